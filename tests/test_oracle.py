"""Pins for the fp64 oracle: each check ties it to something other than itself.

CPU only.  A plausible mistake in the oracle (dropped scale, transposed
operand, off-by-one mask, wrong group map, missing max subtraction, wrong
gradient sign or term) fails at least one test here; the planted-mistake tests
at the bottom show that for several of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from exact_tiled_attention_04_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


TINY = [
    # B, H, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 1, 1, 1, False),
    (1, 1, 1, 5, 5, 3, False),
    (1, 1, 1, 5, 5, 3, True),
    (2, 2, 1, 4, 7, 4, True),    # Nq < Nk, bottom-right causal, GQA
    (1, 4, 2, 6, 6, 8, True),
    (1, 2, 2, 7, 3, 2, True),    # Nq > Nk: first rows see no key
    (1, 3, 3, 8, 8, 5, False),
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal", TINY)
def test_brute_force_agrees(B, H, Hkv, Nq, Nk, d, causal):
    q = _rand((B, H, Nq, d), 1)
    k = _rand((B, Hkv, Nk, d), 2)
    v = _rand((B, Hkv, Nk, d), 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, scale, causal)
    ob, lseb = oracle.brute_force_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    lseb = np.array(lseb)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lseb))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lseb[fin], rtol=0, atol=1e-12)


def test_empty_rows_are_zero_with_neg_inf_lse():
    q = _rand((1, 1, 6, 4), 4)
    k = _rand((1, 1, 2, 4), 5)
    v = _rand((1, 1, 2, 4), 6)
    o, lse = oracle.forward(q, k, v, 0.5, causal=True)
    # Bottom-right alignment: rows 0..3 sit before key 0.
    assert np.all(o[0, 0, :4] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, :4]))
    assert np.all(np.isfinite(lse[0, 0, 4:]))


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows(causal):
    q = _rand((2, 2, 9, 6), 7, 3.0)
    k = _rand((2, 2, 9, 6), 8, 3.0)
    v = _rand((2, 2, 9, 6), 9)
    _, lse, p = oracle.forward_probs(q, k, v, 0.4, causal)
    assert np.all(p >= 0)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    if causal:
        upper = np.triu(np.ones((9, 9), bool), 1)
        assert np.all(p[..., upper] == 0.0)
    # P recomputed from the saved LSE is P itself (the backward's premise).
    s = 0.4 * np.einsum("bhid,bhjd->bhij", q, k)
    p2 = np.exp(s - lse[..., None])
    if causal:
        p2[..., upper] = 0.0
    np.testing.assert_allclose(p2, p, atol=1e-12)


@pytest.mark.parametrize("causal,Nq,Nk", [(False, 7, 7), (True, 7, 7), (True, 4, 9)])
def test_q_zero_closed_form(causal, Nq, Nk):
    """Q = 0: every visible score is 0, so O_i is the mean of the visible V
    rows and LSE_i = ln(number of visible keys)."""
    d = 5
    q = np.zeros((1, 2, Nq, d))
    k = _rand((1, 1, Nk, d), 10)
    v = _rand((1, 1, Nk, d), 11)
    o, lse = oracle.forward(q, k, v, 0.3, causal)
    for i in range(Nq):
        n_vis = (i + (Nk - Nq) + 1) if causal else Nk
        np.testing.assert_allclose(o[0, :, i], np.broadcast_to(
            v[0, 0, :n_vis].mean(0), (2, d)), atol=1e-13)
        np.testing.assert_allclose(lse[0, :, i], math.log(n_vis), atol=1e-13)


@pytest.mark.parametrize("x", [0.5, 3.0, 12.0, 60.0])
def test_one_hot_dominant_score(x):
    """Q_i = a e1, K_j* = b e1, all other K rows orthogonal to e1: the scores
    are x = scale*a*b at j* and 0 elsewhere, so
    O_i = (e^x V_j* + sum_{j != j*} V_j) / (e^x + n - 1)."""
    n, d, jstar = 6, 4, 3
    scale = 0.5
    a = 2.0
    b = x / (scale * a)
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = a
    k = np.zeros((1, 1, n, d))
    k[0, 0, :, 1:] = _rand((n, d - 1), 12)
    k[0, 0, jstar, 0] = b
    v = _rand((1, 1, n, d), 13)
    o, lse = oracle.forward(q, k, v, scale, causal=False)
    others = v[0, 0, [j for j in range(n) if j != jstar]].sum(0)
    expect = (math.exp(x) * v[0, 0, jstar] + others) / (math.exp(x) + n - 1)
    np.testing.assert_allclose(o[0, 0, 0], expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(math.exp(x) + n - 1), rtol=1e-13)
    if x >= 60:
        np.testing.assert_allclose(o[0, 0, 0], v[0, 0, jstar], atol=1e-20 + 1e-24)


def test_key_translation_invariance():
    """Adding u to every key row shifts row i's scores by scale*q_i.u: O is
    unchanged and LSE moves by exactly that amount (softmax is invariant to a
    per-row shift, "Flash attention and IO-aware attention", online softmax)."""
    q = _rand((1, 2, 6, 4), 14)
    k = _rand((1, 2, 6, 4), 15)
    v = _rand((1, 2, 6, 4), 16)
    u = _rand((4,), 17)
    scale = 0.7
    o1, l1 = oracle.forward(q, k, v, scale, causal=False)
    o2, l2 = oracle.forward(q, k + u, v, scale, causal=False)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * (q @ u), atol=1e-12)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (2, 4, 4, 33, 16, False), (2, 4, 4, 33, 16, True),
    (1, 8, 2, 40, 8, True), (1, 6, 3, 17, 32, False)])
def test_torch_sdpa_fp64(B, H, Hkv, N, d, causal):
    """torch's CPU scaled_dot_product_attention in float64 is an independent
    library evaluation of the same definition."""
    q = _rand((B, H, N, d), 18)
    k = _rand((B, Hkv, N, d), 19)
    v = _rand((B, Hkv, N, d), 20)
    scale = 1.0 / math.sqrt(d)
    o, _ = oracle.forward(q, k, v, scale, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=scale, enable_gqa=(H != Hkv))
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


def test_torch_sdpa_rectangular_causal_mask():
    """Nq < Nk causal against SDPA with an explicit lower-triangular mask
    offset by Nk - Nq (torch.tril's diagonal argument)."""
    nq, nk, d = 5, 12, 8
    q = _rand((1, 2, nq, d), 21)
    k = _rand((1, 2, nk, d), 22)
    v = _rand((1, 2, nk, d), 23)
    o, _ = oracle.forward(q, k, v, 0.25, causal=True)
    mask = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=mask, scale=0.25)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


def _blocked_recurrence(q, k, v, scale, causal, block, dt=np.float64):
    """Model of the online-softmax recurrence of "Modern attention kernels"
    ("Online softmax makes tiling exact"), evaluated in the float type ``dt``
    one query row at a time: for each block of keys, the block's scores s,
    the new maximum m' = max(m, max s), the rescale factor exp(m - m'), then
    l <- exp(m - m') l + sum exp(s - m') and o <- exp(m - m') o +
    exp(s - m') V_block; O = o / l and LSE = m + ln l after the last block."""
    q, k, v = (np.asarray(x, dtype=dt) for x in (q, k, v))
    scale = dt(scale)
    nq, d = q.shape
    nk = k.shape[0]
    out = np.zeros((nq, d), dtype=dt)
    lse = np.full(nq, -np.inf)
    for i in range(nq):
        m, ell, acc = dt(-np.inf), dt(0.0), np.zeros(d, dtype=dt)
        for j0 in range(0, nk, block):
            s = scale * (k[j0:j0 + block] @ q[i])
            if causal:
                s = np.where(np.arange(j0, j0 + len(s)) <= i + nk - nq, s, dt(-np.inf))
            m_new = max(m, s.max())
            if m_new == -np.inf:
                continue
            alpha = np.exp(m - m_new) if m > -np.inf else dt(0.0)
            e = np.exp(s - m_new)
            ell = alpha * ell + e.sum()
            acc = alpha * acc + e @ v[j0:j0 + block]
            m = m_new
        if ell > 0:
            out[i] = acc / ell
            lse[i] = float(m) + math.log(float(ell))
    return out, lse


def test_worked_example_fp32_deviation():
    """The worked example of "Flash attention and IO-aware attention": seed 0,
    Q, K, V ~ N(0,1) of [512, 64] drawn in that order, the online softmax in
    float32 over blocks of 128 keys against naive attention; the page prints
    a largest deviation of about 1e-6.  Here the naive side is the fp64
    oracle and the blocked side is the recurrence model above run in float32,
    so the deviation lands at the page's order of magnitude."""
    with open(os.path.join(GOLDEN, "flash_attention_io_aware_worked_example.json")) as f:
        g = json.load(f)
    q, k, v = workloads.prefill(1, 1, 1, g["N"], g["N"], g["d"], dtype="f32", seed=g["seed"])
    # Same draws as seeding the global generator and drawing three [N, d] tensors.
    torch.manual_seed(g["seed"])
    q2, k2, v2 = (torch.randn(g["N"], g["d"]) for _ in range(3))
    assert torch.equal(q[0, 0], q2) and torch.equal(k[0, 0], k2) and torch.equal(v[0, 0], v2)
    o, _ = oracle.forward(q.numpy(), k.numpy(), v.numpy(), g["scale"], causal=False)
    ob, _ = _blocked_recurrence(q2.numpy(), k2.numpy(), v2.numpy(), g["scale"], False,
                                g["block_size"], dt=np.float32)
    assert ob.dtype == np.float32
    dev = float(np.abs(ob.astype(np.float64) - o[0, 0]).max())
    lo, hi = g["accepted_range_for_order_of_magnitude"]
    assert lo <= dev <= hi, dev
    # The page's memory table: N*N*2 bytes in MiB.
    for n, mb in g["memory_table_mb_bf16"].items():
        assert int(n) * int(n) * 2 / 1024 ** 2 == mb


@pytest.mark.parametrize("block", [1, 3, 8, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_equals_definition(block, causal):
    """The recurrence reaches the definition to rounding for any block size,
    including with the row's largest score placed in the last block
    ("Modern attention kernels", "Failure modes": late maximum)."""
    n, d = 37, 6
    q = _rand((n, d), 24)
    k = _rand((n, d), 25)
    v = _rand((n, d), 26)
    k[-1] = 20.0 * q[-1] / np.linalg.norm(q[-1]) ** 2 * 5  # late, dominant key
    o, lse = oracle.forward(q[None, None], k[None, None], v[None, None], 0.9, causal)
    ob, lb = _blocked_recurrence(q, k, v, 0.9, causal, block)
    np.testing.assert_allclose(ob, o[0, 0], atol=1e-12)
    np.testing.assert_allclose(lb, lse[0, 0], atol=1e-11)


@pytest.mark.parametrize("chunks", [1, 2, 7, 16])
def test_split_merge_equals_unsplit(chunks):
    """Split-context merge ("Attention kernels", FlashDecoding): per-chunk
    (o_c unnormalised, m_c, l_c) combined by max-rescaling equals the
    definition over the whole context."""
    n, d = 50, 8
    q = _rand((d,), 27)
    k = _rand((n, d), 28, 2.0)
    v = _rand((n, d), 29)
    scale = 0.35
    o, lse = oracle.forward(q[None, None, None], k[None, None], v[None, None], scale, False)
    edges = np.linspace(0, n, chunks + 1).astype(int)
    parts = []
    for a, b in zip(edges[:-1], edges[1:]):
        s = scale * (k[a:b] @ q)
        m = s.max()
        e = np.exp(s - m)
        parts.append((e @ v[a:b], m, e.sum()))
    big_m = max(p[1] for p in parts)
    w = [math.exp(p[1] - big_m) for p in parts]
    ell = sum(wc * p[2] for wc, p in zip(w, parts))
    om = sum(wc * p[0] for wc, p in zip(w, parts)) / ell
    np.testing.assert_allclose(om, o[0, 0, 0], atol=1e-12)
    np.testing.assert_allclose(big_m + math.log(ell), lse[0, 0, 0], atol=1e-12)


def test_gqa_equals_replicated_heads():
    q = _rand((2, 8, 9, 4), 30)
    k = _rand((2, 2, 11, 4), 31)
    v = _rand((2, 2, 11, 4), 32)
    o1, l1 = oracle.forward(q, k, v, 0.5, causal=True)
    krep = np.repeat(k, 4, axis=1)
    vrep = np.repeat(v, 4, axis=1)
    o2, l2 = oracle.forward(q, krep, vrep, 0.5, causal=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    dq1, dk1, dv1 = oracle.backward(q, k, v, _rand(q.shape, 33), 0.5, True)
    dq2, dk2, dv2 = oracle.backward(q, krep, vrep, _rand(q.shape, 33), 0.5, True)
    np.testing.assert_allclose(dq1, dq2, atol=1e-12)
    np.testing.assert_allclose(dk1, dk2.reshape(2, 2, 4, 11, 4).sum(2), atol=1e-12)
    np.testing.assert_allclose(dv1, dv2.reshape(2, 2, 4, 11, 4).sum(2), atol=1e-12)


# ----------------------------------------------------------------- backward


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.forward(q, k, v, scale, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("causal,Nq,Nk,H,Hkv", [
    (False, 4, 4, 1, 1), (True, 5, 5, 2, 1), (True, 3, 6, 2, 2)])
def test_backward_finite_differences(causal, Nq, Nk, H, Hkv):
    d = 3
    q = _rand((1, H, Nq, d), 34)
    k = _rand((1, Hkv, Nk, d), 35)
    v = _rand((1, Hkv, Nk, d), 36)
    do = _rand((1, H, Nq, d), 37)
    scale = 0.6
    grads = oracle.backward(q, k, v, do, scale, causal)
    eps = 1e-6
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = [q, k, v]; args_p[which] = xp
            args_m = [q, k, v]; args_m[which] = xm
            num[idx] = (_loss(*args_p, do, scale, causal)
                        - _loss(*args_m, do, scale, causal)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_torch_autograd_fp64(causal):
    B, H, Hkv, N, d = 1, 4, 2, 24, 16
    q = _rand((B, H, N, d), 38)
    k = _rand((B, Hkv, N, d), 39)
    v = _rand((B, Hkv, N, d), 40)
    do = _rand((B, H, N, d), 41)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.backward(q, k, v, do, scale, causal)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)


def test_backward_invariants_and_brute_dv():
    """Rows of P sum to 1 so sum_j dV_j = sum_i dO_i; rows of dS sum to 0 so
    sum_j dK_j = 0.  dV also equals a scalar-loop P^T dO."""
    q = _rand((1, 1, 8, 5), 42)
    k = _rand((1, 1, 8, 5), 43)
    v = _rand((1, 1, 8, 5), 44)
    do = _rand((1, 1, 8, 5), 45)
    dq, dk, dv = oracle.backward(q, k, v, do, 0.45, True)
    np.testing.assert_allclose(dv.sum(2), do.sum(2), atol=1e-12)
    np.testing.assert_allclose(dk.sum(2), 0.0, atol=1e-12)
    _, _, p = oracle.forward_probs(q, k, v, 0.45, True)
    np.testing.assert_allclose(dv[0, 0], np.array(
        oracle.brute_force_backward_dv(p[0, 0], do[0, 0])), atol=1e-12)


# ------------------------------------------------------------------- decode


def _small_decode(seed=0, poison=False, **kw):
    args = dict(num_seqs=5, Hq=8, Hkv=2, d=16, ctx_lo=1, ctx_hi=70, block_size=16,
                dtype="f32", seed=seed, poison_tail=poison)
    args.update(kw)
    return workloads.decode(**args)


def test_decode_paged_equals_contiguous_and_last_causal_row():
    w = _small_decode(seed=3)
    scale = 0.25
    o, lse = oracle.decode_paged(w["q"].numpy(), w["k_cache"].numpy(), w["v_cache"].numpy(),
                                 w["block_table"].numpy(), w["context_lens"].numpy(), scale)
    for s in range(w["num_seqs"]):
        ctx = int(w["context_lens"][s])
        ks = oracle.gather_paged(w["k_cache"].numpy(), w["block_table"].numpy(), s, ctx)
        vs = oracle.gather_paged(w["v_cache"].numpy(), w["block_table"].numpy(), s, ctx)
        kk = ks.transpose(1, 0, 2)[None].astype(np.float64)
        vv = vs.transpose(1, 0, 2)[None].astype(np.float64)
        # A causal prefill of ctx queries whose last query is this one.
        qq = np.zeros((1, w["Hq"], ctx, w["d"]))
        qq[0, :, -1] = w["q"][s].numpy()
        of, lf = oracle.forward(qq, kk, vv, scale, causal=True)
        np.testing.assert_allclose(o[s], of[0, :, -1], atol=1e-12)
        np.testing.assert_allclose(lse[s], lf[0, :, -1], atol=1e-12)


def test_decode_permuted_table_equals_identity_table():
    w = _small_decode(seed=4)
    bt = w["block_table"].numpy()
    kc, vc = w["k_cache"].numpy(), w["v_cache"].numpy()
    # Re-lay the same pages out in identity order.
    order = [int(p) for s in range(bt.shape[0]) for p in bt[s] if p >= 0]
    kc2, vc2 = kc[order], vc[order]
    bt2 = np.full_like(bt, -1)
    off = 0
    for s in range(bt.shape[0]):
        n = int((bt[s] >= 0).sum())
        bt2[s, :n] = np.arange(off, off + n)
        off += n
    o1, l1 = oracle.decode_paged(w["q"].numpy(), kc, vc, bt, w["context_lens"].numpy(), 0.3)
    o2, l2 = oracle.decode_paged(w["q"].numpy(), kc2, vc2, bt2, w["context_lens"].numpy(), 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_decode_ignores_poisoned_tail_and_handles_empty():
    w = _small_decode(seed=5, poison=True, context_lens=[0, 1, 16, 17, 33])
    o, lse = oracle.decode_paged(w["q"].numpy(), w["k_cache"].numpy(), w["v_cache"].numpy(),
                                 w["block_table"].numpy(), w["context_lens"].numpy(), 0.25)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(o[1:])) and np.all(np.isfinite(lse[1:]))
    # ctx = 1: the output is the single V row, LSE is the single score.
    phys = int(w["block_table"][1, 0])
    g_of = np.arange(w["Hq"]) // (w["Hq"] // w["Hkv"])
    v_row = w["v_cache"][phys, 0].numpy()[g_of]
    np.testing.assert_allclose(o[1], v_row, atol=1e-12)
    k_row = w["k_cache"][phys, 0].numpy()[g_of]
    np.testing.assert_allclose(lse[1], 0.25 * (w["q"][1].numpy() * k_row).sum(-1), atol=1e-12)


def test_workload_generator_structure():
    w = workloads.decode(num_seqs=6, Hq=4, Hkv=2, d=8, ctx_lo=5, ctx_hi=60,
                         block_size=16, dtype="bf16", seed=1)
    bt = w["block_table"]
    used = bt[bt >= 0]
    assert len(set(used.tolist())) == used.numel() == w["num_blocks"]
    for s, c in enumerate(w["context_lens"].tolist()):
        n = (c + 15) // 16
        assert bool((bt[s, :n] >= 0).all()) and bool((bt[s, n:] == -1).all())
    q, k, v = workloads.prefill(1, 2, 1, 3, 4, 8, dtype="bf16", seed=0)
    assert q.dtype == torch.bfloat16 and k.shape == (1, 1, 4, 8)


# --------------------------------------------------------- planted mistakes


def _pins_pass(monkeypatch_target=None):
    """Run the brute-force and SDPA pins on one causal GQA case."""
    q = _rand((1, 4, 6, 5), 50)
    k = _rand((1, 2, 6, 5), 51)
    v = _rand((1, 2, 6, 5), 52)
    o, lse = oracle.forward(q, k, v, 0.4, True)
    ob, lb = oracle.brute_force_forward(q, k, v, 0.4, True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=True, scale=0.4, enable_gqa=True).numpy()
    return (np.allclose(o, np.array(ob), atol=1e-12) and np.allclose(o, ref, atol=1e-12)
            and np.allclose(lse, np.array(lb), atol=1e-12))


def test_planted_mask_off_by_one_is_caught(monkeypatch):
    assert _pins_pass()
    real = oatt._visible
    monkeypatch.setattr(oatt, "_visible",
                        lambda nq, nk, c, w=None: real(nq, nk + 1, c, w)[:, :nk] if c else real(nq, nk, c, w))
    assert not _pins_pass()


def test_planted_group_map_is_caught(monkeypatch):
    """Plant the interleaved group map (query head h reads KV head h % Hkv
    instead of h // (H / Hkv)): the value pins fail on it."""
    assert _pins_pass()
    monkeypatch.setattr(oatt, "kv_head", lambda h, n_heads, n_kv: h % n_kv)
    assert not _pins_pass()


def test_planted_dropped_scale_is_caught(monkeypatch):
    real = oatt.forward_probs
    monkeypatch.setattr(oatt, "forward_probs", lambda q, k, v, s, c, w=None: real(q, k, v, 1.0, c, w))
    assert not _pins_pass()


def test_planted_transposed_p_in_backward_is_caught(monkeypatch):
    """Hand the backward a transposed P (P^T in place of P, a plausible
    operand mix-up in dV = P^T dO and dS): finite differences fail."""
    q = _rand((1, 1, 4, 3), 53)
    k = _rand((1, 1, 4, 3), 54)
    v = _rand((1, 1, 4, 3), 55)
    do = _rand((1, 1, 4, 3), 56)
    real_fp = oatt.forward_probs

    def transposed_p(q_, k_, v_, s_, c_, w_=None):
        o_, l_, p_ = real_fp(q_, k_, v_, s_, c_, w_)
        return o_, l_, p_.transpose(0, 1, 3, 2)
    monkeypatch.setattr(oatt, "forward_probs", transposed_p)
    dq, dk, dv = oatt.backward(q, k, v, do, 0.5, False)
    monkeypatch.setattr(oatt, "forward_probs", real_fp)
    eps = 1e-6
    num = np.zeros_like(v)
    for idx in np.ndindex(v.shape):
        vp = v.copy(); vp[idx] += eps
        vm = v.copy(); vm[idx] -= eps
        num[idx] = (_loss(q, k, vp, do, 0.5, False) - _loss(q, k, vm, do, 0.5, False)) / (2 * eps)
    assert not np.allclose(dv, num, rtol=1e-6, atol=1e-8)


# ------------------------------------------------------- local (window) band

WINDOWS = [
    # Nq, Nk, causal, (left, right)
    (6, 6, True, (2, None)),      # sliding window of 3 keys
    (6, 6, False, (1, 1)),        # symmetric band
    (5, 8, True, (3, None)),      # rectangular, bottom-right aligned
    (7, 4, False, (0, 2)),        # Nq > Nk: early rows see few or no keys
    (6, 6, False, (None, 0)),     # right = 0 alone is the causal mask
    (6, 6, False, (0, 0)),        # the diagonal only
]


@pytest.mark.parametrize("Nq,Nk,causal,window", WINDOWS)
def test_window_brute_force_agrees(Nq, Nk, causal, window):
    q = _rand((1, 2, Nq, 4), 60)
    k = _rand((1, 1, Nk, 4), 61)
    v = _rand((1, 1, Nk, 4), 62)
    o, lse = oracle.forward(q, k, v, 0.5, causal, window)
    ob, lb = oracle.brute_force_forward(q, k, v, 0.5, causal, window)
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    lb = np.array(lb)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)


def test_window_special_cases():
    """A window wider than the sequence is the plain mask; right = 0 is the
    causal mask; (0, 0) picks exactly the diagonal key: O_i = V_p and
    LSE_i = s_ip."""
    q = _rand((1, 1, 7, 5), 63)
    k = _rand((1, 1, 7, 5), 64)
    v = _rand((1, 1, 7, 5), 65)
    ref_c, lse_c = oracle.forward(q, k, v, 0.7, True)
    for w in [(7, None), (100, 0), (None, None)]:
        o, lse = oracle.forward(q, k, v, 0.7, True, w)
        np.testing.assert_array_equal(o, ref_c)
        np.testing.assert_array_equal(lse, lse_c)
    o, lse = oracle.forward(q, k, v, 0.7, False, (None, 0))
    np.testing.assert_array_equal(o, ref_c)
    ref_f, _ = oracle.forward(q, k, v, 0.7, False)
    o, _ = oracle.forward(q, k, v, 0.7, False, (50, 50))
    np.testing.assert_array_equal(o, ref_f)
    o, lse = oracle.forward(q, k, v, 0.7, False, (0, 0))
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], 0.7 * (q[0, 0] * k[0, 0]).sum(-1), atol=1e-14)


@pytest.mark.parametrize("Nq,Nk,window", [(9, 9, (3, 0)), (6, 10, (2, 1)), (8, 5, (1, 3))])
def test_window_q_zero_closed_form(Nq, Nk, window):
    """Q = 0: O_i is the mean of V over the keys max(0, p - left) ..
    min(Nk - 1, p + right), LSE_i = ln(count); an empty range gives 0, -inf."""
    left, right = window
    q = np.zeros((1, 1, Nq, 3))
    k = _rand((1, 1, Nk, 3), 66)
    v = _rand((1, 1, Nk, 3), 67)
    o, lse = oracle.forward(q, k, v, 0.9, False, window)
    for i in range(Nq):
        p = i + Nk - Nq
        lo, hi = max(0, p - left), min(Nk - 1, p + right)
        if lo > hi:
            assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])
            continue
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, lo:hi + 1].mean(0), atol=1e-14)
        np.testing.assert_allclose(lse[0, 0, i], math.log(hi - lo + 1), atol=1e-14)


def test_window_torch_sdpa_band_mask():
    """torch's fp64 attention with the band written as a boolean mask."""
    B, H, Hkv, Nq, Nk, d = 1, 4, 2, 12, 16, 8
    left, right = 4, 1
    q = _rand((B, H, Nq, d), 68)
    k = _rand((B, Hkv, Nk, d), 69)
    v = _rand((B, Hkv, Nk, d), 70)
    o, _ = oracle.forward(q, k, v, 0.35, False, (left, right))
    i = torch.arange(Nq)[:, None] + (Nk - Nq)
    j = torch.arange(Nk)[None, :]
    band = (j >= i - left) & (j <= i + right)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=band,
        scale=0.35, enable_gqa=True).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)


@pytest.mark.parametrize("causal,window", [(True, (2, None)), (False, (1, 2))])
def test_window_backward_finite_differences(causal, window):
    q = _rand((1, 2, 5, 3), 71)
    k = _rand((1, 1, 6, 3), 72)
    v = _rand((1, 1, 6, 3), 73)
    do = _rand((1, 2, 5, 3), 74)
    scale = 0.8
    grads = oracle.backward(q, k, v, do, scale, causal, window)

    def loss(q_, k_, v_):
        o, _ = oracle.forward(q_, k_, v_, scale, causal, window)
        return float((o * do).sum())
    eps = 1e-6
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            a_p = [q, k, v]; a_p[which] = xp
            a_m = [q, k, v]; a_m[which] = xm
            num[idx] = (loss(*a_p) - loss(*a_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_planted_window_off_by_one_is_caught(monkeypatch):
    """A window that keeps one key too many on the left fails the brute force."""
    q = _rand((1, 1, 6, 4), 75)
    k = _rand((1, 1, 6, 4), 76)
    v = _rand((1, 1, 6, 4), 77)
    real = oatt._visible

    def wrong(nq, nk, c, w=None):
        if w is None:
            return real(nq, nk, c, w)
        return real(nq, nk, c, (w[0] + 1 if w[0] is not None else None, w[1]))
    monkeypatch.setattr(oatt, "_visible", wrong)
    o, _ = oracle.forward(q, k, v, 0.5, True, (2, None))
    ob, _ = oracle.brute_force_forward(q, k, v, 0.5, True, (2, None))
    assert not np.allclose(o, np.array(ob), atol=1e-6)
