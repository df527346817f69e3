"""Pins for the oracle's ragged, paged-prefill and block-sparse definitions.

CPU only.  Each check ties the new oracle functions to something other than
themselves: the scalar brute force (with its own visibility test and its own
gather loop), torch's fp64 attention with an explicit boolean mask, closed
forms, the already-pinned dense forward and paged decode, and planted
mistakes that must be caught.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)


# ------------------------------------------------------------------ ragged

RAGGED = [
    # q lengths, k lengths, causal, window
    ([3, 0, 5, 1], [3, 4, 7, 6], True, None),     # chunks shorter than contexts
    ([4, 2, 6], [4, 2, 6], True, None),           # square sequences
    ([5, 3], [2, 0], True, None),                 # Nq > Nk and an empty context
    ([2, 6, 1], [7, 3, 5], False, None),
    ([6, 4], [6, 8], False, (2, 1)),              # local band within each sequence
]


@pytest.mark.parametrize("qlens,klens,causal,window", RAGGED)
def test_ragged_brute_force(qlens, klens, causal, window):
    """Each packed sequence equals the scalar brute force run on it alone."""
    H, Hkv, d = 4, 2, 3
    cu_q, cu_k = _cu(qlens), _cu(klens)
    q = _rand((cu_q[-1], H, d), 1)
    k = _rand((cu_k[-1], Hkv, d), 2)
    v = _rand((cu_k[-1], Hkv, d), 3)
    scale = 0.6
    o, lse = oracle.prefill_ragged(q, k, v, cu_q, cu_k, scale, causal, window)
    assert o.shape == q.shape and lse.shape == (H, cu_q[-1])
    for s in range(len(qlens)):
        q0, q1, k0, k1 = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        if q1 == q0:
            continue
        # brute force takes [B, H, N, d]: build the per-sequence arrays by hand.
        qs = [[[list(q[i, h]) for i in range(q0, q1)] for h in range(H)]]
        ks = [[[list(k[j, g]) for j in range(k0, k1)] for g in range(Hkv)]]
        vs = [[[list(v[j, g]) for j in range(k0, k1)] for g in range(Hkv)]]
        if k1 == k0:
            assert np.all(o[q0:q1] == 0) and np.all(np.isneginf(lse[:, q0:q1]))
            continue
        ob, lb = oracle.brute_force_forward(qs, ks, vs, scale, causal, window)
        for h in range(H):
            for i in range(q1 - q0):
                np.testing.assert_allclose(o[q0 + i, h], ob[0][h][i], atol=1e-12)
                if math.isinf(lb[0][h][i]):
                    assert np.isneginf(lse[h, q0 + i])
                else:
                    assert abs(lse[h, q0 + i] - lb[0][h][i]) < 1e-12


def test_ragged_equal_lengths_is_dense_batch():
    """All sequences of one length: the packed layout is the dense batch
    [B, H, N, d] transposed to [B*N, H, d]."""
    B, H, N, d = 3, 2, 5, 4
    q = _rand((B, H, N, d), 4)
    k = _rand((B, H, N, d), 5)
    v = _rand((B, H, N, d), 6)
    o, lse = oracle.forward(q, k, v, 0.5, True)
    pack = lambda t: t.transpose(0, 2, 1, 3).reshape(B * N, H, d)  # noqa: E731
    cu = _cu([N] * B)
    o2, lse2 = oracle.prefill_ragged(pack(q), pack(k), pack(v), cu, cu, 0.5, True)
    np.testing.assert_allclose(o2, pack(o), atol=1e-13)
    np.testing.assert_allclose(lse2, lse.transpose(1, 0, 2).reshape(H, B * N), atol=1e-13)


def test_ragged_sequences_are_independent():
    """Changing one sequence's keys leaves the other sequences untouched."""
    cu_q, cu_k = _cu([3, 4]), _cu([5, 6])
    q = _rand((7, 2, 3), 7)
    k = _rand((11, 2, 3), 8)
    v = _rand((11, 2, 3), 9)
    o1, l1 = oracle.prefill_ragged(q, k, v, cu_q, cu_k, 0.5, True)
    k2 = k.copy()
    k2[5:] = _rand(k2[5:].shape, 35)
    o2, l2 = oracle.prefill_ragged(q, k2, v, cu_q, cu_k, 0.5, True)
    np.testing.assert_array_equal(o1[:3], o2[:3])
    np.testing.assert_array_equal(l1[:, :3], l2[:, :3])
    assert not np.allclose(o1[3:], o2[3:])


# ----------------------------------------------------------- paged prefill

def _paged(klens, bs, Hkv, d, seed, perm=True, poison=True):
    """Cache [P, bs, Hkv, d] with each sequence on a slice of a (seeded)
    permutation of pages; slots past a context are NaN; -1 marks unused
    table entries."""
    rng = np.random.default_rng(seed)
    pages = [(c + bs - 1) // bs for c in klens]
    total = sum(pages) + 2
    order = rng.permutation(total) if perm else np.arange(total)
    table = -np.ones((len(klens), max(max(pages), 1)), dtype=np.int64)
    off = 0
    for s, n in enumerate(pages):
        table[s, :n] = order[off:off + n]
        off += n
    kc = rng.standard_normal((total, bs, Hkv, d))
    vc = rng.standard_normal((total, bs, Hkv, d))
    if poison:
        for s, c in enumerate(klens):
            if c % bs:
                kc[table[s, c // bs], c % bs:] = np.nan
                vc[table[s, c // bs], c % bs:] = np.nan
        used = set(table[table >= 0].tolist())
        for p in range(total):
            if p not in used:
                kc[p] = np.nan
                vc[p] = np.nan
    return kc, vc, table


def _gather_loop(cache, table, s, ctx, bs):
    """The paged gather written as a loop over tokens (not ``gather_paged``)."""
    rows = []
    for pos in range(ctx):
        rows.append(cache[table[s][pos // bs]][pos % bs])
    return np.array(rows).reshape(ctx, cache.shape[2], cache.shape[3])


@pytest.mark.parametrize("qlens,klens,causal,window", [
    ([2, 3, 1, 0], [5, 3, 9, 4], True, None),
    ([4, 1], [4, 7], False, None),
    ([3, 2], [8, 6], True, (2, None)),
])
def test_paged_prefill_brute_force(qlens, klens, causal, window):
    bs, H, Hkv, d = 4, 4, 2, 3
    kc, vc, table = _paged(klens, bs, Hkv, d, 10)
    cu_q = _cu(qlens)
    q = _rand((cu_q[-1], H, d), 11)
    o, lse = oracle.prefill_paged(q, kc, vc, table, cu_q, klens, 0.7, causal, window)
    assert np.all(np.isfinite(o))
    for s in range(len(qlens)):
        q0, q1 = cu_q[s], cu_q[s + 1]
        if q1 == q0:
            continue
        ks = _gather_loop(kc, table, s, klens[s], bs)
        vs = _gather_loop(vc, table, s, klens[s], bs)
        qs = [[[list(q[i, h]) for i in range(q0, q1)] for h in range(H)]]
        kk = [[[list(ks[j, g]) for j in range(klens[s])] for g in range(Hkv)]]
        vv = [[[list(vs[j, g]) for j in range(klens[s])] for g in range(Hkv)]]
        ob, lb = oracle.brute_force_forward(qs, kk, vv, 0.7, causal, window)
        for h in range(H):
            for i in range(q1 - q0):
                np.testing.assert_allclose(o[q0 + i, h], ob[0][h][i], atol=1e-12)
                assert abs(lse[h, q0 + i] - lb[0][h][i]) < 1e-12


def test_paged_prefill_chunk_is_tail_of_full_prefill():
    """A chunk of the last q rows equals the last q rows of a causal prefill
    over the whole context (bottom-right alignment), against torch's fp64
    attention with the explicit mask tril(diagonal = k - q)."""
    bs, H, Hkv, d = 8, 2, 1, 5
    klens, qlens = [13, 20], [4, 20]
    kc, vc, table = _paged(klens, bs, Hkv, d, 12)
    cu_q = _cu(qlens)
    q = _rand((cu_q[-1], H, d), 13)
    o, lse = oracle.prefill_paged(q, kc, vc, table, cu_q, klens, 0.4, True)
    for s in range(2):
        ks = _gather_loop(kc, table, s, klens[s], bs)
        vs = _gather_loop(vc, table, s, klens[s], bs)
        qs = q[cu_q[s]:cu_q[s + 1]]
        mask = torch.ones(qlens[s], klens[s], dtype=torch.bool).tril(diagonal=klens[s] - qlens[s])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qs.transpose(1, 0, 2)[None]),
            torch.from_numpy(np.repeat(ks.transpose(1, 0, 2)[None], H // Hkv, axis=1)),
            torch.from_numpy(np.repeat(vs.transpose(1, 0, 2)[None], H // Hkv, axis=1)),
            attn_mask=mask, scale=0.4)
        np.testing.assert_allclose(o[cu_q[s]:cu_q[s + 1]], ref[0].numpy().transpose(1, 0, 2),
                                   atol=1e-12)


def test_paged_prefill_one_row_is_decode():
    """One query row per sequence is exactly paged decode."""
    bs, H, Hkv, d = 4, 4, 2, 6
    klens = [7, 1, 12]
    kc, vc, table = _paged(klens, bs, Hkv, d, 14, poison=False)
    q = _rand((3, H, d), 15)
    o, lse = oracle.prefill_paged(q, kc, vc, table, _cu([1, 1, 1]), klens, 0.5, True)
    od, ld = oracle.decode_paged(q, kc, vc, table, klens, 0.5)
    np.testing.assert_allclose(o, od, atol=1e-13)
    np.testing.assert_allclose(lse.T, ld, atol=1e-13)


def test_paged_prefill_permuted_equals_identity_table():
    bs, H, Hkv, d = 4, 2, 2, 3
    klens, qlens = [9, 5], [3, 5]
    kp, vp, tp = _paged(klens, bs, Hkv, d, 16, perm=True, poison=False)
    ki, vi, ti = _paged(klens, bs, Hkv, d, 16, perm=False, poison=False)
    # Same logical contents: move the identity cache's pages to the permuted slots.
    for s in range(2):
        for lb in range((klens[s] + bs - 1) // bs):
            kp[tp[s, lb]] = ki[ti[s, lb]]
            vp[tp[s, lb]] = vi[ti[s, lb]]
    q = _rand((8, H, d), 17)
    o1, l1 = oracle.prefill_paged(q, kp, vp, tp, _cu(qlens), klens, 0.5, True)
    o2, l2 = oracle.prefill_paged(q, ki, vi, ti, _cu(qlens), klens, 0.5, True)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


# ------------------------------------------------------------ block sparse

def _csr(blocks):
    """CSR block index of a dense boolean [L, R, C] block matrix, written
    independently of ``block_mask_from_index``."""
    n_layouts, rows, _ = blocks.shape
    row_ptr = np.zeros((n_layouts, rows + 1), dtype=np.int64)
    cols = []
    for lay in range(n_layouts):
        for r in range(rows):
            row_ptr[lay, r] = len(cols)
            cols.extend(np.nonzero(blocks[lay, r])[0].tolist())
        row_ptr[lay, rows] = len(cols)
    return row_ptr, np.array(cols, dtype=np.int64)


def test_block_index_round_trip():
    rng = np.random.default_rng(18)
    blocks = rng.random((3, 4, 5)) < 0.4
    row_ptr, col_idx = _csr(blocks)
    np.testing.assert_array_equal(oracle.block_mask_from_index(row_ptr, col_idx, 4, 5), blocks)


@pytest.mark.parametrize("Nq,Nk,bq,bk,causal,L", [
    (8, 8, 2, 2, False, 1), (8, 8, 2, 2, True, 2), (6, 9, 3, 2, True, 4), (7, 5, 2, 3, False, 3)])
def test_block_sparse_brute_force(Nq, Nk, bq, bk, causal, L):
    B, H, d = 2, 2, 3
    rng = np.random.default_rng(19)
    blocks = rng.random((L, -(-Nq // bq), -(-Nk // bk))) < 0.5
    q = _rand((B, H, Nq, d), 20)
    k = _rand((B, 1, Nk, d), 21)
    v = _rand((B, 1, Nk, d), 22)
    o, lse = oracle.block_sparse_forward(q, k, v, 0.5, causal, blocks, bq, bk)
    ob, lb = oracle.brute_force_forward(
        q, k, v, 0.5, causal,
        allowed=lambda b, h, i, j: bool(blocks[(b * H + h) % L][i // bq][j // bk]))
    np.testing.assert_allclose(o, np.array(ob), atol=1e-12)
    lb = np.array(lb)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], lb[fin], atol=1e-12)


def test_block_sparse_special_cases():
    """Every block listed = dense attention; the lower block triangle with
    the causal mask = causal attention (the blocks above the diagonal hold
    no visible pair)."""
    q = _rand((1, 2, 12, 4), 23)
    k = _rand((1, 2, 12, 4), 24)
    v = _rand((1, 2, 12, 4), 25)
    full = np.ones((1, 3, 3), dtype=bool)
    o1, l1 = oracle.block_sparse_forward(q, k, v, 0.5, False, full, 4, 4)
    o2, l2 = oracle.forward(q, k, v, 0.5, False)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    tri = np.tril(np.ones((3, 3), dtype=bool))[None]
    o3, l3 = oracle.block_sparse_forward(q, k, v, 0.5, True, tri, 4, 4)
    o4, l4 = oracle.forward(q, k, v, 0.5, True)
    np.testing.assert_allclose(o3, o4, atol=1e-14)
    np.testing.assert_allclose(l3, l4, atol=1e-14)


def test_block_sparse_torch_sdpa_mask_and_q_zero():
    """torch's fp64 attention with the expanded boolean mask; and Q = 0,
    whose rows are the mean of the V rows of their listed blocks."""
    Nq, Nk, bq, bk, d = 8, 12, 4, 4, 5
    blocks = np.array([[[True, False, True], [False, True, True]]])
    q = _rand((1, 1, Nq, d), 26)
    k = _rand((1, 1, Nk, d), 27)
    v = _rand((1, 1, Nk, d), 28)
    o, _ = oracle.block_sparse_forward(q, k, v, 0.3, False, blocks, bq, bk)
    mask = torch.from_numpy(np.kron(blocks[0], np.ones((bq, bk), dtype=bool)).astype(bool))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.3)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    o0, l0 = oracle.block_sparse_forward(np.zeros_like(q), k, v, 0.3, False, blocks, bq, bk)
    np.testing.assert_allclose(o0[0, 0, :4], np.broadcast_to(v[0, 0, np.r_[0:4, 8:12]].mean(0), (4, d)),
                               atol=1e-13)
    np.testing.assert_allclose(o0[0, 0, 4:], np.broadcast_to(v[0, 0, 4:12].mean(0), (4, d)), atol=1e-13)
    np.testing.assert_allclose(l0[0, 0, :4], math.log(8), atol=1e-13)


def test_planted_block_transpose_is_caught(monkeypatch):
    """Looking the block matrix up as (key block, query block) fails the
    brute-force pin."""
    Nq, Nk, bq, bk = 6, 6, 2, 2
    blocks = np.array([[[True, False, False], [True, True, False], [False, True, True]]])
    q = _rand((1, 1, Nq, 3), 29)
    k = _rand((1, 1, Nk, 3), 30)
    v = _rand((1, 1, Nk, 3), 31)
    real = oatt.forward

    def wrong(q_, k_, v_, s_, c_, w_=None, mask=None):
        return real(q_, k_, v_, s_, c_, w_, mask=None if mask is None else mask.transpose(0, 1, 3, 2))
    monkeypatch.setattr(oatt, "forward", wrong)
    o, _ = oatt.block_sparse_forward(q, k, v, 0.5, False, blocks, bq, bk)
    ob, _ = oracle.brute_force_forward(q, k, v, 0.5, False,
                                       allowed=lambda b, h, i, j: bool(blocks[0][i // bq][j // bk]))
    assert not np.allclose(o, np.array(ob), atol=1e-6)


def test_planted_global_causal_offset_is_caught(monkeypatch):
    """Aligning every sequence with the batch-wide offset total_k - total_q
    instead of its own k - q fails the ragged brute-force pin."""
    qlens, klens = [3, 0, 5, 1], [3, 4, 7, 6]
    cu_q, cu_k = _cu(qlens), _cu(klens)
    q = _rand((cu_q[-1], 2, 3), 32)
    k = _rand((cu_k[-1], 1, 3), 33)
    v = _rand((cu_k[-1], 1, 3), 34)
    good, _ = oracle.prefill_ragged(q, k, v, cu_q, cu_k, 0.5, True)
    real_vis = oatt._visible
    shift = int(cu_k[-1] - cu_q[-1])
    monkeypatch.setattr(oatt, "_visible",
                        lambda nq, nk, c, w=None: real_vis(nq, nq + shift, c, w)[:, :nk]
                        if nq + shift >= nk else real_vis(nq, nk, c, w))
    bad, _ = oatt.prefill_ragged(q, k, v, cu_q, cu_k, 0.5, True)
    assert not np.allclose(good, bad, atol=1e-6)
