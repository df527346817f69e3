"""Paged GQA decode parity: HIP split + merge kernels against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def _to_gpu(w, gpu):
    return {k: (v.to(gpu) if torch.is_tensor(v) else v) for k, v in w.items()}


def _decode(w, gpu, scale, chunk_tokens=0, max_context=None, strides=None):
    g = _to_gpu(w, gpu)
    mc = w["max_context"] if max_context is None else max_context
    o, lse = attn.attn_decode_paged(g["q"], g["k_cache"], g["v_cache"], g["block_table"],
                                    g["context_lens"], scale, max(mc, 1),
                                    chunk_tokens=chunk_tokens, strides=strides)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _oracle(w, scale):
    return oracle.decode_paged(to64(w["q"]), w["k_cache"].float().numpy(),
                               w["v_cache"].float().numpy(), w["block_table"].numpy(),
                               w["context_lens"].numpy(), scale)


CTX_EDGES = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (16, 1)])
def test_decode_page_and_chunk_edges(gpu, d, Hq, Hkv):
    """Context lengths at page (16) and step/chunk (32, 256) boundaries, with
    the slots past each context poisoned with NaN and unused table entries -1."""
    w = workloads.decode(num_seqs=len(CTX_EDGES), Hq=Hq, Hkv=Hkv, d=d, ctx_lo=0, ctx_hi=0,
                         context_lens=CTX_EDGES, dtype="bf16", seed=d + Hq, poison_tail=True,
                         max_blocks_per_seq=70)
    scale = 1.0 / math.sqrt(d)
    o, lse = _decode(w, gpu, scale, chunk_tokens=256)
    o_ref, lse_ref = _oracle(w, scale)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


@pytest.mark.parametrize("block_size", [1, 8, 32, 48])
def test_block_sizes(gpu, block_size):
    """Block sizes other than 16: multiples of 16 take the page-group path
    (several groups per page), the others the per-token path."""
    ctx = [1, 15, 16, 17, 47, 48, 49, 95, 96, 97, 300]
    w = workloads.decode(num_seqs=len(ctx), Hq=16, Hkv=4, d=128, ctx_lo=0, ctx_hi=0,
                         context_lens=ctx, block_size=block_size, dtype="bf16",
                         seed=block_size, poison_tail=True)
    scale = 1.0 / math.sqrt(128)
    o, lse = _decode(w, gpu, scale, chunk_tokens=64)
    o_ref, lse_ref = _oracle(w, scale)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


@pytest.mark.parametrize("chunk", [32, 64, 96, 256, 1024, 0])
def test_split_count_invariance(gpu, chunk):
    """Any work-item length (any number of partials per pair) gives the
    oracle's result."""
    w = workloads.decode(num_seqs=6, Hq=32, Hkv=8, d=128, ctx_lo=900, ctx_hi=3000,
                         dtype="bf16", seed=7, poison_tail=True)
    scale = 1.0 / math.sqrt(128)
    o, lse = _decode(w, gpu, scale, chunk_tokens=chunk)
    o_ref, lse_ref = _oracle(w, scale)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


@pytest.mark.parametrize("block_size", [16, 8])
def test_many_sequences_with_empty_ones(gpu, block_size):
    """More than 64 sequences (the split kernels locate their sequence 64 at
    a time), many of them empty, so the live work items are packed across
    sequence-group boundaries."""
    rng = np.random.default_rng(31)
    ctx = rng.integers(1, 200, size=150)
    ctx[rng.random(150) < 0.3] = 0
    ctx[[0, 63, 64, 127, 128, 149]] = [0, 199, 0, 1, 64, 33]
    w = workloads.decode(num_seqs=150, Hq=8, Hkv=2, d=128, ctx_lo=0, ctx_hi=0,
                         context_lens=ctx.tolist(), block_size=block_size, dtype="bf16",
                         seed=31, poison_tail=True)
    scale = 1.0 / math.sqrt(128)
    o, lse = _decode(w, gpu, scale, chunk_tokens=32)
    o_ref, lse_ref = _oracle(w, scale)
    empty = torch.from_numpy(ctx == 0)
    assert torch.all(o[empty] == 0) and torch.all(torch.isneginf(lse[empty]))
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


@pytest.mark.parametrize("block_size,chunk", [(16, 0), (16, 96), (8, 0), (32, 4064)])
def test_split_ranges_cross_pairs(gpu, block_size, chunk):
    """The split cuts the steps of all (sequence, KV head) pairs, laid end to
    end, into equal ranges: one long context spread over many waves, short
    and empty ones packed several to a wave, ranges starting and ending inside
    pairs.  The automatic split (chunk 0) picks its range length on the device."""
    rng = np.random.default_rng(41)
    ctx = rng.integers(1, 120, size=90)
    ctx[rng.random(90) < 0.2] = 0
    ctx[[0, 5, 40, 64, 89]] = [9000, 0, 4097, 33, 2500]
    w = workloads.decode(num_seqs=90, Hq=24, Hkv=8, d=128, ctx_lo=0, ctx_hi=0,
                         context_lens=ctx.tolist(), block_size=block_size, dtype="bf16",
                         seed=41, poison_tail=True)
    scale = 1.0 / math.sqrt(128)
    o, lse = _decode(w, gpu, scale, chunk_tokens=chunk)
    o_ref, lse_ref = _oracle(w, scale)
    empty = torch.from_numpy(ctx == 0)
    assert torch.all(o[empty] == 0) and torch.all(torch.isneginf(lse[empty]))
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


@pytest.mark.parametrize("d,Hq,Hkv,block_size", [(128, 32, 1, 16), (128, 48, 2, 16),
                                                 (64, 40, 2, 16), (128, 24, 1, 8)])
def test_groups_above_16_heads(gpu, d, Hq, Hkv, block_size):
    """Groups of more than 16 query heads per KV head (multi-query 32:1, 24:1,
    20:1): subgroups of 16 heads are pairs of their own in the split."""
    ctx = [1, 17, 300, 1000, 0, 2049, 64]
    w = workloads.decode(num_seqs=len(ctx), Hq=Hq, Hkv=Hkv, d=d, ctx_lo=0, ctx_hi=0,
                         context_lens=ctx, block_size=block_size, dtype="bf16",
                         seed=Hq + d + block_size, poison_tail=True)
    scale = 1.0 / math.sqrt(d)
    for chunk in (0, 64):
        o, lse = _decode(w, gpu, scale, chunk_tokens=chunk)
        o_ref, lse_ref = _oracle(w, scale)
        check_out(to64(o), o_ref, "bf16")
        check_lse(to64(lse), lse_ref, "bf16")


def test_reused_workspace_other_contexts(gpu):
    """A workspace left by a call with other context lengths (pairs that were
    empty become live and the reverse) gives the oracle's result: the merge
    reads only what this call's split wrote."""
    ctx_a = [0, 700, 33, 0, 1500, 64]
    ctx_b = [900, 0, 31, 2000, 1, 0]
    ws = torch.empty(attn.attn_decode_paged_workspace_size(6, 16, 128, 2048, 64) + 16,
                     dtype=torch.uint8, device=gpu)
    scale = 1.0 / math.sqrt(128)
    for ctx, seed in ((ctx_a, 51), (ctx_b, 52)):
        w = workloads.decode(num_seqs=6, Hq=16, Hkv=4, d=128, ctx_lo=0, ctx_hi=0,
                             context_lens=ctx, dtype="bf16", seed=seed, poison_tail=True,
                             max_blocks_per_seq=128)
        g = _to_gpu(w, gpu)
        o, lse = attn.attn_decode_paged(g["q"], g["k_cache"], g["v_cache"], g["block_table"],
                                        g["context_lens"], scale, 2048, chunk_tokens=64,
                                        workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref = _oracle(w, scale)
        check_out(to64(o.cpu()), o_ref, "bf16")
        check_lse(to64(lse.cpu()), lse_ref, "bf16")


def test_empty_and_clamped_contexts(gpu):
    """ctx <= 0 gives O = 0, LSE = -inf; ctx above max_context is clamped."""
    w = workloads.decode(num_seqs=4, Hq=8, Hkv=2, d=128, ctx_lo=0, ctx_hi=0,
                         context_lens=[0, 40, 100, 100], dtype="bf16", seed=9)
    w["context_lens"][0] = -5
    scale = 0.1
    o, lse = _decode(w, gpu, scale, max_context=64)
    clamped = dict(w)
    clamped["context_lens"] = torch.clamp(w["context_lens"], max=64)
    o_ref, lse_ref = _oracle(clamped, scale)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_permuted_table_equals_identity_table(gpu):
    w = workloads.decode(num_seqs=5, Hq=32, Hkv=8, d=128, ctx_lo=100, ctx_hi=700,
                         dtype="bf16", seed=12)
    bt = w["block_table"]
    order = [int(p) for s in range(bt.shape[0]) for p in bt[s] if p >= 0]
    w2 = dict(w)
    w2["k_cache"] = w["k_cache"][order].contiguous()
    w2["v_cache"] = w["v_cache"][order].contiguous()
    bt2 = torch.full_like(bt, -1)
    off = 0
    for s in range(bt.shape[0]):
        n = int((bt[s] >= 0).sum())
        bt2[s, :n] = torch.arange(off, off + n, dtype=torch.int32)
        off += n
    w2["block_table"] = bt2
    o1, l1 = _decode(w, gpu, 0.09)
    o2, l2 = _decode(w2, gpu, 0.09)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_invalid_block_entries_are_skipped(gpu):
    """A live token whose table entry points outside the cache is excluded
    (page-table mismatch cannot read out of bounds); the result is the
    oracle's over the remaining tokens."""
    w = workloads.decode(num_seqs=3, Hq=8, Hkv=2, d=64, ctx_lo=0, ctx_hi=0,
                         context_lens=[50, 64, 20], dtype="bf16", seed=13)
    bt = w["block_table"].clone()
    bt[0, 1] = w["num_blocks"] + 5   # tokens 16..31 of sequence 0
    bt[1, 3] = -7                    # tokens 48..63 of sequence 1
    w_bad = dict(w)
    w_bad["block_table"] = bt
    o, lse = _decode(w_bad, gpu, 0.125)
    # Oracle over the valid tokens only: drop the bad pages from the context.
    for s, drop in [(0, 1), (1, 3)]:
        ctx = int(w["context_lens"][s])
        keep = [p for p in range(ctx) if p // 16 != drop]
        kk = oracle.gather_paged(w["k_cache"].float().numpy(), w["block_table"].numpy(), s, ctx)[keep]
        vv = oracle.gather_paged(w["v_cache"].float().numpy(), w["block_table"].numpy(), s, ctx)[keep]
        o_ref, lse_ref = oracle.forward(to64(w["q"][s])[None, :, None, :],
                                        kk.transpose(1, 0, 2)[None].astype(np.float64),
                                        vv.transpose(1, 0, 2)[None].astype(np.float64),
                                        0.125, False)
        check_out(to64(o[s]), o_ref[0, :, 0], "bf16")
        check_lse(to64(lse[s]), lse_ref[0, :, 0], "bf16")


def test_non_default_strides(gpu):
    """Cache rows described by strides: head stride padded to 2 d."""
    w = workloads.decode(num_seqs=4, Hq=16, Hkv=4, d=64, ctx_lo=30, ctx_hi=400, dtype="bf16",
                         seed=14, poison_tail=True)
    nb, bs, hkv, d = w["k_cache"].shape
    pad_k = torch.full((nb, bs, hkv, 2 * d), float("nan"), dtype=torch.bfloat16)
    pad_v = pad_k.clone()
    pad_k[..., :d] = w["k_cache"]
    pad_v[..., :d] = w["v_cache"]
    g = _to_gpu(w, gpu)
    o, lse = attn.attn_decode_paged(g["q"], pad_k.to(gpu), pad_v.to(gpu), g["block_table"],
                                    g["context_lens"], 0.125, w["max_context"],
                                    strides=(bs * hkv * 2 * d, hkv * 2 * d, 2 * d))
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(w, 0.125)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_decode_matches_last_row_of_causal_prefill(gpu):
    """Decode of the last token = last row of the causal forward over the same
    contiguous K/V (both on the device)."""
    ctx, hq, hkv, d = 777, 32, 8, 128
    w = workloads.decode(num_seqs=1, Hq=hq, Hkv=hkv, d=d, ctx_lo=0, ctx_hi=0,
                         context_lens=[ctx], dtype="bf16", seed=15)
    kk = torch.from_numpy(oracle.gather_paged(w["k_cache"].float().numpy(),
                                              w["block_table"].numpy(), 0, ctx))
    vv = torch.from_numpy(oracle.gather_paged(w["v_cache"].float().numpy(),
                                              w["block_table"].numpy(), 0, ctx))
    kpre = kk.permute(1, 0, 2)[None].to(torch.bfloat16).contiguous().to(gpu)
    vpre = vv.permute(1, 0, 2)[None].to(torch.bfloat16).contiguous().to(gpu)
    qpre = torch.zeros(1, hq, ctx, d, dtype=torch.bfloat16)
    qpre[0, :, -1] = w["q"][0]
    o_pre, l_pre = attn.attn_fwd(qpre.to(gpu), kpre, vpre, 1 / math.sqrt(d), True)
    o_dec, l_dec = _decode(w, gpu, 1 / math.sqrt(d))
    o_ref, lse_ref = _oracle(w, 1 / math.sqrt(d))
    check_out(to64(o_dec), o_ref, "bf16", what="O decode vs oracle")
    check_lse(to64(l_dec), lse_ref, "bf16", what="LSE decode vs oracle")
    check_out(to64(o_pre[0, :, -1])[None], o_ref, "bf16", what="O prefill last row vs oracle")
    check_lse(to64(l_pre[0, :, -1])[None], lse_ref, "bf16", what="LSE prefill last row vs oracle")
    check_out(to64(o_pre[0, :, -1]), to64(o_dec[0]), "bf16", what="O prefill vs decode kernel")


def test_paged_gqa_decode_64seq_full_size(gpu):
    """64 sequences, Hq=32, Hkv=8, d=128, contexts uniform in [4096, 32768],
    16-token pages from a seeded permutation, tail slots poisoned with NaN;
    full-size launch with the benchmark's automatic split.  Every query head
    of every sequence is compared with the oracle over its gathered context."""
    spec = workloads.WORKLOADS["paged_gqa_decode_bf16_s64_hq32_hkv8_d128"]
    w = workloads.decode(num_seqs=spec["num_seqs"], Hq=spec["Hq"], Hkv=spec["Hkv"], d=spec["d"],
                         ctx_lo=spec["ctx_lo"], ctx_hi=spec["ctx_hi"],
                         block_size=spec["block_size"],
                         max_blocks_per_seq=spec["max_blocks_per_seq"], dtype="bf16",
                         seed=spec["seed"], device=str(gpu), poison_tail=True)
    scale = spec["scale"]
    g = {k: (v.to(gpu) if torch.is_tensor(v) else v) for k, v in w.items()}
    o, lse = attn.attn_decode_paged(g["q"], g["k_cache"], g["v_cache"], g["block_table"],
                                    g["context_lens"], scale, spec["ctx_hi"])
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    bt = w["block_table"]
    bs = spec["block_size"]
    for s in range(spec["num_seqs"]):
        ctx = int(w["context_lens"][s])
        pages = bt[s, : (ctx + bs - 1) // bs].long().to(gpu)
        kk = w["k_cache"][pages].reshape(-1, spec["Hkv"], spec["d"])[:ctx].cpu()
        vv = w["v_cache"][pages].reshape(-1, spec["Hkv"], spec["d"])[:ctx].cpu()
        o_ref, lse_ref = oracle.forward(to64(w["q"][s].cpu())[None, :, None, :],
                                        to64(kk).transpose(1, 0, 2)[None],
                                        to64(vv).transpose(1, 0, 2)[None], scale, False)
        check_out(to64(o[s]), o_ref[0, :, 0], "bf16", what=f"O seq {s}")
        check_lse(to64(lse[s]), lse_ref[0, :, 0], "bf16", what=f"LSE seq {s}")


@pytest.mark.parametrize("d", [64, 128])
def test_head_major_page_layout(gpu, d):
    """Pages stored head-major ([block, head, slot, d], each KV head's 16
    rows contiguous) through the stride arguments: same result as the
    token-major cache it was permuted from."""
    w = workloads.decode(num_seqs=5, Hq=16, Hkv=4, d=d, ctx_lo=1, ctx_hi=700, dtype="bf16",
                         seed=30 + d, poison_tail=True)
    nb, bs, hkv, _ = w["k_cache"].shape
    kh = w["k_cache"].permute(0, 2, 1, 3).contiguous()
    vh = w["v_cache"].permute(0, 2, 1, 3).contiguous()
    g = _to_gpu(w, gpu)
    o, lse = attn.attn_decode_paged(g["q"], kh.to(gpu), vh.to(gpu), g["block_table"],
                                    g["context_lens"], 0.1, w["max_context"], chunk_tokens=64,
                                    strides=(hkv * bs * d, d, bs * d), cache_dims=(nb, bs, hkv))
    torch.cuda.synchronize()
    o_ref, lse_ref = _oracle(w, 0.1)
    check_out(to64(o.cpu()), o_ref, "bf16")
    check_lse(to64(lse.cpu()), lse_ref, "bf16")
