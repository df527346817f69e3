"""Packed ragged prefill and paged (chunked) prefill: HIP kernels against the
fp64 oracle's per-sequence definitions."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu

# Lengths around the 128-row query tile and the 32/64-key tiles, an empty
# sequence, single rows, and contexts longer and shorter than the queries.
RAGGED_CASES = [
    # q_lens, k_lens, (window_left, window_right)
    ([1, 127, 128, 129, 300, 0, 513], [1, 127, 128, 129, 300, 0, 513], (-1, 0)),
    ([1, 127, 128, 129, 300, 0, 513], [1, 127, 128, 129, 300, 0, 513], (-1, -1)),
    ([64, 200, 1, 33], [700, 450, 90, 33], (-1, 0)),     # chunks at the end of longer contexts
    ([300, 20, 150], [100, 0, 149], (-1, 0)),             # more queries than keys; empty context
    ([257, 96], [257, 400], (63, 0)),                     # sliding window of 64 keys
    ([190, 80], [190, 300], (40, 17)),                    # two-sided band
]


def _band(window):
    """The C ABI's window sides as the oracle's band ((-1, 0) is the causal
    mask, (-1, -1) none)."""
    wl, wr = window
    if (wl, wr) == (-1, -1):
        return None
    return (None if wl < 0 else wl, None if wr < 0 else wr)


def _ragged_ref(w, scale, window):
    return oracle.prefill_ragged(to64(w["q"]), to64(w["k"]), to64(w["v"]), w["cu_q"].numpy(),
                                 w["cu_k"].numpy(), scale, False, _band(window))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 2)])
@pytest.mark.parametrize("case", range(len(RAGGED_CASES)))
def test_varlen_parity(gpu, d, H, Hkv, case):
    q_lens, k_lens, window = RAGGED_CASES[case]
    w = workloads.ragged(q_lens, k_lens, H, Hkv, d, seed=case * 10 + d + H)
    scale = 1.0 / math.sqrt(d)
    o, lse = attn.attn_fwd_varlen(w["q"].to(gpu), w["k"].to(gpu), w["v"].to(gpu),
                                  w["cu_q"].to(gpu), w["cu_k"].to(gpu), w["max_q"], scale,
                                  *window)
    torch.cuda.synchronize()
    o_ref, lse_ref = _ragged_ref(w, scale, window)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_varlen_equal_lengths_matches_dense_forward(gpu):
    """All sequences of one length: packed rows give the dense forward's
    values (same kernel arithmetic, different addressing)."""
    B, H, N, d = 3, 4, 200, 128
    q, k, v = workloads.prefill(B, H, H, N, N, d, seed=5)
    o_d, lse_d = attn.attn_fwd(q.to(gpu), k.to(gpu), v.to(gpu), 1 / math.sqrt(d), True)
    pack = lambda t: t.transpose(1, 2).reshape(B * N, H, d).contiguous().to(gpu)  # noqa: E731
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device=gpu)
    o_p, lse_p = attn.attn_fwd_varlen(pack(q), pack(k), pack(v), cu, cu, N, 1 / math.sqrt(d), -1, 0)
    torch.cuda.synchronize()
    assert torch.equal(o_p.cpu(), o_d.transpose(1, 2).reshape(B * N, H, d).cpu())
    assert torch.equal(lse_p.cpu(), lse_d.transpose(0, 1).reshape(H, B * N).cpu())


def _paged_ref(w, scale, window):
    return oracle.prefill_paged(to64(w["q"]), w["k_cache"].float().numpy(),
                                w["v_cache"].float().numpy(), w["block_table"].numpy(),
                                w["cu_q"].numpy(), w["seqlens_k"].numpy(), scale, False,
                                _band(window))


def _paged(w, gpu, scale, window, table=None, num_blocks=None):
    bt = (w["block_table"] if table is None else table).to(gpu)
    o, lse = attn.attn_prefill_paged(w["q"].to(gpu), w["k_cache"].to(gpu), w["v_cache"].to(gpu),
                                     bt, w["cu_q"].to(gpu), w["seqlens_k"].to(gpu), w["max_q"],
                                     scale, *window, num_blocks=num_blocks)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


PAGED_CASES = [
    # q_lens, k_lens, block_size, window
    ([1, 17, 128, 129, 300], [1, 40, 128, 1000, 300], 16, (-1, 0)),
    ([1, 1, 1, 1], [5, 16, 17, 700], 16, (-1, 0)),          # one row per sequence: decode
    ([200, 64, 0, 31], [200, 600, 50, 31], 32, (-1, 0)),    # 32-token pages, an empty query set
    ([150, 70], [333, 70], 48, (-1, 0)),                    # pages that do not divide the tiles
    ([100, 40], [900, 41], 16, (127, 0)),                   # sliding window of 128 keys
    ([90, 33], [90, 200], 16, (-1, -1)),                    # no mask: queries see later tokens too
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4)])
@pytest.mark.parametrize("case", range(len(PAGED_CASES)))
def test_prefill_paged_parity(gpu, d, Hq, Hkv, case):
    """Permuted block tables; slots past each context and unused blocks hold
    NaN, so any read of them that reaches the result shows up."""
    q_lens, k_lens, bs, window = PAGED_CASES[case]
    w = workloads.paged_prefill(q_lens, k_lens, Hq, Hkv, d, block_size=bs, seed=case + d,
                                poison=True, extra_blocks=3)
    scale = 1.0 / math.sqrt(d)
    o, lse = _paged(w, gpu, scale, window)
    o_ref, lse_ref = _paged_ref(w, scale, window)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_prefill_paged_one_row_matches_decode_kernel(gpu):
    """One query per sequence through the prefill kernel agrees with the
    decode kernel within the bf16 tolerance (two kernels, one definition)."""
    k_lens = [33, 500, 4000, 16]
    w = workloads.paged_prefill([1] * 4, k_lens, 32, 8, 128, seed=3, poison=True)
    scale = 1.0 / math.sqrt(128)
    o, lse = _paged(w, gpu, scale, (-1, 0))
    od, ld = attn.attn_decode_paged(w["q"].to(gpu), w["k_cache"].to(gpu), w["v_cache"].to(gpu),
                                    w["block_table"].to(gpu), w["seqlens_k"].to(gpu), scale,
                                    max(k_lens))
    torch.cuda.synchronize()
    o_ref, lse_ref = _paged_ref(w, scale, (-1, 0))
    check_out(to64(o), o_ref, "bf16", what="O prefill kernel vs oracle")
    check_lse(to64(lse), lse_ref, "bf16", what="LSE prefill kernel vs oracle")
    check_out(to64(od), o_ref, "bf16", what="O decode kernel vs oracle")
    check_lse(to64(ld).T, lse_ref, "bf16", what="LSE decode kernel vs oracle")
    check_out(to64(o), to64(od), "bf16", what="O prefill vs decode kernel")
    check_lse(to64(lse).T, to64(ld), "bf16", what="LSE prefill vs decode kernel")


def test_prefill_paged_invalid_entries_are_skipped(gpu):
    """Live tokens whose table entries lie outside the cache get probability
    0 and are never read; the rest match the oracle with those keys masked."""
    q_lens, k_lens = [40, 100], [70, 300]
    w = workloads.paged_prefill(q_lens, k_lens, 8, 2, 128, seed=21, poison=True)
    bt = w["block_table"].clone()
    bt[0, 1] = w["num_blocks"] + 9    # tokens 16..31 of sequence 0
    bt[1, 5] = -3                     # tokens 80..95 of sequence 1
    scale = 1.0 / math.sqrt(128)
    o, lse = _paged(w, gpu, scale, (-1, 0), table=bt)
    cu = w["cu_q"].tolist()
    for s, drop in [(0, 1), (1, 5)]:
        ctx = k_lens[s]
        kk = oracle.gather_paged(w["k_cache"].float().numpy(), w["block_table"].numpy(), s, ctx)
        vv = oracle.gather_paged(w["v_cache"].float().numpy(), w["block_table"].numpy(), s, ctx)
        keep = (np.arange(ctx) // 16 != drop)[None, None, None, :]
        qs = to64(w["q"][cu[s]:cu[s + 1]]).transpose(1, 0, 2)[None]
        o_ref, lse_ref = oracle.forward(qs, kk.transpose(1, 0, 2)[None].astype(np.float64),
                                        vv.transpose(1, 0, 2)[None].astype(np.float64), scale,
                                        True, mask=keep)
        check_out(to64(o[cu[s]:cu[s + 1]]).transpose(1, 0, 2), o_ref[0], "bf16")
        check_lse(to64(lse[:, cu[s]:cu[s + 1]]), lse_ref[0], "bf16")


def test_prefill_paged_chunks_compose_full_prefill(gpu):
    """A context prefilled in two chunks (the second chunk's queries seeing
    the first chunk's keys in the cache) gives the rows of a one-shot causal
    prefill over the whole context, within the bf16 tolerance."""
    n, split = 700, 300
    w = workloads.paged_prefill([n], [n], 8, 2, 128, seed=22)
    scale = 1.0 / math.sqrt(128)
    o_full, lse_full = _paged(w, gpu, scale, (-1, 0))
    # Chunk 1: the first `split` tokens as a context of their own; chunk 2: the rest.
    w1 = dict(w, q=w["q"][:split], cu_q=torch.tensor([0, split], dtype=torch.int32),
              seqlens_k=torch.tensor([split], dtype=torch.int32), max_q=split)
    w2 = dict(w, q=w["q"][split:].contiguous(), cu_q=torch.tensor([0, n - split], dtype=torch.int32),
              max_q=n - split)
    o1, l1 = _paged(w1, gpu, scale, (-1, 0))
    o2, l2 = _paged(w2, gpu, scale, (-1, 0))
    o_ref, lse_ref = _paged_ref(w, scale, (-1, 0))
    check_out(to64(o_full), o_ref, "bf16", what="O one shot vs oracle")
    check_lse(to64(lse_full), lse_ref, "bf16", what="LSE one shot vs oracle")
    check_out(to64(torch.cat([o1, o2])), o_ref, "bf16", what="O two chunks vs oracle")
    check_lse(to64(torch.cat([l1, l2], dim=1)), lse_ref, "bf16", what="LSE two chunks vs oracle")
    check_out(to64(torch.cat([o1, o2])), to64(o_full), "bf16", what="O two chunks vs one shot")


def test_prefill_paged_serving_shape(gpu):
    """The benchmark's serving-shaped workload (16 sequences, GQA 32/8,
    d = 128, 16-token pages) in the benchmark's launch configuration: every
    query row of every sequence against the oracle, for the first query head
    of the first KV group and the last query head of the last (the oracle
    materialises each sequence's scores one head at a time)."""
    pw = workloads.WORKLOADS["paged_prefill_causal_bf16_s16_hq32_hkv8_d128"]
    num_seqs = pw["num_seqs"]
    w = workloads.serving_prefill(num_seqs, pw["q_lo"], pw["q_hi"], pw["ctx_lo"], pw["ctx_hi"],
                                  pw["Hq"], pw["Hkv"], pw["d"], block_size=pw["block_size"],
                                  seed=pw["seed"], device=str(gpu))
    q_lens, k_lens = w["q_lens"], w["k_lens"]
    scale = pw["scale"]
    o, lse = _paged(w, gpu, scale, (-1, 0))
    o, lse = o.cpu(), lse.cpu()
    cu = w["cu_q"].tolist()
    group = pw["Hq"] // pw["Hkv"]
    kc, vc, bt = w["k_cache"].cpu().float().numpy(), w["v_cache"].cpu().float().numpy(), w["block_table"].numpy()
    qh = w["q"].cpu()
    for s in range(num_seqs):
        kk = oracle.gather_paged(kc, bt, s, k_lens[s]).astype(np.float64)
        vv = oracle.gather_paged(vc, bt, s, k_lens[s]).astype(np.float64)
        for h in (0, pw["Hq"] - 1):
            g = h // group
            # The chunk's rows are the last q positions of the context: bottom-right causal.
            qs = to64(qh[cu[s]:cu[s + 1], h])[None, None]
            o_ref, lse_ref = oracle.forward(qs, kk[:, g][None, None], vv[:, g][None, None],
                                            scale, True)
            check_out(to64(o[cu[s]:cu[s + 1], h]), o_ref[0, 0], "bf16", what=f"O seq {s} head {h}")
            check_lse(to64(lse[h, cu[s]:cu[s + 1]]), lse_ref[0, 0], "bf16",
                      what=f"LSE seq {s} head {h}")


def test_varlen_bench_shape(gpu):
    """The benchmark's packed ragged workload (16 sequences of 512..8192
    tokens, GQA 32/8, d = 128, causal) in the benchmark's launch
    configuration: every row of every sequence against the oracle, for the
    first query head of the first KV group and the last query head of the
    last."""
    vw = workloads.WORKLOADS["varlen_causal_bf16_s16_h32_hkv8_d128"]
    lens = workloads.ragged_lengths(vw["num_seqs"], vw["len_lo"], vw["len_hi"], seed=vw["seed"] + 1)
    w = workloads.ragged(lens, lens, vw["H"], vw["Hkv"], vw["d"], seed=vw["seed"], device=str(gpu))
    o, lse = attn.attn_fwd_varlen(w["q"], w["k"], w["v"], w["cu_q"].to(gpu), w["cu_k"].to(gpu),
                                  w["max_q"], vw["scale"], -1, 0)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    qh, kh, vh = w["q"].cpu(), w["k"].cpu(), w["v"].cpu()
    cu = w["cu_q"].tolist()
    group = vw["H"] // vw["Hkv"]
    for s in range(vw["num_seqs"]):
        for h in (0, vw["H"] - 1):
            g = h // group
            qs = to64(qh[cu[s]:cu[s + 1], h])[None, None]
            kk = to64(kh[cu[s]:cu[s + 1], g])[None, None]
            vv = to64(vh[cu[s]:cu[s + 1], g])[None, None]
            o_ref, lse_ref = oracle.forward(qs, kk, vv, vw["scale"], True)
            check_out(to64(o[cu[s]:cu[s + 1], h]), o_ref[0, 0], "bf16", what=f"O seq {s} head {h}")
            check_lse(to64(lse[h, cu[s]:cu[s + 1]]), lse_ref[0, 0], "bf16",
                      what=f"LSE seq {s} head {h}")


def test_prefill_paged_head_major_layout(gpu):
    """The paged prefill through a head-major cache ([block, head, slot, d])
    given by strides equals the oracle on the token-major original."""
    w = workloads.paged_prefill([30, 140], [300, 140], 8, 2, 128, block_size=32, seed=31,
                                poison=True)
    nb, bs, hkv, d = w["k_cache"].shape
    kh = w["k_cache"].permute(0, 2, 1, 3).contiguous()
    vh = w["v_cache"].permute(0, 2, 1, 3).contiguous()
    o, lse = attn.attn_prefill_paged(w["q"].to(gpu), kh.to(gpu), vh.to(gpu),
                                     w["block_table"].to(gpu), w["cu_q"].to(gpu),
                                     w["seqlens_k"].to(gpu), w["max_q"], 0.09, -1, 0,
                                     strides=(hkv * bs * d, d, bs * d), cache_dims=(nb, bs, hkv))
    torch.cuda.synchronize()
    o_ref, lse_ref = _paged_ref(w, 0.09, (-1, 0))
    check_out(to64(o.cpu()), o_ref, "bf16")
    check_lse(to64(lse.cpu()), lse_ref, "bf16")
