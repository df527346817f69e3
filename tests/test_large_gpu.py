"""Maximum sizes: tensors and caches past 2^31 elements and 2^32 bytes.

The kernels address one head (or one page) with 32-bit byte offsets from a
64-bit base; these tests place heads, pages and output rows beyond the first
4 GiB of their buffers and check them against the fp64 oracle, so a base or an
offset computed in 32 bits anywhere on the path shows up as a wrong row.
Inputs are made on the device by the seeded generators (a few GiB each); the
oracle gets copies of the sampled heads or the used pages only.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_grad, check_lse, check_out, to64

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def test_fwd_bwd_tensors_past_4gib(gpu):
    """B=144, H=64, N=2048, d=128, causal bf16: Q, K, V, O, dO, dQ, dK, dV are
    4.5 GiB each (2.4e9 elements).  Whole heads before and after the 4 GiB
    mark against the oracle (forward O and LSE, then the three gradients);
    on every head the invariants sum_j dV_j = sum_i dO_i and sum_j dK_j = 0."""
    B, H, N, d = 144, 64, 2048, 128
    head_bytes = N * d * 2
    assert B * H * head_bytes > GIB4 and B * H * N * d > 2 ** 31
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = workloads.backward(B, H, H, N, N, d, dtype="bf16", seed=11, device=str(gpu))
    o, lse = attn.attn_fwd(q, k, v, scale, True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse).all())
    heads = [(0, 0), (70, 3), (130, 7), (B - 1, H - 1)]
    assert any((b * H + h) * head_bytes >= GIB4 for b, h in heads)
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        qs, ks, vs = to64(q[sl]), to64(k[sl]), to64(v[sl])
        o_ref, lse_ref = oracle.forward(qs, ks, vs, scale, True)
        check_out(to64(o[sl]), o_ref, "bf16", what=f"O[{b},{h}]")
        check_lse(to64(lse[sl]), lse_ref, "bf16")

    dq, dk, dv = attn.attn_bwd(q, k, v, o, do, lse, scale, True)
    torch.cuda.synchronize()
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.backward(to64(q[sl]), to64(k[sl]), to64(v[sl]), to64(do[sl]),
                                     scale, True)
        check_grad(to64(dq[sl]), rq, f"dQ[{b},{h}]")
        check_grad(to64(dk[sl]), rk, f"dK[{b},{h}]")
        check_grad(to64(dv[sl]), rv, f"dV[{b},{h}]")
    # Invariants on every head, reduced on the device in fp32.
    sdv = dv.sum(dim=2, dtype=torch.float32)
    sdo = do.sum(dim=2, dtype=torch.float32)
    assert (sdv - sdo).abs().max().item() <= 0.5
    assert dk.sum(dim=2, dtype=torch.float32).abs().max().item() <= 0.5
    assert bool(torch.isfinite(dq).all())


def _compact_cache(cache, table, used_pages):
    """The used pages of a paged cache, renumbered 0..n-1, and the table that
    addresses them (entries of unused slots stay -1)."""
    pages = torch.as_tensor(sorted(used_pages), dtype=torch.long)
    remap = {int(p): i for i, p in enumerate(pages.tolist())}
    small = cache[pages.to(cache.device)].float().cpu().numpy()
    t = table.clone()
    for (s, j), p in np.ndenumerate(table.numpy()):
        if p >= 0:
            t[s, j] = remap[int(p)]
    return small, t


def test_decode_cache_past_4gib(gpu):
    """8 sequences, Hq=32, Hkv=8, d=128, contexts uniform in [4096, 32768],
    16-token pages drawn at random from a K cache and a V cache with 180,000
    pages more than the sequences use (about 5.8 GiB each, 3.1e9 elements):
    most pages sit past 4 GiB.  Every sequence against the oracle."""
    w = workloads.decode(num_seqs=8, Hq=32, Hkv=8, d=128, ctx_lo=4096, ctx_hi=32768,
                         block_size=16, dtype="bf16", seed=12, device=str(gpu),
                         poison_tail=True, extra_blocks=180_000)
    page_bytes = 16 * 8 * 128 * 2
    bt = w["block_table"]
    assert w["num_blocks"] * page_bytes > GIB4 and int(bt.max()) * page_bytes > GIB4
    scale = 1.0 / math.sqrt(128)
    o, lse = attn.attn_decode_paged(w["q"], w["k_cache"], w["v_cache"], bt.to(gpu),
                                    w["context_lens"].to(gpu), scale, w["max_context"])
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for s in range(8):
        ctx = int(w["context_lens"][s])
        pages = bt[s, : (ctx + 15) // 16].long().to(gpu)
        kk = w["k_cache"][pages].reshape(-1, 8, 128)[:ctx].cpu()
        vv = w["v_cache"][pages].reshape(-1, 8, 128)[:ctx].cpu()
        o_ref, lse_ref = oracle.forward(to64(w["q"][s].cpu())[None, :, None, :],
                                        to64(kk).transpose(1, 0, 2)[None],
                                        to64(vv).transpose(1, 0, 2)[None], scale, False)
        check_out(to64(o[s]), o_ref[0, :, 0], "bf16", what=f"seq {s}")
        check_lse(to64(lse[s]), lse_ref[0, :, 0], "bf16")


def test_prefill_paged_cache_past_4gib(gpu):
    """Chunked prefill (Hq=32, Hkv=8, d=128, 16-token pages) over caches of
    170,000 pages (5.2 GiB each): chunks of 300, 129 and 1 new tokens after
    contexts of 5000, 2000 and 20000 tokens, pages at random over the cache,
    unused pages and tail slots NaN.  All rows against the oracle's paged
    prefill on the used pages renumbered."""
    q_lens, k_lens = [300, 129, 1], [5000, 2000, 20000]
    used = sum((c + 15) // 16 for c in k_lens)
    w = workloads.paged_prefill(q_lens, k_lens, 32, 8, 128, block_size=16, seed=13,
                                device=str(gpu), poison=True, extra_blocks=170_000 - used)
    page_bytes = 16 * 8 * 128 * 2
    bt = w["block_table"]
    assert w["num_blocks"] * page_bytes > GIB4 and int(bt.max()) * page_bytes > GIB4
    scale = 1.0 / math.sqrt(128)
    o, lse = attn.attn_prefill_paged(w["q"], w["k_cache"], w["v_cache"], bt.to(gpu),
                                     w["cu_q"].to(gpu), w["seqlens_k"].to(gpu), w["max_q"],
                                     scale, -1, 0)
    torch.cuda.synchronize()
    live = set(int(p) for p in bt.flatten().tolist() if p >= 0)
    kc, t = _compact_cache(w["k_cache"], bt, live)
    vc, _ = _compact_cache(w["v_cache"], bt, live)
    o_ref, lse_ref = oracle.prefill_paged(to64(w["q"].cpu()), kc, vc, t.numpy(),
                                          w["cu_q"].numpy(), w["seqlens_k"].numpy(), scale,
                                          True, None)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")
