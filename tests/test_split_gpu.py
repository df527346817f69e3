"""Forward with a split key range (attn_fwd_splitkv): partials per key chunk,
merged by max-rescaling, against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def _band(left, right):
    return (None if left < 0 else left, None if right < 0 else right)


@pytest.mark.parametrize("chunk", [64, 128, 192, 256, 1024])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("left,right", [(-1, 0), (-1, -1), (100, 0), (40, 7)])
def test_forced_chunks(gpu, chunk, d, left, right):
    """Chunks of 1..32 key tiles, on and off the band's edges; ragged N."""
    N = 1000 if chunk >= 256 else 333
    q, k, v = workloads.prefill(1, 2, 1, N, N, d, dtype="bf16", seed=chunk + d)
    scale = 1.0 / math.sqrt(d)
    assert attn.attn_fwd_splitkv_workspace_size(1, 2, N, N, d, left, right, chunk) > 0
    o, lse = attn.attn_fwd_splitkv(q.to(gpu), k.to(gpu), v.to(gpu), scale, left, right,
                                   chunk_keys=chunk)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), scale, False, _band(left, right))
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


@pytest.mark.parametrize("Nq,Nk", [(100, 700), (700, 100), (1, 900)])
def test_forced_chunks_rectangular(gpu, Nq, Nk):
    """Bottom-right causal with Nq != Nk: query tiles whose key range is
    empty or shorter than a chunk, rows that see no key."""
    q, k, v = workloads.prefill(1, 2, 2, Nq, Nk, 128, dtype="bf16", seed=Nq)
    o, lse = attn.attn_fwd_splitkv(q.to(gpu), k.to(gpu), v.to(gpu), 0.088, -1, 0, chunk_keys=128)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), 0.088, True)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_planner_leaves_large_grids_unsplit(gpu):
    """32 heads x 64 query tiles fill the chip: the size query asks for no
    workspace.  A small grid through both entry points matches the oracle."""
    assert attn.attn_fwd_splitkv_workspace_size(1, 32, 8192, 8192, 128, -1, 0, 0) == 0
    qc, kc, vc = workloads.prefill(1, 4, 4, 256, 256, 128, dtype="bf16", seed=2)
    q, k, v = qc.to(gpu), kc.to(gpu), vc.to(gpu)
    o1, l1 = attn.attn_fwd(q, k, v, 0.1, True)
    o2, l2 = attn.attn_fwd_splitkv(q, k, v, 0.1, -1, 0)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(qc), to64(kc), to64(vc), 0.1, True)
    check_out(to64(o1), o_ref, "bf16", what="O attn_fwd")
    check_lse(to64(l1), lse_ref, "bf16", what="LSE attn_fwd")
    check_out(to64(o2), o_ref, "bf16", what="O attn_fwd_splitkv")
    check_lse(to64(l2), lse_ref, "bf16", what="LSE attn_fwd_splitkv")


def test_causal_bf16_b1_h4_n8192_d128_split(gpu):
    """The four-head 8192-token causal workload through attn_fwd_splitkv with
    the planner's split: every row of every head against the oracle."""
    B, H, N, d = 1, 4, 8192, 128
    assert attn.attn_fwd_splitkv_workspace_size(B, H, N, N, d, -1, 0, 0) > 0
    q, k, v = workloads.prefill(B, H, H, N, N, d, dtype="bf16", seed=0, device=str(gpu))
    scale = 1.0 / math.sqrt(d)
    o, lse = attn.attn_fwd_splitkv(q, k, v, scale, -1, 0)
    torch.cuda.synchronize()
    q, k, v, o, lse = q.cpu(), k.cpu(), v.cpu(), o.cpu(), lse.cpu()
    for h in range(H):
        sl = (slice(0, 1), slice(h, h + 1))
        o_ref, lse_ref = oracle.forward(to64(q[sl]), to64(k[sl]), to64(v[sl]), scale, True)
        check_out(to64(o[sl]), o_ref, "bf16", what=f"O head {h}")
        check_lse(to64(lse[sl]), lse_ref, "bf16", what=f"LSE head {h}")


@pytest.mark.parametrize("fill", [0x00, 0xFF])
def test_workspace_reuse_repeatable(gpu, fill):
    """A workspace holding any bytes, reused by calls of other sizes and part
    sizes, gives the oracle's result, and repeated calls are bit-identical
    (each tile's partials merge in part order)."""
    ws = torch.full((attn.attn_fwd_splitkv_workspace_size(1, 3, 1000, 1000, 128, -1, 0, 128),),
                    fill, dtype=torch.uint8, device=gpu)
    for N, chunk in ((1000, 1024), (777, 128), (1000, 128)):
        assert ws.numel() >= attn.attn_fwd_splitkv_workspace_size(1, 3, N, N, 128, -1, 0, chunk)
        q, k, v = workloads.prefill(1, 3, 1, N, N, 128, dtype="bf16", seed=N + chunk + fill)
        qg, kg, vg = q.to(gpu), k.to(gpu), v.to(gpu)
        o1, l1 = attn.attn_fwd_splitkv(qg, kg, vg, 0.09, -1, 0, chunk_keys=chunk, workspace=ws)
        o2, l2 = attn.attn_fwd_splitkv(qg, kg, vg, 0.09, -1, 0, chunk_keys=chunk, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"N={N}: repeated calls differ"
        o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), 0.09, True)
        check_out(to64(o1), o_ref, "bf16", what=f"O N={N} chunk={chunk}")
        check_lse(to64(l1), lse_ref, "bf16", what=f"LSE N={N} chunk={chunk}")


def test_planner_split_d64(gpu):
    """The planner's split at d = 64 (64-key tiles; 4 heads x 4096 causal:
    parts of 640 keys, 476 units): every row against the oracle."""
    B, H, N, d = 1, 4, 4096, 64
    assert attn.attn_fwd_splitkv_workspace_size(B, H, N, N, d, -1, 0, 0) > 0
    q, k, v = workloads.prefill(B, H, H, N, N, d, dtype="bf16", seed=5, device=str(gpu))
    o, lse = attn.attn_fwd_splitkv(q, k, v, 0.125, -1, 0)
    torch.cuda.synchronize()
    q, k, v, o, lse = q.cpu(), k.cpu(), v.cpu(), o.cpu(), lse.cpu()
    for h in range(H):
        sl = (slice(0, 1), slice(h, h + 1))
        o_ref, lse_ref = oracle.forward(to64(q[sl]), to64(k[sl]), to64(v[sl]), 0.125, True)
        check_out(to64(o[sl]), o_ref, "bf16", what=f"O head {h}")
        check_lse(to64(lse[sl]), lse_ref, "bf16", what=f"LSE head {h}")


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,left,right", [
    (1, 2, 1, 3000, 3000, 128, -1, 0),      # ragged causal, planner parts
    (2, 3, 3, 1500, 1500, 64, -1, -1),      # no mask, d = 64
    (1, 8, 2, 512, 6000, 128, -1, 0),       # a query chunk against a longer context, GQA
    (1, 4, 4, 2500, 2500, 128, 700, 0),     # local window
])
def test_planner_split_shapes(gpu, B, H, Hkv, Nq, Nk, d, left, right):
    """Shapes whose query tiles leave CUs idle, through the planner's part
    size (chunk_keys = 0): every row against the oracle."""
    assert attn.attn_fwd_splitkv_workspace_size(B, H, Nq, Nk, d, left, right, 0) > 0
    q, k, v = workloads.prefill(B, H, Hkv, Nq, Nk, d, dtype="bf16", seed=Nq + Nk + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = attn.attn_fwd_splitkv(q.to(gpu), k.to(gpu), v.to(gpu), scale, left, right)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), scale, False, _band(left, right))
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_forced_chunks_many_rounds(gpu):
    """128-key parts over 16 causal heads of 2048 keys: 2176 units, about
    three times the workgroups the GPU holds at once, so later units run in
    later rounds; every row against the oracle."""
    B, H, N, d = 1, 16, 2048, 128
    q, k, v = workloads.prefill(B, H, 4, N, N, d, dtype="bf16", seed=21)
    o, lse = attn.attn_fwd_splitkv(q.to(gpu), k.to(gpu), v.to(gpu), 0.09, -1, 0, chunk_keys=128)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), 0.09, True)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_partials_within_their_bound(gpu, d):
    """Each key-split partial is o / l rounded to bf16 once.  Rounding is at
    most 2^-9 relative, and a partial's values are weighted means of V rows, so
    the split output differs from the exact result by at most one rounding of
    P, one of the partial and one of O: 3 * 2^-9 * max|V|; from the unsplit
    kernel (its own P and O roundings) by at most 5 * 2^-9 * max|V|.  V is
    scaled by 64 (|V| up to ~2^8) and the parts are 64 keys long (up to 16
    per query tile)."""
    N = 1000
    q, k, v = workloads.prefill(1, 2, 2, N, N, d, dtype="bf16", seed=70 + d)
    v = (v.float() * 64).to(torch.bfloat16)  # exact: a power-of-two scale
    scale = 1.0 / math.sqrt(d)
    qg, kg, vg = q.to(gpu), k.to(gpu), v.to(gpu)
    o_s, lse_s = attn.attn_fwd_splitkv(qg, kg, vg, scale, -1, 0, chunk_keys=64)
    o_u, _ = attn.attn_fwd(qg, kg, vg, scale, True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), scale, True)
    vmax = float(v.float().abs().max())
    err_ref = float(np.abs(to64(o_s) - o_ref).max())
    err_unsplit = float(np.abs(to64(o_s) - to64(o_u)).max())
    print(f"max|V| {vmax:.1f}: split vs oracle {err_ref:.3g} (bound {3 * 2**-9 * vmax:.3g}), "
          f"vs unsplit {err_unsplit:.3g} (bound {5 * 2**-9 * vmax:.3g})")
    assert err_ref <= 3 * 2**-9 * vmax
    assert err_unsplit <= 5 * 2**-9 * vmax
    check_lse(to64(lse_s), lse_ref, "bf16")
