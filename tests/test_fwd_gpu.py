"""Forward parity: HIP kernels (through the C ABI) against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def _run(gpu, B, H, Hkv, Nq, Nk, d, dtype, causal, seed=0, scale=None, q_mult=1.0,
         mutate=None):
    q, k, v = workloads.prefill(B, H, Hkv, Nq, Nk, d, dtype=dtype, seed=seed)
    if q_mult != 1.0:
        q = (q.float() * q_mult).to(q.dtype)
    if mutate is not None:
        q, k, v = mutate(q, k, v)
    scale = scale if scale is not None else 1.0 / math.sqrt(d)
    o, lse = attn.attn_fwd(q.to(gpu), k.to(gpu), v.to(gpu), scale, causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), scale, causal)
    check_out(to64(o), o_ref, dtype)
    check_lse(to64(lse), lse_ref, dtype)
    return o, lse


def test_single_head_f32_n512_d64(gpu):
    """fp32, B=1, H=1, N=512, d=64, scale 1/8, non-causal, seed 0."""
    _run(gpu, 1, 1, 1, 512, 512, 64, "f32", False, seed=0, scale=1.0 / 8.0)


F32_PATHS = [
    # (B, H, Nq, Nk): fewer 128-row tiles than CUs -> key-split kernel
    # (32-row workgroups, four waves over the keys, merged in LDS) ...
    (1, 1, 512, 512), (1, 3, 33, 33), (2, 2, 17, 200), (1, 2, 200, 17), (1, 1, 1, 1),
    (1, 1, 31, 1000),
    # ... otherwise the 128-row kernel.
    (2, 16, 1030, 1030),
]


@pytest.mark.parametrize("B,H,Nq,Nk", F32_PATHS)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_both_kernels(gpu, B, H, Nq, Nk, d, causal):
    """fp32 on both of its kernels (the plan names which one runs), every
    row against the oracle: ragged tiles, fewer key tiles than waves, Nq > Nk
    (rows with no visible key when causal)."""
    plan = attn.attn_plan_describe(attn.ATTN_PHASE_FWD, B, H, H, Nq, Nk, d, causal,
                                   attn.ATTN_DTYPE_F32)
    assert ("keysplit" in plan) == (B * H * -(-Nq // 128) < 256)
    _run(gpu, B, H, H, Nq, Nk, d, "f32", causal, seed=Nq + Nk + d)


def test_causal_bf16_b4_h16_n2048_d64(gpu):
    """bf16 causal prefill, B=4, H=16, N=2048, d=64, scale 1/8 (full oracle)."""
    _run(gpu, 4, 16, 16, 2048, 2048, 64, "bf16", True, seed=0, scale=1.0 / 8.0)


BOUNDARY_N = [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 257, 1000]


@pytest.mark.parametrize("N", BOUNDARY_N)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_boundary_sweep(gpu, N, d, causal, dtype):
    """Every tile/ragged boundary around the 32/64/128 tile sizes."""
    _run(gpu, 1, 2, 1, N, N, d, dtype, causal, seed=N)


@pytest.mark.parametrize("Nq,Nk", [(1, 300), (17, 200), (130, 129), (200, 17), (64, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_rectangular(gpu, Nq, Nk, causal):
    """Nq != Nk; causal is bottom-right aligned, Nq > Nk leaves empty rows."""
    _run(gpu, 2, 2, 2, Nq, Nk, 128, "bf16", causal, seed=Nq + Nk)


@pytest.mark.parametrize("H,Hkv", [(8, 2), (6, 3), (4, 1)])
def test_gqa_mapping(gpu, H, Hkv):
    _run(gpu, 2, H, Hkv, 300, 300, 64, "bf16", True, seed=H)


@pytest.mark.parametrize("mult", [8.0, 30.0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_logit_range(gpu, mult, dtype):
    """Long rows with large logit ranges (queries scaled up)."""
    _run(gpu, 1, 2, 2, 700, 700, 128, dtype, True, seed=3, q_mult=mult)


@pytest.mark.parametrize("causal", [False, True])
def test_adversarial_late_maximum(gpu, causal):
    """The row maximum arrives in the last key tile: the accumulator must be
    rescaled ("Modern attention kernels", "Failure modes")."""
    def mutate(q, k, v):
        k = k.clone()
        # Last key aligned with every query direction, large enough to dominate.
        k[:, :, -1] = (q[:, :, -1].float() * 6.0).to(k.dtype)
        return q, k, v
    _run(gpu, 1, 2, 2, 513, 513, 128, "bf16", causal, seed=11, mutate=mutate)


def test_deterministic(gpu):
    q, k, v = workloads.prefill(1, 4, 2, 777, 777, 128, dtype="bf16", seed=5)
    q, k, v = q.to(gpu), k.to(gpu), v.to(gpu)
    o1, l1 = attn.attn_fwd(q, k, v, 0.1, True)
    o2, l2 = attn.attn_fwd(q, k, v, 0.1, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _compare_heads(q, k, v, o, lse, scale, causal):
    """Every row of every (batch, head) against the oracle, one head at a time
    (the oracle materialises one head's N x N scores and probabilities)."""
    group = q.shape[1] // k.shape[1]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            g = h // group
            sl = (slice(b, b + 1), slice(h, h + 1))
            o_ref, lse_ref = oracle.forward(to64(q[sl]), to64(k[b:b + 1, g:g + 1]),
                                            to64(v[b:b + 1, g:g + 1]), scale, causal)
            check_out(to64(o[sl]), o_ref, "bf16", what=f"O[{b},{h}]")
            check_lse(to64(lse[sl]), lse_ref, "bf16", what=f"LSE[{b},{h}]")


@pytest.mark.parametrize("H,causal", [(32, True), (32, False), (4, True)])
def test_long_prefill_n8192_d128_full(gpu, H, causal):
    """B=1, N=8192, d=128, scale 1/sqrt(128): H=32 causal and non-causal, and
    H=4 causal (a small grid: the binding takes the key-split path).
    Full-size launch, exactly as the benchmark calls it; every row of every
    head is compared with the oracle (O to the bf16 bounds, LSE to 1e-3)."""
    N, d = 8192, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v = workloads.prefill(1, H, H, N, N, d, dtype="bf16", seed=0)
    qg, kg, vg = q.to(gpu), k.to(gpu), v.to(gpu)
    o, lse = attn.attn_fwd(qg, kg, vg, scale, causal)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    _compare_heads(q, k, v, o, lse, scale, causal)
    # Row 0 under causal sees only key 0: O = V[0] exactly (bf16 in, bf16 out).
    if causal:
        assert torch.equal(o[0, :, 0], v[0, :, 0])


# Wide grids (hundreds of heads) with ragged, rectangular, windowed and
# grouped-query shapes: every workgroup slot of the chip in use at once.
WIDE_CASES = [
    # B, H, Hkv, Nq, Nk, window (left, right) or None for no mask
    (1, 256, 256, 300, 300, (-1, 0)),
    (1, 256, 64, 257, 257, None),
    (2, 128, 32, 200, 900, (-1, 0)),     # Nq < Nk, bottom-right causal
    (1, 256, 256, 900, 200, (-1, 0)),    # Nq > Nk: early rows see no key
    (1, 256, 128, 513, 513, (63, 0)),    # sliding window of 64 keys
    (1, 256, 256, 300, 300, (40, 17)),   # two-sided band
    (1, 256, 256, 1, 64, (-1, 0)),       # one query row per head
]


@pytest.mark.parametrize("case", range(len(WIDE_CASES)))
@pytest.mark.parametrize("d", [64, 128])
def test_wide_grid_edges(gpu, case, d):
    B, H, Hkv, Nq, Nk, window = WIDE_CASES[case]
    q, k, v = workloads.prefill(B, H, Hkv, Nq, Nk, d, dtype="bf16", seed=case * 7 + d)
    scale = 1.0 / math.sqrt(d)
    qg, kg, vg = q.to(gpu), k.to(gpu), v.to(gpu)
    if window is None:
        o, lse = attn.attn_fwd(qg, kg, vg, scale, False)
        band = None
    elif window == (-1, 0):
        o, lse = attn.attn_fwd(qg, kg, vg, scale, True)
        band = None
    else:
        o, lse = attn.attn_fwd_local(qg, kg, vg, scale, *window)
        band = (window[0], window[1])
    torch.cuda.synchronize()
    causal = window == (-1, 0)
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), scale, causal, band)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")
