"""Backward parity: HIP recompute backward against the fp64 oracle's gradients."""

import math

import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_grad, to64

pytestmark = pytest.mark.gpu


def _fwd_bwd(gpu, q, k, v, do, scale, causal):
    qg, kg, vg, dog = (t.to(gpu) for t in (q, k, v, do))
    o, lse = attn.attn_fwd(qg, kg, vg, scale, causal)
    dq, dk, dv = attn.attn_bwd(qg, kg, vg, o, dog, lse, scale, causal)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal", [
    (1, 2, 2, 64, 64, 64, True),
    (1, 2, 2, 128, 128, 128, False),
    (2, 2, 2, 200, 200, 128, True),     # ragged query and key tiles
    (1, 1, 1, 1, 1, 64, True),
    (1, 2, 2, 17, 300, 64, True),      # Nq < Nk, bottom-right causal
    (1, 2, 2, 300, 17, 128, False),
    (1, 2, 2, 129, 100, 64, True),     # Nq > Nk: rows that see no key
    (1, 4, 2, 257, 257, 128, True),    # grouped-query heads
    (1, 8, 1, 96, 96, 64, False),
])
def test_bwd_small(gpu, B, H, Hkv, Nq, Nk, d, causal):
    q, k, v, do = workloads.backward(B, H, Hkv, Nq, Nk, d, dtype="bf16", seed=Nq * 7 + Nk)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = _fwd_bwd(gpu, q, k, v, do, scale, causal)
    rq, rk, rv = oracle.backward(to64(q), to64(k), to64(v), to64(do), scale, causal)
    check_grad(to64(dq), rq, "dQ")
    check_grad(to64(dk), rk, "dK")
    check_grad(to64(dv), rv, "dV")


def test_bwd_large_logits(gpu):
    """Queries scaled by 6: dK (linear in Q) reaches |21|, so the bound is
    magnitude-aware (bf16 output rounding alone exceeds 5e-2 there)."""
    q, k, v, do = workloads.backward(1, 2, 2, 300, 300, 128, dtype="bf16", seed=21)
    q = (q.float() * 6.0).to(torch.bfloat16)
    dq, dk, dv = _fwd_bwd(gpu, q, k, v, do, 1 / math.sqrt(128), True)
    rq, rk, rv = oracle.backward(to64(q), to64(k), to64(v), to64(do), 1 / math.sqrt(128), True)
    check_grad(to64(dq), rq, "dQ", magnitude_aware=True)
    check_grad(to64(dk), rk, "dK", magnitude_aware=True)
    check_grad(to64(dv), rv, "dV", magnitude_aware=True)


def test_bwd_deterministic(gpu):
    """No atomics: all three gradients are bitwise reproducible."""
    q, k, v, do = workloads.backward(1, 4, 4, 333, 333, 128, dtype="bf16", seed=22)
    a = _fwd_bwd(gpu, q, k, v, do, 0.09, True)
    b = _fwd_bwd(gpu, q, k, v, do, 0.09, True)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bwd_very_negative_scores_ragged_keys(gpu):
    """Rows whose scores are all very negative (LSE far below 0) with a ragged
    key tile: masked tail keys must not overflow into dQ."""
    q, k, v, do = workloads.backward(1, 2, 2, 70, 70, 64, dtype="bf16", seed=23)
    u = torch.ones(64, dtype=torch.bfloat16)
    q = (q.float() * 0.05 + 3.0 * u.float()).to(torch.bfloat16)
    k = (k.float() * 0.05 - 3.0 * u.float()).to(torch.bfloat16)   # scores near -72 * 8 * scale
    dq, dk, dv = _fwd_bwd(gpu, q, k, v, do, 1.0, False)
    rq, rk, rv = oracle.backward(to64(q), to64(k), to64(v), to64(do), 1.0, False)
    check_grad(to64(dq), rq, "dQ", magnitude_aware=True)
    check_grad(to64(dk), rk, "dK", magnitude_aware=True)
    check_grad(to64(dv), rv, "dV", magnitude_aware=True)


def test_causal_bwd_b2_h16_n4096_d128(gpu):
    """B=2, H=16, N=4096, d=128, causal, scale 1/sqrt(128): full-size launch,
    exactly as the benchmark calls it.  dQ, dK and dV of every (batch, head)
    are compared with the oracle's gradients, one head at a time."""
    B, H, N, d = 2, 16, 4096, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = workloads.backward(B, H, H, N, N, d, dtype="bf16", seed=0)
    dq, dk, dv = _fwd_bwd(gpu, q, k, v, do, scale, True)
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            rq, rk, rv = oracle.backward(to64(q[sl]), to64(k[sl]), to64(v[sl]), to64(do[sl]),
                                         scale, True)
            check_grad(to64(dq[sl]), rq, f"dQ[{b},{h}]")
            check_grad(to64(dk[sl]), rk, f"dK[{b},{h}]")
            check_grad(to64(dv[sl]), rv, f"dV[{b},{h}]")
