"""Local (banded / sliding-window) attention: forward and backward through
attn_fwd_local / attn_bwd_local against the fp64 oracle with the same band."""

import math

import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_grad, check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def _band(left, right):
    """C-ABI window sides (-1 = no limit) as the oracle's (None = no limit)."""
    return (None if left < 0 else left, None if right < 0 else right)


def _fwd(gpu, B, H, Hkv, Nq, Nk, d, left, right, seed):
    q, k, v = workloads.prefill(B, H, Hkv, Nq, Nk, d, dtype="bf16", seed=seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = attn.attn_fwd_local(q.to(gpu), k.to(gpu), v.to(gpu), scale, left, right)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), scale, False, _band(left, right))
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


WINDOWS = [(0, 0), (1, 0), (31, 0), (32, 0), (33, 0), (63, 0), (64, 0), (100, 0), (255, 0),
           (5, 5), (0, 17), (40, 7), (128, 64), (-1, 3), (7, -1)]


@pytest.mark.parametrize("left,right", WINDOWS)
@pytest.mark.parametrize("d", [64, 128])
def test_window_forward(gpu, left, right, d):
    """Bands narrower and wider than a key tile (32 or 64) and a query tile
    (128), on and off tile boundaries, one- and two-sided, ragged N."""
    _fwd(gpu, 1, 2, 1, 333, 333, d, left, right, seed=left * 7 + right + d)


@pytest.mark.parametrize("Nq,Nk,left,right", [
    (100, 300, 50, 0), (300, 100, 20, 0), (1, 500, 63, 0), (257, 257, 300, 2),
    (64, 4, 1, 1)])
def test_window_forward_rectangular(gpu, Nq, Nk, left, right):
    """Bottom-right alignment with Nq != Nk, including rows whose band holds
    no key (O = 0, LSE = -inf)."""
    _fwd(gpu, 1, 2, 2, Nq, Nk, 128, left, right, seed=Nq + Nk)


def test_window_forward_gqa_sliding_4096(gpu):
    """A sliding window of 1024 keys over 4096 positions, grouped-query heads."""
    _fwd(gpu, 1, 4, 2, 4096, 4096, 128, 1023, 0, seed=5)


def test_unbounded_bands_equal_the_plain_entry_point(gpu):
    """(-1, 0) is the causal mask and (-1, -1) no mask: bit-identical results."""
    q, k, v = (t.to(gpu) for t in workloads.prefill(1, 4, 2, 300, 300, 128, dtype="bf16",
                                                    seed=3))
    for causal, (left, right) in [(True, (-1, 0)), (False, (-1, -1))]:
        o1, l1 = attn.attn_fwd(q, k, v, 0.09, causal)
        o2, l2 = attn.attn_fwd_local(q, k, v, 0.09, left, right)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_window_fp32_only_causal_or_none(gpu):
    q = torch.zeros(1, 1, 8, 64, device=gpu)
    with pytest.raises(attn.AttnError):
        attn.attn_fwd_local(q, q, q, 0.1, 3, 0)
    attn.attn_fwd_local(q, q, q, 0.1, -1, 0)
    attn.attn_fwd_local(q, q, q, 0.1, -1, -1)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,left,right", [
    (1, 2, 2, 200, 200, 128, 31, 0),
    (1, 2, 2, 300, 300, 64, 100, 0),
    (1, 4, 2, 257, 257, 128, 64, 64),
    (1, 2, 1, 150, 400, 128, 40, 5),
    (1, 2, 2, 400, 150, 64, 0, 20),
    (2, 2, 2, 513, 513, 128, 200, 0),
])
def test_window_backward(gpu, B, H, Hkv, Nq, Nk, d, left, right):
    q, k, v, do = workloads.backward(B, H, Hkv, Nq, Nk, d, dtype="bf16", seed=Nq + left)
    scale = 1.0 / math.sqrt(d)
    qg, kg, vg, dog = (t.to(gpu) for t in (q, k, v, do))
    o, lse = attn.attn_fwd_local(qg, kg, vg, scale, left, right)
    dq, dk, dv = attn.attn_bwd_local(qg, kg, vg, o, dog, lse, scale, left, right)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(to64(q), to64(k), to64(v), to64(do), scale, False,
                                 _band(left, right))
    check_grad(to64(dq), rq, "dQ")
    check_grad(to64(dk), rk, "dK")
    check_grad(to64(dv), rv, "dV")
