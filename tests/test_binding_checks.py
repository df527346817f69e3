"""The Python binding rejects mis-shaped calls before anything reaches the C ABI.

The C ABI sees only pointers, so a tensor shorter than the sizes passed with
it would be read or written past its end.  The binding checks every extent,
dtype and row count the kernels rely on and raises ValueError / TypeError
first.  These tests use CPU tensors: every case must fail on a shape or dtype
check, which runs before the device check (a correctly shaped CPU call would
fail on "tensors must live on the GPU" instead, which the match= strings tell
apart).  No kernel can be launched from here.
"""

import pytest
import torch

from exact_tiled_attention_04_amd import attn

bf = torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def lib():
    return attn.load_library()


def _decode_args(num_seqs=3, Hq=8, Hkv=2, d=64, nb=10, bs=16, max_blocks=4):
    return dict(
        q=torch.zeros(num_seqs, Hq, d, dtype=bf),
        k_cache=torch.zeros(nb, bs, Hkv, d, dtype=bf),
        v_cache=torch.zeros(nb, bs, Hkv, d, dtype=bf),
        block_table=torch.zeros(num_seqs, max_blocks, dtype=torch.int32),
        context_lens=torch.ones(num_seqs, dtype=torch.int32),
        scale=0.125, max_context=64)


def _decode(**over):
    a = _decode_args()
    a.update(over)
    return attn.attn_decode_paged(**a)


def test_decode_well_formed_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        _decode()


@pytest.mark.parametrize("over,exc,match", [
    (dict(block_table=torch.zeros(2, 4, dtype=torch.int32)), ValueError, "block_table has 2 rows"),
    (dict(context_lens=torch.ones(4, dtype=torch.int32)), ValueError, "context_lens has 4"),
    (dict(v_cache=torch.zeros(9, 16, 2, 64, dtype=bf)), ValueError, "same shape"),
    (dict(k_cache=torch.zeros(10, 16, 2, 128, dtype=bf),
          v_cache=torch.zeros(10, 16, 2, 128, dtype=bf)), ValueError, "rows hold 128"),
    (dict(k_cache=torch.zeros(10, 16, 2, 64, dtype=torch.float32),
          v_cache=torch.zeros(10, 16, 2, 64, dtype=torch.float32)), TypeError, "share a dtype"),
    (dict(v_cache=torch.zeros(10, 16, 2, 64, dtype=torch.float32)), TypeError, "share a dtype"),
    (dict(out=torch.zeros(3, 8, 32, dtype=bf)), ValueError, "out must have shape"),
    (dict(out=torch.zeros(3, 8, 64, dtype=torch.float32)), TypeError, "out must be"),
    (dict(lse=torch.zeros(3, 4)), ValueError, "lse must have shape"),
    (dict(block_table=torch.zeros(3, 4, dtype=torch.int64)), TypeError, "int32"),
    (dict(workspace=torch.zeros(8, dtype=torch.uint8)), ValueError, "workspace holds 8 bytes"),
    (dict(strides=(16 * 2 * 64, 2 * 64, 64 * 4)), ValueError, "past the"),
    (dict(cache_dims=(11, 16, 2)), ValueError, "past the"),
])
def test_decode_rejects(over, exc, match):
    with pytest.raises(exc, match=match):
        _decode(**over)


def _fwd(**over):
    a = dict(q=torch.zeros(1, 4, 33, 64, dtype=bf), k=torch.zeros(1, 2, 40, 64, dtype=bf),
             v=torch.zeros(1, 2, 40, 64, dtype=bf), scale=0.1, causal=True)
    a.update(over)
    return attn.attn_fwd(**a)


def test_fwd_well_formed_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        _fwd()


@pytest.mark.parametrize("over,exc,match", [
    (dict(v=torch.zeros(1, 2, 39, 64, dtype=bf)), ValueError, "k and v"),
    (dict(k=torch.zeros(1, 2, 40, 128, dtype=bf)), ValueError, "k and v"),
    (dict(v=torch.zeros(1, 2, 40, 64)), TypeError, "share a dtype"),
    (dict(out=torch.zeros(1, 4, 32, 64, dtype=bf)), ValueError, "out must have shape"),
    (dict(lse=torch.zeros(1, 4, 32)), ValueError, "lse must have shape"),
    (dict(lse=torch.zeros(1, 4, 33, dtype=torch.float64)), TypeError, "lse must be"),
    (dict(q=torch.zeros(4, 33, 64, dtype=bf)), ValueError, "4 dimensions"),
])
def test_fwd_rejects(over, exc, match):
    with pytest.raises(exc, match=match):
        _fwd(**over)


def _bwd(**over):
    B, H, Hkv, N, d = 1, 4, 2, 33, 64
    a = dict(q=torch.zeros(B, H, N, d, dtype=bf), k=torch.zeros(B, Hkv, N, d, dtype=bf),
             v=torch.zeros(B, Hkv, N, d, dtype=bf), o=torch.zeros(B, H, N, d, dtype=bf),
             do=torch.zeros(B, H, N, d, dtype=bf), lse=torch.zeros(B, H, N), scale=0.1,
             causal=True)
    a.update(over)
    return attn.attn_bwd(**a)


def test_bwd_well_formed_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        _bwd()


@pytest.mark.parametrize("over,exc,match", [
    (dict(o=torch.zeros(1, 4, 32, 64, dtype=bf)), ValueError, "o must have shape"),
    (dict(do=torch.zeros(1, 4, 33, 64)), TypeError, "do must be"),
    (dict(lse=torch.zeros(1, 4, 34)), ValueError, "lse must have shape"),
    (dict(dq=torch.zeros(1, 4, 33, 32, dtype=bf)), ValueError, "dq must have shape"),
    (dict(dk=torch.zeros(1, 4, 33, 64, dtype=bf)), ValueError, "dk must have shape"),
    (dict(dv=torch.zeros(1, 2, 33, 64)), TypeError, "dv must be"),
    (dict(workspace=torch.zeros(4, dtype=torch.uint8)), ValueError, "workspace holds"),
])
def test_bwd_rejects(over, exc, match):
    with pytest.raises(exc, match=match):
        _bwd(**over)


def test_varlen_rejects_short_outputs():
    q = torch.zeros(50, 4, 64, dtype=bf)
    k = torch.zeros(60, 2, 64, dtype=bf)
    cu = torch.tensor([0, 20, 50], dtype=torch.int32)
    cuk = torch.tensor([0, 30, 60], dtype=torch.int32)
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.attn_fwd_varlen(q, k, k.clone(), cu, cuk, 30, 0.1, lse=torch.zeros(50, 4))
    with pytest.raises(TypeError, match="share a dtype"):
        attn.attn_fwd_varlen(q, k, k.float(), cu, cuk, 30, 0.1)
    with pytest.raises(ValueError, match="GPU"):
        attn.attn_fwd_varlen(q, k, k.clone(), cu, cuk, 30, 0.1)


def test_prefill_paged_rejects():
    q = torch.zeros(20, 8, 64, dtype=bf)
    kc = torch.zeros(10, 16, 2, 64, dtype=bf)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    cu = torch.tensor([0, 5, 20], dtype=torch.int32)
    lens = torch.tensor([30, 40], dtype=torch.int32)
    with pytest.raises(ValueError, match="num_blocks 11 exceeds"):
        attn.attn_prefill_paged(q, kc, kc.clone(), bt, cu, lens, 15, 0.1, num_blocks=11)
    with pytest.raises(ValueError, match="same shape"):
        attn.attn_prefill_paged(q, kc, kc[:9].clone(), bt, cu, lens, 15, 0.1)
    with pytest.raises(ValueError, match="out must have shape"):
        attn.attn_prefill_paged(q, kc, kc.clone(), bt, cu, lens, 15, 0.1,
                                out=torch.zeros(19, 8, 64, dtype=bf))
    with pytest.raises(ValueError, match="GPU"):
        attn.attn_prefill_paged(q, kc, kc.clone(), bt, cu, lens, 15, 0.1)
