"""C-ABI boundary checks that need no GPU.

Every call here fails host-side validation (or is a pure host query), so no
kernel is ever launched: the fake pointers below are never dereferenced.
As a safety net the fake-pointer tests skip themselves where a GPU is
visible: a case that passed validation by mistake would launch a kernel on
pointers that do not exist.
"""

import ctypes
import os
import re

import pytest

from exact_tiled_attention_04_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)
NULL = ctypes.c_void_p(0)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return attn.load_library()


@pytest.fixture()
def cpu_only():
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-pointer validation tests run only where no GPU is visible")


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(attn.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in [(0, "ATTN_OK"), (1, "ATTN_ERR_INVALID_ARG"), (2, "ATTN_ERR_UNSUPPORTED"),
                       (3, "ATTN_ERR_WORKSPACE"), (4, "ATTN_ERR_HIP")]:
        assert attn.attn_status_string(code) == name


def _fwd(lib, q=FAKE, o=FAKE, lse=FAKE, B=1, H=2, Hkv=1, Nq=8, Nk=8, d=64, scale=0.125,
         causal=1, dtype=attn.ATTN_DTYPE_BF16):
    return lib.attn_fwd(q, FAKE, FAKE, o, lse, B, H, Hkv, Nq, Nk, d, scale, causal, dtype, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(lse=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(o=MISALIGNED), attn.ATTN_ERR_INVALID_ARG),
    (dict(B=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Nq=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Nk=-3), attn.ATTN_ERR_INVALID_ARG),
    (dict(H=3, Hkv=2), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=256), attn.ATTN_ERR_UNSUPPORTED),
    (dict(scale=0.0), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=-1.0), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), attn.ATTN_ERR_INVALID_ARG),
    (dict(dtype=7), attn.ATTN_ERR_INVALID_ARG),
])
def test_fwd_validation(lib, cpu_only, kw, status):
    assert _fwd(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def _decode(lib, q=FAKE, ws=FAKE, ws_bytes=1 << 30, num_seqs=2, Hq=8, Hkv=2, d=128,
            block_size=16, num_blocks=10, max_blocks=4, max_context=64, strides=None,
            scale=0.1, dtype=attn.ATTN_DTYPE_BF16, chunk=0, lse=FAKE):
    if strides is None:
        strides = (block_size * Hkv * d, Hkv * d, d)
    return lib.attn_decode_paged(q, FAKE, FAKE, FAKE, FAKE, FAKE, lse, num_seqs, Hq, Hkv, d,
                                 block_size, num_blocks, max_blocks, max_context, strides[0],
                                 strides[1], strides[2], scale, dtype, chunk, ws, ws_bytes, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(num_seqs=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=80), attn.ATTN_ERR_UNSUPPORTED),
    (dict(max_context=65), attn.ATTN_ERR_INVALID_ARG),  # beyond 4 blocks x 16
    (dict(chunk=48), attn.ATTN_ERR_INVALID_ARG),
    (dict(chunk=4096), attn.ATTN_ERR_INVALID_ARG),      # above the 4064-token chunk limit
    (dict(strides=(16 * 2 * 128, 128, 128)), attn.ATTN_ERR_INVALID_ARG),   # token stride < Hkv*d
    (dict(strides=(2 * 128, 2 * 128, 128)), attn.ATTN_ERR_INVALID_ARG),    # block stride too small
    (dict(strides=(16 * 2 * 132, 2 * 132, 130)), attn.ATTN_ERR_INVALID_ARG),  # unaligned head stride
    (dict(dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ws=NULL), attn.ATTN_ERR_WORKSPACE),
    (dict(ws_bytes=16), attn.ATTN_ERR_WORKSPACE),
    (dict(scale=float("inf")), attn.ATTN_ERR_INVALID_ARG),
])
def test_decode_validation(lib, cpu_only, kw, status):
    assert _decode(lib, **kw) == status


def _decode_noalloc(lib, q=FAKE, num_seqs=2, Hq=8, Hkv=2, d=128, max_context=64, max_blocks=4,
                    chunk=0):
    strides = (16 * Hkv * d, Hkv * d, d)
    return lib.attn_decode_paged_noalloc(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, num_seqs, Hq, Hkv,
                                         d, 16, 10, max_blocks, max_context, strides[0],
                                         strides[1], strides[2], 0.1, attn.ATTN_DTYPE_BF16, chunk,
                                         NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=80), attn.ATTN_ERR_UNSUPPORTED),
    (dict(chunk=48), attn.ATTN_ERR_INVALID_ARG),
    # 4096 sequences x 8 KV heads: partials of 33,792 segments x 4 heads x
    # 130 floats, past the 16 MiB scratch.
    (dict(num_seqs=4096, Hq=32, Hkv=8, max_blocks=2048, max_context=32768),
     attn.ATTN_ERR_WORKSPACE),
])
def test_decode_noalloc_validation(lib, cpu_only, kw, status):
    """The no-allocation decode validates like attn_decode_paged and refuses
    sizes whose partials exceed its static scratch, before any device call."""
    assert _decode_noalloc(lib, **kw) == status


def test_decode_noalloc_capacity(lib):
    cap = attn.attn_decode_paged_noalloc_max_bytes()
    assert cap == 16 << 20
    # The benchmark batch (64 sequences, Hq = 32, Hkv = 8, d = 128, contexts
    # up to 32768 tokens) fits: 1024 split waves + 512 pairs, 4 heads each.
    need = (1024 + 512) * 4 * (128 + 2) * 4 + 512 * 2 * 4
    assert need <= cap


def _bwd(lib, ws=FAKE, ws_bytes=1 << 30, dtype=attn.ATTN_DTYPE_BF16, d=128, dq=FAKE, H=4, Hkv=2):
    return lib.attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, 1, H, Hkv, 16, 16, d,
                        0.1, 1, dtype, ws, ws_bytes, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(dq=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(ws=NULL), attn.ATTN_ERR_WORKSPACE),
    (dict(ws_bytes=16), attn.ATTN_ERR_WORKSPACE),     # needs 1*4*16*2*4 = 512
    (dict(H=3, Hkv=2), attn.ATTN_ERR_INVALID_ARG),
])
def test_bwd_validation(lib, cpu_only, kw, status):
    assert _bwd(lib, **kw) == status


def test_workspace_queries(lib):
    # Backward: two floats (D and the base-2 LSE) per query row.
    assert attn.attn_bwd_workspace_size(2, 16, 4096, 128) == 2 * 16 * 4096 * 2 * 4
    assert attn.attn_bwd_workspace_size(1, 1, 1, 96) == 0
    # Decode: (d + 2) floats per query head of every segment (split wave +
    # (sequence, KV head) pair), two ints per pair; the largest over the group
    # sizes G = Hq / Hkv.  4 sequences, Hq = 8, 1000 tokens (32 steps), 256-token
    # items (8 steps): G = 1 gives 32 pairs, 32 * 32 / 8 = 128 waves, 160 ids.
    def ws(pairs, G, waves, d=128):
        return (waves + pairs) * G * (d + 2) * 4 + pairs * 2 * 4
    want = max(ws(4 * 8 // G, G, -(-(4 * 8 // G) * 32 // 8)) for G in (1, 2, 4, 8))
    assert attn.attn_decode_paged_workspace_size(4, 8, 128, 1000, 256) == want == ws(32, 1, 128)
    assert attn.attn_decode_paged_workspace_size(4, 8, 128, 1000, 48) == 0
    # Automatic split: 1024 waves (one workgroup of four per CU); G = 16 needs
    # the most rows here.
    auto = attn.attn_decode_paged_workspace_size(64, 32, 128, 32768, 0)
    assert auto == max(ws(64 * 32 // G, G, 1024) for G in (1, 2, 4, 8, 16)) == ws(128, 16, 1024)
    # A group of more than 16 query heads is split into pairs of 16 heads:
    # Hq = 34 = 17 x 2 (G = 34: one KV head, three pairs of 16, 16 and 2 heads).
    pairs34 = 3
    assert attn.attn_decode_paged_workspace_size(1, 34, 128, 64, 32) >= ws(pairs34, 16, 2)
    # Few steps: the range length never drops below 2 steps (64 tokens).
    assert attn.attn_decode_paged_workspace_size(2, 2, 64, 100, 0) == ws(4, 1, 8, d=64)


def test_plan_describe_per_phase(lib):
    fwd = attn.attn_plan_describe(attn.ATTN_PHASE_FWD, 1, 32, 32, 8192, 8192, 128, True)
    assert "phase=fwd" in fwd and "Br=128" in fwd and "grid=2048" in fwd
    assert "splitkv" not in fwd  # the grid fills the GPU: no key split
    small = attn.attn_plan_describe(attn.ATTN_PHASE_FWD, 1, 4, 4, 8192, 8192, 128, True)
    assert "Br=64" in small  # too few workgroups at Br=128: split the sequence finer
    # ... and the key split attn_fwd_splitkv takes: 1664-key parts, 190 units
    # per head (760 workgroups for 768 resident), at most 5 parts per tile.
    assert "splitkv: Br=128 parts of <= 1664 keys, 190 units per head" in small
    assert "grid=760" in small and "<= 5 parts" in small
    f32 = attn.ATTN_DTYPE_F32
    one = attn.attn_plan_describe(attn.ATTN_PHASE_FWD, 1, 1, 1, 512, 512, 64, False, f32)
    assert "fwd_f32_keysplit" in one and "Br=32" in one and "grid=16" in one
    wide = attn.attn_plan_describe(attn.ATTN_PHASE_FWD, 2, 16, 16, 1030, 1030, 128, True, f32)
    assert "fwd_f32_mfma32x32x2" in wide and "Br=128" in wide and "grid=288" in wide
    dec = attn.attn_plan_describe(attn.ATTN_PHASE_DECODE, 64, 32, 8, 1, 32768, 128, False)
    assert "phase=decode" in dec and "G=4" in dec
    bwd = attn.attn_plan_describe(attn.ATTN_PHASE_BWD, 2, 16, 16, 4096, 4096, 128, True)
    assert "phase=bwd" in bwd
    with pytest.raises(ValueError):
        attn.attn_plan_describe(attn.ATTN_PHASE_FWD, 1, 3, 2, 8, 8, 64, True)


def test_tensor_marshalling_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attn_fwd(q, q, q, 0.125, True)


def _fwd_local(lib, left, right, dtype=attn.ATTN_DTYPE_BF16, Nq=8, Nk=8, d=64):
    return lib.attn_fwd_local(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 1, Nq, Nk, d, 0.125, left, right,
                              dtype, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(left=-2, right=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(left=0, right=-5), attn.ATTN_ERR_INVALID_ARG),
    (dict(left=3, right=0, dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(left=-1, right=2, dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(left=3, right=0, Nk=1 << 23, d=128), attn.ATTN_ERR_UNSUPPORTED),  # > 2 GiB per head
])
def test_fwd_local_validation(lib, cpu_only, kw, status):
    assert _fwd_local(lib, **kw) == status


def test_bwd_local_validation(lib, cpu_only):
    st = lib.attn_bwd_local(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 16, 16,
                            64, 0.1, -3, 0, attn.ATTN_DTYPE_BF16, FAKE, 1 << 20, NULL)
    assert st == attn.ATTN_ERR_INVALID_ARG
    st = lib.attn_bwd_local(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 16, 16,
                            64, 0.1, 4, 0, attn.ATTN_DTYPE_BF16, FAKE, 16, NULL)
    assert st == attn.ATTN_ERR_WORKSPACE


def _one_round_part(tiles, heads, slots, least):
    """Smallest part size in key tiles (at least `least`) whose parts of
    every query tile of every head number at most `slots`, by enumeration."""
    c = least
    while heads * sum(-(-t // c) for t in tiles) > slots:
        c += 1
    return c


def test_fwd_splitkv_workspace_queries(lib):
    # Forced 256-key parts over 1000 causal keys of d = 128 (32-key tiles): the
    # last query tile sees 1000 keys = 32 tiles = 4 parts of 8 tiles.  A
    # partial row is o / l in bf16 (2 d bytes) plus the max and the sum in fp32.
    assert attn.attn_fwd_splitkv_workspace_size(1, 2, 1000, 1000, 128, -1, 0, 256) == \
        2 * 8 * 4 * 128 * (2 * 128 + 8)
    assert attn.attn_fwd_splitkv_workspace_size(1, 2, 1000, 1000, 128, -1, 0, 100) == 0
    assert attn.attn_fwd_splitkv_workspace_size(1, 32, 8192, 8192, 128, -1, 0, 0) == 0
    # Planner, 4 heads x 8192 causal at d = 128: query tile i sees 4 (i + 1)
    # key tiles; parts of 52 tiles (1664 keys) are the shortest whose 760
    # units fit the 768 resident workgroups (3 per CU); the last tile has 5.
    tiles = [4 * (i + 1) for i in range(64)]
    ct = _one_round_part(tiles, 4, 3 * 256, 20)
    assert ct == 52
    assert attn.attn_fwd_splitkv_workspace_size(1, 4, 8192, 8192, 128, -1, 0, 0) == \
        4 * 64 * -(-256 // ct) * 128 * (2 * 128 + 8)
    # d = 64 (64-key tiles, 4 resident workgroups per CU), 4 heads x 4096.
    tiles = [2 * (i + 1) for i in range(32)]
    ct = _one_round_part(tiles, 4, 4 * 256, 10)
    assert attn.attn_fwd_splitkv_workspace_size(1, 4, 4096, 4096, 64, -1, 0, 0) == \
        4 * 32 * -(-64 // ct) * 128 * (2 * 64 + 8)
    # One 128-row query tile against 512 keys: parts of at least 640 keys
    # would not split it.
    assert attn.attn_fwd_splitkv_workspace_size(1, 1, 128, 512, 128, -1, 0, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(chunk=100), attn.ATTN_ERR_INVALID_ARG),
    (dict(chunk=-64), attn.ATTN_ERR_INVALID_ARG),
    (dict(chunk=256, ws=NULL), attn.ATTN_ERR_WORKSPACE),
    (dict(chunk=256, ws_bytes=16), attn.ATTN_ERR_WORKSPACE),
    (dict(chunk=256, dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(left=-4), attn.ATTN_ERR_INVALID_ARG),
])
def test_fwd_splitkv_validation(lib, cpu_only, kw, status):
    chunk = kw.get("chunk", 0)
    st = lib.attn_fwd_splitkv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 2, 1000, 1000, 128, 0.1,
                              kw.get("left", -1), 0, kw.get("dtype", attn.ATTN_DTYPE_BF16), chunk,
                              kw.get("ws", FAKE), kw.get("ws_bytes", 1 << 30), NULL)
    assert st == status


def _varlen(lib, q=FAKE, k=FAKE, cu_q=FAKE, cu_k=FAKE, num_seqs=2, total_q=16, total_k=20,
            max_q=8, H=2, Hkv=1, d=64, scale=0.125, wl=-1, wr=0, dtype=attn.ATTN_DTYPE_BF16):
    return lib.attn_fwd_varlen(q, k, FAKE, FAKE, FAKE, cu_q, cu_k, num_seqs, total_q, total_k,
                               max_q, H, Hkv, d, scale, wl, wr, dtype, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(cu_k=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(k=MISALIGNED), attn.ATTN_ERR_INVALID_ARG),
    (dict(num_seqs=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(max_q=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(max_q=17), attn.ATTN_ERR_INVALID_ARG),       # longer than the packed batch
    (dict(total_k=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(H=3, Hkv=2), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=96), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(wl=-2), attn.ATTN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), attn.ATTN_ERR_INVALID_ARG),
    (dict(total_q=1 << 22, H=64, d=128, max_q=8), attn.ATTN_ERR_UNSUPPORTED),  # > 2 GiB packed
])
def test_fwd_varlen_validation(lib, cpu_only, kw, status):
    assert _varlen(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def _prefill_paged(lib, q=FAKE, kc=FAKE, table=FAKE, num_seqs=2, total_q=16, max_q=8, Hq=4,
                   Hkv=2, d=128, bs=16, num_blocks=10, max_blocks=4, strides=None, wl=-1, wr=0,
                   dtype=attn.ATTN_DTYPE_BF16):
    if strides is None:
        strides = (bs * Hkv * d, Hkv * d, d)
    return lib.attn_prefill_paged(q, kc, FAKE, table, FAKE, FAKE, FAKE, FAKE, num_seqs, total_q,
                                  max_q, Hq, Hkv, d, bs, num_blocks, max_blocks, *strides, 0.088,
                                  wl, wr, dtype, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(table=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(kc=MISALIGNED), attn.ATTN_ERR_INVALID_ARG),
    (dict(bs=8), attn.ATTN_ERR_UNSUPPORTED),            # pages must hold a multiple of 16 tokens
    (dict(bs=24), attn.ATTN_ERR_UNSUPPORTED),
    (dict(num_blocks=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(strides=(16 * 2 * 128, 128, 128)), attn.ATTN_ERR_INVALID_ARG),  # token stride < Hkv*d
    (dict(strides=(100, 256, 128)), attn.ATTN_ERR_INVALID_ARG),           # overlapping blocks
    (dict(Hq=3, Hkv=2), attn.ATTN_ERR_INVALID_ARG),
    (dict(dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(d=80), attn.ATTN_ERR_UNSUPPORTED),
])
def test_prefill_paged_validation(lib, cpu_only, kw, status):
    assert _prefill_paged(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def _sparse(lib, rp=FAKE, ci=FAKE, B=1, H=2, Hkv=1, Nq=256, Nk=256, d=64, layouts=1, nnz=3,
            dtype=attn.ATTN_DTYPE_BF16):
    return lib.attn_fwd_block_sparse(FAKE, FAKE, FAKE, FAKE, FAKE, B, H, Hkv, Nq, Nk, d, 0.125, 1,
                                     rp, ci, layouts, nnz, dtype, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(rp=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(ci=NULL), attn.ATTN_ERR_INVALID_ARG),
    (dict(rp=ctypes.c_void_p((1 << 20) + 2)), attn.ATTN_ERR_INVALID_ARG),
    (dict(layouts=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(nnz=-1), attn.ATTN_ERR_INVALID_ARG),
    (dict(Nq=0), attn.ATTN_ERR_INVALID_ARG),
    (dict(d=32), attn.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=attn.ATTN_DTYPE_F32), attn.ATTN_ERR_UNSUPPORTED),
])
def test_block_sparse_validation(lib, cpu_only, kw, status):
    assert _sparse(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""
