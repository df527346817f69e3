"""Block-sparse forward (visits only the listed 128x128 score blocks): HIP
kernel against the oracle's definition with the expanded block mask."""

import math

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def _run(gpu, q, k, v, scale, causal, row_ptr, col_idx):
    o, lse = attn.attn_fwd_block_sparse(q.to(gpu), k.to(gpu), v.to(gpu), scale, causal,
                                        row_ptr.to(gpu), col_idx.to(gpu))
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _ref(q, k, v, scale, causal, row_ptr, col_idx):
    nq, nk = q.shape[2], k.shape[2]
    blocks = oracle.block_mask_from_index(row_ptr.numpy(), col_idx.numpy(), -(-nq // 128),
                                          -(-nk // 128))
    return oracle.block_sparse_forward(to64(q), to64(k), to64(v), scale, causal, blocks, 128, 128)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,layouts,causal", [
    (1, 4, 4, 1024, 1024, 1, True),
    (2, 4, 2, 700, 700, 4, True),      # ragged tail, per-head layouts, GQA
    (1, 2, 2, 512, 900, 2, False),     # rectangular, non-causal
    (2, 2, 1, 300, 1000, 4, True),     # bottom-right causal with Nq < Nk
])
def test_block_sparse_parity(gpu, d, B, H, Hkv, Nq, Nk, layouts, causal):
    q, k, v = workloads.prefill(B, H, Hkv, Nq, Nk, d, seed=Nq + d)
    nqb, nkb = -(-Nq // 128), -(-Nk // 128)
    row_ptr, col_idx = workloads.block_sparse_index(layouts, nqb, nkb, local=2, n_global=1,
                                                    density=0.3, seed=d + layouts)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(gpu, q, k, v, scale, causal, row_ptr, col_idx)
    o_ref, lse_ref = _ref(q, k, v, scale, causal, row_ptr, col_idx)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_block_sparse_all_blocks_equals_dense(gpu):
    """Listing every block (in reverse order) reproduces the dense causal
    forward within tolerance; the online softmax does not depend on order."""
    B, H, N, d = 1, 4, 640, 128
    q, k, v = workloads.prefill(B, H, H, N, N, d, seed=3)
    nb = N // 128
    row_ptr = torch.arange(0, nb * nb + 1, nb, dtype=torch.int32)[None]
    col_idx = torch.arange(nb - 1, -1, -1, dtype=torch.int32).repeat(nb)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(gpu, q, k, v, scale, True, row_ptr, col_idx)
    od, ld = attn.attn_fwd(q.to(gpu), k.to(gpu), v.to(gpu), scale, True)
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), scale, True)
    check_out(to64(o), o_ref, "bf16", what="O sparse vs oracle")
    check_lse(to64(lse), lse_ref, "bf16", what="LSE sparse vs oracle")
    check_out(to64(o), to64(od), "bf16", what="O sparse vs dense kernel")
    check_lse(to64(lse), to64(ld.cpu()), "bf16", what="LSE sparse vs dense kernel")


def test_block_sparse_empty_rows_and_bad_entries(gpu):
    """A query block listing nothing gets O = 0 and LSE = -inf; entries
    outside the key-block range are ignored."""
    B, H, N, d = 1, 2, 384, 64
    q, k, v = workloads.prefill(B, H, H, N, N, d, seed=4)
    # Row 0: nothing; row 1: block 0 plus out-of-range entries; row 2: blocks 2, 0.
    row_ptr = torch.tensor([[0, 0, 3, 5]], dtype=torch.int32)
    col_idx = torch.tensor([0, 7, -1, 2, 0], dtype=torch.int32)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(gpu, q, k, v, scale, False, row_ptr, col_idx)
    blocks = np.zeros((1, 3, 3), dtype=bool)
    blocks[0, 1, 0] = True
    blocks[0, 2, [0, 2]] = True
    o_ref, lse_ref = oracle.block_sparse_forward(to64(q), to64(k), to64(v), scale, False, blocks,
                                                 128, 128)
    assert torch.all(o[:, :, :128] == 0)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_block_sparse_long_rows_refill(gpu):
    """Rows listing more than 64 key blocks (the index is read 64 entries at a
    time): 100 key blocks, four of every five listed."""
    B, H, Nq, Nk, d = 1, 2, 256, 12800, 64
    q, k, v = workloads.prefill(B, H, H, Nq, Nk, d, seed=6)
    nkb = Nk // 128
    cols = [c for c in range(nkb) if c % 5 != 3]
    row_ptr = torch.tensor([[0, len(cols), 2 * len(cols)]], dtype=torch.int32)
    col_idx = torch.tensor(cols + cols, dtype=torch.int32)
    assert len(cols) > 64
    scale = 1.0 / math.sqrt(d)
    o, lse = _run(gpu, q, k, v, scale, True, row_ptr, col_idx)
    o_ref, lse_ref = _ref(q, k, v, scale, True, row_ptr, col_idx)
    check_out(to64(o), o_ref, "bf16")
    check_lse(to64(lse), lse_ref, "bf16")


def test_block_sparse_bench_shape(gpu):
    """The benchmark's block-sparse workload (B=1, H=32, N=8192, d=128,
    per-head local + global + random blocks, causal) in the benchmark's
    launch configuration: every row of eight heads (eight of the 32 layouts)
    against the oracle, with the block mask and the causal mask written out
    as one boolean mask."""
    bw = workloads.WORKLOADS["block_sparse_causal_bf16_b1_h32_n8192_d128"]
    N, d, H = bw["N"], bw["d"], bw["H"]
    q, k, v = workloads.prefill(bw["B"], H, bw["Hkv"], N, N, d, seed=bw["seed"], device=str(gpu))
    row_ptr, col_idx = workloads.block_sparse_index(bw["layouts"], N // 128, N // 128, bw["local"],
                                                    bw["n_global"], bw["density"], seed=bw["seed"])
    o, lse = _run(gpu, q, k, v, bw["scale"], True, row_ptr, col_idx)
    q, k, v, o, lse = q.cpu(), k.cpu(), v.cpu(), o.cpu(), lse.cpu()
    blocks = oracle.block_mask_from_index(row_ptr.numpy(), col_idx.numpy(), N // 128, N // 128)
    pos = np.arange(N)
    for h in range(0, H, 4):
        vis = np.repeat(np.repeat(blocks[h % bw["layouts"]], 128, axis=0), 128, axis=1)
        vis &= pos[None, :] <= pos[:, None]
        o_ref, lse_ref = oracle.forward(to64(q[0, h])[None, None], to64(k[0, h])[None, None],
                                        to64(v[0, h])[None, None], bw["scale"], False,
                                        mask=vis[None, None])
        check_out(to64(o[0, h]), o_ref[0, 0], "bf16", what=f"O head {h}")
        check_lse(to64(lse[0, h]), lse_ref[0, 0], "bf16", what=f"LSE head {h}")
