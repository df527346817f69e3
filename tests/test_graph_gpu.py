"""The hot path captured in one HIP graph (torch.cuda.CUDAGraph around the
library's launches on the capturing stream): the forward, the key-split
forward, the paged decode and the backward, with every output and workspace
allocated before the capture.  The library allocates nothing and records no
memset, so each replay must equal the eager calls bit for bit; the replays
run with new inputs copied in and eager work (other launches, host syncs)
between them, and every replay is checked."""

import math

import pytest
import torch

import oracle
from exact_tiled_attention_04_amd import attn, workloads
from parity import check_lse, check_out, to64

pytestmark = pytest.mark.gpu


def _inputs(gpu, seed):
    fq, fk, fv = workloads.prefill(1, 4, 2, 1000, 1000, 128, dtype="bf16", seed=seed)
    sq, sk, sv = workloads.prefill(1, 2, 2, 2048, 2048, 128, dtype="bf16", seed=seed + 1)
    dec = workloads.decode(num_seqs=5, Hq=8, Hkv=2, d=128, ctx_lo=40, ctx_hi=700,
                           block_size=16, max_blocks_per_seq=44, dtype="bf16", seed=seed + 2,
                           context_lens=[40, 700, 333, 129, 512])
    bq, bk, bv, bdo = workloads.backward(1, 2, 2, 384, 384, 128, dtype="bf16", seed=seed + 3)
    host = dict(fq=fq, fk=fk, fv=fv, sq=sq, sk=sk, sv=sv, dq=dec["q"], kc=dec["k_cache"],
                vc=dec["v_cache"], bt=dec["block_table"], cl=dec["context_lens"], bq=bq, bk=bk,
                bv=bv, bdo=bdo)
    return {k: v.to(gpu) for k, v in host.items()}, host, dec["max_context"]


def test_hot_path_graph_replays_match_eager(gpu):
    x, _, max_ctx = _inputs(gpu, 11)
    scale = 1.0 / math.sqrt(128)
    # Outputs and workspaces, allocated once.
    fo, flse = torch.empty_like(x["fq"]), torch.empty((1, 4, 1000), dtype=torch.float32, device=gpu)
    so, slse = torch.empty_like(x["sq"]), torch.empty((1, 2, 2048), dtype=torch.float32, device=gpu)
    sws = torch.empty(attn.attn_fwd_splitkv_workspace_size(1, 2, 2048, 2048, 128, -1, 0, 256),
                      dtype=torch.uint8, device=gpu)
    do_, dlse = torch.empty_like(x["dq"]), torch.empty((5, 8), dtype=torch.float32, device=gpu)
    dws = torch.empty(max(attn.attn_decode_paged_workspace_size(5, 8, 128, max_ctx, 0), 16),
                      dtype=torch.uint8, device=gpu)
    bo, blse = torch.empty_like(x["bq"]), torch.empty((1, 2, 384), dtype=torch.float32, device=gpu)
    bdq, bdk, bdv = (torch.empty_like(x["bq"]), torch.empty_like(x["bk"]),
                     torch.empty_like(x["bv"]))
    bws = torch.empty(attn.attn_bwd_workspace_size(1, 2, 384, 128), dtype=torch.uint8,
                      device=gpu)
    fws = torch.empty(max(attn.attn_fwd_splitkv_workspace_size(1, 4, 1000, 1000, 128, -1, 0, 0),
                          16), dtype=torch.uint8, device=gpu)
    bfws = torch.empty(max(attn.attn_fwd_splitkv_workspace_size(1, 2, 384, 384, 128, -1, 0, 0),
                           16), dtype=torch.uint8, device=gpu)
    outs = (fo, flse, so, slse, do_, dlse, bo, blse, bdq, bdk, bdv)

    def step():
        attn.attn_fwd(x["fq"], x["fk"], x["fv"], scale, True, out=fo, lse=flse, workspace=fws)
        attn.attn_fwd_splitkv(x["sq"], x["sk"], x["sv"], scale, -1, 0, chunk_keys=256, out=so,
                              lse=slse, workspace=sws)
        attn.attn_decode_paged(x["dq"], x["kc"], x["vc"], x["bt"], x["cl"], scale, max_ctx,
                               out=do_, lse=dlse, workspace=dws)
        attn.attn_fwd(x["bq"], x["bk"], x["bv"], scale, True, out=bo, lse=blse, workspace=bfws)
        attn.attn_bwd(x["bq"], x["bk"], x["bv"], bo, x["bdo"], blse, scale, True, dq=bdq,
                      dk=bdk, dv=bdv, workspace=bws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager warm-up on the capturing stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep, seed in enumerate((21, 33, 47)):
        fresh, host, _ = _inputs(gpu, seed)
        for k in x:  # same shapes; the decode pages get a new placement
            x[k].copy_(fresh[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = [t.clone() for t in outs]
        junk = torch.randn(512, 512, device=gpu) @ torch.randn(512, 512, device=gpu)
        for t in outs:
            t.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        del junk
        for i, (a, b) in enumerate(zip(replayed, outs)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager call"
        # And the replay is right, not only repeatable (forward against the oracle).
        o_ref, lse_ref = oracle.forward(to64(host["fq"]), to64(host["fk"]), to64(host["fv"]),
                                        scale, True)
        check_out(to64(replayed[0]), o_ref, "bf16", what=f"graph replay {rep} O")
        check_lse(to64(replayed[1]), lse_ref, "bf16", what=f"graph replay {rep} LSE")
