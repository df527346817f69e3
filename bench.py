"""Benchmark of the exact tiled attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over synthetic inputs already
resident in HBM:
  1. causal bf16 forward, B=1, H=32, N=8192, d=128, scale 1/sqrt(128)
     (the headline workload: TFLOP/s and fraction of dense bf16 MFMA peak);
  2. paged GQA decode, 64 sequences, Hq=32, Hkv=8, d=128, contexts uniform
     in [4096, 32768], 16-token pages via a seeded permutation (KV GB/s and
     fraction of HBM peak);
  3. causal bf16 backward, B=2, H=16, N=4096, d=128 (TFLOP/s);
Each call is bracketed by HIP events recorded on the stream the library
launches on (torch's current stream); the K timed steps are bracketed by a
device synchronisation on both sides.  Rank 0 prints one JSON line.

After the timed steps, the other forward configurations (d = 64: B=4, H=16,
N=2048 causal; the headline shape non-causal) and the entry points beyond the
hot path are timed the same way in a loop of their own (K calls each, after W
warm-up calls and 0.3 s of further calls), so they do not change the
conditions the step is measured under:
  * the 4-head variant of (1) through the key split;
  * a packed ragged causal prefill (16 sequences of 512..8192 tokens, GQA
    32/8, d=128);
  * a chunked prefill through the paged cache (16 sequences, 512..2048 new
    tokens after 2048..8192 cached ones, 16-token pages);
  * a block-sparse causal forward (B=1, H=32, N=8192, d=128, per-head local
    + global + random 128x128 blocks).
Their FLOPs count the (query, key) pairs the masks leave visible, times 4 d.

FLOPs follow "Attention kernels" (the FLOPs paragraph): 4 N^2 d per head,
halved under the causal mask; the backward also reports its algorithmic
five-product count 10 N^2 d / 2.  Decode bytes are the K and V cache rows the
contexts cover: 2 * sum(ctx) * Hkv * d * 2 bytes.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector and MFMA)
METRIC = "fwd attention TFLOP/s & % bf16 MFMA peak; paged decode KV GB/s % HBM peak"


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # A GPU coming out of idle runs these kernels ~5% slower for its first
    # tens to hundreds of milliseconds while its clocks and power settle;
    # 400 warm-up steps (~0.7 s) put the timed steps in the steady state.
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the fp64 oracle on the host (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 512 MiB device copy first, so PMC byte counters "
                         "can be scaled against a kernel of known traffic")
    ap.add_argument("--cpu-heads", type=int, default=24,
                    help="heads of the forward workload the oracle is timed on")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line, time a sweep of shapes (batch, lengths, "
                         "heads, head dimension, masks, cache block size) and print one JSON "
                         "line per shape")
    return ap.parse_args()


def _source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel, sources, per_launch_algorithmic):
    """HBM traffic per launch from the committed rocprofv3 PMC summary, when
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    rec = data.get(kernel)
    if not rec or rec.get("source_digest") != _source_digest(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the "
              "library runs on one GPU; sharding across GPUs is not implemented).",
              file=sys.stderr)
        return 2

    import torch
    from exact_tiled_attention_04_amd import attn, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    attn.load_library()  # fails loudly when the HIP library is missing
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    if args.sweep:
        return sweep(args, dev, stream)
    if args.copy_calibration:
        # 512 MiB read + 512 MiB written by one copy kernel.
        src = torch.ones(256 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- inputs (seeded, generated on the device, resident before timing)
    fw = workloads.WORKLOADS["causal_bf16_b1_h32_n8192_d128"]
    q, k, v = workloads.prefill(fw["B"], fw["H"], fw["Hkv"], fw["Nq"], fw["Nk"], fw["d"],
                                dtype="bf16", seed=fw["seed"], device=str(dev))
    o = torch.empty_like(q)
    lse = torch.empty((fw["B"], fw["H"], fw["Nq"]), dtype=torch.float32, device=dev)
    fwd_flops = 4.0 * fw["B"] * fw["H"] * fw["Nq"] * fw["Nk"] * fw["d"] / 2.0

    dw = workloads.WORKLOADS["paged_gqa_decode_bf16_s64_hq32_hkv8_d128"]
    dec = workloads.decode(num_seqs=dw["num_seqs"], Hq=dw["Hq"], Hkv=dw["Hkv"], d=dw["d"],
                           ctx_lo=dw["ctx_lo"], ctx_hi=dw["ctx_hi"], block_size=dw["block_size"],
                           max_blocks_per_seq=dw["max_blocks_per_seq"], dtype="bf16",
                           seed=dw["seed"], device=str(dev))
    dbt = dec["block_table"].to(dev)
    dctx = dec["context_lens"].to(dev)
    dout = torch.empty_like(dec["q"])
    dlse = torch.empty((dw["num_seqs"], dw["Hq"]), dtype=torch.float32, device=dev)
    dws = torch.empty(max(attn.attn_decode_paged_workspace_size(
        dw["num_seqs"], dw["Hq"], dw["d"], dw["ctx_hi"], 0), 16), dtype=torch.uint8, device=dev)
    sum_ctx = int(dec["context_lens"].sum())
    dec_bytes = 2.0 * sum_ctx * dw["Hkv"] * dw["d"] * 2

    # The four-head variant of the same prefill: too few query tiles to fill
    # the chip, so it goes through the key split (partials + merge).
    sw = workloads.WORKLOADS["causal_bf16_b1_h4_n8192_d128"]
    sq, sk, sv = workloads.prefill(sw["B"], sw["H"], sw["Hkv"], sw["Nq"], sw["Nk"], sw["d"],
                                   dtype="bf16", seed=sw["seed"], device=str(dev))
    so = torch.empty_like(sq)
    slse = torch.empty((sw["B"], sw["H"], sw["Nq"]), dtype=torch.float32, device=dev)
    sws_bytes = attn.attn_fwd_splitkv_workspace_size(sw["B"], sw["H"], sw["Nq"], sw["Nk"],
                                                     sw["d"], -1, 0, 0)
    sws = torch.empty(max(sws_bytes, 16), dtype=torch.uint8, device=dev)
    split_flops = 4.0 * sw["B"] * sw["H"] * sw["Nq"] * sw["Nk"] * sw["d"] / 2.0

    bw = workloads.WORKLOADS["causal_bwd_bf16_b2_h16_n4096_d128"]
    bq, bk, bv, bdo = workloads.backward(bw["B"], bw["H"], bw["Hkv"], bw["Nq"], bw["Nk"], bw["d"],
                                         dtype="bf16", seed=bw["seed"], device=str(dev))
    bo, blse = attn.attn_fwd(bq, bk, bv, bw["scale"], True)
    bdq, bdk, bdv = torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv)
    bws = torch.empty(attn.attn_bwd_workspace_size(bw["B"], bw["H"], bw["Nq"], bw["d"]),
                      dtype=torch.uint8, device=dev)
    bwd_flops_fwd_equiv = 4.0 * bw["B"] * bw["H"] * bw["Nq"] * bw["Nk"] * bw["d"] / 2.0
    bwd_flops_algo = 2.5 * bwd_flops_fwd_equiv

    # Packed ragged prefill, chunked prefill through the paged cache, and
    # block-sparse visitation.
    vw = workloads.WORKLOADS["varlen_causal_bf16_s16_h32_hkv8_d128"]
    vlens = workloads.ragged_lengths(vw["num_seqs"], vw["len_lo"], vw["len_hi"], seed=vw["seed"] + 1)
    rg = workloads.ragged(vlens, vlens, vw["H"], vw["Hkv"], vw["d"], seed=vw["seed"], device=str(dev))
    rg_cu = rg["cu_q"].to(dev)
    rg_o = torch.empty_like(rg["q"])
    rg_lse = torch.empty((vw["H"], rg["q"].shape[0]), dtype=torch.float32, device=dev)
    varlen_flops = 4.0 * vw["d"] * vw["H"] * sum(n * (n + 1) / 2 for n in vlens)

    pw = workloads.WORKLOADS["paged_prefill_causal_bf16_s16_hq32_hkv8_d128"]
    pp = workloads.serving_prefill(pw["num_seqs"], pw["q_lo"], pw["q_hi"], pw["ctx_lo"],
                                   pw["ctx_hi"], pw["Hq"], pw["Hkv"], pw["d"],
                                   block_size=pw["block_size"], seed=pw["seed"], device=str(dev))
    pp_bt, pp_cu, pp_k = (pp["block_table"].to(dev), pp["cu_q"].to(dev), pp["seqlens_k"].to(dev))
    pp_o = torch.empty_like(pp["q"])
    pp_lse = torch.empty((pw["Hq"], pp["q"].shape[0]), dtype=torch.float32, device=dev)
    # Query row i of a chunk of q rows sits at position i + k - q and sees keys 0 .. that position.
    paged_flops = 4.0 * pw["d"] * pw["Hq"] * sum(
        q_ * (k_ - q_) + q_ * (q_ + 1) / 2 for q_, k_ in zip(pp["q_lens"], pp["k_lens"]))

    xw = workloads.WORKLOADS["block_sparse_causal_bf16_b1_h32_n8192_d128"]
    xq, xk, xv = workloads.prefill(xw["B"], xw["H"], xw["Hkv"], xw["N"], xw["N"], xw["d"],
                                   seed=xw["seed"], device=str(dev))
    nb = xw["N"] // 128
    x_rp, x_ci = workloads.block_sparse_index(xw["layouts"], nb, nb, xw["local"], xw["n_global"],
                                              xw["density"], seed=xw["seed"])
    sparse_flops = 4.0 * xw["d"] * xw["B"] * sum(
        _sparse_pairs(x_rp[h % xw["layouts"]].tolist(), x_ci.tolist()) for h in range(xw["H"]))
    sparse_density = sparse_flops / (4.0 * xw["d"] * xw["B"] * xw["H"] * xw["N"] * (xw["N"] + 1) / 2)
    x_rp, x_ci = x_rp.to(dev), x_ci.to(dev)
    xo = torch.empty_like(xq)
    xlse = torch.empty((xw["B"], xw["H"], xw["N"]), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(events=None):
        e = events
        if e: e[0].record(stream)
        attn.attn_fwd(q, k, v, fw["scale"], True, out=o, lse=lse, stream=stream)
        if e: e[1].record(stream)
        attn.attn_decode_paged(dec["q"], dec["k_cache"], dec["v_cache"], dbt, dctx, dw["scale"],
                               dw["ctx_hi"], out=dout, lse=dlse, workspace=dws, stream=stream)
        if e: e[2].record(stream)
        attn.attn_bwd(bq, bk, bv, bo, bdo, blse, bw["scale"], True, dq=bdq, dk=bdk, dv=bdv,
                      workspace=bws, stream=stream)
        if e: e[3].record(stream)

    # The other forward configurations: d = 64 (B=4, H=16, N=2048, causal)
    # and the headline shape without the mask.
    c2 = workloads.WORKLOADS["causal_bf16_b4_h16_n2048_d64"]
    c2q, c2k, c2v = workloads.prefill(c2["B"], c2["H"], c2["Hkv"], c2["Nq"], c2["Nk"], c2["d"],
                                      dtype="bf16", seed=c2["seed"], device=str(dev))
    c2o = torch.empty_like(c2q)
    c2lse = torch.empty((c2["B"], c2["H"], c2["Nq"]), dtype=torch.float32, device=dev)
    c2_flops = 4.0 * c2["B"] * c2["H"] * c2["Nq"] * c2["Nk"] * c2["d"] / 2.0
    nc = workloads.WORKLOADS["noncausal_bf16_b1_h32_n8192_d128"]
    nc_flops = 4.0 * nc["B"] * nc["H"] * nc["Nq"] * nc["Nk"] * nc["d"]
    # The single-head fp32 configuration (B=1, H=1, N=512, d=64, non-causal).
    c1 = workloads.WORKLOADS["single_head_f32_n512_d64"]
    c1q, c1k, c1v = workloads.prefill(c1["B"], c1["H"], c1["Hkv"], c1["Nq"], c1["Nk"], c1["d"],
                                      dtype="f32", seed=c1["seed"], device=str(dev))
    c1o = torch.empty_like(c1q)
    c1lse = torch.empty((c1["B"], c1["H"], c1["Nq"]), dtype=torch.float32, device=dev)
    c1_flops = 4.0 * c1["B"] * c1["H"] * c1["Nq"] * c1["Nk"] * c1["d"]

    # Context for the MFMA roofline: the vendor's bf16 GEMM (torch.matmul)
    # on this GPU, timed the same way -- the sustained rate dense MFMA work
    # gets under the chip's power limit.
    ga = torch.randn(16384, 4096, device=dev, dtype=torch.bfloat16)
    gb = torch.randn(4096, 16384, device=dev, dtype=torch.bfloat16)
    gc = torch.empty(16384, 16384, device=dev, dtype=torch.bfloat16)
    gemm_flops = 2.0 * 16384 * 16384 * 4096

    # The vendor GEMM goes last: its sustained MFMA load lowers the clocks
    # the calls after it would get.
    extras = [
        ("fwd_f32_config1", c1_flops, lambda: attn.attn_fwd(c1q, c1k, c1v, c1["scale"], False,
                                                            out=c1o, lse=c1lse, stream=stream)),
        ("fwd_d64", c2_flops, lambda: attn.attn_fwd(c2q, c2k, c2v, c2["scale"], True, out=c2o,
                                                    lse=c2lse, stream=stream)),
        ("fwd_noncausal", nc_flops, lambda: attn.attn_fwd(q, k, v, nc["scale"], False, out=o,
                                                          lse=lse, stream=stream)),
        ("fwd_small_grid", split_flops, lambda: attn.attn_fwd_splitkv(
            sq, sk, sv, sw["scale"], -1, 0, out=so, lse=slse, workspace=sws, stream=stream)),
        ("varlen", varlen_flops, lambda: attn.attn_fwd_varlen(
            rg["q"], rg["k"], rg["v"], rg_cu, rg_cu, rg["max_q"], vw["scale"], -1, 0, out=rg_o,
            lse=rg_lse, stream=stream)),
        ("paged_prefill", paged_flops, lambda: attn.attn_prefill_paged(
            pp["q"], pp["k_cache"], pp["v_cache"], pp_bt, pp_cu, pp_k, pp["max_q"], pw["scale"],
            -1, 0, out=pp_o, lse=pp_lse, stream=stream)),
        ("block_sparse", sparse_flops, lambda: attn.attn_fwd_block_sparse(
            xq, xk, xv, xw["scale"], True, x_rp, x_ci, out=xo, lse=xlse, stream=stream)),
        ("vendor_gemm", gemm_flops, lambda: torch.matmul(ga, gb, out=gc)),
    ]

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # amdsmi's readings lag by hundreds of milliseconds, longer than the
    # timed steps: the clock and power are sampled over two further seconds
    # of the same steps, run back to back right after them.
    clock = _clock_during(step, stream)

    def med(vals):
        s = sorted(vals)
        return s[len(s) // 2]

    # Each one after a few warm-up calls and 0.3 s of further calls, so it
    # runs at the clock its own load settles at rather than its predecessor's.
    extra = {}
    for name, flops, call in extras:
        ms = _time_calls(call, stream, args.steps, min(args.warmup, 3), settle_s=0.3)
        extra[name] = (sum(ms) / len(ms), med(ms), flops, ms)

    fwd_ms = [ev[0].elapsed_time(ev[1]) for ev in events]
    dec_ms = [ev[1].elapsed_time(ev[2]) for ev in events]
    bwd_ms = [ev[2].elapsed_time(ev[3]) for ev in events]
    split_avg = extra["fwd_small_grid"][0]
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    bwd_avg = sum(bwd_ms) / len(bwd_ms)
    fwd_tflops = fwd_flops / (fwd_avg * 1e-3) / 1e12
    dec_gbs = dec_bytes / (dec_avg * 1e-3) / 1e9
    bwd_tflops_algo = bwd_flops_algo / (bwd_avg * 1e-3) / 1e12
    bwd_tflops_fwd_equiv = bwd_flops_fwd_equiv / (bwd_avg * 1e-3) / 1e12

    fwd_src = ["exact_tiled_attention_04_amd/csrc/fwd.hip",
               "exact_tiled_attention_04_amd/csrc/common.hpp",
               "exact_tiled_attention_04_amd/csrc/kernels.hpp"]
    dec_src = ["exact_tiled_attention_04_amd/csrc/decode.hip",
               "exact_tiled_attention_04_amd/csrc/common.hpp",
               "exact_tiled_attention_04_amd/csrc/kernels.hpp"]
    result = {
        "metric": METRIC,
        "value": round(fwd_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal_bf16_b1_h32_n8192_d128 (headline) + "
                        "paged_gqa_decode_bf16_s64_hq32_hkv8_d128 + causal_bwd_bf16_b2_h16_n4096_d128",
            "B": fw["B"], "H": fw["H"], "N": fw["Nq"], "d": fw["d"], "causal": True,
            "plan": attn.attn_plan_describe(attn.ATTN_PHASE_FWD, fw["B"], fw["H"], fw["Hkv"],
                                            fw["Nq"], fw["Nk"], fw["d"], True),
        },
        "roofline": {
            "kernel": "fwd_bf16_kernel<D=128,band=causal,NW=4,BC=32>",
            "bound": "mfma",
            "achieved": round(fwd_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": _traffic("fwd_bf16_kernel<D=128,band=causal,NW=4,BC=32>", fwd_src, None),
            "avg_launch_ms": round(fwd_avg, 4),
            "algorithmic_flop_per_launch": fwd_flops,
            "vendor_bf16_gemm_tflops": round(gemm_flops / (extra["vendor_gemm"][0] * 1e-3) / 1e12, 1),
        },
        "decode": {
            "value": round(dec_gbs, 1),
            "unit": "GB/s",
            "frac_hbm": round(dec_gbs / PEAK_HBM_GBS, 4),
            "avg_call_ms": round(dec_avg, 4),
            "kv_bytes_per_call": dec_bytes,
            "sum_context_tokens": sum_ctx,
            "plan": attn.attn_plan_describe(attn.ATTN_PHASE_DECODE, dw["num_seqs"], dw["Hq"],
                                            dw["Hkv"], 1, dw["ctx_hi"], dw["d"], False),
            "roofline": {"kernel": "decode_split_paged_kernel<128>+decode_merge_kernel", "bound": "hbm",
                         "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
                         "traffic": _traffic("decode_split_paged_kernel<128>", dec_src, None)},
        },
        "bwd": {
            "value": round(bwd_tflops_algo, 2),
            "unit": "TFLOP/s (5-product algorithmic count)",
            "fwd_equivalent_tflops": round(bwd_tflops_fwd_equiv, 2),
            "frac_mfma_peak": round(bwd_tflops_algo / PEAK_BF16_TFLOPS, 4),
            "avg_call_ms": round(bwd_avg, 4),
        },
        "fwd_small_grid": {
            "workload": "causal_bf16_b1_h4_n8192_d128 (attn_fwd_splitkv)",
            "value": round(split_flops / (split_avg * 1e-3) / 1e12, 2),
            "unit": "TFLOP/s",
            "frac_mfma_peak": round(split_flops / (split_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "avg_call_ms": round(split_avg, 4),
            "workspace_bytes": sws_bytes,
        },
        "per_call_ms_median": {"fwd": round(med(fwd_ms), 4), "decode": round(med(dec_ms), 4),
                               "bwd": round(med(bwd_ms), 4),
                               **{k: round(v[1], 4) for k, v in extra.items()}},
        # Tail behaviour ("Benchmarking method": medians plus tails), kernel
        # launches and temporary (workspace) bytes per call.
        "per_call_ms_tail": {"fwd": _tail(fwd_ms), "decode": _tail(dec_ms), "bwd": _tail(bwd_ms),
                             **{k: _tail(v[3]) for k, v in extra.items()}},
        "vendor_gemm": {"workload": "torch.matmul bf16 16384x16384x4096 (hipBLASLt)",
                        "value": round(gemm_flops / (extra["vendor_gemm"][0] * 1e-3) / 1e12, 1),
                        "unit": "TFLOP/s"},
        "launches_and_temporary_bytes": {
            "fwd": [1, 0], "decode": [2, dws.numel()], "bwd": [2, bws.numel()],
            "fwd_small_grid": [2, sws_bytes], "varlen": [1, 0], "paged_prefill": [1, 0],
            "block_sparse": [1, 0]},
    }
    for name, workload, note in [
            ("fwd_d64", "causal_bf16_b4_h16_n2048_d64 (attn_fwd)", "d = 64, 64-key tiles"),
            ("fwd_noncausal", "noncausal_bf16_b1_h32_n8192_d128 (attn_fwd)",
             "the headline shape without the mask"),
            ("varlen", "varlen_causal_bf16_s16_h32_hkv8_d128 (attn_fwd_varlen)",
             f"{len(vlens)} packed sequences, {sum(vlens)} tokens"),
            ("paged_prefill", "paged_prefill_causal_bf16_s16_hq32_hkv8_d128 (attn_prefill_paged)",
             f"{sum(pp['q_lens'])} new tokens over {sum(pp['k_lens'])} cached"),
            ("block_sparse", "block_sparse_causal_bf16_b1_h32_n8192_d128 (attn_fwd_block_sparse)",
             f"visible pairs {100 * sparse_density:.1f}% of causal")]:
        avg, _, flops, _ = extra[name]
        tf = flops / (avg * 1e-3) / 1e12
        result[name] = {"workload": workload, "value": round(tf, 2), "unit": "TFLOP/s",
                        "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                        "avg_call_ms": round(avg, 4), "flop_per_call": flops, "note": note}

    avg, _, flops, _ = extra["fwd_f32_config1"]
    result["config1_f32"] = {
        "workload": "single_head_f32_n512_d64 (attn_fwd, fp32 inputs and accumulation)",
        "ms": round(avg, 4), "value": round(flops / (avg * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "frac_fp32_peak": round(flops / (avg * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 4),
        "flop_per_call": flops,
        "note": "16 workgroups of 32 query rows, 8 waves each over an eighth of the keys, merged in LDS: latency-bound"}
    # Clocks cannot be pinned without administrator rights; the GFX clock and
    # socket power are sampled while the timed steps run.
    result["clock"] = clock
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(q, k, v, fw, args.cpu_heads)
    print(json.dumps(result))
    return 0


def _time_calls(call, stream, calls, warmup, settle_s=0.03):
    """Per-call milliseconds of `calls` back-to-back calls after `warmup`
    calls and then at least `settle_s` seconds of further calls (an idle GPU
    needs some tens of milliseconds of load before its clocks settle)."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(4):
            call()
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(calls):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(calls)]


def sweep(args, dev, stream):
    """The shape space of "Modern attention kernels", "Benchmarking method":
    batch, query and key length, heads and KV heads, head dimension, causal /
    local / block-sparse masks, cache block size.  One JSON line per shape
    with TFLOP/s (visible pairs x 4 d) or KV GB/s, median and tail."""
    import torch
    from exact_tiled_attention_04_amd import attn, workloads

    calls, warm = max(args.steps, 5), max(args.warmup, 2)

    def emit(kind, shape, ms, work, unit):
        t = _tail(ms)
        rate = work / (t["p50"] * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        print(json.dumps({"sweep": kind, **shape, "value": round(rate, 1), "unit": unit,
                          "ms": t}), flush=True)

    # Forward: batch, length, heads / KV heads, head dimension, mask.
    for B, H, Hkv, N, d in [(1, 32, 32, 8192, 128), (1, 32, 8, 8192, 128), (2, 16, 16, 4096, 128),
                            (8, 16, 16, 2048, 128), (4, 16, 16, 2048, 64), (16, 16, 4, 1024, 64),
                            (1, 8, 8, 16384, 128), (32, 32, 8, 512, 128)]:
        q, k, v = workloads.prefill(B, H, Hkv, N, N, d, seed=1, device=str(dev))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        for mask, wl, wr in [("causal", -1, 0), ("none", -1, -1), ("window1024", 1023, 0)]:
            if mask == "window1024" and N <= 1024:
                continue
            call = lambda: attn.attn_fwd_local(q, k, v, 1 / math.sqrt(d), wl, wr, out=o, lse=lse,  # noqa: E731
                                               stream=stream)
            ms = _time_calls(call, stream, calls, warm)
            if mask == "causal":
                pairs = N * (N + 1) / 2
            elif mask == "none":
                pairs = N * N
            else:
                pairs = sum(min(i + 1, wl + 1) for i in range(N))
            emit("fwd", {"B": B, "H": H, "Hkv": Hkv, "N": N, "d": d, "mask": mask}, ms,
                 4.0 * d * B * H * pairs, "TFLOP/s")
        del q, k, v, o, lse
    # Rectangular (a chunk of queries at the end of a longer context), plain
    # and through the key split (which needs a workspace, so only
    # attn_fwd_splitkv takes it).
    for Nq, Nk in [(512, 8192), (2048, 16384)]:
        q, k, v = workloads.prefill(1, 32, 8, Nq, Nk, 128, seed=2, device=str(dev))
        pairs = Nq * (Nk - Nq) + Nq * (Nq + 1) / 2
        ms = _time_calls(lambda: attn.attn_fwd(q, k, v, 1 / math.sqrt(128), True, stream=stream),
                         stream, calls, warm)
        emit("fwd", {"B": 1, "H": 32, "Hkv": 8, "Nq": Nq, "Nk": Nk, "d": 128, "mask": "causal"},
             ms, 4.0 * 128 * 32 * pairs, "TFLOP/s")
        need = attn.attn_fwd_splitkv_workspace_size(1, 32, Nq, Nk, 128, -1, 0, 0)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        ms = _time_calls(lambda: attn.attn_fwd_splitkv(q, k, v, 1 / math.sqrt(128), -1, 0,  # noqa: E731
                                                       workspace=ws, stream=stream),
                         stream, calls, warm)
        emit("fwd_splitkv", {"B": 1, "H": 32, "Hkv": 8, "Nq": Nq, "Nk": Nk, "d": 128,
                             "mask": "causal", "split": need > 0}, ms,
             4.0 * 128 * 32 * pairs, "TFLOP/s")
    # Decode: sequences, context length, GQA group, cache block size.
    for S, Hq, Hkv, lo, hi, bs in [(64, 32, 8, 4096, 32768, 16), (64, 32, 8, 4096, 32768, 32),
                                   (16, 32, 8, 32768, 65536, 16), (256, 32, 8, 1024, 4096, 16),
                                   (64, 64, 8, 8192, 16384, 16), (128, 16, 16, 2048, 8192, 16),
                                   (1, 32, 8, 65536, 65536, 16), (8, 32, 1, 1024, 2048, 16)]:
        w = workloads.decode(num_seqs=S, Hq=Hq, Hkv=Hkv, d=128, ctx_lo=lo, ctx_hi=hi,
                             block_size=bs, max_blocks_per_seq=(hi + bs - 1) // bs,
                             dtype="bf16", seed=3, device=str(dev))
        bt, cl = w["block_table"].to(dev), w["context_lens"].to(dev)
        ws = torch.empty(max(attn.attn_decode_paged_workspace_size(S, Hq, 128, hi, 0), 16),
                         dtype=torch.uint8, device=dev)
        call = lambda: attn.attn_decode_paged(w["q"], w["k_cache"], w["v_cache"], bt, cl,  # noqa: E731
                                              1 / math.sqrt(128), hi, workspace=ws, stream=stream)
        ms = _time_calls(call, stream, calls, warm)
        emit("decode", {"seqs": S, "Hq": Hq, "Hkv": Hkv, "ctx": [lo, hi], "block_size": bs}, ms,
             2.0 * int(w["context_lens"].sum()) * Hkv * 128 * 2, "GB/s")
        del w, bt, cl, ws
    # Backward.
    for B, H, Hkv, N, d in [(2, 16, 16, 4096, 128), (1, 32, 8, 8192, 128), (4, 16, 16, 2048, 64)]:
        q, k, v, do = workloads.backward(B, H, Hkv, N, N, d, seed=4, device=str(dev))
        o, lse = attn.attn_fwd(q, k, v, 1 / math.sqrt(d), True)
        ws = torch.empty(attn.attn_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=dev)
        call = lambda: attn.attn_bwd(q, k, v, o, do, lse, 1 / math.sqrt(d), True, workspace=ws,  # noqa: E731
                                     stream=stream)
        ms = _time_calls(call, stream, calls, warm)
        emit("bwd", {"B": B, "H": H, "Hkv": Hkv, "N": N, "d": d, "mask": "causal"}, ms,
             10.0 * d * B * H * N * (N + 1) / 2, "TFLOP/s")
        del q, k, v, do, o, lse, ws
    return 0


def _tail(ms):
    """p10 / median / p90 / max of per-call milliseconds."""
    v = sorted(ms)
    pick = lambda q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]  # noqa: E731
    return {"p10": round(pick(0.1), 4), "p50": round(pick(0.5), 4), "p90": round(pick(0.9), 4),
            "max": round(v[-1], 4)}


def _sparse_pairs(row_ptr, col_idx, block=128):
    """Causal (query, key) pairs inside the listed blocks of one layout with
    Nq = Nk (square blocks): blocks below the diagonal are full, diagonal
    blocks hold a triangle, blocks above hold none."""
    pairs = 0
    for r in range(len(row_ptr) - 1):
        for c in col_idx[row_ptr[r]:row_ptr[r + 1]]:
            if c < r:
                pairs += block * block
            elif c == r:
                pairs += block * (block + 1) // 2
    return pairs


def _clock_during(call, stream, seconds=2.0):
    """GFX clock and socket power (amdsmi clock and power queries) sampled
    while `call` runs back to back on `stream`: batches of calls are queued,
    two batches stay in flight (so the GPU never waits for the host), and
    both values are read while they run.  Returns the median and range over
    the second half of the samples (amdsmi's readings lag by hundreds of
    milliseconds), the board's power limit, or the error.  (amdsmi's GPU-metrics table is not used: it held the same
    stale idle values for the whole run.)"""
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
        clk = lambda: amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)  # noqa: E731
        pwr = lambda: amdsmi.amdsmi_get_power_info(handle)  # noqa: E731
        first_clk, first_pwr = clk(), pwr()
    except Exception as exc:  # no SMI access: report why, keep the bench line
        return {"error": f"{type(exc).__name__}: {exc}"}

    def num(x):
        try:
            return float(x)
        except (TypeError, ValueError):
            return None

    mhz, watts = [], []
    in_flight = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            call()
        ev = torch.cuda.Event()
        ev.record(stream)
        in_flight.append(ev)
        if len(in_flight) > 2:
            in_flight.pop(0).synchronize()
        try:
            c = num(clk().get("clk"))
            w = num(pwr().get("current_socket_power"))
            if c:
                mhz.append(c)
            if w:
                watts.append(w)
        except Exception:
            pass
    torch.cuda.synchronize()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass

    def stats(v):
        v = sorted(v[len(v) // 2:])
        return (v[len(v) // 2], v[0], v[-1]) if v else (None, None, None)

    c50, c_lo, c_hi = stats(mhz)
    w50, w_lo, w_hi = stats(watts)
    limit = num(first_pwr.get("power_limit"))
    return {"gfx_mhz_median": c50, "gfx_mhz_min": c_lo, "gfx_mhz_max": c_hi,
            "socket_power_w_median": w50, "socket_power_w_min": w_lo, "socket_power_w_max": w_hi,
            "power_limit_w": limit / 1e6 if limit and limit > 1e5 else limit,
            "samples": len(mhz), "driver_max_mhz": first_clk.get("max_clk"),
            "locked": first_clk.get("clk_locked"), "pinned": False,
            "note": "sampled over the second of two seconds of the same steps run back to back "
                    "after the timed ones; peaks are quoted at 2400 MHz; clocks cannot be pinned without root"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(q, k, v, fw, heads):
    """The fp64 oracle, as it stands, timed on the host over a bounded sample:
    `heads` of the forward workload's heads, scaled to TFLOP/s with the same
    per-head FLOP count the GPU figure uses."""
    import numpy as np
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    qs = q[:, :heads].float().cpu().numpy().astype(np.float64)
    ks = k[:, :heads].float().cpu().numpy().astype(np.float64)
    vs = v[:, :heads].float().cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    oracle.forward(qs, ks, vs, fw["scale"], True)
    dt = time.perf_counter() - t0
    flops = 4.0 * heads * fw["Nq"] * fw["Nk"] * fw["d"] / 2.0
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": cores,
        "os_cpu_count": os.cpu_count(),
        "cpu_model": _cpu_model(),
        "blas_threads": cores,
        "kind": "oracle",
        "sample": f"{heads} of {fw['H']} heads of causal_bf16_b1_h32_n8192_d128 "
                  f"(fp64 numpy, materialised S and P), {dt:.1f} s",
    }


if __name__ == "__main__":
    sys.exit(main())
