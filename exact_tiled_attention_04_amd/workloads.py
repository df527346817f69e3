"""Seeded synthetic inputs shared by the HIP path's tests, the benchmark and
the oracle's checks.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic.  Every draw is standard normal in float32 from a torch
generator seeded explicitly, then rounded to the storage dtype with torch's
round-to-nearest-even cast.  Draw order follows the worked example of "Flash
attention and IO-aware attention" (aigrafen.se, the Python listing's
verification step): seed, then Q, K, V in that order, one tensor after the
other; dO (backward) and the decode extras come after.

The shapes are the pages' workloads: prefill tensors are [B, H, N, d]
contiguous; the paged cache is [num_blocks, block_size, Hkv, d] with the
block table assigning each sequence a slice of a seeded random permutation of
the physical blocks ("Modern attention kernels", "Paged attention changes
addressing").
"""

import math

import torch

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name):
    """Storage dtype for a dtype tag ("f32" or "bf16")."""
    try:
        return _DTYPES[name]
    except KeyError:
        raise ValueError(f"unknown dtype tag {name!r}") from None


def _generator(seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _randn(shape, dtype, gen, device, chunk_elems=1 << 28):
    """N(0, 1) float32 draws cast to ``dtype``; large tensors in chunks."""
    numel = math.prod(shape)
    out = torch.empty(numel, dtype=dtype, device=device)
    for start in range(0, numel, chunk_elems):
        stop = min(numel, start + chunk_elems)
        draw = torch.randn(stop - start, generator=gen, dtype=torch.float32,
                           device=device)
        out[start:stop] = draw.to(dtype)
    return out.view(*shape)


def prefill(B, H, Hkv, Nq, Nk, d, dtype="bf16", seed=0, device="cpu"):
    """Q [B,H,Nq,d], K and V [B,Hkv,Nk,d], drawn in the order Q, K, V."""
    dt = torch_dtype(dtype)
    gen = _generator(seed, device)
    q = _randn((B, H, Nq, d), dt, gen, device)
    k = _randn((B, Hkv, Nk, d), dt, gen, device)
    v = _randn((B, Hkv, Nk, d), dt, gen, device)
    return q, k, v


def backward(B, H, Hkv, Nq, Nk, d, dtype="bf16", seed=0, device="cpu"):
    """Q, K, V as :func:`prefill`, then dO [B,H,Nq,d] from the same stream."""
    dt = torch_dtype(dtype)
    gen = _generator(seed, device)
    q = _randn((B, H, Nq, d), dt, gen, device)
    k = _randn((B, Hkv, Nk, d), dt, gen, device)
    v = _randn((B, Hkv, Nk, d), dt, gen, device)
    do = _randn((B, H, Nq, d), dt, gen, device)
    return q, k, v, do


def decode(num_seqs, Hq, Hkv, d, ctx_lo, ctx_hi, block_size=16,
           max_blocks_per_seq=None, dtype="bf16", seed=0, device="cpu",
           context_lens=None, poison_tail=False, extra_blocks=0):
    """Paged decode workload.

    Draw order (one CPU generator for the integer structure, one generator on
    ``device`` for the values, both from ``seed``): context lengths uniform in
    [ctx_lo, ctx_hi] (unless given), the permutation of physical blocks, then
    Q [num_seqs, Hq, d], K cache and V cache [P, block_size, Hkv, d].

    Sequence s owns perm[off_s : off_s + ceil(ctx_s / block_size)] in logical
    order, with off_s the running total; unused table entries are -1.
    ``extra_blocks`` adds physical blocks no sequence uses.  With
    ``poison_tail`` the slots past each sequence's last token in its last page
    hold NaN, so any read of them that reaches the result shows up.

    Returns a dict with q, k_cache, v_cache (on ``device``), block_table,
    context_lens (int32, CPU), and the sizes used.
    """
    cpu_gen = _generator(seed, "cpu")
    if context_lens is None:
        ctx = torch.randint(ctx_lo, ctx_hi + 1, (num_seqs,), generator=cpu_gen,
                            dtype=torch.int64)
    else:
        ctx = torch.as_tensor(context_lens, dtype=torch.int64).clone()
        if ctx.numel() != num_seqs:
            raise ValueError("context_lens must have num_seqs entries")
    pages = [(max(int(c), 0) + block_size - 1) // block_size for c in ctx]
    total_pages = sum(pages) + int(extra_blocks)
    need = max(pages) if pages else 0
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(need, 1)
    if need > max_blocks_per_seq:
        raise ValueError("max_blocks_per_seq is smaller than the longest context")
    perm = torch.randperm(max(total_pages, 1), generator=cpu_gen)[:total_pages]
    table = torch.full((num_seqs, max_blocks_per_seq), -1, dtype=torch.int32)
    off = 0
    for s, n in enumerate(pages):
        table[s, :n] = perm[off:off + n].to(torch.int32)
        off += n

    dt = torch_dtype(dtype)
    gen = _generator(seed, device)
    q = _randn((num_seqs, Hq, d), dt, gen, device)
    nblk = max(total_pages, 1)
    k_cache = _randn((nblk, block_size, Hkv, d), dt, gen, device)
    v_cache = _randn((nblk, block_size, Hkv, d), dt, gen, device)
    if poison_tail:
        for s, c in enumerate(ctx.tolist()):
            if c <= 0 or c % block_size == 0:
                continue
            last = int(table[s, (c - 1) // block_size])
            k_cache[last, c % block_size:] = float("nan")
            v_cache[last, c % block_size:] = float("nan")
    return {
        "q": q,
        "k_cache": k_cache,
        "v_cache": v_cache,
        "block_table": table,
        "context_lens": ctx.to(torch.int32),
        "num_seqs": num_seqs,
        "Hq": Hq,
        "Hkv": Hkv,
        "d": d,
        "block_size": block_size,
        "max_blocks_per_seq": max_blocks_per_seq,
        "max_context": int(ctx.max()) if num_seqs else 0,
        "num_blocks": nblk,
    }


def _offsets(lengths):
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if len(lengths):
        cu[1:] = torch.cumsum(torch.as_tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return cu


def ragged(q_lens, k_lens, H, Hkv, d, dtype="bf16", seed=0, device="cpu"):
    """Packed ragged batch: Q [sum q_lens, H, d], then K and V
    [sum k_lens, Hkv, d] (drawn in that order), with the int32 row offsets
    cu_q, cu_k [num_seqs + 1] (CPU)."""
    dt = torch_dtype(dtype)
    gen = _generator(seed, device)
    tq, tk = int(sum(q_lens)), int(sum(k_lens))
    q = _randn((tq, H, d), dt, gen, device)
    k = _randn((tk, Hkv, d), dt, gen, device)
    v = _randn((tk, Hkv, d), dt, gen, device)
    return {"q": q, "k": k, "v": v, "cu_q": _offsets(q_lens), "cu_k": _offsets(k_lens),
            "max_q": max(int(x) for x in q_lens) if len(q_lens) else 0}


def ragged_lengths(num_seqs, lo, hi, seed=0):
    """num_seqs lengths uniform in [lo, hi] from a seeded CPU generator."""
    gen = _generator(seed, "cpu")
    return torch.randint(lo, hi + 1, (num_seqs,), generator=gen).tolist()


def paged_prefill(q_lens, k_lens, Hq, Hkv, d, block_size=16, dtype="bf16", seed=0,
                  device="cpu", poison=False, extra_blocks=0):
    """Chunked-prefill workload: sequence s has k_lens[s] cached tokens (its
    q_lens[s] new ones last) in a paged cache laid out as for :func:`decode`.

    Draw order: the permutation of physical blocks (CPU generator), then Q
    [sum q_lens, Hq, d], K cache, V cache.  With ``poison`` the slots past
    each context and every block no sequence uses hold NaN.
    Returns q, k_cache, v_cache (on ``device``), block_table, cu_q, seqlens_k
    (int32, CPU) and the sizes used.
    """
    cpu_gen = _generator(seed, "cpu")
    pages = [(max(int(c), 0) + block_size - 1) // block_size for c in k_lens]
    total_pages = sum(pages) + int(extra_blocks)
    nblk = max(total_pages, 1)
    perm = torch.randperm(nblk, generator=cpu_gen)
    table = torch.full((len(k_lens), max(max(pages) if pages else 1, 1)), -1, dtype=torch.int32)
    off = 0
    for s, n in enumerate(pages):
        table[s, :n] = perm[off:off + n].to(torch.int32)
        off += n
    dt = torch_dtype(dtype)
    gen = _generator(seed, device)
    q = _randn((int(sum(q_lens)), Hq, d), dt, gen, device)
    k_cache = _randn((nblk, block_size, Hkv, d), dt, gen, device)
    v_cache = _randn((nblk, block_size, Hkv, d), dt, gen, device)
    if poison:
        used = torch.zeros(nblk, dtype=torch.bool)
        for s, c in enumerate(k_lens):
            n = pages[s]
            used[table[s, :n].long()] = True
            if c > 0 and c % block_size:
                last = int(table[s, (c - 1) // block_size])
                k_cache[last, c % block_size:] = float("nan")
                v_cache[last, c % block_size:] = float("nan")
        idle = (~used).nonzero().flatten().to(k_cache.device)
        k_cache[idle] = float("nan")
        v_cache[idle] = float("nan")
    return {"q": q, "k_cache": k_cache, "v_cache": v_cache, "block_table": table,
            "cu_q": _offsets(q_lens), "seqlens_k": torch.as_tensor(k_lens, dtype=torch.int32),
            "max_q": max(int(x) for x in q_lens), "num_blocks": nblk, "block_size": block_size}


def serving_prefill(num_seqs, q_lo, q_hi, ctx_lo, ctx_hi, Hq, Hkv, d, block_size=16,
                    dtype="bf16", seed=0, device="cpu"):
    """Chunked prefill of a serving batch: new-token counts uniform in
    [q_lo, q_hi] (seed + 1), prior cached context uniform in [ctx_lo, ctx_hi]
    (seed + 2); each sequence's context is prior + new tokens, then
    :func:`paged_prefill` with ``seed``."""
    q_lens = ragged_lengths(num_seqs, q_lo, q_hi, seed=seed + 1)
    prior = ragged_lengths(num_seqs, ctx_lo, ctx_hi, seed=seed + 2)
    k_lens = [q + p for q, p in zip(q_lens, prior)]
    w = paged_prefill(q_lens, k_lens, Hq, Hkv, d, block_size=block_size, dtype=dtype, seed=seed,
                      device=device)
    w["q_lens"], w["k_lens"] = q_lens, k_lens
    return w


def block_sparse_index(n_layouts, n_qblocks, n_kblocks, local, n_global, density, seed=0):
    """CSR block index of a synthetic local + global + random pattern ([AK]
    sparse-attention paragraph: sliding windows, global plus local patterns).

    Query block r (bottom-right aligned onto key block c_r = r + n_kblocks -
    n_qblocks) lists key blocks c_r - local + 1 .. c_r, the first ``n_global``
    blocks, and every other block with probability ``density`` (seeded CPU
    draws, one per candidate).  Returns row_ptr int32 [n_layouts,
    n_qblocks + 1] (offsets into the shared col_idx) and col_idx int32.
    """
    gen = _generator(seed, "cpu")
    row_ptr = torch.zeros((n_layouts, n_qblocks + 1), dtype=torch.int32)
    cols = []
    for lay in range(n_layouts):
        draws = torch.rand((n_qblocks, n_kblocks), generator=gen)
        for r in range(n_qblocks):
            row_ptr[lay, r] = len(cols)
            diag = r + n_kblocks - n_qblocks
            for c in range(n_kblocks):
                near = diag - local < c <= diag
                if near or c < n_global or draws[r, c] < density:
                    cols.append(c)
        row_ptr[lay, n_qblocks] = len(cols)
    return row_ptr, torch.as_tensor(cols, dtype=torch.int32)


# The five workloads the pages' shapes call for (name -> keyword arguments).
WORKLOADS = {
    "single_head_f32_n512_d64": dict(
        kind="fwd", B=1, H=1, Hkv=1, Nq=512, Nk=512, d=64, dtype="f32",
        causal=False, scale=1.0 / 8.0, seed=0),
    "causal_bf16_b4_h16_n2048_d64": dict(
        kind="fwd", B=4, H=16, Hkv=16, Nq=2048, Nk=2048, d=64, dtype="bf16",
        causal=True, scale=1.0 / 8.0, seed=0),
    "causal_bf16_b1_h32_n8192_d128": dict(
        kind="fwd", B=1, H=32, Hkv=32, Nq=8192, Nk=8192, d=128, dtype="bf16",
        causal=True, scale=1.0 / math.sqrt(128.0), seed=0),
    "noncausal_bf16_b1_h32_n8192_d128": dict(
        kind="fwd", B=1, H=32, Hkv=32, Nq=8192, Nk=8192, d=128, dtype="bf16",
        causal=False, scale=1.0 / math.sqrt(128.0), seed=0),
    "causal_bf16_b1_h4_n8192_d128": dict(
        kind="fwd", B=1, H=4, Hkv=4, Nq=8192, Nk=8192, d=128, dtype="bf16",
        causal=True, scale=1.0 / math.sqrt(128.0), seed=0),
    "paged_gqa_decode_bf16_s64_hq32_hkv8_d128": dict(
        kind="decode", num_seqs=64, Hq=32, Hkv=8, d=128, ctx_lo=4096,
        ctx_hi=32768, block_size=16, max_blocks_per_seq=2048, dtype="bf16",
        scale=1.0 / math.sqrt(128.0), seed=0),
    # Rows beyond the five configurations: the serving-engine combination and
    # sparse visitation ("Modern attention kernels", "Paged attention changes
    # addressing"), shaped like the decode and long-prefill workloads.
    "varlen_causal_bf16_s16_h32_hkv8_d128": dict(
        kind="varlen", num_seqs=16, len_lo=512, len_hi=8192, H=32, Hkv=8, d=128,
        dtype="bf16", causal=True, scale=1.0 / math.sqrt(128.0), seed=0),
    "paged_prefill_causal_bf16_s16_hq32_hkv8_d128": dict(
        kind="paged_prefill", num_seqs=16, q_lo=512, q_hi=2048, ctx_lo=2048, ctx_hi=8192,
        Hq=32, Hkv=8, d=128, block_size=16, dtype="bf16", causal=True,
        scale=1.0 / math.sqrt(128.0), seed=0),
    "block_sparse_causal_bf16_b1_h32_n8192_d128": dict(
        kind="block_sparse", B=1, H=32, Hkv=32, N=8192, d=128, layouts=32, local=4,
        n_global=1, density=0.1, dtype="bf16", causal=True, scale=1.0 / math.sqrt(128.0),
        seed=0),
    "causal_bwd_bf16_b2_h16_n4096_d128": dict(
        kind="bwd", B=2, H=16, Hkv=16, Nq=4096, Nk=4096, d=128, dtype="bf16",
        causal=True, scale=1.0 / math.sqrt(128.0), seed=0),
}
