"""Plain fp64 definitions of exact attention (forward, paged decode, backward).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Nothing here is
blocked, fused or reordered: each function materialises the full score matrix
S and probability matrix P for one (batch, head) at a time, exactly as the
definition reads, so it can be compared with the pages by eye.

Sources (web pages, cited by title and section):
  [MAK] "Modern attention kernels" (blog.ecitis.org)
  [FAV] "Flash attention", AI engineering visualised (understandingdata.com)
  [FIO] "Flash attention and IO-aware attention" (aigrafen.se)
  [AK]  "Attention kernels" (inference.tusharamrit.in)

Conventions that the pages leave open (each also listed with its reason in the
design notes):
  * causal alignment is bottom-right: query row i sits at absolute position
    i + (Nk - Nq) and may see key j iff j <= i + (Nk - Nq); with Nq == Nk this
    is the usual lower triangle, and a single query sees the whole cache;
  * a row with no visible key has O = 0 and LSE = -inf;
  * the saved statistic is the natural-log log-sum-exp, LSE = m + ln(l);
  * grouped-query heads map contiguously: query head h reads KV head
    h // (H / Hkv).
"""

import math

import numpy as np


def _visible(nq, nk, causal, window=None):
    """Boolean [nq, nk] visibility of key j from query row i.

    [MAK] "Kernel structure": causal attention hides every key after the
    query's own position; bottom-right aligned as stated in the module notes.
    The same section says local attention changes the range of keys a query
    visits, and [AK]'s sparse-attention paragraph names the sliding window
    (each position sees a fixed number of recent positions).  ``window`` =
    (left, right) keeps key j only if p - left <= j <= p + right, where p is
    the row's bottom-right aligned position; either side may be None
    (unbounded).  A sliding window of W keys is (W - 1, 0).  The window and the
    causal mask combine by intersection.
    """
    row_pos = np.arange(nq)[:, None] + (nk - nq)
    col = np.arange(nk)[None, :]
    vis = np.ones((nq, nk), dtype=bool)
    if causal:
        vis &= col <= row_pos
    if window is not None:
        left, right = window
        if left is not None:
            vis &= col >= row_pos - left
        if right is not None:
            vis &= col <= row_pos + right
    return vis


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d] arrays")
    b, h, _, d = q.shape
    bk, hkv, nk, dk = k.shape
    if bk != b or dk != d or v.shape != k.shape:
        raise ValueError("k and v must be [B, Hkv, Nk, d] with q's B and d")
    if hkv < 1 or h % hkv != 0:
        raise ValueError("H must be a multiple of Hkv")
    return h // hkv


def kv_head(h, n_heads, n_kv):
    """KV head read by query head h, with n_heads query heads over n_kv KV
    heads.  [AK]'s grouped-query paragraph has several query heads share one
    KV head without saying which; the groups are taken contiguous: heads
    h = g * G .. g * G + G - 1 read KV head g, G = n_heads / n_kv."""
    return h // (n_heads // n_kv)


def forward_probs(q, k, v, scale, causal, window=None, mask=None):
    """Materialised attention: returns (O, LSE, P).

    [MAK] "Standard attention materializes quadratic state":
        S = scale * Q K^T,  P = softmax(S) row-wise,  O = P V.
    The softmax is the safe form of [AK] (online-softmax derivation, "standard
    safe softmax"): subtract the row maximum m, exponentiate, sum to l, divide.
    The masked entries are -inf before the softmax, so they get probability
    exactly 0.  LSE = m + ln(l) ([FIO] backward paragraph saves m and l per
    row; one natural-log number carries both).

    q: [B, H, Nq, d]; k, v: [B, Hkv, Nk, d] (any float dtype, computed in fp64).
    window: optional (left, right) local-attention band, see ``_visible``.
    mask: optional boolean array broadcastable to [B, H, Nq, Nk]; True keeps
    the pair.  It is intersected with the causal/window visibility (an
    arbitrary sparse mask, [MAK] "Kernel structure").
    Returns O [B, H, Nq, d], LSE [B, H, Nq], P [B, H, Nq, Nk], all float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    group = _check_shapes(q, k, v)
    bsz, nh, nq, d = q.shape
    nk = k.shape[2]
    vis_all = np.broadcast_to(_visible(nq, nk, causal, window), (bsz, nh, nq, nk))
    if mask is not None:
        vis_all = vis_all & np.broadcast_to(np.asarray(mask, dtype=bool), (bsz, nh, nq, nk))

    out = np.zeros((bsz, nh, nq, d))
    lse = np.full((bsz, nh, nq), -np.inf)
    probs = np.zeros((bsz, nh, nq, nk))
    for b in range(bsz):
        for h in range(nh):
            g = kv_head(h, nh, nh // group)
            s = scale * (q[b, h] @ k[b, g].T)
            s = np.where(vis_all[b, h], s, -np.inf)
            m = s.max(axis=1) if nk > 0 else np.full(nq, -np.inf)
            live = np.isfinite(m)
            e = np.zeros_like(s)
            e[live] = np.exp(s[live] - m[live, None])
            ell = e.sum(axis=1)
            p = np.zeros_like(s)
            p[live] = e[live] / ell[live, None]
            probs[b, h] = p
            out[b, h] = p @ v[b, g]
            lse[b, h, live] = m[live] + np.log(ell[live])
    return out, lse, probs


def forward(q, k, v, scale, causal, window=None, mask=None):
    """(O, LSE) of :func:`forward_probs`."""
    if mask is None:
        out, lse, _ = forward_probs(q, k, v, scale, causal, window)
    else:
        out, lse, _ = forward_probs(q, k, v, scale, causal, window, mask=mask)
    return out, lse


def backward(q, k, v, do, scale, causal, window=None):
    """Gradients of L = sum(O * dO) with respect to Q, K, V.

    [MAK] "Backward pass recomputes scores" and [FIO]'s backward paragraph
    state that the backward needs P again; the pages do not print the
    gradient formulas, so this is the textbook chain rule through
    S = scale Q K^T, P = softmax(S), O = P V:
        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij
        dS = P * (dP - D)          (softmax Jacobian, row by row)
        dQ = scale * dS K
        dK = scale * dS^T Q
    For grouped-query heads, dK and dV of a KV head are the sums over the
    query heads that read it.  P is recomputed here from the definition
    (``forward_probs``), never taken from the device.

    Returns dQ [B, H, Nq, d], dK and dV [B, Hkv, Nk, d] in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    group = _check_shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have Q's shape")
    _, _, p_all = forward_probs(q, k, v, scale, causal, window)
    bsz, nh, _, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(bsz):
        for h in range(nh):
            g = kv_head(h, nh, nh // group)
            p = p_all[b, h]
            dv[b, g] += p.T @ do[b, h]
            dp = do[b, h] @ v[b, g].T
            dsum = (p * dp).sum(axis=1)
            ds = p * (dp - dsum[:, None])
            dq[b, h] = scale * (ds @ k[b, g])
            dk[b, g] += scale * (ds.T @ q[b, h])
    return dq, dk, dv


def gather_paged(cache, block_table, seq, ctx):
    """Contiguous [ctx, Hkv, d] view of one sequence's paged cache rows.

    [MAK] "Paged attention changes addressing": token position pos lives in
    logical block pos // block_size at offset pos % block_size, and the
    sequence's block table maps the logical block to a physical one.
    cache: [num_blocks, block_size, Hkv, d]; block_table: [num_seqs, max_blocks].
    """
    cache = np.asarray(cache)
    block_size = cache.shape[1]
    pos = np.arange(ctx)
    logical = pos // block_size
    offset = pos % block_size
    physical = np.asarray(block_table)[seq, logical]
    if ctx and (physical.min() < 0 or physical.max() >= cache.shape[0]):
        raise ValueError("block table entry out of range for a live token")
    return cache[physical, offset]


def decode_paged(q, k_cache, v_cache, block_table, context_lens, scale):
    """Single-query attention per sequence over a paged KV cache.

    [MAK] "Prefill and decode need different kernels": one query position
    per sequence against its whole cache; "Paged attention changes
    addressing" for the gather; [AK]'s grouped-query paragraph for the
    sharing of one KV head by several query heads.  After the gather this is
    ``forward`` with Nq = 1 and no mask.

    q: [num_seqs, Hq, d]; k_cache, v_cache: [num_blocks, block_size, Hkv, d];
    block_table: int [num_seqs, max_blocks]; context_lens: int [num_seqs].
    Returns O [num_seqs, Hq, d], LSE [num_seqs, Hq] in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    nseq, hq, d = q.shape
    out = np.zeros((nseq, hq, d))
    lse = np.full((nseq, hq), -np.inf)
    for s in range(nseq):
        ctx = int(context_lens[s])
        if ctx <= 0:
            continue
        ks = gather_paged(k_cache, block_table, s, ctx).astype(np.float64)
        vs = gather_paged(v_cache, block_table, s, ctx).astype(np.float64)
        ks = ks.transpose(1, 0, 2)[None]  # [1, Hkv, ctx, d]
        vs = vs.transpose(1, 0, 2)[None]
        o, l_ = forward(q[s][None, :, None, :], ks, vs, scale, causal=False)
        out[s] = o[0, :, 0, :]
        lse[s] = l_[0, :, 0]
    return out, lse


def prefill_ragged(q, k, v, cu_q, cu_k, scale, causal, window=None):
    """Forward over a ragged batch of sequences in packed layout.

    [MAK] "Numerical validation" lists ragged sequence boundaries among the
    cases a fused kernel must get right; a serving engine ("Paged attention
    changes addressing", last paragraph) runs tiled prefill over many
    sequences of different lengths at once.  Each sequence is an independent
    attention problem: sequence s owns query rows cu_q[s] .. cu_q[s+1] - 1 and
    key rows cu_k[s] .. cu_k[s+1] - 1, and this is ``forward`` applied to each
    slice (bottom-right causal alignment within the sequence).

    q: [total_q, H, d]; k, v: [total_k, Hkv, d]; cu_q, cu_k: [num_seqs + 1]
    non-decreasing offsets starting at 0.
    Returns O [total_q, H, d] and LSE [H, total_q], float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    total_q, nh, d = q.shape
    out = np.zeros((total_q, nh, d))
    lse = np.full((nh, total_q), -np.inf)
    for s in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        if q1 <= q0:
            continue
        qs = q[q0:q1].transpose(1, 0, 2)[None]
        ks = k[k0:k1].transpose(1, 0, 2)[None]
        vs = v[k0:k1].transpose(1, 0, 2)[None]
        o, l_ = forward(qs, ks, vs, scale, causal, window)
        out[q0:q1] = o[0].transpose(1, 0, 2)
        lse[:, q0:q1] = l_[0]
    return out, lse


def prefill_paged(q, k_cache, v_cache, block_table, cu_q, seqlens_k, scale, causal,
                  window=None):
    """Ragged prefill whose keys and values live in a paged cache.

    The combination a serving engine runs ([MAK] "Paged attention changes
    addressing", last paragraph): sequence s has seqlens_k[s] tokens in the
    cache, gathered through its block table exactly as for decode, and its
    cu_q[s+1] - cu_q[s] query rows are the LAST positions of that context
    (a prefill chunk whose keys were already appended), bottom-right aligned.
    With one query row this is ``decode_paged``; with as many rows as
    tokens it is a full prefill.

    q: [total_q, Hq, d]; caches [num_blocks, block_size, Hkv, d]; block_table
    [num_seqs, max_blocks]; cu_q [num_seqs + 1]; seqlens_k [num_seqs].
    Returns O [total_q, Hq, d] and LSE [Hq, total_q], float64.
    """
    q = np.asarray(q, dtype=np.float64)
    cu_q = [int(x) for x in cu_q]
    total_q, nh, d = q.shape
    out = np.zeros((total_q, nh, d))
    lse = np.full((nh, total_q), -np.inf)
    for s in range(len(cu_q) - 1):
        q0, q1 = cu_q[s], cu_q[s + 1]
        ctx = max(int(seqlens_k[s]), 0)
        if q1 <= q0:
            continue
        ks = gather_paged(k_cache, block_table, s, ctx).astype(np.float64)
        vs = gather_paged(v_cache, block_table, s, ctx).astype(np.float64)
        qs = q[q0:q1].transpose(1, 0, 2)[None]
        o, l_ = forward(qs, ks.transpose(1, 0, 2)[None], vs.transpose(1, 0, 2)[None], scale,
                        causal, window)
        out[q0:q1] = o[0].transpose(1, 0, 2)
        lse[:, q0:q1] = l_[0]
    return out, lse


def block_mask_from_index(row_ptr, col_idx, n_qblocks, n_kblocks):
    """Dense boolean [L, n_qblocks, n_kblocks] block matrix of a CSR block index.

    [MAK] "Kernel structure": an arbitrary sparse mask needs an index
    structure that tells the kernel which blocks exist.  Here layout l lists,
    for query block r, the key blocks col_idx[row_ptr[l, r] : row_ptr[l, r+1]].
    row_ptr: [L, n_qblocks + 1] offsets into col_idx (int).
    """
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    n_layouts = row_ptr.shape[0]
    blocks = np.zeros((n_layouts, n_qblocks, n_kblocks), dtype=bool)
    for lay in range(n_layouts):
        for r in range(n_qblocks):
            for c in col_idx[row_ptr[lay, r]:row_ptr[lay, r + 1]]:
                blocks[lay, r, c] = True
    return blocks


def block_sparse_forward(q, k, v, scale, causal, blocks, block_q, block_k):
    """Attention restricted to the listed score blocks ([MAK] "Kernel
    structure", sparse masks; "Paged attention changes addressing": sparse
    attention visits selected score blocks).

    blocks: boolean [L, ceil(Nq / block_q), ceil(Nk / block_k)]; (batch b,
    head h) uses layout (b * H + h) % L.  Query row i may see key j iff block
    (i // block_q, j // block_k) is listed, intersected with the causal mask
    when ``causal``.  This is ``forward`` with that boolean mask.
    """
    blocks = np.asarray(blocks, dtype=bool)
    bsz, nh, nq, _ = np.shape(q)
    nk = np.shape(k)[2]
    n_layouts = blocks.shape[0]
    rows = np.arange(nq) // block_q
    cols = np.arange(nk) // block_k
    mask = np.zeros((bsz, nh, nq, nk), dtype=bool)
    for b in range(bsz):
        for h in range(nh):
            mask[b, h] = blocks[(b * nh + h) % n_layouts][rows[:, None], cols[None, :]]
    return forward(q, k, v, scale, causal, mask=mask)


def brute_force_forward(q, k, v, scale, causal, window=None, allowed=None):
    """Scalar pure-Python attention for tiny inputs (N <= 8, d <= 8).

    A second evaluation of the same definition with no numpy arithmetic:
    nested loops, math.exp, and a max taken over the visible keys only (the
    visibility test written out again, not shared with ``_visible``).
    ``allowed(b, h, i, j)``, if given, is an extra predicate a pair must pass.
    Inputs are nested lists or arrays; returns nested lists O, LSE.
    """
    left, right = window if window is not None else (None, None)
    q = np.asarray(q, dtype=np.float64).tolist()
    k = np.asarray(k, dtype=np.float64).tolist()
    v = np.asarray(v, dtype=np.float64).tolist()
    bsz, nh = len(q), len(q[0])
    nq, d = len(q[0][0]), len(q[0][0][0])
    hkv, nk = len(k[0]), len(k[0][0])
    group = nh // hkv
    out = [[[[0.0] * d for _ in range(nq)] for _ in range(nh)] for _ in range(bsz)]
    lse = [[[-math.inf] * nq for _ in range(nh)] for _ in range(bsz)]
    for b in range(bsz):
        for h in range(nh):
            g = h // group
            for i in range(nq):
                scores = []
                for j in range(nk):
                    pos = i + (nk - nq)
                    if causal and j > pos:
                        continue
                    if left is not None and j < pos - left:
                        continue
                    if right is not None and j > pos + right:
                        continue
                    if allowed is not None and not allowed(b, h, i, j):
                        continue
                    dot = 0.0
                    for c in range(d):
                        dot += q[b][h][i][c] * k[b][g][j][c]
                    scores.append((j, scale * dot))
                if not scores:
                    continue
                top = max(sc for _, sc in scores)
                weights = [(j, math.exp(sc - top)) for j, sc in scores]
                total = sum(w for _, w in weights)
                for c in range(d):
                    acc = 0.0
                    for j, w in weights:
                        acc += w * v[b][g][j][c]
                    out[b][h][i][c] = acc / total
                lse[b][h][i] = top + math.log(total)
    return out, lse


def brute_force_backward_dv(p, do):
    """dV = P^T dO for one head with scalar loops (tiny inputs only)."""
    p = np.asarray(p, dtype=np.float64).tolist()
    do = np.asarray(do, dtype=np.float64).tolist()
    nq, nk, d = len(p), len(p[0]), len(do[0])
    dv = [[0.0] * d for _ in range(nk)]
    for j in range(nk):
        for c in range(d):
            acc = 0.0
            for i in range(nq):
                acc += p[i][j] * do[i][c]
            dv[j][c] = acc
    return dv
