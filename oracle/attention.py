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


def forward_probs(q, k, v, scale, causal, window=None):
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
    Returns O [B, H, Nq, d], LSE [B, H, Nq], P [B, H, Nq, Nk], all float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    group = _check_shapes(q, k, v)
    bsz, nh, nq, d = q.shape
    nk = k.shape[2]
    vis = _visible(nq, nk, causal, window)

    out = np.zeros((bsz, nh, nq, d))
    lse = np.full((bsz, nh, nq), -np.inf)
    probs = np.zeros((bsz, nh, nq, nk))
    for b in range(bsz):
        for h in range(nh):
            g = h // group
            s = scale * (q[b, h] @ k[b, g].T)
            s = np.where(vis, s, -np.inf)
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


def forward(q, k, v, scale, causal, window=None):
    """(O, LSE) of :func:`forward_probs`."""
    out, lse, _ = forward_probs(q, k, v, scale, causal, window)
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
            g = h // group
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


def brute_force_forward(q, k, v, scale, causal, window=None):
    """Scalar pure-Python attention for tiny inputs (N <= 8, d <= 8).

    A second evaluation of the same definition with no numpy arithmetic:
    nested loops, math.exp, and a max taken over the visible keys only (the
    visibility test written out again, not shared with ``_visible``).
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
