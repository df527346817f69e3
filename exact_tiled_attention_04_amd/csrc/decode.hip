// Paged grouped-query decode attention with a split-context merge (gfx950).
//
// Method: "Modern attention kernels", sections "Prefill and decode need
// different kernels" (one query per sequence, coalesced cache reads,
// parallel reduction over the context, grouped-query sharing, block
// indirection, many sequences per launch) and "Paged attention changes
// addressing" (logical block = pos / block_size, offset = pos % block_size,
// physical block from the sequence's block table); "Attention kernels",
// FlashDecoding paragraph (split the context into chunks, each chunk yields
// an unnormalised partial output with its max and sum, partials combined by
// the online-softmax rescaling) and its grouped-query paragraph (the query
// heads sharing one KV head read it once).
//
// Split kernel: one wave per (sequence, KV head, context chunk).  The G query
// heads of the group are the columns of a 16x16x32 MFMA (G <= 16), so every
// K and V byte is read from HBM once and used by all G heads.  Per 32 tokens
// (two 16-token groups): K rows go straight from HBM into MFMA A-operand
// registers (S^T = K Q^T); V rows are staged in a wave-private LDS tile and
// read transposed (ds_read_b64_tr_b16) as the A operand of o^T += V^T P^T.
// Block sizes that are multiples of 16 take a path with wave-uniform page
// addressing through buffer resources; other block sizes look each token's
// page up per lane.
// The next 32 tokens are fetched while the current ones are computed.
// Tokens past the context (poisoned or stale page slots) never reach the
// result: their scores are replaced by -inf and their V rows by zeros.
//
// Merge kernel: one workgroup per (query head, sequence), one thread per
// output column: M = max_c m_c, w_c = 2^(m_c - M), l = sum w_c l_c,
// O = sum w_c o_c / l, LSE = (M + log2 l) ln 2.
#include "common.hpp"
#include "kernels.hpp"

namespace eta {

namespace {

constexpr int kTok = 32;  // tokens per inner step (two 16-token pages)
// Longest context chunk one split wave handles (its block-table entries are
// held in four registers: 256 pages of >= 16 tokens).
constexpr int kMaxChunk = 4064;

// Two waves per SIMD (eight per CU), each with the next 32 tokens' K and V
// in flight: enough bytes outstanding to cover HBM latency without spills.
#ifndef ETA_DECODE_WAVES_PER_EU
#define ETA_DECODE_WAVES_PER_EU 2
#endif

// Block sizes that are multiples of 16: each 16-token group of a step lies in
// one page, so its location is wave-uniform.  A group is addressed through a
// raw buffer resource whose base is the group's first cache row and whose
// range ends after its last live token (zero when the group is past the
// chunk or its block-table entry lies outside the cache): K and V rows past
// the context, or of a bad page, arrive as zeros with no branches, and the
// score mask is a compare with the group's live-token count.
#ifndef ETA_DECODE_WG_WAVES
#define ETA_DECODE_WG_WAVES 4
#endif

// Work order of the split kernels.  Work items enumerate the live chunks
// only: first every sequence's full chunks (sequence by sequence), then the
// shorter last chunks of the sequences whose context is not a multiple of
// chunk_tokens, so the short items fill the end of the launch (longest work
// first).  A wave's slot id = item * Hkv + g.  The grid is sized for the
// largest possible count, so the live work is dispatched first and the
// surplus slots at the end exit at once (measured faster than a grid with
// dead slots interleaved through it).  The wave finds its sequence by an
// inclusive scan of the per-sequence counts of 64 sequences at a time.
// Returns g and sets s = -1 for a surplus slot.
__device__ __forceinline__ int live_item(int slot, int Hkv, const int* __restrict__ ctx_lens,
                                         int num_seqs, int max_context, int chunk_tokens,
                                         int lane, int& s_out, int& chunk_out) {
  int item = slot / Hkv;
  const int g = slot % Hkv;
  int s = -1, chunk = 0;
  for (int pass = 0; pass < 2 && s < 0; ++pass) {
    for (int base = 0; base < num_seqs; base += 64) {
      const int sq = base + lane;
      int nc = 0, full = 0;
      if (sq < num_seqs) {
        const int c = min(ctx_lens[sq], max_context);
        full = c > 0 ? c / chunk_tokens : 0;
        nc = pass == 0 ? full : (c > 0 && c % chunk_tokens != 0 ? 1 : 0);
      }
      int incl = nc;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
      }
      const unsigned long long hit = __ballot(incl > item);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        s = base + l;
        chunk = pass == 0 ? item - (__shfl(incl, l, 64) - __shfl(nc, l, 64)) : __shfl(full, l, 64);
        break;
      }
      item -= __shfl(incl, 63, 64);
    }
  }
  s_out = __builtin_amdgcn_readfirstlane(s);
  chunk_out = __builtin_amdgcn_readfirstlane(chunk);
  return g;
}

template <int D>
__global__ __launch_bounds__(64 * ETA_DECODE_WG_WAVES)
__attribute__((amdgpu_waves_per_eu(ETA_DECODE_WAVES_PER_EU)))
void decode_split_paged_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc, const __bf16* __restrict__ Vc,
    const int* __restrict__ block_table, const int* __restrict__ ctx_lens,
    float* __restrict__ part_o, float* __restrict__ part_ml, int num_seqs, int Hq, int Hkv,
    int G, int block_size, int num_blocks, int max_blocks, int max_context, int chunk_tokens,
    int n_chunks_max, long long block_stride, long long token_stride, long long head_stride,
    float scale_log2, unsigned page_magic, int page_shift) {
  constexpr int KS = D / 32;          // k-steps of S^T = K Q^T (32 d each)
  constexpr int NB = D / 16;          // 16-row blocks of o^T
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int VL = kTok * CH / 64;  // V loads per lane per step
  constexpr int TPI = 64 / CH;        // tokens per V load instruction

  __shared__ __attribute__((aligned(16))) __bf16 vs_all[ETA_DECODE_WG_WAVES][kTok * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int s, chunk;
  const int g = live_item(blockIdx.x * ETA_DECODE_WG_WAVES + wave, Hkv, ctx_lens, num_seqs,
                          max_context, chunk_tokens, lane, s, chunk);
  if (s < 0) return;
  const int ctx = min(ctx_lens[s], max_context);
  const int t_begin = chunk * chunk_tokens;
  if (t_begin >= ctx) return;
  const int t_end = min(ctx, t_begin + chunk_tokens);

  __bf16* vs = vs_all[wave];
  const int qc = lane & 15;   // query column (head within the group) / A row
  const int g4 = lane >> 4;   // 16-lane group

  bf16x8 qf[KS];
  {
    const bool ok = qc < G;
    const __bf16* src = Q + ((size_t)s * Hq + (size_t)g * G + (ok ? qc : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = ok ? *(const u32x4*)(src + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const int* bt = block_table + (size_t)s * max_blocks;
  const int ts2 = (int)(token_stride * 2);  // bytes between tokens
  // Per-lane byte offsets inside a 16-token group: the K row of token qc
  // (A operand, d = 32 ks + 8 g4 + e) and this lane's V chunk.
  const int koff = qc * ts2 + 16 * g4;
  const int voff = (lane / CH) * ts2 + (lane % CH) * 16;

  // The chunk's block-table entries (up to 4 * 64 logical pages, enough for
  // kMaxChunk tokens), one per lane of bt_r[i], loaded once: page lookups
  // are register reads (v_readlane), so no step waits on memory before it
  // can issue its K/V loads.
  const int bt_base = t_begin / block_size;
  int bt_r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lp = bt_base + 64 * i + lane;
    bt_r[i] = lp < max_blocks ? bt[lp] : -1;
  }
  auto page_of = [&](int logical) -> int {
    const int idx = logical - bt_base;  // 0 <= idx < 256 by the chunk limit
    const int r = idx >> 6, l = idx & 63;
    const int v = r == 0 ? bt_r[0] : r == 1 ? bt_r[1] : r == 2 ? bt_r[2] : bt_r[3];
    return __builtin_amdgcn_readlane(v, l);
  };

  struct Group {
    buf_rsrc k, v;
    int live;  // tokens of the group inside the chunk (0 if none or bad page)
  };
  // Everything about a group is wave-uniform; readfirstlane makes that
  // visible to the compiler so the buffer resources live in SGPRs.
  auto group = [&](int pos0) -> Group {
    int live = min(t_end - pos0, 16);
    live = live < 0 ? 0 : live;
    long long base = 0;
    if (live > 0) {
      const int logical = (int)(((unsigned long long)(unsigned)pos0 * page_magic) >> page_shift);
      const int slot0 = pos0 - logical * block_size;
      const int ph = page_of(logical);
      if (ph < 0 || ph >= num_blocks) live = 0;
      else
        base = (long long)ph * block_stride + (long long)slot0 * token_stride +
               (long long)g * head_stride;
    }
    live = __builtin_amdgcn_readfirstlane(live);
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)base);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)base >> 32));
    base = (long long)(((unsigned long long)hi << 32) | lo);
    Group r;
    r.k = make_rsrc(Kc + base, (unsigned)(live * ts2));
    r.v = make_rsrc(Vc + base, (unsigned)(live * ts2));
    r.live = live;
    return r;
  };

  u32x4 ka[2][KS], kb[2][KS], kc[2][KS], vr[VL];
  int la[2], lb[2], lc[2];
  auto load_k = [&](int t0, u32x4 (&kd)[2][KS], int (&live)[2]) {
    const Group g0 = group(t0), g1 = group(t0 + 16);
    live[0] = g0.live;
    live[1] = g1.live;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kd[0][ks] = buf_load16(g0.k, koff + 64 * ks, 0);
      kd[1][ks] = buf_load16(g1.k, koff + 64 * ks, 0);
    }
  };
  auto load_v = [&](int t0) {
    const Group g0 = group(t0), g1 = group(t0 + 16);
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int pp = (TPI * it) / 16;
      vr[it] = buf_load16(pp == 0 ? g0.v : g1.v, voff, (TPI * it - 16 * pp) * ts2);
    }
  };

  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto stage_v = [&]() {
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int cid = lane + 64 * it;
      const int tk = cid / CH;
      const int c = cid % CH;
      *(u32x4*)(vs + tk * D + ((c ^ decode_swz<D>(tk)) * 8)) = vr[it];
    }
  };
  auto compute_step = [&](u32x4 (&kd)[2][KS], int (&live)[2]) {
    f32x4 sc[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      sc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[pp] = mfma16(__builtin_bit_cast(bf16x8, kd[pp][ks]), qf[ks], sc[pp]);
    }
    // Lane (qc, g4) register r of sc[pp] is token 16 pp + 4 g4 + r of the step.
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g4 + r >= live[pp]) sc[pp][r] = -INFINITY;
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(__builtin_fmaf(sc[pp][r], scale_log2, -m_use));
        sc[pp][r] = p;
        rs += p;
      }
    l_run = alpha * l_run + rs;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[nb][r] *= alpha;
    u32x4 pw;
    pw[0] = pack_bf16x2(sc[0][0], sc[0][1]);
    pw[1] = pack_bf16x2(sc[0][2], sc[0][3]);
    pw[2] = pack_bf16x2(sc[1][0], sc[1][1]);
    pw[3] = pack_bf16x2(sc[1][2], sc[1][3]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
    const int src = lane & 15;
    const int tr_r = src >> 2;
    const int tr_c = src & 3;
    const int r1 = 4 * g4 + tr_r;
    const int r2 = r1 + 16;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = 16 * nb + 4 * tr_c;
      const int chunk8 = col >> 3;
      const int sub = col & 7;
      const s16x4 lo = lds_read_tr(vs + r1 * D + ((chunk8 ^ decode_swz<D>(r1)) * 8) + sub);
      const s16x4 hi = lds_read_tr(vs + r2 * D + ((chunk8 ^ decode_swz<D>(r2)) * 8) + sub);
      o[nb] = mfma16(join_tr(lo, hi), pb, o[nb]);
    }
    // The next step's LDS writes must follow these reads.
    __asm__ volatile("" ::: "memory");
  };

  // Software pipeline over 32-token steps: K is fetched two steps ahead
  // through a ring of three register sets, V one step ahead (its registers
  // are free once the current step is staged in LDS), so about 24 KiB per
  // wave stay in flight while a step is computed.
  auto iter = [&](int t0, u32x4 (&kcur)[2][KS], int (&lcur)[2], u32x4 (&kfar)[2][KS],
                  int (&lfar)[2]) -> bool {
    stage_v();
    if (t0 + kTok < t_end) load_v(t0 + kTok);
    if (t0 + 2 * kTok < t_end) load_k(t0 + 2 * kTok, kfar, lfar);
    compute_step(kcur, lcur);
    return t0 + kTok < t_end;
  };
  int t0 = t_begin;
  load_k(t0, ka, la);
  load_v(t0);
  if (t0 + kTok < t_end) load_k(t0 + kTok, kb, lb);
  while (true) {
    if (!iter(t0, ka, la, kc, lc)) break;
    t0 += kTok;
    if (!iter(t0, kb, lb, ka, la)) break;
    t0 += kTok;
    if (!iter(t0, kc, lc, kb, lb)) break;
    t0 += kTok;
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot = halves_sum(l_tot);
  if (qc < G) {
    const size_t row = ((size_t)chunk * num_seqs + s) * Hq + (size_t)g * G + qc;
    float* dst = part_o + row * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *(f32x4*)(dst + 16 * nb + 4 * g4) = o[nb];
    if (g4 == 0) {
      part_ml[row * 2 + 0] = m_run;
      part_ml[row * 2 + 1] = l_tot;
    }
  }
}

// Generic block sizes: every token's page is looked up on its own lane.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ETA_DECODE_WAVES_PER_EU)))
void decode_split_generic_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc, const __bf16* __restrict__ Vc,
    const int* __restrict__ block_table, const int* __restrict__ ctx_lens,
    float* __restrict__ part_o, float* __restrict__ part_ml, int num_seqs, int Hq, int Hkv,
    int G, int block_size, int num_blocks, int max_blocks, int max_context, int chunk_tokens,
    int n_chunks_max,
    long long block_stride, long long token_stride, long long head_stride, float scale_log2) {
  constexpr int KS = D / 32;   // k-steps of S^T = K Q^T (32 d each)
  constexpr int NB = D / 16;   // 16-row blocks of o^T
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int VL = kTok * CH / 64;  // V loads per lane per step

  __shared__ __attribute__((aligned(16))) __bf16 vs_all[4][kTok * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int s, chunk;
  const int g = live_item(blockIdx.x * 4 + wave, Hkv, ctx_lens, num_seqs, max_context,
                          chunk_tokens, lane, s, chunk);
  if (s < 0) return;
  const int ctx = min(ctx_lens[s], max_context);
  const int t_begin = chunk * chunk_tokens;
  if (t_begin >= ctx) return;
  const int t_end = min(ctx, t_begin + chunk_tokens);

  __bf16* vs = vs_all[wave];
  const int qc = lane & 15;   // query column (head within the group) / A row
  const int g4 = lane >> 4;   // 16-lane group

  // Q^T as the B operand: lane (qc, g4) holds Q[qc][32 ks + 8 g4 + e].
  bf16x8 qf[KS];
  {
    const bool ok = qc < G;
    const __bf16* src = Q + ((size_t)s * Hq + (size_t)g * G + (ok ? qc : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = ok ? *(const u32x4*)(src + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0};
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const int* bt = block_table + (size_t)s * max_blocks;
  const __bf16* Kg = Kc + (size_t)g * head_stride;
  const __bf16* Vg = Vc + (size_t)g * head_stride;

  // Address of token `pos` of this sequence, or null when pos is past the
  // chunk or its block-table entry lies outside the cache.
  auto tok_ptr = [&](const __bf16* base, int pos) -> const __bf16* {
    if (pos >= t_end) return nullptr;
    const int logical = pos / block_size;
    const int offset = pos - logical * block_size;
    const int physical = bt[logical];
    if (physical < 0 || physical >= num_blocks) return nullptr;
    return base + (size_t)physical * block_stride + (size_t)offset * token_stride;
  };

  u32x4 kr[2][KS], kn[2][KS], vr[VL];
  unsigned long long live_r[2], live_n[2];  // ballot: bit qc of word pp = token t0+16pp+qc is live
  auto load_k = [&](int t0, u32x4 (&kd)[2][KS], unsigned long long (&live)[2]) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const __bf16* p = tok_ptr(Kg, t0 + 16 * pp + qc);
      live[pp] = __ballot(p != nullptr);
      if (p) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kd[pp][ks] = *(const u32x4*)(p + 32 * ks + 8 * g4);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kd[pp][ks] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto load_v = [&](int t0) {
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int cid = lane + 64 * it;
      const int tk = cid / CH;
      const int c = cid % CH;
      const __bf16* p = tok_ptr(Vg, t0 + tk);
      vr[it] = p ? *(const u32x4*)(p + 8 * c) : u32x4{0, 0, 0, 0};
    }
  };

  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // V rows of the current step into the wave's LDS tile (row-major,
  // 16-byte chunks XOR-swizzled by row); frees vr for the next step's loads.
  auto stage_v = [&]() {
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int cid = lane + 64 * it;
      const int tk = cid / CH;
      const int c = cid % CH;
      *(u32x4*)(vs + tk * D + ((c ^ decode_swz<D>(tk)) * 8)) = vr[it];
    }
  };
  auto compute_step = [&](u32x4 (&kd)[2][KS], unsigned long long (&live)[2]) {
    f32x4 sc[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      sc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[pp] = mfma16(__builtin_bit_cast(bf16x8, kd[pp][ks]), qf[ks], sc[pp]);
    }
    // Lane (qc, g4) register r of sc[pp] is token t0 + 16 pp + 4 g4 + r.
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!((live[pp] >> (4 * g4 + r)) & 1ull)) sc[pp][r] = -INFINITY;
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(__builtin_fmaf(sc[pp][r], scale_log2, -m_use));
        sc[pp][r] = p;
        rs += p;
      }
    l_run = alpha * l_run + rs;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[nb][r] *= alpha;
    u32x4 pw;
    pw[0] = pack_bf16x2(sc[0][0], sc[0][1]);
    pw[1] = pack_bf16x2(sc[0][2], sc[0][3]);
    pw[2] = pack_bf16x2(sc[1][0], sc[1][1]);
    pw[3] = pack_bf16x2(sc[1][2], sc[1][3]);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
    const int src = lane & 15;
    const int tr_r = src >> 2;
    const int tr_c = src & 3;
    const int r1 = 4 * g4 + tr_r;
    const int r2 = r1 + 16;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = 16 * nb + 4 * tr_c;
      const int chunk8 = col >> 3;
      const int sub = col & 7;
      const s16x4 lo = lds_read_tr(vs + r1 * D + ((chunk8 ^ decode_swz<D>(r1)) * 8) + sub);
      const s16x4 hi = lds_read_tr(vs + r2 * D + ((chunk8 ^ decode_swz<D>(r2)) * 8) + sub);
      o[nb] = mfma16(join_tr(lo, hi), pb, o[nb]);
    }
    // The next step's LDS writes must follow these reads.
    __asm__ volatile("" ::: "memory");
  };

  // Software pipeline: V of the current step is staged in LDS before the
  // next step's K and V loads are issued, so they fly during the compute.
  int t0 = t_begin;
  load_k(t0, kr, live_r);
  load_v(t0);
  while (true) {
    stage_v();
    int t1 = t0 + kTok;
    if (t1 < t_end) {
      load_v(t1);
      load_k(t1, kn, live_n);
    }
    compute_step(kr, live_r);
    if (t1 >= t_end) break;
    t0 = t1;
    stage_v();
    t1 = t0 + kTok;
    if (t1 < t_end) {
      load_v(t1);
      load_k(t1, kr, live_r);
    }
    compute_step(kn, live_n);
    if (t1 >= t_end) break;
    t0 = t1;
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (qc < G) {
    const size_t row = ((size_t)chunk * num_seqs + s) * Hq + (size_t)g * G + qc;
    float* dst = part_o + row * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *(f32x4*)(dst + 16 * nb + 4 * g4) = o[nb];
    if (g4 == 0) {
      part_ml[row * 2 + 0] = m_run;
      part_ml[row * 2 + 1] = l_tot;
    }
  }
}

template <int D, typename OutT>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int* __restrict__ ctx_lens, OutT* __restrict__ O, float* __restrict__ LSE,
    int num_seqs, int Hq, int chunk_tokens, int max_context) {
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int n = threadIdx.x;
  const int ctx = min(ctx_lens[s], max_context);
  const int nc = ctx > 0 ? (ctx + chunk_tokens - 1) / chunk_tokens : 0;
  // One pass over the chunks, kBatch at a time: all loads of a batch are
  // issued before any is used (the partials are latency-bound, not
  // bandwidth-bound), then the running max absorbs the batch's max and the
  // sums are rescaled by 2^(old - new), as in the online softmax.
  constexpr int kBatch = 8;
  const size_t stride = (size_t)num_seqs * Hq;
  const size_t row0 = (size_t)s * Hq + hq;
  float big_m = -INFINITY, acc = 0.f, ell = 0.f;
  for (int c0 = 0; c0 < nc; c0 += kBatch) {
    float mv[kBatch], lv[kBatch], ov[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool ok = c0 + j < nc;
      const size_t row = (size_t)(ok ? c0 + j : 0) * stride + row0;
      mv[j] = ok ? part_ml[row * 2] : -INFINITY;
      lv[j] = ok ? part_ml[row * 2 + 1] : 0.f;
      ov[j] = ok ? part_o[row * D + n] : 0.f;
    }
    float bm = big_m;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) bm = fmaxf(bm, mv[j]);
    if (bm == -INFINITY) continue;  // every chunk so far saw no key
    const float r = fast_exp2(big_m - bm);  // 0 while big_m is -inf
    acc *= r;
    ell *= r;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float w = fast_exp2(mv[j] - bm);
      ell += w * lv[j];
      acc += w * ov[j];
    }
    big_m = bm;
  }
  const float inv = ell > 0.f ? 1.f / ell : 0.f;
  const size_t orow = (size_t)s * Hq + hq;
  O[orow * D + n] = (OutT)(acc * inv);
  if (n == 0 && LSE) LSE[orow] = ell > 0.f ? (big_m + fast_log2(ell)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  float* part_o = (float*)a.workspace;
  float* part_ml = part_o + (size_t)p.n_chunks_max * a.num_seqs * a.Hq * D;
  if (p.n_chunks_max > 0) {
    const int units = p.n_chunks_max * a.Hkv;
    const bool paged = a.block_size % 16 == 0;
    const int wg_waves = paged ? ETA_DECODE_WG_WAVES : 4;
    // Every (sequence, chunk, KV head) slot the grid could need; the slots
    // beyond the live work exit at once (and come last in launch order).
    const long long slots = (long long)units * a.num_seqs;
    dim3 grid((unsigned)((slots + wg_waves - 1) / wg_waves));
    if (paged) {
      unsigned magic;
      int shift;
      page_magic(a.block_size, magic, shift);
      hipLaunchKernelGGL(decode_split_paged_kernel<D>, grid, dim3(64 * wg_waves), 0, stream,
                         (const __bf16*)a.Q, (const __bf16*)a.K_cache, (const __bf16*)a.V_cache,
                         a.block_table, a.context_lens, part_o, part_ml, a.num_seqs, a.Hq, a.Hkv,
                         a.Hq / a.Hkv, a.block_size, a.num_blocks, a.max_blocks_per_seq,
                         a.max_context, p.chunk_tokens, p.n_chunks_max,
                         (long long)a.block_stride, (long long)a.token_stride,
                         (long long)a.head_stride, a.scale * kLog2e, magic, shift);
    } else {
      hipLaunchKernelGGL(decode_split_generic_kernel<D>, grid, dim3(64 * wg_waves), 0, stream,
                         (const __bf16*)a.Q, (const __bf16*)a.K_cache, (const __bf16*)a.V_cache,
                         a.block_table, a.context_lens, part_o, part_ml, a.num_seqs, a.Hq, a.Hkv,
                         a.Hq / a.Hkv, a.block_size, a.num_blocks, a.max_blocks_per_seq,
                         a.max_context, p.chunk_tokens, p.n_chunks_max,
                         (long long)a.block_stride, (long long)a.token_stride,
                         (long long)a.head_stride, a.scale * kLog2e);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 mgrid((unsigned)a.Hq, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((decode_merge_kernel<D, __bf16>), mgrid, dim3(D), 0, stream, part_o, part_ml,
                     a.context_lens, (__bf16*)a.O, a.LSE, a.num_seqs, a.Hq, p.chunk_tokens,
                     a.max_context);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int num_seqs, int Hq, int d, int n_chunks_max) {
  return (size_t)n_chunks_max * num_seqs * Hq * ((size_t)d + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (a.d == 128) return launch_decode_d<128>(a, p, stream);
  return launch_decode_d<64>(a, p, stream);
}

}  // namespace eta
