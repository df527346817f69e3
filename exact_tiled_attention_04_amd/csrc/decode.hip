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
// Split kernel: the contexts of all (sequence, KV head) pairs, in 32-token
// steps laid end to end, are cut into equal ranges, one per wave (the plan in
// kernels.hpp), so every wave streams the same number of cache bytes and a
// wave whose range crosses a pair boundary writes one partial per pair it
// touches.  Within a pair, the G query heads of the group are the columns
// of a 16x16x32 MFMA, so every K and V byte is read from HBM once and used
// by all G heads; a group of more than 16 heads is split into pairs of 16
// (each reading the KV head again).  Per 32 tokens
// (two 16-token groups): K and V arrive as whole rows, several per load.  On
// the path for block sizes that are multiples of 16 (wave-uniform page
// addressing through buffer resources), K rows are staged in a wave-private
// LDS tile and read back as the MFMA A operand of S^T = K Q^T; on the path
// for other block sizes (each token's page looked up per lane) they go from
// HBM straight into A-operand registers.  V rows are staged in a second LDS
// tile and read transposed (ds_read_b64_tr_b16) as the A operand of
// o^T += V^T P^T.
// The next 32 tokens are fetched while the current ones are computed.  Cache
// rows are loaded non-temporal: each is read once per launch.
// Tokens past the context (poisoned or stale page slots) never reach the
// result: their scores are replaced by -inf and their V rows by zeros.
//
// Merge kernel: one workgroup per (query head, sequence), one thread per
// output column, over the pair's partials c: M = max_c m_c, w_c = 2^(m_c - M),
// l = sum w_c l_c, O = sum w_c o_c / l, LSE = (M + log2 l) ln 2.
#include "common.hpp"
#include "kernels.hpp"

namespace eta {

namespace {

constexpr int kTok = kDecodeStepTokens;  // tokens per inner step (two 16-token groups)

// Swizzle of the decode K tile: chunk c of row r sits at c ^ (r mod chunks per
// row).  The tile is written as whole rows (conflict-free for any swizzle)
// and read in the 16x16x32 A layout (lane: row l % 16, chunk 4 ks + l / 16),
// for which this swizzle measured conflict-free on gfx950 and tile_swz or
// decode_swz measured two-way conflicts.
template <int D>
__device__ __forceinline__ int decode_k_swz(int row) {
  return row & (D / 8 - 1);
}
// The paged kernel walks a segment in pieces of at most kDecodeMaxSteps
// steps (4064 tokens): a piece's block-table entries fit four registers of
// 64 lanes (at most 254 pages of >= 16 tokens, as pieces start on a step
// boundary).
static_assert(kDecodeMaxSteps * kTok <= 4064, "piece block-table entries exceed 256");

// Steps of K and of V in flight ahead of the one being computed (K 3, 4 or
// 5 and V 2 or 3 steps ahead at one wave per SIMD measured the same as 2 and
// 1 with the automatic split).
#ifndef ETA_DECODE_K_AHEAD
#define ETA_DECODE_K_AHEAD 2
#endif
#ifndef ETA_DECODE_V_AHEAD
#define ETA_DECODE_V_AHEAD 1
#endif

// Registers for two waves per SIMD: the automatic split runs one per SIMD,
// a caller-fixed range length can ask for more waves than that.
#ifndef ETA_DECODE_WAVES_PER_EU
#define ETA_DECODE_WAVES_PER_EU 2
#endif

// Block sizes that are multiples of 16: each 16-token group of a step lies in
// one page, so its location is wave-uniform.  A group is addressed through a
// raw buffer resource whose base is the group's first cache row and whose
// range ends after its last live token (zero when the group is past the
// piece or its block-table entry lies outside the cache): K and V rows past
// the context, or of a bad page, arrive as zeros with no branches, and the
// score mask is a compare with the group's live-token count.
#ifndef ETA_DECODE_WG_WAVES
#define ETA_DECODE_WG_WAVES 4
#endif

// Steps of a context of ctx tokens.
__device__ __forceinline__ int ctx_steps(int ctx) { return ctx > 0 ? (ctx + kTok - 1) / kTok : 0; }

__device__ __forceinline__ long long uniform64(long long v) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Where a split wave's work starts.  Pair g of sequence s (one of `units`
// per sequence) owns steps [seq_base(s) + g n_s, seq_base(s) + (g + 1) n_s),
// n_s = ceil(ctx_s / 32);
// wave w takes steps [w q, min((w + 1) q, U)).  The wave reads the
// sequences' contexts 64 at a time (one per lane): a reduction gives U, and
// with it q when the caller left it open; an inclusive scan finds the
// sequence that holds step w q.
struct SplitPos {
  long long a, b;      // the wave's steps [a, b)
  long long seq_base;  // first step of sequence s
  int s, n, ctx, g;    // sequence, its steps, its context, pair within it
};

// False when the wave has no steps.
__device__ __forceinline__ bool split_start(int w, const int* __restrict__ ctx_lens, int num_seqs,
                                            int units, int max_context, int steps_fixed,
                                            int target_waves, int lane, SplitPos& sp) {
  auto ctx_of = [&](int sq) -> int {
    return sq < num_seqs ? max(0, min(ctx_lens[sq], max_context)) : 0;
  };
  long long U = 0;
  for (int base = 0; base < num_seqs; base += 64) {
    long long c = (long long)ctx_steps(ctx_of(base + lane)) * units;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
    U += c;
  }
  U = uniform64(U);
  long long q = steps_fixed;
  if (q <= 0) {
    q = (U + target_waves - 1) / target_waves;
    if (q < kDecodeMinSteps) q = kDecodeMinSteps;
  }
  const long long a = (long long)w * q;
  if (a >= U) return false;
  sp.a = a;
  sp.b = a + q < U ? a + q : U;
  long long run = 0;
  for (int base = 0; base < num_seqs; base += 64) {
    const int ctx = ctx_of(base + lane);
    const int n = ctx_steps(ctx);
    const long long c = (long long)n * units;
    long long incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const unsigned long long hit = __ballot(run + incl > a);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      sp.s = base + l;
      sp.n = __builtin_amdgcn_readfirstlane(__shfl(n, l, 64));
      sp.ctx = __builtin_amdgcn_readfirstlane(__shfl(ctx, l, 64));
      sp.seq_base = uniform64(run + __shfl(incl - c, l, 64));
      sp.g = (int)((a - sp.seq_base) / sp.n);
      return true;
    }
    run += __shfl(incl, 63, 64);
  }
  return false;  // not reached: a < U
}

// One segment of a wave's range: the steps it holds of pair (s, g), as
// tokens [t_begin, t_end) of that pair's context.  After the segment the
// wave moves to the next pair with steps (KV head minor).  Returns false at
// the end of the range.
struct SplitSeg {
  int t_begin, t_end;
  bool first, last;  // the segment holds the pair's first / last step
};
__device__ __forceinline__ SplitSeg split_segment(const SplitPos& sp) {
  const long long P = sp.seq_base + (long long)sp.g * sp.n;
  const int l0 = (int)(sp.a - P);
  const int l1 = sp.b - P < sp.n ? (int)(sp.b - P) : sp.n;
  SplitSeg sg;
  sg.t_begin = l0 * kTok;
  sg.t_end = min(sp.ctx, l1 * kTok);
  sg.first = l0 == 0;
  sg.last = l1 == sp.n;
  return sg;
}
__device__ __forceinline__ bool split_next(SplitPos& sp, const int* __restrict__ ctx_lens,
                                           int num_seqs, int units, int max_context) {
  const long long P = sp.seq_base + (long long)sp.g * sp.n;
  sp.a = sp.b - P < sp.n ? sp.b : P + sp.n;
  if (sp.a >= sp.b) return false;
  if (++sp.g < units) return true;
  sp.g = 0;
  sp.seq_base += (long long)sp.n * units;
  do {
    if (++sp.s >= num_seqs) return false;  // not reached: steps remain
    sp.ctx = max(0, min(ctx_lens[sp.s], max_context));
    sp.n = ctx_steps(sp.ctx);
  } while (sp.n == 0);
  sp.ctx = __builtin_amdgcn_readfirstlane(sp.ctx);
  sp.n = __builtin_amdgcn_readfirstlane(sp.n);
  return true;
}

template <int D>
__global__ __launch_bounds__(64 * ETA_DECODE_WG_WAVES)
__attribute__((amdgpu_waves_per_eu(ETA_DECODE_WAVES_PER_EU)))
void decode_split_paged_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc, const __bf16* __restrict__ Vc,
    const int* __restrict__ block_table, const int* __restrict__ ctx_lens,
    float* __restrict__ part_o, float* __restrict__ part_ml, int* __restrict__ seg_first,
    int* __restrict__ seg_last, int num_seqs, int Hq, int Hkv, int G, int block_size,
    int num_blocks, int max_blocks, int max_context, int steps_fixed, int target_waves,
    long long block_stride, long long token_stride, long long head_stride, float scale_log2,
    unsigned page_magic, int page_shift) {
  constexpr int KS = D / 32;          // k-steps of S^T = K Q^T (32 d each)
  constexpr int NB = D / 16;          // 16-row blocks of o^T
  constexpr int CH = D / 8;           // 16-byte chunks per row
  constexpr int VL = kTok * CH / 64;  // V loads per lane per step
  constexpr int TPI = 64 / CH;        // tokens per V load instruction

  __shared__ __attribute__((aligned(16))) __bf16 vs_all[ETA_DECODE_WG_WAVES][kTok * D];
  // K goes through a wave-private LDS tile too: global loads take whole
  // token rows (4 rows x 256 bytes per instruction at d = 128) and the MFMA
  // operand is read back from LDS; loading the operand layout directly
  // (16 rows x 64 bytes per instruction) reached less of the HBM rate.
  __shared__ __attribute__((aligned(16))) __bf16 ks_all[ETA_DECODE_WG_WAVES][kTok * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * ETA_DECODE_WG_WAVES + wave;
  SplitPos sp;
  // A group of G > 16 query heads is split into subgroups of 16 (the MFMA
  // columns); each (KV head, subgroup) is a pair of its own, re-reading the
  // KV head's cache rows.
  const int nsg = (G + 15) >> 4;
  const int units = Hkv * nsg;     // pairs per sequence
  const int gs = G < 16 ? G : 16;  // partial rows per segment
  if (!split_start(w, ctx_lens, num_seqs, units, max_context, steps_fixed, target_waves, lane, sp))
    return;
  int t_begin = 0, t_end = 0;  // the current piece's tokens of pair (sp.s, sp.g)
  int kvh = 0;                 // the pair's KV head

  __bf16* vs = vs_all[wave];
  __bf16* kst = ks_all[wave];
  const int qc = lane & 15;   // query column (head within the group) / A row
  const int g4 = lane >> 4;   // 16-lane group

  bf16x8 qf[KS];
  const int ts2 = (int)(token_stride * 2);  // bytes between tokens
  // This lane's 16-byte chunk of a K or V row inside a 16-token group (the
  // wave loads TPI whole rows per instruction).
  const int voff = (lane / CH) * ts2 + (lane % CH) * 16;

  // The current piece's block-table entries (up to 4 * 64 logical pages,
  // enough for kDecodeMaxSteps steps), one per lane of bt_r[i], loaded at its
  // start: page lookups are register reads (v_readlane), so no step waits on
  // memory before it can issue its K/V loads.
  int bt_base = 0;
  int bt_r[4];
  auto page_of = [&](int logical) -> int {
    const int idx = logical - bt_base;  // 0 <= idx < 256 by the piece limit
    const int r = idx >> 6, l = idx & 63;
    const int v = r == 0 ? bt_r[0] : r == 1 ? bt_r[1] : r == 2 ? bt_r[2] : bt_r[3];
    return __builtin_amdgcn_readlane(v, l);
  };

  struct Group {
    buf_rsrc k, v;
    int live;  // tokens of the group inside the piece (0 if none or bad page)
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
               (long long)kvh * head_stride;
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

  // Register rings: K of the next NKB - 1 steps and V of the next NVB steps
  // are in flight while a step is computed.
  constexpr int NKB = ETA_DECODE_K_AHEAD + 1;
  constexpr int NVB = ETA_DECODE_V_AHEAD;
  u32x4 kbuf[NKB][VL], vbuf[NVB][VL];
  int lbuf[NKB][2];
  auto load_k = [&](int t0, u32x4 (&kd)[VL], int (&live)[2]) {
    const Group g0 = group(t0), g1 = group(t0 + 16);
    live[0] = g0.live;
    live[1] = g1.live;
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int pp = (TPI * it) / 16;
      kd[it] = buf_load16_nt(pp == 0 ? g0.k : g1.k, voff, (TPI * it - 16 * pp) * ts2);
    }
  };
  auto load_v = [&](int t0, u32x4 (&vr)[VL]) {
    const Group g0 = group(t0), g1 = group(t0 + 16);
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int pp = (TPI * it) / 16;
      vr[it] = buf_load16_nt(pp == 0 ? g0.v : g1.v, voff, (TPI * it - 16 * pp) * ts2);
    }
  };

  f32x4 o[NB];
  float m_run, l_run;

  auto stage_v = [&](const u32x4 (&vr)[VL]) {
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int cid = lane + 64 * it;
      const int tk = cid / CH;
      const int c = cid % CH;
      *(u32x4*)(vs + tk * D + ((c ^ decode_swz<D>(tk)) * 8)) = vr[it];
    }
  };
  auto compute_step = [&](u32x4 (&kd)[VL], int (&live)[2]) {
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int cid = lane + 64 * it;
      const int tk = cid / CH;
      const int c = cid % CH;
      *(u32x4*)(kst + tk * D + ((c ^ decode_k_swz<D>(tk)) * 8)) = kd[it];
    }
    f32x4 sc[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      sc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int tk = 16 * pp + qc;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *(const bf16x8*)(kst + tk * D + (((4 * ks + g4) ^ decode_k_swz<D>(tk)) * 8));
        sc[pp] = mfma16(a, qf[ks], sc[pp]);
      }
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

  // Software pipeline over 32-token steps: step u computes from K ring slot
  // u % NKB after refilling slot (u - 1) % NKB with the K of step u + NKB - 1,
  // and stages V slot u % NVB in LDS before refilling it with the V of step
  // u + NVB (a V slot is free once staged).
  auto iter = [&](int u, int t0) -> bool {
    stage_v(vbuf[u % NVB]);
    if (t0 + NVB * kTok < t_end) load_v(t0 + NVB * kTok, vbuf[u % NVB]);
    if (t0 + (NKB - 1) * kTok < t_end)
      load_k(t0 + (NKB - 1) * kTok, kbuf[(u + NKB - 1) % NKB], lbuf[(u + NKB - 1) % NKB]);
    compute_step(kbuf[u % NKB], lbuf[u % NKB]);
    return t0 + kTok < t_end;
  };
  do {
    const SplitSeg seg = split_segment(sp);
    kvh = sp.g / nsg;
    const int sub = sp.g - kvh * nsg;
    const int heads = min(16, G - 16 * sub);  // query heads of this pair
    {
      const bool ok = qc < heads;
      const __bf16* src =
          Q + ((size_t)sp.s * Hq + (size_t)kvh * G + 16 * sub + (ok ? qc : 0)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = ok ? *(const u32x4*)(src + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;

    // The segment in pieces of at most kDecodeMaxSteps steps, each with its
    // block-table entries in registers (the running o, m, l carry over).
    for (int piece = seg.t_begin; piece < seg.t_end; piece += kDecodeMaxSteps * kTok) {
      t_begin = piece;
      t_end = min(seg.t_end, piece + kDecodeMaxSteps * kTok);
      {
        const int* bt = block_table + (size_t)sp.s * max_blocks;
        bt_base = t_begin / block_size;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int lp = bt_base + 64 * i + lane;
          bt_r[i] = lp < max_blocks ? bt[lp] : -1;
        }
      }
      load_k(t_begin, kbuf[0], lbuf[0]);
#pragma unroll
      for (int u = 0; u < NVB; ++u)
        if (u == 0 || t_begin + u * kTok < t_end) load_v(t_begin + u * kTok, vbuf[u]);
#pragma unroll
      for (int u = 1; u + 1 < NKB; ++u)
        if (t_begin + u * kTok < t_end) load_k(t_begin + u * kTok, kbuf[u], lbuf[u]);
      // Steps in groups of lcm(NKB, NVB), so every ring slot index is a
      // compile-time constant.
      constexpr int kUnroll = NKB % NVB == 0 ? NKB : NKB * NVB;
      for (int t0 = t_begin;;) {
        bool more = true;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (more) {
            more = iter(u, t0);
            t0 += kTok;
          }
        }
        if (!more) break;
      }
    }

    // Partial of segment id w + pair: unique, and consecutive over a pair's
    // segments (both w and the pair index only grow along the steps).
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot = halves_sum(l_tot);
    const int pair = sp.s * units + sp.g;
    const int id = w + pair;
    if (qc < heads) {
      const size_t row = (size_t)id * gs + qc;
      float* dst = part_o + row * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) *(f32x4*)(dst + 16 * nb + 4 * g4) = o[nb];
      if (g4 == 0) {
        part_ml[row * 2 + 0] = m_run;
        part_ml[row * 2 + 1] = l_tot;
      }
    }
    if (lane == 0) {
      if (seg.first) seg_first[pair] = id;
      if (seg.last) seg_last[pair] = id;
    }
  } while (split_next(sp, ctx_lens, num_seqs, units, max_context));
}

// Generic block sizes: every token's page is looked up on its own lane.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ETA_DECODE_WAVES_PER_EU)))
void decode_split_generic_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ Kc, const __bf16* __restrict__ Vc,
    const int* __restrict__ block_table, const int* __restrict__ ctx_lens,
    float* __restrict__ part_o, float* __restrict__ part_ml, int* __restrict__ seg_first,
    int* __restrict__ seg_last, int num_seqs, int Hq, int Hkv, int G, int block_size,
    int num_blocks, int max_blocks, int max_context, int steps_fixed, int target_waves,
    long long block_stride, long long token_stride, long long head_stride, float scale_log2) {
  constexpr int KS = D / 32;   // k-steps of S^T = K Q^T (32 d each)
  constexpr int NB = D / 16;   // 16-row blocks of o^T
  constexpr int CH = D / 8;    // 16-byte chunks per row
  constexpr int VL = kTok * CH / 64;  // V loads per lane per step

  __shared__ __attribute__((aligned(16))) __bf16 vs_all[4][kTok * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * 4 + wave;
  SplitPos sp;
  // A group of G > 16 query heads is split into subgroups of 16 (the MFMA
  // columns); each (KV head, subgroup) is a pair of its own, re-reading the
  // KV head's cache rows.
  const int nsg = (G + 15) >> 4;
  const int units = Hkv * nsg;     // pairs per sequence
  const int gs = G < 16 ? G : 16;  // partial rows per segment
  if (!split_start(w, ctx_lens, num_seqs, units, max_context, steps_fixed, target_waves, lane, sp))
    return;
  int t_begin = 0, t_end = 0;  // the current segment's tokens of pair (sp.s, sp.g)
  int kvh = 0;                 // the pair's KV head

  __bf16* vs = vs_all[wave];
  const int qc = lane & 15;   // query column (head within the group) / A row
  const int g4 = lane >> 4;   // 16-lane group

  // Q^T as the B operand: lane (qc, g4) holds Q[qc][32 ks + 8 g4 + e].
  bf16x8 qf[KS];
  const int* bt = block_table;
  const __bf16* Kg = Kc;
  const __bf16* Vg = Vc;

  // Address of token `pos` of this sequence, or null when pos is past the
  // segment or its block-table entry lies outside the cache.
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
        for (int ks = 0; ks < KS; ++ks)
          kd[pp][ks] = __builtin_nontemporal_load((const u32x4*)(p + 32 * ks + 8 * g4));
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
      vr[it] = p ? __builtin_nontemporal_load((const u32x4*)(p + 8 * c)) : u32x4{0, 0, 0, 0};
    }
  };

  f32x4 o[NB];
  float m_run, l_run;

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
  do {
    const SplitSeg seg = split_segment(sp);
    t_begin = seg.t_begin;
    t_end = seg.t_end;
    kvh = sp.g / nsg;
    const int sub = sp.g - kvh * nsg;
    const int heads = min(16, G - 16 * sub);  // query heads of this pair
    {
      const bool ok = qc < heads;
      const __bf16* src =
          Q + ((size_t)sp.s * Hq + (size_t)kvh * G + 16 * sub + (ok ? qc : 0)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = ok ? *(const u32x4*)(src + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0};
        qf[ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
    bt = block_table + (size_t)sp.s * max_blocks;
    Kg = Kc + (size_t)kvh * head_stride;
    Vg = Vc + (size_t)kvh * head_stride;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;

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
    const int pair = sp.s * units + sp.g;
    const int id = w + pair;
    if (qc < heads) {
      const size_t row = (size_t)id * gs + qc;
      float* dst = part_o + row * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) *(f32x4*)(dst + 16 * nb + 4 * g4) = o[nb];
      if (g4 == 0) {
        part_ml[row * 2 + 0] = m_run;
        part_ml[row * 2 + 1] = l_tot;
      }
    }
    if (lane == 0) {
      if (seg.first) seg_first[pair] = id;
      if (seg.last) seg_last[pair] = id;
    }
  } while (split_next(sp, ctx_lens, num_seqs, units, max_context));
}

// Thread groups per merge workgroup: with PARTS > 1 a pair's partials are
// dealt out to PARTS groups of D threads and their results combined through
// LDS, so a pair with many partials (few, long contexts) takes 1/PARTS of
// the dependent load rounds.  The launcher picks PARTS = 4 when the split
// gives at least 16 waves per pair: with fewer partials per pair the extra
// waves and the LDS step cost more than they save (measured: one 64k
// context +22%, 4 x 4k-8k +10%; 32 x 1k -7% with four groups).
template <int D, int PARTS, typename OutT>
__global__ __launch_bounds__(D * PARTS) void decode_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int* __restrict__ seg_first, const int* __restrict__ seg_last,
    const int* __restrict__ ctx_lens, OutT* __restrict__ O, float* __restrict__ LSE,
    int num_seqs, int Hq, int Hkv, int max_context, long long n_ids) {
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int n = threadIdx.x % D;
  const int part = threadIdx.x / D;
  const int G = Hq / Hkv;
  const int nsg = (G + 15) >> 4;
  const int gs = G < 16 ? G : 16;
  const int g = hq / G;
  const int j = hq - g * G;
  const int pair = (s * Hkv + g) * nsg + (j >> 4);
  const int ctx = min(ctx_lens[s], max_context);
  // The pair's partials are segments seg_first .. seg_last, written by the
  // split waves of this call whenever the pair has a live token.
  int first = 0, nc = 0;
  bool bad = false;
  if (ctx > 0) {
    first = seg_first[pair];
    const int last = seg_last[pair];
    bad = first < 0 || last < first || (long long)last >= n_ids;
    nc = bad ? 0 : last - first + 1;
  }
  // Group `part` takes partials part, part + PARTS, ..., kBatch at a
  // time: all loads of a batch are issued before any is used (the partials
  // are latency-bound, not bandwidth-bound), then the running max absorbs
  // the batch's max and the sums are rescaled by 2^(old - new), as in the
  // online softmax.
  constexpr int kBatch = 8;
  const size_t row0 = (size_t)first * gs + (j & 15);
  float big_m = -INFINITY, acc = 0.f, ell = 0.f;
  for (int c0 = part; c0 < nc; c0 += kBatch * PARTS) {
    float mv[kBatch], lv[kBatch], ov[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = c0 + k * PARTS;
      const bool ok = c < nc;
      const size_t row = row0 + (size_t)(ok ? c : 0) * gs;
      mv[k] = ok ? part_ml[row * 2] : -INFINITY;
      lv[k] = ok ? part_ml[row * 2 + 1] : 0.f;
      ov[k] = ok ? part_o[row * D + n] : 0.f;
    }
    float bm = big_m;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) bm = fmaxf(bm, mv[k]);
    if (bm == -INFINITY) continue;  // every partial so far saw no key
    const float r = fast_exp2(big_m - bm);  // 0 while big_m is -inf
    acc *= r;
    ell *= r;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = fast_exp2(mv[k] - bm);
      ell += w * lv[k];
      acc += w * ov[k];
    }
    big_m = bm;
  }
  float M = big_m;
  if constexpr (PARTS > 1) {
    // The groups' (m, acc, l) combined by the same rescaling.
    __shared__ float sm_m[PARTS][D], sm_a[PARTS][D], sm_l[PARTS][D];
    sm_m[part][n] = big_m;
    sm_a[part][n] = acc;
    sm_l[part][n] = ell;
    __syncthreads();
    if (part != 0) return;
    M = -INFINITY;
#pragma unroll
    for (int p = 0; p < PARTS; ++p) M = fmaxf(M, sm_m[p][n]);
    acc = 0.f;
    ell = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int p = 0; p < PARTS; ++p) {
        const float w = fast_exp2(sm_m[p][n] - M);  // 0 for a group that saw no key
        acc += w * sm_a[p][n];
        ell += w * sm_l[p][n];
      }
    }
  }
  const float inv = ell > 0.f ? 1.f / ell : 0.f;
  const size_t orow = (size_t)s * Hq + hq;
  // Segment ids out of range cannot come from the split kernel; NaN makes
  // such a result impossible to mistake for attention output.
  O[orow * D + n] = bad ? (OutT)NAN : (OutT)(acc * inv);
  if (n == 0 && LSE)
    LSE[orow] = bad ? NAN : ell > 0.f ? (M + fast_log2(ell)) * kLn2 : -INFINITY;
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int gs = G < 16 ? G : 16;
  const long long pairs = decode_pairs(a.num_seqs, a.Hkv, G);
  const long long n_ids = p.n_waves + pairs;
  float* part_o = (float*)a.workspace;
  float* part_ml = part_o + (size_t)n_ids * gs * D;
  int* seg_first = (int*)(part_ml + (size_t)n_ids * gs * 2);
  int* seg_last = seg_first + pairs;
  if (p.n_waves > 0) {
    const bool paged = a.block_size % 16 == 0;
    const int wg_waves = paged ? ETA_DECODE_WG_WAVES : 4;
    dim3 grid((unsigned)((p.n_waves + wg_waves - 1) / wg_waves));
    if (paged) {
      unsigned magic;
      int shift;
      page_magic(a.block_size, magic, shift);
      hipLaunchKernelGGL(decode_split_paged_kernel<D>, grid, dim3(64 * wg_waves), 0, stream,
                         (const __bf16*)a.Q, (const __bf16*)a.K_cache, (const __bf16*)a.V_cache,
                         a.block_table, a.context_lens, part_o, part_ml, seg_first, seg_last,
                         a.num_seqs, a.Hq, a.Hkv, G, a.block_size, a.num_blocks,
                         a.max_blocks_per_seq, a.max_context, p.steps_fixed, p.target_waves,
                         (long long)a.block_stride, (long long)a.token_stride,
                         (long long)a.head_stride, a.scale * kLog2e, magic, shift);
    } else {
      hipLaunchKernelGGL(decode_split_generic_kernel<D>, grid, dim3(64 * wg_waves), 0, stream,
                         (const __bf16*)a.Q, (const __bf16*)a.K_cache, (const __bf16*)a.V_cache,
                         a.block_table, a.context_lens, part_o, part_ml, seg_first, seg_last,
                         a.num_seqs, a.Hq, a.Hkv, G, a.block_size, a.num_blocks,
                         a.max_blocks_per_seq, a.max_context, p.steps_fixed, p.target_waves,
                         (long long)a.block_stride, (long long)a.token_stride,
                         (long long)a.head_stride, a.scale * kLog2e);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 mgrid((unsigned)a.Hq, (unsigned)a.num_seqs);
  if (p.n_waves >= 16 * pairs)
    hipLaunchKernelGGL((decode_merge_kernel<D, 4, __bf16>), mgrid, dim3(D * 4), 0, stream,
                       part_o, part_ml, seg_first, seg_last, a.context_lens, (__bf16*)a.O, a.LSE,
                       a.num_seqs, a.Hq, a.Hkv, a.max_context, n_ids);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, 1, __bf16>), mgrid, dim3(D), 0, stream, part_o,
                       part_ml, seg_first, seg_last, a.context_lens, (__bf16*)a.O, a.LSE,
                       a.num_seqs, a.Hq, a.Hkv, a.max_context, n_ids);
  return hipGetLastError();
}

}  // namespace

long long decode_split_waves(long long pairs, int d, int max_context, int steps_fixed) {
  const long long u_max = pairs * ((max_context + kTok - 1) / kTok);
  if (u_max <= 0) return 0;
  if (steps_fixed > 0) return (u_max + steps_fixed - 1) / steps_fixed;
  // The device's q >= ceil(U / target) and >= kDecodeMinSteps needs at most
  // ceil(U / q) <= min(target, ceil(u_max / kDecodeMinSteps)) waves.
  const long long target = decode_target_waves(d);
  const long long cap = (u_max + kDecodeMinSteps - 1) / kDecodeMinSteps;
  return target < cap ? target : cap;
}

size_t decode_workspace_bytes(long long pairs, int G, int d, long long n_waves) {
  // Partials (d + 2 floats per query head of a pair) of every segment id,
  // then the first and last segment id of every pair.
  const long long rows = (n_waves + pairs) * (G < 16 ? G : 16);
  return (size_t)rows * ((size_t)d + 2) * sizeof(float) + (size_t)pairs * 2 * sizeof(int);
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream) {
  if (a.d == 128) return launch_decode_d<128>(a, p, stream);
  return launch_decode_d<64>(a, p, stream);
}

}  // namespace eta
