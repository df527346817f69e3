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
// (two 16-token pages): K rows go straight from HBM into MFMA A-operand
// registers (S^T = K Q^T); V rows are staged in a wave-private LDS tile and
// read transposed (ds_read_b64_tr_b16) as the A operand of o^T += V^T P^T.
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

// Two waves per SIMD (eight per CU), each with the next 32 tokens' K and V
// in flight: enough bytes outstanding to cover HBM latency without spills.
#ifndef ETA_DECODE_WAVES_PER_EU
#define ETA_DECODE_WAVES_PER_EU 2
#endif

template <int D, bool PAGE16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ETA_DECODE_WAVES_PER_EU)))
void decode_split_kernel(
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
  const int wave = threadIdx.x >> 6;
  const int unit = blockIdx.x * 4 + wave;
  const int s = blockIdx.y;
  if (unit >= n_chunks_max * Hkv) return;
  const int chunk = unit / Hkv;
  const int g = unit % Hkv;
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

  // Physical block of the 16-token page starting at pos0 (a multiple of 16),
  // or -1 when the page lies past the chunk or its entry is outside the cache.
  // pos0 is wave-uniform, so this is a scalar load.
  auto page_phys = [&](int pos0) -> int {
    if (pos0 >= t_end) return -1;
    const int ph = bt[pos0 >> 4];
    return (ph >= 0 && ph < num_blocks) ? ph : -1;
  };

  u32x4 kr[2][KS], kn[2][KS], vr[VL];
  unsigned long long live_r[2], live_n[2];  // ballot: bit qc of word pp = token t0+16pp+qc is live
  auto load_k = [&](int t0, u32x4 (&kd)[2][KS], unsigned long long (&live)[2]) {
    int ph[2] = {0, 0};
    if (PAGE16) {
      ph[0] = page_phys(t0);
      ph[1] = page_phys(t0 + 16);
    }
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const __bf16* p;
      if (PAGE16) {
        const int pos = t0 + 16 * pp + qc;
        p = (ph[pp] >= 0 && pos < t_end)
                ? Kg + (size_t)ph[pp] * block_stride + (size_t)qc * token_stride
                : nullptr;
      } else {
        p = tok_ptr(Kg, t0 + 16 * pp + qc);
      }
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
    int ph[2] = {0, 0};
    if (PAGE16) {
      ph[0] = page_phys(t0);
      ph[1] = page_phys(t0 + 16);
    }
#pragma unroll
    for (int it = 0; it < VL; ++it) {
      const int cid = lane + 64 * it;
      const int tk = cid / CH;
      const int c = cid % CH;
      const __bf16* p;
      if (PAGE16) {
        const int pp = tk >> 4;
        p = (ph[pp] >= 0 && t0 + tk < t_end)
                ? Vg + (size_t)ph[pp] * block_stride + (size_t)(tk & 15) * token_stride
                : nullptr;
      } else {
        p = tok_ptr(Vg, t0 + tk);
      }
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
  float big_m = -INFINITY;
  for (int c = 0; c < nc; ++c) {
    const size_t row = ((size_t)c * num_seqs + s) * Hq + hq;
    big_m = fmaxf(big_m, part_ml[row * 2]);
  }
  const float m_use = big_m == -INFINITY ? 0.f : big_m;
  float acc = 0.f, ell = 0.f;
  for (int c = 0; c < nc; ++c) {
    const size_t row = ((size_t)c * num_seqs + s) * Hq + hq;
    const float w = fast_exp2(part_ml[row * 2] - m_use);
    ell += w * part_ml[row * 2 + 1];
    acc += w * part_o[row * D + n];
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
    dim3 grid((unsigned)((units + 3) / 4), (unsigned)a.num_seqs);
    auto kern = a.block_size == 16 ? decode_split_kernel<D, true> : decode_split_kernel<D, false>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream,
                       (const __bf16*)a.Q, (const __bf16*)a.K_cache, (const __bf16*)a.V_cache,
                       a.block_table, a.context_lens, part_o, part_ml, a.num_seqs, a.Hq, a.Hkv,
                       a.Hq / a.Hkv, a.block_size, a.num_blocks, a.max_blocks_per_seq,
                       a.max_context, p.chunk_tokens, p.n_chunks_max, (long long)a.block_stride, (long long)a.token_stride,
                       (long long)a.head_stride, a.scale * kLog2e);
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
