// Attention backward by recomputation (gfx950).
//
// Method: "Modern attention kernels", "Backward pass recomputes scores" (save
// compact per-row statistics, recompute score tiles, never store P);
// "Flash attention and IO-aware attention", backward paragraph; "Attention
// kernels", recomputation paragraph.  The gradient formulas are the textbook
// chain rule through softmax (the pages do not print them):
//   P = exp(scale Q K^T - LSE), dV = P^T dO, dP = dO V^T,
//   D_i = sum_n dO_in O_in (= sum_j P_ij dP_ij), dS = P (dP - D),
//   dQ = scale dS K, dK = scale dS^T Q.
//
// Kernels (no atomics; every output element has exactly one writer, so all
// three gradients are deterministic):
//   bwd_dkdv: one workgroup per (batch, KV head, 128-key tile), four waves of
//             32 keys.  V of the wave's keys stays in registers and K in a
//             wave-private LDS tile (32 registers fewer: two waves per SIMD
//             without spills, measured 20% faster than K and V in registers
//             at one wave per SIMD); Q, dO, LSE2 and D of each 32-query tile
//             that can see the keys (for every query head of the KV group)
//             are copied straight into LDS, double-buffered.  Each wave forms
//             S = Q K^T and dP = dO V^T with its keys along the lanes, then P
//             and dS, and accumulates dV^T += dO^T P and dK^T += Q^T dS with
//             the transposed operands read by ds_read_b64_tr_b16 (the
//             softmax scale multiplies dK once, at the end).
//   bwd_dq:   runs first.  One workgroup per (batch, head, 128-query tile),
//             four waves of 32 queries, laid out like the forward.  Each lane
//             first forms its row's D = rowsum(dO * O) and LSE2 = LSE log2(e)
//             (rows that see no key get LSE2 = +inf, hence P = 0) and leaves
//             them in the workspace for bwd_dkdv.  Then S^T = K Q^T and
//             dP^T = V dO^T with the queries along the lanes, then
//             dQ^T += K^T dS^T with K^T read transposed from the same LDS
//             tile (scaled once at the end).  K/V tiles arrive by direct
//             copies, double-buffered.
// The split costs two extra products (S and dP are formed in both kernels)
// and buys the removal of the fp32 dQ accumulator and its atomics.
//
// Rows past Nq or Nk arrive as zeros from the buffer loads.  A zero query
// row has dO = 0 and adds nothing to dK or dV, so the dK/dV kernel applies
// only the band (causal or local) mask; the dQ kernel also masks keys past
// Nk (see there).
#include "common.hpp"
#include "kernels.hpp"

namespace eta {

namespace {

constexpr int kBK = 128;  // keys per dK/dV workgroup (32 per wave)
constexpr int kBQ = 32;   // queries per dK/dV inner tile
constexpr int kQB = kBQ / 32;  // 32-row query blocks per inner tile
constexpr int kBC = 32;   // keys per dQ inner tile (measured 1.5% faster than 64)
constexpr int kKB = kBC / 32;  // 32-key blocks per dQ tile
constexpr int kBR = 128;  // queries per dQ workgroup

// Launch order of both main kernels: heaviest causal tiles first.
// Workgroups reach the eight XCDs round robin and, on an XCD, its 32 CUs in
// turn, so in a launch whose grid is (nearly) all resident at once the CU
// that takes workgroup k of a round of 256 also takes workgroup k of the next
// round.  Every other full round runs in reverse CU order (same XCD), so a CU
// pairs a heavy tile with a light one instead of two of similar weight.
__device__ __forceinline__ int snake_order(int w, int n) {
  const int r = w >> 8;
  if ((r & 1) && ((r + 1) << 8) <= n) w = (r << 8) + ((31 - ((w & 255) >> 3)) << 3) + (w & 7);
  return w;
}


// ----------------------------------------------------------------- dK, dV

template <int D, bool BAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2)))
void bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                     const float* __restrict__ LSE2, const float* __restrict__ Dsum,
                     __bf16* __restrict__ dK, __bf16* __restrict__ dV, int B, int H, int Hkv,
                     int Nq, int Nk, float scale, float scale_log2, int win_left,
                     int win_right) {
  constexpr int NT = 256;
  constexpr int CH = D / 8;
  constexpr int KS = D / 16;
  constexpr int NB = D / 32;
  constexpr int ROW = D * 2;
  constexpr int QT = kBQ * ROW;            // bytes of one Q (or dO) tile
  constexpr int NLOAD = kBQ * CH / NT;     // direct copies per thread per tile
  constexpr int STAT = 2 * QT;             // LSE2 then D, kBQ floats each
  constexpr int BUF = STAT + 2 * kBQ * 4;

  __shared__ __attribute__((aligned(16))) char sm0[BUF];
  __shared__ __attribute__((aligned(16))) char sm1[BUF];
  // Each wave's 32 K rows, swizzled like the Q tiles (B operand of S = Q K^T
  // read from LDS instead of held in 32 registers).
  __shared__ __attribute__((aligned(16))) char ksm[4][32 * ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int hh = lane >> 5;
  const int tr_r = (lane & 15) >> 2;
  const int tr_c = lane & 3;

  const int BG = B * Hkv;
  const int wg = snake_order(blockIdx.x, gridDim.x);
  const int kt = wg / BG;  // key tiles seen by the most queries first
  const int bg = wg % BG;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = H / Hkv;
  const int j0 = kt * kBK;
  const int off = Nk - Nq;

  // This wave's 32 keys as B operands: lane (j = li, hh) holds X[j][16 ks + 8 hh + e].
  const int jw = j0 + 32 * wave + li;
  const buf_rsrc krs = make_rsrc(K + ((size_t)b * Hkv + g) * (size_t)Nk * D, (unsigned)Nk * ROW);
  const buf_rsrc vrs = make_rsrc(V + ((size_t)b * Hkv + g) * (size_t)Nk * D, (unsigned)Nk * ROW);
  const char* Kw = ksm[wave];
  {
    // Direct copies of the wave's 32 K rows: instruction it fills slots
    // it * 64 + lane, i.e. row (it * 64 + lane) / CH and swizzled chunk.
#pragma unroll
    for (int it = 0; it < 32 * CH / 64; ++it) {
      const int p = it * 64 + lane;
      const int row = p / CH;
      const int c = (p % CH) ^ tile_swz<D>(row);
      buf_load16_lds(krs, ksm[wave] + it * 1024, (j0 + 32 * wave + row) * ROW + c * 16, 0);
    }
  }
  bf16x8 vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    vf[ks] = __builtin_bit_cast(bf16x8, buf_load16(vrs, jw * ROW + (16 * ks + 8 * hh) * 2, 0));

  // Query tiles that can see this key tile, for each head of the group:
  // query i (position i + off) sees key j iff j - win_right <= i + off <=
  // j + win_left.
  const int n_qt = (Nq + kBQ - 1) / kBQ;
  int qt_begin = 0, qt_end = n_qt - 1;
  if (BAND) {
    const int i_lo = max(0, j0 - win_right - off);
    const int i_hi = min(Nq - 1, j0 + kBK - 1 + win_left - off);
    qt_begin = i_lo / kBQ;
    qt_end = i_lo <= i_hi ? i_hi / kBQ : qt_begin - 1;
  }
  const int per_head = qt_end >= qt_begin ? qt_end - qt_begin + 1 : 0;
  const int n_iter = per_head * G;

  // Loop-invariant byte offsets (the same scheme as the forward).
  int goff[NLOAD];
#pragma unroll
  for (int it = 0; it < NLOAD; ++it) {
    const int p = (wave * NLOAD + it) * 64 + lane;
    const int row = p / CH;
    goff[it] = row * ROW + (((p % CH) ^ tile_swz<D>(row)) * 16);
  }
  int rofs[KS];  // row read: query row li of a 32-row block, chunk 2 ks + hh
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) rofs[ks] = li * ROW + (((2 * ks + hh) ^ tile_swz<D>(li)) * 16);
  int tofs[NB][2];  // transpose read: rows 4 hh + tr_r (+8), columns 32 nb + 16 (li/16) + 4 tr_c
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int rr = 4 * hh + tr_r + 8 * hf;
      const int col = 32 * nb + 16 * (li >> 4) + 4 * tr_c;
      tofs[nb][hf] = rr * ROW + (((col >> 3) ^ tile_swz<D>(rr)) * 16) + (col & 7) * 2;
    }

  f32x16 dv[NB], dk[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    dv[nb] = f32x16{};
    dk[nb] = f32x16{};
  }

  // Tiles run head by head of the group, query tiles in order within a
  // head; (ld_head, ld_qt) is the next tile to copy, c_qt the tile computed.
  int ld_head = 0, ld_qt = qt_begin, c_qt = qt_begin;
  auto load_tiles = [&](char* dst) {
    const int h = g * G + ld_head;
    const int q0 = ld_qt * kBQ;
    if (++ld_qt > qt_end) {
      ld_qt = qt_begin;
      ++ld_head;
    }
    const size_t hb = ((size_t)b * H + h) * (size_t)Nq;
    const buf_rsrc qrs = make_rsrc(Q + hb * D, (unsigned)Nq * ROW);
    const buf_rsrc ors = make_rsrc(dO + hb * D, (unsigned)Nq * ROW);
    const int soff = q0 * ROW;
#pragma unroll
    for (int it = 0; it < NLOAD; ++it) {
      char* slot = dst + (wave * NLOAD + it) * 1024;
      buf_load16_lds(qrs, slot, goff[it], soff);
      buf_load16_lds(ors, slot + QT, goff[it], soff);
    }
    if (wave < 2 && lane < kBQ) {
      // kBQ floats of LSE2 (wave 0) or D (wave 1), 4 bytes per lane.
      const buf_rsrc srs = make_rsrc((wave == 0 ? LSE2 : Dsum) + hb, (unsigned)Nq * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          srs, (__attribute__((address_space(3))) void*)(dst + STAT + wave * kBQ * 4), 4,
          lane * 4, q0 * 4, 0, 0);
    }
  };

  auto step = [&](int itx, const char* cur, char* next) {
    const int q0 = c_qt * kBQ;
    c_qt = c_qt == qt_end ? qt_begin : c_qt + 1;
    if (itx + 1 < n_iter) load_tiles(next);
    const char* Qs = cur;
    const char* Os = cur + QT;
    const float* lse2 = (const float*)(cur + STAT);
    const float* dsum = lse2 + kBQ;
    const bool need_mask = BAND && (j0 + 32 * wave + 31 > q0 + off + win_right ||
                                    j0 + 32 * wave < q0 + kBQ - 1 + off - win_left);

    bf16x8 pb[kQB][2], sb[kQB][2];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const char* qrow = Qs + qb * 32 * ROW;
      const char* orow = Os + qb * 32 * ROW;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(*(const bf16x8*)(qrow + rofs[ks]), *(const bf16x8*)(Kw + rofs[ks]), s);
        dp = mfma32(*(const bf16x8*)(orow + rofs[ks]), vf[ks], dp);
      }
      // Lane (key jw, hh) register r holds query row q0 + 32 qb + 8 (r/4) + 4 hh + r%4.
      // Band edges: scores outside the band become -inf (P = 0), in one
      // block of selects taken only by the edge tiles.
      // With base = q0 + 32 qb + 4 hh + off, register r's row position (query
      // row + off) is base + c for the constant c = 8 (r / 4) + r % 4: the
      // limits are taken relative to base, so each score costs one compare
      // with a constant per limit.
      if (need_mask) {
        const int base = q0 + 32 * qb + 4 * hh + off;
        const int lo_c = jw - win_right - base;  // below: the key is right of the band
        const int hi_c = jw + win_left - base;   // above: the key is left of the band
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 8 * (r >> 2) + (r & 3);
          if (c < lo_c || c > hi_c) s[r] = -INFINITY;
        }
      }
      // dS without the softmax scale, which is applied once to dK at the end.
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rloc = 32 * qb + 8 * r4 + 4 * hh;
        const f32x4 l4 = *(const f32x4*)(lse2 + rloc);
        const f32x4 d4 = *(const f32x4*)(dsum + rloc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -l4[e]));
          s[r] = p;
          dp[r] = p * (dp[r] - d4[e]);
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4 wp, wd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wp[e] = pack_bf16x2(s[8 * s2 + 2 * e], s[8 * s2 + 2 * e + 1]);
          wd[e] = pack_bf16x2(dp[8 * s2 + 2 * e], dp[8 * s2 + 2 * e + 1]);
        }
        pb[qb][s2] = __builtin_bit_cast(bf16x8, wp);
        sb[qb][s2] = __builtin_bit_cast(bf16x8, wd);
      }
    }

    // dV^T += dO^T P and dK^T += Q^T dS.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int base = (32 * qb + 16 * s2) * ROW;
          const bf16x8 dot = join_tr(lds_read_tr(Os + base + tofs[nb][0]),
                                     lds_read_tr(Os + base + tofs[nb][1]));
          const bf16x8 qtt = join_tr(lds_read_tr(Qs + base + tofs[nb][0]),
                                     lds_read_tr(Qs + base + tofs[nb][1]));
          dv[nb] = mfma32(dot, pb[qb][s2], dv[nb]);
          dk[nb] = mfma32(qtt, sb[qb][s2], dk[nb]);
        }
    wait_vmem();
    __syncthreads();
  };

  if (n_iter > 0) load_tiles(sm0);
  wait_vmem();
  __syncthreads();
  for (int itx = 0; itx < n_iter; itx += 2) {
    step(itx, sm0, sm1);
    if (itx + 1 < n_iter) step(itx + 1, sm1, sm0);
  }

  // Lane (key jw, hh) register r of block nb holds column 32 nb + 8 (r/4) + 4 hh + r%4.
  // At d = 64, after the last barrier the wave's K tile is idle: dK, then dV,
  // go out through it as whole rows (the wave's own LDS operations run in
  // order; measured 2% faster).  At d = 128 the staging needs a register
  // the kernel does not have (it spilled, and 32 heads x 8k GQA ran 7%
  // slower), so the C layout is stored directly.
  if constexpr (D == 64) {
    const int k_row0 = j0 + 32 * wave;
    const size_t kv_base = ((size_t)b * Hkv + g) * (size_t)Nk + k_row0;
    store_tile_rows<D>(dk, scale, ksm[wave], dK + kv_base * D, D, Nk - k_row0, lane);
    store_tile_rows<D>(dv, 1.f, ksm[wave], dV + kv_base * D, D, Nk - k_row0, lane);
  } else if (jw < Nk) {
    __bf16* dkp = dK + (((size_t)b * Hkv + g) * (size_t)Nk + jw) * D;
    __bf16* dvp = dV + (((size_t)b * Hkv + g) * (size_t)Nk + jw) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = 32 * nb + 8 * r4 + 4 * hh;
        u32x2 a, c;
        a[0] = pack_bf16x2(dk[nb][4 * r4 + 0] * scale, dk[nb][4 * r4 + 1] * scale);
        a[1] = pack_bf16x2(dk[nb][4 * r4 + 2] * scale, dk[nb][4 * r4 + 3] * scale);
        c[0] = pack_bf16x2(dv[nb][4 * r4 + 0], dv[nb][4 * r4 + 1]);
        c[1] = pack_bf16x2(dv[nb][4 * r4 + 2], dv[nb][4 * r4 + 3]);
        *(u32x2*)(dkp + n) = a;
        *(u32x2*)(dvp + n) = c;
      }
  }
}

// --------------------------------------------------------------------- dQ

template <int D, bool BAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                   const __bf16* __restrict__ O, const float* __restrict__ LSE,
                   float* __restrict__ LSE2, float* __restrict__ Dsum,
                   __bf16* __restrict__ dQ, int B, int H, int Hkv, int Nq, int Nk, float scale,
                   float scale_log2, int n_qtiles, int win_left, int win_right) {
  constexpr int NT = 256;
  constexpr int CH = D / 8;
  constexpr int KS = D / 16;
  constexpr int NB = D / 32;
  constexpr int ROW = D * 2;
  constexpr int TILE = kBC * ROW;
  constexpr int NLOAD = kBC * CH / NT;

  __shared__ __attribute__((aligned(16))) char sm0[2 * TILE];  // K tile | V tile
  __shared__ __attribute__((aligned(16))) char sm1[2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int hh = lane >> 5;
  const int tr_r = (lane & 15) >> 2;
  const int tr_c = lane & 3;

  const int BH = B * H;
  const int wg = snake_order(blockIdx.x, gridDim.x);
  const int qt = n_qtiles - 1 - wg / BH;  // heavy query tiles first
  const int bh = wg % BH;
  const int b = bh / H;
  const int h = bh % H;
  const int g = h / (H / Hkv);
  const int q0 = qt * kBR;
  const int off = Nk - Nq;
  const int qrow = q0 + 32 * wave + li;
  const int wave_row_lo = q0 + 32 * wave;

  int t_lo = 0, t_hi;  // key tiles this query tile sees (as in the forward)
  if (BAND) {
    const int k_lo = max(0, q0 + off - win_left);
    const int k_hi = min(Nk - 1, min(q0 + kBR, Nq) - 1 + off + win_right);
    t_lo = k_lo / kBC;
    t_hi = k_lo <= k_hi ? k_hi / kBC : t_lo - 1;
  } else {
    t_hi = (Nk + kBC - 1) / kBC - 1;
  }

  const size_t hq = ((size_t)b * H + h) * (size_t)Nq;
  const buf_rsrc qrs = make_rsrc(Q + hq * D, (unsigned)Nq * ROW);
  const buf_rsrc ors = make_rsrc(dO + hq * D, (unsigned)Nq * ROW);
  const buf_rsrc krs = make_rsrc(K + ((size_t)b * Hkv + g) * (size_t)Nk * D, (unsigned)Nk * ROW);
  const buf_rsrc vrs = make_rsrc(V + ((size_t)b * Hkv + g) * (size_t)Nk * D, (unsigned)Nk * ROW);
  bf16x8 qf[KS], of[KS];
  // D = rowsum(dO * O) and the base-2 LSE of this lane's row are formed here
  // (the lane and its partner lane ^ 32 hold the two halves of the row) and
  // written to the workspace for the dK/dV kernel, which runs next.  Rows
  // that see no key get LSE2 = +inf, hence P = 0.
  float dd = 0.f;
  {
    const buf_rsrc o_rs = make_rsrc(O + hq * D, (unsigned)Nq * ROW);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int vo = qrow * ROW + (16 * ks + 8 * hh) * 2;
      const u32x4 qv = buf_load16(qrs, vo, 0);
      const u32x4 gv = buf_load16(ors, vo, 0);
      const u32x4 ov = buf_load16(o_rs, vo, 0);
      qf[ks] = __builtin_bit_cast(bf16x8, qv);
      of[ks] = __builtin_bit_cast(bf16x8, gv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dd += bf16_bits_to_float(gv[e] & 0xffff) * bf16_bits_to_float(ov[e] & 0xffff);
        dd += bf16_bits_to_float(gv[e] >> 16) * bf16_bits_to_float(ov[e] >> 16);
      }
    }
    dd += __shfl_xor(dd, 32, 64);
  }
  const float lse_row = qrow < Nq ? LSE[hq + qrow] : 0.f;
  const float lse2 = lse_row == -INFINITY ? INFINITY : lse_row * kLog2e;
  if (hh == 0 && qrow < Nq) {
    Dsum[hq + qrow] = dd;
    LSE2[hq + qrow] = lse2;
  }

  int goff[NLOAD];
#pragma unroll
  for (int it = 0; it < NLOAD; ++it) {
    const int p = (wave * NLOAD + it) * 64 + lane;
    const int row = p / CH;
    goff[it] = row * ROW + (((p % CH) ^ tile_swz<D>(row)) * 16);
  }
  int kofs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kofs[ks] = li * ROW + (((2 * ks + hh) ^ tile_swz<D>(li)) * 16);
  int tofs[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int rr = 4 * hh + tr_r + 8 * hf;
      const int col = 32 * nb + 16 * (li >> 4) + 4 * tr_c;
      tofs[nb][hf] = rr * ROW + (((col >> 3) ^ tile_swz<D>(rr)) * 16) + (col & 7) * 2;
    }

  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};

  auto load_tile = [&](int t, char* dst) {
    const int soff = t * TILE;
#pragma unroll
    for (int it = 0; it < NLOAD; ++it) {
      char* slot = dst + (wave * NLOAD + it) * 1024;
      buf_load16_lds(krs, slot, goff[it], soff);
      buf_load16_lds(vrs, slot + TILE, goff[it], soff);
    }
  };

  auto step = [&](int t, const char* Ks, char* next) {
    const int k0 = t * kBC;
    if (t + 1 <= t_hi) load_tile(t + 1, next);
    const bool wave_live = !BAND || (k0 <= wave_row_lo + 31 + off + win_right &&
                                     k0 + kBC - 1 >= wave_row_lo + off - win_left);
    if (wave_live) {
      const char* Vs = Ks + TILE;
      f32x16 s[kKB], dp[kKB];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
          s[kb] = mfma32(*(const bf16x8*)(Ks + kb * 32 * ROW + kofs[ks]), qf[ks], s[kb]);
          dp[kb] = mfma32(*(const bf16x8*)(Vs + kb * 32 * ROW + kofs[ks]), of[ks], dp[kb]);
        }
      // Band edges, and the ragged key tail: a zero key row past Nk
      // would contribute P * 0, but P = 2^-LSE2 can overflow for rows whose
      // scores are all very negative, so those keys are masked to P = 0.
      const bool need_mask =
          (k0 + kBC > Nk) || (BAND && (k0 + kBC - 1 > wave_row_lo + off + win_right ||
                                       k0 < wave_row_lo + 31 + off - win_left));
      const int lim = BAND ? min(Nk - 1, qrow + off + win_right) : Nk - 1;
      const int lim_lo = BAND ? qrow + off - win_left : 0;
      if (need_mask) {
        // Key k0 + 4 hh + c with the constant c = 32 kb + 8 (r / 4) + r % 4:
        // one compare with a constant per limit.
        const int hi_c = lim - (k0 + 4 * hh);
        const int lo_c = lim_lo - (k0 + 4 * hh);
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
            if (c > hi_c || c < lo_c) s[kb][r] = -INFINITY;
          }
      }
      // dS without the softmax scale, which is applied once to dQ at the end.
      bf16x8 sb[kKB][2];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -lse2));
          dp[kb][r] = p * (dp[kb][r] - dd);
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = pack_bf16x2(dp[kb][8 * s2 + 2 * e], dp[kb][8 * s2 + 2 * e + 1]);
          sb[kb][s2] = __builtin_bit_cast(bf16x8, w);
        }
      }
      // dQ^T += K^T dS^T: K^T from the K tile by transpose reads.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const char* kbase = Ks + (32 * kb + 16 * s2) * ROW;
            const bf16x8 kt_op = join_tr(lds_read_tr(kbase + tofs[nb][0]),
                                         lds_read_tr(kbase + tofs[nb][1]));
            acc[nb] = mfma32(kt_op, sb[kb][s2], acc[nb]);
          }
    }
    wait_vmem();
    __syncthreads();
  };

  if (t_lo <= t_hi) load_tile(t_lo, sm0);
  wait_vmem();
  __syncthreads();
  for (int t = t_lo; t <= t_hi; t += 2) {
    step(t, sm0, sm1);
    if (t + 1 <= t_hi) step(t + 1, sm1, sm0);
  }

  // Lane (query qrow, hh) register r of block nb holds column 32 nb + 8 (r/4) + 4 hh + r%4.
  // Stored as whole rows through the wave's quarter of the idle K/V buffers.
  static_assert(2 * 32 * ROW <= 2 * TILE, "dQ staging fits the K/V buffers");
  store_tile_rows<D>(acc, scale, (wave < 2 ? sm0 : sm1) + (wave & 1) * 32 * ROW,
                     dQ + (hq + wave_row_lo) * D, D, Nq - wave_row_lo, lane);
}

// dQ first: it forms D and the base-2 LSE of every query row on the way and
// leaves them in the workspace for dK/dV (the stream orders the two).
template <int D, bool BAND>
hipError_t launch_main(const BwdArgs& a, float* lse2, float* dsum, hipStream_t stream) {
  const float sl2 = a.scale * kLog2e;
  const int n_qt = (a.Nq + kBR - 1) / kBR;
  hipLaunchKernelGGL((bwd_dq_kernel<D, BAND>), dim3((unsigned)(n_qt * a.B * a.H)), dim3(256), 0,
                     stream, (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V,
                     (const __bf16*)a.dO, (const __bf16*)a.O, a.LSE, lse2, dsum,
                     (__bf16*)a.dQ, a.B, a.H, a.Hkv, a.Nq, a.Nk, a.scale, sl2, n_qt, a.win_left,
                     a.win_right);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_kt = (a.Nk + kBK - 1) / kBK;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, BAND>), dim3((unsigned)(n_kt * a.B * a.Hkv)), dim3(256),
                     0, stream, (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V,
                     (const __bf16*)a.dO, lse2, dsum, (__bf16*)a.dK, (__bf16*)a.dV, a.B, a.H,
                     a.Hkv, a.Nq, a.Nk, a.scale, sl2, a.win_left, a.win_right);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.Nq;
  float* dsum = (float*)a.workspace;
  float* lse2 = dsum + rows;
  return a.band ? launch_main<D, true>(a, lse2, dsum, stream)
                : launch_main<D, false>(a, lse2, dsum, stream);
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int Nq, int d) {
  (void)d;
  return (size_t)B * H * Nq * 2 * sizeof(float);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_bwd_d<128>(a, stream);
  return launch_bwd_d<64>(a, stream);
}

}  // namespace eta
