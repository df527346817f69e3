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
// Kernels:
//   bwd_pre:  D = rowsum(dO * O) in fp32, and zero the fp32 dQ accumulator
//             (a fill kernel, no memset node).
//   bwd_main: one workgroup per (batch, KV head, 128-key tile), four waves of
//             32 keys each.  K and V stay in registers (and K in LDS); for
//             every query head of the KV group and every 64-query tile that
//             can see the keys, Q, dO, LSE and D are staged in LDS
//             (double-buffered through registers).  Each wave computes
//             S = Q K^T and dP = dO V^T with its keys along the lanes, forms
//             P and dS, accumulates dV^T += dO^T P and dK^T += Q^T dS with
//             the transposed operands read by ds_read_b64_tr_b16, then
//             writes scale*dS^T to LDS; after a barrier the waves split
//             dQ = (scale dS) K over all 128 keys into 32x32 blocks and add
//             them to the fp32 accumulator with hardware float atomics.
//   bwd_dq:   dQ fp32 accumulator -> bf16.
#include "common.hpp"
#include "kernels.hpp"

namespace eta {

namespace {

constexpr int kBK = 128;  // keys per workgroup (32 per wave)
constexpr int kBQ = 64;   // queries per inner tile

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ O,
                                                      const __bf16* __restrict__ dO,
                                                      float* __restrict__ Dsum,
                                                      float* __restrict__ dq_acc, long long rows) {
  constexpr int CH = D / 8;
  constexpr int RPB = 256 / CH;  // rows per block
  const int t = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + t / CH;
  const int c = t % CH;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(O + row * D + 8 * c);
    const u32x4 b = *(const u32x4*)(dO + row * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += bf16_bits_to_float(a[e] & 0xffff) * bf16_bits_to_float(b[e] & 0xffff);
      acc += bf16_bits_to_float(a[e] >> 16) * bf16_bits_to_float(b[e] >> 16);
    }
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(dq_acc + row * D + 8 * c) = z;
    *(f32x4*)(dq_acc + row * D + 8 * c + 4) = z;
  }
#pragma unroll
  for (int m = CH / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && c == 0) Dsum[row] = acc;
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ dq_acc,
                                                     __bf16* __restrict__ dQ, long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(dq_acc + 8 * i);
  const f32x4 b = *(const f32x4*)(dq_acc + 8 * i + 4);
  u32x4 w;
  w[0] = pack_bf16x2(a[0], a[1]);
  w[1] = pack_bf16x2(a[2], a[3]);
  w[2] = pack_bf16x2(b[0], b[1]);
  w[3] = pack_bf16x2(b[2], b[3]);
  *(u32x4*)(dQ + 8 * i) = w;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_main_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dsum,
    float* __restrict__ dq_acc, __bf16* __restrict__ dK, __bf16* __restrict__ dV, int B, int H,
    int Hkv, int Nq, int Nk, float scale, float scale_log2) {
  constexpr int CH = D / 8;
  constexpr int KS = D / 16;
  constexpr int NB = D / 32;
  constexpr int QLOAD = kBQ * CH / 256;  // 16-byte loads per thread per Q (or dO) tile
  constexpr int KLOAD = kBK * CH / 256;
  constexpr int DSCH = kBQ / 8;          // chunks per dS^T row

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  __bf16* Ks = (__bf16*)smem_raw;                       // [kBK][D]
  __bf16* Qs = Ks + kBK * D;                            // [2][kBQ][D]
  __bf16* dOs = Qs + 2 * kBQ * D;                       // [2][kBQ][D]
  __bf16* dSt = dOs + 2 * kBQ * D;                      // [kBK][kBQ]
  float* stat = (float*)(dSt + kBK * kBQ);              // [2][2][kBQ]: LSE2, D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int li = lane & 31;
  const int hh = lane >> 5;
  const int src = lane & 15;
  const int tr_r = src >> 2;
  const int tr_c = src & 3;

  const int n_kt = (Nk + kBK - 1) / kBK;
  const int kt = blockIdx.x % n_kt;
  const int bg = blockIdx.x / n_kt;
  const int b = bg / Hkv;
  const int g = bg % Hkv;
  const int G = H / Hkv;
  const int j0 = kt * kBK;
  const int off = Nk - Nq;

  const __bf16* Kp = K + ((size_t)b * Hkv + g) * (size_t)Nk * D;
  const __bf16* Vp = V + ((size_t)b * Hkv + g) * (size_t)Nk * D;

  // K tile into LDS (also the source of this wave's K fragment).
#pragma unroll
  for (int it = 0; it < KLOAD; ++it) {
    const int cid = tid + 256 * it;
    const int row = cid / CH;
    const int c = cid % CH;
    const int key = j0 + row;
    u32x4 v = key < Nk ? *(const u32x4*)(Kp + (size_t)key * D + 8 * c) : u32x4{0, 0, 0, 0};
    *(u32x4*)(Ks + row * D + ((c ^ tile_swz<D>(row)) * 8)) = v;
  }
  // This wave's keys as B operands: lane (j = li, hh) holds X[j][16 ks + 8 hh + e].
  const int jw = j0 + 32 * w + li;
  bf16x8 kf[KS], vf[KS];
  {
    const bool ok = jw < Nk;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 a = ok ? *(const u32x4*)(Kp + (size_t)jw * D + 16 * ks + 8 * hh) : u32x4{0, 0, 0, 0};
      u32x4 v = ok ? *(const u32x4*)(Vp + (size_t)jw * D + 16 * ks + 8 * hh) : u32x4{0, 0, 0, 0};
      kf[ks] = __builtin_bit_cast(bf16x8, a);
      vf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 dv[NB], dk[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    dv[nb] = f32x16{};
    dk[nb] = f32x16{};
  }

  // Query tiles that can see this key tile.
  const int n_qt = (Nq + kBQ - 1) / kBQ;
  int qt_begin = 0;
  if (CAUSAL) {
    const int first_q = j0 - off;  // first query row that sees key j0
    qt_begin = first_q <= 0 ? 0 : first_q / kBQ;
  }
  const int per_head = n_qt > qt_begin ? n_qt - qt_begin : 0;
  const int n_iter = per_head * G;

  u32x4 rq[QLOAD], rdo[QLOAD];
  float rstat = 0.f;
  auto iter_coords = [&](int itx, int& h, int& q0) {
    h = g * G + itx / per_head;
    q0 = (qt_begin + itx % per_head) * kBQ;
  };
  auto load_q = [&](int itx) {
    int h, q0;
    iter_coords(itx, h, q0);
    const size_t hb = ((size_t)b * H + h) * (size_t)Nq;
#pragma unroll
    for (int it = 0; it < QLOAD; ++it) {
      const int cid = tid + 256 * it;
      const int row = cid / CH;
      const int c = cid % CH;
      const int q = q0 + row;
      if (q < Nq) {
        rq[it] = *(const u32x4*)(Q + (hb + q) * D + 8 * c);
        rdo[it] = *(const u32x4*)(dO + (hb + q) * D + 8 * c);
      } else {
        rq[it] = u32x4{0, 0, 0, 0};
        rdo[it] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < 2 * kBQ) {
      const int row = tid % kBQ;
      const int q = q0 + row;
      if (tid < kBQ) {
        // LSE in base 2; rows past Nq or with no visible key give P = 0.
        const float l = q < Nq ? LSE[hb + q] : -INFINITY;
        rstat = l == -INFINITY ? INFINITY : l * kLog2e;
      } else {
        rstat = q < Nq ? Dsum[hb + q] : 0.f;
      }
    }
  };
  auto store_q = [&](int buf) {
    __bf16* qd = Qs + buf * kBQ * D;
    __bf16* dd = dOs + buf * kBQ * D;
#pragma unroll
    for (int it = 0; it < QLOAD; ++it) {
      const int cid = tid + 256 * it;
      const int row = cid / CH;
      const int c = cid % CH;
      const int idx = row * D + ((c ^ tile_swz<D>(row)) * 8);
      *(u32x4*)(qd + idx) = rq[it];
      *(u32x4*)(dd + idx) = rdo[it];
    }
    if (tid < 2 * kBQ) stat[buf * 2 * kBQ + tid] = rstat;
  };

  if (n_iter > 0) {
    load_q(0);
    store_q(0);
  }
  __syncthreads();

  for (int itx = 0; itx < n_iter; ++itx) {
    const int buf = itx & 1;
    int h, q0;
    iter_coords(itx, h, q0);
    if (itx + 1 < n_iter) load_q(itx + 1);
    const __bf16* qs = Qs + buf * kBQ * D;
    const __bf16* ds = dOs + buf * kBQ * D;
    const float* lse2 = stat + buf * 2 * kBQ;
    const float* dsum = lse2 + kBQ;

    const bool need_mask =
        (j0 + kBK > Nk) || (CAUSAL && (j0 + 32 * w + 31 > q0 + off));
    bf16x8 pb[2][2], sb[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const int row = 32 * qb + li;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int idx = row * D + (((2 * ks + hh) ^ tile_swz<D>(row)) * 8);
        s = mfma32(*(const bf16x8*)(qs + idx), kf[ks], s);
        dp = mfma32(*(const bf16x8*)(ds + idx), vf[ks], dp);
      }
      // Lane (key jw, hh) register r holds query row q0 + 32 qb + 8 (r/4) + 4 hh + r%4.
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int rloc = 32 * qb + 8 * r4 + 4 * hh;
        const f32x4 l4 = *(const f32x4*)(lse2 + rloc);
        const f32x4 d4 = *(const f32x4*)(dsum + rloc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -l4[e]));
          if (need_mask) {
            const int qrow = q0 + rloc + e;
            const bool vis = (jw < Nk) && (!CAUSAL || jw <= qrow + off);
            p = vis ? p : 0.f;
          }
          s[r] = p;
          dp[r] = p * (dp[r] - d4[e]) * scale;
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
      // scale*dS^T into LDS: row = key (32 w + li), 4 consecutive queries per store.
      const int krow = 32 * w + li;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qc = 32 * qb + 8 * r4 + 4 * hh;
        const int chunk = qc >> 3;
        u32x2 v;
        v[0] = pack_bf16x2(dp[4 * r4 + 0], dp[4 * r4 + 1]);
        v[1] = pack_bf16x2(dp[4 * r4 + 2], dp[4 * r4 + 3]);
        *(u32x2*)(dSt + krow * kBQ + ((chunk ^ tile_swz<kBQ>(krow)) * 8) + (qc & 7)) = v;
      }
    }

    // dV^T += dO^T P and dK^T += Q^T (scale dS): transposed A operands via LDS tr reads.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = 32 * nb + 16 * (li >> 4) + 4 * tr_c;
      const int chunk = col >> 3;
      const int sub = col & 7;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int r1 = 32 * qb + 16 * s2 + 4 * hh + tr_r;
          const int r2 = r1 + 8;
          const int a1 = r1 * D + ((chunk ^ tile_swz<D>(r1)) * 8) + sub;
          const int a2 = r2 * D + ((chunk ^ tile_swz<D>(r2)) * 8) + sub;
          const bf16x8 dot = join_tr(lds_read_tr(ds + a1), lds_read_tr(ds + a2));
          const bf16x8 qtt = join_tr(lds_read_tr(qs + a1), lds_read_tr(qs + a2));
          dv[nb] = mfma32(dot, pb[qb][s2], dv[nb]);
          dk[nb] = mfma32(qtt, sb[qb][s2], dk[nb]);
        }
    }
    __syncthreads();

    // dQ = (scale dS) K over the 128 keys: work items are (32-query block qb,
    // 32-column slice cs); the four waves take items w, w + 4, ...
    {
      const size_t hb = ((size_t)b * H + h) * (size_t)Nq;
      constexpr int NCS = D / 32;
      for (int item = w; item < 2 * NCS; item += 4) {
        const int qb = item / NCS;
        const int cs = item % NCS;
        const int ncol = 32 * cs + 16 * (li >> 4) + 4 * tr_c;
        const int nchunk = ncol >> 3;
        const int nsub = ncol & 7;
        f32x16 acc = f32x16{};
        const int icol = 32 * qb + 16 * (li >> 4) + 4 * tr_c;
        const int ichunk = icol >> 3;
        const int isub = icol & 7;
#pragma unroll
        for (int kj = 0; kj < kBK / 16; ++kj) {
          const int r1 = 16 * kj + 4 * hh + tr_r;
          const int r2 = r1 + 8;
          // A = (scale dS)[i][j] (rows = queries), B = K[j][n]: both column
          // reads of row-major LDS tiles.
          const bf16x8 ds_op =
              join_tr(lds_read_tr(dSt + r1 * kBQ + ((ichunk ^ tile_swz<kBQ>(r1)) * 8) + isub),
                      lds_read_tr(dSt + r2 * kBQ + ((ichunk ^ tile_swz<kBQ>(r2)) * 8) + isub));
          const bf16x8 k_op = join_tr(lds_read_tr(Ks + r1 * D + ((nchunk ^ tile_swz<D>(r1)) * 8) + nsub),
                                      lds_read_tr(Ks + r2 * D + ((nchunk ^ tile_swz<D>(r2)) * 8) + nsub));
          acc = mfma32(ds_op, k_op, acc);
        }
        // Lane (column 32 cs + li, hh) register r holds query row
        // 32 qb + 8 (r/4) + 4 hh + r%4: each atomic instruction covers two
        // contiguous 128-byte row segments.
        float* dst = dq_acc + (hb + q0 + 32 * qb + 4 * hh) * D + 32 * cs + li;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = 8 * (r >> 2) + (r & 3);
          if (q0 + 32 * qb + 4 * hh + qi < Nq) unsafeAtomicAdd(dst + (size_t)qi * D, acc[r]);
        }
      }
    }

    if (itx + 1 < n_iter) store_q(buf ^ 1);
    __syncthreads();
  }

  // dK = scale * sum dS^T Q was folded into dS; write dK, dV for this wave's keys.
  if (jw < Nk) {
    __bf16* dkp = dK + (((size_t)b * Hkv + g) * (size_t)Nk + jw) * D;
    __bf16* dvp = dV + (((size_t)b * Hkv + g) * (size_t)Nk + jw) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = 32 * nb + 8 * r4 + 4 * hh;
        u32x2 a, c;
        a[0] = pack_bf16x2(dk[nb][4 * r4 + 0], dk[nb][4 * r4 + 1]);
        a[1] = pack_bf16x2(dk[nb][4 * r4 + 2], dk[nb][4 * r4 + 3]);
        c[0] = pack_bf16x2(dv[nb][4 * r4 + 0], dv[nb][4 * r4 + 1]);
        c[1] = pack_bf16x2(dv[nb][4 * r4 + 2], dv[nb][4 * r4 + 3]);
        *(u32x2*)(dkp + n) = a;
        *(u32x2*)(dvp + n) = c;
      }
  }
}

template <int D>
size_t main_lds_bytes() {
  return (size_t)(kBK * D + 4 * kBQ * D + kBK * kBQ) * 2 + 4 * kBQ * sizeof(float);
}

template <int D, bool CAUSAL>
hipError_t launch_main(const BwdArgs& a, float* dq_acc, float* dsum, hipStream_t stream) {
  const size_t lds = main_lds_bytes<D>();
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)bwd_main_kernel<D, CAUSAL>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int n_kt = (a.Nk + kBK - 1) / kBK;
  dim3 grid((unsigned)(n_kt * a.B * a.Hkv));
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL>), grid, dim3(256), lds, stream,
                     (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V,
                     (const __bf16*)a.dO, a.LSE, dsum, dq_acc, (__bf16*)a.dK, (__bf16*)a.dV, a.B,
                     a.H, a.Hkv, a.Nq, a.Nk, a.scale, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  float* dq_acc = (float*)a.workspace;
  float* dsum = dq_acc + (size_t)a.B * a.H * a.Nq * D;
  const long long rows = (long long)a.B * a.H * a.Nq;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, (const __bf16*)a.O, (const __bf16*)a.dO, dsum, dq_acc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = a.causal ? launch_main<D, true>(a, dq_acc, dsum, stream)
               : launch_main<D, false>(a, dq_acc, dsum, stream);
  if (e != hipSuccess) return e;
  const long long n8 = rows * D / 8;
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     dq_acc, (__bf16*)a.dQ, n8);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int Nq, int d) {
  return (size_t)B * H * Nq * ((size_t)d + 1) * sizeof(float);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return launch_bwd_d<128>(a, stream);
  return launch_bwd_d<64>(a, stream);
}

}  // namespace eta
