// Tiled exact attention forward (prefill) for gfx950.
//
// Method ("Modern attention kernels", sections "Online softmax makes tiling
// exact" and "Kernel structure"; "Attention kernels", online-softmax
// derivation): each workgroup owns one query tile of one (batch, head); it
// keeps the queries in registers, streams the key/value tiles its mask allows
// through LDS, and carries a running maximum m, running sum l and an
// unnormalised accumulator o per query row.  After the last tile it divides
// once and writes O and the per-row log-sum-exp; the score and probability
// tiles never leave the chip.
//
// Mapping onto CDNA4:
//   * one wave = 32 query rows; the score tile is computed transposed,
//     S^T = K Q^T, on v_mfma_f32_32x32x16_bf16 so that each lane holds the
//     scores of ONE query row (16 keys per 32-key block); row max and row sum
//     are in-register plus one exchange between the two half-waves;
//   * o^T = V^T P^T on the same MFMA, P taken straight from the score
//     registers (packed to bf16), V^T read from the row-major V tile in LDS
//     with ds_read_b64_tr_b16;
//   * the softmax runs in base 2 with scale*log2(e) folded into one FMA;
//   * K/V tiles are double-buffered in LDS and filled by direct
//     global->LDS buffer copies issued one tile ahead (rows past the end
//     arrive as zeros), one barrier per tile;
//   * the row max is exchanged between half-waves with v_permlane32_swap,
//     and the accumulator is rescaled only when the reference max moves;
//   * grid = batch x head x query tile ("Work partitioning in
//     FlashAttention-2": parallel over the sequence), causal tiles heaviest
//     first, each (batch, KV head) pair owned by one XCD so that its L2
//     serves the heads that share the pair's K and V (grid_tile);
//   * one kernel, four row modes: dense [B, H, N, d]; packed ragged
//     sequences; ragged queries over a paged K/V cache; dense rows visiting
//     only the blocks of a sparse block index.  Only the addressing, the
//     per-sequence lengths and the visited tiles differ between them.
#include "common.hpp"
#include "kernels.hpp"

namespace eta {

namespace {


// Key-tile width per head dimension: 32 keys for d = 128 (32 KiB of LDS
// and 154 VGPRs, so three waves share each SIMD: measured 4% faster than
// 64-key tiles at two waves per SIMD), 64 keys for d = 64 (fewer barriers;
// measured 3% faster than 32).  More waves per SIMD let one wave's softmax
// overlap another's MFMAs.
template <int D>
constexpr int fwd_bc() { return D == 128 ? 32 : 64; }

// Part `chunk` of a key-tile range t_lo .. t_hi cut into
// ceil(n / chunk_tiles) parts of equal size (the last may be shorter):
// narrows the range to that part; false when the part is empty.
__device__ __forceinline__ bool split_part(int& t_lo, int& t_hi, int chunk_tiles, int chunk) {
  const int n = t_hi - t_lo + 1;
  if (n <= 0) return false;
  const int parts = (n + chunk_tiles - 1) / chunk_tiles;
  if (chunk >= parts) return false;
  const int sz = (n + parts - 1) / parts;
  const int lo = t_lo + chunk * sz;
  t_hi = min(t_hi, lo + sz - 1);
  t_lo = lo;
  return t_lo <= t_hi;
}

// Query tile and part of key-split unit u.  Units enumerate the (query
// tile, part) pairs that have work, heaviest (last) query tiles first and
// each tile's parts in order; the wave finds u's tile by an inclusive scan of
// the part counts of 64 tiles at a time.
template <bool BAND>
__device__ __forceinline__ void split_unit(int u, int n_qtiles, int BR, int Nq, int Nk, int BC,
                                           int win_left, int win_right, int chunk_tiles,
                                           int lane, int& qt_out, int& chunk_out) {
  int qt = 0, chunk = 0;
  for (int base = 0; base < n_qtiles; base += 64) {
    const int qr = base + lane;  // position in heavy-first order
    int parts = 0;
    if (qr < n_qtiles) {
      int lo, hi;
      band_tiles(BAND, (n_qtiles - 1 - qr) * BR, BR, Nq, Nk, BC, win_left, win_right, lo, hi);
      parts = hi >= lo ? (hi - lo + chunk_tiles) / chunk_tiles : 0;
    }
    int incl = parts;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    const unsigned long long hit = __ballot(incl > u);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      qt = n_qtiles - 1 - (base + l);
      chunk = u - (__shfl(incl, l, 64) - __shfl(parts, l, 64));
      break;
    }
    u -= __shfl(incl, 63, 64);
  }
  qt_out = __builtin_amdgcn_readfirstlane(qt);
  chunk_out = __builtin_amdgcn_readfirstlane(chunk);
}

// Page of key position `key` (0 <= key < 2^31): key / block_size by a
// multiply-high with the host's magic number m = floor(2^(31+l) / bs) + 1,
// l = ceil(log2 bs), exact for every 31-bit key; scalar instructions only
// (a plain division is a long VALU sequence).
__device__ __forceinline__ int page_div(int key, const FwdSeqArgs& sq) {
  return (int)(((unsigned long long)(unsigned)key * sq.page_magic) >> sq.page_shift);
}

// Query tile and (batch, head) of workgroup wg, heaviest (last) query tiles
// first.  Workgroups reach the eight XCDs round robin (wg % 8), and each XCD
// has its own L2.  When the (batch, KV head) pairs divide evenly over the
// XCDs, XCD x takes the pairs p = x, x + 8, ... and, for each, all query heads
// of the group next to each other: the heads that share K and V run on one
// L2 at the same time, each pair's K/V is fetched by one XCD, and every XCD
// gets the same share of every sequence.  Within an XCD the order is either
// query-tile layers across its pairs (dense rows with a mask: the heaviest
// tiles of every head first) or PAIR_MAJOR, all tiles of one pair before the
// next (packed sequences of different lengths, and dense rows without a
// mask, whose tiles are all equal: a pair's tiles stream its K/V together).
// Otherwise consecutive workgroups take consecutive (batch, head) indices.
template <bool PAIR_MAJOR>
__device__ __forceinline__ void grid_tile(int wg, int n_qtiles, int B, int H, int Hkv, int& qt,
                                          int& bh) {
  const int P = B * Hkv;
  if ((P & 7) == 0) {
    const int G = H / Hkv;
    const int x = wg & 7;
    int k = wg >> 3;
    if (!PAIR_MAJOR) {
      // Every other full round of 32 workgroups on the XCD (one per CU) runs
      // in reverse, so the workgroups that meet on a CU at the start of the
      // launch pair heavier with lighter query tiles (measured +2.7% on
      // 4 x 16 heads x 2k causal, where the whole grid is resident at once).
      const int per_xcd = n_qtiles * (P >> 3) * G;
      const int r = k >> 5;
      if ((r & 1) && (r << 5) + 31 < per_xcd) k = (r << 5) + 31 - (k & 31);
    }
    const int hg = k % G, kk = k / G;
    const int per = P >> 3;
    const int pp = PAIR_MAJOR ? kk / n_qtiles : kk % per;
    const int qt_rev = PAIR_MAJOR ? kk % n_qtiles : kk / per;
    const int p = pp * 8 + x;
    qt = n_qtiles - 1 - qt_rev;
    bh = (p / Hkv) * H + (p % Hkv) * G + hg;
  } else {
    qt = n_qtiles - 1 - wg / (B * H);
    bh = wg % (B * H);
  }
}

// The running maximum is a reference point, not necessarily the exact row
// maximum: it moves (and the accumulator is rescaled) only when a tile's
// maximum exceeds it by more than kSlack in base-2 units.  o / l and
// m + log2 l are the same for any reference point, so the result is exact as
// with a per-tile rescale, while exponents stay <= 2^kSlack.
constexpr float kSlack = 8.f;
constexpr float kSlackExp = 256.f;  // 2^kSlack


// Where a workgroup's rows live and which key tiles it visits.
//   kFwdDense:  Q, O [B, H, N, d]; K, V [B, Hkv, N, d]; a contiguous tile range.
//   kFwdRagged: packed sequences ("Numerical validation": ragged sequence
//            boundaries): Q, O [total_q, H, d], K, V [total_k, Hkv, d];
//            sequence s owns rows cu_q[s] .. cu_q[s+1] - 1 and
//            cu_k[s] .. cu_k[s+1] - 1.
//   kFwdPaged:  packed ragged queries over a paged K/V cache ("Paged attention
//            changes addressing": a token's page comes from the sequence's
//            block table); sequence s has seqlens_k[s] cached tokens.
//   kFwdSparse: dense rows, but the workgroup visits only the 128-key blocks a
//            CSR block index lists for its 128-row query block ("Kernel
//            structure": sparse masks need an index of the blocks that exist).

template <int D, bool BAND, int NW, int BC, bool SPLIT, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(BC == 32 ? 3 : 2)))
void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
    const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
    int B, int H, int Hkv, int Nq, int Nk, float scale_log2, int n_qtiles, int win_left,
    int win_right, int chunk_tiles, int n_chunks, float* __restrict__ part, FwdSeqArgs sq) {
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int NLOAD = BC * CH / NT;       // 16-byte loads per thread per tile
  constexpr int KS = D / 16;                 // k-steps of the QK^T product
  constexpr int NB = D / 32;                 // 32-wide column blocks of o
  constexpr int ROW = D * 2;                 // bytes per row
  constexpr int TILE = BC * ROW;            // bytes per K (or V) tile
  constexpr int KB = BC / 32;                // 32-key blocks per tile
  constexpr int RPI = 64 / CH;               // tile rows per copy instruction
  constexpr int WROWS = NLOAD * RPI;         // tile rows copied by one wave
  constexpr int TPB = 128 / BC;              // key tiles per 128-key sparse block
  constexpr bool PACKED = MODE == kFwdRagged || MODE == kFwdPaged;
  static_assert(BC * CH % NT == 0, "tile load split");
  static_assert(BC == 32 || BC == 64, "tile width");
  static_assert(!(SPLIT && MODE != kFwdDense), "key split on dense rows only");
  static_assert(MODE == kFwdDense || NW == 4, "128-row query tiles");

  // Two LDS buffers (K tile then V tile each) as separate objects, so the
  // direct copies into one are known not to alias reads of the other.
  __shared__ __attribute__((aligned(16))) char smem0[2 * TILE];
  __shared__ __attribute__((aligned(16))) char smem1[2 * TILE];
  // Paged: per buffer, one flag per wave marking its rows of the tile as
  // coming from a page outside the cache (those keys are masked).
  constexpr int NBAD = MODE == kFwdPaged ? NW : 1;
  __shared__ int bad0[NBAD];
  __shared__ int bad1[NBAD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int li = lane & 31;   // query row within the wave / A-row
  const int hh = lane >> 5;   // half-wave
  const int tr_r = (lane & 15) >> 2;
  const int tr_c = lane & 3;

  const int BH = B * H;
  const int wg = blockIdx.x;
  // Heavy (late) query tiles first; with a key split, the chunks of one query
  // tile follow each other (each over every head).
  int qt, bh, chunk = 0;
  if (SPLIT) {
    bh = wg % BH;
    split_unit<BAND>(wg / BH, n_qtiles, BR, Nq, Nk, BC, win_left, win_right, chunk_tiles, lane,
                     qt, chunk);
  } else {
    // Pair-major for packed sequences, and for dense rows without a mask,
    // whose query tiles all carry the same work (no heavy-to-light
    // imbalance for the order to cause).
    grid_tile<MODE == kFwdRagged || MODE == kFwdPaged || (MODE == kFwdDense && !BAND)>(
        wg, n_qtiles, B, H, Hkv, qt, bh);
  }
  const int b = bh / H;       // batch, or sequence of a packed batch
  const int h = bh % H;
  const int g = h / (H / Hkv);
  const int q0 = qt * BR;

  // Rows of this (batch or sequence, head): element offsets of the first
  // query and key row, and byte strides between rows.  Offsets of packed
  // sequences are clamped into the packed tensors, so inconsistent offsets
  // cannot move an access outside them.
  size_t q_elem, k_elem = 0;
  int q_begin = 0;
  if constexpr (PACKED) {
    q_begin = min(max(sq.cu_q[b], 0), sq.total_q);
    const int q_end = min(max(sq.cu_q[b + 1], q_begin), sq.total_q);
    Nq = q_end - q_begin;
    if (q0 >= Nq) return;  // uniform over the workgroup, before any barrier
    if constexpr (MODE == kFwdRagged) {
      const int k_begin = min(max(sq.k_lens[b], 0), sq.total_k);
      Nk = min(max(sq.k_lens[b + 1], k_begin), sq.total_k) - k_begin;
      k_elem = ((size_t)k_begin * Hkv + g) * D;
    } else {
      Nk = min(max(sq.k_lens[b], 0), sq.max_blocks * sq.block_size);
    }
    q_elem = ((size_t)q_begin * H + h) * D;
  } else {
    q_elem = ((size_t)b * H + h) * (size_t)Nq * D;
    k_elem = ((size_t)b * Hkv + g) * (size_t)Nk * D;
  }
  constexpr int QS = PACKED ? 0 : ROW;  // query row stride when known at compile time
  const int qstride = PACKED ? H * ROW : QS;
  const int kstride = MODE == kFwdRagged ? Hkv * ROW : ROW;
  const int off = Nk - Nq;  // bottom-right causal alignment

  const buf_rsrc qrs = make_rsrc(Q + q_elem, (unsigned)Nq * (unsigned)qstride);
  const buf_rsrc krs = make_rsrc(K + k_elem, MODE == kFwdPaged ? 0u : (unsigned)Nk * (unsigned)kstride);
  const buf_rsrc vrs = make_rsrc(V + k_elem, MODE == kFwdPaged ? 0u : (unsigned)Nk * (unsigned)kstride);
  __bf16* Op = O + q_elem;
  float* Lp = PACKED ? LSE + (size_t)h * sq.total_q + q_begin
                     : LSE + ((size_t)b * H + h) * (size_t)Nq;

  const int qrow = q0 + wave * 32 + li;
  const int wave_row_lo = q0 + wave * 32;

  // Key tiles this query tile can see: t_lo .. t_hi.  With a band, the rows
  // of the tile see keys from (first position - win_left) to (last position
  // + win_right); causal is the band (unbounded, 0) ("Kernel structure":
  // causal and local masks change the visited tile range).
  int t_lo, t_hi;
  band_tiles(BAND, q0, BR, Nq, Nk, BC, win_left, win_right, t_lo, t_hi);
  int parts = 1;
  if (SPLIT) {
    // This workgroup's share of the key range ("Attention kernels",
    // FlashDecoding paragraph, applied to a prefill query tile): the tile's
    // key tiles cut into equal parts of at most chunk_tiles tiles.  An empty
    // share exits before any barrier (the condition is uniform over the
    // workgroup).  A tile of one part is written like an unsplit one.
    parts = (t_hi - t_lo + chunk_tiles) / chunk_tiles;
    if (!split_part(t_lo, t_hi, chunk_tiles, chunk)) return;
  }

  // The visited tiles as a sequence j = 0 .. n_iter - 1: the range t_lo ..
  // t_hi, or (sparse) the listed blocks' tiles in list order.  A listed block
  // outside the key range maps to -2: the step copies and computes nothing.
  int n_iter = t_hi - t_lo + 1;
  int sp_lo = 0, sp_base = 0, sp_cols = 0, n_kblk = 0;
  if constexpr (MODE == kFwdSparse) {
    const int lay = bh % sq.num_layouts;
    const int* rp = sq.row_ptr + (size_t)lay * (n_qtiles + 1);
    // Offsets are clamped into col_idx's nnz entries.
    sp_lo = min(max(rp[qt], 0), sq.nnz);
    const int cnt = min(max(rp[qt + 1], sp_lo), sq.nnz) - sp_lo;
    n_iter = cnt * TPB;
    n_kblk = (Nk + 127) / 128;
    sp_cols = lane < cnt ? sq.col_idx[sp_lo + lane] : -1;
  }
  auto tile_at = [&](int j) -> int {
    if constexpr (MODE == kFwdSparse) {
      const int bi = j / TPB;
      if (bi - sp_base >= 64) {  // next 64 entries of the row's list
        sp_base = bi & ~63;
        const int cnt = n_iter / TPB;
        sp_cols = sp_base + lane < cnt ? sq.col_idx[sp_lo + sp_base + lane] : -1;
      }
      const int blk = __builtin_amdgcn_readlane(sp_cols, bi - sp_base);
      const int t = blk * TPB + j % TPB;
      return (blk >= 0 && blk < n_kblk && t >= t_lo && t <= t_hi) ? t : -2;
    } else {
      return t_lo + j;
    }
  };

  // Queries of this lane's row as the B operand (Q^T); rows past Nq read 0.
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = __builtin_bit_cast(bf16x8,
                                buf_load16(qrs, qrow * (QS ? QS : qstride) + (16 * ks + 8 * hh) * 2, 0));

  // Direct copies: instruction `it` of this wave fills 16-byte LDS slots
  // p = (wave * NLOAD + it) * 64 + lane of a tile, i.e. row p / CH and
  // swizzled chunk p % CH; the lane loads the logical chunk that belongs there
  // (paged: relative to the wave's first row, whose page holds all WROWS rows).
  int goff[NLOAD];
#pragma unroll
  for (int it = 0; it < NLOAD; ++it) {
    const int p = (wave * NLOAD + it) * 64 + lane;
    const int row = p / CH;
    const int c = (p % CH) ^ tile_swz<D>(row);
    goff[it] = MODE == kFwdPaged ? (row - wave * WROWS) * (int)(sq.token_stride * 2) + c * 16
                              : row * kstride + c * 16;
  }
  int kofs[KS];   // K row (32 kb + li), chunk 2 ks + hh
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kofs[ks] = li * ROW + (((2 * ks + hh) ^ tile_swz<D>(li)) * 16);
  int vofs[NB][2];  // V transpose reads: rows 4 hh + tr_r (+8), columns 32 nb + 16 (li/16) + 4 tr_c
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int rr = 4 * hh + tr_r + 8 * hf;
      const int col = 32 * nb + 16 * (li >> 4) + 4 * tr_c;
      vofs[nb][hf] = rr * ROW + (((col >> 3) ^ tile_swz<D>(rr)) * 16) + (col & 7) * 2;
    }

  f32x16 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x16{};
  float m_run = -INFINITY;  // reference max, base-2 units (scores * scale * log2 e)
  float l_run = 0.f;        // this lane's partial running sum

  // Paged: the physical page of this wave's rows of tile t, read one step
  // before the copy that needs it.  A vector load (every lane the same
  // address): a scalar load would share its completion counter with the LDS
  // reads, so each step's first LDS wait would also wait for it (measured
  // 1.5% slower).
  const buf_rsrc tbl = make_rsrc(MODE == kFwdPaged ? sq.block_table + (size_t)b * sq.max_blocks
                                                   : nullptr,
                                 MODE == kFwdPaged ? (unsigned)sq.max_blocks * 4u : 0u);
  auto page_of = [&](int t) -> int {
    if constexpr (MODE == kFwdPaged) {
      if (t < 0) return -1;
      const int key = t * BC + wave * WROWS;
      if (key >= Nk) return -1;
      return __builtin_amdgcn_raw_buffer_load_b32(tbl, 0, page_div(key, sq) * 4, 0);
    } else {
      return 0;
    }
  };

  auto load_tile = [&](int t, char* dst, int* bad_dst, int phys) {
    if constexpr (MODE == kFwdPaged) {
      // A buffer resource over this wave's rows in their page: its range
      // ends after the last live token, and is empty for a page outside the
      // cache, so such rows arrive as zeros ("Failure modes": a page-table
      // mismatch must not read outside the cache) and are flagged so that
      // their keys get probability 0.
      phys = __builtin_amdgcn_readfirstlane(phys);
      const int key = t * BC + wave * WROWS;
      int live = min(max(Nk - key, 0), WROWS);
      const bool bad = live > 0 && (phys < 0 || phys >= sq.num_blocks);
      if (bad) live = 0;
      if (lane == 0) bad_dst[wave] = bad ? 1 : 0;
      unsigned long long eo = live ? (unsigned long long)phys * sq.block_stride +
                                         (unsigned long long)(key - page_div(key, sq) * sq.block_size) *
                                             sq.token_stride +
                                         (unsigned long long)g * sq.head_stride
                                   : 0;
      // All of it is wave-uniform; readfirstlane lets the compiler keep the
      // resources in SGPRs (no per-lane loop around the copies).
      live = __builtin_amdgcn_readfirstlane(live);
      const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)eo);
      const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(eo >> 32));
      eo = ((unsigned long long)hi << 32) | lo;
      const unsigned bytes = (unsigned)live * (unsigned)(sq.token_stride * 2);
      const buf_rsrc kp = make_rsrc(K + eo, bytes);
      const buf_rsrc vp = make_rsrc(V + eo, bytes);
#pragma unroll
      for (int it = 0; it < NLOAD; ++it) {
        char* slot = dst + (wave * NLOAD + it) * 1024;
        buf_load16_lds(kp, slot, goff[it], 0);
        buf_load16_lds(vp, slot + TILE, goff[it], 0);
      }
    } else {
      const int soff = t * BC * kstride;  // rows past Nk arrive as zeros (buffer range)
#pragma unroll
      for (int it = 0; it < NLOAD; ++it) {
        char* slot = dst + (wave * NLOAD + it) * 1024;
        buf_load16_lds(krs, slot, goff[it], soff);
        buf_load16_lds(vrs, slot + TILE, goff[it], soff);
      }
    }
  };

  // Pipeline state: tile of the current step, the next one (its copy is
  // issued at the start of the current step) and, paged, the next one's page.
  int t_cur = n_iter > 0 ? tile_at(0) : -2;
  int t_nxt = n_iter > 1 ? tile_at(1) : -1;
  int ph_nxt = page_of(t_nxt);

  auto step = [&](int j, const char* Ks, char* next, const int* Kbad, int* nbad) {
    const int t = t_cur;
    if (t_nxt >= 0) load_tile(t_nxt, next, nbad, ph_nxt);
    const int t_nn = j + 2 < n_iter ? tile_at(j + 2) : -1;
    ph_nxt = page_of(t_nn);
    t_cur = t_nxt;
    t_nxt = t_nn;
    const int k0 = t * BC;
    // Tiles wholly outside this wave's band contribute nothing.
    const bool wave_live = t >= 0 && (!BAND || (k0 <= wave_row_lo + 31 + off + win_right &&
                                               k0 + BC - 1 >= wave_row_lo + off - win_left));
    if (wave_live) {
      const char* Vs = Ks + TILE;
      // S^T for keys 32 kb .. 32 kb + 31 (s[kb]); with two blocks the
      // accumulation chains interleave; each k-step's K operands are read one
      // step ahead.
      f32x16 s[KB];
      bf16x8 a[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = f32x16{};
        a[kb] = *(const bf16x8*)(Ks + 32 * kb * ROW + kofs[0]);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 n[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          n[kb] = (ks + 1 < KS) ? *(const bf16x8*)(Ks + 32 * kb * ROW + kofs[ks + 1]) : a[kb];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) s[kb] = mfma32(a[kb], qf[ks], s[kb]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) a[kb] = n[kb];
      }

      // Mask the band's edges, the ragged key tail and (paged) the rows of
      // pages outside the cache.
      int badm = 0;
      if constexpr (MODE == kFwdPaged) {
#pragma unroll
        for (int w = 0; w < NW; ++w) badm |= (Kbad[w] != 0 ? 1 : 0) << w;
      }
      const bool need_mask =
          (k0 + BC > Nk) || badm != 0 ||
          (BAND && (k0 + BC - 1 > wave_row_lo + off + win_right ||
                    k0 < wave_row_lo + 31 + off - win_left));
      if (need_mask) {
        // Score r of block kb is key k0 + 4 hh + c with the constant
        // c = 32 kb + 8 (r >> 2) + (r & 3); the limits are taken relative to
        // k0 + 4 hh, so each score costs one compare with a constant per
        // limit.
        const int base = k0 + 4 * hh;
        const int hi_rel = (BAND ? min(Nk - 1, qrow + off + win_right) : Nk - 1) - base;
        const int lo_rel = BAND ? qrow + off - win_left - base : -(1 << 30);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * kb + 8 * (r >> 2) + (r & 3);
            const bool bad = MODE == kFwdPaged && ((badm >> ((c + 4 * hh) / WROWS)) & 1);
            if (c > hi_rel || c < lo_rel || bad) s[kb][r] = -INFINITY;
          }
      }

      // Online softmax update for this lane's row, P packed to bf16 as the
      // B operand of o^T += V^T P^T (16 keys per MFMA).  Common path: the
      // exponentials against the current reference, without the tile's
      // maximum.  When every lane's sum is at most 2^kSlack, no probability
      // exceeded 2^kSlack, so the maximum could not have moved the reference
      // and the result is exactly that of the full update below; otherwise
      // (or before the row's first visible key) the full update runs from
      // the scores, which are still intact.
      bf16x8 pb[KB][2];
      float rs = 0.f;
      auto exps = [&](float m_use) {
        rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * s2 + 2 * e;
              const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -m_use));
              const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], scale_log2, -m_use));
              rs += p0;
              rs += p1;
              w[e] = pack_bf16x2(p0, p1);
            }
            pb[kb][s2] = __builtin_bit_cast(bf16x8, w);
          }
      };
      bool full;
      if constexpr (D == 64) {
        // Until every row has seen a key (a wave's first tile) the common
        // path would be computed and thrown away: go straight to the full
        // update.  At d = 64, where the vector work sets the time, this
        // saves 1.5-2%; at d = 128 the extra branch cost as much as it saved.
        full = wave_any(m_run == -INFINITY);
        if (!full) {
          exps(m_run);
          full = wave_any(!(rs <= kSlackExp));
        }
      } else {
        exps(m_run == -INFINITY ? 0.f : m_run);
        full = wave_any(!(rs <= kSlackExp) || m_run == -INFINITY);
      }
      if (full) {
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int kb = 1; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        const float mx2 = halves_max(mx) * scale_log2;
        if (wave_any(mx2 > m_run + kSlack)) {
          const float m_new = fmaxf(m_run, mx2);
          // A row without a key so far has o = 0 and l = 0: the rescale
          // changes nothing, and at d = 64 a wave whose rows are all such
          // (its first tile) skips it (at d = 128 the branch cost six
          // registers for a smaller share of the work).
          if (!(D == 64 && __all(m_run == -INFINITY))) {
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[nb][r] *= alpha;
          }
          m_run = m_new;
        }
        exps(m_run == -INFINITY ? 0.f : m_run);
      }
      l_run += rs;
      // o^T += V^T P^T: 4 MFMAs per 32-column block, V^T operands read one
      // MFMA ahead.
      constexpr int PV = 2 * KB;  // 16-key MFMA steps per tile
      auto vread = [&](int i) {
        const int nb = i / PV, kb = (i % PV) >> 1, s2 = i & 1;
        const char* vb = Vs + (32 * kb + 16 * s2) * ROW;
        return join_tr(lds_read_tr(vb + vofs[nb][0]), lds_read_tr(vb + vofs[nb][1]));
      };
      bf16x8 va = vread(0);
#pragma unroll
      for (int i = 0; i < PV * NB; ++i) {
        const bf16x8 vn = (i + 1 < PV * NB) ? vread(i + 1) : va;
        o[i / PV] = mfma32(va, pb[(i % PV) >> 1][i & 1], o[i / PV]);
        va = vn;
      }
    }
    wait_vmem();
    __syncthreads();
  };

  if (t_cur >= 0) load_tile(t_cur, smem0, bad0, page_of(t_cur));
  wait_vmem();
  __syncthreads();
  // Unrolled by two so each step's LDS buffers are fixed objects.
  for (int j = 0; j < n_iter; j += 2) {
    step(j, smem0, smem1, bad0, bad1);
    if (j + 1 < n_iter) step(j + 1, smem1, smem0, bad1, bad0);
  }

  const float l_tot = halves_sum(l_run);
  if (SPLIT && parts > 1) {
    // Partial of this key range, merged by fwd_merge_kernel: o / l in bf16
    // (whole rows through the wave's slice of the idle K/V buffers, as the
    // final O below), then the base-2 reference max and the sum l in fp32.
    // Normalised, the bf16 rows hold values no larger than V's; the merge
    // weights them by l 2^(m - M), so their rounding adds at most one bf16
    // step of the largest |V| to O.
    const size_t prow0 = (((size_t)bh * n_qtiles + qt) * n_chunks + chunk) * BR + wave * 32;
    __bf16* po = (__bf16*)part;
    static_assert(NW * 32 * ROW <= 4 * TILE, "partial staging fits the K/V buffers");
    store_tile_rows<D>(o, l_tot > 0.f ? 1.f / l_tot : 0.f,
                       wave < 2 ? smem0 + wave * 32 * ROW : smem1 + (wave - 2) * 32 * ROW,
                       po + prow0 * D, D, Nq - wave_row_lo, lane);
    if (qrow < Nq && hh == 0) {
      float* pml = (float*)(po + (size_t)BH * n_qtiles * n_chunks * BR * D) + (prow0 + li) * 2;
      pml[0] = m_run;
      pml[1] = l_tot;
    }
    return;
  }
  // Epilogue: one division per row, O in bf16 stored as whole rows through
  // the wave's slice of the (now idle) K/V buffers, LSE in natural log.
  {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    static_assert(NW * 32 * ROW <= 4 * TILE, "O staging fits the K/V buffers");
    char* stage = wave < 2 ? smem0 + wave * 32 * ROW : smem1 + (wave - 2) * 32 * ROW;
    const size_t rs = PACKED ? (size_t)H * D : (size_t)D;
    store_tile_rows<D>(o, inv, stage, Op + (size_t)wave_row_lo * rs, rs, Nq - wave_row_lo, lane);
    if (qrow < Nq && hh == 0) Lp[qrow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge of the key-split partials of each query row (the split-context
// algebra of "Attention kernels", FlashDecoding paragraph): M = max_c m_c,
// w_c = 2^(m_c - M) l_c, l = sum_c w_c, O = sum_c w_c (o_c / l_c) / l,
// LSE = (M + log2 l) ln 2.  A tile of one part was written by its unit and
// is skipped.  D/4 threads per row, four columns each (8-byte loads); each
// thread takes two rows 256 / (D/4) apart, with up to eight parts' loads of
// both in flight.
template <int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(
    const float* __restrict__ part, __bf16* __restrict__ O, float* __restrict__ LSE, int BH,
    int Nq, int Nk, int n_qtiles, int n_chunks, int chunk_tiles, int band, int win_left,
    int win_right) {
  constexpr int BR = 128;
  constexpr int BC = fwd_bc<D>();
  constexpr int TPR = D / 4;
  constexpr int RPP = 256 / TPR;  // rows per pass of the workgroup
  constexpr int PR = 2;           // rows per thread, their loads in flight together
  constexpr int kBatch = 8;
  static_assert(BR % (PR * RPP) == 0, "a workgroup's rows lie in one query tile");
  const int bh = blockIdx.y;
  const int row_a = blockIdx.x * (PR * RPP) + (int)threadIdx.x / TPR;
  const int n4 = ((int)threadIdx.x % TPR) * 4;
  if (row_a >= Nq) return;
  const int qt = row_a / BR;
  int t_lo, t_hi;
  band_tiles(band != 0, qt * BR, BR, Nq, Nk, BC, win_left, win_right, t_lo, t_hi);
  // Every part of a tile is non-empty: with p = ceil(n / chunk_tiles) parts
  // of ceil(n / p) tiles, the last starts at (p - 1) ceil(n / p) < n.
  int parts = t_lo <= t_hi ? (t_hi - t_lo + chunk_tiles) / chunk_tiles : 0;
  if (parts == 1) return;
  parts = min(parts, n_chunks);
  const __bf16* po = (const __bf16*)part;
  const float* ml = (const float*)(po + (size_t)BH * n_qtiles * n_chunks * BR * D);
  const size_t tile0 = ((size_t)bh * n_qtiles + qt) * n_chunks * BR;
  float big_m[PR], ell[PR];
  f32x4 acc[PR];
#pragma unroll
  for (int i = 0; i < PR; ++i) {
    big_m[i] = -INFINITY;
    ell[i] = 0.f;
    acc[i] = f32x4{};
  }
  for (int c0 = 0; c0 < parts; c0 += kBatch) {
    float mv[PR][kBatch], lv[PR][kBatch];
    f32x4 ov[PR][kBatch];
#pragma unroll
    for (int i = 0; i < PR; ++i)
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int row = row_a + i * RPP;
        const bool ok = c0 + j < parts && row < Nq;
        const size_t prow = tile0 + (size_t)(ok ? c0 + j : 0) * BR + (ok ? row % BR : 0);
        mv[i][j] = ok ? ml[prow * 2] : -INFINITY;
        lv[i][j] = ok ? ml[prow * 2 + 1] : 0.f;
        const u32x2 pv = ok ? *(const u32x2*)(po + prow * D + n4) : u32x2{};
        ov[i][j] = f32x4{__builtin_bit_cast(float, pv[0] << 16),
                         __builtin_bit_cast(float, pv[0] & 0xffff0000u),
                         __builtin_bit_cast(float, pv[1] << 16),
                         __builtin_bit_cast(float, pv[1] & 0xffff0000u)};
      }
#pragma unroll
    for (int i = 0; i < PR; ++i) {
      float bm = big_m[i];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) bm = fmaxf(bm, mv[i][j]);
      if (bm == -INFINITY) continue;
      const float r = fast_exp2(big_m[i] - bm);
      acc[i] *= r;
      ell[i] *= r;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float w = fast_exp2(mv[i][j] - bm) * lv[i][j];
        ell[i] += w;
        acc[i] += w * ov[i][j];
      }
      big_m[i] = bm;
    }
  }
#pragma unroll
  for (int i = 0; i < PR; ++i) {
    const int row = row_a + i * RPP;
    if (row >= Nq) continue;
    const float inv = ell[i] > 0.f ? 1.f / ell[i] : 0.f;
    const size_t orow = (size_t)bh * Nq + row;
    u32x2 w;
    w[0] = pack_bf16x2(acc[i][0] * inv, acc[i][1] * inv);
    w[1] = pack_bf16x2(acc[i][2] * inv, acc[i][3] * inv);
    *(u32x2*)(O + orow * D + n4) = w;
    if (n4 == 0) LSE[orow] = ell[i] > 0.f ? (big_m[i] + fast_log2(ell[i])) * kLn2 : -INFINITY;
  }
}

// fp32 path: the same tiling on v_mfma_f32_32x32x2f32 (P stays fp32).
// One wave = 32 query rows, 32-key tiles.  Lane (i = l%32, h = l/32) holds
// query row i; k-step 4*kk + t pairs lane half h with d = 8*kk + 4*h + t, so
// K and Q operands come from one 16-byte read per four k-steps.
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int B, int H, int Hkv, int Nq, int Nk,
    float scale_log2, int n_qtiles) {
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int BC = 32;
  constexpr int CH = D / 4;   // 16-byte chunks per fp32 row
  constexpr int NLOAD = BC * CH / NT;
  constexpr int KK = D / 8;   // 16-byte groups of k-steps
  constexpr int NB = D / 32;
  static_assert(BC * CH % NT == 0, "tile load split");

  __shared__ __attribute__((aligned(16))) float smem[2][BC * D];  // [K|V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int hh = lane >> 5;

  const int BH = B * H;
  const int wg = blockIdx.x;
  const int qt = n_qtiles - 1 - wg / BH;
  const int bh = wg % BH;
  const int b = bh / H;
  const int h = bh % H;
  const int g = h / (H / Hkv);
  const int q0 = qt * BR;
  const int off = Nk - Nq;

  const float* Qp = Q + ((size_t)b * H + h) * (size_t)Nq * D;
  const float* Kp = K + ((size_t)b * Hkv + g) * (size_t)Nk * D;
  const float* Vp = V + ((size_t)b * Hkv + g) * (size_t)Nk * D;
  float* Op = O + ((size_t)b * H + h) * (size_t)Nq * D;
  float* Lp = LSE + ((size_t)b * H + h) * (size_t)Nq;

  const int qrow = q0 + wave * 32 + li;
  int n_tiles;
  if (CAUSAL) {
    int last = min(Nk - 1, q0 + BR - 1 + off);
    n_tiles = last < 0 ? 0 : last / BC + 1;
  } else {
    n_tiles = (Nk + BC - 1) / BC;
  }

  f32x4 qf[KK];
  {
    const bool ok = qrow < Nq;
    const float* src = Qp + (size_t)(ok ? qrow : 0) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = ok ? *(const f32x4*)(src + 8 * kk + 4 * hh) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  f32x16 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * BC;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NLOAD; ++it) {
      const int cid = tid + it * NT;
      const int row = cid / CH;
      const int c = cid % CH;
      const int key = k0 + row;
      f32x4 kv = f32x4{0.f, 0.f, 0.f, 0.f}, vv = kv;
      if (key < Nk) {
        kv = *(const f32x4*)(Kp + (size_t)key * D + c * 4);
        vv = *(const f32x4*)(Vp + (size_t)key * D + c * 4);
      }
      *(f32x4*)(&smem[0][row * D + ((c ^ (row & (CH - 1))) * 4)]) = kv;
      *(f32x4*)(&smem[1][row * D + c * 4]) = vv;
    }
    __syncthreads();

    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int c = 2 * kk + hh;
      const f32x4 a = *(const f32x4*)(&smem[0][li * D + ((c ^ (li & (CH - 1))) * 4)]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) s = mfma32_f32(a[tt], qf[kk][tt], s);
    }
    const bool need_mask = (k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > q0 + wave * 32 + off));
    if (need_mask) {
      const int lim = CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key > lim) s[r] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -m_use));
      s[r] = p;
      rs += p;
    }
    l_run = alpha * l_run + rs;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nb][r] *= alpha;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
        const float a = smem[1][key * D + 32 * nb + li];
        o[nb] = mfma32_f32(a, s[r], o[nb]);
      }
  }

  const float l_tot = l_run + swap_halves(l_run);
  if (qrow < Nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* dst = Op + (size_t)qrow * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = 32 * nb + 8 * r4 + 4 * hh;
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[nb][4 * r4 + e] * inv;
        *(f32x4*)(dst + n) = w;
      }
    if (hh == 0) Lp[qrow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

// fp32 path for small grids: one workgroup per 32 query rows, its NW
// waves splitting the key range (wave w takes key tiles w, w + NW, ...), each
// with its own running (m, l, o) for the same rows, merged through LDS at the
// end with the split-context algebra of "Attention kernels", FlashDecoding
// paragraph: M = max_w m_w, l = sum_w 2^(m_w - M) l_w, O = sum_w 2^(m_w - M)
// o_w / l.  With few query rows the per-tile chain of fp32 MFMAs is the
// latency; splitting the keys NW ways shortens it.  Each wave stages
// its own K tile, then its V tile, in a private slice of LDS.  Operand
// layouts as in fwd_f32_kernel.
template <int D, bool CAUSAL, int NW, bool PREFETCH>
__global__ __launch_bounds__(NW * 64) void fwd_f32_ksplit_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int B, int H, int Hkv, int Nq, int Nk,
    float scale_log2, int n_rtiles) {
  constexpr int BC = 32;
  constexpr int CH = D / 4;   // 16-byte chunks per fp32 row
  constexpr int LOADS = BC * CH / 64;
  constexpr int KK = D / 8;
  constexpr int NB = D / 32;

  __shared__ __attribute__((aligned(16))) float slice[NW][BC * D];  // K, then V, then o
  __shared__ float part_m[NW][32];
  __shared__ float part_l[NW][32];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31;
  const int hh = lane >> 5;

  const int BH = B * H;
  const int rt = n_rtiles - 1 - (int)blockIdx.x / BH;  // heavy (late) row tiles first
  const int bh = (int)blockIdx.x % BH;
  const int b = bh / H;
  const int h = bh % H;
  const int g = h / (H / Hkv);
  const int q0 = rt * 32;
  const int off = Nk - Nq;
  const int qrow = q0 + li;

  const float* Qp = Q + ((size_t)b * H + h) * (size_t)Nq * D;
  const float* Kp = K + ((size_t)b * Hkv + g) * (size_t)Nk * D;
  const float* Vp = V + ((size_t)b * Hkv + g) * (size_t)Nk * D;
  float* tile = slice[wave];

  int n_tiles;
  if (CAUSAL) {
    const int last = min(Nk - 1, q0 + 31 + off);
    n_tiles = last < 0 ? 0 : last / BC + 1;
  } else {
    n_tiles = (Nk + BC - 1) / BC;
  }

  f32x4 qf[KK];
  {
    const bool ok = qrow < Nq;
    const float* src = Qp + (size_t)(ok ? qrow : 0) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = ok ? *(const f32x4*)(src + 8 * kk + 4 * hh) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  f32x16 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // K and V rows of key tile t into registers (rows past Nk as zeros).
  f32x4 kv[LOADS], vv[LOADS];
  auto fetch = [&](int t) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int cid = lane + it * 64;
      const int key = t * BC + cid / CH;
      const int c = cid % CH;
      kv[it] = vv[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < n_tiles && key < Nk) {
        kv[it] = *(const f32x4*)(Kp + (size_t)key * D + c * 4);
        vv[it] = *(const f32x4*)(Vp + (size_t)key * D + c * 4);
      }
    }
  };
  if (PREFETCH) fetch(wave);
  for (int t = wave; t < n_tiles; t += NW) {
    const int k0 = t * BC;
    // This tile's K goes to the slice now, its V after the scores (the
    // wave's LDS accesses run in program order); with PREFETCH the next
    // tile's rows are fetched meanwhile.
    if (!PREFETCH) fetch(t);
    f32x4 vcur[LOADS];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) vcur[it] = vv[it];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int cid = lane + it * 64;
      const int row = cid / CH;
      const int c = cid % CH;
      *(f32x4*)(&tile[row * D + ((c ^ (row & (CH - 1))) * 4)]) = kv[it];
    }
    if (PREFETCH) fetch(t + NW);
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int c = 2 * kk + hh;
      const f32x4 a = *(const f32x4*)(&tile[li * D + ((c ^ (li & (CH - 1))) * 4)]);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) s = mfma32_f32(a[tt], qf[kk][tt], s);
    }
    const bool need_mask = (k0 + BC > Nk) || (CAUSAL && (k0 + BC - 1 > q0 + off));
    if (need_mask) {
      const int lim = CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key > lim) s[r] = -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(__builtin_fmaf(s[r], scale_log2, -m_use));
      s[r] = p;
      rs += p;
    }
    l_run = alpha * l_run + rs;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[nb][r] *= alpha;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int cid = lane + it * 64;
      *(f32x4*)(&tile[(cid / CH) * D + (cid % CH) * 4]) = vcur[it];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
        o[nb] = mfma32_f32(tile[key * D + 32 * nb + li], s[r], o[nb]);
      }
  }

  // Publish this wave's partial: o as rows of its slice, m and l per row.
  const float l_tot = l_run + swap_halves(l_run);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = o[nb][4 * r4 + e];
      *(f32x4*)(&tile[li * D + 32 * nb + 8 * r4 + 4 * hh]) = w;
    }
  if (hh == 0) {
    part_m[wave][li] = m_run;
    part_l[wave][li] = l_tot;
  }
  __syncthreads();

  // Merge: the workgroup's threads take the 32 rows' 16-byte chunks in turn.
  constexpr int ITEMS = 32 * CH;
#pragma unroll
  for (int i0 = 0; i0 < ITEMS; i0 += NW * 64) {
    const int i = i0 + (int)threadIdx.x;
    if (ITEMS % (NW * 64) != 0 && i >= ITEMS) break;
    const int r = i / CH;
    const int c = i % CH;
    const int row = q0 + r;
    float big_m = part_m[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) big_m = fmaxf(big_m, part_m[w][r]);
    const float m_ref = big_m == -INFINITY ? 0.f : big_m;
    float ell = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2(part_m[w][r] - m_ref);
      ell += wt * part_l[w][r];
      acc += wt * *(const f32x4*)(&slice[w][r * D + c * 4]);
    }
    if (row < Nq) {
      const float inv = ell > 0.f ? 1.f / ell : 0.f;
      *(f32x4*)(O + (((size_t)b * H + h) * (size_t)Nq + row) * D + c * 4) = acc * inv;
      if (c == 0)
        LSE[((size_t)b * H + h) * (size_t)Nq + row] =
            ell > 0.f ? (big_m + fast_log2(ell)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool BAND>
hipError_t launch_bf16(const FwdArgs& a, const FwdPlan& p, hipStream_t stream) {
  constexpr int BC = fwd_bc<D>();
  const float sl2 = a.scale * kLog2e;
  const __bf16* q = (const __bf16*)a.Q;
  const __bf16* k = (const __bf16*)a.K;
  const __bf16* v = (const __bf16*)a.V;
  __bf16* o = (__bf16*)a.O;
  if (a.mode != kFwdDense) {
    // Packed ragged rows, paged K/V or a sparse block list: four waves,
    // 128-row query tiles; a.Nq bounds every sequence's query rows.
    const int n_qt = (a.Nq + 127) / 128;
    dim3 grid((unsigned)((long long)n_qt * a.B * a.H));
#define ETA_LAUNCH_MODE(M)                                                                      \
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BAND, 4, BC, false, M>), grid, dim3(256), 0, stream, q, \
                     k, v, o, a.LSE, a.B, a.H, a.Hkv, a.Nq, a.Nk, sl2, n_qt, a.win_left,         \
                     a.win_right, 0, 0, nullptr, a.seq)
    if (a.mode == kFwdRagged) ETA_LAUNCH_MODE(kFwdRagged);
    else if (a.mode == kFwdPaged) ETA_LAUNCH_MODE(kFwdPaged);
    else ETA_LAUNCH_MODE(kFwdSparse);
#undef ETA_LAUNCH_MODE
    return hipGetLastError();
  }
  if (a.n_chunks > 0) {
    // Key split: always four waves, 128-row query tiles (whatever the
    // unsplit plan's workgroup size), the tiling the host sized the
    // workspace for; partials, then the merge.
    const int n_qt = (a.Nq + 127) / 128;
    float* part = (float*)a.workspace;
    dim3 grid((unsigned)((long long)a.split_units * a.B * a.H));
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BAND, 4, BC, true, kFwdDense>), grid, dim3(256), 0, stream,
                       q, k, v, o, a.LSE, a.B, a.H, a.Hkv, a.Nq, a.Nk, sl2, n_qt, a.win_left,
                       a.win_right, a.chunk_tiles, a.n_chunks, part, FwdSeqArgs{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int rpb = 2 * (256 / (D / 4));
    hipLaunchKernelGGL((fwd_merge_kernel<D>),
                       dim3((unsigned)((a.Nq + rpb - 1) / rpb), (unsigned)(a.B * a.H)), dim3(256), 0,
                       stream, (const float*)part, o, a.LSE, a.B * a.H, a.Nq, a.Nk,
                       n_qt, a.n_chunks, a.chunk_tiles, a.band, a.win_left, a.win_right);
    return hipGetLastError();
  }
  const int br = p.block_rows;  // the planner's tile: 64 or 128 query rows
  if (br != 64 && br != 128) return hipErrorInvalidValue;
  const int n_qtiles = (a.Nq + br - 1) / br;
  dim3 grid((unsigned)(n_qtiles * a.B * a.H));
  if (p.waves == 4) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BAND, 4, BC, false, kFwdDense>), grid, dim3(256), 0, stream,
                       q, k, v, o, a.LSE, a.B, a.H, a.Hkv, a.Nq, a.Nk, sl2, n_qtiles, a.win_left,
                       a.win_right, 0, 0, nullptr, FwdSeqArgs{});
  } else {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BAND, 2, BC, false, kFwdDense>), grid, dim3(128), 0, stream,
                       q, k, v, o, a.LSE, a.B, a.H, a.Hkv, a.Nq, a.Nk, sl2, n_qtiles, a.win_left,
                       a.win_right, 0, 0, nullptr, FwdSeqArgs{});
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdArgs& a, const FwdPlan& p, hipStream_t stream) {
  if (p.key_parts > 1) {
    // d = 64: eight waves (two per SIMD, each covering the other's
    // latencies); d = 128: four waves, each fetching its next tile's rows
    // ahead (two waves would not fit the registers).  Single head, 512 keys:
    // d = 64 with four waves and prefetch 17.0 us, eight without 15.3 us,
    // eight with 16.0 us, sixteen 28.8 us.
    constexpr int NWK = D == 64 ? 8 : 4;
    constexpr bool PF = D != 64;
    const int n_rtiles = (a.Nq + 31) / 32;
    hipLaunchKernelGGL((fwd_f32_ksplit_kernel<D, CAUSAL, NWK, PF>),
                       dim3((unsigned)(n_rtiles * a.B * a.H)), dim3(NWK * 64), 0, stream,
                       (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O,
                       a.LSE, a.B, a.H, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, n_rtiles);
    return hipGetLastError();
  }
  constexpr int NW = 4;
  const int n_qtiles = (a.Nq + NW * 32 - 1) / (NW * 32);
  dim3 grid((unsigned)(n_qtiles * a.B * a.H));
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, NW>), grid, dim3(NW * 64), 0, stream,
                     (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O, a.LSE,
                     a.B, a.H, a.Hkv, a.Nq, a.Nk, a.scale * kLog2e, n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, const FwdPlan& p, hipStream_t stream) {
  if (a.dtype_bf16) {
    if (a.d == 128)
      return a.band ? launch_bf16<128, true>(a, p, stream) : launch_bf16<128, false>(a, p, stream);
    return a.band ? launch_bf16<64, true>(a, p, stream) : launch_bf16<64, false>(a, p, stream);
  }
  if (a.d == 128)
    return a.causal ? launch_f32<128, true>(a, p, stream) : launch_f32<128, false>(a, p, stream);
  return a.causal ? launch_f32<64, true>(a, p, stream) : launch_f32<64, false>(a, p, stream);
}

}  // namespace eta
