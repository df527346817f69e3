// Internal interface between the C-ABI host layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace eta {

// A window side with no limit (larger than any sequence the library accepts).
constexpr int kUnbounded = 1 << 30;

constexpr int kNumCU = 256;  // MI355X compute units

// Extra inputs of the forward's packed-ragged, paged and sparse modes
// (all zero for dense rows).  Device pointers; sizes are host values.
struct FwdSeqArgs {
  const int* cu_q;         // ragged / paged: [num_seqs + 1] query row offsets
  const int* k_lens;       // ragged: cu_k [num_seqs + 1]; paged: seqlens_k [num_seqs]
  const int* block_table;  // paged: [num_seqs, max_blocks]
  const int* row_ptr;      // sparse: [num_layouts, ceil(Nq/128) + 1]
  const int* col_idx;      // sparse: listed 128-key blocks
  int total_q, total_k;    // packed row counts
  int max_blocks, num_blocks, block_size;  // paged cache geometry
  unsigned page_magic;     // paged: key / block_size == (key * page_magic) >> page_shift
  int page_shift;
  int num_layouts;         // sparse: layout of (b, h) = (b * H + h) % num_layouts
  int nnz;                 // sparse: entries of col_idx
  long long block_stride, token_stride, head_stride;  // paged cache strides (elements)
};

// Row layout / tile visitation of the bf16 forward (see fwd.hip).
enum FwdModeTag : int { kFwdDense = 0, kFwdRagged = 1, kFwdPaged = 2, kFwdSparse = 3 };

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int causal;          // fp32 path: causal mask or none
  // Banded mask (bf16 path): key j is visible from query position p (bottom-
  // right aligned) iff p - win_left <= j <= p + win_right; kUnbounded on a
  // side means no limit there.  causal = (kUnbounded, 0).
  int band;            // 0: every key visible (win_* ignored)
  int win_left, win_right;
  bool dtype_bf16;
  // Key split (bf16 path; n_chunks = 0: none): each 128-row query tile's key
  // tiles are cut into equal parts of at most chunk_tiles tiles (n_chunks
  // bounds the part count), computed as separate workgroups into `workspace`
  // and merged.
  int chunk_tiles, n_chunks;
  int split_units;     // (query tile, part) pairs with work (the grid / (B*H))
  void* workspace;
  // Mode (FwdModeTag) and its extra inputs.  Ragged / paged: B = num_seqs,
  // Nq = the longest sequence's query rows, Nk unused.
  int mode;
  FwdSeqArgs seq;
};

// Key tiles of width BC seen by the query rows q0 .. q0 + rows - 1: t_lo .. t_hi
// (empty when t_lo > t_hi).  With a band, the rows see keys from (first
// position - win_left) to (last position + win_right), positions bottom-right
// aligned; causal is the band (kUnbounded, 0).
__host__ __device__ inline void band_tiles(bool band, int q0, int rows, int Nq, int Nk, int BC,
                                           int win_left, int win_right, int& t_lo, int& t_hi) {
  const int off = Nk - Nq;
  if (band) {
    const int last = (q0 + rows < Nq ? q0 + rows : Nq) - 1;
    const int k_lo = q0 + off - win_left > 0 ? q0 + off - win_left : 0;
    const int k_hi = last + off + win_right < Nk - 1 ? last + off + win_right : Nk - 1;
    t_lo = k_lo / BC;
    t_hi = k_lo <= k_hi ? k_hi / BC : t_lo - 1;
  } else {
    t_lo = 0;
    t_hi = (Nk + BC - 1) / BC - 1;
  }
}

// Division of 31-bit token positions by a page size bs without a divide:
// with l = ceil(log2 bs) and m = floor(2^(31+l) / bs) + 1, pos / bs ==
// (pos * m) >> (31 + l) for every 0 <= pos < 2^31 (the error
// pos * (m - 2^(31+l) / bs) / 2^(31+l) stays below 1 / bs), and m < 2^32.
inline void page_magic(int bs, unsigned& magic, int& shift) {
  int l = 0;
  while ((1LL << l) < bs) ++l;
  magic = (unsigned)((1ULL << (31 + l)) / (unsigned long long)bs + 1);
  shift = 31 + l;
}

// Key-tile width of the bf16 forward for head dimension d.
inline int fwd_tile_keys(int d) { return d == 128 ? 32 : 64; }

struct FwdPlan {
  int waves;        // waves per workgroup
  int rows_per_wave;  // query rows per wave
  int block_rows;   // query rows per workgroup
  int block_keys;   // keys per K/V tile
  long long workgroups;
  int key_parts = 1;  // > 1: the waves of a workgroup split the keys of the same rows (fp32)
};

struct DecodeArgs {
  const void* Q;
  const void* K_cache;
  const void* V_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  void* O;
  float* LSE;
  int num_seqs, Hq, Hkv, d, block_size, num_blocks, max_blocks_per_seq, max_context;
  int64_t block_stride, token_stride, head_stride;
  float scale;
  void* workspace;
};

// Split plan of the paged decode.  The live 32-token steps of all (sequence,
// KV head) pairs, laid end to end sequence-major, are cut into equal ranges
// of q steps, one per split wave.  q is fixed by the caller (steps_fixed > 0,
// at most kDecodeMaxSteps) or chosen on the device from the total step
// count U, which only the device knows: q = max(ceil(U / target_waves),
// kDecodeMinSteps).  The grid holds n_waves waves, enough for any U the
// sizes allow; waves past ceil(U / q) exit at once.
constexpr int kDecodeStepTokens = 32;
constexpr int kDecodeMaxSteps = 127;  // 4064 tokens: block-table entries in 4 registers
#ifndef ETA_DECODE_MIN_STEPS
#define ETA_DECODE_MIN_STEPS 2
#endif
constexpr int kDecodeMinSteps = ETA_DECODE_MIN_STEPS;
struct DecodePlan {
  int steps_fixed;      // q when > 0
  int target_waves;     // split waves of the automatic plan
  long long n_waves;    // waves in the split grid
};
// Split waves of the automatic plan for head dimension d: one workgroup of
// four waves per CU.  Measured over six batch shapes (64 x 4k-32k tokens,
// 256 x 1k-4k, 16 x 32k-64k, 128 x 2k-16k with 2 KV heads, 32 x 8k, 8 x 1k-2k):
// 2048 waves (all resident at 2 per SIMD) streamed 1-6% slower at d = 128,
// 17% slower at d = 64; 1536 waves, which leave some CUs with two workgroups
// and others with one, slower still; 768 (192 CUs busy) within 3% either
// way; 512 8-15% slower.  Ranges of equal length gain nothing from uneven
// CU loads, so the count is a multiple of the CU count.
#ifndef ETA_DECODE_WAVES_D128
#define ETA_DECODE_WAVES_D128 1024
#endif
#ifndef ETA_DECODE_WAVES_D64
#define ETA_DECODE_WAVES_D64 1024
#endif
inline int decode_target_waves(int d) {
  return d == 128 ? ETA_DECODE_WAVES_D128 : ETA_DECODE_WAVES_D64;
}
// (sequence, KV head, subgroup of at most 16 query heads) pairs of a decode.
inline long long decode_pairs(int num_seqs, int Hkv, int G) {
  return (long long)num_seqs * Hkv * ((G + 15) / 16);
}
// Waves the split grid needs for that many pairs of at most max_context
// tokens.
long long decode_split_waves(long long pairs, int d, int max_context, int steps_fixed);

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* LSE;
  void* dQ;
  void* dK;
  void* dV;
  int B, H, Hkv, Nq, Nk, d;
  float scale;
  int band;            // as in FwdArgs
  int win_left, win_right;
  void* workspace;
};

hipError_t launch_fwd(const FwdArgs& a, const FwdPlan& p, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
size_t decode_workspace_bytes(long long pairs, int G, int d, long long n_waves);
size_t bwd_workspace_bytes(int B, int H, int Nq, int d);

}  // namespace eta
