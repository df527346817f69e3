// C-ABI entry points: argument validation, planning and launches.
//
// Validation happens entirely on the host before anything is enqueued, so a
// rejected call touches neither the device nor the stream.  The planner is a
// pure function of the shapes ("Modern attention kernels", "Work
// partitioning in FlashAttention-2": kernel selection needs batch, heads,
// sequence length and head dimension; "Prefill and decode need different
// kernels": record the choice per phase).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/attn.h"
#include "kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";

attn_status_t fail(attn_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

attn_status_t ok() {
  g_last_error[0] = '\0';
  return ATTN_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

using eta::kNumCU;

constexpr long long kMaxGrid = 0x7fffffffLL;

}  // namespace

// Scratch of attn_decode_paged_noalloc (the split partials and the pairs'
// segment ids, the same contents as attn_decode_paged's workspace): a
// file-scope device array, so that entry point never allocates.  Every GPU
// the library runs on holds its own copy until the process ends.  In host
// code the name `scratch` is only a stand-in for the symbol: the device
// address comes from hipGetSymbolAddress, once per device (decode_scratch).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev` (the current device), looked
// up on the first call for that device and kept.
attn_status_t decode_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

// ---------------------------------------------------------------- forward

eta::FwdPlan plan_fwd(int B, int H, int Nq, int d, bool bf16) {
  eta::FwdPlan p;
  p.rows_per_wave = 32;
  if (bf16) {
    // One wave = 32 query rows.  Four waves per workgroup share each K/V
    // tile; when that leaves fewer than two workgroups per CU, halve the
    // workgroup so the causal work spreads over more CUs.
    p.waves = 4;
    long long wgs = (long long)B * H * ((Nq + 127) / 128);
    if (wgs < 2LL * kNumCU) p.waves = 2;
    p.block_keys = d == 128 ? 32 : 64;
  } else {
    p.waves = 4;
    p.block_keys = 32;
    // Fewer 128-row tiles than CUs: 32-row workgroups whose waves (8 at
    // d = 64, 4 at d = 128) split the keys (each wave's chain of fp32 MFMAs
    // is the latency there).
    if ((long long)B * H * ((Nq + 127) / 128) < kNumCU) p.key_parts = d == 64 ? 8 : 4;
  }
  p.block_rows = p.key_parts > 1 ? p.rows_per_wave : p.rows_per_wave * p.waves;
  p.workgroups = (long long)B * H * ((Nq + p.block_rows - 1) / p.block_rows);
  return p;
}

attn_status_t check_fwd_shape(int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                              attn_dtype_t dtype) {
  if (B < 1 || H < 1 || Hkv < 1 || Nq < 1 || Nk < 1)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d H=%d Hkv=%d Nq=%d Nk=%d)", B, H,
                Hkv, Nq, Nk);
  if (H % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "H=%d is not a multiple of Hkv=%d", H, Hkv);
  if (dtype != ATTN_DTYPE_F32 && dtype != ATTN_DTYPE_BF16)
    return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(ATTN_ERR_INVALID_ARG, "scale must be positive and finite");
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension %d not in {64,128}", d);
  const long long rows = (long long)B * H * Nq;
  if (rows * d > (1LL << 46)) return fail(ATTN_ERR_INVALID_ARG, "tensor too large");
  // One head's rows are addressed with 32-bit byte offsets.
  const long long elt = dtype == ATTN_DTYPE_BF16 ? 2 : 4;
  if ((long long)(Nq > Nk ? Nq : Nk) * d * elt >= (1LL << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "sequence too long: one head's rows exceed 2 GiB");
  return ATTN_OK;
}

// Layout identity of a paged cache ("Failure modes": page-table mismatch):
// the strides (elements) must place the block_size x Hkv rows of d values
// of a page without overlap, 16-byte aligned, either token-major
// ([block, slot, head, d]: head_stride >= d, token_stride >= Hkv *
// head_stride) or head-major ([block, head, slot, d]: token_stride >= d,
// head_stride >= block_size * token_stride), with pages not overlapping.
bool page_layout_ok(int d, int Hkv, int block_size, int64_t block_stride, int64_t token_stride,
                    int64_t head_stride) {
  if (head_stride % 8 || token_stride % 8 || block_stride % 8) return false;
  if (head_stride >= d && token_stride >= (int64_t)Hkv * head_stride)
    return block_stride >= (int64_t)block_size * token_stride;
  if (token_stride >= d && head_stride >= (int64_t)block_size * token_stride)
    return block_stride >= (int64_t)Hkv * head_stride;
  return false;
}

// Window sides as the kernels take them: -1 (no limit) becomes kUnbounded.
bool window_sides(int window_left, int window_right, int* left, int* right) {
  if (window_left < -1 || window_right < -1) return false;
  *left = window_left < 0 ? eta::kUnbounded : window_left;
  *right = window_right < 0 ? eta::kUnbounded : window_right;
  return true;
}

// ----------------------------------------------------------------- decode

attn_status_t check_decode_shape(int num_seqs, int Hq, int Hkv, int d, int block_size,
                                 int num_blocks, int max_blocks_per_seq, int max_context,
                                 int chunk_tokens) {
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || block_size < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1 || max_context < 0)
    return fail(ATTN_ERR_INVALID_ARG,
                "bad decode sizes (num_seqs=%d Hq=%d Hkv=%d block_size=%d num_blocks=%d "
                "max_blocks_per_seq=%d max_context=%d)",
                num_seqs, Hq, Hkv, block_size, num_blocks, max_blocks_per_seq, max_context);
  if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension %d not in {64,128}", d);
  if ((long long)max_context > (long long)max_blocks_per_seq * block_size)
    return fail(ATTN_ERR_INVALID_ARG, "max_context=%d exceeds block table capacity %lld",
                max_context, (long long)max_blocks_per_seq * block_size);
  if (chunk_tokens < 0 || chunk_tokens % 32 != 0 || chunk_tokens > 4064)
    return fail(ATTN_ERR_INVALID_ARG,
                "chunk_tokens=%d must be 0 or a positive multiple of 32 up to 4064",
                chunk_tokens);
  return ATTN_OK;
}

// --------------------------------------------------------------- backward

attn_status_t check_bwd_shape(int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                              attn_dtype_t dtype) {
  attn_status_t st = check_fwd_shape(B, H, Hkv, Nq, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_BF16) return fail(ATTN_ERR_UNSUPPORTED, "backward supports bf16 only");
  return ATTN_OK;
}


// Key split of the bf16 forward ("Work partitioning in FlashAttention-2":
// too few independent workgroups leave CUs idle; "Attention kernels",
// FlashDecoding paragraph: split the key range and merge the partials).
// When B*H*ceil(Nq/128) query tiles give fewer than two workgroups per CU,
// each tile's key range is cut into equal parts: the shortest parts (of at
// least 640 keys) whose units all fit the split kernel's resident
// workgroups at once (three per CU at d = 128, four at d = 64).  chunk_keys
// > 0 forces the part size.
struct SplitPlan {
  int chunk_tiles = 0;
  int n_chunks = 0;      // most parts of any query tile; 0: no split
  long long units = 0;   // (query tile, part) pairs with work
  size_t ws = 0;
};

SplitPlan plan_fwd_split(int B, int H, int Nq, int Nk, int d, int left, int right,
                         int chunk_keys) {
  SplitPlan sp;
  const int bc = eta::fwd_tile_keys(d);
  const int n_qt = (Nq + 127) / 128;
  const bool band = left != eta::kUnbounded || right != eta::kUnbounded;
  int ct;
  if (chunk_keys > 0) {
    ct = (chunk_keys + bc - 1) / bc;
  } else {
    if ((long long)B * H * n_qt >= 2LL * kNumCU) return sp;
    // One round of units: measured at 4 heads x 8k causal (d = 128), parts
    // of 1664 keys (760 units for 768 resident workgroups) run 85 us, while
    // 1536 keys (816 units: 48 wait for a second round) run 101 us and 1056
    // keys (1136 units) 91 us; fewer units than slots leave CUs idle
    // (2048 keys, 640 units: 93 us).  Parts shorter than 640 keys pay more
    // partial traffic and merge work than they gain in balance.
    std::vector<int> len;
    len.reserve(n_qt);
    int longest = 0;
    for (int qt = 0; qt < n_qt; ++qt) {
      int lo, hi;
      eta::band_tiles(band, qt * 128, 128, Nq, Nk, bc, left, right, lo, hi);
      len.push_back(hi >= lo ? hi - lo + 1 : 0);
      longest = len.back() > longest ? len.back() : longest;
    }
    const long long slots = (long long)kNumCU * (d == 128 ? 3 : 4);
    auto units_for = [&](int c) {
      long long u = 0;
      for (int t : len) u += (t + c - 1) / c;
      return u * B * H;
    };
    // units_for falls as the part size grows; at the longest range every
    // tile is one unit, and B*H*n_qt < 2 * kNumCU <= slots.
    int lo = 640 / bc, hi = longest > lo ? longest : lo;
    if (units_for(lo) <= slots) {
      ct = lo;
    } else {
      while (hi - lo > 1) {
        const int mid = lo + (hi - lo) / 2;
        if (units_for(mid) <= slots) hi = mid; else lo = mid;
      }
      ct = hi;
    }
  }
  // Exact number of (query tile, part) units: the grid holds one workgroup
  // per unit and head, with no idle slots (workgroups reach the XCDs round
  // robin, so idle slots in a fixed pattern would unbalance them).
  long long units = 0;
  int max_parts = 0;
  for (int qt = 0; qt < n_qt; ++qt) {
    int lo, hi;
    eta::band_tiles(band, qt * 128, 128, Nq, Nk, bc, left, right, lo, hi);
    const int parts = hi >= lo ? (hi - lo + ct) / ct : 0;
    units += parts;
    if (parts > max_parts) max_parts = parts;
  }
  if (max_parts <= 1 && chunk_keys == 0) return sp;  // every tile in one part
  const int n_chunks = max_parts > 0 ? max_parts : 1;
  sp.units = units;
  sp.chunk_tiles = ct;
  sp.n_chunks = n_chunks;
  // Per partial row: o / l in bf16, then the max and the sum in fp32.
  sp.ws = (size_t)B * H * n_qt * n_chunks * 128 * (size_t)(2 * d + 2 * sizeof(float));
  return sp;
}

attn_status_t fwd_impl(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                       int H, int Hkv, int Nq, int Nk, int d, float scale, int left, int right,
                       attn_dtype_t dtype, void* stream, const SplitPlan& sp = SplitPlan(),
                       void* workspace = nullptr) {
  if (!Q || !K || !V || !O || !LSE) return fail(ATTN_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return fail(ATTN_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  attn_status_t st = check_fwd_shape(B, H, Hkv, Nq, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  const bool band = left != eta::kUnbounded || right != eta::kUnbounded;
  const bool causal = left == eta::kUnbounded && right == 0;
  if (dtype == ATTN_DTYPE_F32 && band && !causal)
    return fail(ATTN_ERR_UNSUPPORTED, "fp32 forward supports only the causal or no mask");
  if (dtype == ATTN_DTYPE_F32 && sp.n_chunks > 0)
    return fail(ATTN_ERR_UNSUPPORTED, "the key split is bf16 only");
  eta::FwdArgs a{Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, causal ? 1 : 0, band ? 1 : 0,
                 left, right, dtype == ATTN_DTYPE_BF16, sp.chunk_tiles, sp.n_chunks,
                 (int)sp.units, workspace};
  eta::FwdPlan p = plan_fwd(B, H, Nq, d, a.dtype_bf16);
  const long long grid = sp.n_chunks > 0 ? (long long)B * H * sp.units : p.workgroups;
  if (grid > kMaxGrid) return fail(ATTN_ERR_INVALID_ARG, "grid too large");
  hipError_t e = eta::launch_fwd(a, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

attn_status_t bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                       const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int Hkv,
                       int Nq, int Nk, int d, float scale, int left, int right,
                       attn_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV)
    return fail(ATTN_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
    return fail(ATTN_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  attn_status_t st = check_bwd_shape(B, H, Hkv, Nq, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  const size_t need = eta::bwd_workspace_bytes(B, H, Nq, d);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "backward workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const bool band = left != eta::kUnbounded || right != eta::kUnbounded;
  eta::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Hkv, Nq, Nk, d, scale, band ? 1 : 0,
                 left, right, workspace};
  hipError_t e = eta::launch_bwd(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Checks shared by the packed (ragged and paged) forward entry points.
attn_status_t check_packed(const void* Q, const void* O, const float* LSE, const int32_t* cu_q,
                           int num_seqs, int total_q, int max_seqlen_q, int H, int Hkv, int d,
                           float scale, attn_dtype_t dtype) {
  if (!Q || !O || !LSE || !cu_q) return fail(ATTN_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(Q) || !aligned16(O) || ((uintptr_t)LSE & 3u) || ((uintptr_t)cu_q & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "misaligned pointer argument");
  if (num_seqs < 1 || total_q < 1 || max_seqlen_q < 1 || max_seqlen_q > total_q || H < 1 ||
      Hkv < 1)
    return fail(ATTN_ERR_INVALID_ARG,
                "bad sizes (num_seqs=%d total_q=%d max_seqlen_q=%d H=%d Hkv=%d)", num_seqs,
                total_q, max_seqlen_q, H, Hkv);
  if (H % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "H=%d is not a multiple of Hkv=%d", H, Hkv);
  if (dtype != ATTN_DTYPE_BF16) {
    if (dtype != ATTN_DTYPE_F32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    return fail(ATTN_ERR_UNSUPPORTED, "packed and paged forward support bf16 only");
  }
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(ATTN_ERR_INVALID_ARG, "scale must be positive and finite");
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension %d not in {64,128}", d);
  // Packed rows are addressed with 32-bit byte offsets from a sequence's first row.
  if ((long long)total_q * H * d * 2 >= (1LL << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "packed queries exceed 2 GiB");
  if ((long long)((max_seqlen_q + 127) / 128) * num_seqs * H > kMaxGrid)
    return fail(ATTN_ERR_INVALID_ARG, "grid too large");
  return ATTN_OK;
}

attn_status_t launch_mode(eta::FwdArgs& a, void* stream) {
  eta::FwdPlan p{};
  hipError_t e = eta::launch_fwd(a, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int num_seqs, int total_q, int total_k, int max_seqlen_q, int H,
                              int Hkv, int d, float scale, int window_left, int window_right,
                              attn_dtype_t dtype, void* stream) {
  int left, right;
  if (!window_sides(window_left, window_right, &left, &right))
    return fail(ATTN_ERR_INVALID_ARG, "window sides must be >= -1 (got %d, %d)", window_left,
                window_right);
  attn_status_t st = check_packed(Q, O, LSE, cu_seqlens_q, num_seqs, total_q, max_seqlen_q, H,
                                  Hkv, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (!K || !V || !cu_seqlens_k) return fail(ATTN_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(K) || !aligned16(V) || ((uintptr_t)cu_seqlens_k & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "misaligned pointer argument");
  if (total_k < 0) return fail(ATTN_ERR_INVALID_ARG, "total_k=%d must be >= 0", total_k);
  if ((long long)total_k * Hkv * d * 2 >= (1LL << 31))
    return fail(ATTN_ERR_UNSUPPORTED, "packed keys exceed 2 GiB");
  const bool band = left != eta::kUnbounded || right != eta::kUnbounded;
  eta::FwdArgs a{Q, K, V, O, LSE, num_seqs, H, Hkv, max_seqlen_q, 0, d, scale, 0, band ? 1 : 0,
                 left, right, true, 0, 0, 0, nullptr, eta::kFwdRagged, eta::FwdSeqArgs{}};
  a.seq.cu_q = cu_seqlens_q;
  a.seq.k_lens = cu_seqlens_k;
  a.seq.total_q = total_q;
  a.seq.total_k = total_k;
  return launch_mode(a, stream);
}

attn_status_t attn_prefill_paged(const void* Q, const void* K_cache, const void* V_cache,
                                 const int32_t* block_table, const int32_t* cu_seqlens_q,
                                 const int32_t* seqlens_k, void* O, float* LSE, int num_seqs,
                                 int total_q, int max_seqlen_q, int Hq, int Hkv, int d,
                                 int block_size, int num_blocks, int max_blocks_per_seq,
                                 int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                 float scale, int window_left, int window_right,
                                 attn_dtype_t dtype, void* stream) {
  int left, right;
  if (!window_sides(window_left, window_right, &left, &right))
    return fail(ATTN_ERR_INVALID_ARG, "window sides must be >= -1 (got %d, %d)", window_left,
                window_right);
  attn_status_t st = check_packed(Q, O, LSE, cu_seqlens_q, num_seqs, total_q, max_seqlen_q, Hq,
                                  Hkv, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (!K_cache || !V_cache || !block_table || !seqlens_k)
    return fail(ATTN_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(K_cache) || !aligned16(V_cache) || ((uintptr_t)block_table & 3u) ||
      ((uintptr_t)seqlens_k & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "misaligned pointer argument");
  if (block_size < 1 || num_blocks < 1 || max_blocks_per_seq < 1)
    return fail(ATTN_ERR_INVALID_ARG, "bad cache sizes (block_size=%d num_blocks=%d "
                "max_blocks_per_seq=%d)", block_size, num_blocks, max_blocks_per_seq);
  // Each wave's 8 (d = 128) or 16 (d = 64) rows of a key tile must share a page.
  if (block_size % 16 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "paged prefill needs block_size %% 16 == 0 (got %d)",
                block_size);
  if ((long long)max_blocks_per_seq * block_size >= (1LL << 31))
    return fail(ATTN_ERR_INVALID_ARG, "block table capacity exceeds 2^31 tokens");
  if (!page_layout_ok(d, Hkv, block_size, block_stride, token_stride, head_stride))
    return fail(ATTN_ERR_INVALID_ARG,
                "cache strides inconsistent with block_size=%d Hkv=%d d=%d "
                "(block=%lld token=%lld head=%lld)",
                block_size, Hkv, d, (long long)block_stride, (long long)token_stride,
                (long long)head_stride);
  if (token_stride >= (1LL << 24))
    return fail(ATTN_ERR_UNSUPPORTED, "token_stride=%lld elements exceeds 2^24",
                (long long)token_stride);
  const bool band = left != eta::kUnbounded || right != eta::kUnbounded;
  eta::FwdArgs a{Q, K_cache, V_cache, O, LSE, num_seqs, Hq, Hkv, max_seqlen_q, 0, d, scale, 0,
                 band ? 1 : 0, left, right, true, 0, 0, 0, nullptr, eta::kFwdPaged,
                 eta::FwdSeqArgs{}};
  a.seq.cu_q = cu_seqlens_q;
  a.seq.k_lens = seqlens_k;
  a.seq.block_table = block_table;
  a.seq.total_q = total_q;
  a.seq.max_blocks = max_blocks_per_seq;
  a.seq.num_blocks = num_blocks;
  a.seq.block_size = block_size;
  eta::page_magic(block_size, a.seq.page_magic, a.seq.page_shift);
  a.seq.block_stride = block_stride;
  a.seq.token_stride = token_stride;
  a.seq.head_stride = head_stride;
  return launch_mode(a, stream);
}

attn_status_t attn_fwd_block_sparse(const void* Q, const void* K, const void* V, void* O,
                                    float* LSE, int B, int H, int Hkv, int Nq, int Nk, int d,
                                    float scale, int causal, const int32_t* row_ptr,
                                    const int32_t* col_idx, int num_layouts, int nnz,
                                    attn_dtype_t dtype, void* stream) {
  if (!Q || !K || !V || !O || !LSE || !row_ptr || !col_idx)
    return fail(ATTN_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE) ||
      ((uintptr_t)row_ptr & 3u) || ((uintptr_t)col_idx & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "misaligned pointer argument");
  attn_status_t st = check_fwd_shape(B, H, Hkv, Nq, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_BF16)
    return fail(ATTN_ERR_UNSUPPORTED, "block-sparse forward supports bf16 only");
  if (num_layouts < 1) return fail(ATTN_ERR_INVALID_ARG, "num_layouts=%d must be >= 1", num_layouts);
  if (nnz < 0) return fail(ATTN_ERR_INVALID_ARG, "nnz=%d must be >= 0", nnz);
  if ((long long)B * H * ((Nq + 127) / 128) > kMaxGrid)
    return fail(ATTN_ERR_INVALID_ARG, "grid too large");
  eta::FwdArgs a{Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, causal ? 1 : 0, causal ? 1 : 0,
                 eta::kUnbounded, causal ? 0 : eta::kUnbounded, true, 0, 0, 0, nullptr,
                 eta::kFwdSparse, eta::FwdSeqArgs{}};
  a.seq.row_ptr = row_ptr;
  a.seq.col_idx = col_idx;
  a.seq.num_layouts = num_layouts;
  a.seq.nnz = nnz;
  return launch_mode(a, stream);
}


attn_status_t attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                       int H, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                       attn_dtype_t dtype, void* stream) {
  return fwd_impl(Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, eta::kUnbounded,
                  causal ? 0 : eta::kUnbounded, dtype, stream);
}

attn_status_t attn_fwd_local(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                             int window_left, int window_right, attn_dtype_t dtype,
                             void* stream) {
  int left, right;
  if (!window_sides(window_left, window_right, &left, &right))
    return fail(ATTN_ERR_INVALID_ARG, "window sides must be >= -1 (got %d, %d)", window_left,
                window_right);
  return fwd_impl(Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, left, right, dtype, stream);
}

size_t attn_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d, int window_left,
                                       int window_right, int chunk_keys) {
  int left, right;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (d != 64 && d != 128) || chunk_keys < 0 ||
      chunk_keys % 64 != 0 || !window_sides(window_left, window_right, &left, &right))
    return 0;
  return plan_fwd_split(B, H, Nq, Nk, d, left, right, chunk_keys).ws;
}

attn_status_t attn_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                               int window_left, int window_right, attn_dtype_t dtype,
                               int chunk_keys, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int left, right;
  if (!window_sides(window_left, window_right, &left, &right))
    return fail(ATTN_ERR_INVALID_ARG, "window sides must be >= -1 (got %d, %d)", window_left,
                window_right);
  if (chunk_keys < 0 || chunk_keys % 64 != 0)
    return fail(ATTN_ERR_INVALID_ARG, "chunk_keys=%d must be 0 or a positive multiple of 64",
                chunk_keys);
  attn_status_t st = check_fwd_shape(B, H, Hkv, Nq, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  const SplitPlan sp = plan_fwd_split(B, H, Nq, Nk, d, left, right, chunk_keys);
  if (sp.n_chunks > 0) {
    if (!workspace || workspace_bytes < sp.ws)
      return fail(ATTN_ERR_WORKSPACE, "split forward workspace needs %zu bytes, got %zu", sp.ws,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace))
      return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  return fwd_impl(Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, left, right, dtype, stream, sp,
                  workspace);
}

// Workspace of a decode with Hkv = Hq / G KV heads.
size_t decode_ws_for(int num_seqs, int Hq, int G, int d, int max_context, int chunk_tokens) {
  const long long pairs = eta::decode_pairs(num_seqs, Hq / G, G);
  const long long waves = eta::decode_split_waves(pairs, d, max_context, chunk_tokens / 32);
  return eta::decode_workspace_bytes(pairs, G, d, waves);
}

size_t attn_decode_paged_workspace_size(int num_seqs, int Hq, int d, int max_context,
                                        int chunk_tokens) {
  if (num_seqs < 1 || Hq < 1 || (d != 64 && d != 128) || max_context < 0 || chunk_tokens < 0 ||
      chunk_tokens % 32 != 0 || chunk_tokens > 4064)
    return 0;
  // The size depends on the group size G = Hq / Hkv, which the caller has
  // not given: cover every G the decode accepts.
  size_t most = 0;
  for (int G = 1; G <= Hq; ++G)
    if (Hq % G == 0) {
      const size_t b = decode_ws_for(num_seqs, Hq, G, d, max_context, chunk_tokens);
      if (b > most) most = b;
    }
  return most;
}

namespace {

// Validation and launch shared by the two decode entry points.  `workspace`
// is the caller's buffer, or (no_alloc) the library's static scratch, whose
// capacity is workspace_bytes.
attn_status_t decode_impl(const void* Q, const void* K_cache, const void* V_cache,
                          const int32_t* block_table, const int32_t* context_lens, void* O,
                          float* LSE, int num_seqs, int Hq, int Hkv, int d, int block_size,
                          int num_blocks, int max_blocks_per_seq, int max_context,
                          int64_t block_stride, int64_t token_stride, int64_t head_stride,
                          float scale, attn_dtype_t dtype, int chunk_tokens, void* workspace,
                          size_t workspace_bytes, void* stream, bool no_alloc) {
  if (!Q || !K_cache || !V_cache || !block_table || !context_lens || !O)
    return fail(ATTN_ERR_INVALID_ARG, "null pointer argument");
  if (!aligned16(Q) || !aligned16(K_cache) || !aligned16(V_cache) || !aligned16(O) ||
      ((uintptr_t)block_table & 3u) || ((uintptr_t)context_lens & 3u) ||
      (LSE && ((uintptr_t)LSE & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "misaligned pointer argument");
  attn_status_t st = check_decode_shape(num_seqs, Hq, Hkv, d, block_size, num_blocks,
                                        max_blocks_per_seq, max_context, chunk_tokens);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_BF16) {
    if (dtype != ATTN_DTYPE_F32) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    return fail(ATTN_ERR_UNSUPPORTED, "paged decode supports bf16 only");
  }
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(ATTN_ERR_INVALID_ARG, "scale must be positive and finite");
  // Layout identity ("Failure modes": page-table mismatch): the strides must
  // describe disjoint, 16-byte aligned rows.
  if (!page_layout_ok(d, Hkv, block_size, block_stride, token_stride, head_stride))
    return fail(ATTN_ERR_INVALID_ARG,
                "cache strides inconsistent with block_size=%d Hkv=%d d=%d "
                "(block=%lld token=%lld head=%lld)",
                block_size, Hkv, d, (long long)block_stride, (long long)token_stride,
                (long long)head_stride);
  // The kernels address one page with 32-bit byte offsets.
  if (block_stride >= (1LL << 30))
    return fail(ATTN_ERR_UNSUPPORTED, "block_stride=%lld elements exceeds 2^30",
                (long long)block_stride);
  const long long pairs = eta::decode_pairs(num_seqs, Hkv, Hq / Hkv);
  const long long n_waves = eta::decode_split_waves(pairs, d, max_context, chunk_tokens / 32);
  // Segment ids (split wave + pair index) and the split grid stay in int.
  if (n_waves + pairs > kMaxGrid)
    return fail(ATTN_ERR_UNSUPPORTED, "decode needs %lld split waves for %lld pairs",
                n_waves, pairs);
  const size_t need = eta::decode_workspace_bytes(pairs, Hq / Hkv, d, n_waves);
  if (no_alloc) {
    if (need > workspace_bytes)
      return fail(ATTN_ERR_WORKSPACE,
                  "decode needs %zu bytes of scratch, the no-allocation entry point holds %zu",
                  need, workspace_bytes);
    // The scratch pointer belongs to the current device: the stream must too.
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess)
      return fail(ATTN_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
    if (sdev != cur)
      return fail(ATTN_ERR_INVALID_ARG, "stream belongs to device %d, device %d is current",
                  sdev, cur);
    st = decode_scratch(cur, &workspace);
    if (st != ATTN_OK) return st;
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(ATTN_ERR_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace))
      return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  eta::DecodeArgs a{Q,        K_cache,     V_cache,      block_table,  context_lens,
                    O,        LSE,         num_seqs,     Hq,           Hkv,
                    d,        block_size,  num_blocks,   max_blocks_per_seq,
                    max_context, block_stride, token_stride, head_stride, scale,
                    workspace};
  eta::DecodePlan p{chunk_tokens / 32, eta::decode_target_waves(d), n_waves};
  hipError_t e = eta::launch_decode(a, p, (hipStream_t)stream);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

attn_status_t attn_decode_paged(const void* Q, const void* K_cache, const void* V_cache,
                                const int32_t* block_table, const int32_t* context_lens, void* O,
                                float* LSE, int num_seqs, int Hq, int Hkv, int d, int block_size,
                                int num_blocks, int max_blocks_per_seq, int max_context,
                                int64_t block_stride, int64_t token_stride, int64_t head_stride,
                                float scale, attn_dtype_t dtype, int chunk_tokens,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(Q, K_cache, V_cache, block_table, context_lens, O, LSE, num_seqs, Hq, Hkv,
                     d, block_size, num_blocks, max_blocks_per_seq, max_context, block_stride,
                     token_stride, head_stride, scale, dtype, chunk_tokens, workspace,
                     workspace_bytes, stream, false);
}

size_t attn_decode_paged_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

attn_status_t attn_decode_paged_noalloc(const void* Q, const void* K_cache, const void* V_cache,
                                        const int32_t* block_table, const int32_t* context_lens,
                                        void* O, float* LSE, int num_seqs, int Hq, int Hkv, int d,
                                        int block_size, int num_blocks, int max_blocks_per_seq,
                                        int max_context, int64_t block_stride,
                                        int64_t token_stride, int64_t head_stride, float scale,
                                        attn_dtype_t dtype, int chunk_tokens, void* stream) {
  return decode_impl(Q, K_cache, V_cache, block_table, context_lens, O, LSE, num_seqs, Hq, Hkv,
                     d, block_size, num_blocks, max_blocks_per_seq, max_context, block_stride,
                     token_stride, head_stride, scale, dtype, chunk_tokens, nullptr,
                     kNoAllocScratchBytes, stream, true);
}

size_t attn_bwd_workspace_size(int B, int H, int Nq, int d) {
  if (B < 1 || H < 1 || Nq < 1 || (d != 64 && d != 128)) return 0;
  return eta::bwd_workspace_bytes(B, H, Nq, d);
}

attn_status_t attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                       const float* LSE, void* dQ, void* dK, void* dV, int B, int H, int Hkv,
                       int Nq, int Nk, int d, float scale, int causal, attn_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Hkv, Nq, Nk, d, scale, eta::kUnbounded,
                  causal ? 0 : eta::kUnbounded, dtype, workspace, workspace_bytes, stream);
}

attn_status_t attn_bwd_local(const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B,
                             int H, int Hkv, int Nq, int Nk, int d, float scale, int window_left,
                             int window_right, attn_dtype_t dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  int left, right;
  if (!window_sides(window_left, window_right, &left, &right))
    return fail(ATTN_ERR_INVALID_ARG, "window sides must be >= -1 (got %d, %d)", window_left,
                window_right);
  return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, Hkv, Nq, Nk, d, scale, left, right,
                  dtype, workspace, workspace_bytes, stream);
}

int attn_plan_describe(int phase, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                       attn_dtype_t dtype, char* buf, size_t len) {
  char tmp[512];
  int n = -1;
  if (phase == ATTN_PHASE_FWD) {
    if (check_fwd_shape(B, H, Hkv, Nq, Nk, d, 1.f, dtype) != ATTN_OK) return -1;
    const bool bf16 = dtype == ATTN_DTYPE_BF16;
    eta::FwdPlan p = plan_fwd(B, H, Nq, d, bf16);
    if (p.key_parts > 1)
      n = snprintf(tmp, sizeof(tmp),
                   "phase=fwd kernel=fwd_f32_keysplit_mfma32x32x2 d=%d causal=%d Br=%d "
                   "(%d waves split the keys of %d rows, merged in LDS) Bc=%d grid=%lld "
                   "workgroups (B*H*ceil(Nq/Br)) order=heavy-query-tiles-first",
                   d, causal ? 1 : 0, p.block_rows, p.key_parts, p.rows_per_wave, p.block_keys,
                   p.workgroups);
    else
      n = snprintf(tmp, sizeof(tmp),
                   "phase=fwd kernel=%s d=%d causal=%d Br=%d (%d waves x %d rows) Bc=%d "
                   "grid=%lld workgroups (B*H*ceil(Nq/Br)) order=heavy-query-tiles-first "
                   "head-interleaved",
                   bf16 ? "fwd_bf16_mfma32x32x16" : "fwd_f32_mfma32x32x2",
                   d, causal ? 1 : 0, p.block_rows, p.waves, p.rows_per_wave, p.block_keys,
                   p.workgroups);
    // The key split attn_fwd_splitkv would take for the same shape.
    const SplitPlan sp =
        bf16 ? plan_fwd_split(B, H, Nq, Nk, d, eta::kUnbounded, causal ? 0 : eta::kUnbounded, 0)
             : SplitPlan();
    if (sp.n_chunks > 0 && n > 0 && n < (int)sizeof(tmp))
      n += snprintf(tmp + n, sizeof(tmp) - n,
                    "; splitkv: Br=128 parts of <= %d keys, %lld units per head in one round "
                    "(grid=%lld), <= %d parts per query tile, then fwd_merge",
                    sp.chunk_tiles * eta::fwd_tile_keys(d), sp.units, sp.units * B * H,
                    sp.n_chunks);
  } else if (phase == ATTN_PHASE_DECODE) {
    if (check_decode_shape(B, H, Hkv, d, 16, 1, (Nk + 15) / 16 > 0 ? (Nk + 15) / 16 : 1, Nk, 0) !=
        ATTN_OK)
      return -1;
    const long long waves =
        eta::decode_split_waves(eta::decode_pairs(B, Hkv, H / Hkv), d, Nk, 0);
    n = snprintf(tmp, sizeof(tmp),
                 "phase=decode kernel=decode_split_mfma16x16x32+decode_merge d=%d G=%d "
                 "split=balanced (equal 32-token step ranges of all seq x KV-head pairs, "
                 ">= %d steps per wave, %d waves) split_waves<=%lld merge_workgroups=%lld",
                 d, H / Hkv, eta::kDecodeMinSteps, eta::decode_target_waves(d), waves,
                 (long long)B * H);
  } else if (phase == ATTN_PHASE_BWD) {
    if (check_bwd_shape(B, H, Hkv, Nq, Nk, d, 1.f, dtype) != ATTN_OK) return -1;
    n = snprintf(tmp, sizeof(tmp),
                 "phase=bwd kernels=bwd_dq_mfma32x32x16(+D,LSE2)+bwd_dkdv_mfma32x32x16 d=%d "
                 "causal=%d dkdv: key_tile=128 (4 waves x 32 keys, K in LDS) query_tile=32 grid=%lld "
                 "(B*Hkv*ceil(Nk/128)); dq: query_tile=128 key_tile=32 grid=%lld "
                 "(B*H*ceil(Nq/128)); deterministic (no atomics)",
                 d, causal ? 1 : 0, (long long)B * Hkv * ((Nk + 127) / 128),
                 (long long)B * H * ((Nq + 127) / 128));
  } else {
    return -1;
  }
  if (buf && len > 0) {
    strncpy(buf, tmp, len - 1);
    buf[len - 1] = '\0';
  }
  return n;
}

const char* attn_status_string(attn_status_t status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "ATTN_ERR_UNKNOWN";
}

const char* attn_last_error(void) { return g_last_error; }

}  // extern "C"
