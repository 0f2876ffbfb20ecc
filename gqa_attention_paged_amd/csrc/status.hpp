// Error recording shared by the host-side entry points.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "gqap.h"

namespace gqap {

// Message of the last failing call on this host thread.
std::string& last_error_slot();

inline gqap_status fail(gqap_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error_slot() = buf;
  return st;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kBlock = GQAP_BLOCK_SIZE;
// Work-items one launch may hold (grid x workgroup size stays below 2^32).
constexpr int64_t kMaxLaunchItems = ((int64_t)1 << 32) - 256;
constexpr int kDefaultCUs = 256;

// Kernel variants recorded in a decode plan.
enum DecodeKernel : uint32_t {
  kDecodeF32Valu = 1,   // fp32 q / fp32 KV, vector ALU
  kDecodeBf16Mfma = 2,  // bf16 q / bf16 KV, bf16 matrix cores
  kDecodeFp8Mfma = 3,   // bf16 q / fp8 e4m3fn KV, dequantised to bf16 for the matrix cores
};

// Kernel variants recorded in a chunked-prefill plan.
enum ChunkKernel : int32_t {
  kChunkPrefill = 1,         // prefill kernel over the paged cache
  kChunkPrefillMla = 2,      // the same with the shared rope cache
  kChunkPrefillFp8 = 3,      // prefill kernel over an fp8 cache
  kChunkPrefillMlaFp8 = 4,   // fp8 cache with the bf16 rope cache
  kChunkDecode = 5,          // short chunks on the decode workers
  kChunkDecodeFp8 = 6,       // the same over an fp8 cache
};

// Short chunks on the decode workers (decode.hip).  The caller has checked
// the plan, the scales, the pointers and their alignment.
gqap_status chunk_decode_launch(const gqap_chunk_plan_t* plan, const void* q, const void* k_pool,
                                const void* v_pool, const void* kr_pool, const int32_t* block_table,
                                const int32_t* cu_seqlens_q,
                                const int32_t* kv_lens, float scale, bool fp8, float k_scale, float v_scale,
                                void* out, float* lse, void* workspace, uint64_t workspace_bytes, void* stream);

// Byte offsets of the decode workspace regions (shared by planner and launcher).
//   prefix [B + 1] int32              key blocks before each sequence
//   lse    [pieces][cols] float32     base-2 log-sum-exp of each partial
//   o      [pieces][cols][D] float32  normalised partial outputs
// cols = the MFMA columns a piece can hold results for: the query heads of a
// KV head (times the chunk rows in chunk mode), 16 when that needs more than
// one 16-column tile.
struct DecodeWorkspace {
  uint64_t prefix, lse, o, total;
};

inline uint64_t round256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

// Columns per piece slot: `pairs` (token, head) pairs per KV head, in tiles of 16.
inline int64_t piece_cols(int64_t pairs) { return pairs > 16 ? 16 : pairs; }

inline DecodeWorkspace decode_workspace(int64_t B, int64_t pieces, int64_t cols, int64_t D) {
  DecodeWorkspace w;
  w.prefix = 0;
  w.lse = round256((uint64_t)(B + 1) * 4);
  w.o = w.lse + round256((uint64_t)pieces * cols * 4);
  w.total = w.o + round256((uint64_t)pieces * cols * D * 4);
  return w;
}

// Resident worker waves per compute unit for each decode variant.  With the
// streamed K/V reads, three bf16 D = 128 waves per compute unit already keep
// HBM busy, and the fewer pieces shorten the combine; fp8 units carry half
// the bytes, so its workers keep four.  A count that is not a multiple of the
// compute units leaves some with a wave more than others and runs slower.
inline int decode_waves_per_cu(uint32_t kernel, int head_dim) {
  switch (kernel) {
    case kDecodeF32Valu: return 2;
    case kDecodeBf16Mfma: return head_dim == 128 ? 3 : 8;
    default: return head_dim == 128 ? 4 : 8;  // fp8 KV
  }
}

}  // namespace gqap
