// Device-side helpers for gfx950 (CDNA4): vector types, conversions, LDS
// transpose reads and the paged-cache address function.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqap {
namespace dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

#define GQAP_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float f32_from_bits(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t bits_of(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = bits_of(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Upper halves of two floats that are exactly representable in bf16.
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(bits_of(hi), bits_of(lo), 0x07060302u);
}

// Eight OCP e4m3fn bytes (little-endian in w) -> eight bf16 values.  The
// hardware conversion is exact and every e4m3fn value is a bf16 value, so
// truncating the float to its upper half is exact too.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(i32x2 w) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[0], false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w[0], true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w[1], false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w[1], true);
  i32x4 r;
  r[0] = (int)pack_exact_bf16x2(a[0], a[1]);
  r[1] = (int)pack_exact_bf16x2(b[0], b[1]);
  r[2] = (int)pack_exact_bf16x2(c[0], c[1]);
  r[3] = (int)pack_exact_bf16x2(d[0], d[1]);
  return __builtin_bit_cast(bf16x8, r);
}

// Two floats -> packed bf16 pair with the hardware round-to-nearest-even convert.
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 2^x with the hardware transcendental (exp2(-inf) = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane groups),
// with the gfx950 lane-swap instructions instead of LDS-routed shuffles.
__device__ __forceinline__ float wave_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  x = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}
__device__ __forceinline__ float wave_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  x = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

__device__ __forceinline__ i32x4 load16(const void* p) { return *(const i32x4*)p; }
// A streamed read (the load's nontemporal hint): for data read once, such as
// a decode pass over the KV cache.  Hinted reads of a large buffer stream at
// about 6.7 TB/s on this part against about 6.0 for ordinary ones.
__device__ __forceinline__ i32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load((const i32x4*)p);
}
__device__ __forceinline__ void store16(void* p, i32x4 v) { *(i32x4*)p = v; }

// LDS transpose reads (gfx950).  Within each group of 16 lanes:
//   tr16: lane i receives element (i % 4) of the 4 x 16-bit row addressed by
//         lanes 4k + i/4, for k = 0..3;
//   tr8:  lane i receives byte (i % 8) of the 8-byte row addressed by lanes
//         2k + i/8, for k = 0..7.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 GQAP_LDS*)(p));
}
__device__ __forceinline__ i32x2 lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 GQAP_LDS*)(p));
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wait for this wave's outstanding LDS operations; also a compiler barrier.
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Paged-cache addressing (FlashMLA tensor-shape reference: block_table[b, j]
// names the pool block holding logical tokens 64j .. 64j+63; each (block,
// head) is a contiguous 64-row slab).  Byte address of the slab of logical
// block j, KV head g.  Every kernel that touches the pool goes through this.
__device__ __forceinline__ const unsigned char* kv_slab(const unsigned char* pool, const int32_t* bt_row, int j,
                                                        int g, int64_t block_bytes, int64_t head_bytes) {
  return pool + (int64_t)bt_row[j] * block_bytes + (int64_t)g * head_bytes;
}

}  // namespace dev
}  // namespace gqap
