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
constexpr int kDefaultCUs = 256;

// Kernel variants recorded in a decode plan.
enum DecodeKernel : uint32_t {
  kDecodeF32Valu = 1,   // fp32 q / fp32 KV, vector ALU
  kDecodeBf16Mfma = 2,  // bf16 q / bf16 KV, bf16 matrix cores
  kDecodeFp8Mfma = 3,   // bf16 q / fp8 e4m3fn KV, dequantised to bf16 for the matrix cores
};

// Workgroup shape of each decode variant (used by the planner and the launcher).
constexpr int kMfmaWaves = 4;

}  // namespace gqap
