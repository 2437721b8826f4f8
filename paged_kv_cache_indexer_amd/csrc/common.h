// Shared device helpers for libdsa (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "dsa.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- host-side status
void set_last_error(const char* fmt, ...);
dsa_status_t launch_status(const char* what);

#define DSA_CHECK_ARG(cond, ...)                \
  do {                                          \
    if (!(cond)) {                              \
      ::dsa::set_last_error(__VA_ARGS__);       \
      return DSA_ERR_INVALID_ARG;               \
    }                                           \
  } while (0)

// Kernel launch that first clears any error an earlier, unrelated HIP call left behind,
// so that launch_status() afterwards reports this launch only.
#define DSA_LAUNCH(...)                         \
  do {                                          \
    (void)hipGetLastError();                    \
    hipLaunchKernelGGL(__VA_ARGS__);            \
  } while (0)

// Host-side launch parameters (CU counts, occupancy grids, kernel attributes set) are cached
// per device: slot = the current device's id, or -1 past kMaxDevices (then nothing is
// cached).  Concurrent first calls may both compute the value; they store the same one.
constexpr int kMaxDevices = 64;
inline int current_device_slot() {
  int d = -1;
  return (hipGetDevice(&d) == hipSuccess && d >= 0 && d < kMaxDevices) ? d : -1;
}

#define DSA_CHECK_SUPPORTED(cond, ...)          \
  do {                                          \
    if (!(cond)) {                              \
      ::dsa::set_last_error(__VA_ARGS__);       \
      return DSA_ERR_UNSUPPORTED;               \
    }                                           \
  } while (0)

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ void count_error(int32_t* err, int32_t n = 1) {
  if (err) atomicAdd(err, n);
}

// Row address in a dsa_rows_t (paged or dense).  Returns nullptr if the page id or
// row is out of range.
struct RowStore {
  const char* base;
  int64_t num_rows;
  int32_t row_bytes;
  int32_t page_size;
  const int32_t* page_table;
  int32_t pt_stride;
  int64_t req_stride;

  __host__ static RowStore from(const dsa_rows_t& r) {
    RowStore s;
    s.base = static_cast<const char*>(r.base);
    s.num_rows = r.num_rows;
    s.row_bytes = r.row_bytes;
    s.page_size = r.page_size;
    s.page_table = r.page_table;
    s.pt_stride = r.pt_stride;
    s.req_stride = r.req_stride;
    return s;
  }

  // physical row index of token `pos` of request `b`, or -1 if out of range (position past
  // the request's page-table row / dense stride, negative page id, row past num_rows)
  __device__ __forceinline__ int64_t row(int b, int64_t pos) const {
    if (pos < 0) return -1;
    int64_t r;
    if (page_table) {
      const int64_t lp = pos / page_size;
      if (lp >= pt_stride) return -1;
      const int32_t pg = page_table[(int64_t)b * pt_stride + lp];
      if (pg < 0) return -1;
      r = (int64_t)pg * page_size + (pos - lp * page_size);
    } else {
      if (req_stride > 0 && pos >= req_stride) return -1;
      r = (int64_t)b * req_stride + pos;
    }
    return (r < num_rows) ? r : -1;
  }
};

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Four e4m3 codes (one dword) -> two dwords of packed bf16 (exact: every e4m3 value is a bf16).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t v) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// 8 e4m3 codes (two dwords) -> bf16x8
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t a, uint32_t b) {
  u32x2 x = e4m3x4_to_bf16x4(a);
  u32x2 y = e4m3x4_to_bf16x4(b);
  u32x4 r = {x.x, x.y, y.x, y.y};
  return __builtin_bit_cast(bf16x8, r);
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0.0 maps as +0.0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Load of a wave-uniform address through the constant address space, which lets the
// backend emit a scalar (SMEM) load: it is counted by lgkmcnt and does not wait behind
// outstanding vector loads.  Only for data that no kernel writes while it runs.
template <typename T>
__device__ __forceinline__ T scalar_load(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace dsa
