// Peak probes for the roofline: what HBM streaming and the matrix cores reach on the running
// device, measured beside the published figures (8 TB/s; 2.5 PF/s bf16, 5.0 PF/s fp8 dense).
// Not part of libdsa's interface; the benchmark loads this library on its own.
//
//   dsa_peak_stream_read  non-temporal 16-byte loads over a buffer, grid-stride; one 4-byte
//                         XOR per wave is written so the loads cannot be dropped
//   dsa_peak_stream_copy  non-temporal 16-byte loads and stores, grid-stride
//   dsa_peak_mfma         back-to-back 32x32 MFMAs on eight independent accumulators per wave
//                         (bf16 32x32x16, or fp8 e4m3 32x32x64 through the scaled form with
//                         unit scales), operands all ones: every accumulator element ends at
//                         K * iters exactly, which the caller checks.  One value per wave.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* src, int64_t n, uint32_t* out) {
  uint32_t x = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

__global__ void __launch_bounds__(256) stream_copy_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

constexpr int kAcc = 8;   // independent accumulators per wave

template <bool FP8>
__global__ void __launch_bounds__(256) mfma_loop_kernel(int iters, float* out) {
  f32x16 acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = f32x16{};
  if constexpr (FP8) {
    // e4m3 1.0 = 0x38 in every byte
    const int one4 = 0x38383838;
    const i32x8 a = {one4, one4, one4, one4, one4, one4, one4, one4};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kAcc; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, acc[j], 0, 0, 0, 127, 0, 127);
    }
  } else {
    const bf16x8 a = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[j], 0, 0, 0);
    }
  }
  // every element equals K * iters; the wave reports the smallest and the largest element
  float lo = acc[0][0], hi = acc[0][0];
#pragma unroll
  for (int j = 0; j < kAcc; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      lo = fminf(lo, acc[j][e]);
      hi = fmaxf(hi, acc[j][e]);
    }
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
  }
  if ((threadIdx.x & 63) == 0) {
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    out[2 * w] = lo;
    out[2 * w + 1] = hi;
  }
}

}  // namespace

// Returns 0, or a HIP error code.  n16: number of 16-byte elements; out: blocks * 4 uint32.
extern "C" int dsa_peak_stream_read(const void* src, int64_t n16, int blocks, uint32_t* out, hipStream_t stream) {
  if (!src || !out || n16 < 1 || blocks < 1) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src), n16,
                     out);
  return (int)hipGetLastError();
}

extern "C" int dsa_peak_stream_copy(const void* src, void* dst, int64_t n16, int blocks, hipStream_t stream) {
  if (!src || !dst || n16 < 1 || blocks < 1) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), n16);
  return (int)hipGetLastError();
}

// fp8 = 0: bf16 32x32x16 (K = 16); fp8 = 1: e4m3 32x32x64 (K = 64).  out: blocks * 4 * 2 floats
// (smallest and largest accumulator element of each wave).  Flops per launch:
// blocks * 4 waves * iters * 8 MFMAs * 2 * 32 * 32 * K.
extern "C" int dsa_peak_mfma(int fp8, int iters, int blocks, float* out, hipStream_t stream) {
  if (!out || iters < 1 || blocks < 1) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();
  if (fp8)
    hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(blocks), dim3(256), 0, stream, iters, out);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(blocks), dim3(256), 0, stream, iters, out);
  return (int)hipGetLastError();
}
