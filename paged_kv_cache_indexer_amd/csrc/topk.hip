// Top-k selection of indexer scores ("Shared-Indexer KV Cache Offload for GLM-5.2",
// §2.1: the 2048 best positions per query feed sparse attention).
//
// Order: score descending, then position ascending; -0.0 == +0.0.  Scores map to
// order-preserving uint32 keys; an MSB-first radix select (digits of up to 11 bits,
// starting below the bits every key of the row shares) finds the k-th largest key T
// and how many keys equal to T are taken ("need").  A final ordered compaction emits
// every position with key > T plus the first `need` positions with key == T, so the
// output is ascending by position.  One 1024-thread work-group per query row; the row
// is re-read from L2 on each pass.
#include "common.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

// block-wide exclusive scan of one int per thread; returns prefix, writes total
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int t = (lane < kTopkWaves) ? wave_tot[lane] : 0;
    int s = t;
#pragma unroll
    for (int o = 1; o < kTopkWaves; o <<= 1) {
      const int y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < kTopkWaves) wave_tot[kTopkWaves + lane] = s - t;   // exclusive wave offsets
    if (lane == kTopkWaves - 1) wave_tot[2 * kTopkWaves] = s;
  }
  __syncthreads();
  const int res = wave_tot[kTopkWaves + wave] + x - v;
  total = wave_tot[2 * kTopkWaves];
  __syncthreads();
  return res;
}

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const float* __restrict__ scores, int64_t stride,
                                                            const int32_t* __restrict__ seq_lens, int Sq, int k,
                                                            int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kBins];
  __shared__ int wave_tot[2 * kTopkWaves + 1];
  __shared__ uint32_t red[2 * kTopkWaves];
  __shared__ uint32_t sel_digit;
  __shared__ int sel_above;

  const int row = blockIdx.x;
  const int b = row / Sq, t = row % Sq;
  int n = seq_lens[b] - Sq + 1 + t;
  if (n < 0) n = 0;
  int32_t* out = idx + (int64_t)row * k;
  const float* src = scores + (int64_t)row * stride;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  if (n <= k) {
    for (int i = tid; i < k; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }

  // ---- pass 0: min / max key of the row
  uint32_t kmin = 0xffffffffu, kmax = 0;
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = float_key(src[i]);
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) {
    red[wave] = kmin;
    red[kTopkWaves + wave] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0;
  for (int w = 0; w < kTopkWaves; ++w) {
    kmin = min(kmin, red[w]);
    kmax = max(kmax, red[kTopkWaves + w]);
  }

  // ---- radix select of the k-th largest key
  uint32_t prefix;
  int remaining = k;
  int hi;                                   // bits >= hi of the answer are known
  if (kmin == kmax) {
    prefix = kmin;
    hi = 0;
  } else {
    const int top = 31 - __builtin_clz(kmin ^ kmax);   // highest differing bit
    hi = top + 1;
    prefix = (hi == 32) ? 0u : (kmin & ~((1u << hi) - 1u));
  }
  while (hi > 0) {
    const int nb = hi < kDigitBits ? hi : kDigitBits;
    const int sh = hi - nb;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = float_key(src[i]);
      const bool match = (hi == 32) ? true : ((key >> hi) == (prefix >> hi));
      if (match) atomicAdd(&hist[(key >> sh) & dmask], 1u);
    }
    __syncthreads();
    // suffix counts from the top digit down; thread i covers digits 2047-2i, 2046-2i
    const int d_hi = kBins - 1 - 2 * tid, d_lo = d_hi - 1;
    const int c_hi = (int)hist[d_hi], c_lo = (int)hist[d_lo];
    int tot;
    const int before = block_exclusive_scan(c_hi + c_lo, wave_tot, tot);
    if (before < remaining && remaining <= before + c_hi) {
      sel_digit = (uint32_t)d_hi;
      sel_above = before;
    } else if (before + c_hi < remaining && remaining <= before + c_hi + c_lo) {
      sel_digit = (uint32_t)d_lo;
      sel_above = before + c_hi;
    }
    __syncthreads();
    prefix |= sel_digit << sh;
    remaining -= sel_above;
    hi = sh;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const int need = remaining;               // keys == T to take, lowest positions first

  // ---- ordered compaction
  int sel_base = 0, eq_base = 0;
  for (int c0 = 0; c0 < n && sel_base < k; c0 += kTopkThreads) {
    const int i = c0 + tid;
    const uint32_t key = (i < n) ? float_key(src[i]) : 0u;
    const bool gt = (i < n) && key > T;
    const bool eq = (i < n) && key == T;
    int eq_tot;
    const int eq_rank = eq_base + block_exclusive_scan(eq ? 1 : 0, wave_tot, eq_tot);
    const bool take = gt || (eq && eq_rank < need);
    int sel_tot;
    const int pos = sel_base + block_exclusive_scan(take ? 1 : 0, wave_tot, sel_tot);
    if (take && pos < k) out[pos] = i;
    sel_base += sel_tot;
    eq_base += eq_tot;
  }
  for (int i = sel_base + tid; i < k; i += kTopkThreads) out[i] = -1;   // unreachable when n > k
}

}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int B, int Sq, int k) {
  (void)B;
  (void)Sq;
  (void)k;
  return 0;
}

extern "C" dsa_status_t dsa_topk(const float* scores, int64_t score_stride, const int32_t* seq_lens, int B, int Sq,
                                 int k, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && k >= 1, "dsa_topk: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(scores && seq_lens && idx, "dsa_topk: null pointer");
  DSA_CHECK_ARG(score_stride >= 1, "dsa_topk: score_stride < 1");
  DSA_CHECK_SUPPORTED(k <= 8192, "dsa_topk: k > 8192");
  DSA_CHECK_ARG((int64_t)B * Sq <= 0x7fffffff, "dsa_topk: too many rows");
  hipLaunchKernelGGL(dsa::topk_kernel, dim3((unsigned)(B * Sq)), dim3(dsa::kTopkThreads), 0, stream, scores,
                     score_stride, seq_lens, Sq, k, idx);
  return dsa::launch_status("dsa_topk");
}
