// De-duplicated union of the query tokens' selections ("Shared-Indexer KV Cache Offload for
// GLM-5.2": §4.2, the plan classifies a step's top-k ids once and de-duplicates repeated
// misses; §5.1, MTP draft steps reuse the first decode step's selection, so the positions
// a request's draft tokens select largely coincide).
//
// One work-group per request.  The Sq selection rows (ascending, -1 padding at the end, as
// dsa_topk writes them) are staged in LDS.  An entry x of row t owns its value when no
// earlier row and no earlier entry of row t holds x.  Every distinct value has exactly one
// owner, so the union index of x is the number of owners, over all rows, whose value is
// below x: sum over rows t' of (owners of row t' before lower_bound_t'(x)), read from an
// exclusive prefix count of the owner flags.  Each entry records its union index and sets
// its bit in its row's membership mask; owners write the union.
#include "common.h"

namespace dsa {

constexpr int kUnionThreads = 1024;
constexpr int kUnionMax = 8192;             // Sq * k
constexpr int kUnionMaxSq = 16;
constexpr int kUnionPer = kUnionMax / kUnionThreads;

struct UnionArgs {
  const int32_t* topk;   // [B, Sq, k]
  int Sq, k;
  int32_t* uni;          // [B, Sq * k]
  int32_t* count;        // [B]
  int32_t* uidx;         // [B, Sq, k] or null
  uint32_t* member;      // [B, Sq, W] or null
  int W;                 // ceil(Sq * k / 32)
  int32_t* err;
};

// first index i in [0, n) of the ascending row with row[i] >= x (n if none)
__device__ __forceinline__ int lower_bound_lds(const int32_t* row, int n, int32_t x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(kUnionThreads) union_kernel(UnionArgs a) {
  __shared__ int32_t vals[kUnionMax];           // rows; padding as INT32_MAX (above every position)
  __shared__ int32_t pre[kUnionMax + 1];        // exclusive prefix count of the owner flags
  __shared__ uint32_t mem[kUnionMaxSq * (kUnionMax / 32)];  // membership bits, row t at t * W
  __shared__ int32_t wave_tot[2 * (kUnionThreads / 64) + 1];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Sq = a.Sq, k = a.k, n = Sq * k;
  const int32_t* src = a.topk + (int64_t)b * n;
  for (int e = tid; e < n; e += kUnionThreads) {
    const int32_t v = src[e];
    vals[e] = v >= 0 ? v : INT32_MAX;
  }
  for (int i = tid; i < Sq * a.W; i += kUnionThreads) mem[i] = 0;
  __syncthreads();

  // owner flags, kUnionPer consecutive entries per thread (element order = scan order)
  int own[kUnionPer];
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < kUnionPer; ++r) {
    const int e = tid * kUnionPer + r;
    own[r] = 0;
    if (e < n) {
      const int32_t x = vals[e];
      const int t = e / k, j = e - t * k;
      if (x != INT32_MAX) {
        bool o = !(j > 0 && vals[e - 1] == x);
        if (j > 0 && vals[e - 1] > x) count_error(a.err);   // a row out of order
        for (int t2 = 0; t2 < t && o; ++t2) {
          const int lb = lower_bound_lds(vals + t2 * k, k, x);
          o = !(lb < k && vals[t2 * k + lb] == x);
        }
        own[r] = o ? 1 : 0;
      }
    }
    cnt += own[r];
  }
  // block exclusive scan of the per-thread counts
  int x = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  constexpr int NWV = kUnionThreads / 64;
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  if (wave == 0) {
    const int t = (lane < NWV) ? wave_tot[lane] : 0;
    int s = t;
#pragma unroll
    for (int o = 1; o < NWV; o <<= 1) {
      const int y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < NWV) wave_tot[NWV + lane] = s - t;
    if (lane == NWV - 1) wave_tot[2 * NWV] = s;
  }
  __syncthreads();
  int run = wave_tot[NWV + wave] + x - cnt;
#pragma unroll
  for (int r = 0; r < kUnionPer; ++r) {
    const int e = tid * kUnionPer + r;
    if (e < n) pre[e] = run;
    run += own[r];
  }
  const int total = wave_tot[2 * NWV];
  if (tid == 0) pre[n] = total;
  __syncthreads();

  // union index of every entry; owners write the union
  int32_t* uni = a.uni + (int64_t)b * n;
  for (int e = tid; e < n; e += kUnionThreads) {
    const int32_t x = vals[e];
    const int t = e / k, j = e - t * k;
    int u = -1;
    if (x != INT32_MAX) {
      u = 0;
      for (int t2 = 0; t2 < Sq; ++t2) {
        const int lb = (t2 == t) ? lower_bound_lds(vals + t * k, j + 1, x) : lower_bound_lds(vals + t2 * k, k, x);
        u += pre[t2 * k + lb] - pre[t2 * k];
      }
      atomicOr(&mem[t * a.W + (u >> 5)], 1u << (u & 31));
      if (pre[e + 1] != pre[e]) uni[u] = x;     // this entry owns x
    }
    if (a.uidx) a.uidx[(int64_t)b * n + e] = u;
  }
  for (int u = total + tid; u < n; u += kUnionThreads) uni[u] = -1;
  if (tid == 0) a.count[b] = total;
  __syncthreads();
  if (a.member)
    for (int i = tid; i < Sq * a.W; i += kUnionThreads) a.member[(int64_t)b * Sq * a.W + i] = mem[i];
}

}  // namespace dsa

extern "C" dsa_status_t dsa_topk_union(const int32_t* topk, int B, int Sq, int k, int32_t* uni, int32_t* count,
                                       int32_t* uidx, uint32_t* member, int32_t* err_count, hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && k >= 1, "dsa_topk_union: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(topk && uni && count, "dsa_topk_union: null pointer");
  DSA_CHECK_SUPPORTED(Sq <= kUnionMaxSq && (int64_t)Sq * k <= kUnionMax,
                      "dsa_topk_union: needs Sq <= 16 and Sq * k <= 8192");
  UnionArgs a{};
  a.topk = topk;
  a.Sq = Sq;
  a.k = k;
  a.uni = uni;
  a.count = count;
  a.uidx = uidx;
  a.member = member;
  a.W = (Sq * k + 31) / 32;
  a.err = err_count;
  DSA_LAUNCH(union_kernel, dim3((unsigned)B), dim3(kUnionThreads), 0, stream, a);
  return launch_status("dsa_topk_union");
}
