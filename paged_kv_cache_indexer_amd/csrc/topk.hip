// Top-k selection of indexer scores ("Shared-Indexer KV Cache Offload for GLM-5.2",
// §2.1: the 2048 best positions per query feed sparse attention).
//
// Order: score descending, then position ascending; -0.0 == +0.0.  Scores map to
// order-preserving uint32 keys.
//
// Stage 1 (many work-groups per row): the row's n positions are cut into chunks of C
// positions; chunk c (len_c positions) keeps its r_c = min(len_c, 2 ceil(k len_c / n)) best
// keys as candidates, in position order, and records its r_c-th largest key X_c.
// Stage 2 (one work-group per row): the exact select over the ~2k candidates gives the
// row's k-th key T; it is the row's answer whenever every chunk that left keys out has
// X_c < T.  Otherwise the row is selected again from its scores, filtered by a lower bound
// of the k-th key derived from the X_c (see topk_select_kernel).
//
// Both stages use the same select: an MSB-first radix search for the r-th largest key T
// (digits of up to 11 bits, starting below the bits that the smallest and the largest
// key share) and `need`, the number of keys equal to T that are taken (lowest positions
// first).
#include <algorithm>

#include "common.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kMaxChunkElems = 32768;     // stage-1 LDS staging: 128 KB of keys
constexpr int kTargetChunks = 8;

struct TopkShared {
  uint32_t hist[kBins];
  int wave_tot[2 * kTopkWaves + 1];
  uint32_t red[2 * kTopkWaves];
  uint32_t sel_digit;
  int sel_above;
};

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

// k-th largest key T among keys[0..n) (n > k) and how many keys == T are taken.
// KEY(i) returns the i-th key; reads are repeated once per pass.
template <typename KeyFn>
__device__ void radix_select(KeyFn KEY, int n, int k, TopkShared& sh, uint32_t& T_out, int& need_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0;
  for (int i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = KEY(i);
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) {
    sh.red[wave] = kmin;
    sh.red[kTopkWaves + wave] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0;
  for (int w = 0; w < kTopkWaves; ++w) {
    kmin = min(kmin, sh.red[w]);
    kmax = max(kmax, sh.red[kTopkWaves + w]);
  }
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
    const int sh_ = hi - nb;
    const uint32_t dmask = (1u << nb) - 1u;
    for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = KEY(i);
      const bool match = (hi == 32) ? true : ((key >> hi) == (prefix >> hi));
      if (match) atomicAdd(&sh.hist[(key >> sh_) & dmask], 1u);
    }
    __syncthreads();
    // suffix counts from the top digit down; thread i covers digits 2047-2i, 2046-2i
    const int d_hi = kBins - 1 - 2 * tid, d_lo = d_hi - 1;
    const int c_hi = (int)sh.hist[d_hi], c_lo = (int)sh.hist[d_lo];
    int tot;
    const int before = block_exclusive_scan(c_hi + c_lo, sh.wave_tot, tot);
    if (before < remaining && remaining <= before + c_hi) {
      sh.sel_digit = (uint32_t)d_hi;
      sh.sel_above = before;
    } else if (before + c_hi < remaining && remaining <= before + c_hi + c_lo) {
      sh.sel_digit = (uint32_t)d_lo;
      sh.sel_above = before + c_hi;
    }
    __syncthreads();
    prefix |= sh.sel_digit << sh_;
    remaining -= sh.sel_above;
    hi = sh_;
    __syncthreads();
  }
  T_out = prefix;
  need_out = remaining;
}

// Ordered compaction: for i ascending, take i if key > T, or key == T among the first
// `need` such; EMIT(slot, i, key) for each taken element.  Each thread owns PER
// consecutive elements per round so the scan order is element order.
template <int PER, typename KeyFn, typename EmitFn>
__device__ void ordered_take(KeyFn KEY, int n, uint32_t T, int need, int k, TopkShared& sh, EmitFn EMIT) {
  const int tid = threadIdx.x;
  int sel_base = 0, eq_base = 0;
  for (int c0 = 0; c0 < n && sel_base < k; c0 += kTopkThreads * PER) {
    uint32_t key[PER];
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = c0 + tid * PER + r;
      key[r] = (i < n) ? KEY(i) : 0u;
      n_gt += (i < n && key[r] > T);
      n_eq += (i < n && key[r] == T);
    }
    int eq_tot, gt_tot;
    int eq_rank = eq_base + block_exclusive_scan(n_eq, sh.wave_tot, eq_tot);
    // taken by this thread: all its > T, plus its == T while the rank is below need
    int take_eq = need - eq_rank;
    take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
    int sel_tot;
    int pos = sel_base + block_exclusive_scan(n_gt + take_eq, sh.wave_tot, sel_tot);
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = c0 + tid * PER + r;
      if (i >= n) break;
      bool take = key[r] > T;
      if (key[r] == T) {
        take = eq_rank < need;
        ++eq_rank;
      }
      if (take) {
        if (pos < k) EMIT(pos, i, key[r]);
        ++pos;
      }
    }
    (void)gt_tot;
    sel_base += sel_tot;
    eq_base += eq_tot;
  }
}

struct TopkArgs {
  const float* scores;
  int64_t stride;
  const int32_t* seq_lens;
  int Sq, k;
  int chunk;          // C: positions per stage-1 chunk
  int max_chunks;     // chunk slots per row in the workspace
  int cap;            // candidate slots per chunk: min(C, 2k)
  uint32_t* xc;       // [rows, max_chunks] cut key of each chunk
  uint2* cand;        // [rows, max_chunks, cap] (key, position) candidates
  int32_t* idx;
};

__device__ __forceinline__ int row_len(const TopkArgs& a, int row) {
  const int b = row / a.Sq, t = row % a.Sq;
  const int n = a.seq_lens[b] - a.Sq + 1 + t;
  return n < 0 ? 0 : n;
}

// candidates kept by a chunk of `len` of the row's `n` positions: twice its share
// ceil(k * len / n) of the k, at most len.  The shares add up to at least k.
__device__ __forceinline__ int chunk_keep(int k, int len, int n) {
  const int share = (int)(((int64_t)k * len + n - 1) / n);
  return min(len, 2 * share);
}

// stage 1, grid (max_chunks, rows): chunk c keeps its r_c best keys (r_c = chunk_keep) as
// (key, position) candidates in position order; X_c = its r_c-th largest key, so every key
// it left out is < X_c, or == X_c at a later position.
__global__ void __launch_bounds__(kTopkThreads) topk_chunk_kernel(TopkArgs a) {
  extern __shared__ uint32_t skeys[];
  __shared__ TopkShared sh;
  const int row = blockIdx.y, c = blockIdx.x;
  const int n = row_len(a, row);
  if (n <= a.k) return;                       // stage 2 writes 0..n-1 directly
  const int lo = c * a.chunk;
  if (lo >= n) return;
  const int len = min(a.chunk, n - lo);
  const int r = chunk_keep(a.k, len, n);
  const float* src = a.scores + (int64_t)row * a.stride + lo;
  uint2* out = a.cand + ((int64_t)row * a.max_chunks + c) * a.cap;
  uint32_t kmin = 0xffffffffu;
  for (int i0 = 0; i0 < len; i0 += 8 * kTopkThreads) {      // 8 independent loads in flight
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {                 // unconditional (clamped) loads stay in flight together
      const int i = i0 + q * kTopkThreads + threadIdx.x;
      v[q] = src[min(i, len - 1)];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = i0 + q * kTopkThreads + threadIdx.x;
      if (i < len) {
        const uint32_t key = float_key(v[q]);
        skeys[i] = key;
        kmin = min(kmin, key);
      }
    }
  }
  __syncthreads();
  uint32_t T;
  if (r >= len) {                              // the whole chunk is kept; X_c = its smallest key
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = kmin;
    __syncthreads();
    T = 0xffffffffu;
    for (int w = 0; w < kTopkWaves; ++w) T = min(T, sh.red[w]);
    for (int i = threadIdx.x; i < len; i += kTopkThreads) out[i] = make_uint2(skeys[i], (uint32_t)(lo + i));
  } else {
    int need;
    radix_select([&](int i) { return skeys[i]; }, len, r, sh, T, need);
    ordered_take<8>([&](int i) { return skeys[i]; }, len, T, need, r, sh,
                    [&](int slot, int i, uint32_t key) { out[slot] = make_uint2(key, (uint32_t)(lo + i)); });
  }
  if (threadIdx.x == 0) a.xc[(int64_t)row * a.max_chunks + c] = T;
}

// stage 2: one work-group per row.  The chunks' candidates (about 2k, concatenated in
// chunk order, so in position order) are staged in LDS and the exact select runs there,
// giving the k-th key T.  The answer is exact if every chunk that left keys out has
// X_c < T: all keys it left out are then below T.  Otherwise (ties at a chunk's cut, or
// more than twice a chunk's share in the answer) the row is selected again from its
// scores: the bound M is the largest X_c such that the chunks whose X is >= X_c hold at
// least k keys >= it, which makes M a lower bound of the row's k-th key; the row's keys
// >= M are compacted in position order into LDS and selected exactly; if ties at the
// bound leave more keys than LDS holds, the select runs over the whole row.
constexpr int kFiltPer = 16;                       // keys per thread per filter round
constexpr int kFiltLds = 8192;                     // candidates / filtered keys kept in LDS
static_assert(kFiltPer * kTopkWaves == 256, "the filter scan covers 4 counts per lane of one wave");
constexpr int kSelectLds = kFiltLds * 2;           // 32-bit words of dynamic LDS: keys + positions
constexpr int kMaxChunks = 64;                     // chunks one wave combines
__global__ void __launch_bounds__(kTopkThreads) topk_select_kernel(TopkArgs a) {
  extern __shared__ uint32_t fl[];                 // [kFiltLds] keys, then [kFiltLds] positions
  __shared__ TopkShared sh;
  __shared__ uint32_t m_sh;
  __shared__ int ok_sh;
  __shared__ int coff[kMaxChunks + 1];
  __shared__ int fcnt[kFiltPer * kTopkWaves];
  __shared__ int ftot;
  const int row = blockIdx.x;
  const int n = row_len(a, row);
  int32_t* out = a.idx + (int64_t)row * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  const float* src = a.scores + (int64_t)row * a.stride;
  const int nch = (n + a.chunk - 1) / a.chunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t* fkey = fl;
  uint32_t* fpos = fl + kFiltLds;
  uint32_t xj = 0;                                 // wave 0, lane j < nch: X_j
  int rj = 0, lenj = 0;
  if (wave == 0) {
    if (lane < nch) {
      xj = a.xc[(int64_t)row * a.max_chunks + lane];
      lenj = min(a.chunk, n - lane * a.chunk);
      rj = chunk_keep(a.k, lenj, n);
    }
    int incl = rj;                                 // candidate offsets of the chunks
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane < nch) coff[lane] = incl - rj;
    if (lane == nch - 1) coff[nch] = incl;
  }
  __syncthreads();
  const int n_cand = coff[nch];
  uint32_t T;
  int need;
  if (n_cand <= kFiltLds) {
    // stage the candidates: slot j belongs to the last chunk whose offset is <= j
    for (int j0 = 0; j0 < n_cand; j0 += 4 * kTopkThreads) {
      uint2 v[4];
      int jj[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = min(j0 + q * kTopkThreads + (int)threadIdx.x, n_cand - 1);
        int lo = 0, hi = nch - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (coff[mid] <= j) lo = mid; else hi = mid - 1;
        }
        jj[q] = j;
        v[q] = a.cand[((int64_t)row * a.max_chunks + lo) * a.cap + (j - coff[lo])];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (j0 + q * kTopkThreads + (int)threadIdx.x < n_cand) {
          fkey[jj[q]] = v[q].x;
          fpos[jj[q]] = v[q].y;
        }
      }
    }
    __syncthreads();
    radix_select([&](int j) { return fkey[j]; }, n_cand, a.k, sh, T, need);
    if (wave == 0) {
      const bool bad = lane < nch && rj < lenj && !(xj < T);
      const uint64_t any_bad = __builtin_amdgcn_ballot_w64(bad);
      if (lane == 0) ok_sh = (any_bad == 0);
    }
    __syncthreads();
    if (ok_sh) {
      ordered_take<4>([&](int j) { return fkey[j]; }, n_cand, T, need, a.k, sh,
                      [&](int slot, int j, uint32_t) { out[slot] = (int32_t)fpos[j]; });
      return;
    }
  }
  // ---- select again from the row's scores
  if (wave == 0) {
    // lane j tests X_j as the bound: keys guaranteed >= X_j = sum of r_c over X_c >= X_j
    int64_t guaranteed = 0;
    for (int c = 0; c < nch; ++c) {
      const uint32_t x = (uint32_t)__shfl((int)xj, c);
      const int r = __shfl(rj, c);
      if (x >= xj) guaranteed += r;
    }
    uint32_t m = (lane < nch && guaranteed >= a.k) ? xj : 0u;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if (lane == 0) m_sh = m;
  }
  __syncthreads();
  const uint32_t M = m_sh;
  // ordered compaction of the keys >= M.  Loads are coalesced (i = round base + q*1024 +
  // thread); order is (q, wave, lane), so a ballot per load plus one scan over the
  // (q, wave) counts gives every kept key its position-ordered slot.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int n_f = 0;
  for (int i0 = 0; i0 < n; i0 += kTopkThreads * kFiltPer) {
    uint32_t key[kFiltPer];
    uint64_t keep[kFiltPer];
#pragma unroll
    for (int q = 0; q < kFiltPer; ++q) {          // unconditional (clamped) loads stay in flight together
      const int i = i0 + q * kTopkThreads + threadIdx.x;
      key[q] = float_key(src[min(i, n - 1)]);
    }
#pragma unroll
    for (int q = 0; q < kFiltPer; ++q) {
      const int i = i0 + q * kTopkThreads + threadIdx.x;
      keep[q] = __builtin_amdgcn_ballot_w64(i < n && key[q] >= M);
      if (lane == 0) fcnt[q * kTopkWaves + wave] = __builtin_popcountll(keep[q]);
    }
    __syncthreads();
    if (wave == 0) {                               // exclusive scan of the 256 (q, wave) counts
      int c4[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c4[i] = fcnt[lane * 4 + i];
        s += c4[i];
      }
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      int run = incl - s;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fcnt[lane * 4 + i] = run;
        run += c4[i];
      }
      if (lane == 63) ftot = incl;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kFiltPer; ++q) {
      if ((keep[q] >> lane) & 1ull) {
        const int pos = n_f + fcnt[q * kTopkWaves + wave] + __builtin_popcountll(keep[q] & lt_mask);
        if (pos < kFiltLds) {
          fkey[pos] = key[q];
          fpos[pos] = (uint32_t)(i0 + q * kTopkThreads + threadIdx.x);
        }
      }
    }
    n_f += ftot;
    __syncthreads();
  }
  if (n_f <= kFiltLds) {
    if (n_f <= a.k) {                              // only when ties make the bound keep exactly k
      for (int i = threadIdx.x; i < a.k; i += kTopkThreads) out[i] = (i < n_f) ? (int32_t)fpos[i] : -1;
      return;
    }
    radix_select([&](int j) { return fkey[j]; }, n_f, a.k, sh, T, need);
    ordered_take<4>([&](int j) { return fkey[j]; }, n_f, T, need, a.k, sh,
                    [&](int slot, int j, uint32_t) { out[slot] = (int32_t)fpos[j]; });
  } else {                                         // many keys tie at the bound: select over the whole row
    radix_select([&](int i) { return float_key(src[i]); }, n, a.k, sh, T, need);
    ordered_take<4>([&](int i) { return float_key(src[i]); }, n, T, need, a.k, sh,
                    [&](int slot, int i, uint32_t) { out[slot] = i; });
  }
}

static void topk_geometry(int64_t stride, int k, int& chunk, int& max_chunks, int& cap) {
  // about kTargetChunks chunks of the longest row, at most 128 KB of keys each
  int64_t c = (stride + kTargetChunks - 1) / kTargetChunks;
  c = (c + 1023) / 1024 * 1024;
  if (c > kMaxChunkElems) c = kMaxChunkElems;
  chunk = (int)c;
  max_chunks = (int)((stride + c - 1) / c);
  cap = (int)std::min<int64_t>(c, 2 * (int64_t)k);
}

}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int B, int Sq, int k, int64_t score_stride) {
  if (B <= 0 || Sq <= 0 || k <= 0 || score_stride <= 0) return 0;
  int chunk, max_chunks, cap;
  dsa::topk_geometry(score_stride, k, chunk, max_chunks, cap);
  return (size_t)B * Sq * max_chunks * ((size_t)cap * sizeof(uint2) + sizeof(uint32_t));
}

extern "C" dsa_status_t dsa_topk(const float* scores, int64_t score_stride, const int32_t* seq_lens, int B, int Sq,
                                 int k, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && k >= 1, "dsa_topk: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(scores && seq_lens && idx, "dsa_topk: null pointer");
  DSA_CHECK_ARG(score_stride >= 1 && score_stride < ((int64_t)1 << 31), "dsa_topk: bad score_stride");
  DSA_CHECK_SUPPORTED(k <= 8192, "dsa_topk: k > 8192");
  DSA_CHECK_ARG((int64_t)B * Sq <= 65535, "dsa_topk: more than 65535 rows");
  TopkArgs a{};
  a.scores = scores;
  a.stride = score_stride;
  a.seq_lens = seq_lens;
  a.Sq = Sq;
  a.k = k;
  topk_geometry(score_stride, k, a.chunk, a.max_chunks, a.cap);
  DSA_CHECK_SUPPORTED(a.max_chunks <= kMaxChunks, "dsa_topk: score_stride above %d", kMaxChunks * kMaxChunkElems);
  const size_t need = dsa_topk_workspace_size(B, Sq, k, score_stride);
  if (ws == nullptr || ws_bytes < need) {
    set_last_error("dsa_topk: workspace %zu < %zu bytes", ws_bytes, need);
    return DSA_ERR_WORKSPACE;
  }
  DSA_CHECK_ARG(((uintptr_t)ws & 7) == 0, "dsa_topk: workspace not 8-byte aligned");
  const size_t rows = (size_t)B * Sq;
  a.cand = static_cast<uint2*>(ws);
  a.xc = reinterpret_cast<uint32_t*>(a.cand + rows * a.max_chunks * a.cap);
  a.idx = idx;
  const size_t lds = (size_t)a.chunk * sizeof(uint32_t);
  static bool attr = false;
  if (!attr) {
    hipFuncSetAttribute((const void*)topk_chunk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)(kMaxChunkElems * sizeof(uint32_t)));
    hipFuncSetAttribute((const void*)topk_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)(kSelectLds * sizeof(uint32_t)));
    attr = true;
  }
  DSA_LAUNCH(topk_chunk_kernel, dim3(a.max_chunks, B * Sq), dim3(kTopkThreads), lds, stream, a);
  dsa_status_t st = launch_status("dsa_topk(chunk)");
  if (st != DSA_OK) return st;
  DSA_LAUNCH(topk_select_kernel, dim3(B * Sq), dim3(kTopkThreads), kSelectLds * sizeof(uint32_t), stream, a);
  return launch_status("dsa_topk(select)");
}
