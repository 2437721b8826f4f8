// Top-k selection of indexer scores ("Shared-Indexer KV Cache Offload for GLM-5.2",
// §2.1: the 2048 best positions per query feed sparse attention).
//
// Order: score descending, then position ascending; -0.0 == +0.0.  Scores map to
// order-preserving uint32 keys.
//
// Stage 1 cuts each row into chunks; chunk c (len_c positions) keeps at most r_c =
// min(len_c, 2 ceil(k len_c / n) + slack) of its best keys as candidates, in position
// order, in fixed slots (unused slots hold key 0, which no select takes), and records its
// candidate count and a cut key X_c: every key it left out is <= X_c, and one equal to X_c
// sits after every kept key equal to it.  The chunks' slots are laid back to back per row,
// so the row's candidate list is in position order.  Two forms:
//   * wave chunks (rows up to 256K positions whose candidate bound fits the exact select's
//     registers): one wave per 1024 positions, a threshold search whose count lands in a
//     window just below r_c (see topk_wave_kernel); no barriers, no LDS;
//   * work-group chunks of 8192 or, when the grid would otherwise take more than one
//     round of the chip's work-group slots, 16384 positions: an exact select of r_c
//     (slack 0).
// Stage 2 (one work-group per row): the exact select over the candidates is the row's
// answer whenever every chunk that left keys out has X_c below the smallest key the
// answer may take.  Otherwise the row is selected again from its scores, filtered by a
// lower bound of the k-th key derived from the X_c and the counts (see
// topk_select_kernel).
//
// The work-group selects keep each thread's keys in registers: an MSB-first radix search
// (digits of up to 11 bits, starting below the bits the smallest and largest key share;
// two barriers per digit; it stops as soon as the chosen digit's keys are all taken), then
// one ordered take from per-wave ballots.  The rare re-select runs the same search over
// keys staged in LDS.
#include <algorithm>

#include "topk_wave.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kPer = 8;                            // keys per thread held in registers
constexpr int kChunk = kTopkThreads * kPer;        // stage-1 chunk: 8192 positions
constexpr int kLongPer = 16;                       // keys per thread of the long-row chunks
constexpr int kMaxChunks = kTopkMaxChunks;         // rows up to 2^21 positions
// Stage-1 work-groups that run in one round: 256 CUs x 2 work-groups of 1024 threads (the
// chunk kernel fits eight waves per SIMD).  A larger grid switches to 16384-position chunks.
constexpr int64_t kChunkRound = 512;
constexpr int kMaxCand = kTopkMaxCand;             // stage-2 candidates held in registers
static_assert(kMaxCand == kTopkThreads * kPer, "stage 2 holds kPer candidates per thread");
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;

// ---- LDS-resident select (the rare re-select over a row's scores) ----

template <int NT>
struct TopkShared {
  static_assert(NT % 64 == 0 && (1 << 11) % NT == 0, "whole waves; digits split evenly over threads");
  uint32_t hist[kBins];
  int wave_tot[2 * (NT / 64) + 1];
  uint32_t red[2 * (NT / 64)];
  uint32_t sel_digit;
  int sel_above;
};

// block-wide exclusive scan of one int per thread; returns prefix, writes total
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  constexpr int NW = NT / 64;
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
    int t = (lane < NW) ? wave_tot[lane] : 0;
    int s = t;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const int y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < NW) wave_tot[NW + lane] = s - t;   // exclusive wave offsets
    if (lane == NW - 1) wave_tot[2 * NW] = s;
  }
  __syncthreads();
  const int res = wave_tot[NW + wave] + x - v;
  total = wave_tot[2 * NW];
  __syncthreads();
  return res;
}

// k-th largest key T among keys[0..n) (n > k) and how many keys == T are taken.
// KEY(i) returns the i-th key; reads are repeated once per pass.
template <int NT, typename KeyFn>
__device__ void radix_select(KeyFn KEY, int n, int k, TopkShared<NT>& sh, uint32_t& T_out, int& need_out) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0;
  for (int i = tid; i < n; i += NT) {
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
    sh.red[NW + wave] = kmax;
  }
  __syncthreads();
  kmin = 0xffffffffu;
  kmax = 0;
  for (int w = 0; w < NW; ++w) {
    kmin = min(kmin, sh.red[w]);
    kmax = max(kmax, sh.red[NW + w]);
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
    for (int i = tid; i < kBins; i += NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = KEY(i);
      const bool match = (hi == 32) ? true : ((key >> hi) == (prefix >> hi));
      if (match) atomicAdd(&sh.hist[(key >> sh_) & dmask], 1u);
    }
    __syncthreads();
    // suffix counts from the top digit down; thread i covers the BPT digits below
    // kBins-1-BPT*i, highest first
    constexpr int BPT = kBins / NT;
    const int d0 = kBins - 1 - BPT * tid;
    int cnt[BPT], sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      cnt[j] = (int)sh.hist[d0 - j];
      sum += cnt[j];
    }
    int tot;
    int before = block_exclusive_scan<NT>(sum, sh.wave_tot, tot);
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (before < remaining && remaining <= before + cnt[j]) {
        sh.sel_digit = (uint32_t)(d0 - j);
        sh.sel_above = before;
      }
      before += cnt[j];
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

// Ordered compaction (the re-select path): for i ascending, take i if key > T, or key == T among the first
// `need` such; EMIT(slot, i, key) for each taken element.  Each thread owns PER
// consecutive elements per round so the scan order is element order.
template <int NT, int PER, typename KeyFn, typename EmitFn>
__device__ void ordered_take(KeyFn KEY, int n, uint32_t T, int need, int k, TopkShared<NT>& sh, EmitFn EMIT) {
  const int tid = threadIdx.x;
  int sel_base = 0, eq_base = 0;
  for (int c0 = 0; c0 < n && sel_base < k; c0 += NT * PER) {
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
    int eq_rank = eq_base + block_exclusive_scan<NT>(n_eq, sh.wave_tot, eq_tot);
    // taken by this thread: all its > T, plus its == T while the rank is below need
    int take_eq = need - eq_rank;
    take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
    int sel_tot;
    int pos = sel_base + block_exclusive_scan<NT>(n_gt + take_eq, sh.wave_tot, sel_tot);
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

// ---- register-resident select (both stages' hot path) ----

struct alignas(16) RadixShared {
  uint32_t hist[2][kBins];                 // digit histograms, alternating per pass
  uint32_t red[2 * kTopkWaves];            // per-wave min / max, then per-wave digit counts
  int cnt[kLongPer * kTopkWaves];          // ordered take: packed counts per (slot q, wave)
  uint32_t sel_digit;
  int sel_above;
  int sel_count;
};

// Sum of x over lanes below `upto` (a wave-uniform lane count <= 64), for x held by lane i
// as the i-th value.
__device__ __forceinline__ int wave_prefix_below(int x, int upto) {
  const int incl = wave_sum_incl(x);
  return upto == 0 ? 0 : __builtin_amdgcn_readlane(incl, upto - 1);
}

// Block min / max (each thread passes its own); also clears both histograms.  One barrier.
__device__ __forceinline__ void block_minmax(uint32_t& kmin, uint32_t& kmax, RadixShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  if (lane == 0) {
    sh.red[wave] = kmin;
    sh.red[kTopkWaves + wave] = kmax;
  }
  for (int i = threadIdx.x; i < 2 * kBins; i += kTopkThreads) (&sh.hist[0][0])[i] = 0;
  __syncthreads();
  kmin = wave_min(lane < kTopkWaves ? sh.red[lane] : 0xffffffffu);
  kmax = wave_max(lane < kTopkWaves ? sh.red[kTopkWaves + lane] : 0u);
}

// Threshold of the k best keys of the work-group: every key > T is taken, and the first
// `need` keys == T in position order.  Empty slots hold key 0, which no select takes:
// float_key maps every non-NaN float above 2^23 - 2, the first digit pass skips 0, and
// the later passes' prefix does not match it.
// kmin / kmax are the block min / max of the real keys (block_minmax, which also clears
// the histograms).  Per digit: histogram atomics, a block scan of the counts from the top
// digit down, and the one thread whose digits hold the `remaining`-th key publishes it:
// three barriers.  When a digit's keys are all taken before the last digit, T is one below
// that digit's smallest key and need = 0.
template <int PER>
__device__ void radix_select_reg(const uint32_t (&key)[PER], int k, uint32_t kmin, uint32_t kmax,
                                 RadixShared& sh, uint32_t& T_out, int& need_out) {
  static_assert(kBins == 2 * kTopkThreads, "each thread owns two digits");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t prefix;
  int hi;
  if (kmin == kmax) {
    prefix = kmin;
    hi = 0;
  } else {
    hi = 32 - __builtin_clz(kmin ^ kmax);
    prefix = (hi == 32) ? 0u : (kmin & ~((1u << hi) - 1u));
  }
  int remaining = k;
  int p = 0;
  while (hi > 0) {
    const int nb = hi < kDigitBits ? hi : kDigitBits;
    const int s = hi - nb;
    uint32_t* h = sh.hist[p & 1];
    if (p == 0) {                                  // every real key shares the prefix; empty slots skipped
#pragma unroll
      for (int q = 0; q < PER; ++q)
        if (key[q] != 0u) atomicAdd(&h[__builtin_amdgcn_ubfe(key[q], s, nb)], 1u);
    } else {
      const uint32_t mhi = ~((1u << hi) - 1u);     // hi <= 21 here
#pragma unroll
      for (int q = 0; q < PER; ++q)
        if ((key[q] & mhi) == prefix) atomicAdd(&h[__builtin_amdgcn_ubfe(key[q], s, nb)], 1u);
    }
    __syncthreads();
    // thread t owns digits kBins-1-2t (c_hi) and kBins-2-2t (c_lo): thread order is
    // descending digit order, so a block scan of c_hi + c_lo counts the keys above.
    const uint2 pair = *reinterpret_cast<const uint2*>(h + kBins - 2 - 2 * threadIdx.x);
    const int c_lo = (int)pair.x, c_hi = (int)pair.y, c2 = c_hi + c_lo;
    const int incl = wave_sum_incl(c2);
    if (lane == 63) sh.red[wave] = (uint32_t)incl;
    // the other histogram was last read before the previous pass's last barrier
    uint32_t* hz = sh.hist[(p + 1) & 1];
    for (int i = threadIdx.x; i < kBins; i += kTopkThreads) hz[i] = 0;
    __syncthreads();
    const int before = wave_prefix_below(lane < kTopkWaves ? (int)sh.red[lane] : 0, wave) + incl - c2;
    if (before < remaining && remaining <= before + c2) {   // exactly one thread
      const bool top = remaining <= before + c_hi;
      sh.sel_digit = (uint32_t)(kBins - 1 - 2 * (int)threadIdx.x - (top ? 0 : 1));
      sh.sel_above = top ? before : before + c_hi;
      sh.sel_count = top ? c_hi : c_lo;
    }
    __syncthreads();
    prefix |= sh.sel_digit << s;
    remaining -= sh.sel_above;
    const int count = sh.sel_count;
    hi = s;
    ++p;
    if (hi > 0 && count == remaining) {            // the whole digit is taken: keys >= prefix
      T_out = prefix - 1u;
      need_out = 0;
      return;
    }
  }
  T_out = prefix;
  need_out = remaining;
}

// Ordered take of the keys chosen by (T, need): slot q of thread t is the work-group's
// element q * kTopkThreads + t, so element order is (q, wave, lane); per (q, wave) ballots
// give each kept key its rank.  EMIT(slot, q) for each kept key.  Two barriers.
template <int PER, typename EmitFn>
__device__ void take_reg(const uint32_t (&key)[PER], uint32_t T, int need, RadixShared& sh, EmitFn EMIT) {
  static_assert(PER <= 64, "lane q publishes slot q's counts");
  constexpr int NC = PER * kTopkWaves;             // (slot, wave) counts
  static_assert(NC <= kLongPer * kTopkWaves, "counts fit sh.cnt");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t gtm[PER], eqm[PER];
  int mine = 0;                                    // lane q: packed (eq, gt) counts of slot q
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    gtm[q] = __builtin_amdgcn_ballot_w64(key[q] > T);
    eqm[q] = need > 0 ? __builtin_amdgcn_ballot_w64(key[q] == T) : 0ull;
    const int packed = (__builtin_popcountll(eqm[q]) << 16) | __builtin_popcountll(gtm[q]);
    mine = lane == q ? packed : mine;
  }
  if (lane < PER) sh.cnt[lane * kTopkWaves + wave] = mine;
  __syncthreads();
  if (wave == 0) {                                 // exclusive scan of the packed counts
    constexpr int E = (NC + 63) / 64;
    int c[E], sum = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      c[e] = lane * E + e < NC ? sh.cnt[lane * E + e] : 0;
      sum += c[e];
    }
    int run = wave_sum_incl(sum) - sum;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (lane * E + e < NC) sh.cnt[lane * E + e] = run;
      run += c[e];
    }
  }
  __syncthreads();
  auto slot_of = [&](int q, uint64_t gt, uint64_t eq) {   // slot of a kept key, -1 if not kept
    const int base = __builtin_amdgcn_readfirstlane(sh.cnt[q * kTopkWaves + wave]);
    const int gb = lanes_below(gt, base & 0xffff);
    if (eq == 0)                                   // no key == T in this wave's slot q
      return key[q] > T ? gb + min(need, base >> 16) : -1;
    const int eb = lanes_below(eq, base >> 16);
    return key[q] > T ? gb + min(need, eb) : ((key[q] == T && eb < need) ? gb + eb : -1);
  };
  if constexpr (PER <= kPer) {
    int slot[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) slot[q] = slot_of(q, gtm[q], eqm[q]);
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (slot[q] >= 0) EMIT(slot[q], q);
  } else {
    // sixteen keys per thread: the ballots are taken again here rather than held across the
    // scan, which keeps the kernel within the registers of eight waves per SIMD
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const uint64_t gt = __builtin_amdgcn_ballot_w64(key[q] > T);
      const uint64_t eq = need > 0 ? __builtin_amdgcn_ballot_w64(key[q] == T) : 0ull;
      const int s = slot_of(q, gt, eq);
      if (s >= 0) EMIT(s, q);
    }
  }
}

// stage 1, grid (max_chunks, rows), PER keys per thread (a.chunk = kTopkThreads * PER).
// Chunk c's candidates start at c * r_full in the row's list (r_full: the keep of a full
// chunk; only the last chunk can be shorter).  Eight waves per SIMD (two work-groups per
// CU) for either PER: with sixteen keys the compiler keeps a few scalars in VGPR lanes.
template <int PER>
__global__ void __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
topk_chunk_kernel(TopkArgs a) {
  constexpr int kC = kTopkThreads * PER;
  __shared__ RadixShared sh;
  const int row = blockIdx.y, c = blockIdx.x;
  const int lo = c * kC;
  if (lo >= a.stride) return;
  // the loads are clamped to the row's stride, not its length, so they issue before the
  // length arrives; positions past the length are masked below
  // 32-bit byte offsets from the row's base (the row holds < 2^21 positions): one VGPR per load
  const char* src = reinterpret_cast<const char*>(a.scores + (int64_t)row * a.stride);
  const int last = (int)a.stride - 1;
  float v[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q)
    v[q] = *reinterpret_cast<const float*>(src + (uint32_t)min(lo + q * kTopkThreads + (int)threadIdx.x, last) * 4u);
  const int n = row_len(a, row);
  if (n <= a.k) return;                       // stage 2 writes 0..n-1 directly
  if (lo >= n) return;
  const int len = min(kC, n - lo);
  const int r = chunk_keep(a.k, len, n, a.slack);
  uint2* out = a.cand + (int64_t)row * a.cand_stride + (int64_t)c * chunk_keep(a.k, kC, n, a.slack);
  uint32_t key[PER], kmin = 0xffffffffu, kmax = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {                  // empty slots: key 0
    const bool in = q * kTopkThreads + (int)threadIdx.x < len;
    key[q] = in ? float_key(v[q]) : 0u;
    kmin = min(kmin, in ? key[q] : 0xffffffffu);
    kmax = max(kmax, key[q]);
  }
  block_minmax(kmin, kmax, sh);
  uint32_t T;
  if (r >= len) {                              // the whole chunk is kept; X_c = its smallest key
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = q * kTopkThreads + threadIdx.x;
      if (i < len) out[i] = make_uint2(key[q], (uint32_t)(lo + i));
    }
    T = kmin;
  } else {
    int need;
    radix_select_reg<PER>(key, r, kmin, kmax, sh, T, need);
    take_reg<PER>(key, T, need, sh, [&](int slot, int q) {
      if (slot < r) out[slot] = make_uint2(key[q], (uint32_t)(lo + q * kTopkThreads + (int)threadIdx.x));
    });
  }
  if (threadIdx.x == 0) {
    a.xc[(int64_t)row * a.max_chunks + c] = T;
    a.cc[(int64_t)row * a.max_chunks + c] = min(r, len);
  }
}

// stage 1 on wave chunks, a 1-D grid of rows x G work-groups (G = ceil(max_chunks / 4)):
// wave w of group g owns chunk 4g + w, its slots [c * r_full, c * r_full + r_c) of the row,
// its cut key xc and its candidate count cc.  Work-groups are handed to the eight XCDs in
// turn by their index, and stage 2 runs row r's select on XCD r % 8; when the row count is
// a multiple of 8, the groups of row r are given indices on that same XCD, so that the
// select reads its candidates from the XCD's own L2.
__global__ void __launch_bounds__(kWaveThreads) topk_wave_kernel(TopkArgs a, int groups, int rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int row, grp;
  if ((rows & 7) == 0) {
    const int j = (int)(blockIdx.x >> 3);
    row = (int)(blockIdx.x & 7) + 8 * (j / groups);
    grp = j % groups;
  } else {
    row = (int)blockIdx.x / groups;
    grp = (int)blockIdx.x % groups;
  }
  const int c = grp * (kWaveThreads / 64) + wave;
  const int lo = c * kWaveChunk;
  if (lo >= a.stride) return;                     // whole waves leave; no barrier follows
  // loads issued before the row's length arrives: a chunk inside the stride reads its 4 KB
  // from one base address; the stride's last chunk clamps its positions
  const float* src = a.scores + (int64_t)row * a.stride + lo;
  float v[kWavePer];
  if (lo + kWaveChunk <= a.stride) {
#pragma unroll
    for (int q = 0; q < kWavePer; ++q) v[q] = src[q * 64 + lane];
  } else {
    const int last = (int)a.stride - 1 - lo;
#pragma unroll
    for (int q = 0; q < kWavePer; ++q) v[q] = src[min(q * 64 + lane, last)];
  }
  const int n = row_len(a, row);
  if (n <= a.k) return;                           // stage 2 writes 0..n-1 directly
  if (lo >= n) return;
  const int len = min(kWaveChunk, n - lo);
  const int r = chunk_keep(a.k, len, n, a.slack);
  const int share = (int)(((int64_t)a.k * len + n - 1) / n);
  uint2* out = a.cand + (int64_t)row * a.cand_stride + (int64_t)c * chunk_keep(a.k, kWaveChunk, n, a.slack);
  uint32_t T;
  const int kept = len == kWaveChunk ? wave_chunk<true>(v, len, r, share, lo, out, T)
                                     : wave_chunk<false>(v, len, r, share, lo, out, T);
  if (lane == 0) {
    a.xc[(int64_t)row * a.max_chunks + c] = T;
    a.cc[(int64_t)row * a.max_chunks + c] = kept;
  }
}

// Exact select of the k best of the row's n_cand candidates, PER per thread (candidate j =
// q * kTopkThreads + t in slot q of thread t).  Writes the row's answer and returns true
// unless a chunk that left keys out (cut_t, cut key x_t, one chunk per thread) could hold
// part of it: then it returns false, having written nothing.
template <int PER>
__device__ bool select_candidates(const uint2 (&cv)[kPer], int n_cand, int k, bool cut_t, uint32_t x_t,
                                  RadixShared& rs, int32_t* out) {
  uint32_t key[PER], pos[PER], kmin = 0xffffffffu, kmax = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {                  // slots past n_cand and empty slots: key 0
    const bool in = q * kTopkThreads + (int)threadIdx.x < n_cand;
    key[q] = in ? cv[q].x : 0u;
    pos[q] = cv[q].y;
    kmin = min(kmin, key[q] != 0u ? key[q] : 0xffffffffu);
    kmax = max(kmax, key[q]);
  }
  block_minmax(kmin, kmax, rs);
  uint32_t T;
  int need;
  radix_select_reg<PER>(key, k, kmin, kmax, rs, T, need);
  const uint32_t V = need > 0 ? T : T + 1u;       // smallest key the answer may take
  if (__syncthreads_or(cut_t && !(x_t < V))) return false;
  take_reg<PER>(key, T, need, rs, [&](int slot, int q) {
    if (slot < k) out[slot] = (int32_t)pos[q];
  });
  return true;
}

// stage 2: one work-group per row.  The candidates (about 2k, in position order) are held
// in registers and the exact select over them gives the threshold (T, need); the smallest
// key the answer may take is V = T, or T + 1 when need = 0.  The answer is exact if every
// chunk that left keys out has X_c < V: all keys it left out are then below V.  Otherwise
// (ties at a chunk's cut, or more than twice a chunk's share in the answer) the row is
// selected again from its scores: the bound M is the largest X_c such that the chunks
// whose X is >= X_c hold at least k candidates (all of them >= their chunk's X), which
// makes M a lower bound of the row's k-th key; the row's keys >= M are compacted in
// position order into LDS and selected exactly; if ties at the bound leave more keys than
// LDS holds, the select runs over the whole row.
constexpr int kFiltPer = 16;                       // keys per thread per filter round
constexpr int kFiltLds = 8192;                     // filtered keys kept in LDS
static_assert(kFiltPer * kTopkWaves == 256, "the filter scan covers 4 counts per lane of one wave");
constexpr int kSelectLds = kFiltLds * 2;           // 32-bit words of dynamic LDS: keys + positions
__global__ void __launch_bounds__(kTopkThreads) topk_select_kernel(TopkArgs a) {
  extern __shared__ uint32_t fl[];                 // [kFiltLds] keys, then [kFiltLds] positions
  __shared__ RadixShared rs;
  __shared__ TopkShared<kTopkThreads> sh;
  __shared__ uint32_t xs[kMaxChunks];
  __shared__ int rsz[kMaxChunks];
  __shared__ uint32_t m_sh;
  __shared__ int fcnt[kFiltPer * kTopkWaves];
  __shared__ int ftot;
  const int row = blockIdx.x;
  // the row's candidate slots and cut keys are loaded before its length arrives (clamped
  // to the row's workspace; slots past the row's count are masked below)
  const uint2* cr = a.cand + (int64_t)row * a.cand_stride;
  uint2 cv[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) cv[q] = cr[min(q * kTopkThreads + (int)threadIdx.x, a.cand_stride - 1)];
  const uint32_t x_ld = a.xc[(int64_t)row * a.max_chunks + min((int)threadIdx.x, a.max_chunks - 1)];
  const int c_ld = a.cc[(int64_t)row * a.max_chunks + min((int)threadIdx.x, a.max_chunks - 1)];
  const int n = row_len(a, row);
  int32_t* out = a.idx + (int64_t)row * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kTopkThreads) out[i] = (i < n) ? i : -1;
    return;
  }
  const float* src = a.scores + (int64_t)row * a.stride;
  const int chunk = a.chunk;
  const int nch = (n + chunk - 1) / chunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r_full = chunk_keep(a.k, chunk, n, a.slack);
  const int n_cand = (nch - 1) * r_full + chunk_keep(a.k, n - (nch - 1) * chunk, n, a.slack);
  // thread t < nch: chunk t's cut key, keep, and whether it left keys out
  uint32_t x_t = 0;
  int r_t = 0;
  bool cut_t = false;
  if ((int)threadIdx.x < nch) {
    const int len_t = min(chunk, n - (int)threadIdx.x * chunk);
    x_t = x_ld;
    r_t = c_ld;
    cut_t = r_t < len_t;
    xs[threadIdx.x] = x_t;
    rsz[threadIdx.x] = r_t;
  }
  uint32_t* fkey = fl;
  uint32_t* fpos = fl + kFiltLds;
  uint32_t T;
  int need;
  // the register select sized to the candidate count (its work scales with the slots)
  if (n_cand <= kTopkThreads * 2) {
    if (select_candidates<2>(cv, n_cand, a.k, cut_t, x_t, rs, out)) return;
  } else if (n_cand <= kTopkThreads * 4) {
    if (select_candidates<4>(cv, n_cand, a.k, cut_t, x_t, rs, out)) return;
  } else if (n_cand <= kTopkThreads * 5) {
    if (select_candidates<5>(cv, n_cand, a.k, cut_t, x_t, rs, out)) return;
  } else if (n_cand <= kTopkThreads * 6) {
    if (select_candidates<6>(cv, n_cand, a.k, cut_t, x_t, rs, out)) return;
  } else if (n_cand <= kMaxCand) {
    if (select_candidates<kPer>(cv, n_cand, a.k, cut_t, x_t, rs, out)) return;
  }
  // ---- select again from the row's scores
  if (threadIdx.x == 0) m_sh = 0;
  __syncthreads();
  if ((int)threadIdx.x < nch) {
    // keys guaranteed >= X_t: the candidates of every chunk whose X is >= X_t
    int64_t guaranteed = 0;
    for (int c = 0; c < nch; ++c)
      if (xs[c] >= x_t) guaranteed += rsz[c];
    if (guaranteed >= a.k) atomicMax(&m_sh, x_t);
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
    radix_select<kTopkThreads>([&](int j) { return fkey[j]; }, n_f, a.k, sh, T, need);
    ordered_take<kTopkThreads, 4>([&](int j) { return fkey[j]; }, n_f, T, need, a.k, sh,
                    [&](int slot, int j, uint32_t) { out[slot] = (int32_t)fpos[j]; });
  } else {                                         // many keys tie at the bound: select over the whole row
    radix_select<kTopkThreads>([&](int i) { return float_key(src[i]); }, n, a.k, sh, T, need);
    ordered_take<kTopkThreads, 4>([&](int i) { return float_key(src[i]); }, n, T, need, a.k, sh,
                    [&](int slot, int i, uint32_t) { out[slot] = i; });
  }
}

void topk_geometry(int64_t stride, int k, int chunk, int slack, int& max_chunks, int& cand_stride) {
  max_chunks = (int)((stride + chunk - 1) / chunk);
  // sum over chunks of min(len_c, 2 ceil(k len_c / n) + slack) <= min(n, 2k + (2 + slack) * chunks)
  cand_stride = (int)std::min<int64_t>(stride, 2 * (int64_t)k + (2 + (int64_t)slack) * max_chunks);
}

// Wave chunks serve rows of up to kWaveMaxStride positions whose candidate lists fit the
// exact select's registers: the slack is the largest one up to kWaveSlack that keeps the
// candidate bound within kMaxCand.  Returns -1 when it would fall below kWaveMinSlack
// (longer rows or larger k take the work-group chunks).
int topk_wave_slack(int64_t stride, int k) {
  if (stride > kWaveMaxStride) return -1;
  if (stride <= kMaxCand) return kWaveSlack;
  const int64_t nch = (stride + kWaveChunk - 1) / kWaveChunk;
  const int64_t slack = std::min<int64_t>(kWaveSlack, (kMaxCand - 2 * (int64_t)k) / nch - 2);
  return slack >= kWaveMinSlack ? (int)slack : -1;
}

dsa_status_t topk_setup(const char* who, const float* scores, int64_t score_stride, const int32_t* seq_lens, int B,
                        int Sq, int k, int32_t* idx, bool need_idx, void* ws, size_t ws_bytes, TopkArgs& a,
                        bool& wave_chunks) {
  DSA_CHECK_ARG(scores && seq_lens && (idx || !need_idx), "%s: null pointer", who);
  DSA_CHECK_ARG(score_stride >= 1 && score_stride < ((int64_t)1 << 31), "%s: bad score_stride", who);
  DSA_CHECK_SUPPORTED(k <= 8192, "%s: k > 8192", who);
  DSA_CHECK_ARG((int64_t)B * Sq <= 65535, "%s: more than 65535 rows", who);
  DSA_CHECK_SUPPORTED(score_stride <= (int64_t)kMaxChunks * kChunk, "%s: score_stride above %d", who,
                      kMaxChunks * kChunk);
  a = TopkArgs{};
  a.scores = scores;
  a.stride = score_stride;
  a.seq_lens = seq_lens;
  a.Sq = Sq;
  a.k = k;
  const int wave_slack = topk_wave_slack(score_stride, k);
  wave_chunks = wave_slack >= 0;
  const int64_t grid8 = (int64_t)B * Sq * ((score_stride + kChunk - 1) / kChunk);
  const bool long_chunks = !wave_chunks && grid8 > kChunkRound;
  a.chunk = wave_chunks ? kWaveChunk : (long_chunks ? kTopkThreads * kLongPer : kChunk);
  a.slack = wave_chunks ? wave_slack : 0;
  topk_geometry(score_stride, k, a.chunk, a.slack, a.max_chunks, a.cand_stride);
  const size_t need = dsa_topk_workspace_size(B, Sq, k, score_stride);
  if (ws == nullptr || ws_bytes < need) {
    set_last_error("%s: workspace %zu < %zu bytes", who, ws_bytes, need);
    return DSA_ERR_WORKSPACE;
  }
  DSA_CHECK_ARG(((uintptr_t)ws & 7) == 0, "%s: workspace not 8-byte aligned", who);
  const size_t rows = (size_t)B * Sq;
  a.cand = static_cast<uint2*>(ws);
  a.xc = reinterpret_cast<uint32_t*>(a.cand + rows * a.cand_stride);
  a.cc = reinterpret_cast<int32_t*>(a.xc + rows * a.max_chunks);
  a.idx = idx;
  return DSA_OK;
}

dsa_status_t topk_launch_select(const TopkArgs& a, int rows, hipStream_t stream) {
  static std::atomic<bool> attr_by_dev[kMaxDevices];
  const int slot = current_device_slot();
  if (slot < 0 || !attr_by_dev[slot].load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute((const void*)topk_select_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)(kSelectLds * sizeof(uint32_t)));
    if (e != hipSuccess) {
      set_last_error("top-k select: hipFuncSetAttribute: %s", hipGetErrorString(e));
      return DSA_ERR_HIP;
    }
    if (slot >= 0) attr_by_dev[slot].store(true, std::memory_order_relaxed);
  }
  DSA_LAUNCH(topk_select_kernel, dim3(rows), dim3(kTopkThreads), kSelectLds * sizeof(uint32_t), stream, a);
  return launch_status("top-k select");
}

}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int B, int Sq, int k, int64_t score_stride) {
  if (B <= 0 || Sq <= 0 || k <= 0 || score_stride <= 0) return 0;
  // the wave-chunk geometry when it serves the rows, else the 8192-position one (the
  // 16384-position one needs no more: half the chunk slots, no more candidate slots)
  int max_chunks, cand_stride;
  const int slack = dsa::topk_wave_slack(score_stride, k);
  if (slack >= 0)
    dsa::topk_geometry(score_stride, k, dsa::kWaveChunk, slack, max_chunks, cand_stride);
  else
    dsa::topk_geometry(score_stride, k, dsa::kChunk, 0, max_chunks, cand_stride);
  return (size_t)B * Sq * ((size_t)cand_stride * sizeof(uint2) + (size_t)max_chunks * 2 * sizeof(uint32_t));
}

extern "C" dsa_status_t dsa_topk(const float* scores, int64_t score_stride, const int32_t* seq_lens, int B, int Sq,
                                 int k, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && k >= 1, "dsa_topk: bad sizes");
  if (B == 0) return DSA_OK;
  TopkArgs a;
  bool wave_chunks = false;
  if (dsa_status_t st = topk_setup("dsa_topk", scores, score_stride, seq_lens, B, Sq, k, idx, true, ws, ws_bytes, a,
                                   wave_chunks);
      st != DSA_OK)
    return st;
  if (wave_chunks) {
    const int groups = (a.max_chunks + kWaveThreads / 64 - 1) / (kWaveThreads / 64);
    DSA_LAUNCH(topk_wave_kernel, dim3((unsigned)(groups * B * Sq)), dim3(kWaveThreads), 0, stream, a, groups,
               B * Sq);
  } else if (a.chunk == kTopkThreads * kLongPer) {
    DSA_LAUNCH(topk_chunk_kernel<kLongPer>, dim3(a.max_chunks, B * Sq), dim3(kTopkThreads), 0, stream, a);
  } else {
    DSA_LAUNCH(topk_chunk_kernel<kPer>, dim3(a.max_chunks, B * Sq), dim3(kTopkThreads), 0, stream, a);
  }
  dsa_status_t st = launch_status("dsa_topk(chunk)");
  if (st != DSA_OK) return st;
  return topk_launch_select(a, B * Sq, stream);
}

extern "C" dsa_status_t dsa_topk_select_chunks(const float* scores, int64_t score_stride, const int32_t* seq_lens,
                                               int B, int k, int32_t* idx, void* ws, size_t ws_bytes,
                                               hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && k >= 1, "dsa_topk_select_chunks: bad sizes");
  if (B == 0) return DSA_OK;
  TopkArgs a;
  bool wave_chunks = false;
  if (dsa_status_t st = topk_setup("dsa_topk_select_chunks", scores, score_stride, seq_lens, B, 1, k, idx, true, ws,
                                   ws_bytes, a, wave_chunks);
      st != DSA_OK)
    return st;
  DSA_CHECK_SUPPORTED(wave_chunks, "dsa_topk_select_chunks: rows of %lld positions with k = %d do not take wave "
                      "chunks", (long long)score_stride, k);
  return topk_launch_select(a, B, stream);
}
