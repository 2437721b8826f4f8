// Shared-group cache-pool plan ("Shared-Indexer KV Cache Offload for GLM-5.2", §3,
// §4.2-4.3 and §5: "DsaPlan" classifies the shared top-k once per group of layers,
// records per entry whether it is served from the device pool or from the host, emits
// a compact miss list, and picks replacement slots in a set-associative pool whose
// sets are replaced FIFO through one pointer per set that only installs advance).
//
// One 1024-thread work-group per request, all state in LDS:
//   1. U = sorted, de-duplicated valid positions of the Sq top-k rows (already sorted
//      for Sq = 1 and skipped then; bitonic sort otherwise).
//   2. hit iff id_to_slot[u] != -1.
//   3. misses ranked within their set in ascending position order: bitonic sort of
//      (set << 13 | index in U); rank = sorted position - first position of the set.
//   4. way = (ptr[s] + rank) mod W; survives iff rank >= m_s - W.
//   5. outputs per entry and the ascending miss list; optional commit.
#include "common.h"

namespace dsa {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanMaxE = 8192;        // Sq * k
constexpr int kPlanMaxSets = 4096;

struct PlanArgs {
  const int32_t* topk;
  int Sq, k;
  int32_t* pool_ids;
  int32_t* id_to_slot;
  int32_t* ptr;
  int n_sets, ways, id_range;
  uint8_t* is_hit;
  int32_t* slot;
  int32_t* miss_pos;
  int32_t* miss_slot;
  int32_t* miss_count;
  int commit;
  int32_t* err;
};

__device__ __forceinline__ int plan_scan(int v, int* wave_tot, int& total) {
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
    int t = (lane < kPlanWaves) ? wave_tot[lane] : 0;
    int s = t;
#pragma unroll
    for (int o = 1; o < kPlanWaves; o <<= 1) {
      const int y = __shfl_up(s, o);
      if (lane >= o) s += y;
    }
    if (lane < kPlanWaves) wave_tot[kPlanWaves + lane] = s - t;
    if (lane == kPlanWaves - 1) wave_tot[2 * kPlanWaves] = s;
  }
  __syncthreads();
  const int res = wave_tot[kPlanWaves + wave] + x - v;
  total = wave_tot[2 * kPlanWaves];
  __syncthreads();
  return res;
}

// ascending bitonic sort of n (power of two) uint32 keys in LDS
__device__ void bitonic_sort(uint32_t* a, int n) {
  for (int kk = 2; kk <= n; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += kPlanThreads) {
        const int lo = 2 * i - (i & (j - 1));
        const int hi = lo + j;
        const bool up = (lo & kk) == 0;
        const uint32_t x = a[lo], y = a[hi];
        if ((x > y) == up) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(kPlanThreads) plan_kernel(PlanArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem;                                  // [kPlanMaxE]  entries, then sort keys
  uint32_t* upos = keys + kPlanMaxE;                      // [kPlanMaxE]  U
  int32_t* uslot = reinterpret_cast<int32_t*>(upos + kPlanMaxE);   // [kPlanMaxE]
  int32_t* sstart = uslot + kPlanMaxE;                    // [kPlanMaxSets + 1]
  uint8_t* uhit = reinterpret_cast<uint8_t*>(sstart + kPlanMaxSets + 1);  // [kPlanMaxE]
  __shared__ int wave_tot[2 * kPlanWaves + 1];
  __shared__ int flag;

  const int b = blockIdx.x, tid = threadIdx.x;
  const int E = a.Sq * a.k;
  const int W = a.ways, NS = a.n_sets, NSLOT = a.n_sets * a.ways;
  const int32_t* tk = a.topk + (int64_t)b * E;
  int32_t* its = a.id_to_slot + (int64_t)b * a.id_range;
  int32_t* pids = a.pool_ids + (int64_t)b * NSLOT;
  int32_t* ptr = a.ptr + (int64_t)b * NS;

  int Ep = 1;
  while (Ep < E) Ep <<= 1;

  // ---- 1. U
  if (tid == 0) flag = 0;
  __syncthreads();
  for (int i = tid; i < Ep; i += kPlanThreads) {
    uint32_t v = 0xffffffffu;
    if (i < E) {
      const int32_t p = tk[i];
      if (p >= 0) v = (uint32_t)p;
    }
    keys[i] = v;
  }
  __syncthreads();
  if (a.Sq > 1) {
    flag = 1;
  } else {
    for (int i = 1 + tid; i < E; i += kPlanThreads)
      if (keys[i] != 0xffffffffu && keys[i] <= keys[i - 1]) flag = 1;
  }
  __syncthreads();
  if (flag) bitonic_sort(keys, Ep);
  int n_u = 0;
  {
    // ordered compaction of first occurrences; each thread owns a contiguous run
    constexpr int PER = kPlanMaxE / kPlanThreads;
    uint32_t v[PER];
    int cnt = 0;
    const int base = tid * PER;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = base + r;
      uint32_t x = 0xffffffffu;
      if (i < Ep) {
        x = keys[i];
        if (x != 0xffffffffu && i > 0 && keys[i - 1] == x) x = 0xffffffffu;
      }
      v[r] = x;
      cnt += (x != 0xffffffffu);
    }
    const int off = plan_scan(cnt, wave_tot, n_u);
    int o = off;
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (v[r] != 0xffffffffu) upos[o++] = v[r];
  }
  __syncthreads();

  // ---- 2. classify against the pre-step state
  for (int i = tid; i < n_u; i += kPlanThreads) {
    const uint32_t u = upos[i];
    int st = -1;
    uint8_t h = 0;
    if (u >= (uint32_t)a.id_range) {
      st = -2;                                  // invalid id
      count_error(a.err);
    } else {
      const int32_t s = its[u];
      if (s >= 0) {
        if (s < NSLOT) {
          st = s;
          h = 1;
        } else {
          st = -2;
          count_error(a.err);
        }
      }
    }
    uslot[i] = st;
    uhit[i] = h;
  }
  for (int s = tid; s <= NS; s += kPlanThreads) sstart[s] = 0;
  __syncthreads();

  // ---- 3. per-set miss counts, set starts, sort keys (set, U index)
  for (int i = tid; i < n_u; i += kPlanThreads)
    if (uslot[i] == -1) atomicAdd(&sstart[upos[i] % (uint32_t)NS], 1);
  __syncthreads();
  int m = 0;
  {
    constexpr int SPER = (kPlanMaxSets + kPlanThreads - 1) / kPlanThreads;
    int c[SPER];
    int tot = 0;
#pragma unroll
    for (int r = 0; r < SPER; ++r) {
      const int s = tid * SPER + r;
      c[r] = (s < NS) ? sstart[s] : 0;
      tot += c[r];
    }
    int off = plan_scan(tot, wave_tot, m);
#pragma unroll
    for (int r = 0; r < SPER; ++r) {
      const int s = tid * SPER + r;
      if (s < NS) sstart[s] = off;
      off += c[r];
    }
    if (tid == 0) sstart[NS] = m;
  }
  __syncthreads();
  int Mp = 1;
  while (Mp < m) Mp <<= 1;
  {
    // compact miss keys (order irrelevant: the sort orders them)
    constexpr int PER = kPlanMaxE / kPlanThreads;
    uint32_t v[PER];
    int cnt = 0;
    const int base = tid * PER;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = base + r;
      uint32_t x = 0xffffffffu;
      if (i < n_u && uslot[i] == -1) x = ((upos[i] % (uint32_t)NS) << 13) | (uint32_t)i;
      v[r] = x;
      cnt += (x != 0xffffffffu);
    }
    int tot;
    int o = plan_scan(cnt, wave_tot, tot);
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (v[r] != 0xffffffffu) keys[o++] = v[r];
    for (int i = m + tid; i < Mp; i += kPlanThreads) keys[i] = 0xffffffffu;
  }
  __syncthreads();
  if (m > 1) bitonic_sort(keys, Mp);

  // ---- 4. FIFO ways and survivors
  for (int p = tid; p < m; p += kPlanThreads) {
    const uint32_t key = keys[p];
    const int s = (int)(key >> 13), ui = (int)(key & 0x1fffu);
    const int rank = p - sstart[s];
    const int ms = sstart[s + 1] - sstart[s];
    const int p0 = ((ptr[s] % W) + W) % W;
    uslot[ui] = (rank >= ms - W) ? s * W + (p0 + rank) % W : -3;   // -3: miss that does not survive
  }
  __syncthreads();

  // ---- 5. miss list (ascending) and per-entry outputs
  {
    constexpr int PER = kPlanMaxE / kPlanThreads;
    int cnt = 0;
    const int base = tid * PER;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = base + r;
      cnt += (i < n_u && !uhit[i] && uslot[i] != -2);
    }
    int tot;
    int o = plan_scan(cnt, wave_tot, tot);
    int32_t* mp = a.miss_pos + (int64_t)b * E;
    int32_t* ms = a.miss_slot + (int64_t)b * E;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = base + r;
      if (i < n_u && !uhit[i] && uslot[i] != -2) {
        mp[o] = (int32_t)upos[i];
        ms[o] = uslot[i] >= 0 ? uslot[i] : -1;
        ++o;
      }
    }
    if (tid == 0) a.miss_count[b] = tot;
  }
  for (int e = tid; e < E; e += kPlanThreads) {
    const int32_t p = tk[e];
    uint8_t h = 0;
    int32_t sl = -1;
    if (p >= 0) {
      int lo = 0, hi = n_u - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (upos[mid] < (uint32_t)p) lo = mid + 1; else hi = mid;
      }
      if (n_u > 0 && upos[lo] == (uint32_t)p) {
        h = uhit[lo];
        sl = uslot[lo] >= 0 ? uslot[lo] : -1;
      }
    }
    a.is_hit[(int64_t)b * E + e] = h;
    a.slot[(int64_t)b * E + e] = sl;
  }

  // ---- 6. commit
  if (a.commit) {
    __syncthreads();       // every read of id_to_slot / ptr above is done
    for (int i = tid; i < n_u; i += kPlanThreads) {
      if (uhit[i] || uslot[i] < 0) continue;
      const int sl = uslot[i];
      const int32_t old = pids[sl];
      if (old >= 0 && old < a.id_range) its[old] = -1;
    }
    __syncthreads();
    for (int i = tid; i < n_u; i += kPlanThreads) {
      if (uhit[i] || uslot[i] < 0) continue;
      const int sl = uslot[i];
      pids[sl] = (int32_t)upos[i];
      its[upos[i]] = sl;
    }
    for (int s = tid; s < NS; s += kPlanThreads) {
      const int ms = sstart[s + 1] - sstart[s];
      if (ms) ptr[s] = (int)((((ptr[s] % W) + W) % W + ms) % W);
    }
  }
}

static size_t plan_smem() {
  return (size_t)kPlanMaxE * 4 * 3 + (kPlanMaxSets + 1) * 4 + kPlanMaxE;
}

}  // namespace dsa

extern "C" dsa_status_t dsa_plan(const int32_t* topk, int B, int Sq, int k, int32_t* pool_ids, int32_t* id_to_slot,
                                 int32_t* ptr, int n_sets, int ways, int id_range, uint8_t* is_hit, int32_t* slot,
                                 int32_t* miss_pos, int32_t* miss_slot, int32_t* miss_count, int commit,
                                 int32_t* err_count, hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && k >= 1 && n_sets >= 1 && ways >= 1 && id_range >= 1, "dsa_plan: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(topk && pool_ids && id_to_slot && ptr && is_hit && slot && miss_pos && miss_slot && miss_count,
                "dsa_plan: null pointer");
  DSA_CHECK_SUPPORTED((int64_t)Sq * k <= kPlanMaxE && n_sets <= kPlanMaxSets && ways <= 64 &&
                          (int64_t)n_sets * ways <= (1 << 24),
                      "dsa_plan: needs Sq*k <= 8192, n_sets <= 4096, ways <= 64");
  static std::atomic<bool> attr_by_dev[kMaxDevices];
  const int dev_slot = current_device_slot();
  if (dev_slot < 0 || !attr_by_dev[dev_slot].load(std::memory_order_relaxed)) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)plan_smem());
    if (e != hipSuccess) {
      set_last_error("dsa_plan: hipFuncSetAttribute: %s", hipGetErrorString(e));
      return DSA_ERR_HIP;
    }
    if (dev_slot >= 0) attr_by_dev[dev_slot].store(true, std::memory_order_relaxed);
  }
  PlanArgs args{topk, Sq, k, pool_ids, id_to_slot, ptr, n_sets, ways, id_range, is_hit, slot,
                miss_pos, miss_slot, miss_count, commit, err_count};
  DSA_LAUNCH(plan_kernel, dim3((unsigned)B), dim3(kPlanThreads), plan_smem(), stream, args);
  return launch_status("dsa_plan");
}
