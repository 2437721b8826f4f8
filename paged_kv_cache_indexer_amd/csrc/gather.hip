// Per-layer serve and install ("Shared-Indexer KV Cache Offload for GLM-5.2", §2.1:
// selected rows are scattered over the full cache and must be gathered; §4.4 and §5:
// "DsaServe" prepares them from the device pool on a hit and the host cache on a miss,
// "DsaInstall" backfills the surviving misses into their pool slots off the critical
// path).
//
// Rows are copied in 16-byte chunks; consecutive lanes take consecutive chunks of one
// row, so every row read (device HBM or mapped pinned host memory over the host link)
// and every row write is a contiguous run.
#include "common.h"

namespace dsa {

struct GatherArgs {
  const int32_t* topk;      // [B, Sq, k]
  const uint8_t* is_hit;    // [B, Sq, k] or null
  const int32_t* slot;      // [B, Sq, k] or null
  int Sq, k;
  RowStore src;
  char* pool;               // [B, pool_rows, row_bytes]
  int64_t pool_rows;
  int row_bytes;
  char* sel;                // [B, Sq, k, row_bytes]
  int32_t* sel_idx;         // [B, Sq, k] or null (SERVE: t * k + j where a row was served, else -1)
  int32_t* err;
};

// SERVE: grid-stride over (entry, chunk)
__global__ void __launch_bounds__(256) serve_kernel(GatherArgs a, int64_t n_entries) {
  const int cpr = a.row_bytes >> 4;
  const int64_t total = n_entries * cpr;
  const int E = a.Sq * a.k;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < total;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = it / cpr;
    const int c = (int)(it - e * cpr);
    const int b = (int)(e / E);
    const int32_t p = a.topk[e];
    u32x4 v = {0, 0, 0, 0};
    bool served = false;
    if (p >= 0) {
      const char* rowp = nullptr;
      if (a.is_hit && a.is_hit[e]) {
        const int32_t s = a.slot[e];
        if (s >= 0 && s < a.pool_rows) rowp = a.pool + ((int64_t)b * a.pool_rows + s) * a.row_bytes;
      } else {
        const int64_t r = a.src.row(b, p);
        if (r >= 0) rowp = a.src.base + r * a.src.row_bytes;
      }
      if (rowp) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp) + c);
      } else if (c == 0) {
        count_error(a.err);
      }
      served = rowp != nullptr;
    }
    *(reinterpret_cast<u32x4*>(a.sel + e * a.row_bytes) + c) = v;
    if (a.sel_idx && c == 0) a.sel_idx[e] = served ? (int32_t)(e - (int64_t)b * E) : -1;
  }
}

// INSTALL: pool[b, slot] = sel[b, t, j] for surviving misses, first occurrence only
__global__ void __launch_bounds__(256) install_kernel(GatherArgs a, int64_t n_entries) {
  const int cpr = a.row_bytes >> 4;
  const int64_t total = n_entries * cpr;
  const int E = a.Sq * a.k;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < total;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = it / cpr;
    const int c = (int)(it - e * cpr);
    if (a.is_hit[e]) continue;
    const int32_t s = a.slot[e];
    const int32_t p = a.topk[e];
    if (s < 0 || p < 0) continue;
    const int b = (int)(e / E);
    const int within = (int)(e - (int64_t)b * E);
    const int t = within / a.k;
    // an earlier query row holding the same position installs it instead
    bool dup = false;
    for (int t2 = 0; t2 < t && !dup; ++t2) {
      const int32_t* row = a.topk + (int64_t)b * E + (int64_t)t2 * a.k;
      int lo = 0, hi = a.k - 1;
      while (lo < hi) {                          // rows are ascending, -1 padding last
        const int mid = (lo + hi) >> 1;
        const int32_t v = row[mid];
        if (v >= 0 && v < p) lo = mid + 1; else hi = mid;
      }
      dup = (row[lo] == p);
    }
    if (dup) continue;
    if (s >= a.pool_rows) {
      if (c == 0) count_error(a.err);
      continue;
    }
    const u32x4 v = *(reinterpret_cast<const u32x4*>(a.sel + e * a.row_bytes) + c);
    *(reinterpret_cast<u32x4*>(a.pool + ((int64_t)b * a.pool_rows + s) * a.row_bytes) + c) = v;
  }
}

}  // namespace dsa

extern "C" dsa_status_t dsa_gather_kv(const int32_t* topk, const uint8_t* is_hit, const int32_t* slot, int B, int Sq,
                                      int k, const dsa_rows_t* src, void* pool, int64_t pool_rows, int32_t row_bytes,
                                      void* sel, int32_t* sel_idx, int mode, int32_t* err_count,
                                      hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && k >= 1, "dsa_gather_kv: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(row_bytes > 0 && row_bytes % 16 == 0 && row_bytes <= 4096, "dsa_gather_kv: bad row_bytes");
  DSA_CHECK_ARG(topk && sel, "dsa_gather_kv: null pointer");
  DSA_CHECK_ARG(((uintptr_t)sel & 15) == 0, "dsa_gather_kv: sel not 16-byte aligned");
  DSA_CHECK_ARG(((uintptr_t)sel_idx & 3) == 0, "dsa_gather_kv: sel_idx not 4-byte aligned");
  DSA_CHECK_ARG(mode == DSA_GATHER_SERVE || mode == DSA_GATHER_INSTALL, "dsa_gather_kv: bad mode");
  if (is_hit || mode == DSA_GATHER_INSTALL) {
    DSA_CHECK_ARG(is_hit && slot && pool && pool_rows > 0, "dsa_gather_kv: pool mode needs is_hit, slot, pool");
    DSA_CHECK_ARG(((uintptr_t)pool & 15) == 0, "dsa_gather_kv: pool not 16-byte aligned");
  }
  GatherArgs a{};
  a.topk = topk;
  a.is_hit = is_hit;
  a.slot = slot;
  a.Sq = Sq;
  a.k = k;
  a.pool = static_cast<char*>(pool);
  a.pool_rows = pool_rows;
  a.row_bytes = row_bytes;
  a.sel = static_cast<char*>(sel);
  a.sel_idx = mode == DSA_GATHER_SERVE ? sel_idx : nullptr;
  a.err = err_count;
  if (mode == DSA_GATHER_SERVE) {
    DSA_CHECK_ARG(src && src->base, "dsa_gather_kv: null src");
    DSA_CHECK_ARG(src->row_bytes == row_bytes, "dsa_gather_kv: src row_bytes mismatch");
    DSA_CHECK_ARG(((uintptr_t)src->base & 15) == 0, "dsa_gather_kv: src not 16-byte aligned");
    if (src->page_table) DSA_CHECK_ARG(src->page_size > 0, "dsa_gather_kv: bad page_size");
    a.src = RowStore::from(*src);
  }
  const int64_t n = (int64_t)B * Sq * k;
  const int64_t items = n * (row_bytes / 16);
  int64_t blocks = (items + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (mode == DSA_GATHER_SERVE)
    DSA_LAUNCH(serve_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n);
  else
    DSA_LAUNCH(install_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n);
  return launch_status("dsa_gather_kv");
}
