// Top-k pieces shared by the top-k kernels and the indexer scan, whose epilogue can run the
// wave-chunk stage of the top-k on the scores it has just staged ("Shared-Indexer KV Cache
// Offload for GLM-5.2", §2.1: the 2048 best positions per query feed sparse attention).
#pragma once

#include "common.h"

namespace dsa {

constexpr int kTopkMaxChunks = 256;                // chunk slots per row
constexpr int kTopkMaxCand = 8192;                 // stage-2 candidates held in registers
constexpr int kWaveChunk = 1024;
constexpr int kWavePer = kWaveChunk / 64;
constexpr int kWaveSlack = 16;                     // candidates kept beyond twice the share
constexpr int kWaveMinSlack = 8;                   // below this, the rows take the work-group chunks
constexpr int kWaveThreads = 256;
constexpr int64_t kWaveMaxStride = (int64_t)kTopkMaxChunks * kWaveChunk;
constexpr int kWaveInterp = 6;                     // regula-falsi probes before bisection

// Wave-wide inclusive scans through DPP lane moves (no LDS round trips): four row
// shifts build each 16-lane row's prefix, then row broadcasts of lanes 15 and 31 carry
// the rows' totals forward.  Lanes with no source lane take the identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROWS, 0xf, false);
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t x, uint32_t identity, Op op) {
  x = op(x, dpp_move<0x111, 0xf>(x, identity));   // row_shr:1
  x = op(x, dpp_move<0x112, 0xf>(x, identity));   // row_shr:2
  x = op(x, dpp_move<0x114, 0xf>(x, identity));   // row_shr:4
  x = op(x, dpp_move<0x118, 0xf>(x, identity));   // row_shr:8
  x = op(x, dpp_move<0x142, 0xa>(x, identity));   // row_bcast:15 into rows 1 and 3
  x = op(x, dpp_move<0x143, 0xc>(x, identity));   // row_bcast:31 into rows 2 and 3
  return x;
}
__device__ __forceinline__ int wave_sum_incl(int x) {
  return (int)wave_scan_incl((uint32_t)x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  x = wave_scan_incl(x, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = wave_scan_incl(x, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// number of set bits of m below this lane, plus acc
__device__ __forceinline__ int lanes_below(uint64_t m, int acc) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)acc));
}

struct TopkArgs {
  const float* scores;
  int64_t stride;
  const int32_t* seq_lens;
  int Sq, k;
  int chunk;          // positions per stage-1 chunk: kWaveChunk, or kTopkThreads * (kPer or kLongPer)
  int slack;          // extra candidates kept per chunk beyond twice its share (wave chunks)
  int max_chunks;     // chunk slots per row
  int cand_stride;    // candidate slots per row (>= the sum of the r_c)
  uint32_t* xc;       // [rows, max_chunks] cut key of each chunk
  int32_t* cc;        // [rows, max_chunks] candidates each chunk kept (at most its r_c slots)
  uint2* cand;        // [rows, cand_stride] (key, position) candidates, position order
  int32_t* idx;
};

// visible positions of the row, clamped to [0, stride]
__device__ __forceinline__ int row_len(const TopkArgs& a, int row) {
  const int b = row / a.Sq, t = row % a.Sq;
  const int64_t n = (int64_t)a.seq_lens[b] - a.Sq + 1 + t;
  return n < 0 ? 0 : (int)(n < a.stride ? n : a.stride);
}

// candidates kept by a chunk of `len` of the row's `n` positions: twice its share
// ceil(k * len / n) of the k plus `slack`, at most len.  The shares add up to at least k.
__device__ __forceinline__ int chunk_keep(int k, int len, int n, int slack) {
  const int share = (int)(((int64_t)k * len + n - 1) / n);
  return min(len, 2 * share + slack);
}

// ---- stage 1 on wave chunks (no work-group barriers, no LDS) ----
//
// Each wave owns one chunk of kWaveChunk positions, kWavePer keys per lane (position
// lo + 64 q + lane in slot q, so slot-major lane order is position order).  Instead of an
// exact select of r_c keys, the wave searches for a threshold T whose count of keys above
// it lies in a window [lo_c, r_c] just below its slot budget, and keeps exactly those keys
// (fewer than r_c candidates are fine: the slots left over hold key 0, which no select
// takes, and stage 2 is exact for any cut key that bounds what was left out).  Each probe
// of the search is one compare per key and a wave sum.  The first probe is the chunk's
// mean plus z standard deviations, z the normal upper-tail quantile of the target
// fraction (Abramowitz and Stegun 26.2.23); later probes are Illinois regula falsi in key
// space, then bisection, on the bracket [kmin - 1, kmax].  When ties leave no threshold
// inside the window the bracket closes on adjacent keys (A, B = A + 1): T = B, and the
// first r_c - count(> B) keys equal to B are taken in position order, as an exact select.

// wave sum of a float through DPP lane moves (the scan's last lane holds the total)
__device__ __forceinline__ float wave_fsum(float x) {
  const uint32_t t = wave_scan_incl(__float_as_uint(x), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)t, 63));
}

// number of the wave's keys above m (empty slots hold key 0, below every probe)
template <int P>
__device__ __forceinline__ int wave_count_above(const uint32_t (&key)[P], uint32_t m) {
  int c = 0;
#pragma unroll
  for (int q = 0; q < P; ++q) c += key[q] > m ? 1 : 0;
  const int incl = wave_sum_incl(c);
  return __builtin_amdgcn_readlane(incl, 63);
}

// upper-tail standard normal quantile: P(Z > z) = p for 0 < p <= 0.5 (Abramowitz and
// Stegun 26.2.23, absolute error below 4.5e-4)
__device__ __forceinline__ float normal_upper_quantile(float p) {
  const float t = __builtin_amdgcn_sqrtf(-2.0f * __logf(p));
  return t - (2.515517f + t * (0.802853f + t * 0.010328f)) *
                 __builtin_amdgcn_rcpf(1.0f + t * (1.432788f + t * (0.189269f + t * 0.001308f)));
}

// the order-preserving key of float_key without its branches: -0.0 folds into +0.0, then
// negative floats are inverted and positive ones get the top bit
__device__ __forceinline__ uint32_t float_key_fast(float f) {
  uint32_t u = __float_as_uint(f);
  u = u == 0x80000000u ? 0u : u;
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// One wave chunk (FULL: all kWaveChunk positions inside the row, no masks).  v: the
// chunk's scores; returns the candidate count, writes the cut key to T.
template <bool FULL>
__device__ __forceinline__ int wave_chunk(const float (&v)[kWavePer], int len, int r, int share, int lo, uint2* out,
                                          uint32_t& T) {
  const int lane = threadIdx.x & 63;
  uint32_t key[kWavePer], kmin = 0xffffffffu, kmax = 0u;
  float xs = 0.0f, xq = 0.0f;
#pragma unroll
  for (int q = 0; q < kWavePer; ++q) {
    const bool in = FULL || q * 64 + lane < len;
    const uint32_t kq = float_key_fast(v[q]);
    key[q] = in ? kq : 0u;
    kmin = min(kmin, in ? kq : 0xffffffffu);
    kmax = max(kmax, key[q]);
    const float x = in ? v[q] : 0.0f;
    xs += x;
    xq = fmaf(x, x, xq);
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  char* const ob = reinterpret_cast<char*>(out);
  const uint32_t p0 = (uint32_t)(lo + lane);
  if (r >= len) {                                 // the whole chunk is kept; X_c = its smallest key
#pragma unroll
    for (int q = 0; q < kWavePer; ++q)
      if (FULL || q * 64 + lane < len)
        *reinterpret_cast<uint2*>(ob + (uint32_t)(q * 64 + lane) * 8u) = make_uint2(key[q], p0 + q * 64);
    T = kmin;
    return len;
  }
  const int lo_c = r - max(2, (r - share) / 4);
  const float tc = 0.5f * (float)(lo_c + r);
  // first probe: mean + z * deviation of the chunk's scores (one pass; a poor guess only
  // costs probes)
  const float inv_len = __builtin_amdgcn_rcpf((float)len);
  const float mean = wave_fsum(xs) * inv_len;
  const float sd = __builtin_amdgcn_sqrtf(fmaxf(wave_fsum(xq) * inv_len - mean * mean, 0.0f));
  const float p_up = tc * inv_len;                // target fraction of the chunk above T
  const float z = p_up <= 0.5f ? normal_upper_quantile(p_up) : -normal_upper_quantile(1.0f - p_up);
  const float g = fmaf(z, sd, mean);
  uint32_t A = kmin - 1u, B = kmax;               // count(> A) = len > r, count(> B) = 0 < lo_c
  int cB = 0;                                     // exact count above B
  float fA = (float)len, fB = 0.0f;               // Illinois-damped counts at the bracket ends
  uint32_t m = (g == g && fabsf(g) <= 3.0e38f) ? float_key_fast(g) : A + (B - A) / 2u;
  int side = 0, probes = 0;
  while (B - A > 1u) {                            // the bracket shrinks at every probe
    m = min(max(m, A + 1u), B - 1u);
    const int cm = wave_count_above(key, m);
    ++probes;
    if (cm > r) {
      A = m;
      fA = (float)cm;
      if (side < 0) fB = 0.5f * (fB + tc);
      side = -1;
    } else if (cm < lo_c) {
      B = m;
      cB = cm;
      fB = (float)cm;
      if (side > 0) fA = 0.5f * (fA + tc);
      side = 1;
    } else {                                      // inside the window: keep the keys above m
      T = m;
      int base = 0;
#pragma unroll
      for (int q = 0; q < kWavePer; ++q) {
        const uint64_t tm = __builtin_amdgcn_ballot_w64(key[q] > m);
        const int slot = lanes_below(tm, base);
        if (key[q] > m) *reinterpret_cast<uint2*>(ob + (uint32_t)slot * 8u) = make_uint2(key[q], p0 + q * 64);
        base += (int)__builtin_popcountll(tm);
      }
      for (int i = cm + lane; i < r; i += 64) *reinterpret_cast<uint2*>(ob + (uint32_t)i * 8u) = make_uint2(0u, 0u);
      return cm;
    }
    if (probes < kWaveInterp && fA > fB) {
      const float f = fminf(fmaxf((fA - tc) * __builtin_amdgcn_rcpf(fA - fB), 0.0f), 1.0f);
      m = A + (uint32_t)((float)(B - A) * f);
    } else {
      m = A + (B - A) / 2u;
    }
  }
  // adjacent bracket (ties across the window): exact select of r at T = B, the first
  // `need` keys equal to B in position order
  T = B;
  const int need = r - cB;
  int base = 0, eq_base = 0;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int q = 0; q < kWavePer; ++q) {
    const bool eq = key[q] == B;                   // never an empty slot: B > 0
    const uint64_t em = __builtin_amdgcn_ballot_w64(eq);
    const bool take = key[q] > B || (eq && eq_base + (int)__builtin_popcountll(em & lt) < need);
    const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
    const int slot = lanes_below(tm, base);
    if (take && slot < r) *reinterpret_cast<uint2*>(ob + (uint32_t)slot * 8u) = make_uint2(key[q], p0 + q * 64);
    base += (int)__builtin_popcountll(tm);
    eq_base += (int)__builtin_popcountll(em);
  }
  return r;
}

// ---- host side (topk.hip)

// Geometry of the candidate workspace: chunk slots per row and candidate slots per row.
void topk_geometry(int64_t stride, int k, int chunk, int slack, int& max_chunks, int& cand_stride);
// Slack of the wave-chunk form for rows of `stride` positions and k, or -1 when the rows
// take the work-group chunks.
int topk_wave_slack(int64_t stride, int k);
// Checks the arguments of a top-k over [B, Sq, stride] scores and fills `a` for the form
// that serves them (wave_chunks: the wave-chunk geometry).  Enqueues nothing.
// need_idx: the call writes indices (a fused scan fills only the candidate workspace).
dsa_status_t topk_setup(const char* who, const float* scores, int64_t stride, const int32_t* seq_lens, int B, int Sq,
                        int k, int32_t* idx, bool need_idx, void* ws, size_t ws_bytes, TopkArgs& a,
                        bool& wave_chunks);
// Stage 2 of a top-k whose candidates are in `a`'s workspace.
dsa_status_t topk_launch_select(const TopkArgs& a, int rows, hipStream_t stream);

}  // namespace dsa
