// Lightning-Indexer scan ("Shared-Indexer KV Cache Offload for GLM-5.2", §2.1: the
// indexer scores every history token so that the most relevant ones can be kept).
//
//   score[b,t,s] = sum_h w[b,t,h] * max(0, sigma_s * <q[b,t,h,:], k[b,s,:]>)
//
// Three kernels on one entry point:
//   * indexer_f32_kernel   fp32 q and keys on the VALU (one thread per token).
//   * indexer_mfma_kernel  D = 128 keys streamed from the paged cache, heads on the
//     MFMA M axis and 32 tokens on N, so the ReLU-weighted head sum is an in-lane
//     reduction plus one cross-half add.  bf16 queries use v_mfma_f32_32x32x16_bf16 with
//     the keys widened to bf16 in registers (exact); e4m3 queries use the scaled
//     v_mfma_scale_f32_32x32x64_f8f6f4 directly on the key bytes.
//     Keys are e4m3 (128 B per token, optional per-token fp32 scale) or MXFP4 (64 B of
//     E2M1 codes plus four E8M0 block scales per token: the FP4 indexer cache, read as
//     OCP MXFP4).  MXFP4 keys are widened with v_cvt_scalef32_pk_bf16_fp4, which applies
//     the block scale while converting (exact: every scaled E2M1 value is a bf16), or fed
//     to the scaled MFMA as its fp4 B operand with the E8M0 byte as the B scale.
//
// Key loads: a 32-token tile (4 KB for e4m3, 2 KB for MXFP4; contiguous inside its page)
// is read with 16-byte loads per lane where each instruction covers 1 KB contiguously
// (lane i, load c: bytes 1024c + 16i), the streaming shape that reaches full HBM
// bandwidth.  The tile is then re-laid through a per-wave LDS buffer so that lane
// (n = lane%32, g = lane/32) holds the second half (g = 1) or first half (g = 0) of token
// n's key bytes for the MFMA B operand.  The contraction order over d is the same
// permutation for the A (query) and B (key) operands, so any d -> (lane group, register
// slot) assignment is valid, provided (MXFP4) that each scaled-MFMA lane operand stays
// inside one 32-element block.
#include <type_traits>

#include "topk_wave.h"

namespace dsa {

// ------------------------------------------------------------------------- fp32 VALU
constexpr int kF32MaxQ = 4096;

__global__ void __launch_bounds__(256) indexer_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ w, RowStore keys,
    const float* __restrict__ k_scale, const int32_t* __restrict__ seq_lens, int Sq, int H, int D,
    int64_t score_stride, float* __restrict__ scores, int32_t* err) {
  __shared__ float qs[kF32MaxQ];
  __shared__ float ws[256];
  const int b = blockIdx.y;
  const int L = seq_lens[b];
  const int n_q = Sq * H * D;
  for (int i = threadIdx.x; i < n_q; i += blockDim.x) qs[i] = q[(int64_t)b * n_q + i];
  for (int i = threadIdx.x; i < Sq * H; i += blockDim.x) ws[i] = w[(int64_t)b * Sq * H + i];
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= L || s >= score_stride) return;        // a length past the row is clamped to it
  const int64_t r = keys.row(b, s);
  float* out = scores + (int64_t)b * Sq * score_stride + s;
  if (r < 0) {
    count_error(err);
    for (int t = 0; t < Sq; ++t) out[(int64_t)t * score_stride] = -INFINITY;
    return;
  }
  const float* k = reinterpret_cast<const float*>(keys.base + r * keys.row_bytes);
  const float sig = k_scale ? k_scale[r] : 1.0f;
  for (int t = 0; t < Sq; ++t) {
    const int vis = L - Sq + 1 + t;
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) {
      const float* qh = qs + (t * H + h) * D;
      float dot = 0.0f;
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(k + d);
        dot = fmaf(qh[d], kv.x, dot);
        dot = fmaf(qh[d + 1], kv.y, dot);
        dot = fmaf(qh[d + 2], kv.z, dot);
        dot = fmaf(qh[d + 3], kv.w, dot);
      }
      const float v = dot * sig;
      acc = fmaf(ws[t * H + h], v > 0.0f ? v : 0.0f, acc);
    }
    out[(int64_t)t * score_stride] = (s < vis) ? acc : -INFINITY;
  }
}

// ------------------------------------------------------------------------- MFMA scan
constexpr int kTile = 32;      // tokens per wave tile (MFMA N)
constexpr int kMaxB = 1024;    // requests per launch on this path

struct MfmaArgs {
  const void* q;               // [B, Sq, H, 128] bf16 or e4m3
  const float* w;              // [B, Sq, H]
  RowStore keys;               // 128-byte e4m3 rows or 64-byte MXFP4 rows
  const void* k_scale;         // e4m3: float per row, or null; MXFP4: 4 E8M0 bytes per row
  const int32_t* seq_lens;     // [B]
  int B, Sq, H;
  int64_t score_stride;
  float* scores;
  int32_t* err;
  // fused top-k chunk stage (FUSE): one query row per request, 1024-position units, each
  // unit's candidates, cut key and count written into the top-k workspace described here
  TopkArgs tk;
};

// HMT: 32-row M tiles per query (H / 32); NQ: queries per wave; RG: waves that share one
// token tile (each covers NQ of the Sq queries).  MT_W = HMT * NQ M tiles per wave.
//
// Work is cut into units of up to `ut` tiles inside one request.  A wave loads the
// request's queries once per unit, then streams the unit's tiles through kSlots fixed
// register slots (kSlots - 1 tiles in flight behind the one being computed).  Every fetch is
// issued unconditionally (past the unit's end it re-reads the last tile, an L2 hit), and
// the unit's page lookups are done once, one tile per lane, so the steady-state loop never
// waits on more than the tile it is about to use.  The unit size is derived on the device from the total
// tile count so that the units fill the grid's wave slots in one round.
constexpr int kPrefixPerThread = (kMaxB + 255) / 256;
// register slots per wave: kSlots - 1 tiles in flight behind the one computed (two slots
// measured 1.5% faster than three; four to eight were no faster)
constexpr int kSlots = 2;
constexpr int kMaxUnit = (64 / kSlots) * kSlots;   // tiles per unit: at most one per lane

// tiles per unit for `total` tiles over `wave_slots` waves: one round, whole passes over the
// register slots, at most one tile per lane
__device__ __forceinline__ int unit_tiles(int total, int wave_slots, int max_unit) {
  int ut = (total + wave_slots - 1) / wave_slots;
  ut = ((ut + kSlots - 1) / kSlots) * kSlots;
  if (ut < kSlots) ut = kSlots;
  if (ut > max_unit) ut = max_unit;
  return ut;
}

// unit_off[b] = first unit of request b (units of ut tiles), unit_off[B] = total; len_sh[b] =
// request b's length clamped to [0, stride] (a longer one is counted once, by work-group 0);
// returns ut
__device__ int indexer_units(const int32_t* seq_lens, int B, int64_t stride, int wave_slots, int max_unit,
                              int fixed_ut, int* unit_off, int* len_sh, int* wsum, int32_t* err) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tiles[kPrefixPerThread];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPrefixPerThread; ++i) {
    const int b = tid * kPrefixPerThread + i;
    int len = (b < B) ? seq_lens[b] : 0;
    if (len > stride) {
      if (blockIdx.x == 0) count_error(err);
      len = (int)stride;
    }
    len = max(len, 0);
    if (b < B) len_sh[b] = len;
    tiles[i] = (len + kTile - 1) / kTile;
    mine += tiles[i];
  }
  auto block_scan = [&](int v, int& total) {     // exclusive scan over the 256 threads
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int s = wsum[w];
      if (w < wave) before += s;
      total += s;
    }
    __syncthreads();
    return before + incl - v;
  };
  int total_tiles = 0;
  block_scan(mine, total_tiles);
  const int ut = fixed_ut > 0 ? fixed_ut : unit_tiles(total_tiles, wave_slots, max_unit);
  int units[kPrefixPerThread];
  int my_units = 0;
#pragma unroll
  for (int i = 0; i < kPrefixPerThread; ++i) {
    units[i] = (tiles[i] + ut - 1) / ut;
    my_units += units[i];
  }
  int total_units = 0;
  int off = block_scan(my_units, total_units);
#pragma unroll
  for (int i = 0; i < kPrefixPerThread; ++i) {
    const int b = tid * kPrefixPerThread + i;
    if (b < B) unit_off[b] = off;
    off += units[i];
  }
  if (tid == 0) unit_off[B] = total_units;
  __syncthreads();
  return ut;
}

// E8M0 code (low 8 bits of c) -> the float 2^(c - 127); code 0 is the subnormal 2^-127
__device__ __forceinline__ float e8m0_to_float(uint32_t c) {
  c &= 0xFFu;
  return __uint_as_float(c ? (c << 23) : 0x00400000u);
}

// 8 E2M1 codes (one dword, element i in nibble i) times a power-of-two scale -> bf16x8
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t v, float scale) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3);
  const u32x4 r = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                   __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(bf16x8, r);
}

// max(x, 0) as a signed-integer max of the bits: a float with the sign bit set (including
// -0.0) is a negative integer and becomes +0.0; one instruction, where fmaxf would first
// quiet its NaN operand
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

typedef __attribute__((address_space(3))) const float lds_f32;

// Top-k wave chunk t_begin / 32 of row b (positions [lo, lo + len) of its n), from the unit's
// scores staged in LDS.  Not inlined: inside the scan its address arithmetic was hoisted
// across the unit loop and spilled under the loop's register pressure.
__device__ __attribute__((noinline)) void fused_chunk_select(lds_f32* sb, int b, int t_begin, int n, uint2* cand,
                                                             uint32_t* xc, int32_t* cc, int cand_stride,
                                                             int max_chunks, int k, int slack) {
  const int lane = threadIdx.x & 63;
  const int c = t_begin / (kWaveChunk / kTile);
  const int lo = t_begin * kTile;
  const int len = min(kWaveChunk, n - lo);
  const int r = chunk_keep(k, len, n, slack);
  const int share = (int)(((int64_t)k * len + n - 1) / n);
  uint2* out = cand + (int64_t)b * cand_stride + (int64_t)c * chunk_keep(k, kWaveChunk, n, slack);
  float v[kWavePer];
#pragma unroll
  for (int q = 0; q < kWavePer; ++q) v[q] = sb[q * 64 + lane];   // positions past len are masked
  uint32_t T;
  const int kept = len == kWaveChunk ? wave_chunk<true>(v, len, r, share, lo, out, T)
                                     : wave_chunk<false>(v, len, r, share, lo, out, T);
  if (lane == 0) {
    xc[(int64_t)b * max_chunks + c] = T;
    cc[(int64_t)b * max_chunks + c] = kept;
  }
}

// FUSE (one query row per request, one query per wave): units are exactly kWaveChunk / 32
// tiles, so unit u of a request is top-k wave chunk u of its row; after writing the unit's
// scores the wave runs the chunk's threshold search on the scores still staged in its LDS
// buffer (topk_wave.h) and writes the chunk's candidates, cut key and count.
template <bool QFP8, bool KFP4, int HMT, int NQ, int RG, bool FUSE>
__global__ void __launch_bounds__(256, 2) indexer_mfma_kernel(MfmaArgs a) {
  static_assert(!FUSE || (NQ == 1 && RG == 1), "the fused top-k stage takes one query per wave");
  constexpr int MT_W = HMT * NQ;
  constexpr int WPU = 4 / RG;                      // units processed side by side per work-group
  constexpr int KSTEPS = QFP8 ? 2 : 8;
  constexpr int kRowBytes = KFP4 ? 64 : 128;       // key bytes per token
  constexpr int kLoads = kRowBytes * kTile / 1024; // 16-byte loads per lane per tile
  constexpr int kHalf = kRowBytes / 2;             // key bytes per lane group after the re-layout
  __shared__ int unit_off[kMaxB + 1];              // prefix of units per request
  __shared__ int len_sh[kMaxB];                    // request lengths, clamped to the score row
  __shared__ __attribute__((aligned(16))) float wsm[4][MT_W * 32];   // per-wave head weights
  constexpr int kStageStride = kRowBytes + 16;                        // key rows, padded
  __shared__ __attribute__((aligned(16))) char kstage[4][kTile * kStageStride];
  // Scores are staged here, kBufTiles tiles per query, and written when the buffer is full or
  // the unit ends (with one query per wave, once per unit).  Stores share the vector-memory
  // counter with loads, so a score store issued inside the tile loop made every later wait
  // for key data also wait for that store's write acknowledgement (measured: 55.8 us with
  // per-tile stores, 49.2 us without stores).
  constexpr int kBufTiles = kMaxUnit / NQ;         // NQ * kBufTiles * 32 scores per wave
  static_assert(kBufTiles % kSlots == 0, "a buffer is whole passes over the register slots");
  __shared__ __attribute__((aligned(16))) float sbuf[4][kMaxUnit * kTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave % RG;
  const int us = wave / RG;
  const int n = lane & 31;                         // token within tile / row within M tile
  const int g = lane >> 5;                         // lane group
  const int ps = a.keys.page_size;
  const int tpp = ps / kTile;                       // tiles per page (ps % 32 == 0 on this path)
  const int tpp_shift = (tpp > 0 && (tpp & (tpp - 1)) == 0) ? __builtin_ctz(tpp) : -1;

  __shared__ int scan_wsum[4];
  static_assert(!FUSE || (kWaveChunk % kTile == 0 && kWaveChunk / kTile <= kMaxUnit / NQ), "a fused unit fits the score buffer");
  const int ut = __builtin_amdgcn_readfirstlane(indexer_units(a.seq_lens, a.B, a.score_stride, gridDim.x * WPU,
                                                              kMaxUnit, FUSE ? kWaveChunk / kTile : 0, unit_off,
                                                              len_sh, scan_wsum, a.err));
  const int total_units = __builtin_amdgcn_readfirstlane(unit_off[a.B]);
  const int row0 = rg * MT_W * 32;                 // first query row (t*H + h) of this wave

  typedef typename std::conditional<QFP8, i32x8, bf16x8>::type qop_t;
  qop_t qa[MT_W][KSTEPS];

  struct Slot {
    u32x4 kb[kLoads];
    uint32_t sig;                                  // e4m3: fp32 scale bits; MXFP4: 4 E8M0 codes
    bool valid;
  };

  for (int u = blockIdx.x * WPU + us; u < total_units; u += gridDim.x * WPU) {
    int b = 0;
    {
      int lo = 0, hi = a.B - 1;                    // last b with unit_off[b] <= u
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (unit_off[mid] <= u) lo = mid; else hi = mid - 1;
      }
      b = __builtin_amdgcn_readfirstlane(lo);
    }
    const int L = __builtin_amdgcn_readfirstlane(len_sh[b]);
    const int n_tiles_b = (L + kTile - 1) / kTile;
    const int t_begin = (u - __builtin_amdgcn_readfirstlane(unit_off[b])) * ut;
    const int t_end = min(t_begin + ut, n_tiles_b);

    // first key row of each tile of the unit, one tile per lane (-1: its page is missing or
    // out of range); a fetch reads its tile's row back with readlane, so no memory wait sits
    // between a tile's LDS re-layout and the refill of its slot
    int64_t my_row = -1;
    {
      const int t = t_begin + lane;
      if (t < t_end) {
        const int s0 = t * kTile;                  // positions fit in 31 bits
        int64_t r0 = -1;
        if (a.keys.page_table) {
          const int lp = tpp_shift >= 0 ? (t >> tpp_shift) : t / tpp;
          if (lp < a.keys.pt_stride) {
            const int32_t pg = a.keys.page_table[(int64_t)b * a.keys.pt_stride + lp];
            if (pg >= 0) r0 = (int64_t)pg * ps + (s0 - lp * ps);
          }
        } else if (a.keys.req_stride <= 0 || s0 < a.keys.req_stride) {
          r0 = (int64_t)b * a.keys.req_stride + s0;
        }
        my_row = (r0 >= 0 && r0 + kTile <= a.keys.num_rows) ? r0 : -1;
      }
    }
    const int row_lo = (int)(uint32_t)my_row, row_hi = (int)(my_row >> 32);
    auto fetch = [&](Slot& sl, int t) {
      t = min(t, t_end - 1);
      const int i = t - t_begin;                   // < kMaxUnit <= 64
      const int64_t r0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane(row_hi, i) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane(row_lo, i));
      sl.valid = r0 >= 0;
      const int64_t r = (sl.valid ? r0 : 0) + n;
      const char* kp = a.keys.base + (sl.valid ? r0 : 0) * kRowBytes + lane * 16;
      // non-temporal loads: every key is read once per step, and plain loads (which allocate
      // in the last-level cache) measured 9% slower when successive calls read different caches
#pragma unroll
      for (int c = 0; c < kLoads; ++c)
        sl.kb[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + c * 1024));
      // always issue the scale load (a dummy in-bounds read when there is no scale), so
      // every fetch adds the same number of outstanding loads; an e4m3 scale is only looked
      // at in the epilogue, so nothing waits for it here (MXFP4 is required to pass one)
      sl.sig = a.k_scale ? static_cast<const uint32_t*>(a.k_scale)[r]
                         : *reinterpret_cast<const uint32_t*>(a.keys.base);
    };

    // queries and weights of request b for this wave's rows
#pragma unroll
    for (int mt = 0; mt < MT_W; ++mt) {
      const int64_t qoff = ((int64_t)b * a.Sq * a.H + row0 + mt * 32 + n) * 128;
      if constexpr (QFP8 && KFP4) {
        // The scaled MFMA takes an 8-bit A lane (row, half g) as K = 16g + [0, 16) and
        // 32 + 16g + [0, 16), but an fp4 B lane (column, half g) as K = 32g + [0, 32).  Step
        // j's key lane (n, g) holds dimensions 64g + 32j + [0, 32), so the query lane (row, g)
        // takes dimensions 32j + 16g + [0, 16) and 64 + 32j + 16g + [0, 16).
        const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qoff + g * 16;
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(qp + j * 32);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(qp + 64 + j * 32);
          qa[mt][j] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
      } else if constexpr (QFP8) {
        const uint8_t* qp = static_cast<const uint8_t*>(a.q) + qoff + g * 64;
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(qp + j * 32);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(qp + j * 32 + 16);
          qa[mt][j] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
      } else {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qoff + g * 64;
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j) qa[mt][j] = *reinterpret_cast<const bf16x8*>(qp + j * 8);
      }
    }
    float wreg[(MT_W * 32 + 63) / 64];
#pragma unroll
    for (int r = 0; r < (MT_W * 32 + 63) / 64; ++r) {
      const int i = lane + 64 * r;
      wreg[r] = (i < MT_W * 32) ? a.w[(int64_t)b * a.Sq * a.H + row0 + i] : 0.0f;
    }
    // tile prefetches go out after the query loads, so the loop below is entered with the
    // same outstanding-load order as its back edge (no full drain at the loop header)
    Slot sl[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; ++k) fetch(sl[k], t_begin + k);
#pragma unroll
    for (int r = 0; r < (MT_W * 32 + 63) / 64; ++r) {
      const int i = lane + 64 * r;
      if (i < MT_W * 32) wsm[wave][i] = wreg[r];
    }

    // compute tile t from slot `cur`; once its bytes are in the LDS re-layout buffer the
    // slot is refilled with tile t_next, so that load is in flight during this tile's MFMAs
    auto compute = [&](Slot& cur, int t, bool live, int t_next) {
      // re-lay the tile: load c of lane i holds token (1024c + 16i) / kRowBytes, bytes
      // (16i) % kRowBytes .. +16
      constexpr int kLanesPerRow = kRowBytes / 16;
      char* st = kstage[wave];
#pragma unroll
      for (int c = 0; c < kLoads; ++c)
        *reinterpret_cast<u32x4*>(st + (c * (64 / kLanesPerRow) + lane / kLanesPerRow) * kStageStride +
                                  (lane % kLanesPerRow) * 16) = cur.kb[c];
      const uint32_t sig = cur.sig;
      const bool valid = cur.valid;
      fetch(cur, t_next);
      u32x4 kb[kLoads];
#pragma unroll
      for (int c = 0; c < kLoads; ++c)
        kb[c] = *reinterpret_cast<const u32x4*>(st + n * kStageStride + g * kHalf + c * 16);
      f32x16 acc[MT_W];
#pragma unroll
      for (int mt = 0; mt < MT_W; ++mt) acc[mt] = f32x16{};
      if constexpr (KFP4) {
        // lane group g holds key dimensions [64g, 64g+64) = blocks 2g and 2g+1; their E8M0
        // codes are bytes 0 and 1 of sg
        const uint32_t sg = sig >> (16 * g);
        if constexpr (QFP8) {
          // step j: this lane's 32 dimensions [64g + 32j, +32) are MFMA K = 32g + [0, 32), key
          // block 2g + j; the MFMA takes the scale of K-block g of column n from lane n + 32g,
          // which is this lane, so its B scale is byte j of sg
          const i32x8 b0 = i32x8{(int)kb[0].x, (int)kb[0].y, (int)kb[0].z, (int)kb[0].w, 0, 0, 0, 0};
          const i32x8 b1 = i32x8{(int)kb[1].x, (int)kb[1].y, (int)kb[1].z, (int)kb[1].w, 0, 0, 0, 0};
#pragma unroll
          for (int mt = 0; mt < MT_W; ++mt) {
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt][0], b0, acc[mt], 0, 4, 0, 127, 0, (int)sg);
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt][1], b1, acc[mt], 0, 4, 0, 127, 1, (int)sg);
          }
        } else {
          // step j: dimensions [64g + 8j, +8), in block 2g + j/4
          const float s0 = e8m0_to_float(sg), s1 = e8m0_to_float(sg >> 8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const u32x4 kc = kb[j >> 2];
            const uint32_t v = (j & 3) == 0 ? kc.x : (j & 3) == 1 ? kc.y : (j & 3) == 2 ? kc.z : kc.w;
            const bf16x8 bop = fp4x8_to_bf16x8(v, j < 4 ? s0 : s1);
#pragma unroll
            for (int mt = 0; mt < MT_W; ++mt)
              acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][j], bop, acc[mt], 0, 0, 0);
          }
        }
      } else if constexpr (QFP8) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 k0 = kb[2 * j], k1 = kb[2 * j + 1];
          const i32x8 bop = i32x8{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                                  (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
#pragma unroll
          for (int mt = 0; mt < MT_W; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mt][j], bop, acc[mt], 0, 0, 0, 127, 0, 127);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4 kc = kb[j >> 1];
          const bf16x8 bop = (j & 1) ? e4m3x8_to_bf16x8(kc.z, kc.w) : e4m3x8_to_bf16x8(kc.x, kc.y);
#pragma unroll
          for (int mt = 0; mt < MT_W; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[mt][j], bop, acc[mt], 0, 0, 0);
        }
      }
      // epilogue: per query, sum over this lane's 16 rows of each M tile, plus the other half
      const int64_t s = (int64_t)t * kTile + n;
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) {
        float part = 0.0f;
#pragma unroll
        for (int hm = 0; hm < HMT; ++hm) {
          const int mt = qq * HMT + hm;
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 wv = *reinterpret_cast<const f32x4*>(&wsm[wave][mt * 32 + i4 * 8 + g * 4]);
            part = fmaf(wv.x, relu(acc[mt][i4 * 4 + 0]), part);
            part = fmaf(wv.y, relu(acc[mt][i4 * 4 + 1]), part);
            part = fmaf(wv.z, relu(acc[mt][i4 * 4 + 2]), part);
            part = fmaf(wv.w, relu(acc[mt][i4 * 4 + 3]), part);
          }
        }
        part += __shfl_xor(part, 32);
        const int tq = rg * NQ + qq;
        const int vis = L - a.Sq + 1 + tq;
        float v = (!KFP4 && a.k_scale) ? part * __uint_as_float(sig) : part;
        if (!valid || s >= vis) v = -INFINITY;
        if (live && g == 0) sbuf[wave][(qq * kBufTiles + (t - t_begin) % kBufTiles) * kTile + n] = v;
      }
      // one error per unresolvable token (the tile's positions below L), as the fp32 path counts
      if (live && !valid && lane == 0 && rg == 0) count_error(a.err, min(kTile, L - t * kTile));
    };

    // write the staged scores of tiles [t_lo, t_hi): positions [t_lo * 32, min(t_hi * 32, L))
    // of each query; t_lo is the first tile of its buffer fill
    auto flush = [&](int t_lo, int t_hi) {
      const int s0 = t_lo * kTile;
      const int ntok = min(t_hi * kTile, L) - s0;
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) {
        const int tq = rg * NQ + qq;
        float* dst = a.scores + ((int64_t)b * a.Sq + tq) * a.score_stride + s0;
        const float* src = &sbuf[wave][qq * kBufTiles * kTile];
        int i0 = 0;
        if (((uintptr_t)dst & 15) == 0) {
          for (int i = lane * 4; i + 4 <= ntok; i += 256)
            *reinterpret_cast<f32x4*>(dst + i) = *reinterpret_cast<const f32x4*>(src + i);
          i0 = ntok & ~3;
        }
        for (int i = i0 + lane; i < ntok; i += 64) dst[i] = src[i];
      }
    };

    // fixed-shape body: no exit between the fetches (tiles past the unit's end are computed
    // from the clamped tile and not stored)
    int t_flushed = t_begin;
    for (int t = t_begin; t < t_end; t += kSlots) {
#pragma unroll
      for (int k = 0; k < kSlots; ++k) compute(sl[k], t + k, k == 0 || t + k < t_end, t + k + kSlots);
      if (t + kSlots - t_flushed == kBufTiles && t + kSlots < t_end) {   // buffer full, unit goes on
        flush(t_flushed, t + kSlots);
        t_flushed = t + kSlots;
      }
    }
    flush(t_flushed, t_end);
    if constexpr (FUSE) {
      // one query row: every position below L is visible
      if (L > a.tk.k)
        fused_chunk_select((const lds_f32*)&sbuf[wave][0], b, t_begin, L, a.tk.cand, a.tk.xc, a.tk.cc,
                           a.tk.cand_stride, a.tk.max_chunks, a.tk.k, a.tk.slack);
    }
  }
}

template <bool QFP8, bool KFP4, int HMT, int NQ, int RG, bool FUSE = false>
static dsa_status_t launch_mfma(const MfmaArgs& a, hipStream_t stream) {
  static std::atomic<int> grid_by_dev[kMaxDevices];
  const int slot = current_device_slot();
  int grid = slot >= 0 ? grid_by_dev[slot].load(std::memory_order_relaxed) : 0;
  if (grid == 0) {
    int cus = 256, per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, slot < 0 ? 0 : slot) != hipSuccess ||
        cus < 1)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, indexer_mfma_kernel<QFP8, KFP4, HMT, NQ, RG, FUSE>, 256,
                                                     0) !=
            hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    grid = cus * per_cu;
    if (slot >= 0) grid_by_dev[slot].store(grid, std::memory_order_relaxed);
  }
  DSA_LAUNCH((indexer_mfma_kernel<QFP8, KFP4, HMT, NQ, RG, FUSE>), dim3(grid), dim3(256), 0, stream, a);
  return launch_status("dsa_indexer_scores");
}

}  // namespace dsa

namespace dsa {
// Argument checks of the MFMA path (every check runs before anything is enqueued); fills the
// launch arguments and the template selectors.
static dsa_status_t mfma_setup(const char* who, const void* q, dsa_dtype_t q_dtype, const float* w,
                               const dsa_rows_t* keys, dsa_dtype_t k_dtype, const void* k_scale,
                               const int32_t* seq_lens, int B, int Sq, int H, int D, int64_t score_stride,
                               float* scores, int32_t* err_count, MfmaArgs& a, bool& f8, bool& fp4, int& HMT) {
  DSA_CHECK_SUPPORTED((k_dtype == DSA_E4M3 || k_dtype == DSA_MXFP4) && (q_dtype == DSA_BF16 || q_dtype == DSA_E4M3),
                      "%s: supported dtypes are (f32,f32) and q bf16/e4m3 with k e4m3/mxfp4", who);
  DSA_CHECK_SUPPORTED(D == 128 && H % 32 == 0 && (int64_t)Sq * H <= 256 && B <= kMaxB,
                      "%s: MFMA path needs D == 128, H %% 32 == 0, Sq*H <= 256, B <= 1024", who);
  fp4 = k_dtype == DSA_MXFP4;
  if (fp4) {
    DSA_CHECK_ARG(keys->row_bytes == 64, "%s: MXFP4 row_bytes != 64", who);
    DSA_CHECK_ARG(k_scale && ((uintptr_t)k_scale & 3) == 0, "%s: MXFP4 keys need 4-byte aligned E8M0 block scales",
                  who);
  } else {
    DSA_CHECK_ARG(keys->row_bytes == 128, "%s: row_bytes != 128", who);
  }
  if (keys->page_table) DSA_CHECK_SUPPORTED(keys->page_size % 32 == 0, "%s: page_size %% 32 != 0", who);
  // the MFMA path reads whole 32-token tiles (an unresolvable tile reads rows 0..31 as a
  // stand-in), so the key rows hold at least one tile, and a dense tile never straddles the
  // end of the rows or the boundary between two requests
  DSA_CHECK_SUPPORTED(keys->num_rows >= kTile, "%s: MFMA path needs num_rows >= 32", who);
  if (!keys->page_table)
    DSA_CHECK_SUPPORTED(keys->num_rows % kTile == 0 && keys->req_stride % kTile == 0,
                        "%s: dense keys on the MFMA path need num_rows and req_stride multiples of 32", who);
  DSA_CHECK_SUPPORTED((int64_t)B * ((score_stride + kTile - 1) / kTile) < ((int64_t)1 << 31),
                      "%s: B * ceil(score_stride / 32) must be below 2^31", who);
  a = MfmaArgs{q, w, RowStore::from(*keys), k_scale, seq_lens, B, Sq, H, score_stride, scores, err_count, TopkArgs{}};
  HMT = H / 32;
  f8 = q_dtype == DSA_E4M3;
  {
    // the (H / 32, Sq) combinations instantiated below
    static const int kInst[][2] = {{1, 1}, {1, 2}, {1, 4}, {1, 8}, {2, 1}, {2, 2}, {2, 4}, {4, 1}, {4, 2}};
    bool known = false;
    for (const auto& c : kInst) known = known || (HMT == c[0] && Sq == c[1]);
    DSA_CHECK_SUPPORTED(known, "%s: unsupported (Sq, H) combination for the MFMA path", who);
  }
  return DSA_OK;
}

// the stream joins the load stream only once every argument check has passed, so a rejected
// call enqueues nothing
static dsa_status_t join_ready(const char* who, hipEvent_t ready, hipStream_t stream) {
  if (!ready) return DSA_OK;
  const hipError_t e = hipStreamWaitEvent(stream, ready, 0);
  if (e != hipSuccess) {
    set_last_error("%s: hipStreamWaitEvent: %s", who, hipGetErrorString(e));
    return DSA_ERR_HIP;
  }
  return DSA_OK;
}
}  // namespace dsa

extern "C" dsa_status_t dsa_indexer_scores(const void* q, dsa_dtype_t q_dtype, const float* w,
                                           const dsa_rows_t* keys, dsa_dtype_t k_dtype, const void* k_scale,
                                           const int32_t* seq_lens, int B, int Sq, int H, int D,
                                           int64_t score_stride, float* scores, int32_t* err_count,
                                           hipEvent_t ready, hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && H >= 1 && D >= 1, "dsa_indexer_scores: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(q && w && keys && keys->base && seq_lens && scores, "dsa_indexer_scores: null pointer");
  DSA_CHECK_ARG(score_stride >= 1, "dsa_indexer_scores: score_stride < 1");
  DSA_CHECK_ARG(keys->num_rows >= 1, "dsa_indexer_scores: num_rows < 1");
  DSA_CHECK_ARG(((uintptr_t)keys->base & 15) == 0, "dsa_indexer_scores: keys not 16-byte aligned");
  if (keys->page_table) DSA_CHECK_ARG(keys->page_size > 0 && keys->pt_stride >= 0, "dsa_indexer_scores: bad paging");
  if (q_dtype == DSA_F32 && k_dtype == DSA_F32) {
    DSA_CHECK_SUPPORTED((int64_t)Sq * H * D <= kF32MaxQ && (int64_t)Sq * H <= 256 && D % 4 == 0,
                        "dsa_indexer_scores: fp32 path needs Sq*H*D <= 4096, Sq*H <= 256, D %% 4 == 0");
    DSA_CHECK_ARG(keys->row_bytes == D * 4, "dsa_indexer_scores: row_bytes != D*4");
    DSA_CHECK_ARG(score_stride <= (int64_t)65535 * 256, "dsa_indexer_scores: score_stride too large");
    DSA_CHECK_SUPPORTED(B <= 65535, "dsa_indexer_scores: fp32 path takes at most 65535 requests (grid y)");
    const int64_t gx = (score_stride + 255) / 256;
    if (dsa_status_t st = join_ready("dsa_indexer_scores", ready, stream); st != DSA_OK) return st;
    DSA_LAUNCH(indexer_f32_kernel, dim3((unsigned)gx, (unsigned)B), dim3(256), 0, stream,
                       static_cast<const float*>(q), w, RowStore::from(*keys), static_cast<const float*>(k_scale),
                       seq_lens, Sq, H, D, score_stride, scores, err_count);
    return launch_status("dsa_indexer_scores");
  }
  MfmaArgs a;
  bool f8 = false, fp4 = false;
  int HMT = 0;
  if (dsa_status_t st = mfma_setup("dsa_indexer_scores", q, q_dtype, w, keys, k_dtype, k_scale, seq_lens, B, Sq, H,
                                   D, score_stride, scores, err_count, a, f8, fp4, HMT);
      st != DSA_OK)
    return st;
  if (dsa_status_t st = join_ready("dsa_indexer_scores", ready, stream); st != DSA_OK) return st;
  // one wave covers up to 4 M tiles; queries beyond that go to a second wave on the same tile
#define DSA_CASE(HM, NQ_, RG_)                                                                  \
  if (HMT == HM && Sq == NQ_ * RG_) {                                                            \
    if (fp4)                                                                                     \
      return f8 ? launch_mfma<true, true, HM, NQ_, RG_>(a, stream)                               \
                : launch_mfma<false, true, HM, NQ_, RG_>(a, stream);                             \
    return f8 ? launch_mfma<true, false, HM, NQ_, RG_>(a, stream)                                \
              : launch_mfma<false, false, HM, NQ_, RG_>(a, stream);                              \
  }
  DSA_CASE(1, 1, 1) DSA_CASE(1, 2, 1) DSA_CASE(1, 4, 1) DSA_CASE(1, 4, 2)
  DSA_CASE(2, 1, 1) DSA_CASE(2, 2, 1) DSA_CASE(2, 2, 2)
  DSA_CASE(4, 1, 1) DSA_CASE(4, 1, 2)
#undef DSA_CASE
  set_last_error("dsa_indexer_scores: unsupported (Sq, H) combination for the MFMA path");
  return DSA_ERR_UNSUPPORTED;
}

extern "C" dsa_status_t dsa_indexer_topk_chunks(const void* q, dsa_dtype_t q_dtype, const float* w,
                                                const dsa_rows_t* keys, dsa_dtype_t k_dtype, const void* k_scale,
                                                const int32_t* seq_lens, int B, int H, int D, int64_t score_stride,
                                                float* scores, int k, void* ws, size_t ws_bytes, int32_t* err_count,
                                                hipEvent_t ready, hipStream_t stream) {
  using namespace dsa;
  const char* who = "dsa_indexer_topk_chunks";
  DSA_CHECK_ARG(B >= 0 && H >= 1 && D >= 1 && k >= 1, "%s: bad sizes", who);
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(q && w && keys && keys->base && seq_lens && scores, "%s: null pointer", who);
  DSA_CHECK_ARG(score_stride >= 1, "%s: score_stride < 1", who);
  DSA_CHECK_ARG(keys->num_rows >= 1, "%s: num_rows < 1", who);
  DSA_CHECK_ARG(((uintptr_t)keys->base & 15) == 0, "%s: keys not 16-byte aligned", who);
  if (keys->page_table) DSA_CHECK_ARG(keys->page_size > 0 && keys->pt_stride >= 0, "%s: bad paging", who);
  MfmaArgs a;
  bool f8 = false, fp4 = false;
  int HMT = 0;
  if (dsa_status_t st = mfma_setup(who, q, q_dtype, w, keys, k_dtype, k_scale, seq_lens, B, 1, H, D, score_stride,
                                   scores, err_count, a, f8, fp4, HMT);
      st != DSA_OK)
    return st;
  bool wave_chunks = false;
  if (dsa_status_t st = topk_setup(who, scores, score_stride, seq_lens, B, 1, k, nullptr, false, ws, ws_bytes, a.tk,
                                   wave_chunks);
      st != DSA_OK)
    return st;
  DSA_CHECK_SUPPORTED(wave_chunks, "%s: rows of %lld positions with k = %d do not take wave chunks", who,
                      (long long)score_stride, k);
  if (dsa_status_t st = join_ready(who, ready, stream); st != DSA_OK) return st;
#define DSA_CASE(HM)                                                                             \
  if (HMT == HM) {                                                                               \
    if (fp4)                                                                                     \
      return f8 ? launch_mfma<true, true, HM, 1, 1, true>(a, stream)                             \
                : launch_mfma<false, true, HM, 1, 1, true>(a, stream);                           \
    return f8 ? launch_mfma<true, false, HM, 1, 1, true>(a, stream)                              \
              : launch_mfma<false, false, HM, 1, 1, true>(a, stream);                            \
  }
  DSA_CASE(1) DSA_CASE(2) DSA_CASE(4)
#undef DSA_CASE
  set_last_error("%s: unsupported head count for the MFMA path", who);
  return DSA_ERR_UNSUPPORTED;
}
