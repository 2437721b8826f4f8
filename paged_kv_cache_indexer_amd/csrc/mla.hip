// Sparse MLA decode over the selected rows (TokenSpeed audit page, "MLA
// (tokenspeed-mla)": one 576-wide latent row per token is both key (all 576 values)
// and value (the first 512); "Shared-Indexer KV Cache Offload for GLM-5.2", §2.1:
// attention reads only the top-k positions).  Split-KV decode with fp32 partial
// (o, lse) and an LSE-rescaling merge (TokenSpeed audit, two-stage split-KV decode).
//
// Work-group = 2*HG waves (one per SIMD) for 32*HG heads of one query row and one split
// of its selected rows.  Wave (hg, half) owns heads [32hg, 32hg+32) and computes
//   S^T[32 tokens x 32 heads] partial = K_tile[:, half] . q^T[half]   (bf16 MFMA 32x32x16,
//     18 steps over its 288 of the 576 latent dims, q^T resident in VGPRs); the two
//     halves of a head group swap partial S^T through LDS and both hold the full sum;
//   O^T[256 dims x 32 heads] += V^T[half] . P^T                        (bf16 MFMA 32x32x16)
//     over its 256 of the 512 value dims.  Heads sit on the N axis, so each lane owns one
//     head's running max / sum and the rescale is a per-lane scalar; P^T is the S^T
//     accumulator itself (rounded to bf16).  The V^T operand is read straight from the
//     token-major K tile with LDS transpose reads (ds_read_b64_tr_b16: within each 16-lane
//     group, lane i receives element i%4 of the 8-byte rows addressed by lanes i/4, 4+i/4,
//     8+i/4, 12+i/4), so no transposed copy is made.
// Selected rows stream into a ring of three LDS tiles with LDS-direct loads
// (global_load_lds_dwordx4: lane i of a wave instruction lands at M0 + 16 i), two tiles
// ahead of the one being computed; no VGPRs hold rows in flight.  A tile is stored as
// 1 KB blocks of 8 tokens x 128 bytes (block = chunk group cg * 4 + token group), so one
// wave instruction fetches eight whole 128-byte lines and each lane streams one row.
// Inside a block, 16-byte chunk c of token m sits at position m*8 + ((c%8) ^ swz(m)),
// which keeps both the K reads (one chunk of 32 tokens) and the transpose reads (two
// chunks of 4 tokens) free of LDS bank conflicts.
// Online softmax in base 2 with a lazy rescale (the running max is only moved when it
// grows by more than 2^8), which leaves o and lse mathematically unchanged.
#include "common.h"

namespace dsa {

constexpr int kRowEl = 576;                 // latent 512 + rope 64
constexpr int kVDim = 512;
constexpr int kRowBytes = kRowEl * 2;
constexpr int kTT = 32;                     // tokens per tile
constexpr int kChunks = kRowBytes / 16;     // 72 x 16 B per row
constexpr int kTileSlots = kTT * kChunks;   // 2304 chunk slots per tile
constexpr int kTileBytes = kTileSlots * 16; // 36864
constexpr int kRing = 3;                    // LDS tiles: one computed, two in flight
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;
constexpr int kMaxSplit = 1024;             // selected rows per split (row offsets kept in LDS)

struct MlaArgs {
  const uint16_t* q;       // [QR, H, 576] bf16
  const int32_t* idx;      // [QR, k]
  RowStore rows;
  int Sq, H, k;
  int splits, per_split;   // per_split: entries per split (multiple of 32)
  float scale_log2;
  void* o;                 // [QR, H, 512] (o_f32 ? float : bf16)   -- splits == 1
  int o_f32;
  float* lse;              // [QR, H]                                 -- splits == 1
  void* part_o;            // [QR, splits, H, 512] in o's dtype, normalised   -- splits > 1
  float* part_lse;         // [QR, splits, H]
  int32_t* err;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// chunk swizzle of token m (mod 8) inside a 1 KB block
__device__ __forceinline__ int chunk_swz(int m) { return ((m << 1) & 6) | ((m >> 2) & 1); }

// byte offset of 16-byte chunk c of token n inside a tile
__device__ __forceinline__ int chunk_byte(int n, int c) {
  return ((((c >> 3) << 2) + (n >> 3)) * 64 + (n & 7) * 8 + ((c & 7) ^ chunk_swz(n & 7))) * 16;
}

// 16 bytes from global memory into LDS at M0 + 16 * lane (M0 = lds_addr, wave-uniform).  No
// instruction offset is used: it would move the LDS destination as well.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr) : "m0");
}

// LDS-direct loads R..CPT-1 of one tile: load r fetches chunk group r / NSRC of the row in
// src[r % NSRC] into 1 KB block r * NW of the wave's stripe
template <int R, int CPT, int NSRC, int NW>
__device__ __forceinline__ void dma_tile(const char* const* src, uint32_t dst) {
  if constexpr (R < CPT) {
    lds_dma16(src[R % NSRC] + (R / NSRC) * 128, dst + R * NW * 1024);
    dma_tile<R + 1, CPT, NSRC, NW>(src, dst);
  }
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ u32x2 lds_read_tr16(const lds_u8* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// grid position -> (unit = query row x split, head block).  The head blocks of one unit
// read the same rows; they are placed on one XCD (work-groups go round-robin over the 8
// XCDs) so that the second reader finds the rows in that XCD's L2.
__device__ __forceinline__ void mla_block_unit(int nhb, int& unit, int& hb) {
  const int x = blockIdx.x, G = gridDim.x;
  if (G % (8 * nhb) == 0) {
    const int xcd = x & 7, kk = x >> 3;
    hb = kk % nhb;
    unit = (kk / nhb) * 8 + xcd;
  } else {
    hb = x % nhb;
    unit = x / nhb;
  }
}

template <int HG>
__global__ void __launch_bounds__(128 * HG, 1) mla_decode_kernel(MlaArgs a) {
  constexpr int NW = 2 * HG;
  constexpr int NT = 64 * NW;
  constexpr int CPT = kTileSlots / NT;      // LDS-direct loads per thread per tile
  static_assert(kTileSlots % NT == 0, "tile must split evenly over the threads");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][kTileBytes];
  __shared__ f32x4 xch[NW][4][64];          // partial S^T exchange between the halves
  __shared__ int64_t rowoff[kMaxSplit];     // byte offset of each selected row of the split, -1 = none
  __shared__ uint32_t tmask[kMaxSplit / kTT];  // valid-row bits per tile

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave >> 1, half = wave & 1;
  const int n = lane & 31, g = lane >> 5;
  const int nhb = (a.H + 32 * HG - 1) / (32 * HG);
  int unit, hb;
  mla_block_unit(nhb, unit, hb);
  const int qr = unit / a.splits;
  const int split = unit - qr * a.splits;
  const int b = qr / a.Sq;
  const int head = hb * 32 * HG + hg * 32 + n;
  const bool head_ok = head < a.H;

  const int e_begin = split * a.per_split;
  const int e_end = min(e_begin + a.per_split, a.k);
  const int ntiles = (e_end - e_begin + kTT - 1) / kTT;
  const int32_t* idx = a.idx + (int64_t)qr * a.k;
  // rows that are padding or unresolvable are loaded from this query row instead (finite
  // values; their probabilities are exactly zero)
  const char* stand_in = reinterpret_cast<const char*>(a.q + (int64_t)qr * a.H * kRowEl);

  // ---- q^T operand: 18 k-steps of 16 over this wave's 288 latent dims
  bf16x8 qb[18];
  {
    const uint16_t* qp = a.q + ((int64_t)qr * a.H + (head_ok ? head : 0)) * kRowEl + half * 288 + g * 8;
#pragma unroll
    for (int j = 0; j < 18; ++j) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + j * 16);
      if (!head_ok) v = bf16x8{};
      qb[j] = v;
    }
  }

  // ---- resolve every selected row of this split once: index -> page table -> byte offset
  for (int e = tid; e < ntiles * kTT; e += NT) {
    int64_t off = -1;
    if (e_begin + e < e_end) {
      const int32_t p = idx[e_begin + e];
      const int64_t row = a.rows.row(b, p);
      if (row < 0 && p >= 0) count_error(a.err);
      if (row >= 0) off = row * kRowBytes;
    }
    rowoff[e] = off;
    const uint64_t m = __builtin_amdgcn_ballot_w64(off >= 0);
    if (lane == 0) {            // e is a multiple of 64 here: lanes 0-31 and 32-63 are two tiles
      tmask[e >> 5] = (uint32_t)m;
      if ((e >> 5) + 1 < ntiles) tmask[(e >> 5) + 1] = (uint32_t)(m >> 32);
    }
  }

  // ---- per-lane constants of the three access patterns
  constexpr int NSRC = 4 / NW;  // token groups one lane streams per tile
  // LDS-direct load r of this lane: token group (wave + NW * (r % NSRC)), chunk group
  // r / NSRC; the lane fetches chunk ((lane & 7) ^ swz) of token 8 * group + lane / 8
  const int dlane = ((lane & 7) ^ chunk_swz(lane >> 3)) * 16;
  int qoff[4];                  // K operand of k-step j: qoff[j % 4] + 4096 (j / 4)
#pragma unroll
  for (int j = 0; j < 4; ++j) qoff[j] = chunk_byte(n, half * 36 + 2 * j + g);
  int voff[2];                  // V^T operand (transpose read) of m-tile mt: voff[mt % 2] + 4096 (mt / 2)
  {
    const int blk = lane >> 4, s16 = lane & 15, jj = s16 >> 2, qq = s16 & 3;
    const int tok = (blk >> 1) * 4 + jj;
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
      voff[mp] = chunk_byte(tok, half * 32 + mp * 4 + (blk & 1) * 2 + (qq >> 1)) + (qq & 1) * 8;
  }
  wait_vmcnt<0>();              // q^T is resident before any row load is in flight
  __syncthreads();              // rowoff / tmask ready

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&ring[0][0];
  const char* nsrc[NSRC];       // rows of the next tile to issue
  auto prepare = [&](int t) {
#pragma unroll
    for (int p = 0; p < NSRC; ++p) {
      const int64_t off = rowoff[t * kTT + (wave + NW * p) * 8 + (lane >> 3)];
      nsrc[p] = (off >= 0 ? a.rows.base + off : stand_in) + dlane;
    }
  };
  auto issue = [&](int t) {
    const uint32_t dst = ring_lds + (uint32_t)((t % kRing) * kTileBytes + wave * 1024);
    dma_tile<0, CPT, NSRC, NW>(nsrc, dst);
  };

  prepare(0);
  issue(0);
  if (ntiles > 1) {
    prepare(1);
    issue(1);
  }
  if (ntiles > 2) prepare(2);

  f32x16 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x16{};
  float m_used = -INFINITY;     // log2-domain running max used for p
  float l_part = 0.0f;          // this lane's share of sum p (fp32 p: for lse)
  float lr_part = 0.0f;         // this lane's share of sum bf16(p) (the PV weights: for o)

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles)
      wait_vmcnt<CPT>();        // this wave's loads of tile t are done (tile t+1 may be in flight)
    else
      wait_vmcnt<0>();
    __syncthreads();            // tile t complete for all waves; slot (t+2)%3 and xch free
    if (t + 2 < ntiles) {
      issue(t + 2);
      if (t + 3 < ntiles) prepare(t + 3);
    }
    const lds_u8* tile = (const lds_u8*)(uintptr_t)(ring_lds + (uint32_t)((t % kRing) * kTileBytes));

    // ---- partial S^T over this wave's half of the latent dims; operand reads run ahead
    f32x16 s = f32x16{};
    {
      auto kop = [&](int j) {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(tile + qoff[j & 3] + (j >> 2) * 4096);
      };
      bf16x8 rk[4];
#pragma unroll
      for (int j = 0; j < 3; ++j) rk[j] = kop(j);
#pragma unroll
      for (int j = 0; j < 18; ++j) {
        if (j + 3 < 18) rk[(j + 3) & 3] = kop(j + 3);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rk[j & 3], qb[j], s, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) xch[wave][i4][lane] = f32x4{s[4 * i4], s[4 * i4 + 1], s[4 * i4 + 2], s[4 * i4 + 3]};
    __syncthreads();            // partial S^T of both halves ready
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 o = xch[wave ^ 1][i4][lane];
      s[4 * i4] += o.x;
      s[4 * i4 + 1] += o.y;
      s[4 * i4 + 2] += o.z;
      s[4 * i4 + 3] += o.w;
    }

    // ---- online softmax for head n (tokens of lane group g)
    const uint32_t vmask = __builtin_amdgcn_readfirstlane(tmask[t]);
    if (vmask != 0xffffffffu) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = (i >> 2) * 8 + g * 4 + (i & 3);
        if (!((vmask >> tok) & 1u)) s[i] = -INFINITY;
      }
    }
    float tmax = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, s[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * a.scale_log2;   // scale > 0 keeps the order
    const bool grow = tmax > m_used + kLazy || (m_used == -INFINITY && tmax > -INFINITY);
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? tmax : m_used;
      const float alpha = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) oacc[i] *= alpha;
      l_part *= alpha;
      lr_part *= alpha;
      m_used = m_new;
    }
    const float msub = (m_used == -INFINITY) ? 0.0f : m_used;
    uint32_t pb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], a.scale_log2, -msub));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], a.scale_log2, -msub));
      const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
      pb[i] = w;
      l_part += p0 + p1;
      lr_part += __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
    }
    const bf16x8 p_lo = __builtin_bit_cast(bf16x8, u32x4{pb[0], pb[1], pb[2], pb[3]});
    const bf16x8 p_hi = __builtin_bit_cast(bf16x8, u32x4{pb[4], pb[5], pb[6], pb[7]});

    // ---- O^T += V^T . P^T over this wave's 256 value dims; operand reads run ahead
    {
      auto vop = [&](int i) {   // i = 2*mt + ks: tokens ks*16 + {g*4.., 8 + g*4..}
        const lds_u8* p = tile + voff[(i >> 1) & 1] + (i >> 2) * 4096 + (i & 1) * 2048;   // ks: token groups 2ks, 2ks+1
        const u32x2 lo = lds_read_tr16(p);
        const u32x2 hi = lds_read_tr16(p + 1024);
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      };
      bf16x8 rv[4];
#pragma unroll
      for (int i = 0; i < 3; ++i) rv[i] = vop(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + 3 < 16) rv[(i + 3) & 3] = vop(i + 3);
        oacc[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rv[i & 3], (i & 1) ? p_hi : p_lo, oacc[i >> 1], 0, 0, 0);
      }
    }
  }

  // ---- finish: l over both lane groups, normalise, write this wave's 256 dims
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float lr_tot = lr_part + __shfl_xor(lr_part, 32);
  const float inv = (lr_tot > 0.0f) ? 1.0f / lr_tot : 0.0f;
  const float lse = (l_tot > 0.0f) ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
  if (!head_ok) return;
  const bool direct = a.splits == 1;
  const int64_t obase = (direct ? ((int64_t)qr * a.H + head) : ((((int64_t)qr * a.splits + split) * a.H + head))) *
                            kVDim + half * 256;
  if (!direct) {
    // split partials keep the precision of the final output
    if (a.o_f32) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.part_o) + obase + mt * 32 + i4 * 8 + g * 4) =
              f32x4{oacc[mt][i4 * 4 + 0] * inv, oacc[mt][i4 * 4 + 1] * inv, oacc[mt][i4 * 4 + 2] * inv,
                    oacc[mt][i4 * 4 + 3] * inv};
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.part_o) + obase + mt * 32 + i4 * 8 + g * 4) =
              u32x2{pack_bf16x2(oacc[mt][i4 * 4 + 0] * inv, oacc[mt][i4 * 4 + 1] * inv),
                    pack_bf16x2(oacc[mt][i4 * 4 + 2] * inv, oacc[mt][i4 * 4 + 3] * inv)};
    }
    if (g == 0 && half == 0) a.part_lse[((int64_t)qr * a.splits + split) * a.H + head] = lse;
  } else if (a.o_f32) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + obase + mt * 32 + i4 * 8 + g * 4) =
            f32x4{oacc[mt][i4 * 4 + 0] * inv, oacc[mt][i4 * 4 + 1] * inv, oacc[mt][i4 * 4 + 2] * inv,
                  oacc[mt][i4 * 4 + 3] * inv};
    if (g == 0 && half == 0) a.lse[(int64_t)qr * a.H + head] = lse;
  } else {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + obase + mt * 32 + i4 * 8 + g * 4) =
            u32x2{pack_bf16x2(oacc[mt][i4 * 4 + 0] * inv, oacc[mt][i4 * 4 + 1] * inv),
                  pack_bf16x2(oacc[mt][i4 * 4 + 2] * inv, oacc[mt][i4 * 4 + 3] * inv)};
    if (g == 0 && half == 0) a.lse[(int64_t)qr * a.H + head] = lse;
  }
}

// merge of split partials: 64 threads per (query row, head), 8 value dims per thread
constexpr int kMergeHeads = 4;   // heads per 256-thread work-group

__global__ void __launch_bounds__(64 * kMergeHeads) mla_merge_kernel(MlaArgs a) {
  const int qr = blockIdx.y;
  const int head = blockIdx.x * kMergeHeads + (threadIdx.x >> 6);
  if (head >= a.H) return;
  const int S = a.splits;
  const int d = (threadIdx.x & 63) * 8;
  const float* pl = a.part_lse + (int64_t)qr * S * a.H + head;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, pl[(int64_t)s * a.H]);
  float wsum = 0.0f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (mx > -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float l = pl[(int64_t)s * a.H];
      const float w = (l == -INFINITY) ? 0.0f : __expf(l - mx);
      wsum += w;
      const int64_t pb = (((int64_t)qr * S + s) * a.H + head) * kVDim + d;
      if (a.o_f32) {
        const f32x4 v0 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.part_o) + pb);
        const f32x4 v1 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.part_o) + pb + 4);
        for (int i = 0; i < 4; ++i) {
          acc[i] += w * v0[i];
          acc[4 + i] += w * v1[i];
        }
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.part_o) + pb);
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += w * __uint_as_float(v[i] << 16);
          acc[2 * i + 1] += w * __uint_as_float(v[i] & 0xffff0000u);
        }
      }
    }
    const float inv = 1.0f / wsum;
    for (int i = 0; i < 8; ++i) acc[i] *= inv;
  }
  const int64_t ob = ((int64_t)qr * a.H + head) * kVDim + d;
  if (a.o_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + ob) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + ob + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  } else {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + ob) =
        u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
              pack_bf16x2(acc[6], acc[7])};
  }
  if ((threadIdx.x & 63) == 0) a.lse[(int64_t)qr * a.H + head] = (mx > -INFINITY) ? mx + __logf(wsum) : -INFINITY;
}

static int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  return cus;
}

static void mla_split_plan(int B, int Sq, int H, int k, int& splits, int& per_split) {
  const int wg_heads = (H > 32) ? 64 : 32;
  const int64_t wgs = (int64_t)B * Sq * ((H + wg_heads - 1) / wg_heads);
  const int tiles = (k + kTT - 1) / kTT;
  // one work-group per CU
  int s = (int)((device_cus() + wgs - 1) / wgs);
  if (s < 1) s = 1;
  if (s > tiles) s = tiles;
  const int min_s = (tiles + kMaxSplit / kTT - 1) / (kMaxSplit / kTT);
  if (s < min_s) s = min_s;
  const int tps = (tiles + s - 1) / s;
  per_split = tps * kTT;
  splits = (k + per_split - 1) / per_split;
  if (splits < 1) splits = 1;
}

}  // namespace dsa

extern "C" size_t dsa_sparse_mla_workspace_size(int B, int Sq, int H, int k) {
  if (B <= 0 || Sq <= 0 || H <= 0 || k <= 0) return 0;
  int splits, per;
  dsa::mla_split_plan(B, Sq, H, k, splits, per);
  if (splits <= 1) return 0;
  return (size_t)B * Sq * splits * H * (dsa::kVDim + 1) * sizeof(float);
}

extern "C" dsa_status_t dsa_sparse_mla_decode(const void* q, const int32_t* idx, const dsa_rows_t* rows, int B, int Sq,
                                              int H, int k, float scale, void* o, dsa_dtype_t o_dtype, float* lse,
                                              void* ws, size_t ws_bytes, int32_t* err_count, hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && H >= 1 && k >= 1, "dsa_sparse_mla_decode: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(q && idx && rows && rows->base && o && lse, "dsa_sparse_mla_decode: null pointer");
  DSA_CHECK_ARG(rows->row_bytes == kRowBytes, "dsa_sparse_mla_decode: row_bytes must be 1152");
  DSA_CHECK_ARG(((uintptr_t)rows->base & 15) == 0 && ((uintptr_t)q & 15) == 0,
                "dsa_sparse_mla_decode: rows and q must be 16-byte aligned");
  DSA_CHECK_ARG(o_dtype == DSA_BF16 || o_dtype == DSA_F32, "dsa_sparse_mla_decode: o_dtype must be BF16 or F32");
  DSA_CHECK_ARG(scale > 0.0f && scale < INFINITY, "dsa_sparse_mla_decode: scale must be positive and finite");
  DSA_CHECK_SUPPORTED(H % 16 == 0 && k <= 65536, "dsa_sparse_mla_decode: needs H %% 16 == 0 and k <= 65536");
  if (rows->page_table) DSA_CHECK_ARG(rows->page_size > 0, "dsa_sparse_mla_decode: bad page_size");
  int splits, per;
  mla_split_plan(B, Sq, H, k, splits, per);
  const size_t need = dsa_sparse_mla_workspace_size(B, Sq, H, k);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) {
    set_last_error("dsa_sparse_mla_decode: workspace %zu < %zu bytes", ws_bytes, need);
    return DSA_ERR_WORKSPACE;
  }
  MlaArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.idx = idx;
  a.rows = RowStore::from(*rows);
  a.Sq = Sq;
  a.H = H;
  a.k = k;
  a.splits = splits;
  a.per_split = per;
  a.scale_log2 = scale * kLog2e;
  a.o = o;
  a.o_f32 = (o_dtype == DSA_F32);
  a.lse = lse;
  if (splits > 1) {
    a.part_lse = static_cast<float*>(ws);
    a.part_o = a.part_lse + (size_t)B * Sq * splits * H;
  }
  const int QR = B * Sq;
  if (H > 32) {
    DSA_LAUNCH(mla_decode_kernel<2>, dim3(splits * QR * ((H + 63) / 64)), dim3(256), 0, stream, a);
  } else {
    DSA_LAUNCH(mla_decode_kernel<1>, dim3(splits * QR), dim3(128), 0, stream, a);
  }
  dsa_status_t st = launch_status("dsa_sparse_mla_decode");
  if (st != DSA_OK || splits == 1) return st;
  DSA_LAUNCH(mla_merge_kernel, dim3((H + kMergeHeads - 1) / kMergeHeads, QR), dim3(64 * kMergeHeads), 0,
                     stream, a);
  return launch_status("dsa_sparse_mla_decode(merge)");
}
