// Sparse MLA decode over the selected rows (TokenSpeed audit page, "MLA
// (tokenspeed-mla)": one 576-wide latent row per token is both key (all 576 values)
// and value (the first 512); "Shared-Indexer KV Cache Offload for GLM-5.2", §2.1:
// attention reads only the top-k positions).  Split-KV decode: each split writes its
// normalised partial o (in o's dtype) and its lse, and an LSE-rescaling merge combines
// them (TokenSpeed audit, two-stage split-KV decode).
//
// Two work-group forms share the tile layout, the row loads and the online softmax:
//  * mla_roles_kernel (64 heads per work-group, used whenever H >= 64): eight waves in two
//    roles.  Four score waves each keep q^T of 16 heads in VGPRs and compute
//      S^T[32 tokens x 16 heads] = K_tile . q^T  (bf16 MFMA 16x16x32: two 16-token M tiles x 18
//      steps of 32 latent dims)
//    and the softmax; they hand P^T to four value waves through LDS.  Value wave d keeps O^T
//    for value dims 128d..128d+127 of all 64 heads and computes
//      O^T[128 dims x 64 heads] += V^T . P^T  (bf16 MFMA 16x16x32, K = the tile's 32 tokens),
//    so each V^T operand read serves 64 heads.  Details at the kernel.
//  * mla_decode_kernel<NW, 2> (16 to 48 heads): two token streams of NW waves (one per SIMD
//    per stream) for 16*NW heads; stream s takes tiles T with T % 2 == s, and the streams'
//    softmax states are merged through LDS at the end.  Each wave owns 16 heads over the
//    whole latent row and computes both products itself.
// In both, heads sit on the N axis of S^T: the four lanes of a head (lane % 16) hold its
// running max / sums, and P^T is the S^T accumulator rounded to bf16; lane group g = lane / 16
// holds tokens 4g..4g+3 and 16+4g..16+4g+3, which are also its eight K slots of the PV
// product.  The V^T operand is read straight from the token-major K tile with LDS transpose
// reads (ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4 of the
// 8-byte rows addressed by lanes i/4, 4+i/4, 8+i/4, 12+i/4), so no transposed copy is made.
// Selected rows stream into a ring of four LDS tiles with LDS-direct loads
// (global_load_lds_dwordx4: lane i of a wave instruction lands at M0 + 16 i); no VGPRs hold
// rows in flight.  A tile is stored as 1 KB
// blocks of 8 tokens x 128 bytes (block = chunk group cg * 4 + token group), so one wave
// instruction fetches eight whole 128-byte lines; the placement inside a block
// (chunk_byte) keeps both operand reads free of LDS bank conflicts.
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
constexpr int kTileBytes = 36 * 1024;       // 36 blocks of 8 tokens x 128 bytes
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;
constexpr int kMaxSplit = 1152;             // selected rows of one work-group piece (row table in LDS)

struct MlaArgs {
  const uint16_t* q;       // [QR, H, 576] bf16
  const int32_t* idx;      // [QR, k]
  RowStore rows;
  int Sq, H, k;
  int splits, per_split;   // per_split: entries per split (multiple of 32)
  float scale_log2;
  void* o;                 // [QR, H, 512] (o_f32 ? float : bf16)   -- written directly when splits == 1
  int o_f32;
  float* lse;              // [QR, H]
  void* part_o;            // split partials, 512 values per row in o's dtype, normalised:
  float* part_lse;         //   [QR, splits, H] rows (split form) or the row-stream slots
  int32_t* err;
  // union form (query tokens folded into the head axis): entries of row qr past counts[qr]
  // are skipped; wave heads of query t = head / fold_h only see entries whose bit is set in
  // member[(qr * fold_sq + t) * mwords + entry / 32]
  const int32_t* counts;   // [QR] or null
  const uint32_t* member;  // or null
  int fold_h, fold_sq, mwords;
  // row-stream form of the 64-head kernel (sk_groups > 0, split form otherwise): the
  // sk_groups work-groups of each head block share its QR x sk_tpu tiles evenly; partials
  // in nhb x (sk_groups + QR) slots of 64 rows (see mla_pieces)
  int QR, sk_groups, sk_tpu;
};

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// max over lanes l, l^16, l^32, l^48 (the four lanes of a head) with the row-swap permutes
// (VALU; a shuffle through LDS would wait behind the tile's operand reads).  Each swap
// pairs lane l with l^16 (v_permlane16_swap) or l^32 (v_permlane32_swap) across its two
// results; lane check on the device: a probe of both swaps against l ^ 16 and l ^ 32.
__device__ __forceinline__ float head_max4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// Byte offset of 16-byte chunk c of token n inside a tile.  Token group tg = n / 8 and
// chunk group cg = c / 8 select block cg * 4 + tg (1 KB, unpadded); inside it, chunk
// cc = c % 8 of token m = n % 8 sits at 16-byte slot m * 8 + (cc ^ 2(m/2)).  One LDS-direct
// load instruction fills a block with eight whole 128-byte lines (eight consecutive lanes
// per token).
// LDS banks (64 x 4 bytes), as measured with PMC bank-conflict counts on single-wave probes:
// a ds_read_b128 is served as four 16-lane sets, each 32-lane half split by the parity of
// the lane's quad index (lane / 4), and a set takes one cycle per access to its most used
// 16-byte bank group (address / 16 mod 16).  The K operand read (lane (n, g) reads chunk
// 4j + g of token n) then gives every set 16 distinct groups; with a 16-byte padding per
// block it cost four extra cycles per read.  The transpose reads measure conflict-free too.
constexpr int kBlockBytes = 1024;
__device__ __forceinline__ int chunk_byte(int n, int c) {
  const int m = n & 7, cc = c & 7;
  return (((c >> 3) << 2) + (n >> 3)) * kBlockBytes + (m * 8 + (cc ^ ((m >> 1) << 1))) * 16;
}

// 16 bytes from global memory into LDS at M0 + 16 * lane (M0 = lds_addr, wave-uniform).  No
// instruction offset is used: it would move the LDS destination as well.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_addr) : "m0");
}

// LDS-direct loads R..CPT-1 of one tile: load r fetches chunk group r / NSRC of the row in
// src[r % NSRC] into block r * NW of the wave's stripe
template <int R, int CPT, int NSRC, int NW>
__device__ __forceinline__ void dma_tile(const char* const* src, uint32_t dst) {
  if constexpr (R < CPT) {
    lds_dma16(src[R % NSRC] + (R / NSRC) * 128, dst + R * NW * kBlockBytes);
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

// grid position -> (unit = query row x split, head block).  Work-groups go round robin over
// the 8 XCDs, each with its own L2.  When the query rows split evenly over the XCDs (QR % 8 ==
// 0), every work-group of one query row runs on XCD qr % 8: its head blocks read the same
// selected rows and its splits the same q from that L2, and the merge of its split partials
// (mla_merge_unit) runs there too.  Otherwise the head blocks of one unit share an XCD.
__device__ __forceinline__ void mla_block_unit(int nhb, int splits, int& unit, int& hb) {
  const int x = blockIdx.x, G = gridDim.x;
  const int per_qr = splits * nhb;
  if (G % (8 * per_qr) == 0) {
    const int xcd = x & 7, kk = x >> 3;
    const int local = kk % per_qr;
    hb = local % nhb;
    unit = ((kk / per_qr) * 8 + xcd) * splits + local / nhb;
  } else if (G % (8 * nhb) == 0) {
    const int xcd = x & 7, kk = x >> 3;
    hb = kk % nhb;
    unit = (kk / nhb) * 8 + xcd;
  } else {
    hb = x % nhb;
    unit = x / nhb;
  }
}

// merge grid position -> (query row, head block of kMergeHeads): with QR % 8 == 0 the merge
// of query row qr runs on XCD qr % 8, where the decode work-groups wrote its partials
__device__ __forceinline__ void mla_merge_unit(int hblocks, int& qr, int& hblk) {
  const int x = blockIdx.x, G = gridDim.x;
  if (G % (8 * hblocks) == 0) {
    const int xcd = x & 7, kk = x >> 3;
    hblk = kk % hblocks;
    qr = (kk / hblocks) * 8 + xcd;
  } else {
    qr = x / hblocks;
    hblk = x - qr * hblocks;
  }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// NW waves per stream (16 heads each), NS token streams: stream s handles tiles T with
// T % NS == s, so NS waves share each SIMD and hide each other's latencies.  Each stream
// keeps its own online-softmax state; the streams are merged through LDS at the end.
template <int NW, int NS>
__global__ void __launch_bounds__(64 * NW * NS, 1) mla_decode_kernel(MlaArgs a) {
  constexpr int NT = 64 * NW * NS;
  constexpr int NTS = 64 * NW;              // threads of one stream
  constexpr int CPT = kTileSlots / NTS;     // LDS-direct loads per thread per tile
  static_assert(kTileSlots % NTS == 0, "tile must split evenly over a stream's threads");
  constexpr int NSRC = 4 / NW;              // token groups one lane streams per tile
  static_assert(NSRC * NW == 4, "NW must divide the 4 token groups of a tile");
  constexpr int PD = (NS == 1) ? 2 : 1;     // iterations a tile is loaded ahead
  constexpr int RING = NS * (PD + 1);       // LDS tiles
  static_assert(RING * kTileBytes + kMaxSplit * 8 + 128 + NW * kMaxSplit / 8 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) uint8_t ring[RING][kTileBytes];
  __shared__ int64_t rowoff[kMaxSplit];     // byte offset of each selected row of the split, -1 = none
  __shared__ uint32_t tmask[kMaxSplit / kTT];  // valid-row bits per tile
  __shared__ uint32_t mmask[NW][kMaxSplit / kTT];   // union form: the entries each head group's query selected

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int stream = wave / NW, ws = wave % NW;
  const int n = lane & 15, g = lane >> 4;
  const int nhb = (a.H + 16 * NW - 1) / (16 * NW);
  int unit, hb;
  mla_block_unit(nhb, a.splits, unit, hb);
  const int qr = unit / a.splits;
  const int split = unit - qr * a.splits;
  const int b = qr / a.Sq;
  const int head = hb * 16 * NW + ws * 16 + n;
  const bool head_ok = head < a.H;

  const int kq = a.counts ? max(0, min(a.k, a.counts[qr])) : a.k;   // entries of this row
  // with a per-row count the row's entries are spread evenly over its splits (never more
  // per split than the host sized for)
  const int per = a.counts ? min(a.per_split, (((kq + a.splits - 1) / a.splits) + kTT - 1) / kTT * kTT) : a.per_split;
  const int e_begin = split * per;
  const int e_end = min(e_begin + per, kq);
  const int ntiles = e_end > e_begin ? (e_end - e_begin + kTT - 1) / kTT : 0;
  const int32_t* idx = a.idx + (int64_t)qr * a.k;
  // rows that are padding or unresolvable are loaded from this query row instead (finite
  // values; their probabilities are exactly zero)
  const char* stand_in = reinterpret_cast<const char*>(a.q + (int64_t)qr * a.H * kRowEl);

  // ---- q^T operand: 18 k-steps of 32 latent dims; lane (n, g) holds dims 32j + 8g .. +8
  bf16x8 qb[18];
  {
    const uint16_t* qp = a.q + ((int64_t)qr * a.H + (head_ok ? head : 0)) * kRowEl + g * 8;
#pragma unroll
    for (int j = 0; j < 18; ++j) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + j * 32);
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
      if (row < 0 && p >= 0 && hb == 0) count_error(a.err);   // once per entry, not per head block
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
  // LDS-direct load r of this lane: token group tg = ws + NW * (r % NSRC), chunk group
  // r / NSRC; the lane fetches chunk (lane % 8) ^ 2(m/2) of token m = 8 tg + lane / 8
  const int dlane = ((lane & 7) ^ (((lane >> 4) & 3) << 1)) * 16;
  int koff[2][2];               // K operand of M tile mt, k-step j: koff[j % 2][mt] + 4 blocks (j / 2)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) koff[j][mt] = chunk_byte(n + 16 * mt, 4 * j + g);
  int voff[4];                  // V^T operand (transpose read) of value tile vt: voff[vt % 4] + 4 blocks (vt / 4)
  {
    const int jj = n >> 2, qq = n & 3;          // source lane n = 4 jj + qq of this 16-lane group
    const int tok = 4 * g + jj;
#pragma unroll
    for (int vm = 0; vm < 4; ++vm) voff[vm] = chunk_byte(tok, 2 * vm + (qq >> 1)) + (qq & 1) * 8;
  }
  if (a.member && stream == 0 && lane < ntiles) {
    // the query of this wave's 16 heads (fold_h is a multiple of 16, so they share one)
    const int t = (hb * 16 * NW + ws * 16) / a.fold_h;
    mmask[ws][lane] = (t < a.fold_sq) ? a.member[((int64_t)qr * a.fold_sq + t) * a.mwords + e_begin / kTT + lane] : 0u;
  }
  wait_vmcnt<0>();              // q^T is resident before any row load is in flight
  __syncthreads();              // rowoff / tmask / mmask ready

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&ring[0][0];
  const char* nsrc[NSRC];       // rows of the next tile this wave issues
  auto prepare = [&](int T) {
#pragma unroll
    for (int p = 0; p < NSRC; ++p) {
      const int64_t off = rowoff[T * kTT + (ws + NW * p) * 8 + (lane >> 3)];
      nsrc[p] = (off >= 0 ? a.rows.base + off : stand_in) + dlane;
    }
  };
  auto issue = [&](int T) {
    const uint32_t dst = ring_lds + (uint32_t)((T % RING) * kTileBytes + ws * kBlockBytes);
    dma_tile<0, CPT, NSRC, NW>(nsrc, dst);
  };

  const int iters = (ntiles + NS - 1) / NS;  // tile of iteration i for this stream: i*NS + stream
#pragma unroll
  for (int i = 0; i < PD; ++i) {
    const int T = i * NS + stream;
    if (T < ntiles) {
      prepare(T);
      issue(T);
    }
  }
  if (PD * NS + stream < ntiles) prepare(PD * NS + stream);

  f32x4 oacc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) oacc[i] = f32x4{};
  float m_used = -INFINITY;     // log2-domain running max used for p
  float l_part = 0.0f;          // this lane's share of sum p (fp32 p: for lse)
  float lr_part = 0.0f;         // this lane's share of sum bf16(p) (the PV weights: for o)

  for (int i = 0; i < iters; ++i) {
    const int T = i * NS + stream;
    if (PD == 2 && T + NS < ntiles)
      wait_vmcnt<CPT>();        // this wave's loads of tile T are done (the next one may be in flight)
    else
      wait_vmcnt<0>();
    __syncthreads();            // this iteration's tiles complete; the slots of iteration i-1 are free
    const int Tn = T + PD * NS;
    if (Tn < ntiles) {
      issue(Tn);
      if (Tn + NS < ntiles) prepare(Tn + NS);
    }
    if (T >= ntiles) continue;  // stream without a tile in the last iteration
    const lds_u8* tile = (const lds_u8*)(uintptr_t)(ring_lds + (uint32_t)((T % RING) * kTileBytes));

    // ---- S^T over the 576 latent dims: two independent 16-token chains
    f32x4 s0 = f32x4{}, s1 = f32x4{};
    {
      auto kop = [&](int j, int mt) {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(tile + koff[j & 1][mt] +
                                                                                 (j >> 1) * 4 * kBlockBytes);
      };
      constexpr int RK = (NS == 1) ? 2 : 1;    // operand reads issued ahead (none under the tighter budget)
      bf16x8 r0[RK], r1[RK];
      if constexpr (RK == 2) {
        r0[0] = kop(0, 0);
        r1[0] = kop(0, 1);
      }
#pragma unroll
      for (int j = 0; j < 18; ++j) {
        if constexpr (RK == 2) {
          if (j + 1 < 18) {
            r0[(j + 1) & 1] = kop(j + 1, 0);
            r1[(j + 1) & 1] = kop(j + 1, 1);
          }
        } else {
          r0[0] = kop(j, 0);
          r1[0] = kop(j, 1);
        }
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0[j % RK], qb[j], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r1[j % RK], qb[j], s1, 0, 0, 0);
      }
    }
    float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};   // tokens 4g+i, 16+4g+i

    // ---- online softmax for head n
    uint32_t vmask = __builtin_amdgcn_readfirstlane(tmask[T]);
    if (a.member) vmask &= __builtin_amdgcn_readfirstlane(mmask[ws][T]);
    if (vmask != 0xffffffffu) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int tok = (c >> 2) * 16 + g * 4 + (c & 3);
        if (!((vmask >> tok) & 1u)) s[c] = -INFINITY;
      }
    }
    float tmax = s[0];
#pragma unroll
    for (int c = 1; c < 8; ++c) tmax = fmaxf(tmax, s[c]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * a.scale_log2;   // scale > 0 keeps the order
    const bool grow = tmax > m_used + kLazy || (m_used == -INFINITY && tmax > -INFINITY);
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? tmax : m_used;
      const float alpha = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - m_new);
#pragma unroll
      for (int c = 0; c < 32; ++c) oacc[c] *= alpha;
      l_part *= alpha;
      lr_part *= alpha;
      m_used = m_new;
    }
    const float msub = (m_used == -INFINITY) ? 0.0f : m_used;
    uint32_t pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * c], a.scale_log2, -msub));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * c + 1], a.scale_log2, -msub));
      const uint32_t w = pack_bf16x2(p0, p1);
      pb[c] = w;
      l_part += p0 + p1;
      lr_part += __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
    }
    const bf16x8 pt = __builtin_bit_cast(bf16x8, u32x4{pb[0], pb[1], pb[2], pb[3]});

    // ---- O^T += V^T . P^T over 32 value tiles of 16 dims; operand reads run ahead
    {
      auto vop = [&](int vt) {  // tokens 4g.. (first 8 bytes) and 16+4g.. (last 8 bytes)
        const lds_u8* p = tile + voff[vt & 3] + (vt >> 2) * 4 * kBlockBytes;
        const u32x2 lo = lds_read_tr16(p);
        const u32x2 hi = lds_read_tr16(p + 2 * kBlockBytes);   // tokens + 16: two token groups on
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      };
      constexpr int RV = (NS == 1) ? 4 : 2;    // operand reads in flight (2 under the tighter register budget)
      bf16x8 rv[RV];
#pragma unroll
      for (int c = 0; c < RV - 1; ++c) rv[c] = vop(c);
#pragma unroll
      for (int vt = 0; vt < 32; ++vt) {
        if (vt + RV - 1 < 32) rv[(vt + RV - 1) % RV] = vop(vt + RV - 1);
        oacc[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rv[vt % RV], pt, oacc[vt], 0, 0, 0);
      }
    }
  }

  if constexpr (NS == 2) {
    // ---- merge stream 1 into stream 0 through the (now idle) ring
    __syncthreads();
    f32x4* xo = reinterpret_cast<f32x4*>(&ring[0][0]);                  // [NW][32][64]
    float* xs = reinterpret_cast<float*>(xo + NW * 32 * 64);             // [NW][3][64]
    static_assert(NW * 32 * 64 * 16 + NW * 3 * 64 * 4 <= RING * kTileBytes, "merge staging fits the ring");
    if (stream == 1) {
#pragma unroll
      for (int vt = 0; vt < 32; ++vt) xo[(ws * 32 + vt) * 64 + lane] = oacc[vt];
      xs[(ws * 3 + 0) * 64 + lane] = m_used;
      xs[(ws * 3 + 1) * 64 + lane] = l_part;
      xs[(ws * 3 + 2) * 64 + lane] = lr_part;
    }
    __syncthreads();
    if (stream == 1) return;
    const float m1 = xs[(ws * 3 + 0) * 64 + lane];
    const float m_new = fmaxf(m_used, m1);
    const float a0 = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - m_new);
    const float a1 = (m1 == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m1 - m_new);
    l_part = l_part * a0 + xs[(ws * 3 + 1) * 64 + lane] * a1;
    lr_part = lr_part * a0 + xs[(ws * 3 + 2) * 64 + lane] * a1;
#pragma unroll
    for (int vt = 0; vt < 32; ++vt) oacc[vt] = oacc[vt] * a0 + xo[(ws * 32 + vt) * 64 + lane] * a1;
    m_used = m_new;
  }

  // ---- finish: l over the head's four lanes, normalise, write 512 dims
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float lr_tot = lr_part + __shfl_xor(lr_part, 16);
  lr_tot += __shfl_xor(lr_tot, 32);
  const float inv = (lr_tot > 0.0f) ? 1.0f / lr_tot : 0.0f;
  const float lse = (l_tot > 0.0f) ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
  if (!head_ok) return;
  const bool direct = a.splits == 1;
  const int64_t obase = (direct ? ((int64_t)qr * a.H + head) : ((((int64_t)qr * a.splits + split) * a.H + head))) *
                            kVDim + g * 4;
  void* dst = direct ? a.o : a.part_o;
  if (a.o_f32) {
#pragma unroll
    for (int vt = 0; vt < 32; ++vt)
      *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + obase + vt * 16) = oacc[vt] * inv;
  } else {
#pragma unroll
    for (int vt = 0; vt < 32; ++vt)
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst) + obase + vt * 16) =
          u32x2{pack_bf16x2(oacc[vt].x * inv, oacc[vt].y * inv), pack_bf16x2(oacc[vt].z * inv, oacc[vt].w * inv)};
  }
  if (g == 0) {
    if (direct)
      a.lse[(int64_t)qr * a.H + head] = lse;
    else
      a.part_lse[((int64_t)qr * a.splits + split) * a.H + head] = lse;
  }
}

// A piece of a 64-head work-group's work: entries e_begin..e_end of query row qr's selection
// for head block hb.  Its normalised o and lse go to rows orow0 + (head - 64 hb) of the
// caller's o and lse (direct) or of the partial arrays.
struct MlaPiece {
  int qr, hb, e_begin, e_end;
  int64_t orow0;
  bool direct;
};

// The pieces of this work-group.  Split form: one piece, the (query row, split) of the grid
// position.  Row-stream form (sk_groups = G > 0): the G work-groups of head block hb share
// its QR x Tu tiles of 32 entries (row by row) evenly, work-group w taking tiles
// [w T / G, (w + 1) T / G) of T = QR Tu.  The host picks this form only when a share is at
// most one row's Tu tiles, so a work-group meets at most two rows: piece 0 writes partial
// slot w, a second piece (which starts row r) slot G + r, among head block hb's G + QR slots
// of 64 rows.  Work-group w of every head block runs on XCD w % 8 (round-robin placement),
// so the head blocks read the same rows from one L2.
template <bool SK>
__device__ __forceinline__ int mla_pieces(const MlaArgs& a, int nhb, MlaPiece (&pc)[2]) {
  if constexpr (!SK) {
    int unit, hb;
    mla_block_unit(nhb, a.splits, unit, hb);
    const int qr = unit / a.splits;
    const int split = unit - qr * a.splits;
    const int kq = a.counts ? max(0, min(a.k, a.counts[qr])) : a.k;
    // with a per-row count the row's entries are spread evenly over its splits (never more
    // per split than the host sized for)
    const int per =
        a.counts ? min(a.per_split, (((kq + a.splits - 1) / a.splits) + kTT - 1) / kTT * kTT) : a.per_split;
    pc[0].qr = qr;
    pc[0].hb = hb;
    pc[0].e_begin = split * per;
    pc[0].e_end = min(pc[0].e_begin + per, kq);
    pc[0].direct = a.splits == 1;
    pc[0].orow0 = (pc[0].direct ? (int64_t)qr * a.H : ((int64_t)qr * a.splits + split) * a.H) + hb * 64;
    return 1;
  } else {
  const int G = a.sk_groups, Tu = a.sk_tpu;
  const int x = blockIdx.x, xcd = x & 7, kk = x >> 3;
  const int hb = kk % nhb;
  const int w = (kk / nhb) * 8 + xcd;
  const int64_t T = (int64_t)a.QR * Tu;
  const int64_t start = (int64_t)w * T / G, end = (int64_t)(w + 1) * T / G;
  const int r0 = (int)(start / Tu);
  const int64_t slots = (int64_t)hb * (G + a.QR);
  pc[0].qr = r0;
  pc[0].hb = hb;
  pc[0].e_begin = (int)(start - (int64_t)r0 * Tu) * kTT;
  pc[0].e_end = min((int)min(end - (int64_t)r0 * Tu, (int64_t)Tu) * kTT, a.k);
  pc[0].direct = false;
  pc[0].orow0 = (slots + w) * 64;
  if (end <= (int64_t)(r0 + 1) * Tu) return 1;
  const int r1 = r0 + 1;
  pc[1].qr = r1;
  pc[1].hb = hb;
  pc[1].e_begin = 0;
  pc[1].e_end = min((int)(end - (int64_t)r1 * Tu) * kTT, a.k);
  pc[1].direct = false;
  pc[1].orow0 = (slots + G + r1) * 64;
  return 2;
  }
}

// ---- role-split form: 64 heads per work-group, eight waves in two roles
// Score waves 0-3: wave w keeps q^T of heads 16w..16w+15 in VGPRs and computes
//   S^T[32 tokens x 16 heads] = K_tile . q^T exactly as the two-stream form does, then the
//   online softmax of its heads; it writes P^T (bf16, already in the B-operand lane layout of
//   the value product) and, when its running max moved, the heads' rescale factors to LDS.
// Value waves 4-7: wave 4+d keeps O^T for value dims 128d..128d+127 of all 64 heads (32
//   accumulator tiles of 16 dims x 16 heads) and adds V^T . P^T for the tile the score waves
//   finished one iteration earlier.  Each V^T operand read serves the four head groups, so a
//   tile's V^T bytes are read from LDS once per 64 heads instead of once per 16.  The value
//   waves also issue the row loads (token group d of every tile).
// Iteration i: score waves take tile i, value waves tile i-1, one barrier.  Ring slot i % 4
// holds tile i from its load (issued in iteration i-2) until the value waves are done with it
// (iteration i+1), so two tiles are always in flight.
// Waves w and w + 4 of a work-group share a SIMD (measured placement), so each SIMD runs one
// score and one value wave: 36 + 32 MFMAs 16x16x32 per tile.  Per tile and CU the LDS serves
// 144 KB of K-operand reads (ds_read_b128, measured 250 B/clk per CU), 32 KB of V^T transpose
// reads (ds_read_b64_tr_b16, measured 62.5 B/clk per CU) and 36 KB of row loads: about 1,400
// LDS cycles against 1,088 MFMA cycles per SIMD.  The operand reads are kept ahead of their
// MFMAs with scheduling barriers; left alone, the scheduler sinks each read next to its use.
// Tried and slower: two 32-head score waves alone on their SIMDs (six waves; K read once per
// 32 heads, but 72 score MFMAs and the softmax of 32 heads on one SIMD per tile), and a second
// barrier that keeps the value MFMAs off the matrix cores until the score MFMAs are issued.
constexpr int kRolesRing = 4;
constexpr int kScoreRK = 4;     // K-operand read buffers of a score wave (reads 3 k-steps ahead)
constexpr int kValueRV = 3;     // V^T operand buffers of a value wave (reads 2 value tiles ahead)

template <bool SK>   // row-stream form (a.sk_groups > 0), else the split form
__global__ void __launch_bounds__(512, 1) mla_roles_kernel(MlaArgs a) {
  constexpr int NT = 512;
  constexpr int CPT = kTileSlots / 256;     // LDS-direct loads per value-wave thread per tile
  static_assert(CPT == 9, "a tile is 36 blocks, nine per value wave");
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRolesRing][kTileBytes];
  __shared__ int32_t rowix[kMaxSplit];      // row index of each selected row of the split, -1 = none
  __shared__ uint32_t tmask[kMaxSplit / kTT];          // valid-row bits per tile
  __shared__ uint32_t mmask[4][kMaxSplit / kTT];       // union form: the entries each head group's query selected
  __shared__ bf16x8 pbuf[2][4][64];         // P^T of a tile per head group, lane (n, g) as the B operand
  __shared__ float abuf[2][4][16];          // rescale factor per (head group, head), valid when aflag is set
  __shared__ __attribute__((aligned(16))) uint32_t aflag[2][4];
  __shared__ float xinv[4][16];             // 1 / sum of the bf16 weights per head, for the output
  static_assert(kRolesRing * kTileBytes + kMaxSplit * 4 + (kMaxSplit / kTT) * 4 * 5 + 2 * 4 * 64 * 16 +
                        2 * 4 * 16 * 4 + 2 * 4 * 4 + 4 * 16 * 4 <= 160 * 1024,
                "LDS budget");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nhb = (a.H + 63) / 64;
  MlaPiece pcs[2];
  const int npc = mla_pieces<SK>(a, nhb, pcs);

  for (int pi = 0; pi < npc; ++pi) {
  const MlaPiece pc = pi == 0 ? pcs[0] : pcs[1];
  const int qr = pc.qr, hb = pc.hb, e_begin = pc.e_begin, e_end = pc.e_end;
  const int b = qr / a.Sq;
  const int ntiles = e_end > e_begin ? (e_end - e_begin + kTT - 1) / kTT : 0;
  const int32_t* idx = a.idx + (int64_t)qr * a.k;

  // ---- resolve every selected row of this split once: index -> page table -> row
  for (int e = tid; e < ntiles * kTT; e += NT) {
    int32_t r = -1;
    if (e_begin + e < e_end) {
      const int32_t p = idx[e_begin + e];
      const int64_t row = a.rows.row(b, p);
      if (row < 0 && p >= 0 && hb == 0) count_error(a.err);   // once per entry, not per head block
      if (row >= 0) r = (int32_t)row;       // num_rows < 2^31 (checked on the host)
    }
    rowix[e] = r;
    const uint64_t m = __builtin_amdgcn_ballot_w64(r >= 0);
    if (lane == 0) {            // e is a multiple of 64 here: lanes 0-31 and 32-63 are two tiles
      tmask[e >> 5] = (uint32_t)m;
      if ((e >> 5) + 1 < ntiles) tmask[(e >> 5) + 1] = (uint32_t)(m >> 32);
    }
  }

  if (wave < 4) {
    // ================================================================ score wave
    const int w = wave;
    const int head = hb * 64 + w * 16 + n;
    const bool head_ok = head < a.H;
    // q^T: lane (n, g) holds dims 32j + 8g .. +8 of head n.  A head past H reads head 0 instead
    // (finite values; nothing of it is stored), so no select waits for these loads before the
    // first barrier, which the value waves' first row loads wait behind.
    bf16x8 qb[18];
    {
      const uint16_t* qp = a.q + ((int64_t)qr * a.H + (head_ok ? head : 0)) * kRowEl + g * 8;
#pragma unroll
      for (int j = 0; j < 18; ++j) qb[j] = *reinterpret_cast<const bf16x8*>(qp + j * 32);
    }
    int koff[2][2];             // K operand of M tile mt, k-step j: koff[j % 2][mt] + 4 blocks (j / 2)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) koff[j][mt] = chunk_byte(n + 16 * mt, 4 * j + g);
    if (a.member && lane < ntiles) {
      // the query of this wave's 16 heads (fold_h is a multiple of 16, so they share one)
      const int t = (hb * 64 + w * 16) / a.fold_h;
      mmask[w][lane] = (t < a.fold_sq) ? a.member[((int64_t)qr * a.fold_sq + t) * a.mwords + e_begin / kTT + lane] : 0u;
    }
    __syncthreads();            // rowix / tmask / mmask ready

    const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&ring[0][0];
    float m_used = -INFINITY;   // log2-domain running max used for p
    float l_part = 0.0f;        // this lane's share of sum p (fp32 p: for lse)
    float lr_part = 0.0f;       // this lane's share of sum bf16(p) (the PV weights: for o)
    for (int i = 0; i <= ntiles; ++i) {
      __syncthreads();          // tile i is in its slot; the value waves are done with P of tile i-2
      if (i >= ntiles) continue;
      const lds_u8* tile = (const lds_u8*)(uintptr_t)(ring_lds + (uint32_t)((i % kRolesRing) * kTileBytes));

      // ---- S^T over the 576 latent dims: two independent 16-token chains, operand reads
      // kScoreRK - 1 steps ahead
      f32x4 s0 = f32x4{}, s1 = f32x4{};
      {
        auto kop = [&](int j, int mt) {
          return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(tile + koff[j & 1][mt] +
                                                                                   (j >> 1) * 4 * kBlockBytes);
        };
        bf16x8 r0[kScoreRK], r1[kScoreRK];
#pragma unroll
        for (int c = 0; c < kScoreRK - 1; ++c) {
          r0[c] = kop(c, 0);
          r1[c] = kop(c, 1);
        }
#pragma unroll
        for (int j = 0; j < 18; ++j) {
          if (j + kScoreRK - 1 < 18) {
            r0[(j + kScoreRK - 1) % kScoreRK] = kop(j + kScoreRK - 1, 0);
            r1[(j + kScoreRK - 1) % kScoreRK] = kop(j + kScoreRK - 1, 1);
          }
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r0[j % kScoreRK], qb[j], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r1[j % kScoreRK], qb[j], s1, 0, 0, 0);
          // keep the reads kScoreRK - 1 steps ahead: the scheduler would otherwise sink each
          // read next to its MFMA and every MFMA would wait out a full LDS latency
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};   // tokens 4g+i, 16+4g+i

      // ---- online softmax for head n
      uint32_t vmask = __builtin_amdgcn_readfirstlane(tmask[i]);
      if (a.member) vmask &= __builtin_amdgcn_readfirstlane(mmask[w][i]);
      if (vmask != 0xffffffffu) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int tok = (c >> 2) * 16 + g * 4 + (c & 3);
          if (!((vmask >> tok) & 1u)) s[c] = -INFINITY;
        }
      }
      float tmax = s[0];
#pragma unroll
      for (int c = 1; c < 8; ++c) tmax = fmaxf(tmax, s[c]);
      tmax = head_max4(tmax) * a.scale_log2;   // scale > 0 keeps the order
      const bool grow = tmax > m_used + kLazy || (m_used == -INFINITY && tmax > -INFINITY);
      uint32_t rescaled = 0;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? tmax : m_used;
        const float alpha = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - m_new);
        l_part *= alpha;
        lr_part *= alpha;
        m_used = m_new;
        if (g == 0) abuf[i & 1][w][n] = alpha;
        rescaled = 1;
      }
      const float msub = (m_used == -INFINITY) ? 0.0f : m_used;
      uint32_t pb[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * c], a.scale_log2, -msub));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * c + 1], a.scale_log2, -msub));
        const uint32_t wd = pack_bf16x2(p0, p1);
        pb[c] = wd;
        l_part += p0 + p1;
        lr_part += __uint_as_float(wd << 16) + __uint_as_float(wd & 0xffff0000u);
      }
      pbuf[i & 1][w][lane] = __builtin_bit_cast(bf16x8, u32x4{pb[0], pb[1], pb[2], pb[3]});
      if (lane == 0) aflag[i & 1][w] = rescaled;
    }

    // ---- finish: l over the head's four lanes; the value waves normalise and write o
    float l_tot = l_part + __shfl_xor(l_part, 16);
    l_tot += __shfl_xor(l_tot, 32);
    float lr_tot = lr_part + __shfl_xor(lr_part, 16);
    lr_tot += __shfl_xor(lr_tot, 32);
    if (g == 0) xinv[w][n] = (lr_tot > 0.0f) ? 1.0f / lr_tot : 0.0f;
    const float lse = (l_tot > 0.0f) ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;
    if (g == 0 && head_ok) (pc.direct ? a.lse : a.part_lse)[pc.orow0 + w * 16 + n] = lse;
    __syncthreads();            // xinv ready
    continue;
  }

  // ================================================================== value wave
  const int d = wave - 4;       // value dims 128d .. 128d + 127 = value tiles 8d .. 8d + 7
  // LDS-direct load r of this lane: token group d, chunk group r; the lane fetches chunk
  // (lane % 8) ^ 2(m/2) of token m = 8d + lane / 8
  const int dlane = ((lane & 7) ^ (((lane >> 4) & 3) << 1)) * 16;
  int voff[4];                  // V^T operand of value tile vt: voff[vt % 4] + 4 blocks (vt / 4)
  {
    const int jj = n >> 2, qq = n & 3;          // source lane n = 4 jj + qq of this 16-lane group
    const int tok = 4 * g + jj;
#pragma unroll
    for (int vm = 0; vm < 4; ++vm) voff[vm] = chunk_byte(tok, 2 * vm + (qq >> 1)) + (qq & 1) * 8;
  }
  // rows that are padding or unresolvable are loaded from this query row instead (finite
  // values; their probabilities are exactly zero)
  const char* stand_in = reinterpret_cast<const char*>(a.q + (int64_t)qr * a.H * kRowEl);
  __syncthreads();              // rowix / tmask / mmask ready

  const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&ring[0][0];
  const char* nsrc[1];          // row of the next tile this lane loads
  auto prepare = [&](int T) {
    const int32_t r = rowix[T * kTT + d * 8 + (lane >> 3)];
    nsrc[0] = (r >= 0 ? a.rows.base + (int64_t)r * kRowBytes : stand_in) + dlane;
  };
  auto issue = [&](int T) {
    const uint32_t dst = ring_lds + (uint32_t)((T % kRolesRing) * kTileBytes + d * kBlockBytes);
    dma_tile<0, CPT, 1, 4>(nsrc, dst);
  };
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    if (T < ntiles) {
      prepare(T);
      issue(T);
    }
  }
  if (2 < ntiles) prepare(2);

  f32x4 oacc[4][8];             // [head group][value tile 8d + v]
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int v = 0; v < 8; ++v) oacc[h][v] = f32x4{};

  for (int i = 0; i <= ntiles; ++i) {
    if (i + 1 < ntiles)
      wait_vmcnt<CPT>();        // this wave's loads of tile i are done (tile i+1's may be in flight)
    else
      wait_vmcnt<0>();
    __syncthreads();            // tile i complete; P of tile i-1 written; the slot of tile i-2 is free
    if (i + 2 < ntiles) {
      issue(i + 2);
      if (i + 3 < ntiles) prepare(i + 3);
    }
    if (i == 0) continue;
    const int T = i - 1;
    const int pslot = T & 1;
    const lds_u8* tile = (const lds_u8*)(uintptr_t)(ring_lds + (uint32_t)((T % kRolesRing) * kTileBytes));
    // ---- O^T += V^T . P^T over this wave's 8 value tiles, each read once for the 4 head groups
    auto vop = [&](int v) {     // tokens 4g.. (first 8 bytes) and 16+4g.. (last 8 bytes)
      const int vt = 8 * d + v;
      const lds_u8* p = tile + voff[vt & 3] + (vt >> 2) * 4 * kBlockBytes;
      const u32x2 lo = lds_read_tr16(p);
      const u32x2 hi = lds_read_tr16(p + 2 * kBlockBytes);   // tokens + 16: two token groups on
      return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    };
    bf16x8 rv[kValueRV];
#pragma unroll
    for (int c = 0; c < kValueRV - 1; ++c) rv[c] = vop(c);
    bf16x8 pt[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pt[h] = pbuf[pslot][h][lane];
    const u32x4 fl = *reinterpret_cast<const u32x4*>(&aflag[pslot][0]);
    __builtin_amdgcn_sched_barrier(0);      // the first operand reads are in flight before any wait
    if (__builtin_amdgcn_readfirstlane(fl.x | fl.y | fl.z | fl.w)) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (__builtin_amdgcn_readfirstlane(fl[h])) {
          const float alpha = abuf[pslot][h][n];
#pragma unroll
          for (int v = 0; v < 8; ++v) oacc[h][v] *= alpha;
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      if (v + kValueRV - 1 < 8) rv[(v + kValueRV - 1) % kValueRV] = vop(v + kValueRV - 1);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        oacc[h][v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rv[v % kValueRV], pt[h], oacc[h][v], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);    // reads stay kValueRV - 1 value tiles ahead
    }
  }

  __syncthreads();              // xinv ready
  void* dst = pc.direct ? a.o : a.part_o;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int head = hb * 64 + h * 16 + n;
    if (head >= a.H) continue;
    const float inv = xinv[h][n];
    const int64_t obase = (pc.orow0 + h * 16 + n) * kVDim + d * 128 + g * 4;
    if (a.o_f32) {
#pragma unroll
      for (int v = 0; v < 8; ++v)
        *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + obase + v * 16) = oacc[h][v] * inv;
    } else {
#pragma unroll
      for (int v = 0; v < 8; ++v)
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(dst) + obase + v * 16) =
            u32x2{pack_bf16x2(oacc[h][v].x * inv, oacc[h][v].y * inv),
                  pack_bf16x2(oacc[h][v].z * inv, oacc[h][v].w * inv)};
    }
  }
  }                             // pieces
}

// merge of split partials: 64 threads per (query row, head), 8 value dims per thread.  With
// SMAX > 0 (splits <= SMAX) every lse and partial load is issued before any is used, so a
// thread waits for memory once; SMAX == 0 handles any split count in batches of that kind.  F32: o and the partials
// are float32, else bf16.
constexpr int kMergeHeads = 4;   // heads per 256-thread work-group
constexpr int kMergeUnrolled = 8;
constexpr int kMergeUnrolledF32 = 4;

template <bool F32>
__device__ __forceinline__ void merge_load(const void* part_o, int64_t pb, u32x4& v0, u32x4& v1) {
  if constexpr (F32) {
    v0 = *reinterpret_cast<const u32x4*>(static_cast<const float*>(part_o) + pb);
    v1 = *reinterpret_cast<const u32x4*>(static_cast<const float*>(part_o) + pb + 4);
  } else {
    v0 = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(part_o) + pb);
  }
}

template <bool F32>
__device__ __forceinline__ void merge_add(float w, const u32x4& v0, const u32x4& v1, float* acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (F32) {
      acc[i] += w * __uint_as_float(v0[i]);
      acc[4 + i] += w * __uint_as_float(v1[i]);
    } else {
      acc[2 * i] += w * __uint_as_float(v0[i] << 16);
      acc[2 * i + 1] += w * __uint_as_float(v0[i] & 0xffff0000u);
    }
  }
}

template <int SMAX, bool F32, bool SK>
__global__ void __launch_bounds__(64 * kMergeHeads) mla_merge_kernel(MlaArgs a) {
  const int hblocks = (a.H + kMergeHeads - 1) / kMergeHeads;   // 1-D grid: query row x head block
  int qr, hblk;
  mla_merge_unit(hblocks, qr, hblk);
  const int head = hblk * kMergeHeads + (threadIdx.x >> 6);
  if (head >= a.H) return;
  const int d = (threadIdx.x & 63) * 8;
  // partial row of this head's s-th partial: split form, split s of row qr; row-stream
  // form, the pieces of the work-groups w0.. whose tile ranges meet row qr (mla_pieces)
  int S;
  int64_t srow0 = 0, sstep = 0;       // split form: row srow0 + s * sstep
  int sk_w0 = 0;
  int64_t sk_base = 0, sk_T = 0, sk_x0 = 0;
  if constexpr (!SK) {
    S = a.splits;
    srow0 = (int64_t)qr * S * a.H + head;
    sstep = a.H;
  } else {
    const int G = a.sk_groups, Tu = a.sk_tpu;
    sk_T = (int64_t)a.QR * Tu;
    sk_x0 = (int64_t)qr * Tu;
    const int64_t x1 = sk_x0 + Tu - 1;
    sk_w0 = (int)(((sk_x0 + 1) * G - 1) / sk_T);        // the work-group holding tile x0
    S = (int)(((x1 + 1) * G - 1) / sk_T) - sk_w0 + 1;
    sk_base = (int64_t)(head >> 6) * (G + a.QR);
  }
  auto prow = [&](int s) -> int64_t {
    if constexpr (!SK) {
      return srow0 + s * sstep;
    } else {
      const int G = a.sk_groups, w = sk_w0 + s;
      const int64_t slot = ((int64_t)w * sk_T / G < sk_x0) ? (int64_t)G + qr : (int64_t)w;
      return (sk_base + slot) * 64 + (head & 63);
    }
  };
  float mx = -INFINITY, wsum = 0.0f;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (SMAX > 0) {
    float lv[SMAX];
    u32x4 v0[SMAX], v1[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      lv[s] = -INFINITY;
      v0[s] = u32x4{};
      v1[s] = u32x4{};
      if (s < S) {
        const int64_t r = prow(s);
        lv[s] = a.part_lse[r];
        merge_load<F32>(a.part_o, r * kVDim + d, v0[s], v1[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < SMAX; ++s) mx = fmaxf(mx, lv[s]);
    if (mx > -INFINITY) {
#pragma unroll
      for (int s = 0; s < SMAX; ++s) {
        const float w = (lv[s] == -INFINITY) ? 0.0f : __expf(lv[s] - mx);
        wsum += w;
        merge_add<F32>(w, v0[s], v1[s], acc);
      }
    }
  } else {
    // any part count, in batches whose loads are all issued before any is used (a plain loop
    // waited out one memory latency per part)
    constexpr int NB = F32 ? kMergeUnrolledF32 : kMergeUnrolled;
    for (int s0 = 0; s0 < S; s0 += NB) {
      float lv[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) lv[j] = (s0 + j < S) ? a.part_lse[prow(s0 + j)] : -INFINITY;
#pragma unroll
      for (int j = 0; j < NB; ++j) mx = fmaxf(mx, lv[j]);
    }
    if (mx > -INFINITY) {
      for (int s0 = 0; s0 < S; s0 += NB) {
        float lv[NB];
        u32x4 v0[NB], v1[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          lv[j] = -INFINITY;
          v0[j] = u32x4{};
          v1[j] = u32x4{};
          if (s0 + j < S) {
            const int64_t r = prow(s0 + j);
            lv[j] = a.part_lse[r];
            merge_load<F32>(a.part_o, r * kVDim + d, v0[j], v1[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const float w = (lv[j] == -INFINITY) ? 0.0f : __expf(lv[j] - mx);
          wsum += w;
          merge_add<F32>(w, v0[j], v1[j], acc);
        }
      }
    }
  }
  if (mx > -INFINITY) {
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= inv;
  }
  const int64_t ob = ((int64_t)qr * a.H + head) * kVDim + d;
  if constexpr (F32) {
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
  static std::atomic<int> cus_by_dev[kMaxDevices];
  const int slot = current_device_slot();
  int cus = slot >= 0 ? cus_by_dev[slot].load(std::memory_order_relaxed) : 0;
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, slot < 0 ? 0 : slot) != hipSuccess ||
        cus <= 0)
      cus = 256;
    if (slot >= 0) cus_by_dev[slot].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// waves per work-group: 16 heads each, up to one per SIMD
static int mla_waves(int H) { return H >= 64 ? 4 : (H > 16 ? 2 : 1); }

// Splits per (query row, head block): one work-group fits a CU (its LDS ring), so a launch of
// W work-groups runs in ceil(W / CUs) rounds and takes about rounds x (F + tiles per split)
// tile-times, F being the per-work-group start-up and finish in tile-times (≈ 8: 18.8 µs for
// a one-tile work-group against 1.74 µs per further tile).  The plan takes the split count
// with the least such estimate (ties: fewer splits, fewer partials), from the fewest that
// keep a split within kMaxSplitRows rows up to four times the count that covers the CUs.
// With 264 work-groups at 2 splits, a 66-row batch ran a second round of 8; 3 splits make
// two full rounds of shorter work-groups.
// The 64-head kernel can instead share each head block's tiles evenly over a fixed set of
// work-groups (the row-stream form, mla_pieces): one round of F + tiles per work-group, plus
// a second start-up (≈ kPieceStartTiles) where a share crosses into a second row.  It is
// taken when its estimate is lower, a share is at most one row and fits the LDS row table,
// and the rows carry no per-row counts (the union form keeps splits).
constexpr int kSplitStartTiles = 8;
constexpr int kPieceStartTiles = 4;
constexpr int kMaxSplitRows = 1024;         // rows per split of the split form

struct MlaPlan {
  int splits = 1, per_split = 0;
  int sk_groups = 0, sk_tpu = 0;            // row-stream form when sk_groups > 0
  int sk_max_parts = 0;                     // most partials one (row, head) gets in that form
};

static MlaPlan mla_plan(int B, int Sq, int H, int k, bool row_stream) {
  MlaPlan p;
  const int nhb = (H + 16 * mla_waves(H) - 1) / (16 * mla_waves(H));
  const int64_t QR = (int64_t)B * Sq;
  const int64_t wgs = QR * nhb;
  const int tiles = (k + kTT - 1) / kTT;
  const int64_t cus = device_cus();
  const int min_s = (tiles + kMaxSplitRows / kTT - 1) / (kMaxSplitRows / kTT);
  const int cover = (int)std::min<int64_t>(tiles, (cus + wgs - 1) / wgs);
  const int max_s = std::max(min_s, std::min(tiles, 4 * std::max(cover, 1)));
  int s = min_s;
  int64_t best = -1;
  for (int c = min_s; c <= max_s; ++c) {
    const int64_t rounds = (wgs * c + cus - 1) / cus;
    const int64_t cost = rounds * (kSplitStartTiles + (tiles + c - 1) / c);
    if (best < 0 || cost < best) {
      best = cost;
      s = c;
    }
  }
  const int tps = (tiles + s - 1) / s;
  p.per_split = tps * kTT;
  p.splits = std::max(1, (k + p.per_split - 1) / p.per_split);
  if (row_stream && mla_waves(H) == 4) {
    const int64_t G = (cus / nhb) / 8 * 8;  // work-groups per head block, whole XCD rounds
    const int64_t T = QR * tiles;
    if (G >= 8 && T >= G && QR < ((int64_t)1 << 24)) {
      const int64_t tpw = (T + G - 1) / G;
      if (tpw <= tiles && tpw * kTT <= kMaxSplit) {
        const int64_t cost = kSplitStartTiles + tpw + (tpw < tiles ? kPieceStartTiles : 0);
        if (cost < best) {
          p.sk_groups = (int)G;
          p.sk_tpu = tiles;
          const int64_t tmin = T / G;       // every share holds at least this many tiles
          p.sk_max_parts = (int)((tiles + tmin - 1) / tmin + 1);
        }
      }
    }
  }
  return p;
}

// bytes of split partials the plan writes: float32 lse, then o in float32 (the larger dtype)
static size_t mla_workspace_bytes(int B, int Sq, int H, int k, bool row_stream) {
  if (B <= 0 || Sq <= 0 || H <= 0 || k <= 0) return 0;
  const MlaPlan p = mla_plan(B, Sq, H, k, row_stream);
  size_t rows;
  if (p.sk_groups > 0)
    rows = (size_t)((H + 63) / 64) * (p.sk_groups + (size_t)B * Sq) * 64;
  else if (p.splits > 1)
    rows = (size_t)B * Sq * p.splits * H;
  else
    return 0;
  return rows * (kVDim + 1) * sizeof(float);
}

}  // namespace dsa

extern "C" size_t dsa_sparse_mla_workspace_size(int B, int Sq, int H, int k) {
  return dsa::mla_workspace_bytes(B, Sq, H, k, true);
}

namespace dsa {
struct MlaUnion {
  const int32_t* counts = nullptr;
  const uint32_t* member = nullptr;
  int fold_h = 0, fold_sq = 0, mwords = 0;
};
static dsa_status_t mla_decode_impl(const void* q, const int32_t* idx, const dsa_rows_t* rows, int B, int Sq, int H,
                                    int k, float scale, void* o, dsa_dtype_t o_dtype, float* lse, void* ws,
                                    size_t ws_bytes, int32_t* err_count, hipStream_t stream, const MlaUnion& un);
}  // namespace dsa

extern "C" dsa_status_t dsa_sparse_mla_decode(const void* q, const int32_t* idx, const dsa_rows_t* rows, int B, int Sq,
                                              int H, int k, float scale, void* o, dsa_dtype_t o_dtype, float* lse,
                                              void* ws, size_t ws_bytes, int32_t* err_count, hipStream_t stream) {
  return dsa::mla_decode_impl(q, idx, rows, B, Sq, H, k, scale, o, o_dtype, lse, ws, ws_bytes, err_count, stream,
                              dsa::MlaUnion{});
}

extern "C" size_t dsa_sparse_mla_union_workspace_size(int B, int Sq, int H, int U) {
  if (B <= 0 || Sq <= 0 || H <= 0 || U <= 0 || (int64_t)Sq * H > (1 << 20)) return 0;
  return dsa::mla_workspace_bytes(B, 1, Sq * H, U, false);
}

extern "C" dsa_status_t dsa_sparse_mla_decode_union(const void* q, const int32_t* uni, const int32_t* count,
                                                    const uint32_t* member, const dsa_rows_t* rows, int B, int Sq,
                                                    int H, int U, float scale, void* o, dsa_dtype_t o_dtype,
                                                    float* lse, void* ws, size_t ws_bytes, int32_t* err_count,
                                                    hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && H >= 1 && U >= 1, "dsa_sparse_mla_decode_union: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(member, "dsa_sparse_mla_decode_union: null member");
  DSA_CHECK_SUPPORTED(H % 16 == 0 && (int64_t)Sq * H <= (1 << 20),
                      "dsa_sparse_mla_decode_union: needs H %% 16 == 0 and Sq * H <= 2^20");
  MlaUnion un;
  un.counts = count;
  un.member = member;
  un.fold_h = H;
  un.fold_sq = Sq;
  un.mwords = (U + 31) / 32;
  // query tokens folded into the head axis: one row of Sq * H heads per request
  return mla_decode_impl(q, uni, rows, B, 1, Sq * H, U, scale, o, o_dtype, lse, ws, ws_bytes, err_count, stream, un);
}

static dsa_status_t dsa::mla_decode_impl(const void* q, const int32_t* idx, const dsa_rows_t* rows, int B, int Sq,
                                         int H, int k, float scale, void* o, dsa_dtype_t o_dtype, float* lse,
                                         void* ws, size_t ws_bytes, int32_t* err_count, hipStream_t stream,
                                         const MlaUnion& un) {
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
  DSA_CHECK_SUPPORTED(rows->num_rows < ((int64_t)1 << 31), "dsa_sparse_mla_decode: num_rows must be below 2^31");
  DSA_CHECK_SUPPORTED((int64_t)B * Sq * ((H + 15) / 16) <= (1 << 24),
                      "dsa_sparse_mla_decode: more than 2^24 (query row, 16-head group) pairs");
  const bool row_stream = un.counts == nullptr;
  const MlaPlan plan = mla_plan(B, Sq, H, k, row_stream);
  const int splits = plan.splits;
  const int QR = B * Sq;
  const int nw = mla_waves(H);
  const int nhb = (H + 16 * nw - 1) / (16 * nw);
  const int64_t blocks = plan.sk_groups > 0 ? (int64_t)nhb * plan.sk_groups : (int64_t)splits * QR * nhb;
  // the launch's work-items (blocks x threads) must fit the 32-bit grid size
  DSA_CHECK_SUPPORTED(blocks * 128 * nw < ((int64_t)1 << 32),
                      "dsa_sparse_mla_decode: %lld work-groups exceed one launch", (long long)blocks);
  const size_t need = mla_workspace_bytes(B, Sq, H, k, row_stream);
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
  a.per_split = plan.per_split;
  a.scale_log2 = scale * kLog2e;
  a.o = o;
  a.o_f32 = (o_dtype == DSA_F32);
  a.lse = lse;
  a.err = err_count;
  a.counts = un.counts;
  a.member = un.member;
  a.fold_h = un.fold_h;
  a.fold_sq = un.fold_sq;
  a.mwords = un.mwords;
  a.QR = QR;
  a.sk_groups = plan.sk_groups;
  a.sk_tpu = plan.sk_tpu;
  const bool merged = plan.sk_groups > 0 || splits > 1;
  if (merged) {
    const size_t part_rows = plan.sk_groups > 0 ? (size_t)nhb * (plan.sk_groups + (size_t)QR) * 64
                                                : (size_t)QR * splits * H;
    a.part_lse = static_cast<float*>(ws);
    a.part_o = a.part_lse + part_rows;
  }
  const dim3 grid((unsigned)blocks);
  if (nw == 4 && plan.sk_groups > 0)
    DSA_LAUNCH(mla_roles_kernel<true>, grid, dim3(512), 0, stream, a);
  else if (nw == 4)
    DSA_LAUNCH(mla_roles_kernel<false>, grid, dim3(512), 0, stream, a);
  else if (nw == 2)
    DSA_LAUNCH((mla_decode_kernel<2, 2>), grid, dim3(256), 0, stream, a);
  else
    DSA_LAUNCH((mla_decode_kernel<1, 2>), grid, dim3(128), 0, stream, a);
  dsa_status_t st = launch_status("dsa_sparse_mla_decode");
  if (st != DSA_OK || !merged) return st;
  const dim3 mgrid((unsigned)(((H + kMergeHeads - 1) / kMergeHeads) * QR));
  const dim3 mblock(64 * kMergeHeads);
  // float32 partials take twice the registers per part: up to kMergeUnrolledF32 parts unrolled
  if (plan.sk_groups > 0) {
    if (a.o_f32 && plan.sk_max_parts <= kMergeUnrolledF32)
      DSA_LAUNCH((mla_merge_kernel<kMergeUnrolledF32, true, true>), mgrid, mblock, 0, stream, a);
    else if (a.o_f32)
      DSA_LAUNCH((mla_merge_kernel<0, true, true>), mgrid, mblock, 0, stream, a);
    else if (plan.sk_max_parts <= kMergeUnrolled)
      DSA_LAUNCH((mla_merge_kernel<kMergeUnrolled, false, true>), mgrid, mblock, 0, stream, a);
    else
      DSA_LAUNCH((mla_merge_kernel<0, false, true>), mgrid, mblock, 0, stream, a);
  } else {
    if (a.o_f32 && splits <= kMergeUnrolledF32)
      DSA_LAUNCH((mla_merge_kernel<kMergeUnrolledF32, true, false>), mgrid, mblock, 0, stream, a);
    else if (a.o_f32)
      DSA_LAUNCH((mla_merge_kernel<0, true, false>), mgrid, mblock, 0, stream, a);
    else if (splits <= kMergeUnrolled)
      DSA_LAUNCH((mla_merge_kernel<kMergeUnrolled, false, false>), mgrid, mblock, 0, stream, a);
    else
      DSA_LAUNCH((mla_merge_kernel<0, false, false>), mgrid, mblock, 0, stream, a);
  }
  return launch_status("dsa_sparse_mla_decode(merge)");
}

namespace dsa {

// Merge of R partial attention results over disjoint row sets (the ranks of a page-sharded
// cache, TokenSpeed audit page "MLA": split-KV partials combined by LSE rescaling; HiCache
// page §1.1: each rank holds and attends over its own pages only).  64 threads per output
// row n, 8 values per thread per pass.  Parts are [R, N, V] (the layout an all-gather of the
// ranks' outputs produces); PF32 / OF32: float32 parts / output, else bf16.
template <bool PF32, bool OF32>
__global__ void __launch_bounds__(256) rank_merge_kernel(const void* parts, const float* plse, int R, int64_t N,
                                                          int V, void* o, float* lse) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int lane = threadIdx.x & 63;
  float mx = -INFINITY;
  for (int r = 0; r < R; ++r) mx = fmaxf(mx, plse[(int64_t)r * N + n]);
  float wsum = 0.0f;
  if (mx > -INFINITY)
    for (int r = 0; r < R; ++r) {
      const float l = plse[(int64_t)r * N + n];
      wsum += (l == -INFINITY) ? 0.0f : expf(l - mx);
    }
  const float inv = (mx > -INFINITY) ? 1.0f / wsum : 0.0f;
  for (int d = lane * 8; d < V; d += 512) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (mx > -INFINITY)
      for (int r = 0; r < R; ++r) {
        const float l = plse[(int64_t)r * N + n];
        if (l == -INFINITY) continue;
        const float w = expf(l - mx) * inv;
        const int64_t off = ((int64_t)r * N + n) * V + d;
        if constexpr (PF32) {
          const f32x4 v0 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(parts) + off);
          const f32x4 v1 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(parts) + off + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[i] += w * v0[i];
            acc[4 + i] += w * v1[i];
          }
        } else {
          const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(parts) + off);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[2 * i] += w * __uint_as_float(v[i] << 16);
            acc[2 * i + 1] += w * __uint_as_float(v[i] & 0xffff0000u);
          }
        }
      }
    const int64_t ob = n * V + d;
    if constexpr (OF32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(o) + ob) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(static_cast<float*>(o) + ob + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(o) + ob) =
          u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                pack_bf16x2(acc[6], acc[7])};
    }
  }
  if (lane == 0) lse[n] = (mx > -INFINITY) ? mx + logf(wsum) : -INFINITY;
}

}  // namespace dsa

extern "C" dsa_status_t dsa_merge_partials(const void* o_parts, dsa_dtype_t part_dtype, const float* lse_parts, int R,
                                           int64_t N, int V, void* o, dsa_dtype_t o_dtype, float* lse,
                                           hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(R >= 1 && N >= 0 && V >= 8 && V % 8 == 0, "dsa_merge_partials: bad sizes");
  if (N == 0) return DSA_OK;
  DSA_CHECK_ARG(o_parts && lse_parts && o && lse, "dsa_merge_partials: null pointer");
  DSA_CHECK_ARG(((uintptr_t)o_parts & 15) == 0 && ((uintptr_t)o & 15) == 0,
                "dsa_merge_partials: o_parts and o must be 16-byte aligned");
  DSA_CHECK_ARG((part_dtype == DSA_F32 || part_dtype == DSA_BF16) && (o_dtype == DSA_F32 || o_dtype == DSA_BF16),
                "dsa_merge_partials: dtypes must be F32 or BF16");
  DSA_CHECK_SUPPORTED((N + 3) / 4 < ((int64_t)1 << 31) && (int64_t)R * N < ((int64_t)1 << 40),
                      "dsa_merge_partials: N too large for one launch");
  const dim3 grid((unsigned)((N + 3) / 4)), block(256);
  const bool pf = part_dtype == DSA_F32, of = o_dtype == DSA_F32;
  if (pf && of)
    DSA_LAUNCH((rank_merge_kernel<true, true>), grid, block, 0, stream, o_parts, lse_parts, R, N, V, o, lse);
  else if (pf)
    DSA_LAUNCH((rank_merge_kernel<true, false>), grid, block, 0, stream, o_parts, lse_parts, R, N, V, o, lse);
  else if (of)
    DSA_LAUNCH((rank_merge_kernel<false, true>), grid, block, 0, stream, o_parts, lse_parts, R, N, V, o, lse);
  else
    DSA_LAUNCH((rank_merge_kernel<false, false>), grid, block, 0, stream, o_parts, lse_parts, R, N, V, o, lse);
  return launch_status("dsa_merge_partials");
}

// ---------------------------------------------------------------------------------------------
// dsa_sparse_mla_decode_noalloc: the same kernels with their split partials in a scratch array
// of the library instead of a caller workspace, for callers that cannot allocate.  Host code
// never names `scratch` itself (its host-side symbol is a stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, once per device, with that device current.
namespace dsa {

constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

static std::atomic<void*> g_scratch_by_dev[kMaxDevices];

// device address of this device's scratch array, or nullptr (error text set)
static void* scratch_for_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_last_error("dsa_sparse_mla_decode_noalloc: no current device below %d (%s)", kMaxDevices,
                   hipGetErrorString(e));
    return nullptr;
  }
  void* p = g_scratch_by_dev[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // concurrent first calls on one device both obtain the same address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_last_error("dsa_sparse_mla_decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_by_dev[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace dsa

extern "C" size_t dsa_sparse_mla_noalloc_max_workspace(void) { return dsa::kNoAllocScratchBytes; }

extern "C" dsa_status_t dsa_sparse_mla_decode_noalloc(const void* q, const int32_t* idx, const dsa_rows_t* rows,
                                                      int B, int Sq, int H, int k, float scale, void* o,
                                                      dsa_dtype_t o_dtype, float* lse, int32_t* err_count,
                                                      hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && H >= 1 && k >= 1, "dsa_sparse_mla_decode_noalloc: bad sizes");
  if (B == 0) return DSA_OK;
  const size_t need = dsa_sparse_mla_workspace_size(B, Sq, H, k);
  DSA_CHECK_SUPPORTED(need <= kNoAllocScratchBytes,
                      "dsa_sparse_mla_decode_noalloc: needs %zu bytes of split partials, above the %zu-byte "
                      "scratch array (use dsa_sparse_mla_decode with a workspace)",
                      need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_for_current_device();
    if (ws == nullptr) return DSA_ERR_HIP;
  }
  return dsa_sparse_mla_decode(q, idx, rows, B, Sq, H, k, scale, o, o_dtype, lse, ws, need, err_count, stream);
}
