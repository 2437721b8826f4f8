// Sparse MLA decode over the selected rows (TokenSpeed audit page, "MLA
// (tokenspeed-mla)": one 576-wide latent row per token is both key (all 576 values)
// and value (the first 512); "Shared-Indexer KV Cache Offload for GLM-5.2", §2.1:
// attention reads only the top-k positions).  Split-KV decode with fp32 partial
// (o, lse) and an LSE-rescaling merge (TokenSpeed audit, two-stage split-KV decode).
//
// Work-group = 2*HG waves (one per SIMD) for 32*HG heads of one query row and one split
// of its selected rows.  Wave (hg, half) owns heads [32hg, 32hg+32) and
//   S^T[32 tokens x 32 heads] partial = K_tile[:, half] . q^T[half]   (bf16 MFMA 32x32x16,
//     18 steps over its 288 of the 576 latent dims, q^T resident in VGPRs); the two
//     halves of a head group swap partial S^T through LDS and both hold the full sum;
//   O^T[256 dims x 32 heads] += V^T[half] . P^T                        (bf16 MFMA 32x32x16)
//     over its 256 of the 512 value dims.  Heads sit on the N axis, so each lane owns one
//     head's running max / sum and the rescale is a per-lane scalar; P^T is the S^T
//     accumulator itself (rounded to bf16), and V^T is written to LDS in the token order
//     that layout implies.
// The K tile is double-buffered in LDS; the next tile's rows are loaded into registers
// while the current one is computed.
// Online softmax in base 2 with a lazy rescale (the running max is only moved when it
// grows by more than 2^8), which leaves o and lse mathematically unchanged.
#include "common.h"

namespace dsa {

constexpr int kRowEl = 576;                 // latent 512 + rope 64
constexpr int kVDim = 512;
constexpr int kRowBytes = kRowEl * 2;
constexpr int kTT = 32;                     // tokens per tile
constexpr int kChunks = kRowBytes / 16;     // 72 x 16 B per row
constexpr int kTileChunks = kTT * kChunks;  // 2304
constexpr int kKStride = kRowEl + 8;        // K tile row stride (bf16), 1168 B
constexpr int kVStride = kTT + 8;           // V^T row stride (bf16), 80 B
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
  float* part_o;           // [QR, splits, H, 512]                    -- splits > 1
  float* part_lse;         // [QR, splits, H]
  int32_t* err;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

template <int HG>
__global__ void __launch_bounds__(128 * HG, 1) mla_decode_kernel(MlaArgs a) {
  constexpr int NW = 2 * HG;
  constexpr int NT = 64 * NW;
  constexpr int CPT = (kTileChunks + NT - 1) / NT;      // 16-byte chunks per thread per tile
  __shared__ __attribute__((aligned(16))) uint16_t klds[2][kTT * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kVDim * kVStride];
  __shared__ __attribute__((aligned(16))) float xch[NW][16][64];      // partial S^T exchange
  __shared__ int64_t rowoff[kMaxSplit];  // byte offset of each selected row of the split, -1 = none
  __shared__ int tvalid[2][kTT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hg = wave >> 1, half = wave & 1;
  const int n = lane & 31, g = lane >> 5;
  const int nhb = (a.H + 32 * HG - 1) / (32 * HG);
  const int qr = blockIdx.y / nhb;
  const int hb = blockIdx.y % nhb;
  const int b = qr / a.Sq;
  const int split = blockIdx.x;
  const int head = hb * 32 * HG + hg * 32 + n;
  const bool head_ok = head < a.H;

  const int e_begin = split * a.per_split;
  int e_end = e_begin + a.per_split;
  if (e_end > a.k) e_end = a.k;
  const int32_t* idx = a.idx + (int64_t)qr * a.k;

  // resolve every selected row of this split once: index -> page table -> byte offset
  for (int e = e_begin + tid; e < e_end; e += NT) {
    const int32_t p = idx[e];
    const int64_t row = a.rows.row(b, p);
    if (row < 0 && p >= 0) count_error(a.err);
    rowoff[e - e_begin] = row >= 0 ? row * kRowBytes : -1;
  }
  for (int e = e_end + tid; e < e_begin + a.per_split && e - e_begin < kMaxSplit; e += NT) rowoff[e - e_begin] = -1;
  __syncthreads();

  u32x4 stage[CPT];
  auto load_tile = [&](int e0) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + NT * r;
      stage[r] = u32x4{0, 0, 0, 0};
      if (c < kTileChunks) {
        const int tok = c / kChunks, ch = c - tok * kChunks;
        const int64_t off = rowoff[e0 - e_begin + tok];
        if (off >= 0) stage[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.rows.base + off) + ch);
      }
    }
  };
  auto store_tile = [&](int bf, int e0) {
#pragma unroll
    for (int r = 0; r < CPT; ++r) {
      const int c = tid + NT * r;
      if (c < kTileChunks) {
        const int tok = c / kChunks, ch = c - tok * kChunks;
        *reinterpret_cast<u32x4*>(&klds[bf][tok * kKStride + ch * 8]) = stage[r];
      }
    }
    if (tid < kTT) tvalid[bf][tid] = rowoff[e0 - e_begin + tid] >= 0;
  };

  // ---- prologue: tile 0 into K buffer 0
  if (e_begin < e_end) {
    load_tile(e_begin);
    store_tile(0, e_begin);
  }

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

  f32x16 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x16{};
  float m_used = -INFINITY;     // log2-domain running max used for p
  float l_part = 0.0f;          // this lane's share of sum p (fp32 p: for lse)
  float lr_part = 0.0f;         // this lane's share of sum bf16(p) (the PV weights: for o)

  int cur = 0;
  for (int e0 = e_begin; e0 < e_end; e0 += kTT, cur ^= 1) {
    const bool has_next = e0 + kTT < e_end;
    __syncthreads();              // K[cur] ready; V^T, xch and K[cur^1] free

    // ---- V^T from K[cur]: 8 tokens x 8 dims blocks, transposed through registers
    for (int blk = tid; blk < 4 * (kVDim / 8); blk += NT) {
      const int grp = blk & 3, db = blk >> 2;        // token group (ks, gg), dim block
      const int ks = grp >> 1, gg = grp & 1;
      u32x4 r8[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int tok = ks * 16 + (s >> 2) * 8 + gg * 4 + (s & 3);
        r8[s] = *reinterpret_cast<const u32x4*>(&klds[cur][tok * kKStride + db * 8]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;   // high or low halves
        u32x4 ov;
        ov.x = __builtin_amdgcn_perm(r8[1][w], r8[0][w], sel);
        ov.y = __builtin_amdgcn_perm(r8[3][w], r8[2][w], sel);
        ov.z = __builtin_amdgcn_perm(r8[5][w], r8[4][w], sel);
        ov.w = __builtin_amdgcn_perm(r8[7][w], r8[6][w], sel);
        *reinterpret_cast<u32x4*>(vt + (db * 8 + e) * kVStride + ks * 16 + gg * 8) = ov;
      }
    }
    if (has_next) load_tile(e0 + kTT);

    // ---- partial S^T over this wave's half of the latent dims; operand reads run ahead
    f32x16 s = f32x16{};
    {
      const uint16_t* kp = &klds[cur][n * kKStride + half * 288 + g * 8];
      bf16x8 ring[4];
#pragma unroll
      for (int j = 0; j < 3; ++j) ring[j] = *reinterpret_cast<const bf16x8*>(kp + j * 16);
#pragma unroll
      for (int j = 0; j < 18; ++j) {
        if (j + 3 < 18) ring[(j + 3) & 3] = *reinterpret_cast<const bf16x8*>(kp + (j + 3) * 16);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[j & 3], qb[j], s, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) xch[wave][i][lane] = s[i];
    __syncthreads();              // partial S^T of both halves and V^T ready
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] += xch[wave ^ 1][i][lane];

    // ---- online softmax for head n (tokens of lane group g)
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = (i >> 2) * 8 + g * 4 + (i & 3);
      const float x = tvalid[cur][tok] ? s[i] * a.scale_log2 : -INFINITY;
      s[i] = x;
      tmax = fmaxf(tmax, x);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool grow = tmax > m_used + kLazy || (m_used == -INFINITY && tmax > -INFINITY);
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? tmax : m_used;
      const float alpha = (m_used == -INFINITY) ? 0.0f : exp2f(m_used - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) oacc[i] *= alpha;
      l_part *= alpha;
      lr_part *= alpha;
      m_used = m_new;
    }
    uint32_t pb[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = (s[i] == -INFINITY) ? 0.0f : exp2f(s[i] - m_used);
      const float p1 = (s[i + 1] == -INFINITY) ? 0.0f : exp2f(s[i + 1] - m_used);
      const uint32_t w = pack_bf16x2(p0, p1);
      pb[i >> 1] = w;
      l_part += p0 + p1;
      lr_part += bf16_bits_to_f32(w & 0xffffu) + bf16_bits_to_f32(w >> 16);
    }
    const bf16x8 p_lo = __builtin_bit_cast(bf16x8, u32x4{pb[0], pb[1], pb[2], pb[3]});
    const bf16x8 p_hi = __builtin_bit_cast(bf16x8, u32x4{pb[4], pb[5], pb[6], pb[7]});

    // ---- O^T += V^T . P^T over this wave's 256 value dims; operand reads run ahead
    {
      const uint16_t* vp = vt + (half * 256 + n) * kVStride + g * 8;
      auto vop = [&](int i) {   // i = 2*mt + ks
        return *reinterpret_cast<const bf16x8*>(vp + (i >> 1) * 32 * kVStride + (i & 1) * 16);
      };
      bf16x8 ring[4];
#pragma unroll
      for (int i = 0; i < 3; ++i) ring[i] = vop(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + 3 < 16) ring[(i + 3) & 3] = vop(i + 3);
        oacc[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i & 3], (i & 1) ? p_hi : p_lo, oacc[i >> 1], 0,
                                                               0, 0);
      }
    }

    if (has_next) store_tile(cur ^ 1, e0 + kTT);
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
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4*>(a.part_o + obase + mt * 32 + i4 * 8 + g * 4) =
            f32x4{oacc[mt][i4 * 4 + 0] * inv, oacc[mt][i4 * 4 + 1] * inv, oacc[mt][i4 * 4 + 2] * inv,
                  oacc[mt][i4 * 4 + 3] * inv};
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

// merge of split partials: one work-group of 128 threads per (query row, head)
__global__ void __launch_bounds__(128) mla_merge_kernel(MlaArgs a) {
  const int qr = blockIdx.y, head = blockIdx.x;
  const int S = a.splits;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, a.part_lse[((int64_t)qr * S + s) * a.H + head]);
  float wsum = 0.0f;
  f32x4 acc = {0, 0, 0, 0};
  const int d = threadIdx.x * 4;
  if (mx > -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const int64_t pb = ((int64_t)qr * S + s) * a.H + head;
      const float l = a.part_lse[pb];
      if (l == -INFINITY) continue;
      const float w = __expf(l - mx);
      wsum += w;
      const f32x4 v = *reinterpret_cast<const f32x4*>(a.part_o + pb * kVDim + d);
      acc += w * v;
    }
    acc *= 1.0f / wsum;
  }
  const int64_t ob = ((int64_t)qr * a.H + head) * kVDim + d;
  if (a.o_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + ob) = acc;
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + ob) =
        u32x2{pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w)};
  }
  if (threadIdx.x == 0) a.lse[(int64_t)qr * a.H + head] = (mx > -INFINITY) ? mx + __logf(wsum) : -INFINITY;
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
    a.part_o = static_cast<float*>(ws);
    a.part_lse = a.part_o + (size_t)B * Sq * splits * H * kVDim;
  }
  const int QR = B * Sq;
  if (H > 32) {
    hipLaunchKernelGGL(mla_decode_kernel<2>, dim3(splits, QR * ((H + 63) / 64)), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(mla_decode_kernel<1>, dim3(splits, QR), dim3(128), 0, stream, a);
  }
  dsa_status_t st = launch_status("dsa_sparse_mla_decode");
  if (st != DSA_OK || splits == 1) return st;
  hipLaunchKernelGGL(mla_merge_kernel, dim3(H, QR), dim3(128), 0, stream, a);
  return launch_status("dsa_sparse_mla_decode(merge)");
}
