// KV write path of one decode step: the new tokens' entries are quantized and scattered
// into the paged caches in one launch (TokenSpeed engine audit page, "Attention
// integration / KV host tiering": a fused FP8 KV-pack kernel; "MLA (tokenspeed-mla)": one
// 576-wide latent row per token; "Shared-Indexer KV Cache Offload for GLM-5.2", §2.1: fp8
// indexer keys).
//
// One wave per new token (b, t), at position p = seq_lens[b] - Sq + t:
//   * the bf16 latent row (1152 bytes) is copied to its paged row of the KV cache;
//   * the indexer key (D values, bf16 or fp32) is quantized with one scale per token,
//       sigma = max_d |k_d| / 448,   code_d = e4m3(k_d / sigma)   (float32 divisions;
//       e4m3 = nearest OCP E4M3FN value, ties to even, saturating at 448),
//     and written with sigma to its paged row of the indexer cache (a zero key stores
//     sigma = 0 and zero codes);
//   * or, for the FP4 indexer cache (read as OCP MXFP4), quantized per block of 32
//     dimensions following the OCP MX conversion: E8M0 scale code = floor(log2(block
//     max |k|)) - 2 + 127 clamped to 0..254 (0 for a zero block), elements = nearest E2M1
//     value of k / 2^(code - 127), ties to the even mantissa, saturating at 6; the codes go
//     two per byte (element 2i in the low nibble) with the four scale codes beside them.
#include "common.h"

namespace dsa {

constexpr int kLatentBytes = 576 * 2;

// float32 -> OCP E4M3FN code: nearest finite value, ties to the even code, |x| >= 448
// saturating to 448; -0.0 and negative values that round to zero keep the sign bit.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e00000u) {                          // |x| >= 448
    code = 0x7eu;
  } else if (a >= 0x3c800000u) {                   // |x| >= 2^-6: normal, exponent bias 7
    const uint32_t q = ((((a >> 23) - 127u + 7u) << 3) | ((a >> 20) & 7u));
    const uint32_t rem = a & 0xfffffu;              // the 20 mantissa bits dropped
    const uint32_t r = q + ((rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u);
    code = r > 0x7eu ? 0x7eu : r;                    // a carry moves into the exponent field
  } else {                                          // below 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling; 8 is 2^-6
  }
  return sign | code;
}

// float32 -> E2M1 code: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even mantissa,
// magnitudes above 6 saturating; the sign bit is kept (also for values that round to 0).
// Each comparison passes one boundary between neighbouring values; at a boundary that is a
// tie the comparison is strict when the lower neighbour has the even mantissa.
__device__ __forceinline__ uint32_t e2m1_encode(float x) {
  const float a = fabsf(x);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

struct KvWriteArgs {
  const uint16_t* latent;      // [B, Sq, 576] bf16
  const void* key;             // [B, Sq, D] bf16 or fp32
  int key_f32;
  const int32_t* seq_lens;     // [B]
  int B, Sq, D;
  RowStore kv;                 // 1152-byte latent rows (written)
  RowStore ic;                 // D-byte e4m3 rows or D/2-byte MXFP4 rows (written)
  void* iscale;                // e4m3: float per row; MXFP4: D/32 E8M0 bytes per row (written)
  int32_t* err;
};

template <bool FP4>
__global__ void __launch_bounds__(256) kv_write_kernel(KvWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (tok >= a.B * a.Sq) return;
  const int b = tok / a.Sq, t = tok - b * a.Sq;
  const int64_t pos = (int64_t)a.seq_lens[b] - a.Sq + t;
  const int64_t rk = a.kv.row(b, pos), ri = a.ic.row(b, pos);
  if (rk < 0 || ri < 0) {
    if (lane == 0) count_error(a.err);
    return;
  }
  // latent row: 72 chunks of 16 bytes
  const u32x4* src = reinterpret_cast<const u32x4*>(a.latent + (int64_t)tok * 576);
  u32x4* dst = reinterpret_cast<u32x4*>(const_cast<char*>(a.kv.base) + rk * kLatentBytes);
  dst[lane] = src[lane];
  if (lane < kLatentBytes / 16 - 64) dst[64 + lane] = src[64 + lane];
  // key: lane i holds values 2i, 2i+1 (D <= 128, even)
  const bool live = 2 * lane < a.D;
  float k0 = 0.0f, k1 = 0.0f;
  if (live) {
    if (a.key_f32) {
      const f32x2 v = reinterpret_cast<const f32x2*>(static_cast<const float*>(a.key) + (int64_t)tok * a.D)[lane];
      k0 = v.x;
      k1 = v.y;
    } else {
      const uint32_t v = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.key) + (int64_t)tok * a.D)[lane];
      k0 = __uint_as_float(v << 16);
      k1 = __uint_as_float(v & 0xffff0000u);
    }
  }
  float amax = fmaxf(fabsf(k0), fabsf(k1));
  if constexpr (FP4) {
    // block j = dimensions [32j, 32j + 32) = lanes [16j, 16j + 16)
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const int eb = (int)((__float_as_uint(amax) >> 23) & 0xffu);   // floor(log2 amax) + 127 if normal
    const uint32_t code = (uint32_t)min(max(eb - 2, 0), 254);        // 0 for zero / tiny blocks
    const float X = __uint_as_float(code ? (code << 23) : 0x00400000u);
    const uint32_t byte = e2m1_encode(k0 / X) | (e2m1_encode(k1 / X) << 4);
    char* row = const_cast<char*>(a.ic.base) + ri * (a.D / 2);
    if (live) reinterpret_cast<uint8_t*>(row)[lane] = (uint8_t)byte;
    if ((lane & 15) == 0 && 2 * lane < a.D)
      static_cast<uint8_t*>(a.iscale)[ri * (a.D / 32) + (lane >> 4)] = (uint8_t)code;
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float sigma = amax / 448.0f;
    uint32_t pair = 0;
    if (amax > 0.0f) pair = e4m3_encode(k0 / sigma) | (e4m3_encode(k1 / sigma) << 8);
    if (live)
      reinterpret_cast<uint16_t*>(const_cast<char*>(a.ic.base) + ri * a.D)[lane] = (uint16_t)pair;
    if (lane == 0) static_cast<float*>(a.iscale)[ri] = sigma;
  }
}

}  // namespace dsa

extern "C" dsa_status_t dsa_kv_write(const void* latent, const void* idx_k, dsa_dtype_t idx_k_dtype,
                                     const int32_t* seq_lens, int B, int Sq, int D, const dsa_rows_t* kv,
                                     const dsa_rows_t* idx_cache, dsa_dtype_t idx_cache_dtype, void* idx_scale,
                                     int32_t* err_count, hipStream_t stream) {
  using namespace dsa;
  DSA_CHECK_ARG(B >= 0 && Sq >= 1 && D >= 2, "dsa_kv_write: bad sizes");
  if (B == 0) return DSA_OK;
  DSA_CHECK_ARG(latent && idx_k && seq_lens && kv && idx_cache && kv->base && idx_cache->base && idx_scale,
                "dsa_kv_write: null pointer");
  DSA_CHECK_ARG(idx_k_dtype == DSA_BF16 || idx_k_dtype == DSA_F32, "dsa_kv_write: idx_k must be BF16 or F32");
  DSA_CHECK_ARG(idx_cache_dtype == DSA_E4M3 || idx_cache_dtype == DSA_MXFP4,
                "dsa_kv_write: the indexer cache must be E4M3 or MXFP4");
  const bool fp4 = idx_cache_dtype == DSA_MXFP4;
  DSA_CHECK_SUPPORTED(D <= 128 && D % 2 == 0, "dsa_kv_write: needs an even D <= 128");
  if (fp4) DSA_CHECK_SUPPORTED(D % 32 == 0, "dsa_kv_write: MXFP4 needs D a multiple of 32");
  DSA_CHECK_ARG(kv->row_bytes == kLatentBytes, "dsa_kv_write: kv row_bytes must be 1152");
  DSA_CHECK_ARG(idx_cache->row_bytes == (fp4 ? D / 2 : D),
                "dsa_kv_write: indexer-cache row_bytes must be D (E4M3) or D/2 (MXFP4)");
  DSA_CHECK_ARG(((uintptr_t)latent & 15) == 0 && ((uintptr_t)kv->base & 15) == 0,
                "dsa_kv_write: latent and kv base must be 16-byte aligned");
  DSA_CHECK_ARG(((uintptr_t)idx_k & 7) == 0 && (fp4 || ((uintptr_t)idx_cache->base & 1) == 0),
                "dsa_kv_write: idx_k must be 8-byte and an E4M3 indexer cache 2-byte aligned");
  if (!fp4) DSA_CHECK_ARG(((uintptr_t)idx_scale & 3) == 0, "dsa_kv_write: idx_scale must be 4-byte aligned");
  if (kv->page_table) DSA_CHECK_ARG(kv->page_size > 0, "dsa_kv_write: bad kv page_size");
  if (idx_cache->page_table) DSA_CHECK_ARG(idx_cache->page_size > 0, "dsa_kv_write: bad indexer page_size");
  DSA_CHECK_ARG((int64_t)B * Sq <= ((int64_t)1 << 31) - 4, "dsa_kv_write: too many tokens");
  KvWriteArgs a{};
  a.latent = static_cast<const uint16_t*>(latent);
  a.key = idx_k;
  a.key_f32 = idx_k_dtype == DSA_F32;
  a.seq_lens = seq_lens;
  a.B = B;
  a.Sq = Sq;
  a.D = D;
  a.kv = RowStore::from(*kv);
  a.ic = RowStore::from(*idx_cache);
  a.iscale = idx_scale;
  a.err = err_count;
  const int tokens = B * Sq;
  if (fp4)
    DSA_LAUNCH(kv_write_kernel<true>, dim3((tokens + 3) / 4), dim3(256), 0, stream, a);
  else
    DSA_LAUNCH(kv_write_kernel<false>, dim3((tokens + 3) / 4), dim3(256), 0, stream, a);
  return launch_status("dsa_kv_write");
}
