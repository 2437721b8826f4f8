"""KV write path of one decode step, for the oracle (test infrastructure only).

The TokenSpeed engine audit page, section "Attention integration / KV host tiering",
lists a fused FP8 KV-pack kernel that quantizes the new token's entries and scatter-
writes them into the paged caches in one launch, and (section "MLA (tokenspeed-mla)")
one 576-wide latent row per token.  The pages do not fix the key quantization; the
reading taken here is the per-token scale of the indexer-cache layout the rest of the
path reads ("Shared-Indexer KV Cache Offload for GLM-5.2", §2.1: fp8 indexer keys):

    sigma = max_d |k_d| / 448            (float32 division; 448 = largest e4m3 value)
    code_d = e4m3(k_d / sigma)           (float32 division, then nearest e4m3, ties to even)
    a zero key stores sigma = 0 and all-zero codes.

With the FP4 indexer cache (read as OCP MXFP4, as the indexer oracle does) the key is
instead quantized per block of 32 dimensions, following the OCP MX conversion: the shared
exponent is floor(log2(max |k| of the block)) - 2 (2 being the exponent of E2M1's largest
value, 6 = 1.5 * 2^2), clamped to the E8M0 range, so the scale is X = 2^(that exponent);
each element is k / X rounded to the nearest E2M1 value, ties to even, with magnitudes
above 6 saturated to 6.  An all-zero block stores scale code 0 and zero codes.

The latent row is stored unchanged (bf16).  The Sq new tokens of request b occupy its
last Sq positions, seq_lens[b] - Sq + t, and go to the paged row of that position.
"""
import numpy as np

from .formats import MX_BLOCK, bf16_to_f64, f64_to_e4m3_codes

E4M3_MAX = np.float32(448.0)


def quantize_key(k) -> tuple:
    """One key row (float32 values) -> (e4m3 codes uint8, sigma float32)."""
    k = np.asarray(k, dtype=np.float32)
    amax = np.max(np.abs(k)).astype(np.float32)
    if amax == 0:
        return np.zeros(k.shape, dtype=np.uint8), np.float32(0.0)
    sigma = np.float32(amax / E4M3_MAX)
    x = (k / sigma).astype(np.float32)
    return f64_to_e4m3_codes(x.astype(np.float64)), sigma


# E2M1 magnitude (times 2) -> code, for the values 0, 0.5, 1, 1.5, 2, 3, 4, 6
_E2M1_CODE = {0: 0, 1: 1, 2: 2, 3: 3, 4: 4, 6: 5, 8: 6, 12: 7}


def e2m1_round(y: float) -> int:
    """float y -> E2M1 code: nearest value, ties to even, magnitudes above 6 saturate.

    Rounding counts quanta: below 2 the spacing is 0.5, in [2, 4) it is 1 and in [4, 6]
    it is 2; round-half-even on the count gives the even mantissa at ties.
    """
    a = abs(float(y))
    if a >= 6.0:
        mag2 = 12
    else:
        e = max(int(np.floor(np.log2(a))), 0) if a > 0 else 0
        quantum = 2.0 ** (e - 1)
        mag = float(np.rint(a / quantum)) * quantum
        mag2 = min(int(mag * 2), 12)
    code = _E2M1_CODE[mag2]
    return code | (8 if np.signbit(y) else 0)


def quantize_key_mxfp4(k) -> tuple:
    """One key row (float32, D a multiple of 32) -> (packed codes uint8 [D/2], E8M0 scales
    uint8 [D/32]); element 2i is the low nibble of byte i."""
    k = np.asarray(k, dtype=np.float32)
    D = k.shape[0]
    assert D % MX_BLOCK == 0
    codes = np.zeros(D, dtype=np.uint8)
    scales = np.zeros(D // MX_BLOCK, dtype=np.uint8)
    for j in range(D // MX_BLOCK):
        blk = k[j * MX_BLOCK:(j + 1) * MX_BLOCK]
        amax = float(np.max(np.abs(blk)))
        if amax == 0.0:
            continue                                   # scale code 0, zero codes
        shared = int(np.floor(np.log2(amax))) - 2
        code = min(max(shared + 127, 0), 254)
        X = np.float32(2.0 ** (code - 127))
        y = (blk / X).astype(np.float32)               # exact: X is a power of two
        scales[j] = code
        codes[j * MX_BLOCK:(j + 1) * MX_BLOCK] = [e2m1_round(v) for v in y]
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    return packed, scales


def kv_write(latent_bits, idx_k, seq_lens, page_table, page_size: int, kv, icache, iscale, cache="e4m3"):
    """Write the new tokens of every request into copies of the caches.

    latent_bits [B, Sq, 576] uint16 (bf16 bits); idx_k [B, Sq, D] float32 or uint16 bf16
    bits; page_table [B, P] int32; kv [rows, 576] uint16.  cache "e4m3": icache [rows, D]
    uint8 codes, iscale [rows] float32; cache "mxfp4": icache [rows, D/2] uint8 packed
    codes, iscale [rows, D/32] uint8 E8M0 scales.  Returns (kv, icache, iscale, errors): a
    token whose position is negative, past its page-table row, on a negative page id, or
    past the caches' rows is skipped and counted.
    """
    kv, icache, iscale = kv.copy(), icache.copy(), iscale.copy()
    B, Sq = latent_bits.shape[:2]
    keys = idx_k if idx_k.dtype == np.float32 else bf16_to_f64(idx_k).astype(np.float32)
    errors = 0
    for b in range(B):
        for t in range(Sq):
            p = int(seq_lens[b]) - Sq + t
            lp = p // page_size if p >= 0 else -1
            pg = int(page_table[b, lp]) if 0 <= lp < page_table.shape[1] else -1
            row = pg * page_size + p % page_size if pg >= 0 else -1
            if row < 0 or row >= kv.shape[0] or row >= icache.shape[0]:
                errors += 1
                continue
            kv[row] = latent_bits[b, t]
            if cache == "mxfp4":
                icache[row], iscale[row] = quantize_key_mxfp4(keys[b, t])
            else:
                icache[row], iscale[row] = quantize_key(keys[b, t])
    return kv, icache, iscale, errors
