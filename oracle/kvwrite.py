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

The latent row is stored unchanged (bf16).  The Sq new tokens of request b occupy its
last Sq positions, seq_lens[b] - Sq + t, and go to the paged row of that position.
"""
import numpy as np

from .formats import bf16_to_f64, f64_to_e4m3_codes

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


def kv_write(latent_bits, idx_k, seq_lens, page_table, page_size: int, kv, icache, iscale):
    """Write the new tokens of every request into copies of the caches.

    latent_bits [B, Sq, 576] uint16 (bf16 bits); idx_k [B, Sq, D] float32 or uint16 bf16
    bits; page_table [B, P] int32; kv [rows, 576] uint16; icache [rows, D] uint8;
    iscale [rows] float32.  Returns (kv, icache, iscale, errors): a token whose position
    is negative, past its page-table row, on a negative page id, or past the caches'
    rows is skipped and counted.
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
            icache[row], iscale[row] = quantize_key(keys[b, t])
    return kv, icache, iscale, errors
