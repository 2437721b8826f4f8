/*
 * libdsa — one decode step of DSA-style sparse attention on AMD MI355X (gfx950).
 *
 * The step (sources are web pages describing the method):
 *   [GLM52] "Shared-Indexer KV Cache Offload for GLM-5.2 on CANN" (lmnt.cn news 268566)
 *   [HCCP]  "HiCache across parallel modes and distributed serving" (dujian.net)
 *   [TSA]   TokenSpeed engine code audit (devpress.csdn.net, AMD channel)
 *   [GLM5R] Zhipu GLM-5 serving report (hkstock.com.hk news 808716)
 *
 *   dsa_indexer_scores     Lightning-Indexer scan over every visible cached token   [GLM52] §2.1
 *   dsa_topk               top-k positions per query (k = 2048 in the pages)        [GLM52] §2.1
 *   dsa_topk_union         de-duplicated union of a request's query selections     [GLM52] §4.2, §5.1
 *   dsa_plan               shared-group pool plan, set-associative FIFO            [GLM52] §3, §4.2-4.3, §5
 *   dsa_gather_kv          per-layer serve (pool / paged / host rows) and install  [GLM52] §4.4, §5
 *   dsa_sparse_mla_decode  MLA latent attention over the selected rows only        [TSA] "MLA", [GLM52] §2.1
 *   dsa_sparse_mla_decode_union  the same over the union, query tokens packed       [TSA] "MLA", [GLM52] §5.1
 *   dsa_merge_partials     LSE merge of per-rank (or per-split) partial attention  [TSA] "MLA", [HCCP] §1.1
 *   dsa_page_translate     page-sharded ownership closed form                      [HCCP] §1.1
 *   dsa_kv_write           new tokens' latent rows and e4m3 or MXFP4 indexer keys into the
 *                          paged caches (fused quantise + scatter)                 [TSA] "KV host tiering"
 *
 * Conventions shared by every call
 *   - Pointers are device pointers owned by the caller, unless stated otherwise.  The
 *     library never allocates memory: scratch space is a caller buffer sized by the
 *     matching *_workspace_size() call.
 *   - Every call only enqueues work on `stream` (a hipStream_t; 0 = the null stream)
 *     and returns; nothing synchronises.  There is no global mutable state, except the
 *     scratch array that dsa_sparse_mla_decode_noalloc uses instead of a workspace.
 *   - Argument checks that need no device access (null pointers, sizes, dtypes,
 *     alignment) happen before anything is enqueued and return DSA_ERR_INVALID_ARG or
 *     DSA_ERR_UNSUPPORTED; then nothing was enqueued.  A failed launch returns
 *     DSA_ERR_HIP, with the HIP error text in dsa_last_error() (thread-local).
 *   - Data-dependent indices (page ids, positions, slots) are checked on the device:
 *     an out-of-range entry is treated as absent (score -inf / row skipped / entry
 *     invalid, as each call states) and, if `err_count` is not NULL, one is added to
 *     *err_count (a device int32 the caller zeroes).  No kernel reads or writes
 *     outside the buffers described here.
 *   - Integer layouts are row-major C arrays; strides are in elements.
 */
#ifndef LIBDSA_DSA_H
#define LIBDSA_DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, dtype or alignment              */
  DSA_ERR_UNSUPPORTED = -2,  /* valid request outside what this library implements      */
  DSA_ERR_HIP = -3,          /* a HIP launch/runtime call failed; see dsa_last_error()   */
  DSA_ERR_WORKSPACE = -4     /* workspace pointer NULL or smaller than *_workspace_size  */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,   /* IEEE binary32                                            */
  DSA_BF16 = 1,  /* bfloat16 (upper half of binary32)                        */
  DSA_E4M3 = 2,  /* OCP FP8 E4M3FN (bias 7, max 448, no infinities)          */
  DSA_MXFP4 = 3  /* OCP MX FP4: E2M1 codes two per byte (element 2i in the    *
                  * low nibble of byte i) with one E8M0 scale byte 2^(c-127)  *
                  * per 32 elements, held in a separate scale array           */
} dsa_dtype_t;

/*
 * A per-token row store: the paged caches (indexer keys, latent KV rows), a device
 * pool, a dense selection buffer, or mapped pinned host memory.
 *
 * Paged (page_table != NULL): token `pos` of request b lives at physical row
 *     page_table[b * pt_stride + pos / page_size] * page_size + pos % page_size
 *   and physical page ids must lie in [0, num_rows / page_size).  Only the entries
 *   of pages that hold positions < the request's length are read.  (Page-table
 *   metadata kept apart from the physical rows: [TSA] "req_to_token_pool vs KV
 *   allocator".)
 * Dense (page_table == NULL): token `pos` of request b lives at row
 *     b * req_stride + pos,  which must be < num_rows.
 * Row r starts at (const char*)base + r * row_bytes.  `base` may be a device
 * pointer or a host pointer from hipHostMalloc(..., hipHostMallocMapped) (or its
 * device alias); it must be 16-byte aligned and row_bytes a multiple of 16.
 */
typedef struct {
  const void* base;
  int64_t num_rows;
  int32_t row_bytes;
  int32_t page_size;
  const int32_t* page_table;
  int32_t pt_stride;
  int32_t reserved;
  int64_t req_stride;
} dsa_rows_t;

/* Library version (major*10000 + minor*100 + patch). */
int dsa_version(void);

/* Text of the last DSA_ERR_HIP / DSA_ERR_INVALID_ARG on the calling thread ("" if none). */
const char* dsa_last_error(void);

/*
 * dsa_indexer_scores — Lightning-Indexer scan ([GLM52] §2.1: the indexer scores every
 * history token against the current query; the score is the ReLU-gated,
 * head-weighted dot product below).
 *
 *   score[b,t,s] = sum_h w[b,t,h] * max(0, sigma_s * sum_d q[b,t,h,d] * k[b,s,d])
 *
 * for s < vis(b,t) = seq_lens[b] - Sq + 1 + t  (query t of an MTP verify step sees the
 * history and the draft tokens up to its own), and -inf for vis(b,t) <= s < seq_lens[b].
 * Entries at s >= seq_lens[b] (up to score_stride) are not written.
 *
 *   q        [B, Sq, H, D]  dtype q_dtype (F32, BF16 or E4M3)
 *   w        [B, Sq, H]     float32 head weights
 *   keys     row store of keys: row_bytes = D * sizeof(k_dtype) for F32 and E4M3, D / 2
 *            for MXFP4
 *   k_scale  F32 / E4M3 keys: float32 sigma_s per key row (same row index as `keys`,
 *            sigma_s > 0), or NULL (1.0).
 *            MXFP4 keys (the optional FP4 indexer cache of the TokenSpeed audit page,
 *            "DSA"; read as OCP MXFP4): required; uint8 [num_rows, D/32] E8M0 block
 *            scales, 4-byte aligned, key dimension d scaled by byte d/32 of its row.
 *            The score then has no sigma_s (sigma_s = 1).
 *   seq_lens [B] int32 cache length per request (history + Sq query tokens), >= Sq
 *   scores   [B, Sq, score_stride] float32, score_stride >= max(seq_lens)
 *   ready    if not NULL, the stream waits on this event before the scan starts: the
 *            load stream records it after the indexer-cache copy, so the scan can never
 *            read keys that are not yet resident ([GLM5R] "BugFix#2": the indexer must
 *            sync with the load stream before it launches; [HCCP] §1.3 ordering).
 *
 * Supported: (q F32, k F32): any H*D <= 4096, Sq*H <= 256, B <= 65535; q BF16 or E4M3 with
 * k E4M3 or MXFP4: D = 128, (H / 32, Sq) in {(1,1), (1,2), (1,4), (1,8), (2,1), (2,2), (2,4),
 * (4,1), (4,2)}, B <= 1024, B * ceil(score_stride / 32) < 2^31, keys->num_rows >= 32 (the
 * scan reads whole 32-token tiles); paged keys: page size a multiple of 32; dense keys:
 * num_rows and req_stride multiples of 32.  Outside these the call returns
 * DSA_ERR_UNSUPPORTED before anything is enqueued (the wait on `ready` included).
 * MXFP4 block-scale codes: 0x00..0xFE with E4M3 queries (the scaled MFMA applies them);
 * 0x00..0xFE with BF16 queries as long as every scaled key element is a finite bf16
 * (|element| * 2^(c-127) < 2^128).  Code 0xFF (NaN) gives an unspecified score.
 * Out-of-range page ids: the affected tokens score -inf, and each adds one to err_count.
 * A seq_lens[b] above score_stride is clamped to score_stride (nothing is written past a
 * score row); on the BF16 / E4M3 path each such request also adds one to err_count.
 */
dsa_status_t dsa_indexer_scores(const void* q, dsa_dtype_t q_dtype, const float* w,
                                const dsa_rows_t* keys, dsa_dtype_t k_dtype, const void* k_scale,
                                const int32_t* seq_lens, int B, int Sq, int H, int D,
                                int64_t score_stride, float* scores, int32_t* err_count,
                                hipEvent_t ready, hipStream_t stream);

/*
 * dsa_topk — keep the k best-scoring visible positions of each query ([GLM52] §2.1:
 * top-2048 feeds sparse attention).  Order: score descending, then position ascending
 * (lowest position wins a tie); -0.0 and +0.0 compare equal.  Output per (b,t) is the
 * selected positions in ascending order, padded with -1 when vis(b,t) < k.
 *
 *   scores   [B, Sq, score_stride] float32 (positions < vis(b,t) are read; no NaNs;
 *            a vis(b,t) above score_stride is clamped to score_stride)
 *   idx      [B, Sq, k] int32 output
 *   ws       workspace of at least dsa_topk_workspace_size(B, Sq, k, score_stride) bytes,
 *            8-byte aligned, contents on entry ignored: per row, the best keys of each
 *            chunk of positions as candidates (1024-position chunks for rows of up to
 *            262144 positions whose candidates fit, else 8192 or 16384) plus each chunk's
 *            cut key and candidate count, for a two-stage select (chunk c keeps at most
 *            twice its share ceil(k*len_c/n) of the k plus a slack; the exact select over
 *            the candidates is checked against the cut keys and redone over the row's
 *            scores when a chunk could hold more)
 * Supported: 1 <= k <= 8192, B*Sq <= 65535, score_stride <= 2^21.
 */
size_t dsa_topk_workspace_size(int B, int Sq, int k, int64_t score_stride);
dsa_status_t dsa_topk(const float* scores, int64_t score_stride, const int32_t* seq_lens, int B,
                      int Sq, int k, int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dsa_indexer_topk_chunks + dsa_topk_select_chunks — the same two results as
 * dsa_indexer_scores followed by dsa_topk, for one query token per request (Sq = 1), with
 * the top-k's chunk stage run inside the scan ([GLM52] §2.1: the indexer scores feed the
 * top-2048 directly).  Each wave of the scan owns a 1024-position unit of one request;
 * after writing the unit's scores it keeps the unit's candidates for the top-k in `ws`,
 * as dsa_topk's wave-chunk stage does.  dsa_topk_select_chunks then runs the exact select
 * over those candidates (re-selecting a row from `scores` when its candidates could miss
 * part of the answer).  scores and idx are bit-identical to the two separate calls.
 *
 *   dsa_indexer_topk_chunks: the arguments of dsa_indexer_scores with Sq = 1 on the MFMA
 *            path (q BF16 or E4M3, keys E4M3 or MXFP4, H in {32, 64, 128}), plus k and the
 *            top-k workspace ws / ws_bytes (dsa_topk_workspace_size(B, 1, k, score_stride)
 *            bytes, 8-byte aligned, contents on entry ignored).  `ready` and err_count as
 *            for dsa_indexer_scores.
 *   dsa_topk_select_chunks: the arguments of dsa_topk with Sq = 1; ws must hold what
 *            dsa_indexer_topk_chunks wrote for the same scores, seq_lens, k and
 *            score_stride, on the same stream or after it.
 * Supported: 1 <= k <= 8192, score_stride <= 262144 with candidate lists that fit the
 * select (dsa_topk's wave-chunk form; otherwise DSA_ERR_UNSUPPORTED with nothing
 * enqueued, and the caller takes the two separate calls).
 */
dsa_status_t dsa_indexer_topk_chunks(const void* q, dsa_dtype_t q_dtype, const float* w, const dsa_rows_t* keys,
                                     dsa_dtype_t k_dtype, const void* k_scale, const int32_t* seq_lens, int B, int H,
                                     int D, int64_t score_stride, float* scores, int k, void* ws, size_t ws_bytes,
                                     int32_t* err_count, hipEvent_t ready, hipStream_t stream);
dsa_status_t dsa_topk_select_chunks(const float* scores, int64_t score_stride, const int32_t* seq_lens, int B, int k,
                                    int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dsa_topk_union — the de-duplicated union of each request's Sq selections ([GLM52] §4.2: the
 * planner works on the de-duplicated union of a step's top-k positions; §5.1: the draft
 * tokens of speculative decoding select overlapping positions), for serving each distinct row
 * once and for attention over the union with per-query membership.
 *
 *   topk    [B, Sq, k] int32, each row ascending with -1 padding at the end (as dsa_topk writes)
 *   uni     [B, Sq * k] int32 out: the distinct valid positions of request b, ascending, then -1
 *   count   [B] int32 out: number of distinct positions
 *   uidx    [B, Sq, k] int32 out, optional: index in uni[b] of each entry's position, -1 for
 *           padding (so uni[b][uidx[b,t,j]] == topk[b,t,j])
 *   member  [B, Sq, W] uint32 out, optional, W = ceil(Sq * k / 32): bit u % 32 of word u / 32
 *           of row (b, t) is set iff uni[b][u] is one of query t's positions
 * A row found out of order adds one to err_count per out-of-order entry (the union is then
 * unspecified).  Supported: Sq <= 16, Sq * k <= 8192.
 */
dsa_status_t dsa_topk_union(const int32_t* topk, int B, int Sq, int k, int32_t* uni, int32_t* count,
                            int32_t* uidx, uint32_t* member, int32_t* err_count, hipStream_t stream);

/*
 * dsa_plan — shared-group pool plan ("DsaPlan", [GLM52] §4.2 and §5), run once per
 * decode step for a group of layers that share one top-k ([GLM52] §4.1, groups of 4).
 * The device pool of each request has n_sets sets of `ways` slots; id u belongs to
 * set u mod n_sets and may use any way of it; each set has one FIFO pointer that moves
 * once per install and never on a hit ([GLM52] §4.3).  Per request:
 *   U = ascending de-duplicated union of the valid (>= 0) positions of all Sq rows;
 *   u is a hit iff id_to_slot[u] != -1; the misses M (ascending) of set s get ways
 *   (ptr[s] + i) mod ways, i = 0..m_s-1, slot = s*ways + way, and survive iff
 *   i >= m_s - ways; ptr[s] advances by m_s mod ways.
 *
 *   topk        [B, Sq, k] int32 positions (-1 = padding), each row ascending
 *   pool_ids    [B, n_sets*ways] int32  id held by each slot, -1 = empty
 *   id_to_slot  [B, id_range] int32     slot of each id, -1 = not pooled
 *   ptr         [B, n_sets] int32       FIFO pointer per set
 *   is_hit      [B, Sq, k] uint8 out    1 = served from the pool
 *   slot        [B, Sq, k] int32 out    hit: its slot; surviving miss: its new slot;
 *                                       other miss and padding: -1
 *   miss_pos    [B, Sq*k] int32 out     the misses, ascending (first miss_count[b] valid)
 *   miss_slot   [B, Sq*k] int32 out     slot of each miss, -1 if it does not survive
 *   miss_count  [B] int32 out
 *   commit      1: apply the step to pool_ids / id_to_slot / ptr in the same launch (clear
 *               each evicted occupant's id_to_slot, install survivors, advance ptr).  The
 *               outputs above carry everything serve and install need, so committing at
 *               plan time equals the pages' commit at the end of the group.  0: leave the
 *               metadata untouched.
 * Positions >= id_range, and stored slots outside [0, n_sets*ways), are treated as
 * invalid entries (is_hit 0, slot -1, not counted as misses) and counted in err_count.
 * Supported: Sq*k <= 8192, n_sets <= 4096, ways <= 64, n_sets*ways <= 2^24.
 */
dsa_status_t dsa_plan(const int32_t* topk, int B, int Sq, int k, int32_t* pool_ids,
                      int32_t* id_to_slot, int32_t* ptr, int n_sets, int ways, int id_range,
                      uint8_t* is_hit, int32_t* slot, int32_t* miss_pos, int32_t* miss_slot,
                      int32_t* miss_count, int commit, int32_t* err_count, hipStream_t stream);

/*
 * dsa_gather_kv — per-layer serve and install ("DsaServe" / "DsaInstall", [GLM52] §4.4
 * and §5; the basic offload gather of selected rows from the host cache, §2.1).
 *
 * mode DSA_GATHER_SERVE: for every entry (b,t,j) with p = topk[b,t,j]:
 *     sel[b,t,j,:] = pool[b, slot[b,t,j], :]   if is_hit != NULL and is_hit[b,t,j]
 *                  = src row (b, p)            otherwise (p >= 0)
 *                  = zeros                     if p == -1
 * mode DSA_GATHER_INSTALL: for every entry with is_hit == 0 and slot >= 0 (a surviving
 *     miss; the first entry of a repeated position only):  pool[b, slot, :] = sel[b,t,j,:]
 *     The backfill reads the already-served row from `sel` rather than from `src`, so a
 *     miss crosses the host link once.  Run it after the layer's serve and after every
 *     reader of the overwritten pool rows ([GLM52] §4.4: backfill is off the critical
 *     path, on an auxiliary stream).
 *
 *   src      row store of the full cache for this layer (paged device cache, dense device
 *            rows, or mapped pinned host rows); row_bytes must equal `row_bytes`
 *   pool     [B, pool_rows, row_bytes] bytes (NULL allowed when is_hit is NULL in SERVE)
 *   sel      [B, Sq, k, row_bytes] bytes
 *   sel_idx  SERVE only, optional (NULL = not written): [B, Sq, k] int32, t * k + j where
 *            entry (b,t,j) received a row and -1 where it got the zero row (padding or an
 *            invalid entry).  Passed as `idx` to dsa_sparse_mla_decode together with a dense
 *            row store over `sel` (req_stride = Sq * k), attention then skips the padded
 *            entries instead of weighting their zero rows.  4-byte aligned.
 * Supported: row_bytes a multiple of 16, <= 4096.  Invalid slots / positions: zero row
 * (SERVE) or skipped (INSTALL), counted in err_count.
 */
#define DSA_GATHER_SERVE 0
#define DSA_GATHER_INSTALL 1
dsa_status_t dsa_gather_kv(const int32_t* topk, const uint8_t* is_hit, const int32_t* slot, int B,
                           int Sq, int k, const dsa_rows_t* src, void* pool, int64_t pool_rows,
                           int32_t row_bytes, void* sel, int32_t* sel_idx, int mode,
                           int32_t* err_count, hipStream_t stream);

/*
 * dsa_sparse_mla_decode — MLA latent attention over the selected rows only.  One
 * 576-wide bf16 latent row per token serves as key (all 576) and value (first 512)
 * ([TSA] "MLA (tokenspeed-mla)"); attention reads only the top-k rows ([GLM52] §2.1).
 * Per (b, t, h):
 *     logit_j = scale * <q[b,t,h,:], K_j>     over valid entries j of idx[b,t,:]
 *     lse     = ln sum_j exp(logit_j)
 *     o       = sum_j exp(logit_j - lse) * K_j[:512]
 * Empty selection: o = 0, lse = -inf.  The rows are split over work-groups and the
 * partial (o, lse) are merged by LSE rescaling ([TSA] two-stage split-KV decode).
 *
 *   q      [B, Sq, H, 576] bf16
 *   idx    [B, Sq, k] int32 positions into `rows` (-1 = skip).  A position >= 0 that resolves
 *          to no row (past the request's page-table row or dense stride, on a page whose id
 *          is negative, or at a row >= num_rows) is skipped like -1 and adds one to
 *          err_count.
 *   rows   row store of latent rows, row_bytes = 1152
 *   o      [B, Sq, H, 512], o_dtype BF16 (round-to-nearest-even) or F32
 *   lse    [B, Sq, H] float32
 *   scale  softmax scale, positive and finite (else DSA_ERR_INVALID_ARG)
 *   ws     workspace of dsa_sparse_mla_workspace_size(B, Sq, H, k) bytes (16-byte aligned);
 *          NULL allowed when that size is 0.  Holds the split partials: lse as float32,
 *          o normalised in o_dtype.  Its contents are scratch between calls.
 * Supported: H a multiple of 16 (H >= 64 runs 64-head work-groups of score and value waves;
 * 32 and 48 heads run 32-head, 16 heads 16-head work-groups), k <= 65536, rows->num_rows
 * < 2^31, at most 2^24 (query row, 16-head group) pairs, and a split grid that fits one
 * launch (fewer than 2^32 work-items); beyond those limits the call returns
 * DSA_ERR_UNSUPPORTED.
 */
size_t dsa_sparse_mla_workspace_size(int B, int Sq, int H, int k);
dsa_status_t dsa_sparse_mla_decode(const void* q, const int32_t* idx, const dsa_rows_t* rows,
                                   int B, int Sq, int H, int k, float scale, void* o,
                                   dsa_dtype_t o_dtype, float* lse, void* ws, size_t ws_bytes,
                                   int32_t* err_count, hipStream_t stream);

/*
 * dsa_sparse_mla_decode_union — sparse MLA for the Sq query tokens of a request over the union
 * of their selections (dsa_topk_union), with the query tokens packed into the head axis of
 * the work-groups ([TSA] "MLA (tokenspeed-mla)": fold_sq_factor folds the query tokens of a
 * step into the MMA M dimension; [GLM52] §5.1: draft tokens share most of their selection).
 * Each union row is loaded once per work-group and every query token attends only over the
 * entries its membership bits mark, so the result per (b, t, h) is dsa_sparse_mla_decode's
 * over that query's own selection (up to rounding order).
 *
 *   q       [B, Sq, H, 576] bf16
 *   uni     [B, U] int32 positions into `rows` (-1 = skip), from dsa_topk_union (U = Sq * k),
 *           or any row list with its membership masks
 *   count   [B] int32 or NULL: entries past count[b] are not read
 *   member  [B, Sq, ceil(U / 32)] uint32 membership bits (as dsa_topk_union writes them)
 *   rows, o [B, Sq, H, 512], lse [B, Sq, H], scale, err_count: as dsa_sparse_mla_decode
 *   ws      workspace of dsa_sparse_mla_union_workspace_size(B, Sq, H, U) bytes
 * Packing pays when one work-group holds more query heads than one query token has (a
 * work-group holds 64 heads): then a row shared by several query tokens is loaded once
 * instead of once per token.  Supported: H a multiple of 16, Sq * H <= 2^20, and the limits of
 * dsa_sparse_mla_decode for B requests of Sq * H heads over U entries.
 */
size_t dsa_sparse_mla_union_workspace_size(int B, int Sq, int H, int U);
dsa_status_t dsa_sparse_mla_decode_union(const void* q, const int32_t* uni, const int32_t* count,
                                         const uint32_t* member, const dsa_rows_t* rows, int B, int Sq,
                                         int H, int U, float scale, void* o, dsa_dtype_t o_dtype,
                                         float* lse, void* ws, size_t ws_bytes, int32_t* err_count,
                                         hipStream_t stream);

/*
 * dsa_sparse_mla_decode_noalloc — dsa_sparse_mla_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the split partials go to a scratch array inside the library instead of a
 * caller workspace; the caller still passes q, idx, rows, o and lse.  Arguments, results and
 * errors are those of dsa_sparse_mla_decode.
 *   - The scratch array holds dsa_sparse_mla_noalloc_max_workspace() bytes (64 MiB) on every
 *     device the library runs on, until the process ends.  A call whose
 *     dsa_sparse_mla_workspace_size(B, Sq, H, k) exceeds it returns DSA_ERR_UNSUPPORTED with
 *     nothing enqueued.
 *   - The call allocates nothing.  Its first call on a device looks up that device's copy
 *     of the array (hipGetSymbolAddress).
 *   - Every call on a device shares that device's array: calls that may overlap on one
 *     device (other streams, other threads) race on it and must be ordered by the caller.
 *     Nothing in it needs to start at zero; each call writes every partial it reads.
 */
size_t dsa_sparse_mla_noalloc_max_workspace(void);
dsa_status_t dsa_sparse_mla_decode_noalloc(const void* q, const int32_t* idx, const dsa_rows_t* rows,
                                           int B, int Sq, int H, int k, float scale, void* o,
                                           dsa_dtype_t o_dtype, float* lse, int32_t* err_count,
                                           hipStream_t stream);

/*
 * dsa_merge_partials — combine R partial attention results, each over its own disjoint set
 * of rows, into the result over the union of the rows ([TSA] "MLA": split-KV partials merged
 * by LSE rescaling; [HCCP] §1.1: under page-sharded KV each rank attends over the pages it
 * owns, so the ranks' partials are merged this way).  For every output row n:
 *     lse[n] = ln sum_r exp(lse_r[n])
 *     o[n,:] = sum_r exp(lse_r[n] - lse[n]) * o_r[n,:]
 * A part with lse_r = -inf (no rows) contributes nothing; if every part is empty the result is
 * o = 0, lse = -inf.
 *
 *   o_parts    [R, N, V] part_dtype (F32 or BF16), 16-byte aligned: rank r's normalised o
 *              (e.g. [R, B, Sq, H, 512] from dsa_sparse_mla_decode with o_dtype F32)
 *   lse_parts  [R, N] float32
 *   o          [N, V] o_dtype (F32 or BF16, round to nearest even), 16-byte aligned
 *   lse        [N] float32
 * Supported: V a multiple of 8, ceil(N / 4) < 2^31.
 */
dsa_status_t dsa_merge_partials(const void* o_parts, dsa_dtype_t part_dtype, const float* lse_parts, int R,
                                int64_t N, int V, void* o, dsa_dtype_t o_dtype, float* lse,
                                hipStream_t stream);

/*
 * dsa_page_translate — owner rank and owner-local row of logical cache slots under
 * page-based KV sharding ([HCCP] §1.1): q = floor(x / page_size), rank = q mod n_ranks,
 * local_row = floor(q / n_ranks) * page_size + (x mod page_size).  Arithmetic only,
 * no lookup table.
 *
 *   x          [n] int64 logical slots (>= 0; negative slots give rank -1, row -1 and
 *              count in err_count)
 *   rank       [n] int32 out
 *   local_row  [n] int64 out
 */
dsa_status_t dsa_page_translate(const int64_t* x, int64_t n, int page_size, int n_ranks,
                                int32_t* rank, int64_t* local_row, int32_t* err_count,
                                hipStream_t stream);

/*
 * dsa_kv_write — the KV write path of a decode step: quantise and scatter the new tokens
 * into the paged caches in one launch ([TSA] "Attention integration / KV host tiering":
 * the fused KV-pack kernel; [TSA] "MLA": one 576-wide latent row per token; [GLM52] §2.1:
 * fp8 indexer keys).  The Sq new tokens of request b sit at its last Sq positions,
 * p = seq_lens[b] - Sq + t (seq_lens counts them already).  For each:
 *     kv row of (b, p)        = latent[b, t, :]                  (bf16, copied bit for bit)
 *     sigma                   = max_d |idx_k[b, t, d]| / 448      (float32 division)
 *     idx_cache row of (b, p) = e4m3(idx_k[b, t, d] / sigma)     (float32 division, nearest
 *                               OCP E4M3FN value, ties to even, saturating at 448)
 *     idx_scale[that row]     = sigma
 * A zero key stores sigma = 0 and zero codes (it dequantises to 0).  The pages do not fix
 * the key quantisation; this is the per-token-scale layout dsa_indexer_scores reads.
 * With idx_cache_dtype = DSA_MXFP4 (the FP4 indexer cache, [TSA] "DSA", read as OCP MXFP4)
 * the key is quantised per block j of 32 dimensions instead (OCP MX conversion):
 *     code_j                  = clamp(floor(log2 max_{d in j} |idx_k[b,t,d]|) - 2 + 127, 0, 254)
 *                               (0 for an all-zero block); X_j = 2^(code_j - 127)
 *     element d               = nearest E2M1 value of idx_k[b,t,d] / X_j, ties to the even
 *                               mantissa, magnitudes above 6 saturating to 6
 *     idx_cache row of (b, p) = the D codes, element 2i in the low nibble of byte i
 *     idx_scale[row][j]       = code_j
 *
 *   latent      [B, Sq, 576] bf16, 16-byte aligned
 *   idx_k       [B, Sq, D] bf16 or float32 (idx_k_dtype), 8-byte aligned; D even, <= 128
 *   kv          rows of the latent cache (row_bytes 1152, base 16-byte aligned), written
 *   idx_cache   rows of the indexer cache, written; it may use its own page table.
 *               E4M3: row_bytes D, base 2-byte aligned.  MXFP4: row_bytes D / 2, D a
 *               multiple of 32.
 *   idx_scale   E4M3: [idx_cache rows] float32 (4-byte aligned); MXFP4: [idx_cache rows,
 *               D / 32] uint8 E8M0 codes; written at each written row
 * A token whose position or page is out of range in either cache is skipped and counted
 * in err_count.  Two tokens mapping to the same row race (the caller's pages are distinct).
 */
dsa_status_t dsa_kv_write(const void* latent, const void* idx_k, dsa_dtype_t idx_k_dtype,
                          const int32_t* seq_lens, int B, int Sq, int D, const dsa_rows_t* kv,
                          const dsa_rows_t* idx_cache, dsa_dtype_t idx_cache_dtype, void* idx_scale,
                          int32_t* err_count, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBDSA_DSA_H */
