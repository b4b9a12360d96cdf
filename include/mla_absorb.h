/*
 * mla_absorb.h - C ABI of an MI355X (gfx950) library for Multi-head Latent
 * Attention decode in the weight-absorbed form over a paged latent KV cache.
 *
 * The method: each cached position stores only the compressed latent c (D_C
 * wide) and one rotary key k_rope (D_R wide) shared by all heads ("DeepSeek's
 * KV Cache: From 3.9 MB to 890 B per Token", Figure 3 and section "Calculating
 * V2's KV cache").  A decode step never expands per-head keys or values:
 *   1. mla_absorb_q    q_lat[h] = W_UK[h] q_nope[h]    (Figure 5, form (2))
 *   2. mla_decode_attn score_j = scale*(q_lat[h].c_j + q_rope[h].k_rope_j),
 *                      softmax over the visible positions, and the weighted
 *                      latent U[h] = sum_j p_j c_j      (Figures 4, 5 (2), 6 (2))
 *      optionally restricted to a picked subset of positions (Figure 10)
 *   3. mla_combine     log-sum-exp merge of split partials (exact identity of
 *                      softmax over a union of disjoint position sets)
 *   4. mla_out_up      out[h] = W_UV[h] U[h]            (Figure 6, form (2))
 *   3+4. mla_combine_out_up  both in one launch, without storing U
 *
 * Conventions common to every call
 *  - All pointers except *_host ones are device pointers.  The caller owns
 *    every buffer; the library allocates nothing, keeps no state between
 *    calls and never synchronises.  Kernels are enqueued on `stream` (a
 *    hipStream_t; NULL = the default stream) and run asynchronously: buffers
 *    must stay alive until the stream has passed them.
 *  - Each call validates its host-visible arguments first.  On any error it
 *    enqueues nothing and returns the error code.  MLA_ERR_LAUNCH reports a
 *    failed kernel launch (hipGetLastError after the launch).
 *  - Dense tensors are row-major with the shapes given below, element type
 *    act_dtype (queries, weights, outputs) unless stated.  Pointers must be
 *    16-byte aligned.
 *  - Device-resident metadata (seq_lens, block tables, index lists) is not
 *    read on the host.  Contract: 1 <= seq_lens[b]; block-table entries of the
 *    pages a request uses are valid page ids; index lists are sorted,
 *    distinct, within [0, seq_lens[b]) or -1 as padding.  Kernels never fault
 *    on bad metadata: positions whose index is negative or >= seq_lens[b], and
 *    positions whose page id is outside [0, num_pages), are skipped as if
 *    masked.  mla_check_decode_inputs_host() checks the contract on host
 *    copies and reports the first violation.
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1
#define MLA_PAGE_TOKENS 64 /* positions per cache page */
#define MLA_TILE_TOKENS 32 /* positions per attention tile; split granularity */

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null or misaligned pointer, bad size, too small workspace */
  MLA_ERR_UNSUPPORTED = 2, /* a dims / dtype combination the library has no kernel for */
  MLA_ERR_LAUNCH = 3,      /* the HIP runtime refused a launch */
  MLA_ERR_SCRATCH = 4      /* the call needs more than the library's static
                              scratch holds (mla_decode_noalloc only) */
} mla_status;

typedef enum {
  MLA_F32 = 0,
  MLA_BF16 = 1,
  MLA_FP8_E4M3 = 2,     /* OCP E4M3: bias 7, max 448, no infinities (cache only);
                           one float32 scale per position */
  MLA_FP8_E4M3_G128 = 3 /* the same codes with one float32 scale per 128
                           consecutive latent channels of each position
                           ("DeepSeek's KV Cache", section "Calculating V3.2's
                           KV cache": the 656-byte main KV item; cache only) */
} mla_dtype;

/* Model dimensions and types.  Supported combinations:
 *   cache F32,  act F32 : any dims with num_heads*d_latent <= 8192,
 *                         d_latent, d_rope <= 512 (generic fp32 kernels)
 *   cache BF16, act BF16: num_heads = 128, d_latent = 512, d_rope = 64
 *                         (DeepSeek-V2 dims; MFMA kernels), d_nope and d_v
 *                         multiples of 16
 *   cache FP8,  act BF16: as BF16, latent stored as E4M3 with one float32
 *                         scale per position, rotary key in BF16
 *   cache FP8_E4M3_G128, act BF16: as FP8, with D_C / 128 float32 scales per
 *                         position; channel d of the latent uses scale d / 128
 *   The FP8 latent is dequantised (code value times its scale) to BF16 inside
 *   the kernel, one rounding per element, before the matrix products. */
typedef struct {
  int32_t num_heads;     /* H */
  int32_t d_latent;      /* D_C, width of the cached latent c */
  int32_t d_rope;        /* D_R, width of the shared rotary key */
  int32_t d_nope;        /* D_N, per-head content query width */
  int32_t d_v;           /* D_V, per-head value width */
  int32_t block_size;    /* positions per page, must be MLA_PAGE_TOKENS */
  float softmax_scale;   /* > 0, usually 1/sqrt(d_nope + d_rope) */
  int32_t cache_dtype;   /* mla_dtype */
  int32_t act_dtype;     /* mla_dtype, F32 or BF16 */
} mla_config;

/* Split plan for mla_decode_attn / mla_combine. */
typedef struct {
  int32_t num_workers;    /* work-groups that share the position tiles of all requests, 1..65536 */
  int32_t num_slots;      /* partial results the workers can emit: num_workers + batch - 1 */
  size_t workspace_bytes; /* bytes mla_decode_attn needs for partials */
} mla_plan;

/* ABI version compiled into the library (MLA_ABI_VERSION). */
int32_t mla_abi_version(void);

/* Static text for a status code. */
const char* mla_status_string(mla_status status);

/* Byte layout of one cache page (structure of arrays, sections 16-byte
 * aligned, positions in order inside each section):
 *   F32 : c [64][D_C] f32,  k_rope [64][D_R] f32
 *   BF16: c [64][D_C] bf16, k_rope [64][D_R] bf16
 *   FP8 : c [64][D_C] e4m3, k_rope [64][D_R] bf16, scale [64] f32
 *   FP8_E4M3_G128: c [64][D_C] e4m3, k_rope [64][D_R] bf16,
 *         scale [64][D_C / 128] f32
 * Outputs the page size and the offsets of the rope and scale sections.  Host
 * only. */
mla_status mla_page_layout(const mla_config* cfg, size_t* page_bytes, size_t* rope_offset,
                           size_t* scale_offset);

/* Append one new token per request to the cache, before the decode step
 * that reads it ("DeepSeek's KV Cache", section "MLA: the cache holds one
 * latent", Figure 3: the latent is stored without rotation, the shared rotary
 * key with RoPE applied; section "Calculating V3.2's KV cache" for the FP8
 * item).
 *   c_new [batch][D_C], k_new [batch][D_R]: activation dtype (16-byte
 *     aligned); k_new is the rotary key before rotation.
 *   rope_cos, rope_sin [rope_rows][D_R / 2] float32, or both NULL to store
 *     k_new as given: pair i (elements 2i, 2i+1) of the key at position p
 *     becomes (x cos - y sin, x sin + y cos) with cos = rope_cos[p][i],
 *     sin = rope_sin[p][i].
 *   positions [batch] int32: the position the token takes; it is written to
 *     row p % 64 of page block_table[b][p / 64].
 *   kv_pool, num_pages, block_table, block_table_stride: as mla_decode_attn.
 * Storage: F32 and BF16 caches store the values (BF16 activations as they
 * are); FP8 caches store scale = max|c| / 448 over the token (over each 128
 * channels for MLA_FP8_E4M3_G128; 1 when that maximum is 0) and the E4M3
 * codes nearest to c / scale (float32 quotient clamped to +-448, ties to
 * even), the rotary key in BF16 (rounded to nearest even).  Only the token's
 * row of each section is written.  A request whose position is negative, not
 * below 64 * block_table_stride (or rope_rows when tables are given), or on a
 * page id out of range writes nothing.
 * Errors: null or misaligned pointers, batch < 1, only one table given,
 * rope_rows < 1 with tables -> MLA_ERR_INVALID_ARG; odd d_rope ->
 * MLA_ERR_UNSUPPORTED. */
mla_status mla_cache_append(const mla_config* cfg, const void* c_new, const void* k_new, const float* rope_cos,
                            const float* rope_sin, int32_t rope_rows, const int32_t* positions, void* kv_pool,
                            int64_t num_pages, const int32_t* block_table, int32_t block_table_stride,
                            int32_t batch, void* stream);

/* ---- Prefill (many queries of one request) on the expanded path ----
 * With many queries a key expanded once is shared by all of them ("DeepSeek's
 * KV Cache", the paragraph after Figure 5 on when absorption wins; Figure 5
 * (1) and Figure 6 (1) for the expanded forms).  V2 dims, a BF16 or FP8
 * cache, BF16 activations, d_nope = d_v = 128 (MLA_ERR_UNSUPPORTED
 * otherwise).
 *
 * mla_prepare_w_uk_t: the weight layout the expansion reads, once per set of
 * weights: w_uk_t[h][n][c] = w_uk[h][c][n] ([H][D_N][D_C], BF16). */
mla_status mla_prepare_w_uk_t(const mla_config* cfg, const void* w_uk, void* w_uk_t, void* stream);

/* mla_prefill_expand: for positions 0 .. T-1 of one request (pages
 * block_table[0 .. ceil(T/64) - 1] of kv_pool), write
 *   k_nope[s][h][n] = sum_c c_s[c] w_uk[h][c][n]   [T][H][D_N] BF16
 *   v[s][h][n]      = sum_c w_uv[h][n][c] c_s[c]    [T][H][D_V] BF16
 *   k_rope[s][r]    = the cached rotary key         [T][D_R]    BF16
 * (float32 accumulation, one BF16 rounding).  The cache is BF16 or FP8
 * ("DeepSeek's KV Cache", section "Calculating V3.2's KV cache": c_s is the
 * E4M3 value times its scale): with one scale per position the sums run on
 * the exact code values and are multiplied by the position's scale in
 * float32; with one scale per 128 channels each value times its group's
 * scale is rounded once to BF16 first.  Positions on a page id out of range
 * get unspecified values (never a fault).  Errors: null or misaligned
 * pointers, T < 1 -> MLA_ERR_INVALID_ARG; a float32 cache ->
 * MLA_ERR_UNSUPPORTED. */
mla_status mla_prefill_expand(const mla_config* cfg, const void* kv_pool, int64_t num_pages,
                              const int32_t* block_table, int32_t T, const void* w_uk_t, const void* w_uv,
                              void* k_nope, void* v, void* k_rope, void* stream);

/* mla_prefill_attn: n_queries queries at positions q_start .. q_start +
 * n_queries - 1 (q_start + n_queries <= T), query i attending to positions
 * 0 .. q_start + i of the expanded keys and values:
 *   q_nope [n][H][D_N], q_rope [n][H][D_R] BF16 (rotated);
 *   out [n][H][D_V] BF16 = softmax(scale (q_nope . k_nope + q_rope . k_rope)) v;
 *   lse_out [n][H] float32 (natural log of the softmax sum) or NULL.
 * Errors: null or misaligned pointers, n_queries < 1, q_start < 0,
 * q_start + n_queries > T -> MLA_ERR_INVALID_ARG. */
mla_status mla_prefill_attn(const mla_config* cfg, const void* q_nope, const void* q_rope, const void* k_nope,
                            const void* v, const void* k_rope, int32_t T, int32_t q_start, int32_t n_queries,
                            void* out, float* lse_out, void* stream);

/* Choose the number of workers for a batch and size the partial workspace.
 * seq_lens_host: host copy of the per-request lengths (used only to count
 * tiles; may be NULL, then every request is assumed to be max_len long).
 * topk: 0 for dense attention, else the index-list length per request.
 * num_cus: compute units of the device (256 on MI355X).  Host only. */
mla_status mla_decode_plan(const mla_config* cfg, int32_t batch, const int32_t* seq_lens_host,
                           int32_t max_len, int32_t topk, int32_t num_cus, mla_plan* plan);

/* Step 1 (Figure 5 (2)): absorb W_UK into the query.
 *   q_nope [batch][H][D_N], w_uk [H][D_C][D_N] (k_nope_j = c_j W_UK[h], i.e.
 *   W^UK_h as an [input, output] matrix), q_lat [batch][H][D_C]:
 *   q_lat[b][h][c] = sum_n w_uk[h][c][n] * q_nope[b][h][n]  (fp32 accumulate) */
mla_status mla_absorb_q(const mla_config* cfg, const void* q_nope, const void* w_uk, void* q_lat,
                        int32_t batch, void* stream);

/* Step 2: attention of every head over the latent cache.
 *   q_lat [batch][H][D_C], q_rope [batch][H][D_R] (act_dtype)
 *   kv_pool: num_pages pages laid out as mla_page_layout() describes
 *   block_table [batch][block_table_stride] int32 page ids, logical page
 *     i of request b holds positions 64i..64i+63
 *   seq_lens [batch] int32 cached positions per request (all visible)
 *   topk_idx: NULL for dense attention, else [batch][topk] int32 positions
 *     (sorted, distinct, -1 = padding); only those positions are read and
 *     the softmax runs over them alone (Figure 10)
 * Two output modes:
 *   o_lat != NULL: one work-group per request writes the final weighted latent
 *     o_lat [batch][H][D_C] (act_dtype) and, if lse_out != NULL, lse_out
 *     [batch][H] = log sum_j exp(score_j).  workspace is not used.
 *   o_lat == NULL: plan->num_workers work-groups share all position tiles of
 *     all requests and write partials (the normalised weighted latent, BF16
 *     when act_dtype is BF16 and float32 otherwise, and its float32
 *     log-sum-exp) into workspace; mla_combine() or mla_combine_out_up()
 *     finishes.
 * A request whose positions are all skipped yields zeros and lse = -inf. */
mla_status mla_decode_attn(const mla_config* cfg, const void* q_lat, const void* q_rope,
                           const void* kv_pool, int64_t num_pages, const int32_t* block_table,
                           int32_t block_table_stride, const int32_t* seq_lens,
                           const int32_t* topk_idx, int32_t topk, int32_t batch,
                           const mla_plan* plan, void* workspace, size_t workspace_bytes,
                           void* o_lat, float* lse_out, void* stream);

/* Step 3: merge the partials of mla_decode_attn (o_lat == NULL mode):
 *   o_lat[b][h] = sum_s exp(lse_s - LSE) o_s,  LSE = log sum_s exp(lse_s)
 * over the partials that request b received.  seq_lens, topk, batch and plan
 * must be those given to mla_decode_attn.  lse_out [batch][H] may be NULL. */
mla_status mla_combine(const mla_config* cfg, const void* workspace, size_t workspace_bytes,
                       const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                       void* o_lat, float* lse_out, void* stream);

/* Step 4 (Figure 6 (2)): up-project the weighted latent.
 *   o_lat [batch][H][D_C], w_uv [H][D_V][D_C] (v_j = W_UV[h] c_j),
 *   out [batch][H][D_V]: out[b][h][v] = sum_c w_uv[h][v][c] * o_lat[b][h][c] */
mla_status mla_out_up(const mla_config* cfg, const void* o_lat, const void* w_uv, void* out,
                      int32_t batch, void* stream);

/* Steps 3 and 4 in one launch: out[b][h] = W_UV[h] o_lat[b][h] with o_lat[b][h]
 * the merge mla_combine computes (rounded to BF16 as mla_combine stores it),
 * never written to memory (Figure 6, form (2), after the exact log-sum-exp
 * merge).  workspace, seq_lens, topk, batch and plan as for mla_combine;
 * w_uv and out as for mla_out_up; lse_out [batch][H] may be NULL.  Served for
 * act_dtype BF16 at H = 128, D_C = 512, D_V = 128; other configurations return
 * MLA_ERR_UNSUPPORTED (use mla_combine, then mla_out_up). */
mla_status mla_combine_out_up(const mla_config* cfg, const void* workspace, size_t workspace_bytes,
                              const int32_t* seq_lens, int32_t topk, int32_t batch, const mla_plan* plan,
                              const void* w_uv, void* out, float* lse_out, void* stream);

/* Bytes of the static device buffer mla_decode_noalloc keeps its split
 * partials in (one buffer per GPU, held until the process ends). */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the split
 * decode of mla_decode_attn (with `plan`) followed by its merge, in one call,
 * with the split partials kept in a static device buffer the library owns
 * instead of a caller workspace.  Nothing is allocated or freed by this call.
 *   Arguments as mla_decode_attn (split mode) and mla_combine /
 *   mla_combine_out_up.  Exactly one output form:
 *     o_lat != NULL (w_uv and out NULL): the merged weighted latent, as
 *       mla_combine writes it;
 *     out != NULL with w_uv: the merged up-projection, as mla_combine_out_up
 *       writes it (BF16, D_V = 128 only; o_lat is not written).
 *   lse_out [batch][H] may be NULL.
 * Capacity: the partials take (num_workers + batch - 1) * (H * D_C * e + H *
 * 4) bytes, each section rounded up to 16, with e = 2 for BF16 activations and
 * 4 for F32; calls needing more than MLA_NOALLOC_SCRATCH_BYTES return
 * MLA_ERR_SCRATCH and enqueue nothing (at V2 dims: 382 slots, e.g. 256
 * workers and up to 127 requests).
 * Sharing: every call on a GPU uses that GPU's one buffer.  Calls that may
 * overlap on one GPU (different streams, or host threads without ordering)
 * race on it and must not be issued; calls in order on one stream are safe.
 * The buffer keeps the last call's contents; nothing in it needs clearing,
 * because the merge reads only partials written by the same call.
 * The first call on a device looks up that device's buffer address (with the
 * device current); later calls reuse it.
 * Errors: as mla_decode_attn and the merge calls, plus both or neither
 * output given -> MLA_ERR_INVALID_ARG, capacity -> MLA_ERR_SCRATCH. */
mla_status mla_decode_noalloc(const mla_config* cfg, const void* q_lat, const void* q_rope, const void* kv_pool,
                              int64_t num_pages, const int32_t* block_table, int32_t block_table_stride,
                              const int32_t* seq_lens, const int32_t* topk_idx, int32_t topk, int32_t batch,
                              const mla_plan* plan, void* o_lat, const void* w_uv, void* out, float* lse_out,
                              void* stream);

/* Host-side check of the device-metadata contract on host copies: lengths
 * >= 1, enough block-table columns, page ids in [0, num_pages) for every page
 * a request uses, index lists sorted, distinct, in range, -1 only as trailing
 * padding.  topk_idx may be NULL (dense).  Returns MLA_OK or
 * MLA_ERR_INVALID_ARG and, if err_index != NULL, the request that failed. */
mla_status mla_check_decode_inputs_host(const mla_config* cfg, int32_t batch,
                                        const int32_t* seq_lens, const int32_t* block_table,
                                        int32_t block_table_stride, int64_t num_pages,
                                        const int32_t* topk_idx, int32_t topk,
                                        int32_t* err_index);

#ifdef __cplusplus
}
#endif
#endif /* MLA_ABSORB_H */
