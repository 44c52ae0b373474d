/*
 * librba — relative-bias grouped-query attention on AMD Instinct MI355X (gfx950).
 *
 * What is computed (the method, restated from the pages):
 *   "Inkling-Small on Gaudi 2", sections "Why it needed a port" and
 *   "Attention with a relative bias": every attention logit gets a learned
 *   per-query, per-head, per-distance term rel[i, h, i - j] in place of RoPE;
 *   rel is produced for the tokens of the current call (one row per query
 *   token) and handed to the attention call; chunked prefill and prefix hits
 *   attend to the cached context plus the new tokens; key positions in a paged
 *   cache are block ordinal * block size + slot.
 *   Same page, "What was built": GQA (32 query / 8 KV heads, head size 128),
 *   local layers with a 512-token window (relative extent 512), global layers
 *   without a window (relative extent 1024).
 *   Same page, "Decode window": the window holds exactly W keys including the
 *   query's own key.
 *   "Inkling on Two DGX Sparks ...", section "Wall 1": the value head size may
 *   differ from the query/key head size (128 vs 64); decode splits the KV range
 *   and must not read device values on the host (graph capture).
 *   "vLLM TML Inkling Support", section "Low-Latency Collectives and Kernels":
 *   the number of KV splits is chosen from batch size and KV length.
 *   "Inkling 2 Small on vLLM: Day-0 Support", integration section: decode and
 *   verify read each KV block once for all query heads that share it.
 *
 *   For query row t (absolute position i) of sequence b, query head h, KV head
 *   g = h / (Hq / Hkv):
 *     x_j      = scale * <q[t,h,:], K_b[j,g,:]> + (i - j < R ? rel[t,h,i-j] : 0)
 *     visible  = j <= i  and  (W == 0 or i - j < W)
 *     out[t,h] = sum_j softmax_j(x) * V_b[j,g,:]      (fp32)
 *     lse[t,h] = log sum_j exp(x_j)                   (fp32, natural log)
 *   The bias for distances i - j >= R is 0: the pages do not define it and this
 *   library fixes it to zero.
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers are device memory owned by the caller;
 *     the library allocates nothing, frees nothing and keeps no pointer after
 *     the call returns. `params` and other host pointers are read during the
 *     call only.
 *   - Layouts are dense row-major. bf16 is IEEE bfloat16 (uint16 storage).
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *     and return without waiting. No call reads device memory on the host, so
 *     calls may be captured into a HIP graph. Calls are thread-safe.
 *   - All argument checks run on the host before anything is launched; a call
 *     that returns an error has enqueued nothing and written nothing.
 *   - Return 0 on success or a negative RBA_ERR_* code; rba_last_error()
 *     then describes the problem (thread-local).
 *   - Alignment: q, k_cache, v_cache, out, workspace, r and rel_proj must be
 *     16-byte aligned; rel, lse, cu_q, seq_lens, block_tables, sink, gate and
 *     logit_scale 4-byte aligned (RBA_ERR_UNSUPPORTED otherwise).
 *   - Values the library cannot check without reading device memory are the
 *     caller's contract: q_len_b <= seq_lens[b] <= max_seq_len, cu_q
 *     non-decreasing with cu_q[batch] = the rows of q, and q_len_b <=
 *     max_q_len. A seq_lens[b] below q_len_b (or n_q), above what the
 *     block-table row addresses (max_blocks_per_seq * 128), or (decode) above
 *     what the split plan for max_seq_len covers makes sequence b's rows NaN;
 *     no block-table entry past the row is read. Table entries for blocks a
 *     query can see must be in [0, num_blocks); an entry outside that range
 *     makes the affected rows NaN instead of being dereferenced. Entries for
 *     blocks that no query of the call can see (wholly outside every window)
 *     are never read and may hold anything, e.g. -1. Other violations give
 *     undefined results, never out-of-bounds accesses.
 *   - Slots of the last block past seq_lens[b] are never used: whatever they
 *     hold (NaN included) contributes exactly 0.
 */
#ifndef RBA_H
#define RBA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RBA_OK 0
#define RBA_ERR_NULL (-1)        /* a required pointer is NULL                      */
#define RBA_ERR_SHAPE (-2)       /* inconsistent sizes or counts                     */
#define RBA_ERR_UNSUPPORTED (-3) /* valid in principle, not supported by the kernels */
#define RBA_ERR_WORKSPACE (-4)   /* workspace missing or too small                   */
#define RBA_ERR_HIP (-5)         /* a HIP runtime call failed                        */

#define RBA_BLOCK_SIZE 128       /* tokens per KV-cache block                        */
#define RBA_HEAD_DIM_QK 128      /* supported query/key head size                    */

typedef struct rba_attn_params {
    int32_t num_heads_q;   /* Hq >= 1                                                */
    int32_t num_heads_kv;  /* Hkv >= 1, Hq % Hkv == 0; query head h uses KV head    */
                           /* h / (Hq / Hkv)                                         */
    int32_t head_dim_qk;   /* must be 128                                            */
    int32_t head_dim_v;    /* 64 or 128                                              */
    int32_t rel_extent;    /* R >= 1: bias defined for distances 0 <= i-j < R, 0     */
                           /* beyond                                                 */
    int32_t window;        /* W: 0 = no window; else key visible iff 0 <= i-j < W    */
    float scale;           /* finite multiplier of q.k (e.g. 1/sqrt(128))            */
    int32_t block_size;    /* must be RBA_BLOCK_SIZE                                 */
} rba_attn_params;

/* Library version string, e.g. "librba 0.1.0 gfx950". */
const char* rba_version(void);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* rba_last_error(void);

/*
 * Prefill / chunked prefill / prefix-cache extension.
 * Source: "Inkling-Small on Gaudi 2", section "Attention with a relative
 * bias" (a chunk attends to all cached context plus itself; key positions
 * from block ordinals; local layers need only the blocks inside the window).
 *
 *   q            device bf16 [total_q, Hq, 128]; rows of all sequences packed,
 *                sequence b owns rows [cu_q[b], cu_q[b+1])
 *   k_cache      device bf16 [num_blocks, Hkv, 128, 128]   (block, head, slot, dim)
 *   v_cache      device bf16 [num_blocks, Hkv, 128, dv]
 *   num_blocks   number of blocks in the cache pool (>= 1)
 *   rel          device fp32 [total_q, Hq, R]; row t is the bias row of query row t
 *   cu_q         device int32 [batch + 1]; query-row offsets, cu_q[0] = 0
 *   seq_lens     device int32 [batch]; keys of sequence b INCLUDING this call's
 *                tokens, whose K/V must already be in the cache. The query rows
 *                of b are its last q_len_b = cu_q[b+1]-cu_q[b] positions.
 *   block_tables device int32 [batch, max_blocks_per_seq]; entry n is the physical
 *                block holding positions [128 n, 128 n + 128) of the sequence
 *   batch        number of sequences (0 = nothing to do)
 *   max_q_len    host upper bound of every q_len_b (sets the grid)
 *   max_seq_len  host upper bound of every seq_lens[b]; max_blocks_per_seq must be
 *                >= ceil(max_seq_len / 128)
 *   out          device fp32 [total_q, Hq, dv]  (written)
 *   lse          device fp32 [total_q, Hq] or NULL (written if non-NULL)
 *   stream       hipStream_t
 * Errors: RBA_ERR_NULL, RBA_ERR_SHAPE, RBA_ERR_UNSUPPORTED, RBA_ERR_HIP.
 */
int rba_prefill(const rba_attn_params* params,
                const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                float* out, float* lse, void* stream);

/*
 * Prefill with the bias produced inside the kernel from its source, instead
 * of read from a materialised rel tensor. Source: "Inkling-Small on Gaudi 2",
 * section "Attention with a relative bias" (each layer forms rel as the
 * product of r, the R branch of the fused QKVR projection, with the layer's
 * rel_logits_proj, and hands it to the attention call). Reading: r has one
 * vector of width d_r per token and query head; the projection is one
 * [d_r, R] matrix shared by all heads or one per query head; the pages give
 * neither the width nor the sharing.
 *
 *   r            device bf16 [total_q, Hq, d_r], rows as q
 *   rel_proj     device bf16 [proj_heads, R, d_r], the projection in a linear
 *                layer's weight layout: element (hp, d, c) multiplies r[..., c]
 *                into the bias at distance d. Head h uses hp = h when
 *                proj_heads == Hq, hp = 0 when proj_heads == 1.
 *   d_r          32, 64 or 128 (RBA_ERR_UNSUPPORTED otherwise)
 *   proj_heads   1 or Hq (RBA_ERR_SHAPE otherwise)
 *   sink, gate   as rba_prefill_gated (NULL: not applied)
 *   all other arguments as rba_prefill. The bias of distance d is
 *   sum_c r[t, h, c] * rel_proj[hp, d, c] (products exact, fp32 sum) for
 *   0 <= d < R and 0 beyond. r and rel_proj must be 16-byte aligned.
 * Errors: as rba_prefill.
 */
int rba_prefill_relproj(const rba_attn_params* params,
                        const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                        const void* r, const void* rel_proj, int32_t d_r, int32_t proj_heads,
                        const int32_t* cu_q, const int32_t* seq_lens,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                        const float* sink, const float* gate,
                        float* out, float* lse, void* stream);

/*
 * Prefill and decode with a per-row logit scale: every logit of query row t,
 * scale * q.k + bias, is multiplied by logit_scale[t]. Source: "Inkling-Small
 * on Gaudi 2", section "What was built" (global layers apply a log-position
 * scale to q and to the rel logits beyond 128K positions). The pages give no
 * formula for the scale, so the caller computes one value per query row (for
 * example from its absolute position); applying it to q and to the bias is
 * the same as multiplying the row's logits by it.
 *
 *   logit_scale  device fp32, [total_q] for rba_prefill_logpos (row t of q)
 *                and [batch * n_q] for rba_decode_logpos; finite values
 *   all other arguments as rba_prefill / rba_decode (bf16 K/V; no sink or
 *   gate: rba_prefill_ex / rba_decode_ex combine them). Errors: as
 *   rba_prefill / rba_decode; RBA_ERR_NULL if logit_scale
 *   is NULL for a non-empty call, RBA_ERR_UNSUPPORTED if it is not 4-byte
 *   aligned.
 */
int rba_prefill_logpos(const rba_attn_params* params,
                       const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                       const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                       const float* logit_scale, float* out, float* lse, void* stream);

int rba_decode_logpos(const rba_attn_params* params,
                      const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                      const float* rel, const int32_t* seq_lens,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                      void* workspace, size_t workspace_bytes, const float* logit_scale,
                      float* out, float* lse, void* stream);

/* Host-only argument check of rba_prefill (no HIP call; same return codes). */
int rba_validate_prefill(const rba_attn_params* params,
                         const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                         const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                         const float* out);

/*
 * Paged decode / speculative verify with split-KV and a log-sum-exp combine.
 * Sources: "Inkling-Small on Gaudi 2", section "Attention with a relative
 * bias" (decode keys at block-ordinal positions); "vLLM TML Inkling Support",
 * section "Low-Latency Collectives and Kernels" (split count chosen from batch
 * and KV length); "Inkling on Two DGX Sparks ...", section "Wall 1" (split-KV
 * decode, dv may be 64, no device-to-host reads); "Inkling 2 Small on vLLM:
 * Day-0 Support", integration section (each KV block read once for all query
 * heads sharing it; several verify tokens per sequence).
 *
 *   q            device bf16 [batch * n_q, Hq, 128]; row b*n_q + u is token u of
 *                sequence b, at position seq_lens[b] - n_q + u
 *   k_cache, v_cache, num_blocks, block_tables, max_blocks_per_seq: as rba_prefill
 *   rel          device fp32 [batch * n_q, Hq, R]
 *   seq_lens     device int32 [batch]; includes the n_q new tokens (n_q <= seq_lens[b])
 *   n_q          query tokens per sequence, 1 <= n_q and G * n_q <= 256
 *                (G = Hq / Hkv); causal among themselves
 *   max_seq_len  host upper bound of seq_lens (sets the split plan and the grid)
 *   num_splits   0 = automatic (rba_decode_plan_splits with this device's CU
 *                count), else 1 <= num_splits <= 1024
 *   workspace    device memory of at least rba_decode_workspace_size(...) bytes
 *                (partial outputs; contents on entry are ignored)
 *   out          device fp32 [batch * n_q, Hq, dv]; lse device fp32 [batch*n_q, Hq]
 *                or NULL
 * Errors: RBA_ERR_NULL, RBA_ERR_SHAPE, RBA_ERR_UNSUPPORTED, RBA_ERR_WORKSPACE,
 * RBA_ERR_HIP.
 */
int rba_decode(const rba_attn_params* params,
               const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
               const float* rel, const int32_t* seq_lens,
               const int32_t* block_tables, int32_t max_blocks_per_seq,
               int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
               void* workspace, size_t workspace_bytes,
               float* out, float* lse, void* stream);

/* Host-only argument check of rba_decode (no HIP call; same return codes). */
int rba_validate_decode(const rba_attn_params* params,
                        const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                        const float* rel, const int32_t* seq_lens,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                        const void* workspace, size_t workspace_bytes, const float* out);

/*
 * Split plan (host only, pure function). Returns the number of KV splits
 * rba_decode uses for num_splits = 0 on a device with `num_cus` compute units.
 * Work units are (sequence, KV head, 32-column group, split); up to two run
 * per CU at a time. With 33 to 64 columns (G * n_q) one unit covers both
 * column groups and one runs per CU. If one unit per CU (num_cus units)
 * covers max_seq_len with at most 32 blocks per split, and the kernel that
 * runs keeps the next block's loads in flight (G * n_q <= 16, head_dim_v <=
 * 64, or 33 to 64 columns), that is used; else if one round of units (two per
 * CU, one with 33 to 64 columns) covers it with at most 128 blocks per split,
 * that round; otherwise splits of ~32 blocks of max_seq_len. Never fewer than
 * ~16 blocks per split, at most 256 splits.
 * Returns a negative RBA_ERR_* code on bad arguments.
 */
int32_t rba_decode_plan_splits(const rba_attn_params* params, int32_t batch, int32_t n_q,
                               int32_t max_seq_len, int32_t num_cus);

/*
 * Bytes of workspace rba_decode needs (host only). num_splits = 0 plans with
 * the current device's CU count (256 when no device is visible). Returns 0 on
 * bad arguments.
 * Layout: fp32 partial outputs [batch*n_q, Hq, splits, dv] followed by fp32
 * partial log-sum-exp [batch*n_q, Hq, splits].
 */
size_t rba_decode_workspace_size(const rba_attn_params* params, int32_t batch, int32_t n_q,
                                 int32_t max_seq_len, int32_t num_splits);

/*
 * The two stages of rba_decode, callable one at a time (rba_decode is exactly
 * rba_decode_split followed by rba_decode_combine on the same stream).
 * rba_decode_split writes, for every (row, head, split), the split's
 * normalised partial output and its log-sum-exp into `workspace` (a split
 * that sees no key gets lse = -inf). rba_decode_combine merges them:
 *   LSE = log sum_s exp(lse_s),  out = sum_s exp(lse_s - LSE) * O_s.
 * `num_splits` must be the resolved count (>= 1) for both calls.
 */
int rba_decode_split(const rba_attn_params* params,
                     const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                     const float* rel, const int32_t* seq_lens,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                     void* workspace, size_t workspace_bytes, void* stream);

int rba_decode_combine(const rba_attn_params* params, int32_t batch, int32_t n_q,
                       int32_t num_splits, const void* workspace, size_t workspace_bytes,
                       float* out, float* lse, void* stream);

/*
 * Gated attention output (Inkling 2 Small). Source: "Inkling 2 Small on vLLM:
 * Day-0 Support", model-architecture section (the attention-output row of the
 * comparison table, and the paragraph on the Inkling backbone and recent
 * advances: a sigmoid gate on each head's output, paired with a per-token
 * attention sink). No formula is given; this library reads:
 *   sink  device fp32 [rows, Hq] or NULL: a logit (natural-log units, finite
 *         or -inf) per (query token, head) that joins the softmax normaliser
 *         with a zero value vector:
 *           out = sum_j e^(x_j) V_j / (sum_j e^(x_j) + e^sink),
 *           lse = log(sum_j e^(x_j) + e^sink)
 *   gate  device fp32 [rows, Hq] or NULL: out is multiplied by 1 / (1 + e^-gate)
 *         (lse is unchanged)
 * rows = total_q (prefill) or batch * n_q (decode). With both NULL each call
 * is exactly its ungated counterpart. sink and gate must be 4-byte aligned
 * (RBA_ERR_UNSUPPORTED otherwise); every other argument and error is as in
 * rba_prefill / rba_decode / rba_decode_combine. The decode's split stage is
 * unchanged (rba_decode_split or rba_decode_split_fp8); the sink and gate are
 * applied by the combine.
 */
int rba_prefill_gated(const rba_attn_params* params,
                      const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                      const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                      const float* sink, const float* gate,
                      float* out, float* lse, void* stream);

int rba_decode_gated(const rba_attn_params* params,
                     const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                     const float* rel, const int32_t* seq_lens,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                     void* workspace, size_t workspace_bytes,
                     const float* sink, const float* gate,
                     float* out, float* lse, void* stream);

int rba_decode_combine_gated(const rba_attn_params* params, int32_t batch, int32_t n_q,
                             int32_t num_splits, const void* workspace, size_t workspace_bytes,
                             const float* sink, const float* gate,
                             float* out, float* lse, void* stream);

/*
 * Decode over an FP8 KV cache. Source: "vLLM TML Inkling Support", section
 * "Future Roadmap" (FP8 for global attention, to cut the KV-cache cost). The
 * pages give no format or scale convention; this library reads:
 *   k_cache, v_cache  device e4m3 (OCP FP8: 1 sign, 4 exponent bits with bias
 *                7, 3 mantissa bits, no infinities, S.1111.111 = NaN), one
 *                byte per element, same [num_blocks, Hkv, 128, 128] and
 *                [num_blocks, Hkv, 128, dv] layouts as the bf16 cache
 *   k_scale, v_scale  per-tensor dequantization scales: the key / value used is
 *                the e4m3 value times the scale (finite, > 0)
 * Everything else (arguments, workspace, split plan, combine, errors) is as
 * rba_decode / rba_decode_split; the output is attention over the dequantized
 * K/V. rba_decode_fp8 = rba_decode_split_fp8 + rba_decode_combine.
 */
int rba_decode_fp8(const rba_attn_params* params,
                   const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                   float k_scale, float v_scale, const float* rel, const int32_t* seq_lens,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                   void* workspace, size_t workspace_bytes,
                   float* out, float* lse, void* stream);

int rba_decode_split_fp8(const rba_attn_params* params,
                         const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                         float k_scale, float v_scale, const float* rel, const int32_t* seq_lens,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Any combination of the optional terms above in one call: the gated output
 * (sink, gate; rba_prefill_gated / rba_decode_gated), the per-row logit scale
 * (rba_prefill_logpos / rba_decode_logpos) and the e4m3 K/V cache
 * (rba_decode_fp8; here also for the prefill, whose chunks attend to a cached
 * context held in FP8). Sources: those entry points' sections above. The
 * terms act at different places, so their composition is fixed: the logit
 * scale multiplies every logit of its row (scale * q.k + bias); the sink is a
 * separate logit that joins the softmax normaliser unscaled; the gate
 * multiplies the normalised output; with e4m3 K/V the keys and values used are
 * the dequantised ones. A NULL `options`, or one with every pointer NULL and
 * kv_e4m3 = 0, is the plain call (rba_prefill, rba_prefill_relproj without
 * sink and gate, rba_decode, rba_decode_split).
 */
typedef struct rba_call_options {
    const float* sink;         /* device fp32 [rows, Hq] or NULL (rows: total_q or batch * n_q)  */
    const float* gate;         /* device fp32 [rows, Hq] or NULL                                  */
    const float* logit_scale;  /* device fp32 [rows] or NULL; finite values                       */
    int32_t kv_e4m3;           /* 0: bf16 K/V; 1: e4m3 K/V (every entry point taking options);    */
                               /* other values RBA_ERR_SHAPE                                      */
    float k_scale, v_scale;    /* with kv_e4m3 = 1: dequantization scales (finite, > 0)           */
} rba_call_options;

/* rba_prefill with options (sink, gate, logit_scale, e4m3 K/V). Other
 * arguments and errors as rba_prefill (and rba_decode_fp8 for the cache
 * format and scales); sink, gate and logit_scale must be 4-byte aligned. */
int rba_prefill_ex(const rba_attn_params* params,
                   const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                   const float* rel, const int32_t* cu_q, const int32_t* seq_lens,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                   const rba_call_options* options, float* out, float* lse, void* stream);

/* rba_prefill_relproj with options (sink, gate, logit_scale, e4m3 K/V; the
 * logit scale also multiplies the bias made in the kernel). Other arguments
 * and errors as rba_prefill_relproj. */
int rba_prefill_relproj_ex(const rba_attn_params* params,
                           const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                           const void* r, const void* rel_proj, int32_t d_r, int32_t proj_heads,
                           const int32_t* cu_q, const int32_t* seq_lens,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t batch, int32_t max_q_len, int32_t max_seq_len,
                           const rba_call_options* options, float* out, float* lse, void* stream);

/* rba_decode with options (sink, gate, logit_scale, e4m3 K/V). Other
 * arguments and errors as rba_decode (and rba_decode_fp8 for the scales). */
int rba_decode_ex(const rba_attn_params* params,
                  const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                  const float* rel, const int32_t* seq_lens,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                  void* workspace, size_t workspace_bytes, const rba_call_options* options,
                  float* out, float* lse, void* stream);

/* rba_decode_split with options (logit_scale, e4m3 K/V). The sink and gate
 * act in the merge (rba_decode_combine_gated), so they must be NULL here
 * (RBA_ERR_UNSUPPORTED otherwise). num_splits must be resolved (>= 1). */
int rba_decode_split_ex(const rba_attn_params* params,
                        const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                        const float* rel, const int32_t* seq_lens,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                        void* workspace, size_t workspace_bytes, const rba_call_options* options,
                        void* stream);

/*
 * Decode with the bias made from the R branch instead of a materialised rel.
 * Source: "Inkling-Small on Gaudi 2", section "Attention with a relative
 * bias" (each layer forms rel as r times its rel_logits_proj and hands it to
 * the attention call); the same reading as rba_prefill_relproj (one r vector
 * of width d_r per token and query head; one projection shared by the heads
 * or one per head). A decode step's bias covers only its batch * n_q query
 * rows, batch * n_q * Hq * R floats, small next to the cached context the
 * step reads; so the call first forms those rows with a small kernel, into
 * the workspace, and then runs the rba_decode kernels on them.
 *
 *   r            device bf16 [batch * n_q, Hq, d_r], rows as q
 *   rel_proj     device bf16 [proj_heads, R, d_r], as rba_prefill_relproj
 *   d_r          32, 64 or 128 (RBA_ERR_UNSUPPORTED otherwise)
 *   proj_heads   1 or Hq (RBA_ERR_SHAPE otherwise)
 *   workspace    device memory of at least
 *                rba_decode_relproj_workspace_size(...) bytes, 16-byte
 *                aligned: the split partials as for rba_decode, then, from the
 *                next multiple of 256 bytes, the bias rows fp32
 *                [batch * n_q, Hq, R]. Its contents on entry are ignored.
 *   options      as rba_decode_ex (NULL: none)
 *   all other arguments as rba_decode. The bias of distance d is
 *   sum_c r[t, h, c] * rel_proj[hp, d, c] (exact products, fp32 sum in
 *   the order of c) for 0 <= d < R and 0 beyond. r and rel_proj must be
 *   16-byte aligned.
 * Errors: as rba_decode_ex; every check runs before the first launch.
 */
size_t rba_decode_relproj_workspace_size(const rba_attn_params* params, int32_t batch, int32_t n_q,
                                         int32_t max_seq_len, int32_t num_splits);

int rba_decode_relproj(const rba_attn_params* params,
                       const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                       const void* r, const void* rel_proj, int32_t d_r, int32_t proj_heads,
                       const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                       int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                       void* workspace, size_t workspace_bytes, const rba_call_options* options,
                       float* out, float* lse, void* stream);

/*
 * rba_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The split partials go to a scratch array that the
 * library's code object holds on each GPU (RBA_NOALLOC_SCRATCH_BYTES bytes per
 * GPU, kept until the process ends); the call allocates nothing and calls no
 * allocating routine. Its contents on entry are ignored (every partial is
 * written before it is read), so nothing needs clearing between calls; but
 * every call on one GPU shares that GPU's array, so calls that overlap on one
 * GPU (several streams or threads at once) race and give wrong results.
 * Arguments, results and errors are as rba_decode (same kernels, same split
 * plan); RBA_ERR_WORKSPACE if the call needs more than
 * RBA_NOALLOC_SCRATCH_BYTES (see rba_decode_workspace_size), RBA_ERR_HIP if
 * the scratch address cannot be taken on the current device.
 */
#define RBA_NOALLOC_SCRATCH_BYTES (16u << 20)

int rba_decode_noalloc(const rba_attn_params* params,
                       const void* q, const void* k_cache, const void* v_cache, int32_t num_blocks,
                       const float* rel, const int32_t* seq_lens,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       int32_t batch, int32_t n_q, int32_t max_seq_len, int32_t num_splits,
                       float* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RBA_H */
