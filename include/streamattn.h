/*
 * streamattn -- forward multi-head attention for streaming video models on MI355X (gfx950).
 *
 * C ABI of libstreamattn.so. Plain pointers and sizes only; no framework types.
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers (HIP global memory) unless stated otherwise.
 *   - Layouts are token-major and contiguous in the last dimension:
 *       queries / outputs  [B, Lq, Hq, d]
 *       keys / values      [B, Lk, Hkv, d]
 *     This is the [batch, length, heads, head_dim] layout of the page "flashdreams.accelerated",
 *     section "Multi Head Attention Definition" (reshaped Q, K, V) and of its FlashAttention2
 *     backend description (token-major queries, keys and values).
 *   - 16-bit element types: bfloat16 (SA_DTYPE_BF16) or IEEE binary16 (SA_DTYPE_F16). The
 *     accelerated-module guide restricts inputs to FP16/BF16 and head dims to powers of two in
 *     [16, 256]; this library builds d = 64 and d = 128 and rejects the rest with
 *     SA_ERR_UNSUPPORTED (no fallback kernel is ever substituted).
 *   - Element strides and offsets are int64.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Every call only
 *     enqueues kernels on that stream and returns; none synchronises.
 *   - Ownership: the caller allocates and frees every buffer, including the K/V cache. The
 *     library allocates no device memory at run time and keeps no caller pointer after a call
 *     returns; its only device memory is the scratch array of attn_forward_ws_static, part of
 *     its loaded code object.
 *   - Errors: arguments are validated on the host before anything is launched. A negative
 *     status means nothing was enqueued by that call (except SA_ERR_HIP, which reports a failed
 *     launch). sa_last_error() returns a thread-local text for the last failing call.
 *   - Base pointers must be 16-byte aligned (SA_ERR_ALIGN otherwise).
 */
#ifndef STREAMATTN_H
#define STREAMATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SA_OK = 0,
    SA_ERR_NULL = -1,        /* a required pointer is NULL */
    SA_ERR_SHAPE = -2,       /* inconsistent sizes (e.g. Hq % Hkv != 0, causal with Lq > Lk) */
    SA_ERR_UNSUPPORTED = -3, /* valid request outside what is built (e.g. d not in {64, 128}) */
    SA_ERR_ALIGN = -4,       /* a base pointer or stride is not 16-byte aligned */
    SA_ERR_RANGE = -5,       /* a size is negative or an element count overflows */
    SA_ERR_HIP = -6          /* the HIP runtime reported an error at launch */
} sa_status;

/* Element types. SA_DTYPE_FP8_E4M3 (attention inputs only): OCP FP8 E4M3, the unscaled
 * float8_e4m3fn of the quantized-SDPA option (page "flashdreams.accelerated", section
 * OptimizedMultiHeadAttention); q, k and v are one byte per element, out is bf16.
 * SA_DTYPE_BF16_F16V (attention only): q, k and out bf16, v f16 -- for a cache that keeps V in
 * the f16 type the P*V product uses (kv_cache_append_ex bf16 -> f16); the result is identical to
 * bf16 v with the same values rounded to f16, minus the per-tile conversion.
 * SA_DTYPE_FP8_E4M3_P8 (attention only, opt-in): as SA_DTYPE_FP8_E4M3, and the softmax
 * probabilities are rounded to E4M3 for an FP8 P*V product with V kept in E4M3 -- the FP8
 * softmax probabilities of the same page's quantized-SDPA option, which the page warns can make
 * attention inaccurate. Each probability p = 2^(s*scale*log2(e) - m + 8), m the row's running
 * maximum, carries a relative rounding error of at most 2^-4 while the row's scores span at most
 * 14 binades below it; the row sum adds the rounded values, so
 * |out - exact| <= (1/15) sum_j w_j |v_j - exact| + one bf16 ulp per element. */
enum { SA_DTYPE_BF16 = 0, SA_DTYPE_F16 = 1, SA_DTYPE_FP8_E4M3 = 2, SA_DTYPE_BF16_F16V = 3,
       SA_DTYPE_FP8_E4M3_P8 = 4 };

/* Q/K normalisation scope: none, per head (m = d), or inner (m = H*d: all heads of a token). */
enum { SA_NORM_NONE = 0, SA_NORM_HEAD = 1, SA_NORM_INNER = 2 };

/* RoPE pairing: none, split-half pairs (r, r + d/2), interleaved pairs (2r, 2r + 1).
 * SA_ROPE_AFTER_CACHE may be OR-ed into a pairing for qk_norm_rope: the queries are rotated,
 * the keys only normalised (the cache stores unrotated keys; kv_cache_rope rotates them). */
enum { SA_ROPE_NONE = 0, SA_ROPE_SPLIT = 1, SA_ROPE_INTERLEAVED = 2, SA_ROPE_AFTER_CACHE = 4 };

/*
 * qk_norm_rope -- Q/K prologue: RMSNorm, then RoPE, one rounding to bf16.
 *
 * Page "flashdreams.accelerated", section "Multi Head Attention Definition": the RMSNorm
 * equation gamma * z / sqrt(mean(z^2) + eps) with head scope (m = d, each head separately) or
 * inner scope (m = H*d, all heads of a token together), followed by the pair rotation
 * [[cos t, -sin t], [sin t, cos t]] with angle t = theta_{p,r}; V is neither normalised nor
 * rotated. With before-cache RoPE the rotated keys are what the K/V cache stores, so k_out may
 * point straight into a cache (see below). With after-cache RoPE (rope_style |
 * SA_ROPE_AFTER_CACHE) the keys are normalised and stored unrotated and only the queries are
 * rotated here; kv_cache_rope rotates the visible keys before attention.
 *
 *   q_in      [B, L, Hq, d] bf16 (device). q_out: [B, L, Hq, d] bf16, batch stride
 *             q_out_bstride elements (>= L*Hq*d; q_out == q_in is allowed: in place).
 *   k_in      [B, L, Hkv, d] bf16, or NULL for a query-only prologue (cross-attention).
 *   k_out     destination of the processed keys, row (b, p, h) at
 *             k_out + b*k_out_bstride + (p*Hkv + h)*d. To write into a cache
 *             [B, S, Hkv, d] at token slot s0, pass cache_k + s0*Hkv*d and S*Hkv*d.
 *             NULL iff k_in is NULL.
 *   gamma_q, gamma_k  fp32 RMSNorm weights, [d] for SA_NORM_HEAD, [Hq*d] / [Hkv*d] for
 *             SA_NORM_INNER (16-byte aligned); both NULL iff norm_scope == SA_NORM_NONE
 *             (gamma_k may be NULL when k_in is NULL). Inner scope with keys requires
 *             Hq == Hkv (the accelerated-module guide rules out inner-width norms for grouped
 *             heads); SA_ERR_UNSUPPORTED otherwise.
 *   rope_angles fp32 [L, d/2] host-built angles theta_{p,r} for the L positions of this chunk
 *             (device pointer); NULL iff rope_style == SA_ROPE_NONE. The same angles rotate q
 *             and k (positions are shared by the chunk's queries and keys).
 *   eps       RMSNorm epsilon (>= 0).
 * Arithmetic in fp32; the only rounding to bf16 is the final store.
 * Returns SA_OK, or SA_ERR_* as described at the top of this file.
 */
int qk_norm_rope(const void* q_in, void* q_out, int64_t q_out_bstride,
                 const void* k_in, void* k_out, int64_t k_out_bstride,
                 const float* gamma_q, const float* gamma_k, const float* rope_angles,
                 int B, int L, int Hq, int Hkv, int d, float eps,
                 int norm_scope, int rope_style, void* stream);

/*
 * qk_norm_rope_ex -- qk_norm_rope with a choice of output type.
 *
 * out_dtype SA_DTYPE_BF16 is qk_norm_rope. SA_DTYPE_FP8_E4M3 rounds the fp32 results once to
 * OCP FP8 E4M3 (nearest even; a value past 448 after rounding becomes NaN), the unscaled
 * float8_e4m3fn cast of the quantized-SDPA option (page "flashdreams.accelerated", section
 * OptimizedMultiHeadAttention), so q_out and k_out (e.g. an FP8 K cache) hold one byte per
 * element; their batch strides (elements) must then be multiples of 16.
 */
int qk_norm_rope_ex(const void* q_in, void* q_out, int64_t q_out_bstride,
                    const void* k_in, void* k_out, int64_t k_out_bstride,
                    const float* gamma_q, const float* gamma_k, const float* rope_angles,
                    int B, int L, int Hq, int Hkv, int d, float eps,
                    int norm_scope, int rope_style, int out_dtype, void* stream);

/*
 * qk_norm_rope_v -- qk_norm_rope_ex that also copies the chunk's values and can write the
 * cos/sin table of its angles: the per-chunk prologue of streaming self-attention in one launch
 * (the Q/K prologue and the value half of the "K/V cache updates" of page
 * "flashdreams.accelerated", section "Generic Multi Head Attention Interface").
 *
 * Arguments as qk_norm_rope_ex, and:
 *   q_in, q_out  may both be NULL (no query rows; gamma_q must then be NULL and Hq is ignored),
 *             for a caller that normalises the queries inside the attention (attn_forward_qnorm).
 *   v_in      [B, L, Hkv, d] bf16 contiguous values, or NULL; v_out receives them unchanged
 *             (rounded to E4M3 for out_dtype SA_DTYPE_FP8_E4M3) at v_out + b*v_out_bstride +
 *             (p*Hkv + h)*d, e.g. a cache's value rows at the chunk's slot. NULL iff v_in is NULL.
 *   rope_cs_out  fp32 [L, d], 16-byte aligned, device memory, or NULL: row p receives cos then
 *             sin (fp32, as used for the keys) of the d/2 angles of position p -- the table
 *             attn_forward_qnorm reads. Requires rope_style != SA_ROPE_NONE.
 * At least one of q_in, k_in, v_in must be given. The keys are rotated unless rope_style has
 * SA_ROPE_AFTER_CACHE; the values are never normalised or rotated.
 */
int qk_norm_rope_v(const void* q_in, void* q_out, int64_t q_out_bstride,
                   const void* k_in, void* k_out, int64_t k_out_bstride,
                   const void* v_in, void* v_out, int64_t v_out_bstride,
                   const float* gamma_q, const float* gamma_k, const float* rope_angles, float* rope_cs_out,
                   int B, int L, int Hq, int Hkv, int d, float eps,
                   int norm_scope, int rope_style, int out_dtype, void* stream);

/*
 * kv_cache_slot -- rolling sink + window cache: where chunk `chunk_idx` is written and how
 * many cached tokens the chunk then attends to. Pure host integer function (no device work).
 *
 * Page "flashdreams.accelerated", section "Generic Multi Head Attention Interface": the
 * BlockKVCache storage is [B, sink_size + window_size, H, d]; before_update(chunk_idx) precedes
 * the attention call and the current chunk is written into the rolling cache before it is
 * queried. Page "Accelerated building blocks" (section "Cache lifecycle"): chunk, window and
 * sink sizes are fixed. Slot rule (sizes in tokens, multiples of chunk_len Lc;
 * n_sink = sink_size/Lc, n_win = window_size/Lc >= 1):
 *     slot_base(c)   = c*Lc                                   if c < n_sink (sinks stay)
 *                    = sink_size + ((c - n_sink) mod n_win)*Lc otherwise (window ring)
 *     visible_len(c) = min((c + 1)*Lc, sink_size + window_size)
 * Attention over physical slots [0, visible_len) equals attention over the chunks in arrival
 * order, because non-causal attention does not depend on key order and before-cache RoPE has
 * already placed the positions in the stored keys.
 *   slot_base_out, visible_len_out: HOST pointers receiving the results.
 * Returns SA_OK, SA_ERR_NULL, or SA_ERR_RANGE (negative chunk index, Lc <= 0, sizes not
 * multiples of Lc, window_size < Lc, or a result that does not fit).
 */
int kv_cache_slot(int64_t chunk_idx, int chunk_len, int sink_size, int window_size,
                  int64_t* slot_base_out, int* visible_len_out);

/*
 * kv_cache_append -- copy one chunk of keys and/or values into its cache slot range.
 *
 * Same page and section as kv_cache_slot ("K/V cache updates" of the streaming attention).
 *   k_new, v_new   [B, Lc, Hkv, d] 16-bit (device); either may be NULL (skipped), not both.
 *                  k_new is NULL when qk_norm_rope already wrote the rotated keys.
 *   cache_k, cache_v  [B, sink_size + window_size, Hkv, d]; a cache whose source is NULL may
 *                  also be NULL.
 * Rows [slot_base, slot_base + Lc) of every batch are overwritten (slot_base from
 * kv_cache_slot); all other rows are untouched. A byte copy: bit-exact.
 */
int kv_cache_append(const void* k_new, const void* v_new, void* cache_k, void* cache_v,
                    int B, int Lc, int Hkv, int d, int sink_size, int window_size,
                    int64_t chunk_idx, void* stream);

/*
 * kv_cache_positions -- logical row of every visible physical row of the rolling cache after
 * chunk `chunk_idx` has been written. Pure host integer function (no device work).
 *
 * Same cache as kv_cache_slot. The visible keys in logical (arrival) order are the sink chunks,
 * then the window chunks oldest first; physical row s holds logical row logical_rows_out[s] for
 * s in [0, visible_len). This is the position order after-cache RoPE uses (kv_cache_rope).
 *   logical_rows_out  HOST array of `capacity` >= visible_len entries.
 * Returns SA_OK, SA_ERR_NULL, or SA_ERR_RANGE (as kv_cache_slot, or capacity too small).
 */
int kv_cache_positions(int64_t chunk_idx, int chunk_len, int sink_size, int window_size,
                       int64_t* logical_rows_out, int capacity);

/*
 * kv_cache_rope -- after-cache RoPE: rotate every visible cached key for the current step.
 *
 * Page "flashdreams.accelerated", section "Multi Head Attention Definition", RoPE after the K/V
 * cache update: the cache stores unrotated keys, and right before attention every visible key
 * is rotated with the angles of its current position; the page "Accelerated building blocks"
 * (section "Cache lifecycle") calls these cache-relative frequencies. The current position of
 * a key is its logical row in the visible sequence (kv_cache_positions).
 *   cache_k      [B, S, Hkv, d] bf16 unrotated keys, S = sink_size + window_size (device).
 *   k_rot        [B, S, Hkv, d] bf16 output (device, must not be cache_k): rows
 *                [0, visible_len) of every batch get the rotated keys of the same physical
 *                rows, so attention over k_rot pairs each key with the value in its cache row.
 *                Other rows are not written.
 *   rope_angles  fp32 [visible_len, d/2] (device), row r = angles theta_{r, .} of logical row r;
 *                the current chunk's queries use rows [visible_len - chunk_len, visible_len).
 *   rope_style   SA_ROPE_SPLIT or SA_ROPE_INTERLEAVED.
 * fp32 arithmetic, one rounding to bf16. Returns SA_OK or SA_ERR_* (kv_cache_slot's checks,
 * d not in {64, 128}, null or aliased pointers).
 */
int kv_cache_rope(const void* cache_k, void* k_rot, const float* rope_angles,
                  int B, int Hkv, int d, int chunk_len, int sink_size, int window_size,
                  int64_t chunk_idx, int rope_style, void* stream);

/*
 * kv_cache_append_ex -- kv_cache_append for caches kept in another element type.
 *
 * (src_dtype, cache_dtype): (bf16, bf16), (f16, f16) and (fp8, fp8) copy bytes; (bf16, fp8)
 * rounds each value to OCP FP8 E4M3 (nearest even, NaN past 448: the quantized-SDPA option
 * stores its K/V cache in float8_e4m3fn); (bf16, f16) rounds to binary16 (exact for |v| in
 * [2^-14, 65504]). Any other pair is SA_ERR_UNSUPPORTED. Same slot rule and layout as
 * kv_cache_append, with one cache element per source element.
 */
int kv_cache_append_ex(const void* k_new, const void* v_new, void* cache_k, void* cache_v,
                       int B, int Lc, int Hkv, int d, int sink_size, int window_size,
                       int64_t chunk_idx, int src_dtype, int cache_dtype, void* stream);

/*
 * attn_forward -- scaled dot-product attention forward pass, bf16 in and out.
 *
 * Page "flashdreams.accelerated", section "Multi Head Attention Definition", attention
 * equation: out_h = softmax(Q_h K_h^T * scale) V_h for every head h (scale = 1/sqrt(d) in
 * that equation; passed explicitly here). Computed tile by tile with an online softmax, so
 * the Lq x Lk score matrix is never stored; the result equals the definition up to rounding.
 *   q, out   [B, Lq, Hq, d] bf16; k, v [B, Lk, Hkv, d] bf16 (all device, contiguous).
 *   Hq % Hkv == 0: query head h reads key/value head h / (Hq / Hkv) (grouped heads).
 *   causal   0 or 1. With 1, query i sees key j iff j <= i + (Lk - Lq) (queries aligned to
 *            the end of the keys); requires Lq <= Lk.
 *   Lk >= 1; Lq == 0 or B == 0 is a successful no-op. d in {64, 128}.
 * Accumulation in fp32; probabilities enter the P*V product as fp16 (V converted exactly for
 * |v| in [2^-17, 65504]); the output is rounded once to bf16.
 */
int attn_forward(const void* q, const void* k, const void* v, void* out,
                 int B, int Hq, int Hkv, int Lq, int Lk, int d,
                 float scale, int causal, void* stream);

/* attn_forward_f16 -- the same operation with IEEE binary16 q, k, v and out. */
int attn_forward_f16(const void* q, const void* k, const void* v, void* out,
                     int B, int Hq, int Hkv, int Lq, int Lk, int d,
                     float scale, int causal, void* stream);

/*
 * attn_forward_kvstride -- attention over the first Lk tokens of a larger K/V buffer, such as
 * a rolling cache [B, S, Hkv, d] with S >= Lk (streaming self-attention) or a static context
 * cache (cross-attention). kv_bstride is the element distance between batches of k and v
 * (S*Hkv*d for a cache; >= Lk*Hkv*d; a multiple of 16 bytes). dtype is SA_DTYPE_BF16 or
 * SA_DTYPE_F16 for all four tensors, SA_DTYPE_FP8_E4M3 (or, opt-in, SA_DTYPE_FP8_E4M3_P8) for q,
 * k and v with a bf16 out, or SA_DTYPE_BF16_F16V (bf16 q, k, out; f16 v).
 * FP8: Q K^T runs on the FP8 MFMA with fp32 accumulation from the exact E4M3 values; V is
 * widened exactly to f16 and P V is computed as for 16-bit inputs (f16 probabilities), so the
 * only FP8 rounding is the caller's cast of Q, K and V. Otherwise identical to attn_forward.
 */
int attn_forward_kvstride(const void* q, const void* k, const void* v, void* out,
                          int B, int Hq, int Hkv, int Lq, int Lk, int d,
                          float scale, int causal, int64_t kv_bstride, int dtype, void* stream);

/*
 * attn_forward_window -- local (sliding-window) attention over a K/V buffer with batch stride.
 *
 * Page "optimizing-attention-flash", workflow 2, "Step 3: Enable advanced features": sliding
 * window (local) attention, a (left, right) window around each query. Query i sits at key
 * position p_i = i + (Lk - Lq) (queries aligned to the end of the keys, as with causal) and
 * sees key j iff p_i - window_left <= j <= p_i + window_right; a bound of -1 is unbounded.
 * (-1, 0) is causal attention, (-1, -1) full attention; a causal window of w tokens back is
 * (w, 0), the page's causal=True with a left window.
 *   window_left, window_right  >= -1. With window_right >= 0, Lq <= Lk + window_right is
 *            required so that every query sees at least one key (SA_ERR_SHAPE otherwise).
 * Key tiles that lie outside every query's band of a workgroup are skipped, so the work is
 * proportional to the keys in the band. Everything else (dtypes included) as
 * attn_forward_kvstride.
 */
int attn_forward_window(const void* q, const void* k, const void* v, void* out,
                        int B, int Hq, int Hkv, int Lq, int Lk, int d,
                        float scale, int window_left, int window_right,
                        int64_t kv_bstride, int dtype, void* stream);

/*
 * attn_forward_workspace_bytes -- size of the workspace that lets attn_forward_ws balance any
 * launch of head dim d on the current device (two partial-result slots per persistent
 * workgroup, one workgroup per CU: 37.7 MB at d = 128 and 21.0 MB at d = 64 on 256 CUs).
 * Returns the byte count, or SA_ERR_UNSUPPORTED for d not in {64, 128}. Host function.
 */
int64_t attn_forward_workspace_bytes(int d);

/*
 * attn_forward_ws -- attn_forward_window with a caller-provided device workspace.
 *
 * Same operation, arguments and results as attn_forward_window (dtype as attn_forward_kvstride;
 * window (-1, -1) is full attention). The workspace (16-byte aligned device memory of
 * workspace_bytes, no initialisation needed; NULL or too small: the plain launch) lets grids
 * of 256-row query blocks whose rounds would keep the CUs under 90 % busy -- e.g. 40 heads x 7
 * blocks = 280 blocks on 256 CUs -- run balanced: one persistent 8-wave workgroup per CU takes
 * the same number of whole query blocks, then an equal piece of the key tiles of the remaining
 * blocks; each piece hands over its partial (O, row maximum, row sum) through the workspace, and
 * a second kernel merges the pieces of each split block in key order (deterministic, no
 * atomics). Only for full-range (no causal, no window) attention whose key loop has at least 16
 * tiles of 64 keys (Lk > 960); other calls take the plain launch. Whole query blocks are
 * computed exactly as by the 8-wave plain launch; split ones equal it up to the rounding of the
 * merge (within the same bounds). At d = 128, grids with at most a quarter as many 128-row query
 * blocks as CUs over key loops of at least 32 tiles (Lk > 1984; few query rows over a long
 * context) split every block's key tiles the same way, into equal pieces on up to one
 * workgroup per CU. Calls that overlap on one workspace race.
 */
int attn_forward_ws(const void* q, const void* k, const void* v, void* out,
                    int B, int Hq, int Hkv, int Lq, int Lk, int d,
                    float scale, int window_left, int window_right, int64_t kv_bstride, int dtype,
                    void* workspace, int64_t workspace_bytes, void* stream);

/*
 * attn_forward_ws_static -- attn_forward_ws without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). This call allocates nothing: the partial results of a balanced launch go
 * to a scratch array the library holds in device memory, one per GPU (its address is looked up
 * on the first call on each device and kept), sized for one persistent workgroup per CU on up
 * to 256 CUs at d = 128 (37.7 MB; attn_forward_workspace_bytes(d) of an MI355X). A device that
 * would need more returns SA_ERR_UNSUPPORTED before anything is launched.
 * Operation, arguments, results and errors otherwise as attn_forward_ws with a workspace of
 * that size: the same kernels, so the same bits. Every call on one GPU shares that GPU's array
 * (it keeps the last call's partials; nothing needs clearing), so calls that overlap on one GPU
 * -- on different streams or host threads -- race; serialise them. The stream must belong to the
 * current device.
 */
int attn_forward_ws_static(const void* q, const void* k, const void* v, void* out,
                           int B, int Hq, int Hkv, int Lq, int Lk, int d,
                           float scale, int window_left, int window_right, int64_t kv_bstride, int dtype,
                           void* stream);

/*
 * attn_forward_qnorm -- attn_forward_ws with the query prologue fused into the attention: each
 * query row z is replaced by gamma_q * z / sqrt(mean(z^2) + eps) (RMSNorm, head scope), then,
 * when rope_style is SA_ROPE_SPLIT or SA_ROPE_INTERLEAVED, rotated by RoPE with the cos/sin
 * table rope_cs, and rounded once to the query type as it is loaded and attended with. Page
 * "flashdreams.accelerated", section "Multi Head Attention Definition" (RMSNorm of Q per head,
 * then RoPE, before attention; the cross-attention example normalises Q without RoPE).
 *
 * q is read as given and not modified; the result equals qk_norm_rope (Q rows, head scope, the
 * same angles) followed by attn_forward_ws, up to the summation order of the row's sum of
 * squares (the normalised query can differ by one ulp of the query type in rare rounding ties).
 *   gamma_q   fp32 [d], 16-byte aligned, device memory. eps >= 0 and finite.
 *   rope_cs   fp32 [Lq, d], 16-byte aligned, device memory: row i holds cos then sin of query
 *             row i's d/2 angles (the table qk_norm_rope_v writes), the same for every batch;
 *             NULL with rope_style SA_ROPE_NONE (0).
 * dtype SA_DTYPE_BF16, SA_DTYPE_F16 or SA_DTYPE_BF16_F16V (FP8 queries: SA_ERR_UNSUPPORTED).
 * Every other argument, the workspace (may be NULL) and the errors as attn_forward_ws.
 */
int attn_forward_qnorm(const void* q, const void* k, const void* v, void* out, const float* gamma_q, float eps,
                       const float* rope_cs, int rope_style, int B, int Hq, int Hkv, int Lq, int Lk, int d,
                       float scale, int window_left, int window_right, int64_t kv_bstride, int dtype,
                       void* workspace, int64_t workspace_bytes, void* stream);

/* Text describing the last non-zero status returned to this thread ("" if none). */
const char* sa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* STREAMATTN_H */
