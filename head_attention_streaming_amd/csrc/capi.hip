// C entry points of libstreamattn.so (declared in include/streamattn.h): host-side argument
// validation, the rolling-cache slot rule, and dispatch to the gfx950 kernels. Nothing here
// allocates device memory or synchronises; every failure is reported before any launch.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "sa_internal.h"
#include "streamattn.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return SA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
    return ok();
}

// element count a*b*c*d without overflow (int64), -1 if it would overflow
int64_t mul4(int64_t a, int64_t b, int64_t c, int64_t d) {
    const int64_t lim = INT64_C(1) << 62;
    int64_t r = 1;
    for (int64_t x : {a, b, c, d}) {
        if (x != 0 && r > lim / x) return -1;
        r *= x;
    }
    return r;
}

int check_attn(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int Lq,
               int Lk, int d, float scale, int win_left, int win_right, int64_t kv_bstride, int dtype) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Lq < 0 || Lk < 0)
        return fail(SA_ERR_RANGE, "attn_forward: negative or zero size (B=%d Hq=%d Hkv=%d Lq=%d Lk=%d)", B, Hq,
                    Hkv, Lq, Lk);
    if (dtype != SA_DTYPE_BF16 && dtype != SA_DTYPE_F16 && dtype != SA_DTYPE_FP8_E4M3 && dtype != SA_DTYPE_BF16_F16V &&
        dtype != SA_DTYPE_FP8_E4M3_P8)
        return fail(SA_ERR_UNSUPPORTED,
                    "attn_forward: dtype %d is not bf16 (0), f16 (1), fp8 e4m3 (2), bf16 with f16 v (3) or fp8 e4m3 with "
                    "fp8 probabilities (4)", dtype);
    if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "attn_forward: head dim %d not built (64, 128)", d);
    if (Hq % Hkv != 0) return fail(SA_ERR_SHAPE, "attn_forward: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (win_left < -1 || win_right < -1)
        return fail(SA_ERR_RANGE, "attn_forward: window bounds must be >= -1 (left=%d right=%d)", win_left, win_right);
    // with a right bound every query must see at least one key: the first query's band ends at
    // Lk - Lq + win_right, which must not fall before key 0
    if (win_right >= 0 && (int64_t)Lq > (int64_t)Lk + win_right)
        return fail(SA_ERR_SHAPE, "attn_forward: causal or right-bounded window needs Lq <= Lk + right (Lq=%d Lk=%d right=%d)",
                    Lq, Lk, win_right);
    if (!(scale > 0.f) || scale > 1e30f) return fail(SA_ERR_RANGE, "attn_forward: scale must be positive and finite");
    if (B == 0 || Lq == 0) return SA_OK + 1;  // nothing to do
    if (Lk == 0) return fail(SA_ERR_SHAPE, "attn_forward: Lk must be >= 1 when Lq > 0");
    if (!q || !k || !v || !out) return fail(SA_ERR_NULL, "attn_forward: null tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(SA_ERR_ALIGN, "attn_forward: tensor pointers must be 16-byte aligned");
    const int64_t nq = mul4(B, Lq, Hq, d);
    const int64_t nkv = mul4(1, Lk, Hkv, d);
    if (nq < 0 || nkv < 0 || (int64_t)Lq * Hq * d > INT32_MAX || (int64_t)Lk * Hkv * d > INT64_C(1) << 40)
        return fail(SA_ERR_RANGE, "attn_forward: tensor too large");
    if (kv_bstride < nkv) return fail(SA_ERR_SHAPE, "attn_forward: kv_bstride %lld < Lk*Hkv*d %lld",
                                      (long long)kv_bstride, (long long)nkv);
    const int elem_bytes = dtype == SA_DTYPE_FP8_E4M3 || dtype == SA_DTYPE_FP8_E4M3_P8 ? 1 : 2;
    if ((kv_bstride * elem_bytes) % 16)
        return fail(SA_ERR_ALIGN, "attn_forward: kv_bstride must be a multiple of 16 bytes");
    if (mul4(B, kv_bstride, 1, 1) < 0) return fail(SA_ERR_RANGE, "attn_forward: K/V extent overflows");
    const int64_t nblocks = (int64_t)((Lq + 127) / 128) * Hq * B;
    if (nblocks > INT32_MAX) return fail(SA_ERR_RANGE, "attn_forward: grid too large");
    return SA_OK;
}

int run_attn(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int Lq, int Lk, int d,
             float scale, int win_left, int win_right, int64_t kv_bstride, int dtype, void* stream,
             void* workspace = nullptr, int64_t workspace_bytes = 0, const float* gamma_q = nullptr,
             float q_eps = 0.f, const float* q_cs = nullptr, int q_rope = 0) {
    const int st = check_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, win_left, win_right, kv_bstride, dtype);
    if (st < 0) return st;
    if (st > 0) return ok();
    if (workspace && (!aligned16(workspace) || workspace_bytes < 0))
        return fail(SA_ERR_ALIGN, "attn_forward_ws: workspace must be 16-byte aligned");
    sa::AttnArgs a{};
    a.ws = workspace;
    a.ws_bytes = workspace ? workspace_bytes : 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Lq = Lq;
    a.Lk = Lk;
    a.d = d;
    a.q_bstride = (int64_t)Lq * Hq * d;
    a.kv_bstride = kv_bstride;
    a.scale = scale;
    // A bound that every query's band already reaches is dropped: query i sits at key i + Lk - Lq,
    // so left >= Lk - 1 reaches key 0 for all queries and right >= Lq - 1 reaches key Lk - 1.
    a.win_left = win_left >= Lk - 1 ? -1 : win_left;
    a.win_right = win_right >= Lq - 1 ? -1 : win_right;
    a.dtype = dtype;
    a.gamma_q = gamma_q;
    a.q_eps = q_eps;
    a.q_cs = q_cs;
    a.q_rope = q_rope;
    return hip_status(sa::launch_attn_fwd(a, static_cast<hipStream_t>(stream)), "attn_forward launch");
}

int check_causal(int causal) {
    return causal == 0 || causal == 1 ? SA_OK : fail(SA_ERR_RANGE, "attn_forward: causal must be 0 or 1");
}

}  // namespace

extern "C" {

const char* sa_last_error(void) { return g_err; }

int attn_forward(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int Lq, int Lk,
                 int d, float scale, int causal, void* stream) {
    if (check_causal(causal)) return SA_ERR_RANGE;
    return run_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, -1, causal ? 0 : -1, (int64_t)Lk * Hkv * d,
                    SA_DTYPE_BF16, stream);
}

int attn_forward_f16(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int Lq,
                     int Lk, int d, float scale, int causal, void* stream) {
    if (check_causal(causal)) return SA_ERR_RANGE;
    return run_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, -1, causal ? 0 : -1, (int64_t)Lk * Hkv * d,
                    SA_DTYPE_F16, stream);
}

int attn_forward_kvstride(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int Lq,
                          int Lk, int d, float scale, int causal, int64_t kv_bstride, int dtype, void* stream) {
    if (check_causal(causal)) return SA_ERR_RANGE;
    return run_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, -1, causal ? 0 : -1, kv_bstride, dtype, stream);
}

int64_t attn_forward_workspace_bytes(int d) {
    if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "attn_forward_workspace_bytes: head dim %d not built", d);
    ok();
    return sa::attn_workspace_bytes(d);
}

int attn_forward_ws(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int Lq, int Lk,
                    int d, float scale, int window_left, int window_right, int64_t kv_bstride, int dtype,
                    void* workspace, int64_t workspace_bytes, void* stream) {
    return run_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, window_left, window_right, kv_bstride, dtype, stream,
                    workspace, workspace_bytes);
}

int attn_forward_ws_static(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int Lq,
                           int Lk, int d, float scale, int window_left, int window_right, int64_t kv_bstride, int dtype,
                           void* stream) {
    // same validation as attn_forward_ws first, so bad arguments never touch the scratch array
    const int st = check_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, window_left, window_right, kv_bstride, dtype);
    if (st < 0) return st;
    if (st > 0) return ok();
    const int64_t need = sa::attn_workspace_bytes(d);
    if (need > sa::attn_scratch_bytes())
        return fail(SA_ERR_UNSUPPORTED, "attn_forward_ws_static: this device needs %lld bytes of partial-result scratch, "
                    "the library holds %lld (one workgroup per CU on up to 256 CUs)", (long long)need,
                    (long long)sa::attn_scratch_bytes());
    void* ptr = nullptr;
    const hipError_t e = sa::attn_scratch(&ptr);
    if (e != hipSuccess) return hip_status(e, "attn_forward_ws_static: scratch address");
    return run_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, window_left, window_right, kv_bstride, dtype, stream,
                    ptr, sa::attn_scratch_bytes());
}

int attn_forward_qnorm(const void* q, const void* k, const void* v, void* out, const float* gamma_q, float eps,
                       const float* rope_cs, int rope_style, int B, int Hq, int Hkv, int Lq, int Lk, int d,
                       float scale, int window_left, int window_right, int64_t kv_bstride, int dtype, void* workspace,
                       int64_t workspace_bytes, void* stream) {
    if (!gamma_q) return fail(SA_ERR_NULL, "attn_forward_qnorm: gamma_q is null");
    if (!aligned16(gamma_q)) return fail(SA_ERR_ALIGN, "attn_forward_qnorm: gamma_q must be 16-byte aligned");
    if (!(eps >= 0.f) || eps > 1e30f) return fail(SA_ERR_RANGE, "attn_forward_qnorm: eps must be >= 0 and finite");
    if (dtype == SA_DTYPE_FP8_E4M3 || dtype == SA_DTYPE_FP8_E4M3_P8)
        return fail(SA_ERR_UNSUPPORTED, "attn_forward_qnorm: the fused query norm takes 16-bit queries");
    if (rope_style != SA_ROPE_NONE && rope_style != SA_ROPE_SPLIT && rope_style != SA_ROPE_INTERLEAVED)
        return fail(SA_ERR_UNSUPPORTED, "attn_forward_qnorm: unknown RoPE pairing %d", rope_style);
    if ((rope_style != SA_ROPE_NONE) != (rope_cs != nullptr))
        return fail(SA_ERR_NULL, "attn_forward_qnorm: the cos/sin table must be given iff RoPE is enabled");
    if (rope_cs && !aligned16(rope_cs)) return fail(SA_ERR_ALIGN, "attn_forward_qnorm: rope_cs must be 16-byte aligned");
    return run_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, window_left, window_right, kv_bstride, dtype, stream,
                    workspace, workspace_bytes, gamma_q, eps, rope_cs, rope_style);
}

int attn_forward_window(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int Lq,
                        int Lk, int d, float scale, int window_left, int window_right, int64_t kv_bstride, int dtype,
                        void* stream) {
    return run_attn(q, k, v, out, B, Hq, Hkv, Lq, Lk, d, scale, window_left, window_right, kv_bstride, dtype,
                    stream);
}

int kv_cache_slot(int64_t chunk_idx, int chunk_len, int sink_size, int window_size, int64_t* slot_base_out,
                  int* visible_len_out) {
    if (!slot_base_out || !visible_len_out) return fail(SA_ERR_NULL, "kv_cache_slot: null output pointer");
    if (chunk_idx < 0 || chunk_len <= 0 || sink_size < 0 || window_size < chunk_len)
        return fail(SA_ERR_RANGE, "kv_cache_slot: need chunk_idx >= 0, chunk_len > 0, sink >= 0, window >= chunk");
    if (sink_size % chunk_len || window_size % chunk_len)
        return fail(SA_ERR_RANGE, "kv_cache_slot: sink (%d) and window (%d) must be multiples of chunk_len (%d)",
                    sink_size, window_size, chunk_len);
    if ((int64_t)sink_size + window_size > INT32_MAX) return fail(SA_ERR_RANGE, "kv_cache_slot: cache too large");
    const int64_t n_sink = sink_size / chunk_len;
    const int64_t n_win = window_size / chunk_len;
    const int64_t cap = (int64_t)sink_size + window_size;
    if (chunk_idx < n_sink)
        *slot_base_out = chunk_idx * chunk_len;
    else
        *slot_base_out = sink_size + ((chunk_idx - n_sink) % n_win) * chunk_len;
    const int64_t seen = chunk_idx >= cap / chunk_len ? cap : (chunk_idx + 1) * chunk_len;
    *visible_len_out = (int)(seen < cap ? seen : cap);
    return ok();
}

int kv_cache_append_ex(const void* k_new, const void* v_new, void* cache_k, void* cache_v, int B, int Lc, int Hkv,
                       int d, int sink_size, int window_size, int64_t chunk_idx, int src_dtype, int cache_dtype,
                       void* stream) {
    int64_t slot = 0;
    int vis = 0;
    const int st = kv_cache_slot(chunk_idx, Lc, sink_size, window_size, &slot, &vis);
    if (st != SA_OK) return st;
    if (B < 0 || Hkv <= 0) return fail(SA_ERR_RANGE, "kv_cache_append: B >= 0 and Hkv > 0 required");
    if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "kv_cache_append: head dim %d not built (64, 128)", d);
    int cvt = -1;
    if (src_dtype == cache_dtype && (src_dtype == SA_DTYPE_BF16 || src_dtype == SA_DTYPE_F16)) cvt = 0;
    else if (src_dtype == SA_DTYPE_FP8_E4M3 && cache_dtype == SA_DTYPE_FP8_E4M3) cvt = 3;
    else if (src_dtype == SA_DTYPE_BF16 && cache_dtype == SA_DTYPE_FP8_E4M3) cvt = 1;
    else if (src_dtype == SA_DTYPE_BF16 && cache_dtype == SA_DTYPE_F16) cvt = 2;
    if (cvt < 0)
        return fail(SA_ERR_UNSUPPORTED, "kv_cache_append: no conversion from dtype %d to cache dtype %d", src_dtype,
                    cache_dtype);
    if (!k_new && !v_new) return fail(SA_ERR_NULL, "kv_cache_append: both k_new and v_new are NULL");
    if ((k_new && !cache_k) || (v_new && !cache_v)) return fail(SA_ERR_NULL, "kv_cache_append: null cache pointer");
    for (const void* p : {k_new, v_new, (const void*)cache_k, (const void*)cache_v})
        if (p && !aligned16(p)) return fail(SA_ERR_ALIGN, "kv_cache_append: pointers must be 16-byte aligned");
    const int64_t row = (int64_t)Hkv * d;
    const int64_t chunk_elems = mul4(Lc, row, 1, 1);
    const int64_t cap = (int64_t)sink_size + window_size;
    if (chunk_elems < 0 || mul4(B, cap, row, 1) < 0) return fail(SA_ERR_RANGE, "kv_cache_append: tensor too large");
    if (B == 0) return ok();
    const int64_t nvec = chunk_elems / 8;
    if ((nvec + 1023) / 1024 > INT32_MAX || B > 65535) return fail(SA_ERR_RANGE, "kv_cache_append: grid too large");
    for (int which = 0; which < 2; ++which) {
        const void* src = which ? v_new : k_new;
        void* dst = which ? cache_v : cache_k;
        if (!src) continue;
        sa::CopyArgs c{};
        c.src = src;
        c.dst = dst;
        c.B = B;
        c.row_elems = chunk_elems;
        c.dst_bstride = cap * row;
        c.dst_offset = slot * row;
        c.cvt = cvt;
        const int s = hip_status(sa::launch_copy_rows(c, static_cast<hipStream_t>(stream)), "kv_cache_append launch");
        if (s != SA_OK) return s;
    }
    return ok();
}

int kv_cache_append(const void* k_new, const void* v_new, void* cache_k, void* cache_v, int B, int Lc, int Hkv,
                    int d, int sink_size, int window_size, int64_t chunk_idx, void* stream) {
    // a 16-bit byte copy: bf16 and f16 move alike
    return kv_cache_append_ex(k_new, v_new, cache_k, cache_v, B, Lc, Hkv, d, sink_size, window_size, chunk_idx,
                              SA_DTYPE_BF16, SA_DTYPE_BF16, stream);
}

int qk_norm_rope_v(const void* q_in, void* q_out, int64_t q_out_bstride, const void* k_in, void* k_out,
                   int64_t k_out_bstride, const void* v_in, void* v_out, int64_t v_out_bstride, const float* gamma_q,
                   const float* gamma_k, const float* rope_angles, float* rope_cs_out, int B, int L, int Hq, int Hkv,
                   int d, float eps, int norm_scope, int rope_style, int out_dtype, void* stream) {
    if (out_dtype != SA_DTYPE_BF16 && out_dtype != SA_DTYPE_FP8_E4M3)
        return fail(SA_ERR_UNSUPPORTED, "qk_norm_rope: output dtype %d is not bf16 (0) or fp8 e4m3 (2)", out_dtype);
    if (B < 0 || L < 0 || (q_in && Hq <= 0) || ((k_in || v_in) && Hkv <= 0))
        return fail(SA_ERR_RANGE, "qk_norm_rope: negative or zero size");
    if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "qk_norm_rope: head dim %d not built (64, 128)", d);
    if (norm_scope != SA_NORM_NONE && norm_scope != SA_NORM_HEAD && norm_scope != SA_NORM_INNER)
        return fail(SA_ERR_UNSUPPORTED, "qk_norm_rope: unknown norm scope %d", norm_scope);
    const int pairing = rope_style & ~SA_ROPE_AFTER_CACHE;
    if ((rope_style & ~(SA_ROPE_AFTER_CACHE | 3)) || pairing > SA_ROPE_INTERLEAVED ||
        (rope_style == SA_ROPE_AFTER_CACHE))
        return fail(SA_ERR_UNSUPPORTED, "qk_norm_rope: unknown RoPE style %d", rope_style);
    if (norm_scope == SA_NORM_INNER && q_in && k_in && Hkv != Hq)
        return fail(SA_ERR_UNSUPPORTED, "qk_norm_rope: inner-scope norm needs Hq == Hkv (grouped heads use head scope)");
    if (!(eps >= 0.f) || eps > 1e30f) return fail(SA_ERR_RANGE, "qk_norm_rope: eps must be >= 0 and finite");
    if (B == 0 || L == 0) return ok();
    if ((q_in == nullptr) != (q_out == nullptr)) return fail(SA_ERR_NULL, "qk_norm_rope: q_in and q_out must both be set or both NULL");
    if ((k_in == nullptr) != (k_out == nullptr)) return fail(SA_ERR_NULL, "qk_norm_rope: k_in and k_out must both be set or both NULL");
    if ((v_in == nullptr) != (v_out == nullptr)) return fail(SA_ERR_NULL, "qk_norm_rope: v_in and v_out must both be set or both NULL");
    if (!q_in && !k_in && !v_in) return fail(SA_ERR_NULL, "qk_norm_rope: no input rows");
    if (norm_scope != SA_NORM_NONE && ((q_in && !gamma_q) || (k_in && !gamma_k)))
        return fail(SA_ERR_NULL, "qk_norm_rope: RMSNorm weights required");
    if ((norm_scope == SA_NORM_NONE && (gamma_q || gamma_k)) || (!q_in && gamma_q) || (!k_in && gamma_k))
        return fail(SA_ERR_SHAPE, "qk_norm_rope: weights given for rows that are not normalised");
    if ((pairing != SA_ROPE_NONE) != (rope_angles != nullptr))
        return fail(SA_ERR_NULL, "qk_norm_rope: angles must be given iff RoPE is enabled");
    if (rope_cs_out && pairing == SA_ROPE_NONE)
        return fail(SA_ERR_SHAPE, "qk_norm_rope: a cos/sin table needs RoPE angles");
    for (const void* p : {q_in, (const void*)q_out, k_in, (const void*)k_out, v_in, (const void*)v_out,
                          (const void*)gamma_q, (const void*)gamma_k, (const void*)rope_cs_out})
        if (p && !aligned16(p)) return fail(SA_ERR_ALIGN, "qk_norm_rope: pointers must be 16-byte aligned");
    const int64_t nq = mul4(1, L, q_in ? Hq : 1, d);
    const int64_t nkv = mul4(1, L, (k_in || v_in) ? Hkv : 1, d);
    if (nq < 0 || nkv < 0 || mul4(B, L, (k_in || v_in) ? Hkv : 1, d) < 0 || mul4(B, L, q_in ? Hq : 1, d) < 0)
        return fail(SA_ERR_RANGE, "qk_norm_rope: tensor too large");
    const int align_elems = out_dtype == SA_DTYPE_FP8_E4M3 ? 16 : 8;  // 16-byte aligned batch strides
    if (q_in && (q_out_bstride < nq || q_out_bstride % align_elems)) return fail(SA_ERR_SHAPE, "qk_norm_rope: bad q_out_bstride");
    if (k_in && (k_out_bstride < nkv || k_out_bstride % align_elems))
        return fail(SA_ERR_SHAPE, "qk_norm_rope: bad k_out_bstride");
    if (v_in && (v_out_bstride < nkv || v_out_bstride % align_elems))
        return fail(SA_ERR_SHAPE, "qk_norm_rope: bad v_out_bstride");
    if ((int64_t)B * L > INT32_MAX) return fail(SA_ERR_RANGE, "qk_norm_rope: grid too large");
    sa::NormRopeArgs a{};
    a.q_in = q_in;
    a.q_in_bstride = q_in ? nq : 0;
    a.q_out = q_out;
    a.q_out_bstride = q_out_bstride;
    a.k_in = k_in;
    a.k_out = k_out;
    a.k_out_bstride = k_out_bstride;
    a.v_in = v_in;
    a.v_out = v_out;
    a.v_out_bstride = v_out_bstride;
    a.cs_out = rope_cs_out;
    a.gamma_q = gamma_q;
    a.gamma_k = gamma_k;
    a.angles = rope_angles;
    a.B = B;
    a.L = L;
    a.Hq = q_in ? Hq : 0;
    a.Hkv = (k_in || v_in) ? Hkv : 0;
    a.d = d;
    a.eps = eps;
    a.norm_scope = norm_scope;
    a.rope_style = pairing;
    a.rope_keys = (rope_style & SA_ROPE_AFTER_CACHE) ? 0 : 1;
    a.out_fp8 = out_dtype == SA_DTYPE_FP8_E4M3;
    return hip_status(sa::launch_qk_norm_rope(a, static_cast<hipStream_t>(stream)), "qk_norm_rope launch");
}

int qk_norm_rope_ex(const void* q_in, void* q_out, int64_t q_out_bstride, const void* k_in, void* k_out,
                    int64_t k_out_bstride, const float* gamma_q, const float* gamma_k, const float* rope_angles, int B,
                    int L, int Hq, int Hkv, int d, float eps, int norm_scope, int rope_style, int out_dtype,
                    void* stream) {
    if (out_dtype != SA_DTYPE_BF16 && out_dtype != SA_DTYPE_FP8_E4M3)
        return fail(SA_ERR_UNSUPPORTED, "qk_norm_rope: output dtype %d is not bf16 (0) or fp8 e4m3 (2)", out_dtype);
    if (B < 0 || L < 0 || Hq <= 0 || (k_in && Hkv <= 0))
        return fail(SA_ERR_RANGE, "qk_norm_rope: negative or zero size");
    if (B > 0 && L > 0 && (!q_in || !q_out)) {
        if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "qk_norm_rope: head dim %d not built (64, 128)", d);
        return fail(SA_ERR_NULL, "qk_norm_rope: null q pointer");
    }
    return qk_norm_rope_v(q_in, q_out, q_out_bstride, k_in, k_out, k_out_bstride, nullptr, nullptr, 0, gamma_q, gamma_k,
                          rope_angles, nullptr, B, L, Hq, Hkv, d, eps, norm_scope, rope_style, out_dtype, stream);
}

int qk_norm_rope(const void* q_in, void* q_out, int64_t q_out_bstride, const void* k_in, void* k_out,
                 int64_t k_out_bstride, const float* gamma_q, const float* gamma_k, const float* rope_angles, int B,
                 int L, int Hq, int Hkv, int d, float eps, int norm_scope, int rope_style, void* stream) {
    return qk_norm_rope_ex(q_in, q_out, q_out_bstride, k_in, k_out, k_out_bstride, gamma_q, gamma_k, rope_angles, B,
                           L, Hq, Hkv, d, eps, norm_scope, rope_style, SA_DTYPE_BF16, stream);
}

int kv_cache_positions(int64_t chunk_idx, int chunk_len, int sink_size, int window_size, int64_t* logical_rows_out,
                       int capacity) {
    int64_t base = 0;
    int vis = 0;
    const int st = kv_cache_slot(chunk_idx, chunk_len, sink_size, window_size, &base, &vis);
    if (st) return st;
    if (!logical_rows_out) return fail(SA_ERR_NULL, "kv_cache_positions: null output pointer");
    if (capacity < vis) return fail(SA_ERR_RANGE, "kv_cache_positions: output holds %d rows, %d visible", capacity, vis);
    for (int s = 0; s < vis; ++s)
        logical_rows_out[s] = sa::ring_logical_row(s, chunk_len, sink_size / chunk_len, window_size / chunk_len, chunk_idx);
    return ok();
}

int kv_cache_rope(const void* cache_k, void* k_rot, const float* rope_angles, int B, int Hkv, int d, int chunk_len,
                  int sink_size, int window_size, int64_t chunk_idx, int rope_style, void* stream) {
    int64_t base = 0;
    int vis = 0;
    const int st = kv_cache_slot(chunk_idx, chunk_len, sink_size, window_size, &base, &vis);
    if (st) return st;
    if (B < 0 || Hkv <= 0) return fail(SA_ERR_RANGE, "kv_cache_rope: negative or zero size");
    if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "kv_cache_rope: head dim %d not built (64, 128)", d);
    if (rope_style != SA_ROPE_SPLIT && rope_style != SA_ROPE_INTERLEAVED)
        return fail(SA_ERR_UNSUPPORTED, "kv_cache_rope: RoPE style must be split or interleaved");
    if (B == 0) return ok();
    if (!cache_k || !k_rot || !rope_angles) return fail(SA_ERR_NULL, "kv_cache_rope: null pointer");
    if (cache_k == k_rot) return fail(SA_ERR_SHAPE, "kv_cache_rope: k_rot must not be the cache (keys stay unrotated)");
    if (!aligned16(cache_k) || !aligned16(k_rot))
        return fail(SA_ERR_ALIGN, "kv_cache_rope: pointers must be 16-byte aligned");
    const int64_t S = (int64_t)sink_size + window_size;
    const int64_t bstride = mul4(S, Hkv, d, 1);
    if (bstride < 0 || mul4(B, bstride, 1, 1) < 0 || (int64_t)B * vis > INT32_MAX)
        return fail(SA_ERR_RANGE, "kv_cache_rope: cache too large");
    sa::NormRopeArgs a{};
    a.q_in = cache_k;
    a.q_in_bstride = bstride;
    a.q_out = k_rot;
    a.q_out_bstride = bstride;
    a.angles = rope_angles;
    a.B = B;
    a.L = vis;
    a.Hq = Hkv;
    a.Hkv = 0;
    a.d = d;
    a.norm_scope = SA_NORM_NONE;
    a.rope_style = rope_style;
    a.rope_keys = 1;
    a.ring_lc = chunk_len;
    a.ring_nsink = sink_size / chunk_len;
    a.ring_nwin = window_size / chunk_len;
    a.ring_chunk = chunk_idx;
    return hip_status(sa::launch_qk_norm_rope(a, static_cast<hipStream_t>(stream)), "kv_cache_rope launch");
}

}  // extern "C"
