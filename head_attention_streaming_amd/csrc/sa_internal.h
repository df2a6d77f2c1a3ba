// Internal declarations shared by the HIP sources of libstreamattn.so (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// Attention launch description. Element strides are in 16-bit elements.
struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    int B, Hq, Hkv, Lq, Lk, d;
    int64_t q_bstride;   // between batches of q and out (= Lq*Hq*d)
    int64_t kv_bstride;  // between batches of k and v
    float scale;
    int win_left;        // visible keys of query i: [i+s-win_left, i+s+win_right], s = Lk - Lq;
    int win_right;       // -1 = unbounded (causal is (-1, 0))
    int dtype;           // SA_DTYPE_*
    void* ws;            // optional device workspace for balanced launches (null: none)
    int64_t ws_bytes;
    const float* gamma_q;  // optional RMSNorm weights [d] applied to each query row (null: none)
    float q_eps;
    const float* q_cs;     // optional RoPE table [Lq, d] (cos then sin per row) after the norm
    int q_rope;            // its pairing: 1 split, 2 interleaved
};

struct NormRopeArgs {
    const void* q_in;
    int64_t q_in_bstride;   // elements between batches of q_in (L*Hq*d when contiguous)
    void* q_out;
    int64_t q_out_bstride;
    const void* k_in;       // [B, L, Hkv, d] contiguous, or null
    void* k_out;
    int64_t k_out_bstride;
    const float* gamma_q;   // [d] (head scope) or [Hq*d] (inner scope)
    const float* gamma_k;   // [d] or [Hkv*d]
    const float* angles;    // [rows, d/2]; row of token p: p, or its logical cache row (ring_lc > 0)
    int B, L, Hq, Hkv, d;
    float eps;
    int norm_scope;         // 0 none, 1 head, 2 inner
    int rope_style;         // 0 none, 1 split, 2 interleaved
    int rope_keys;          // rotate the k rows too (0: keys are normalised only)
    int out_fp8;            // outputs are OCP FP8 E4M3 (1 byte) instead of bf16; strides in elements
    int ring_lc, ring_nsink, ring_nwin;  // ring_lc > 0: token p is physical row p of a rolling
    int64_t ring_chunk;                  // cache after chunk ring_chunk was written
    const void* v_in;       // [B, L, Hkv, d] contiguous, or null: value rows copied (cast to the
    void* v_out;            // output type) unnormalised and unrotated
    int64_t v_out_bstride;
    float* cs_out;          // [L, d] fp32, or null: cos then sin of token p's angles in row p
};

// Rolling sink + window cache after chunk c has been written (sizes in chunks of Lc tokens):
// the logical (arrival-order) row of physical row s, for s below the visible length. Sink
// chunk u sits in slot u; window chunk c' sits in slot n_sink + (c' - n_sink) mod n_win; the
// visible sequence is the sinks, then the window chunks oldest first.
__host__ __device__ inline int64_t ring_logical_row(int64_t s, int Lc, int n_sink, int n_win, int64_t c) {
    const int64_t u = s / Lc, i = s % Lc;
    if (u < n_sink) return s;
    const int64_t w = u - n_sink;                                   // window slot
    const int64_t held = c - (((c - n_sink - w) % n_win) + n_win) % n_win;  // chunk in slot w
    const int64_t first = c - n_win + 1 > n_sink ? c - n_win + 1 : n_sink;  // oldest visible window chunk
    return ((int64_t)n_sink + (held - first)) * Lc + i;
}

struct CopyArgs {
    const void* src;
    void* dst;
    int B;
    int64_t row_elems;   // elements per (batch) block to copy = Lc*Hkv*d
    int64_t dst_bstride; // elements between batches of dst
    int64_t dst_offset;  // element offset of the first destination row in each batch
    int cvt;             // 0: same-type 16-bit copy, 1: bf16 -> FP8 E4M3, 2: bf16 -> f16, 3: FP8 byte copy
};

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream);
int64_t attn_workspace_bytes(int d);  // workspace that lets every shape of this device run balanced
int64_t attn_scratch_bytes();          // size of the library-held scratch array (per GPU)
hipError_t attn_scratch(void** out);   // its device address on the current GPU
hipError_t launch_qk_norm_rope(const NormRopeArgs& a, hipStream_t stream);
hipError_t launch_copy_rows(const CopyArgs& a, hipStream_t stream);

}  // namespace sa
