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
};

struct NormRopeArgs {
    const void* q_in;
    void* q_out;
    int64_t q_out_bstride;
    const void* k_in;
    void* k_out;
    int64_t k_out_bstride;
    const float* gamma_q;
    const float* gamma_k;
    const float* angles;
    int B, L, Hq, Hkv, d;
    float eps;
    int norm_scope, rope_style;
};

struct CopyArgs {
    const void* src;
    void* dst;
    int B;
    int64_t row_elems;   // elements per (batch) block to copy = Lc*Hkv*d
    int64_t dst_bstride; // elements between batches of dst
    int64_t dst_offset;  // element offset of the first destination row in each batch
};

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream);
hipError_t launch_qk_norm_rope(const NormRopeArgs& a, hipStream_t stream);
hipError_t launch_copy_rows(const CopyArgs& a, hipStream_t stream);

}  // namespace sa
