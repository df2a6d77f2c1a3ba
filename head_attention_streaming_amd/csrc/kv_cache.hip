// Rolling K/V cache append for gfx950: copy one chunk [B, Lc, Hkv, d] into rows
// [slot_base, slot_base + Lc) of a cache [B, S, Hkv, d] (the "K/V cache updates" of streaming
// self-attention on the page "flashdreams.accelerated", section "Generic Multi Head Attention
// Interface"). Per batch the source chunk and the destination rows are each one contiguous
// range, so the kernel is a 16-byte vector copy; it is bit-exact and HBM-bound.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;

__global__ void __launch_bounds__(kThreads) copy_rows_kernel(CopyArgs a, int64_t nvec_per_batch) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* src = static_cast<const u32x4*>(a.src);
    u32x4* dst = static_cast<u32x4*>(a.dst);
    const int b = blockIdx.y;
    const int64_t dst0 = (b * a.dst_bstride + a.dst_offset) / 8;  // in 16-byte vectors
    const int64_t src0 = b * nvec_per_batch;
    const int64_t base = (int64_t)blockIdx.x * kThreads * kVecPerThread + threadIdx.x;
    u32x4 r[kVecPerThread];
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        if (i < nvec_per_batch) r[u] = __builtin_nontemporal_load(src + src0 + i);  // read once
    }
#pragma unroll
    for (int u = 0; u < kVecPerThread; ++u) {
        const int64_t i = base + (int64_t)u * kThreads;
        if (i < nvec_per_batch) dst[dst0 + i] = r[u];
    }
}

}  // namespace

hipError_t launch_copy_rows(const CopyArgs& a, hipStream_t stream) {
    const int64_t nvec = a.row_elems / 8;
    const int64_t per_block = (int64_t)kThreads * kVecPerThread;
    const dim3 grid((unsigned)((nvec + per_block - 1) / per_block), (unsigned)a.B);
    hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(kThreads), 0, stream, a, nvec);
    return hipGetLastError();
}

}  // namespace sa
