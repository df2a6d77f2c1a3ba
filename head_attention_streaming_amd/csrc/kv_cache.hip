// Rolling K/V cache append for gfx950: copy one chunk [B, Lc, Hkv, d] into rows
// [slot_base, slot_base + Lc) of a cache [B, S, Hkv, d] (the "K/V cache updates" of streaming
// self-attention on the page "flashdreams.accelerated", section "Generic Multi Head Attention
// Interface"). Per batch the source chunk and the destination rows are each one contiguous
// range, so the kernel is a 16-byte vector copy; it is bit-exact and HBM-bound. Variants cast
// bf16 values to FP8 E4M3 or f16 on the way, for caches kept in those types.
#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;
// Two 16-byte vectors per thread: of 2, 4 and 8, the most workgroups in flight and the fastest
// append of a 1785-token chunk (8.1 us against 8.3 and 15.4 for 36.6 MB).
constexpr int kVecPerThread = 2;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// bf16 pair (one dword) -> two floats, exactly
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 bf16 -> 8 OCP FP8 E4M3, round to nearest even (the unscaled float8_e4m3fn cast)
__device__ __forceinline__ u32x2 bf16x8_to_e4m3x8(u32x4 x) {
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(x.x), bf16_hi(x.x), 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(x.y), bf16_hi(x.y), w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(x.z), bf16_hi(x.z), 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(x.w), bf16_hi(x.w), w1, true);
    return u32x2{(uint32_t)w0, (uint32_t)w1};
}

// 8 bf16 -> 8 f16, round to nearest even (exact for |v| in [2^-14, 65504])
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 x) {
    auto cv = [](uint32_t w) {
        f32x2 v = {bf16_lo(w), bf16_hi(w)};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    };
    return u32x4{cv(x.x), cv(x.y), cv(x.z), cv(x.w)};
}

// CVT 0: 16-bit copy, 3: byte copy (both 16 bytes -> 16 bytes); 1: bf16 -> E4M3 (16 -> 8 bytes);
// 2: bf16 -> f16 (16 -> 16 bytes). nvec = 16-byte source vectors per batch.
template <int CVT>
__global__ void __launch_bounds__(kThreads) copy_rows_kernel(CopyArgs a, int64_t nvec_per_batch) {
    constexpr int DST_EPV = CVT == 3 ? 16 : 8;  // destination elements per source vector
    using DstV = std::conditional_t<CVT == 1, u32x2, u32x4>;
    const u32x4* src = static_cast<const u32x4*>(a.src);
    DstV* dst = static_cast<DstV*>(a.dst);
    const int b = blockIdx.y;
    const int64_t dst0 = (b * a.dst_bstride + a.dst_offset) / DST_EPV;  // in destination vectors
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
        if (i < nvec_per_batch) {
            if constexpr (CVT == 1) dst[dst0 + i] = bf16x8_to_e4m3x8(r[u]);
            else if constexpr (CVT == 2) dst[dst0 + i] = bf16x8_to_f16x8(r[u]);
            else __builtin_nontemporal_store(r[u], dst + dst0 + i);  // streams out: -3 % against cached stores
        }
    }
}

}  // namespace

hipError_t launch_copy_rows(const CopyArgs& a, hipStream_t stream) {
    const int64_t nvec = a.row_elems / (a.cvt == 3 ? 16 : 8);
    const int64_t per_block = (int64_t)kThreads * kVecPerThread;
    const dim3 grid((unsigned)((nvec + per_block - 1) / per_block), (unsigned)a.B);
    switch (a.cvt) {
        case 1: hipLaunchKernelGGL(copy_rows_kernel<1>, grid, dim3(kThreads), 0, stream, a, nvec); break;
        case 2: hipLaunchKernelGGL(copy_rows_kernel<2>, grid, dim3(kThreads), 0, stream, a, nvec); break;
        case 3: hipLaunchKernelGGL(copy_rows_kernel<3>, grid, dim3(kThreads), 0, stream, a, nvec); break;
        default: hipLaunchKernelGGL(copy_rows_kernel<0>, grid, dim3(kThreads), 0, stream, a, nvec); break;
    }
    return hipGetLastError();
}

}  // namespace sa
