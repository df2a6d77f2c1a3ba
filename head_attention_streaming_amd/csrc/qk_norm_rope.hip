// Q/K prologue for gfx950: per-head RMSNorm, then RoPE, one rounding to bf16.
//
// Page "flashdreams.accelerated", section "Multi Head Attention Definition": RMSNorm with head
// scope maps each head's feature vector z (m = d) to gamma * z / sqrt(mean(z^2) + eps); RoPE then
// rotates feature pair r of position p by theta_{p,r} (split-half pairs (r, r + d/2) or
// interleaved pairs (2r, 2r + 1)); normalisation comes before RoPE, and V is untouched.
//
// Memory-bound: each element is read once and written once. One workgroup handles one token
// (all query heads, then all key heads), so the token's d/2 angles are turned into cos/sin once
// (in LDS) and reused by every head. A head row of d features is spread over d/8 lanes holding 8
// features (one 16-byte load/store) each; the RMS reduction and the split-half partner exchange
// are lane shuffles inside that group.
#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

// 256 threads: 16 head rows per pass at d = 128, and eight passes of rows in flight per thread, so
// a token's Q, K and V rows load in one batch. Against 512-thread workgroups with four passes:
// twice the bytes in flight per CU; the one-launch prologue 4 % faster, kv_cache_rope 12 %.
constexpr int kThreads = 256;

// Cross-lane moves inside a 16-lane DPP row (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kQuadReverse = 0x1B;    // quad_perm [3,2,1,0]
constexpr int kRowMirror = 0x140;     // lane i <- lane 15-i of its 16-lane row
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7-i of its 8-lane half row
constexpr int kRowRotate8 = 0x128;    // lane i <- lane (i + 8) mod 16 of its row, i.e. i ^ 8

// Sum over the LPR (8 or 16) lanes holding one head row; every lane gets the total.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp<kQuadXor1>(x);
    x += dpp<kQuadXor2>(x);
    x += dpp<kRowHalfMirror>(x);
    if constexpr (LPR == 16) x += dpp<kRowMirror>(x);
    return x;
}

// Value held by the lane whose feature slice is half a head away (lane ^ LPR/2 within the group).
template <int LPR>
__device__ __forceinline__ float split_partner(float x) {
    if constexpr (LPR == 16) return dpp<kRowRotate8>(x);                      // i ^ 8 within 16 lanes
    else return dpp<kQuadReverse>(dpp<kRowHalfMirror>(x));                    // i ^ 4 within 8 lanes
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack_bf16x8(u32x4 w, float* f) {
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(a[i] << 16);
        f[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
    }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 pack_bf16x8(const float* f) {
    uint32_t a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x2 v = {f[2 * i], f[2 * i + 1]};
        a[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
    return u32x4{a[0], a[1], a[2], a[3]};
}

// 8 floats -> 8 OCP FP8 E4M3 bytes, round to nearest even; beyond 448 after rounding gives NaN
// (the unscaled float8_e4m3fn cast)
__device__ __forceinline__ u32x2_t pack_e4m3x8(const float* f) {
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
    return u32x2_t{(uint32_t)w0, (uint32_t)w1};
}

// NORM: the norm scope (0 none, 1 head, 2 inner) as a template parameter, so the head-scope
// kernel carries no inner-scope state. OUT8: outputs are FP8 E4M3 (one byte per element) instead
// of bf16. Seven 256-thread workgroups per CU (at most 72 VGPRs): the 1785 one-token workgroups
// of a 1785-token chunk are all resident at once instead of leaving a partial second round
// (A/B on one box against five per CU: one-launch Q/K/V prologue 23.7 -> 21.0 us, Q/K prologue
// -4 %).
template <int D, int NORM, bool OUT8>
__global__ void __launch_bounds__(kThreads, 7) qk_norm_rope_kernel(NormRopeArgs a) {
    using Out = std::conditional_t<OUT8, uint8_t, uint16_t>;
    constexpr int LPR = D / 8;            // lanes per head row
    constexpr int RPP = kThreads / LPR;   // head rows per pass
    constexpr int HALF = D / 2;
    __shared__ float cs[HALF], sn[HALF];
    __shared__ float gsh[2][D];  // head-scope weights of the query and key rows

    const int tok = blockIdx.x;           // b * L + p
    const int b = tok / a.L, p = tok % a.L;
    const int tid = threadIdx.x;
    const int li = tid % LPR;             // which 8-feature slice of the row
    const int rs = tid / LPR;             // row slot within a pass
    const int f0 = 8 * li;

    // rows of the token: Hq query rows, then Hkv key rows (if k_in), then Hkv value rows (if v_in)
    const int nk = a.k_in ? a.Hkv : 0;
    const int rows = a.Hq + nk + (a.v_in ? a.Hkv : 0);
    const uint16_t* qin = a.q_in ? static_cast<const uint16_t*>(a.q_in) + b * a.q_in_bstride + (int64_t)p * a.Hq * D : nullptr;
    const uint16_t* kin = a.k_in ? static_cast<const uint16_t*>(a.k_in) + ((int64_t)b * a.L + p) * a.Hkv * D : nullptr;
    const uint16_t* vin = a.v_in ? static_cast<const uint16_t*>(a.v_in) + ((int64_t)b * a.L + p) * a.Hkv * D : nullptr;
    Out* qout = a.q_out ? static_cast<Out*>(a.q_out) + b * a.q_out_bstride + (int64_t)p * a.Hq * D : nullptr;
    Out* kout = a.k_out ? static_cast<Out*>(a.k_out) + b * a.k_out_bstride + (int64_t)p * a.Hkv * D : nullptr;
    Out* vout = a.v_out ? static_cast<Out*>(a.v_out) + b * a.v_out_bstride + (int64_t)p * a.Hkv * D : nullptr;

    // Rows are handled NB passes at a time: all NB loads are issued before any is used, so each
    // thread keeps NB 16-byte reads in flight. rows_padded keeps every lane of a row group in
    // the loop (the shuffles need all of them); lanes past the last row compute on zeros.
    constexpr int NB = 8;
    const int rows_padded = (rows + RPP - 1) / RPP * RPP;
    u32x4 raw[NB];
    auto load_batch = [&](int base) __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int row = base + rs + nb * RPP;
            raw[nb] = u32x4{0u, 0u, 0u, 0u};
            if (row < rows) {
                const uint16_t* src = row < a.Hq        ? qin + row * D
                                      : row < a.Hq + nk ? kin + (row - a.Hq) * D
                                                        : vin + (row - a.Hq - nk) * D;
                raw[nb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + f0));
            }
        }
    };
    load_batch(0);  // in flight while the angles are turned into cos/sin

    if (a.rope_style != 0) {
        const int64_t arow = a.ring_lc > 0 ? ring_logical_row(p, a.ring_lc, a.ring_nsink, a.ring_nwin, a.ring_chunk) : p;
        for (int r = tid; r < HALF; r += kThreads) {
            float s, c;
            sincosf(a.angles[arow * HALF + r], &s, &c);
            cs[r] = c;
            sn[r] = s;
            if (a.cs_out && b == 0) {  // the table the attention's fused query RoPE reads
                a.cs_out[(int64_t)p * D + r] = c;
                a.cs_out[(int64_t)p * D + HALF + r] = s;
            }
        }
    }
    if constexpr (NORM == 1) {
        for (int r = tid; r < D; r += kThreads) {
            gsh[0][r] = a.q_in ? a.gamma_q[r] : 1.f;
            gsh[1][r] = a.k_in ? a.gamma_k[r] : 1.f;
        }
    }
    __syncthreads();

    // The per-lane constants (cos/sin of the lane's pairs, the weights of its features) are read
    // from LDS in every pass rather than held in registers: the offsets go through an empty asm
    // statement so that the compiler does not hoist the reads out of the loop. Split pairs:
    // features f0..f0+7 belong to pairs (f0 % HALF) + e; interleaved: pairs f0/2 + e for e < 4.
    const int cs_lane = a.rope_style == 1 ? f0 % HALF : f0 / 2;

    // Inner scope: one RMS over all of the token's query features (and one over its key
    // features), so the sums of squares are reduced over the workgroup before any row is
    // normalised. The first batch of rows is already in registers; later batches are read twice.
    float r_q = 1.f, r_k = 1.f;
    if constexpr (NORM == 2) {
        float sq = 0.f, sk = 0.f;
        for (int base = 0; base < rows_padded; base += NB * RPP) {
            if (base > 0) load_batch(base);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = base + rs + nb * RPP;
                float z[8];
                unpack_bf16x8(raw[nb], z);  // zeros past the last row
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += z[e] * z[e];
                if (row < a.Hq) sq += ss;
                else if (row < a.Hq + nk) sk += ss;
            }
        }
        __shared__ float red[2][kThreads / 64];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            sq += __shfl_xor(sq, off);
            sk += __shfl_xor(sk, off);
        }
        if ((tid & 63) == 0) {
            red[0][tid >> 6] = sq;
            red[1][tid >> 6] = sk;
        }
        __syncthreads();
        sq = sk = 0.f;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
            sq += red[0][w];
            sk += red[1][w];
        }
        r_q = 1.f / sqrtf(sq / (float)(a.Hq * D) + a.eps);
        if (a.Hkv) r_k = 1.f / sqrtf(sk / (float)(a.Hkv * D) + a.eps);
        if (rows_padded > NB * RPP) load_batch(0);
    }

    for (int base = 0; base < rows_padded; base += NB * RPP) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int row = base + rs + nb * RPP;
            if (base + nb * RPP >= rows_padded) break;  // uniform: past the last pass
            const bool valid = row < rows;
            const bool is_q = row < a.Hq;
            const bool is_v = row >= a.Hq + nk;  // copied as is (uniform per row group)
            float z[8];
            unpack_bf16x8(raw[nb], z);
            if constexpr (NORM == 1) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += z[e] * z[e];
                ss = group_sum<LPR>(ss);
                const float r = is_v ? 1.f : 1.f / sqrtf(ss / (float)D + a.eps);
                int goff = (is_q ? 0 : D) + f0;
                asm volatile("" : "+v"(goff));
                const float* gl = &gsh[0][0] + goff;
#pragma unroll
                for (int e = 0; e < 8; ++e) z[e] = (is_v ? 1.f : gl[e]) * (z[e] * r);
            } else if (NORM == 2 && valid && !is_v) {
                // weights of this row's features: gamma[h*d + f0 .. + 8]
                const f32x4* pg = reinterpret_cast<const f32x4*>(
                    is_q ? a.gamma_q + row * D + f0 : a.gamma_k + (row - a.Hq) * D + f0);
                const f32x4 g0 = pg[0], g1 = pg[1];
                const float r = is_q ? r_q : r_k;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z[e] = g0[e] * (z[e] * r);
                    z[e + 4] = g1[e] * (z[e + 4] * r);
                }
            }
            const int style = is_v ? 0 : (is_q || a.rope_keys) ? a.rope_style : 0;  // uniform per row group
            float o[8];
            if (style == 1) {
                const bool first = li < LPR / 2;
                int coff = cs_lane;
                asm volatile("" : "+v"(coff));
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float c = cs[coff + e], sv = sn[coff + e];
                    const float other = split_partner<LPR>(z[e]);
                    o[e] = first ? c * z[e] - sv * other : sv * other + c * z[e];
                }
            } else if (style == 2) {
                int coff = cs_lane;
                asm volatile("" : "+v"(coff));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float c = cs[coff + e], sv = sn[coff + e];
                    const float x0 = z[2 * e], x1 = z[2 * e + 1];
                    o[2 * e] = c * x0 - sv * x1;
                    o[2 * e + 1] = sv * x0 + c * x1;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = z[e];
            }
            if (valid) {
                // nontemporal stores: the rows stream out instead of lingering as dirty L2 lines
                // that the end of the kernel must write back (A/B on one box: the one-launch
                // prologue 4 % faster, kv_cache_rope 5 %, the streaming step that reads the rows
                // right after unchanged)
                Out* dst = is_q ? qout + row * D : !is_v ? kout + (row - a.Hq) * D : vout + (row - a.Hq - nk) * D;
                if constexpr (OUT8)
                    __builtin_nontemporal_store(pack_e4m3x8(o), reinterpret_cast<u32x2_t*>(dst + f0));
                else
                    __builtin_nontemporal_store(pack_bf16x8(o), reinterpret_cast<u32x4*>(dst + f0));
            }
        }
        if (base + NB * RPP < rows_padded) load_batch(base + NB * RPP);
    }
}

}  // namespace

template <int D, bool OUT8>
void launch_d(const NormRopeArgs& a, dim3 grid, hipStream_t stream) {
    if (a.norm_scope == 1)
        hipLaunchKernelGGL((qk_norm_rope_kernel<D, 1, OUT8>), grid, dim3(kThreads), 0, stream, a);
    else if (a.norm_scope == 2)
        hipLaunchKernelGGL((qk_norm_rope_kernel<D, 2, OUT8>), grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((qk_norm_rope_kernel<D, 0, OUT8>), grid, dim3(kThreads), 0, stream, a);
}

hipError_t launch_qk_norm_rope(const NormRopeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.B * a.L));
    if (a.d == 128) {
        if (a.out_fp8) launch_d<128, true>(a, grid, stream);
        else launch_d<128, false>(a, grid, stream);
    } else {
        if (a.out_fp8) launch_d<64, true>(a, grid, stream);
        else launch_d<64, false>(a, grid, stream);
    }
    return hipGetLastError();
}

}  // namespace sa
