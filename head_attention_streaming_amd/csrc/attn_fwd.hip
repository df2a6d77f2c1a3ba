// Attention forward kernel for gfx950 (MI355X): out = softmax(Q K^T * scale) V per head.
//
// The operation is the scaled dot-product attention equation of the page
// "flashdreams.accelerated", section "Multi Head Attention Definition". It is evaluated as an
// exact tiled attention with an online softmax (the IO-aware tiling the FlashAttention papers
// describe, which the "optimizing-attention-flash" page cites): keys are streamed in tiles, a
// running row maximum m and row sum l are kept in registers, and the partial output is
// rescaled by exp2(m_old - m_new) when the maximum grows far enough past m to matter (m may lag
// the true maximum; see the two checks at m's declaration). No score matrix is stored.
//
// Work decomposition (one workgroup = 128 or 256 query rows of one (batch, head)):
//   * each wave owns 32 query rows; its Q^T slice stays in registers as the MFMA B operand;
//   * K and V tiles of 32 or 64 keys are staged global -> registers -> LDS, double buffered, so
//     the next tile's global loads are in flight while the current tile is computed; an 8-wave
//     workgroup may instead split the keys between two groups of 4 waves, merged at the end;
//   * S^T = K Q^T with v_mfma_f32_32x32x16 (bf16 or f16): each lane then holds 16 scores of ONE
//     query column, so row max/sum are in-lane reductions plus one v_permlane32_swap;
//   * O^T += V^T P^T with v_mfma_f32_32x32x16_f16: the score registers, converted to f16, are
//     directly the B operand (no shuffle); V^T comes from LDS through ds_read_b64_tr_b16,
//     which returns 4 consecutive keys of one feature column per lane;
//   * exp2 with log2(e) folded into the scale; the output is divided by l once at the end.
// Probabilities use f16 (11-bit significand) for the P*V product; bf16 V is converted to f16
// when it is staged into LDS (exact for |v| in [2^-17, 65504]).
#include <mutex>
#include <type_traits>

#include "sa_internal.h"

// SA_LDS_CHECK=1 builds a check variant of the kernels (a separate library, compared bit for bit
// with the fast one by the tests): one LDS slot for K and one for V instead of two, each written
// only after a barrier that follows every read of its previous tile, and V staged after the
// P*V product that read the previous V. A barrier missing from the fast build's double-buffered
// pipeline would let a wave read a tile being overwritten; the check variant cannot, so the two
// builds' outputs would differ.
#ifndef SA_LDS_CHECK
#define SA_LDS_CHECK 0
#endif

namespace sa {
namespace {

constexpr bool kLdsCheck = SA_LDS_CHECK != 0;
// LDS slot of key tile t: double buffering, or the single slot of the check variant
__device__ __forceinline__ int lds_slot(int t) { return kLdsCheck ? 0 : (t & 1); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes as a native vector
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kLog2e = 1.4426950408889634f;

// Input element types (template parameter DT): bf16 or f16 (output in the same type), FP8 E4M3
// (OCP float8_e4m3fn, one byte; output bf16), or bf16 Q/K/out with f16 V (a cache that keeps V
// in the type the P*V product uses, so no tile is converted).
// FP8P: FP8 E4M3 q, k, v as kDtFP8, and the probabilities rounded to E4M3 for an FP8 P*V product
// with V kept in E4M3 (the quantized-SDPA option's FP8 softmax probabilities; opt-in).
// BF16P (chosen by the launch, not an ABI type): bf16 q, k, v with the probabilities rounded to
// bf16 for a bf16 P*V product, V staged as is -- for rows that all see at least
// kBf16ProbMinKeys keys, where the rounding averages out well inside the output bounds.
constexpr int kDtBF16 = 0, kDtF16 = 1, kDtFP8 = 2, kDtBF16VF16 = 3, kDtFP8P = 4, kDtBF16P = 5;

struct KParams {
    const void* q;  // [B, Lq, Hq, D] of the input type; strides below are in its elements
    const void* k;
    const void* v;
    uint16_t* out;  // [B, Lq, Hq, D] bf16 (f16 for f16 input)
    int Hq, Hkv, Lq, Lk, group, n_qblk, nblocks;
    int win_left, win_right;  // visible keys of query i: [i+s-left, i+s+right], s = Lk-Lq; -1 = unbounded
    int64_t q_bstride, kv_bstride;
    int q_tstride, kv_tstride;
    float c;  // scale * log2(e)
    // Balanced launches: each of the sk_wgs workgroups takes sk_full whole units, and the
    // surplus units from sk_full * sk_wgs on (sk_work = surplus x sk_tiles key tiles) are cut
    // into sk_wgs equal contiguous pieces whose partial results go to ws (2 slots per workgroup).
    int sk_tiles, sk_wgs, sk_full;
    int64_t sk_work;
    float* ws;
    // Optional RMSNorm of every query row (head scope) applied as it is loaded: weights [D]
    // (null: queries are used as given) and epsilon.
    const float* gamma_q;
    float q_eps;
    // Optional RoPE of the normalised query rows: table [Lq, D] fp32 (row i: cos then sin of
    // query row i's angles), pairing 1 split (r, r + D/2) or 2 interleaved (2r, 2r + 1).
    const float* q_cs;
    int q_rope;
    // Four key groups only: 1 = each workgroup takes the pair of query blocks (i, n_qblk - 1 - i)
    // of one (batch, head), its key groups divided between the two (causal rows, no left edge).
    int pair;
};

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 8 bf16 -> 8 f16 (exact for |v| in [2^-17, 65504]): each bf16 is widened to f32 (the low one
// by a shift, the high one by clearing the other half) and pairs are packed with RNE.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 x) {
    u32x4 r;
    r.x = pack_f16x2(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u));
    r.y = pack_f16x2(__uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u));
    r.z = pack_f16x2(__uint_as_float(x.z << 16), __uint_as_float(x.z & 0xffff0000u));
    r.w = pack_f16x2(__uint_as_float(x.w << 16), __uint_as_float(x.w & 0xffff0000u));
    return r;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// S^T block += K (32 keys x 64 features) * Q^T (64 features x 32 queries), FP8 E4M3 operands,
// unit block scales (E8M0 exponent 127). Lane (g, i) holds features [32g, 32g + 32) of its row
// in both operands (any feature order works if both operands use the same one).
__device__ __forceinline__ f32x16 mfma_qk_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16 FP8 E4M3 values -> 16 f16 (exact: every E4M3 value is an f16 value)
__device__ __forceinline__ uint32_t fp8x2_lo_to_f16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi_to_f16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}
__device__ __forceinline__ void fp8x16_to_f16x16(u32x4 x, u32x4& lo, u32x4& hi) {
    lo = u32x4{fp8x2_lo_to_f16x2(x.x), fp8x2_hi_to_f16x2(x.x), fp8x2_lo_to_f16x2(x.y), fp8x2_hi_to_f16x2(x.y)};
    hi = u32x4{fp8x2_lo_to_f16x2(x.z), fp8x2_hi_to_f16x2(x.z), fp8x2_lo_to_f16x2(x.w), fp8x2_hi_to_f16x2(x.w)};
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma_qk(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Calls f(integral_constant<int, i>) for i = 0 .. N-1, so array indices are compile-time
// constants and the staging arrays stay in registers.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (N > 0) {
        static_for<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// max / sum of a value with its copy in the other 32-lane half of the wave
__device__ __forceinline__ float half_swap_max(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Launch shapes. Every wave owns 32 query rows and every lane stays within 256 registers, so
// two waves share each SIMD:
//   8 waves, one key group (256 query rows) per workgroup, one workgroup per CU, 64-key tiles:
//     K/V tiles are staged once for 256 rows, so each thread converts and stores half as much;
//   4 waves (128 rows), two workgroups per CU: twice as many workgroups, for grids that would
//     otherwise leave CUs idle;
//   8 waves as two key groups of 4 (128 rows, each group half of the keys): for grids with at
//     most one 128-row workgroup per CU.
// Keys per tile, every shape (at d = 128 a 4-wave workgroup's double-buffered K/V tiles take
// 75.8 KB of LDS, so two workgroups per CU still fit; against 32-key tiles for that shape:
// cross-attention 1785 x 512 keys 1.5-3 % faster, d = 128 windows and causal within 2 %).
constexpr int kTileKeys = 64;

// 16-byte chunks a lane hands over for one partial unit: its O^T accumulators divided by the
// unit's row sum, as f16 pairs (a weighted mean of V rows, so within V's f16 range), two chunks
// per 32-feature block, then one chunk holding the running offset m and the row sum l of the
// piece's keys (fp32). Chunk c of the wave's 64 lanes is 1 KB contiguous ([chunk][lane]), so
// every hand-over store and merge load is 16 bytes per lane and coalesced.
template <int D>
constexpr int partial_chunks() { return 2 * (D / 32) + 1; }

// Integer min / max of 64-bit values (in device code the generic min / max of int64_t go through
// double precision).
__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

// Fourth word of a raw buffer resource on gfx9-family GPUs (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;

// Workgroup w of a balanced launch owns surplus positions [w_begin(w), w_begin(w + 1)).
__device__ __forceinline__ int64_t w_begin(const KParams& p, int w) { return p.sk_work * w / p.sk_wgs; }

template <int D, int DT, int NW, int KS, bool SK, bool BIG>
__global__ void __launch_bounds__(NW * 64, 8 / NW) attn_fwd_kernel(KParams p) {
    constexpr bool P8 = DT == kDtFP8P;                 // E4M3 probabilities and V in P*V
    constexpr bool FP8 = DT == kDtFP8 || P8;           // E4M3 q, k, v
    constexpr bool PB = DT == kDtBF16P;                        // bf16 probabilities and V in P*V
    constexpr bool BF16 = DT == kDtBF16 || DT == kDtBF16VF16 || PB;  // bf16 Q and K
    constexpr bool V_BF16 = DT == kDtBF16;                     // bf16 V, converted to f16 when staged
    constexpr bool OUT_BF16 = DT != kDtF16;                    // bf16 output
    using In = std::conditional_t<FP8, uint8_t, uint16_t>;
    constexpr int EPC = FP8 ? 16 : 8;            // input elements per 16-byte chunk
    constexpr int kRW = NW / KS;          // row waves per key group
    constexpr int kGThreads = kRW * 64;   // threads of one key group (they stage its tiles)
    constexpr int kBM = kRW * 32;         // query rows per workgroup
    // Four key groups split 64-row blocks for balance (d = 64 only: their double-buffered
    // 64-key tiles take 147 KB of LDS).
    static_assert(KS != 4 || D == 64, "four key groups only at d = 64");
    constexpr int kBN = kTileKeys;
    constexpr int KB = kBN / 32;  // 32-key score blocks per tile
    constexpr int KC = kBN / 16;  // 16-key P*V chunks per tile
    // LDS row stride of a K tile (input elements): 16 bytes of padding keep the b128 reads of
    // 16 consecutive rows on distinct banks
    constexpr int KST = D + 16 / (int)sizeof(In);
    // LDS row stride of a V tile: conflict-free transposed reads (D + 16 with four key groups,
    // whose tiles would not fit the LDS otherwise)
    constexpr int VST = KS == 4 ? D + 16 : D + 32;
    constexpr int DC = FP8 ? D / 64 : D / 16;  // QK MFMAs per 32-key block (64 or 16 features each)
    constexpr int DB = D / 32;    // 32-feature blocks of the O^T accumulator
    constexpr int CPR = D / EPC;  // 16-byte chunks per key row (global memory)
    constexpr int kChunks = kBN * CPR;
    constexpr int NCH = kChunks >= kGThreads ? kChunks / kGThreads : 1;  // chunks per thread per tile
    constexpr int RSTEP = kGThreads / CPR;      // key rows between a thread's chunks
    static_assert(kChunks < kGThreads ? kGThreads % kChunks == 0 && kChunks % 64 == 0
                                      : NCH * kGThreads == kChunks,
                  "tile must split evenly over the key group (or over whole waves of it)");
    static_assert(KS == 1 || KS == 2 || KS == 4, "one, two or four key groups");

    // Each key group owns two K slots and two V slots (double buffering) in LDS. K and V are
    // separate arrays so every LDS offset stays within the 16-bit immediate of ds_read/ds_write.
    constexpr int kKSlot = kBN * KST, kVSlot = kBN * VST;
    __shared__ __attribute__((aligned(16))) In Ks[KS][2 * kKSlot];
    // V tiles: f16 (converted from bf16 or E4M3 when staged), or the E4M3 bytes themselves for P8
    // (row stride D + 32 bytes: the transposed byte reads of eight rows then hit every bank once)
    using VT = std::conditional_t<P8, uint8_t, uint16_t>;
    __shared__ __attribute__((aligned(16))) VT Vs[KS][2 * kVSlot];
    // Output rows leave through LDS (see the epilogue): one area of 32 rows per row wave, waves
    // [0, kRW/2) in the K tile array and the others in the V tile array, when they fit.
    constexpr int OST = D + 8;         // LDS row stride of the output block (elements)
    constexpr int kOArea = 32 * OST;   // elements per row wave
    constexpr bool kLdsOut = !FP8 && (kRW / 2) * kOArea * 2 <= (int)sizeof(Ks) &&
                             (kRW - kRW / 2) * kOArea * 2 <= (int)sizeof(Vs);
    // (with paired blocks the lead of block B uses its own group's buffers)
    static_assert(KS != 4 || !kLdsOut || ((kRW / 2) * kOArea * 2 <= (int)sizeof(Ks) / KS &&
                                          (kRW - kRW / 2) * kOArea * 2 <= (int)sizeof(Vs) / KS),
                  "an output area must fit one group's tile buffers");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform over the wave: say so, so that values derived from it (the key
    // group, its tile indices, the buffer offsets) stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ks = KS == 1 ? 0 : wave / kRW;     // key group of this wave
    const int rw = KS == 1 ? wave : wave % kRW;  // row wave within the group
    const int g = lane >> 5;   // half of the wave
    const int j = lane & 31;   // query column owned by this lane

    // Workgroups are dealt round-robin to the 8 XCDs; regroup them so that each XCD works on a
    // contiguous range of (batch, head, query block) and its L2 serves the same K/V head.
    int bid = blockIdx.x;
    {
        const int nb = p.nblocks, base = nb >> 3, rem = nb & 7, x = bid & 7;
        bid = x * base + (x < rem ? x : rem) + (bid >> 3);
    }
    // One unit = one (batch, head, query block), over key tiles [seg_ta, seg_tb) when given
    // (balanced launches; otherwise the tiles the block's rows can see). part_slot >= 0: store
    // the unnormalised partial result there instead of the output.
    auto unit = [&](int ubid, int seg_ta, int seg_tb, int part_slot) __attribute__((always_inline)) {
    int qblk = ubid % p.n_qblk;
    int bh = ubid / p.n_qblk;
    if (p.win_right >= 0) qblk = p.n_qblk - 1 - qblk;  // causal-like bands: longest rows first
    // Paired blocks (four key groups, causal rows with no left edge): blocks A = i and
    // B = n_qblk - 1 - i see nA + nB = about n_qblk + 1 key tiles together; groups [0, kA) take A
    // and [kA, 4) take B, kA chosen so that the longer of the two groups' runs is shortest. Every
    // group runs S steps (they share the barriers); steps past a group's own run are dead. Both
    // blocks have at least one key tile (the entry points require Lq <= Lk + right, so every
    // query sees a key), so the step loop below runs for the groups of both blocks.
    const bool paired = KS == 4 && p.pair;
    int kA = KS, pS = 0;  // groups on block A; steps of every group
    if (paired) {
        const int npair = (p.n_qblk + 1) / 2;
        const int pi = ubid % npair;
        bh = ubid / npair;
        const int blkB = p.n_qblk - 1 - pi;
        auto tiles = [&](int blk) __attribute__((always_inline)) {
            const int last = min(blk * kBM + kBM, p.Lq) - 1;
            return (min(p.Lk, last + (p.Lk - p.Lq) + p.win_right + 1) + kBN - 1) / kBN;
        };
        const int nA = tiles(pi), nB = blkB != pi ? tiles(blkB) : 0;
        pS = (nA + KS - 1) / KS;
        if (nB > 0) {
            pS = 1 << 30;
            for (int k = 1; k < KS; ++k) {
                const int sk = max((nA + k - 1) / k, (nB + KS - k - 1) / (KS - k));
                if (sk < pS) { pS = sk; kA = k; }
            }
        }
        qblk = ks < kA ? pi : blkB;
    }
    const int h = bh % p.Hq;
    const int b = bh / p.Hq;
    const int hk = h / p.group;

    const int qb0 = qblk * kBM;
    const int r0 = qb0 + rw * 32;    // this wave's first query row
    const int qrow = r0 + j;
    const int shift = p.Lk - p.Lq;   // query i sits at key position i + shift
    const int qlast = min(qb0 + kBM, p.Lq) - 1;

    // Key tiles [t0, nkt) hold every key some row of the workgroup can see. Tiles in [t0, tl)
    // cut the left window edge and tiles in [tr, nkt) the right edge or the key tail for some
    // row; only those get per-element masks.
    const int kbeg = p.win_left >= 0 ? max(0, qb0 + shift - p.win_left) : 0;
    const int kend = p.win_right >= 0 ? min(p.Lk, qlast + shift + p.win_right + 1) : p.Lk;
    const int t0 = SK ? seg_ta : kbeg / kBN;
    const int nkt = SK ? seg_tb : (kend + kBN - 1) / kBN;
    int tl = t0;
    if (p.win_left >= 0) tl = max(t0, (qlast + shift - p.win_left + kBN - 1) / kBN);
    int tr = p.Lk / kBN;
    if (p.win_right >= 0) tr = min(tr, max(0, (qb0 + shift + p.win_right + 1) / kBN));
    // Key groups split [t0, nkt) into consecutive runs of nsteps tiles; every group runs the same
    // number of steps (they share the barriers), so the last group may step over tiles >= nkt:
    // those re-read the last tile and are masked out entirely (tr <= nkt).
    int nsteps = KS == 1 ? nkt - t0 : (nkt - t0 + KS - 1) / KS;
    int ta = t0 + ks * nsteps;
    int tend = KS == 1 ? nkt : ta + nsteps;
    int tv = tend;  // end of this group's own tiles
    if (paired) {  // this group's share of its block, then dead steps up to the common count
        const int ngrp = ks < kA ? kA : KS - kA, jg = ks < kA ? ks : ks - kA;
        nsteps = (nkt - t0 + ngrp - 1) / ngrp;
        ta = t0 + jg * nsteps;
        tv = ta + nsteps;
        tend = ta + pS;
        tr = min(tr, tv);
    }
    // this lane's visible keys [key_lo, key_lo + key_span] (rows past Lq may get an empty or
    // wrapped range; their scores are never stored)
    int key_lo, key_hi;
    {
        const int64_t pos = (int64_t)qrow + shift;
        key_lo = p.win_left >= 0 ? (int)max64(0, pos - p.win_left) : 0;
        key_hi = p.win_right >= 0 ? (int)min64(p.Lk - 1, pos + p.win_right) : p.Lk - 1;
        if (paired) key_hi = min(key_hi, tv * kBN - 1);
    }
    const unsigned key_span = (unsigned)(key_hi - key_lo);
    // keys some row of this wave can see, [wave_lo, wave_hi] (rows past Lq only widen it): an
    // edge tile outside it is skipped by this wave (its MFMAs, softmax and P*V), while the wave
    // still stages tiles and meets every barrier
    const int wave_lo = p.win_left >= 0 ? (int)max64(0, (int64_t)r0 + shift - p.win_left) : 0;
    const int wave_hi = min(p.win_right >= 0 ? (int)min64(p.Lk - 1, (int64_t)r0 + 31 + shift + p.win_right) : p.Lk - 1,
                            paired ? tv * kBN - 1 : 0x7fffffff);
    auto dead_tile = [&](int tt) __attribute__((always_inline)) { return tt * kBN > wave_hi || tt * kBN + kBN - 1 < wave_lo; };
    // Balanced launches have no windows or causal masks (only key tails), so no tile is dead
    // there; their kernel, at its register limit, keeps the plain sequence of steps.
    constexpr bool kSkipDead = !SK;

    // Q^T operand: lane (g, j) holds features [16c + 8g, 16c + 8g + 8) of its row (16-bit
    // inputs), or [64c + 32g, 64c + 32g + 32) (FP8, two 16-byte loads per MFMA).
    const In* const pq = static_cast<const In*>(p.q);
    const In* const pk = static_cast<const In*>(p.k);
    const In* const pv = static_cast<const In*>(p.v);
    using QOp = std::conditional_t<FP8, i32x8, u32x4>;
    QOp qf[DC];
    {
        const In* qp = pq + b * p.q_bstride + (int64_t)min(qrow, p.Lq - 1) * p.q_tstride + h * D + (FP8 ? 32 : 8) * g;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            if constexpr (FP8) {
                const u32x4 lo = *reinterpret_cast<const u32x4*>(qp + 64 * c);
                const u32x4 hi = *reinterpret_cast<const u32x4*>(qp + 64 * c + 16);
                qf[c] = __builtin_bit_cast(i32x8, (u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}));
            } else {
                qf[c] = *reinterpret_cast<const u32x4*>(qp + 16 * c);
            }
        }
    }
    // Staging geometry: thread tid copies 16-byte chunks (key row srow0 + u*RSTEP, EPC input
    // features from scol) of every tile; rows past Lk re-read row Lk - 1 (their scores are
    // masked). When a tile has fewer chunks than the group has threads, whole waves sit out.
    const int tid_g = KS == 1 ? tid : tid % kGThreads;
    const bool stager = kChunks >= kGThreads || tid_g < kChunks;
    const int srow0 = tid_g / CPR, scol = (tid_g % CPR) * EPC;
    // K and V rows of this (batch, K/V head) are read through buffer resources that end at row
    // Lk: rows at or past Lk fall outside the range and read as zero (their scores are masked).
    // A thread's byte offset is a constant plus the tile's first row; when the rows up to one
    // tile past Lk span 4 GiB or more (BIG), each tile gets a resource rebased at its first row
    // instead, so every offset stays within 32 bits.
    const char* const kbase = reinterpret_cast<const char*>(pk + b * p.kv_bstride + hk * D);
    const char* const vbase = reinterpret_cast<const char*>(pv + b * p.kv_bstride + hk * D);
    const uint32_t row_bytes = (uint32_t)p.kv_tstride * (uint32_t)sizeof(In);
    const uint32_t tile_bytes = (uint32_t)kBN * row_bytes;
    const uint32_t voff0 = (uint32_t)srow0 * row_bytes + (uint32_t)(scol * sizeof(In));
    const uint32_t region_bytes = BIG ? 0u : (uint32_t)p.Lk * row_bytes;
    const auto k_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase), (short)0, (int)region_bytes, kBufferWord3);
    const auto v_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase), (short)0, (int)region_bytes, kBufferWord3);
    auto tile_rsrc = [&](const char* base, int kt) __attribute__((always_inline)) {
        const int64_t row0 = (int64_t)kt * kBN;
        const int64_t bytes = min64(max64(0, p.Lk - row0) * row_bytes, 0xffffffffLL);
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + row0 * row_bytes), (short)0,
                                                  (int)(uint32_t)bytes, kBufferWord3);
    };
    In* const Kg = &Ks[ks][0];  // this group's K and V slots (V always f16 in LDS)
    VT* const Vg = &Vs[ks][0];
    In* ks_st = Kg + srow0 * KST + scol;
    VT* vs_st = Vg + srow0 * VST + scol;
    u32x4 kreg[NCH], vreg[NCH];
    auto load_rows = [&](u32x4 (&dst)[NCH], const char* base, const __amdgpu_buffer_rsrc_t& whole, int kt)
                         __attribute__((always_inline)) {
        if (!stager) return;
        if constexpr (!BIG) {
            const uint32_t toff = (uint32_t)kt * tile_bytes;
            static_for<NCH>([&](auto u) __attribute__((always_inline)) {
                dst[u] = __builtin_amdgcn_raw_buffer_load_b128(whole, voff0 + (toff + (uint32_t)(u * RSTEP) * row_bytes), 0, 0);
            });
        } else {
            const auto r = tile_rsrc(base, kt);
            static_for<NCH>([&](auto u) __attribute__((always_inline)) {
                dst[u] = __builtin_amdgcn_raw_buffer_load_b128(r, voff0 + (uint32_t)(u * RSTEP) * row_bytes, 0, 0);
            });
        }
    };
    auto load_k = [&](int kt) __attribute__((always_inline)) { load_rows(kreg, kbase, k_rsrc, kt); };
    auto load_v = [&](int kt) __attribute__((always_inline)) { load_rows(vreg, vbase, v_rsrc, kt); };
    auto store_k = [&](int slot) __attribute__((always_inline)) {
        if (!stager) return;
        static_for<NCH>([&](auto u) __attribute__((always_inline)) {
            *reinterpret_cast<u32x4*>(ks_st + slot * (kBN * KST) + u * RSTEP * KST) = kreg[u];
        });
    };
    auto store_v = [&](int slot) __attribute__((always_inline)) {
        if (!stager) return;
        static_for<NCH>([&](auto u) __attribute__((always_inline)) {
            VT* dst = vs_st + slot * (kBN * VST) + u * RSTEP * VST;
            if constexpr (P8) {
                *reinterpret_cast<u32x4*>(dst) = vreg[u];
            } else if constexpr (FP8) {
                u32x4 lo, hi;
                fp8x16_to_f16x16(vreg[u], lo, hi);
                *reinterpret_cast<u32x4*>(dst) = lo;
                *reinterpret_cast<u32x4*>(dst + 8) = hi;
            } else {
                *reinterpret_cast<u32x4*>(dst) = V_BF16 ? bf16x8_to_f16x8(vreg[u]) : vreg[u];
            }
        });
    };

    // The first tiles' loads go out right behind the query loads -- K(ta), V(ta) and K(ta + 1),
    // the last into registers of its own -- so for short key loops their latency overlaps the
    // queries' and the query norm's instead of following them (V(ta) and K(ta + 1) used to wait
    // for K(ta) to reach LDS). Balanced launches (key loops of 16+ tiles, at their register
    // limit) load K(ta + 1) after K(ta) is staged, as before.
    u32x4 knext[NCH];
    if (nkt > t0) {
        load_k(ta);
        load_v(ta);
        if constexpr (!SK) load_rows(knext, kbase, k_rsrc, min(ta + 1, nkt - 1));
    }
    if constexpr (!FP8) {
        if (p.gamma_q) {  // uniform. RMSNorm of the query row, then one rounding to the input type:
            // gamma * (z * r), r = 1 / sqrt(mean(z^2) + eps); this lane holds half of the row's
            // features, lane j + 32 (or j - 32) the other half
            float z[DC][8];
            float ss = 0.f;
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) {
                const uint32_t w[4] = {qf[cc].x, qf[cc].y, qf[cc].z, qf[cc].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (BF16) {
                        z[cc][2 * i] = __uint_as_float(w[i] << 16);
                        z[cc][2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
                    } else {
                        const f16x2 h2 = __builtin_bit_cast(f16x2, w[i]);
                        z[cc][2 * i] = (float)h2[0];
                        z[cc][2 * i + 1] = (float)h2[1];
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += z[cc][e] * z[cc][e];
            }
            const float r = 1.f / sqrtf(half_swap_sum(ss) / (float)D + p.q_eps);
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) {
                const f32x4* gp = reinterpret_cast<const f32x4*>(p.gamma_q + 16 * cc + 8 * g);
                const f32x4 g0 = gp[0], g1 = gp[1];
                const float gw[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
#pragma unroll
                for (int e = 0; e < 8; ++e) z[cc][e] = gw[e] * (z[cc][e] * r);
            }
            if (p.q_cs) {  // uniform. RoPE of the normalised row; both features of a pair are in this lane
                const float* cs_row = p.q_cs + (int64_t)min(qrow, p.Lq - 1) * D;
                if (p.q_rope == 1) {  // split pairs (r, r + D/2): feature 16c + 8g + e of chunks c, c + DC/2
#pragma unroll
                    for (int cc = 0; cc < DC / 2; ++cc) {
                        const f32x4* cp = reinterpret_cast<const f32x4*>(cs_row + 16 * cc + 8 * g);
                        const f32x4* sp = reinterpret_cast<const f32x4*>(cs_row + D / 2 + 16 * cc + 8 * g);
                        const f32x4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
                        const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                        const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float a0 = z[cc][e], b0 = z[cc + DC / 2][e];
                            z[cc][e] = cv[e] * a0 - sv[e] * b0;
                            z[cc + DC / 2][e] = sv[e] * a0 + cv[e] * b0;
                        }
                    }
                } else {  // interleaved pairs (2r, 2r + 1): r = 8c + 4g + e for e < 4
#pragma unroll
                    for (int cc = 0; cc < DC; ++cc) {
                        const f32x4 cv = *reinterpret_cast<const f32x4*>(cs_row + 8 * cc + 4 * g);
                        const f32x4 sv = *reinterpret_cast<const f32x4*>(cs_row + D / 2 + 8 * cc + 4 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float a0 = z[cc][2 * e], b0 = z[cc][2 * e + 1];
                            z[cc][2 * e] = cv[e] * a0 - sv[e] * b0;
                            z[cc][2 * e + 1] = sv[e] * a0 + cv[e] * b0;
                        }
                    }
                }
            }
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) {
                uint32_t w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[i] = BF16 ? pack_bf16x2(z[cc][2 * i], z[cc][2 * i + 1]) : pack_f16x2(z[cc][2 * i], z[cc][2 * i + 1]);
                qf[cc] = u32x4{w[0], w[1], w[2], w[3]};
            }
        }
    }

    // LDS read addresses (address space 3, so constant offsets fold into the instructions).
    typedef __attribute__((address_space(3))) const u32x4 lds_u4;
    // P8 reads the K rows of each 32-key block in the order 8a + 4b + c -> key 16(a >> 1) + 8b +
    // 4(a & 1) + c, so that score registers 0-7 (8-15) of lane half g hold the 8 consecutive keys
    // 8g + [0, 8) (16 + 8g + [0, 8)): the runs the transposed byte reads of V deliver.
    const int krow = P8 ? 16 * (j >> 4) + 8 * ((j >> 2) & 1) + 4 * ((j >> 3) & 1) + (j & 3) : j;
    lds_u4* kq_lane = (lds_u4*)(Kg + krow * KST + (FP8 ? 32 : 8) * g);
    // V^T operand addressing for ds_read_b64_tr_b16: loader lane L (within its 16-lane group G)
    // reads 4 features of key row (L / 4); the transpose hands lane L the 4 keys of feature L.
    const int G = lane >> 4, L16 = lane & 15;
    lds_i16x4* v_lane = (lds_i16x4*)(Vg + (4 * (G >> 1) + (L16 >> 2)) * VST + 16 * (G & 1) + 4 * (L16 & 3));
    // P8: ds_read_b64_tr_b8 -- loader lane L of a 16-lane group reads 8 bytes of key row L / 2 at
    // byte 8 (L % 2); lane i then holds byte i of those 8 rows (measured on the device). Group G
    // reads the keys of lane half g = G / 2 and features 16 (G % 2) + [0, 16) of a 32-feature block.
    lds_i32x2* v8_lane = (lds_i32x2*)((const uint8_t*)Vg + (8 * (G >> 1) + (L16 >> 1)) * VST + 16 * (G & 1) +
                                      8 * (L16 & 1));

    const float c = p.c;
    // Exponent offset m (log2 domain), a running maximum of the scores that may lag the true one;
    // a finite start value, so exp2 never sees inf - inf. Two ways to keep the lag safe:
    //  * max check: each step takes the tile's maximum right after S = K Q^T and raises m only
    //    when it exceeds m by more than kRescaleSlack (2^8 for 16-bit probabilities, so most
    //    tiles skip the O rescale and probabilities stay below 2^8);
    //  * sum check (kLazyMax): a tile's probabilities are computed against the current m, and
    //    this lane's sum of them -- the row-sum term the kernel forms anyway -- checks the lag:
    //    while every lane's sum is at most 2^15, every probability is at most 2^15 (inside f16
    //    range; fp32 O and l stay far from overflow) and the tile needs no maximum at all;
    //    otherwise (an f16 overflow shows as inf) the wave takes the tile's maximum, raises m to
    //    it, rescales O and l and computes the probabilities again. The first tile always does;
    //    later ones only when a tile's scores rise ~10 binades past m, so for such data m, and
    //    every result, is the same as with the max check. It saves the per-step maximum (16
    //    max3 of 32 scores, a lane swap, a ballot) and frees the score registers earlier.
    //    Measured on MI355X against the max check (A/B in one process; the same bits where no
    //    later tile rises 8+ binades past m): cross-attention 2 x 1785 x 512 keys -4 to -6 %
    //    time, causal [1,4096,64,128] -8 %, window (1024, 0) [1,8192,16,128] -7.5 %, balanced
    //    streaming attention -0.3 to -1.5 % (the 4-wave and balanced d = 128 kernels spill 9 and
    //    11 registers instead of 23 and 17), d = 64 8-wave launches of one key group -2.5 to
    //    -2.8 %; the plain launch with bf16 probabilities +0.7 %, FP8 +1.8 %, the other d = 64
    //    shapes (4-wave windows, four key groups) +2.8 to +4.4 %: those keep the max check.
    // P8 rounds the probabilities to E4M3 (largest 448), so it raises m with every new maximum and
    // offsets the exponent by 8: p = 2^(s c - m + 8) <= 2^8, normal down to 14 binades below m.
    constexpr bool kLazyMax = !FP8 && !(PB && !SK) && (D == 128 || (NW == 8 && KS == 1));
    constexpr float kRescaleSlack = P8 ? 0.0f : 8.0f;
    constexpr float kPOff = P8 ? 8.0f : 0.0f;
    constexpr float kSumLimit = 32768.0f;
    float m_run = -1e30f;
    float l_run = 0.f;  // this lane's share of the row sum (its own keys)
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    f32x16 s0[KB], s1[KB];  // scores of tile t live in s[(t - ta) & 1]
    u32x4 pf[KC];           // f16 probabilities of the previous tile (P^T operands)
    i32x8 pf8;              // P8: the previous tile's E4M3 probabilities (one 64-key P^T operand)

    // the largest score of a (masked) tile for this lane's query row, in log2 units
    auto tile_max = [&](const f32x16 (&sx)[KB]) __attribute__((always_inline)) {
        float mk[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            mk[kb] = fmaxf(sx[kb][0], sx[kb][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) mk[kb] = fmaxf(fmaxf(mk[kb], sx[kb][r]), sx[kb][r + 1]);
        }
        float mloc = mk[0];
#pragma unroll
        for (int kb = 1; kb < KB; ++kb) mloc = fmaxf(mloc, mk[kb]);
        return half_swap_max(mloc) * c;
    };
    // raise m to tmax (if larger) and rescale O and l to the new offset
    auto rescale = [&](float tmax) __attribute__((always_inline)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    };

    // One pipeline step t:  S(t) = K(t) Q^T  ||  P(t-1) = exp2(S(t-1) c - m)  [MFMA || VALU]
    //                       O += V(t-1) P(t-1)  ||  stage K(t+1), V(t); masks (max check: row max) of S(t)
    // K(t) and V(t) live in LDS slot t%2; step t overwrites the slots step t-1 read, and the
    // barrier closing each step orders those writes before the next step's reads.
    auto step = [&](auto do_qk, auto do_pv, auto do_mask, int t, f32x16 (&sc)[KB], f32x16 (&sp)[KB]) __attribute__((always_inline)) {
        constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value, MASK = decltype(do_mask)::value;
        // This wave's S = K Q^T products issue ahead of the other wave's softmax work on the SIMD:
        // raised issue priority until they are queued (measured +0.3 to +4 % across launch shapes).
        const bool qk_dead = kSkipDead && QK && MASK && dead_tile(t);   // uniform over the wave
        const bool pv_dead = kSkipDead && PV && MASK && dead_tile(t - 1);
        __builtin_amdgcn_s_setprio(1);
        if (QK && !qk_dead) {
            if constexpr (!FP8 && D == 64) {
                // d = 64: the K fragment reads run four MFMAs ahead of their products, an issue
                // order pinned for the scheduler (which otherwise waits on each read right
                // before its MFMA). Measured +2-5 % at d = 64; at d = 128 it gains nothing and
                // the extra registers cost the balanced launch 7-10 %.
                constexpr int NQ = KB * DC, kLook = NQ > 4 ? 4 : NQ - 1;
                static_assert(NQ > kLook, "more products than reads in flight");
                u32x4 kbuf[NQ];
                auto kread = [&](int i) __attribute__((always_inline)) {
                    kbuf[i] = kq_lane[(lds_slot(t) * kBN * KST + (i / DC) * 32 * KST + 16 * (i % DC)) / 8];
                };
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
                for (int i = 0; i < kLook; ++i) kread(i);
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    if (i + kLook < NQ) kread(i + kLook);
                    sc[i / DC] = mfma_qk<BF16>(kbuf[i], qf[i % DC], sc[i / DC]);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, kLook, 0);  // kLook LDS reads
#pragma unroll
                for (int i = 0; i < NQ - kLook; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, kLook, 0);
            } else {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
#pragma unroll
                    for (int cc = 0; cc < DC; ++cc) {
                        if constexpr (FP8) {
                            const int off = (lds_slot(t) * kBN * KST + kb * 32 * KST + 64 * cc) / 16;
                            const u32x4 lo = kq_lane[off], hi = kq_lane[off + 1];
                            sc[kb] = mfma_qk_fp8(__builtin_bit_cast(i32x8, (u32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w})),
                                                 qf[cc], sc[kb]);
                        } else {
                            sc[kb] = mfma_qk<BF16>(kq_lane[(lds_slot(t) * kBN * KST + kb * 32 * KST + 16 * cc) / 8], qf[cc], sc[kb]);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
        if (P8 && PV && !pv_dead) {
            // P(t-1) as E4M3: dword w holds contraction index 4w .. 4w + 3, i.e. score registers
            // (kb, r) = (w / 4, 4 (w % 4) + e); the row sum adds the rounded values (widened
            // exactly to f16 pairs) that the product uses
            const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
            const float mo = m_run - kPOff;
            float acc0 = 0.f, acc1 = 0.f;
            int pw[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int kb = w >> 2, r0 = 4 * (w & 3);
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sp[kb][r0 + e], c, -mo));
                int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
                v = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], v, true);
                pw[w] = v;
                acc0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, fp8x2_lo_to_f16x2((uint32_t)v)), one2, acc0, false);
                acc1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, fp8x2_hi_to_f16x2((uint32_t)v)), one2, acc1, false);
            }
            pf8 = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
            l_run += acc0 + acc1;
        }
        if (!P8 && PV && !pv_dead) {
            // P(t-1) as f16 (bf16) operands; the row sum adds the rounded values the product uses
            auto probs = [&]() __attribute__((always_inline)) {
                const f16x2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
                float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const int kb = kc >> 1, hh = kc & 1;
                    uint32_t w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sp[kb][8 * hh + 2 * e], c, -m_run));
                        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sp[kb][8 * hh + 2 * e + 1], c, -m_run));
                        if constexpr (PB) {
                            w[e] = pack_bf16x2(x0, x1);
                            const bf16x2 one_b = {(__bf16)1.0f, (__bf16)1.0f};
                            if (e & 1)
                                acc1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), one_b, acc1, false);
                            else
                                acc0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), one_b, acc0, false);
                        } else {
                            w[e] = pack_f16x2(x0, x1);
                            if (e & 1)
                                acc1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w[e]), one2, acc1, false);
                            else
                                acc0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w[e]), one2, acc0, false);
                        }
                    }
                    pf[kc] = u32x4{w[0], w[1], w[2], w[3]};
                }
                return acc0 + acc1;
            };
            float acc;
            if constexpr (kLazyMax) {
                // at most two passes (one copy of the code): the second after raising m to the
                // tile maximum when the first finds that m lags too far
                for (int pass = 0;; ++pass) {
                    acc = probs();
                    if (pass > 0 || !__builtin_amdgcn_ballot_w64(!(acc <= kSumLimit))) break;
                    rescale(tile_max(sp));
                }
            } else {
                acc = probs();
            }
            l_run += acc;
        }
        if constexpr (QK) {
            if constexpr (kLdsCheck) __syncthreads();  // every wave has read K(t) from the one K slot
            store_k(lds_slot(t + 1));  // K(t+1) (slot content unused when t + 1 == nkt)
            if constexpr (!kLdsCheck) store_v(lds_slot(t));  // V(t)
            load_k(min(t + 2, nkt - 1));
            if constexpr (!kLdsCheck) load_v(min(t + 1, nkt - 1));
        }
        if (P8 && PV && !pv_dead) {
            // O^T += V^T P^T on the FP8 MFMA, 64 keys per product: read m of a 32-feature block
            // brings keys 8 (2m + g) + [0, 8) of this lane's feature
            const int slot = lds_slot(t - 1);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                i32x2 r[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    r[m] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(v8_lane + (slot * kBN * VST + 16 * m * VST + 32 * db) / 8);
                const i32x8 va = {r[0].x, r[0].y, r[1].x, r[1].y, r[2].x, r[2].y, r[3].x, r[3].y};
                o[db] = mfma_qk_fp8(va, pf8, o[db]);
            }
        }
        if (!P8 && PV && !pv_dead) {
            const int slot = lds_slot(t - 1);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int off = (slot * kBN * VST + 16 * kc * VST + 32 * db) / 4;
                    const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(v_lane + off);
                    const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(v_lane + off + 2 * VST);
                    const i16x8 a8 = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                    if constexpr (PB)
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8),
                                                                         __builtin_bit_cast(bf16x8, pf[kc]), o[db], 0, 0, 0);
                    else
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a8),
                                                                        __builtin_bit_cast(f16x8, pf[kc]), o[db], 0, 0, 0);
                }
        }
        if constexpr (QK && kLdsCheck) {
            __syncthreads();  // every wave has read V(t-1) from the one V slot
            store_v(lds_slot(t));
            load_v(min(t + 1, nkt - 1));
        }
        if (QK && !qk_dead) {
            if constexpr (MASK) {
                // one unsigned compare and a select per score: key - key_lo in [0, key_span]
                // key of score register (kb, r) in lane half g: kb 32 + 8 (r / 4) + 4 g + r % 4, or
                // with P8's row order kb 32 + 8 g + r + 8 (r / 8)
                const int rel0 = t * kBN + (P8 ? 8 : 4) * g - key_lo;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const unsigned rel = (unsigned)(rel0 + kb * 32 + (P8 ? r + 8 * (r >> 3) : 8 * (r >> 2) + (r & 3)));
                        sc[kb][r] = rel <= key_span ? sc[kb][r] : -INFINITY;
                    }
            }
            if constexpr (!kLazyMax) {
                const float tmax = tile_max(sc);
                if (__builtin_amdgcn_ballot_w64(tmax > m_run + kRescaleSlack)) rescale(tmax);
            }
        }
        __syncthreads();
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    // steps t in [a, b) with both halves; S(t) lives in s0 when t - ta is even, s1 when odd
    auto middle = [&](auto do_mask, int a, int t1) __attribute__((always_inline)) {
        int t = a;
        if (t < t1 && ((t - ta) & 1)) step(T_{}, T_{}, do_mask, t++, s1, s0);
        for (; t + 1 < t1; t += 2) {
            step(T_{}, T_{}, do_mask, t, s0, s1);
            step(T_{}, T_{}, do_mask, t + 1, s1, s0);
        }
        if (t < t1) step(T_{}, T_{}, do_mask, t, s0, s1);
    };

    if (nkt > t0) {  // uniform over the workgroup: every group runs nsteps + 1 steps
        store_k(lds_slot(ta));
        if constexpr (SK)
            load_k(min(ta + 1, nkt - 1));
        else
            static_for<NCH>([&](auto u) __attribute__((always_inline)) { kreg[u] = knext[u]; });
        __syncthreads();
        const bool mask0 = ta < tl || ta >= tr;
        if (mask0) step(T_{}, F_{}, T_{}, ta, s0, s1);
        else step(T_{}, F_{}, F_{}, ta, s0, s1);
        // steps ta+1 .. tend-1 in three segments: left-edge masked, unmasked, right-edge masked.
        // A masked step also decides whether this wave skips the previous tile's softmax and
        // P*V, so when the tile before the unmasked run is masked, the run starts one step later
        // (that step's mask passes every score).
        auto masked = [&](int tt) __attribute__((always_inline)) { return tt < tl || tt >= tr; };
        int e1 = min(max(tl, ta + 1), tend);
        const int e2 = max(e1, min(tr, tend));
        if (kSkipDead && e1 < e2 && masked(e1 - 1)) ++e1;
        middle(T_{}, ta + 1, e1);
        middle(F_{}, e1, e2);
        middle(T_{}, e2, tend);
        const bool mlast = kSkipDead && masked(tend - 1);
        if ((tend - ta) & 1) {  // S(tend-1) in s0 when tend-1-ta is even
            if (mlast) step(F_{}, T_{}, T_{}, tend, s1, s0);
            else step(F_{}, T_{}, F_{}, tend, s1, s0);
        } else {
            if (mlast) step(F_{}, T_{}, T_{}, tend, s0, s1);
            else step(F_{}, T_{}, F_{}, tend, s0, s1);
        }
    }

    // the group that merges and stores this group's block: group 0, or kA for block B of a pair
    const int lead = paired && ks >= kA ? kA : 0;
    if constexpr (KS > 1) {
        // Merge the key groups' partial results through LDS (the tiles are no longer read: every
        // step ended with a barrier): (m, l, O) = (max_i m_i, sum_i l_i a_i, sum_i O_i a_i) with
        // a_i = exp2(m_i - m). The other groups of a block hand over m and l through the K
        // buffers and O through the V buffers, DBR 32-feature blocks per round; the block's lead
        // group merges and stores.
        constexpr int kOut = KS - 1;           // groups that hand over
        constexpr int kPerDb = kRW * 16 * 64;  // floats of one 32-feature block, all row waves of a group
        constexpr int kFit = (int)(sizeof(Vs) / 4 / (kPerDb * kOut));
        constexpr int DBR = kFit < DB ? kFit : DB;
        static_assert(DBR >= 1 && kOut * kRW * 128 * 4 <= (int)sizeof(Ks), "merge areas must fit in the tile buffers");
        float* const ml_base = reinterpret_cast<float*>(&Ks[0][0]) + rw * 128 + lane;
        float* const area_base = reinterpret_cast<float*>(&Vs[0][0]) + rw * (DBR * 16 * 64) + lane;
        auto ml = [&](int g) __attribute__((always_inline)) { return ml_base + (g - 1) * kRW * 128; };
        auto area = [&](int g) __attribute__((always_inline)) { return area_base + (g - 1) * kRW * (DBR * 16 * 64); };
        // Group gg hands its result to this wave's lead (uniform over the wave). Every group but
        // 0 writes its slot (block B's lead too), so a lead reads finite values from every slot
        // and weights the other block's groups by exp2(-inf) = 0, without branches.
        const int lead_end = paired && ks < kA ? kA : KS;
        auto member = [&](int gg) __attribute__((always_inline)) { return gg > lead && gg < lead_end; };
        if (ks > 0) {
            ml(ks)[0] = m_run;
            ml(ks)[64] = l_run;
        }
        __syncthreads();
        float a0 = 1.f, ag[kOut];
        if (ks == lead) {
            float mg[kOut], mn = m_run;
#pragma unroll
            for (int gg = 1; gg < KS; ++gg) {
                mg[gg - 1] = member(gg) ? ml(gg)[0] : -INFINITY;
                mn = fmaxf(mn, mg[gg - 1]);
            }
            a0 = __builtin_amdgcn_exp2f(m_run - mn);
            l_run *= a0;
#pragma unroll
            for (int gg = 1; gg < KS; ++gg) {
                ag[gg - 1] = __builtin_amdgcn_exp2f(mg[gg - 1] - mn);
                l_run += ml(gg)[64] * ag[gg - 1];
            }
        }
#pragma unroll
        for (int d0 = 0; d0 < DB; d0 += DBR) {
            if (ks > 0) {
                float* const mine = area(ks);
#pragma unroll
                for (int db = d0; db < d0 + DBR && db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mine[((db - d0) * 16 + r) * 64] = o[db][r];
            }
            __syncthreads();
            if (ks == lead) {
#pragma unroll
                for (int db = d0; db < d0 + DBR && db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float acc = o[db][r] * a0;
#pragma unroll
                        for (int gg = 1; gg < KS; ++gg) acc += area(gg)[((db - d0) * 16 + r) * 64] * ag[gg - 1];
                        o[db][r] = acc;
                    }
            }
            // the next round overwrites the areas, and after the last round the output rows
            // pass through the same buffers
            if (d0 + DBR < DB || kLdsOut) __syncthreads();
        }
        if (ks != lead) return;
    }

    if constexpr (SK) {
        if (part_slot >= 0) {  // split unit: hand over O / l, m, l (merged by attn_merge_kernel)
            constexpr int NC = partial_chunks<D>();
            u32x4* dst = reinterpret_cast<u32x4*>(p.ws) + ((int64_t)part_slot * NW + wave) * NC * 64 + lane;
            const float lt = half_swap_sum(l_run);
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            auto pk = [&](int db, int i) __attribute__((always_inline)) {
                return pack_f16x2(o[db][2 * i] * inv, o[db][2 * i + 1] * inv);
            };
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    dst[(2 * db + hh) * 64] = u32x4{pk(db, 4 * hh), pk(db, 4 * hh + 1), pk(db, 4 * hh + 2), pk(db, 4 * hh + 3)};
            dst[2 * DB * 64] = u32x4{__float_as_uint(m_run), __float_as_uint(lt), 0u, 0u};
            return;
        }
    }

    // ---- epilogue: O / l, one rounding to the output dtype
    const float l = half_swap_sum(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    auto packed = [&](int db, int rg) __attribute__((always_inline)) {  // features 32db + 8rg + 4g + [0, 4)
        const float x0 = o[db][4 * rg + 0] * inv, x1 = o[db][4 * rg + 1] * inv;
        const float x2 = o[db][4 * rg + 2] * inv, x3 = o[db][4 * rg + 3] * inv;
        u32x2 w;
        if constexpr (OUT_BF16) {
            w.x = pack_bf16x2(x0, x1);
            w.y = pack_bf16x2(x2, x3);
        } else {
            w.x = pack_f16x2(x0, x1);
            w.y = pack_f16x2(x2, x3);
        }
        return w;
    };
    // Rows leave through LDS (free after the last step's or merge round's barrier): each row wave
    // writes its 32 x D block to an area of its own, then stores whole rows, 16 bytes per lane. A
    // lane's own features are 4 of every 8, so storing from registers would take 8-byte stores
    // that touch 32 rows each; the whole-row stores need 8x fewer cache-line requests, which
    // matters when every workgroup of a round stores at once (short key loops).
    if constexpr (kLdsOut) {
        // (the lead group's own tile buffers: the two leads of a pair store at the same time)
        uint16_t* const area = rw < kRW / 2 ? reinterpret_cast<uint16_t*>(&Ks[lead][0]) + rw * kOArea
                                            : &Vs[lead][0] + (rw - kRW / 2) * kOArea;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
                *reinterpret_cast<u32x2*>(area + j * OST + 32 * db + 8 * rg + 4 * g) = packed(db, rg);
        // only this wave reads its area: its writes complete before its reads are issued
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int kLpr = D / 8;        // lanes per row, 16 bytes each
        constexpr int kRpi = 64 / kLpr;    // rows per store instruction
        const int col = 8 * (lane % kLpr);
        uint16_t* const ob = p.out + b * p.q_bstride + h * D + col;
#pragma unroll
        for (int i = 0; i < 32 / kRpi; ++i) {
            const int rr = i * kRpi + lane / kLpr;
            const u32x4 val = *reinterpret_cast<const u32x4*>(area + rr * OST + col);
            if (r0 + rr < p.Lq) *reinterpret_cast<u32x4*>(ob + (int64_t)(r0 + rr) * p.q_tstride) = val;
        }
        if constexpr (SK) __syncthreads();  // the next unit stages its tiles into the same LDS
    } else if (qrow < p.Lq) {
        uint16_t* op = p.out + b * p.q_bstride + (int64_t)qrow * p.q_tstride + h * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) *reinterpret_cast<u32x2*>(op + 32 * db + 8 * rg + 4 * g) = packed(db, rg);
    }
    };  // unit

    if constexpr (SK) {
        // Balanced launch: this workgroup's whole units, then its piece of the surplus units. A
        // piece is shorter than one unit's key loop, so it lies in one unit or spans the end of
        // one and the start of the next: first part -> slot 2w, second part -> slot 2w + 1.
        // (one loop over both kinds of task, so the unit body is inlined once)
        const int nT = p.sk_tiles;
        int64_t w = w_begin(p, bid);
        const int64_t w1 = w_begin(p, bid + 1);
        for (int i = 0, slot = 2 * bid;; ++i) {
            if (i < p.sk_full) {
                unit(bid * p.sk_full + i, 0, nT, -1);
            } else {
                if (w >= w1) break;
                const int u = (int)(w / nT), ta = (int)(w % nT);
                const int tb = (int)min64(nT, ta + (w1 - w));
                unit(p.sk_full * p.sk_wgs + u, ta, tb, slot++);
                w += tb - ta;
            }
        }
    } else {
        unit(bid, -1, -1, -1);
    }
}

// Output of the surplus units of a balanced launch: unit e's key tiles were cut into pieces held
// by consecutive workgroups; merged in key order, normalised, rounded once. One workgroup per
// (unit, 32-feature block), so the partials are read by D/32 times as many CUs; the maximum is
// taken first so that every piece's loads are independent and several are in flight at once.
template <int D, int DT, int NW>
__global__ void __launch_bounds__(NW * 64) attn_merge_kernel(KParams p) {
    constexpr bool OUT_BF16 = DT != kDtF16;
    constexpr int DB = D / 32;
    constexpr int NC = partial_chunks<D>();
    constexpr int kBM = NW * 32;
    const int e = blockIdx.x / DB, db = blockIdx.x % DB;
    const int nT = p.sk_tiles, P = p.sk_wgs;
    const int64_t lo = (int64_t)e * nT, hi = lo + nT;  // the unit's surplus positions
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, j = lane & 31;
    // first workgroup whose piece holds position lo: the last w with w_begin(w) <= lo (its piece
    // is never empty: the next one starts after lo, or it is the last and ends at sk_work > lo)
    int w0 = (int)(lo * P / p.sk_work);
    while (w0 + 1 < P && w_begin(p, w0 + 1) <= lo) ++w0;
    while (w0 > 0 && w_begin(p, w0) > lo) --w0;
    const int64_t beg0 = w_begin(p, w0);
    const int rem0 = (int)(p.sk_work * w0 % P);
    const int64_t step_q = p.sk_work / P;
    const int step_r = (int)(p.sk_work % P);
    const u32x4* base = reinterpret_cast<const u32x4*>(p.ws) + (int64_t)wave * NC * 64 + lane;
    constexpr int64_t kSlot = (int64_t)NW * NC * 64;
    const u32x4* first = base + (beg0 >= lo ? 2 * w0 : 2 * w0 + 1) * kSlot;
    // the pieces of workgroups w0, w0 + 1, ... that start before hi, stepping
    // w_begin(w + 1) = w_begin(w) + step_q (+1 when the remainder of sk_work * w wraps)
    auto next = [&](int64_t& beg, int& rem) __attribute__((always_inline)) {
        const int s = rem + step_r;
        const int64_t nb = beg + step_q + (s >= P ? 1 : 0);
        rem = s >= P ? s - P : s;
        return nb;
    };
    int n = 0;
    for (int64_t beg = beg0, rem_ = rem0; w0 + n < P && beg < hi; ++n) {
        int rem = (int)rem_;
        beg = next(beg, rem);
        rem_ = rem;
    }
    // calls f(src, nonempty) for each of the n pieces; a counted loop with unconditional loads, so
    // the loads of several pieces are in flight together (an empty piece wrote nothing: it reads
    // `first`, which always holds a partial, with weight 0)
    auto each_piece = [&](auto&& f) __attribute__((always_inline)) {
        int64_t beg = beg0;
        int rem = rem0;
#pragma unroll 4
        for (int i = 0; i < n; ++i) {
            const int w = w0 + i;
            const int64_t nb = next(beg, rem);
            const bool ne = nb > beg;
            f(ne ? base + (beg >= lo ? 2 * w : 2 * w + 1) * kSlot : first, ne);
            beg = nb;
        }
    };
    // one pass in key order with a running maximum: piece i holds O_i / l_i, so the output is
    // sum_i w_i (O_i / l_i) / sum_i w_i with w_i = l_i 2^(m_i - M); the loads of every piece are
    // independent of the running state, so several pieces' loads are in flight together
    float M = -1e30f, l = 0.f;
    float o[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) o[r] = 0.f;
    each_piece([&](const u32x4* src, bool ne) {
        const u32x4 ml = src[2 * DB * 64];
        const float mv = __uint_as_float(ml.x), lv = __uint_as_float(ml.y);
        const u32x4 c0 = src[(2 * db) * 64], c1 = src[(2 * db + 1) * 64];
        const uint32_t ow[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float mi = ne ? mv : -1e30f;
        const float mn = fmaxf(M, mi);
        const float a = __builtin_amdgcn_exp2f(M - mn);
        const float f = ne ? lv * __builtin_amdgcn_exp2f(mi - mn) : 0.f;
        l = l * a + f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f16x2 h = __builtin_bit_cast(f16x2, ow[i]);
            o[2 * i] = o[2 * i] * a + (float)h[0] * f;
            o[2 * i + 1] = o[2 * i + 1] * a + (float)h[1] * f;
        }
        M = mn;
    });
    const float inv = l > 0.f ? 1.f / l : 0.f;  // l is already the whole row's weight
    const int u = p.sk_full * p.sk_wgs + e;
    const int qblk = u % p.n_qblk, bh = u / p.n_qblk, h = bh % p.Hq, b = bh / p.Hq;
    const int qrow = qblk * kBM + wave * 32 + j;
    if (qrow >= p.Lq) return;
    uint16_t* op = p.out + b * p.q_bstride + (int64_t)qrow * p.q_tstride + h * D + 32 * db;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
        const float x0 = o[4 * rg + 0] * inv, x1 = o[4 * rg + 1] * inv;
        const float x2 = o[4 * rg + 2] * inv, x3 = o[4 * rg + 3] * inv;
        u32x2 v;
        if constexpr (OUT_BF16) {
            v.x = pack_bf16x2(x0, x1);
            v.y = pack_bf16x2(x2, x3);
        } else {
            v.x = pack_f16x2(x0, x1);
            v.y = pack_f16x2(x2, x3);
        }
        *reinterpret_cast<u32x2*>(op + 8 * rg + 4 * g) = v;
    }
}

// Balanced launches run 8-wave workgroups (256 query rows, 64-key tiles).
constexpr int kBalancedWaves = 8;

// Workspace of a balanced launch: two partial slots per workgroup, one per wave and lane.
constexpr int64_t balanced_workspace_bytes(int d, int wgs) {
    return (int64_t)2 * wgs * kBalancedWaves * 64 * (2 * (d / 32) + 1) * (int64_t)sizeof(u32x4);
}

// Library-held partial results for callers that cannot allocate device memory: one array per
// GPU (each device's copy of this code object holds its own), kept until the process ends. It
// covers a balanced launch at the largest head dim built (d = 128) with one persistent
// workgroup per CU on up to 256 CUs (MI355X): 37.7 MB. Its contents persist from call to call;
// a balanced launch writes every partial before it reads it, so nothing needs clearing.
constexpr int kScratchMaxCUs = 256;
constexpr int64_t kScratchBytes = balanced_workspace_bytes(128, kScratchMaxCUs);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kScratchMaxDevices = 64;

constexpr int kBalancedMinTiles = 16;
// Key loops (64-key tiles) from which grids far smaller than the CUs split them (launch_shape).
constexpr int kSplitMinTiles = 32;

// A balanced launch pays when the grid's rounds would keep the slots under 90 % busy, for
// full-range attention (every unit the same number of key tiles), more units than slots and key
// loops of at least 16 tiles; shorter ones spend too much on handing over partial results.
// Measured on MI355X against the plain launch for 1785 x 40-head blocks (B = 2, d = 128): 2 tiles
// -22 %, 8 tiles -13 %, 12-14 tiles within 2 %, 16 tiles +3-4 %, 24 tiles +10 %; the streaming
// grid (280 blocks, 112 tiles) +23 %.
bool balanced_pays(const AttnArgs& a, int64_t units, int64_t slots, int tiles) {
    if (a.win_left >= 0 || a.win_right >= 0 || units <= slots || tiles < kBalancedMinTiles) return false;
    const int64_t rounds = (units + slots - 1) / slots;
    return units * 10 < rounds * slots * 9;
}

int device_cu_count() {
    static thread_local int cached_dev = -1, cached_cus = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev != cached_dev) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached_dev = dev;
        cached_cus = cus;
    }
    return cached_cus;
}

template <int D, int DT, int NW, int KS>
KParams make_params(const AttnArgs& a) {
    constexpr int kBM = NW / KS * 32;
    KParams p{};
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.out = static_cast<uint16_t*>(a.out);
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.Lq = a.Lq;
    p.Lk = a.Lk;
    p.group = a.Hq / a.Hkv;
    p.n_qblk = (a.Lq + kBM - 1) / kBM;
    p.win_left = a.win_left;
    p.win_right = a.win_right;
    p.q_bstride = a.q_bstride;
    p.kv_bstride = a.kv_bstride;
    p.q_tstride = a.Hq * D;
    p.kv_tstride = a.Hkv * D;
    p.c = a.scale * kLog2e;
    p.gamma_q = a.gamma_q;
    p.q_eps = a.q_eps;
    p.q_cs = a.q_cs;
    p.q_rope = a.q_rope;
    p.nblocks = (int)((int64_t)p.n_qblk * a.Hq * a.B);
    return p;
}

template <int D, int DT, int NW, int KS, bool BIG = false>
hipError_t launch(const AttnArgs& a, hipStream_t stream, bool paired = false) {
    KParams p = make_params<D, DT, NW, KS>(a);
    if (paired) {  // one workgroup per pair of 64-row blocks (four key groups)
        p.pair = 1;
        p.nblocks = (int)((int64_t)((p.n_qblk + 1) / 2) * a.Hq * a.B);
    }
    hipLaunchKernelGGL((attn_fwd_kernel<D, DT, NW, KS, false, BIG>), dim3((unsigned)p.nblocks), dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
}

// Balanced launch: wgs persistent 8-wave workgroups (one per CU), then the merge of the split
// units.
template <int D, int DT>
hipError_t launch_balanced(const AttnArgs& a, int wgs, hipStream_t stream) {
    constexpr int NW = kBalancedWaves;
    KParams p = make_params<D, DT, NW, 1>(a);
    const int units = p.nblocks;
    p.sk_tiles = (a.Lk + kTileKeys - 1) / kTileKeys;
    p.sk_wgs = wgs;
    p.sk_full = units / wgs;
    const int surplus = units - p.sk_full * wgs;  // > 0: balanced_pays requires a partial last round
    p.sk_work = (int64_t)surplus * p.sk_tiles;
    p.ws = static_cast<float*>(a.ws);
    p.nblocks = wgs;  // the XCD regrouping works on the persistent workgroups
    hipLaunchKernelGGL((attn_fwd_kernel<D, DT, NW, 1, true, false>), dim3((unsigned)wgs), dim3(NW * 64), 0, stream, p);
    hipLaunchKernelGGL((attn_merge_kernel<D, DT, NW>), dim3((unsigned)(surplus * (D / 32))), dim3(NW * 64), 0,
                       stream, p);
    return hipGetLastError();
}

template <int D, int DT>
hipError_t launch_shape(const AttnArgs& a, hipStream_t stream) {
    // 256-row workgroups when there are at least four per CU (long sequences). Otherwise 128-row
    // workgroups of 4 waves, two per CU -- unless even those leave CUs with a single 4-wave
    // workgroup (at most one per CU) over a long key loop: then 8 waves split the keys in two
    // halves, so every CU runs 8 waves on half as many keys each. Measured on MI355X: the split
    // pays for [2, 2048, 8, 64] causal (256 workgroups, +15 %), but not for grids above one
    // workgroup per CU (the shared barriers of the two halves cost more than the finer
    // balancing gains) nor for loops of a few tiles (the merge does not amortise).
    // With a caller workspace, grids of 256-row blocks that would leave the CUs under 90 % busy
    // over their rounds (e.g. 280 blocks on 256 CUs) run balanced on one persistent 8-wave
    // workgroup per CU. Measured on MI355X, this beats the plain launches of those grids (also
    // the 4-wave one, whose last round still gives every CU a workgroup), and beats balancing
    // 4-wave workgroups: 8 waves per workgroup stage each tile once for twice the rows.
    // K/V regions whose rows up to one tile past Lk span 4 GiB or more: the plain 8-wave shape
    // with per-tile buffer resources (any grid)
    const int64_t elem = DT == kDtFP8 || DT == kDtFP8P ? 1 : 2;
    if (((int64_t)a.Lk + 64) * a.Hkv * D * elem > 0xffffffffLL) return launch<D, DT, 8, 1, true>(a, stream);
    const int64_t cus = device_cu_count();
    const int64_t wg256 = (int64_t)((a.Lq + 255) / 256) * a.Hq * a.B;
    const int tiles8 = (a.Lk + kTileKeys - 1) / kTileKeys;
    if (a.ws && a.ws_bytes >= balanced_workspace_bytes(a.d, (int)cus) && balanced_pays(a, wg256, cus, tiles8))
        return launch_balanced<D, DT>(a, (int)cus, stream);
    // Grids of at most a quarter as many 128-row blocks as CUs over long key loops (a few query
    // rows per head over a long context) are set by the loop's serial steps, not by the CUs: with
    // a workspace and full-range rows, every 256-row unit's key tiles are cut into equal pieces,
    // one persistent workgroup each (up to one per CU), and the merge kernel combines them.
    // Measured on MI355X against the plain launch (d = 128, two key groups there): 16 heads x 64
    // queries over 4096 keys (64 tiles) 2.35x faster, over 3072 keys 2.0x; 8 x 1024 queries over
    // 2048 keys (32 tiles) 1.34x, 8 x 256 queries 1.13x; one query row per head over 8192 keys
    // 1.6x; shorter loops lose (16 tiles -5 %, 8 x 257 over 257 keys -32 %: the second launch
    // and the merge outweigh the steps saved). At d = 64 the four key groups of one workgroup
    // are faster (the split: -13 % to -32 %).
    const int64_t wg128 = (int64_t)((a.Lq + 127) / 128) * a.Hq * a.B;
    if (D == 128 && a.ws && a.win_left < 0 && a.win_right < 0 && wg128 * 4 <= cus && tiles8 >= kSplitMinTiles) {
        const int wgs = (int)std::min<int64_t>(cus, wg256 * tiles8);
        if (a.ws_bytes >= balanced_workspace_bytes(a.d, wgs)) return launch_balanced<D, DT>(a, wgs, stream);
    }
    // Banded rows -- a window of at most 2048 + 1 keys, or causal rows of at most 4096 keys --
    // waste less on edge tiles in 128-row blocks, which halves the keys a block visits beyond
    // its rows' bands. Measured on MI355X with two or more 256-row blocks per CU: window (256, 0)
    // d = 64 +41 %, (1024, 0) +14 %, (2048, 0) +2 %, (4096, 0) -4.5 %; causal 2048-4096 keys
    // +6-8 %, 8192 keys -7 %.
    const bool banded = a.win_right >= 0 && (a.win_left >= 0 ? (int64_t)a.win_left + a.win_right <= 2048 : a.Lk <= 4096);
    if (banded && wg256 >= 2 * cus) return launch<D, DT, 4, 1>(a, stream);
    // 256-row workgroups for four or more blocks per CU, or for one or more per CU whose rounds
    // keep the CUs at least 90 % busy over key loops of at least 2048 keys. Measured: one or two
    // full rounds +12-14 % (64 heads x 2048 x 7140 keys, [1,4096,16,128], causal
    // [2,2048,16,128]); 1.25-2.25 rounds lose 2-6 % (one slot per CU quantises coarser than two
    // 128-row slots) and loops of 512-1024 keys 9 %, so those keep 128-row blocks.
    const bool full8 = wg256 >= cus && wg256 * 10 >= (wg256 + cus - 1) / cus * cus * 9;
    if (wg256 >= 4 * cus || (full8 && a.Lk >= 2048)) return launch<D, DT, 8, 1>(a, stream);
    if (wg128 <= cus && a.Lk >= 512) {
        // d = 64, rows over at least 1024 keys with no left window edge: four key groups over
        // 64-row blocks (twice the blocks, each group a quarter of the loop) when causal rows
        // make the blocks' loops unequal -- dispatched longest first, a CU's second block is as
        // short as its first was long, so the rounds even out without a merge across
        // workgroups -- or when 128-row blocks would leave half the CUs idle. Measured on MI355X
        // against the two-group shape: causal [2,1024,8,64] +20 %, [1,4096,8,64] +13 %,
        // [2,2048,8,64] +2 %, non-causal [1,2048,4,64] +26 %; a (256, 0) window over the same
        // grid -64 %, so banded rows keep two groups.
        // Causal blocks that would need a second round of such workgroups are paired instead
        // (block i with block n - 1 - i, one round, the groups divided between the two).
        if constexpr (D == 64)
            if (a.win_left < 0 && a.Lk >= 1024 && (a.win_right >= 0 || 2 * wg128 <= cus)) {
                const int64_t nq64 = (a.Lq + 63) / 64;
                const bool pair = a.win_right >= 0 && nq64 * a.Hq * a.B > cus &&
                                  (nq64 + 1) / 2 * a.Hq * a.B <= cus;
                return launch<D, DT, 8, 4>(a, stream, pair);
            }
        return launch<D, DT, 8, 2>(a, stream);
    }
    return launch<D, DT, 4, 1>(a, stream);
}

}  // namespace

int64_t attn_workspace_bytes(int d) { return balanced_workspace_bytes(d, device_cu_count()); }

int64_t attn_scratch_bytes() { return kScratchBytes; }

// Device address of the current GPU's scratch array, looked up once per device with that device
// current. Host code uses only this address: the array's own name is a host-side stand-in.
hipError_t attn_scratch(void** out) {
    static std::mutex mu;
    static void* addr[kScratchMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

// Every row of a full-range (no causal mask, no window) bf16 launch with at least this many keys
// takes bf16 probabilities: each probability then carries a relative rounding error of at most
// 2^-8 (zero-mean for independent mantissas), so the output error is a weighted sum of those
// errors times (v_j - o), whose mean shrinks like 1/sqrt(keys): at 2048 keys it stays 2x below
// the mean-abs bound on unit-variance data (and the worst case, 2^-8 / (1 - 2^-8) times the
// weighted mean of |v_j - o|, below the max-abs bound). Shorter rows keep f16 probabilities.
constexpr int kBf16ProbMinKeys = 2048;

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t stream) {
    const bool bf16_probs = a.dtype == kDtBF16 && a.win_left < 0 && a.win_right < 0 && a.Lk >= kBf16ProbMinKeys;
    if (bf16_probs) return a.d == 128 ? launch_shape<128, kDtBF16P>(a, stream) : launch_shape<64, kDtBF16P>(a, stream);
    if (a.d == 128) {
        if (a.dtype == kDtFP8) return launch_shape<128, kDtFP8>(a, stream);
        if (a.dtype == kDtFP8P) return launch_shape<128, kDtFP8P>(a, stream);
        if (a.dtype == kDtBF16VF16) return launch_shape<128, kDtBF16VF16>(a, stream);
        return a.dtype == kDtBF16 ? launch_shape<128, kDtBF16>(a, stream) : launch_shape<128, kDtF16>(a, stream);
    }
    if (a.dtype == kDtFP8) return launch_shape<64, kDtFP8>(a, stream);
    if (a.dtype == kDtFP8P) return launch_shape<64, kDtFP8P>(a, stream);
    if (a.dtype == kDtBF16VF16) return launch_shape<64, kDtBF16VF16>(a, stream);
    return a.dtype == kDtBF16 ? launch_shape<64, kDtBF16>(a, stream) : launch_shape<64, kDtF16>(a, stream);
}

}  // namespace sa
