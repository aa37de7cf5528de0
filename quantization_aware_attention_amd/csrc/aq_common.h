// Shared device helpers for the Attn-QAT HIP kernels (gfx950 / CDNA4).
//
// Layout conventions used by every kernel in this library:
//  * bf16 values travel as raw uint16_t patterns.
//  * Matrix products use v_mfma_f32_32x32x16_bf16 (wave64). For lane l,
//    with h = l / 32 and c = l % 32:
//      A operand (32 x 16):  A[c][8h + j], j = 0..7  (8 bf16 per lane)
//      B operand (16 x 32):  B[8h + j][c]
//      C/D (32 x 32, fp32):  C[row(r, h)][c], r = 0..15,
//                            row(r, h) = 8 (r / 4) + 4 h + r % 4.
//    The k index of A and B only has to agree between the two operands, so a
//    C tile can feed the next product directly when its row index is the
//    contraction index: registers r = 0..7 hold k-slots 8h + j of the first
//    16-row half, r = 8..15 those of the second, with k-slot 8h + j holding
//    row 8 (j / 4) + 4 h + j % 4 of that half.
//  * Operands that must be read along the contraction index are stored
//    transposed ([D][N]). K^T, which multiplies a score tile held in this
//    accumulator order, has the tokens of every 16-token group permuted so
//    that the k-slot order becomes contiguous: position p holds token
//    perm16(p), which swaps the 4-token chunks 1 and 2. Score tiles whose
//    keys are loaded in perm32 order (below) need no such permutation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;

__host__ __device__ constexpr int perm16(int p) {
    // swap chunk 1 (positions 4..7) with chunk 2 (positions 8..11); an involution
    return ((p & 12) == 4) ? p + 4 : (((p & 12) == 8) ? p - 4 : p);
}

__device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Same product with fp16 operands (used where both operands are NVFP4 values,
// which fp16 represents exactly).
__device__ __forceinline__ f32x16 mfma_f16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Nearest bf16 (ties to even) of a double, returned as bits.
__device__ __forceinline__ uint16_t bf16_from_double(double x) {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    u = (u + ((1ull << 44) - 1) + ((u >> 45) & 1ull)) & ~((1ull << 45) - 1);
    const float f = (float)__longlong_as_double((long long)u);  // exact: 8 significant bits
    return (uint16_t)(__float_as_uint(f) >> 16);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Pack two floats whose values are exactly representable in bf16 (low 16 bits zero).
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// Round two floats to bf16 (nearest even) and pack them.
__device__ __forceinline__ uint32_t pack_rne(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Larger of two scores. IEEE maximum (NaN-propagating) instead of fmaxf:
// fmaxf must quiet signalling NaNs, so on values the compiler cannot prove
// canonical (matrix-unit results) it inserts a self-max before every use,
// while maximum lowers to one v_maximum3_f32 per two new values. The two
// agree on everything the kernels feed them (finite values and -inf).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Debug builds (AQ_LDS_POISON) fill the LDS arrays in which a kernel stages
// operands and partial results with the 32-bit word 0x7FF87FF8 before their
// first use, then synchronise the workgroup. Read as bf16, fp16, fp32 or
// fp64 every element is a NaN, so a read of LDS that the kernel never wrote
// shows up as NaN in its outputs. Release builds compile the call to
// nothing. Integer arrays (block lists) are never passed: a poisoned index
// would address memory instead of producing a NaN.
template <class... T>
__device__ __forceinline__ void lds_poison(T&... x) {
#ifdef AQ_LDS_POISON
    const unsigned nt = blockDim.x * blockDim.y * blockDim.z;
    const unsigned tid = threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z);
    auto fill = [&](auto& v) {
        static_assert(sizeof(v) % 4 == 0, "LDS arrays are poisoned in 4-byte words");
        uint32_t* w = reinterpret_cast<uint32_t*>(&v);
        for (unsigned i = tid; i < sizeof(v) / 4; i += nt) w[i] = 0x7FF87FF8u;
    };
    (fill(x), ...);
    __syncthreads();
#else
    ((void)x, ...);
#endif
}

// Value of x held by lane l ^ 32.
__device__ __forceinline__ float partner_lane(float x) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return (__lane_id() < 32) ? __uint_as_float(sw[1]) : __uint_as_float(sw[0]);
}

// ---------------------------------------------------------------------------
// NVFP4 scale: s = E4M3(v), v = amax / 6 >= 0, round to nearest even onto the
// OCP E4M3FN grid, saturating at 448. Below 2^-6 the grid is m * 2^-9;
// above, the fp32 significand is rounded to 3 fraction bits.
__device__ __forceinline__ float e4m3_round(float v) {
    float sub = __builtin_rintf(v * 512.0f) * (1.0f / 512.0f);
    uint32_t b = __float_as_uint(v);
    b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
    float nrm = __uint_as_float(b);
    float s = (v < 0.015625f) ? sub : nrm;
    return fminf(s, 448.0f);
}

// OCP E4M3FN code of a value produced by e4m3_round.
__device__ __forceinline__ uint8_t e4m3_code(float s) {
    if (s < 0.015625f) return (uint8_t)(int)(s * 512.0f);
    const uint32_t b = __float_as_uint(s);
    const int e = (int)((b >> 23) & 0xFFu) - 127;
    return (uint8_t)(((e + 7) << 3) | ((b >> 20) & 7u));
}

// Exact NVFP4 element for bf16 inputs: returns sign(x) * E2M1(|x| / s) * s,
// decided by comparing |x| with the rounding midpoints t * s (each product is
// exact in fp32), so exact ties go to the even E2M1 code. s == 0 gives +-0.
__device__ __forceinline__ float fq_elem_exact(float x, float s) {
    float ax = fabsf(x);
    float y = 0.0f;
    y = (ax > 0.25f * s) ? 0.5f * s : y;
    y = (ax >= 0.75f * s) ? 1.0f * s : y;
    y = (ax > 1.25f * s) ? 1.5f * s : y;
    y = (ax >= 1.75f * s) ? 2.0f * s : y;
    y = (ax > 2.5f * s) ? 3.0f * s : y;
    y = (ax >= 3.5f * s) ? 4.0f * s : y;
    y = (ax > 5.0f * s) ? 6.0f * s : y;
    return __builtin_copysignf(y, x);
}

// Key order inside a 32-key block of a score tile S^T = K Q^T. The MFMA
// accumulator puts tile row 8 (r / 4) + 4 h + r % 4 in register r of lane
// half h; loading key 16 h + r into that row gives each lane one whole
// 16-key group (keys 16 h .. 16 h + 15) in registers 0..15. perm32(row) is the
// key stored at tile row `row`.
__host__ __device__ constexpr int perm32(int p) {
    return 16 * ((p >> 2) & 1) + 4 * (p >> 3) + (p & 3);
}

// NVFP4 fake quantization of P for one 16-key group held in one lane:
// P_j = 2^(x_j c - lse2) with x_j the raw scores (masked keys at -inf).
// The scale s = E4M3(max_j P_j / 6) comes from an FP8 round trip (nearest
// even). The division by s is folded into the exponent,
// P_j / s = 2^(x_j c - lse2 - log2 s), and the E2M1 rounding of that ratio
// (nearest even, saturating at 6) is the FP4 conversion unit's. An all-zero
// group (s = 0) multiplies every code by 0. Outputs: the 16 values
// q_j * s in key order as 8 packed pairs, fp16 (F16, exact: q * s has at
// most 6 significant bits and lies in [2^-10, 6]) or bf16 (also exact).
template <bool F16>
__device__ __forceinline__ void quant_p_group16(const float* x, float c, float lse2, u32x4* out) {
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = vmax(mx, x[j]);
    const float pmax = __builtin_amdgcn_exp2f(__builtin_fmaf(mx, c, -lse2));
    const float a6 = pmax * (1.0f / 6.0f);
    const i16x2 z = {0, 0};
    const i16x2 c8 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a6, a6, 1.0f, false);
    const int code2 = __builtin_bit_cast(int, c8);  // the scale code in bytes 0 and 1
    const float s = __builtin_amdgcn_cvt_scalef32_f32_fp8(code2, 1.0f, 0);
    const float t = lse2 + __builtin_fmaxf(__builtin_amdgcn_logf(s), -64.0f);
    float r[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, -t));
    uint32_t codes[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const float* rw = r + 8 * w;
        uint32_t cw = 0u;
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, rw[0], rw[1], 1.0f, 0);
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, rw[2], rw[3], 1.0f, 1);
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, rw[4], rw[5], 1.0f, 2);
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, rw[6], rw[7], 1.0f, 3);
        codes[w] = cw;
    }
    if (F16) {
        const f16x2 s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((short)code2, 1.0f, false);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const f16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[w], 1.0f, 0);
            const f16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[w], 1.0f, 1);
            const f16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[w], 1.0f, 2);
            const f16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes[w], 1.0f, 3);
            out[w] = u32x4{__builtin_bit_cast(uint32_t, q0 * s2), __builtin_bit_cast(uint32_t, q1 * s2),
                           __builtin_bit_cast(uint32_t, q2 * s2), __builtin_bit_cast(uint32_t, q3 * s2)};
        }
    } else {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[w], 1.0f, 0);
            const f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[w], 1.0f, 1);
            const f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[w], 1.0f, 2);
            const f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes[w], 1.0f, 3);
            out[w] = u32x4{pack_rne(q0[0] * s, q0[1] * s), pack_rne(q1[0] * s, q1[1] * s),
                           pack_rne(q2[0] * s, q2[1] * s), pack_rne(q3[0] * s, q3[1] * s)};
        }
    }
}

// Backward form of quant_p_group16 (bf16 output): also returns r_j = P_j / s'
// and s', so that the unquantized P_j = r_j s' (for dS) can be folded into
// later products; s' = s, or 2^-64 for an all-zero group (an exact
// power-of-two rescaling).
__device__ __forceinline__ void quant_p_group16_bwd(const float* x, float c, float lse2, u32x4* out,
                                                    float* r, float& sp_out) {
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) mx = vmax(mx, x[j]);
    const float pmax = __builtin_amdgcn_exp2f(__builtin_fmaf(mx, c, -lse2));
    const float a6 = pmax * (1.0f / 6.0f);
    const i16x2 z = {0, 0};
    const i16x2 c8 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a6, a6, 1.0f, false);
    const float s = __builtin_amdgcn_cvt_scalef32_f32_fp8(__builtin_bit_cast(int, c8), 1.0f, 0);
    const float sp = (s > 0.0f) ? s : 0x1p-64f;
    const float t = lse2 + __builtin_amdgcn_logf(sp);
    sp_out = sp;
#pragma unroll
    for (int j = 0; j < 16; ++j) r[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], c, -t));
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const float* rw = r + 8 * w;
        uint32_t cw = 0u;
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, rw[0], rw[1], 1.0f, 0);
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, rw[2], rw[3], 1.0f, 1);
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, rw[4], rw[5], 1.0f, 2);
        cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, rw[6], rw[7], 1.0f, 3);
        const f32x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
        const f32x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
        const f32x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
        const f32x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
        out[w] = u32x4{pack_rne(q0[0] * s, q0[1] * s), pack_rne(q1[0] * s, q1[1] * s),
                       pack_rne(q2[0] * s, q2[1] * s), pack_rne(q3[0] * s, q3[1] * s)};
    }
}

// 16-bit transposing LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, lane m supplies the address of 4 consecutive 16-bit elements M[m][0..3];
// lane i receives M[4 j + i / 4][i % 4] for j = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}

}  // namespace aq
