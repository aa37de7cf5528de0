// Memory-bound kernels: NVFP4 fake quantization (standalone and operand
// preparation), the permuted transpose used to lay operands out for MFMA, and
// the backward preprocess Dl = rowsum(dO * O).
//
// Fake quantization follows the NVFP4 block format of the FastVideo VSA
// checkpoint metadata (linear_quantization.format: E2M1 values, 16-element
// blocks, FP8 E4M3 block scales) with no global scale, as its
// attention.precision flags state for Q, K, V and P.
#include "aq_kernels.h"

namespace aq {

// One thread per 16-element group along the contiguous head dimension.
// Rows n in [N, Nout) are written as zeros (padding for tiled kernels).
template <bool QUANT>
__global__ __launch_bounds__(256) void fq_axis_d_kernel(FqArgs a) {
    const int G = a.D / 16;
    const int64_t total = (int64_t)a.BH * a.Nout * G;
    for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < total;
         gi += (int64_t)gridDim.x * blockDim.x) {
        const int gd = (int)(gi % G);
        const int64_t row = (gi / G) % a.Nout;
        const int64_t bh = gi / ((int64_t)G * a.Nout);
        const int64_t b = bh / a.H, h = bh % a.H;
        uint16_t* yp = a.y + b * a.ysb + h * a.ysh + row * a.ysn + gd * 16;
        if (row >= a.N) {
            u32x4 z = {0u, 0u, 0u, 0u};
            *(u32x4*)yp = z;
            *(u32x4*)(yp + 8) = z;
            continue;
        }
        const uint16_t* xp = a.x + b * a.xsb + h * a.xsh + row * a.xsn + gd * 16;
        u32x4 w0 = *(const u32x4*)xp;
        u32x4 w1 = *(const u32x4*)(xp + 8);
        if (!QUANT) {
            *(u32x4*)yp = w0;
            *(u32x4*)(yp + 8) = w1;
            continue;
        }
        uint32_t w[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fmaxf(fabsf(bf_lo(w[i])), fabsf(bf_hi(w[i]))));
        const float s = e4m3_round(amax / 6.0f);
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            o[i] = pack_exact(fq_elem_exact(bf_lo(w[i]), s), fq_elem_exact(bf_hi(w[i]), s));
        u32x4 o0 = {o[0], o[1], o[2], o[3]}, o1 = {o[4], o[5], o[6], o[7]};
        *(u32x4*)yp = o0;
        *(u32x4*)(yp + 8) = o1;
        if (a.codes) a.codes[(bh * a.N + row) * G + gd] = e4m3_code(s);
    }
}

// One thread per (16-token group, CW columns). Tokens >= N read as zero;
// rows in [N, Nout) are written as zeros. Two columns per thread (one 4-byte
// word per row): a wave reads and writes whole 256-byte rows, with four times
// as many threads as 8 columns (16-byte words) would give (measured on 6 x
// 31,200 x 128 tokens: 0.045 -> 0.044 ms resident, 0.051 -> 0.046 ms after
// a cache flush).
template <bool QUANT, int CW>
__global__ __launch_bounds__(256) void fq_axis_n_kernel(FqArgs a) {
    static_assert(CW == 2 || CW == 8, "columns per thread");
    constexpr int W = CW / 2;  // 32-bit words (bf16 pairs) per row
    typedef uint32_t word_t __attribute__((ext_vector_type(W)));
    const int CG = a.D / CW;
    const int64_t NGo = (a.Nout + 15) / 16;
    const int64_t total = (int64_t)a.BH * NGo * CG;
    for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < total;
         gi += (int64_t)gridDim.x * blockDim.x) {
        const int dc = (int)(gi % CG);
        const int64_t tg = (gi / CG) % NGo;
        const int64_t bh = gi / ((int64_t)CG * NGo);
        const int64_t b = bh / a.H, h = bh % a.H;
        const uint16_t* xb = a.x + b * a.xsb + h * a.xsh + dc * CW;
        uint16_t* yb = a.y + b * a.ysb + h * a.ysh + dc * CW;
        word_t v[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int64_t row = tg * 16 + t;
            if (row < a.N) v[t] = *(const word_t*)(xb + row * a.xsn);
            else v[t] = word_t{};
        }
        if (QUANT) {
            float s[CW];
#pragma unroll
            for (int c = 0; c < CW; ++c) {
                float amax = 0.0f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const uint32_t wd = v[t][c >> 1];
                    amax = fmaxf(amax, fabsf((c & 1) ? bf_hi(wd) : bf_lo(wd)));
                }
                s[c] = e4m3_round(amax / 6.0f);
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
#pragma unroll
                for (int c2 = 0; c2 < W; ++c2) {
                    const uint32_t wd = v[t][c2];
                    v[t][c2] = pack_exact(fq_elem_exact(bf_lo(wd), s[2 * c2]),
                                          fq_elem_exact(bf_hi(wd), s[2 * c2 + 1]));
                }
            }
            if (a.codes && tg * 16 < a.N) {
                uint8_t* cp = a.codes + (bh * ((a.N + 15) / 16) + tg) * a.D + dc * CW;
#pragma unroll
                for (int c = 0; c < CW; ++c) cp[c] = e4m3_code(s[c]);
            }
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int64_t row = tg * 16 + t;
            if (row < a.Nout) *(word_t*)(yb + row * a.ysn) = v[t];
        }
    }
}

// Fake quantization of V along the tokens fused with its transpose, for the
// forward (which reads V only as V^T): y[bh][d][p] = FQ_tokens(x)[bh][p][d]
// for p < Nout (tokens >= N are zero), the same 16-token groups and exact
// arithmetic as fq_axis_n_kernel, so the values are bit-identical; with F16
// they are stored as fp16 (exact for NVFP4 values). One 64-token x 64-column
// tile per workgroup, staged in LDS (rows padded by 4 bytes); in the middle
// each thread quantizes one 16-token group of one column in place.
template <bool QUANT, bool F16>
__global__ __launch_bounds__(256) void fq_n_transpose_kernel(FqArgs a) {
    __shared__ uint16_t tile[64][64 + 2];
    lds_poison(tile);
    const int64_t bh = blockIdx.z, b = bh / a.H, h = bh % a.H;
    const int n0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
    const uint16_t* s = a.x + b * a.xsb + h * a.xsh;
    const int tid = threadIdx.x;
    for (int i = tid; i < 64 * 8; i += 256) {
        const int r = i / 8, cc = i % 8;
        const int64_t row = n0 + r;
        u32x4 w = {0u, 0u, 0u, 0u};
        if (row < a.N) w = *(const u32x4*)(s + row * a.xsn + d0 + cc * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tile[r][cc * 8 + 2 * j] = (uint16_t)(w[j] & 0xFFFFu);
            tile[r][cc * 8 + 2 * j + 1] = (uint16_t)(w[j] >> 16);
        }
    }
    __syncthreads();
    if (QUANT) {
        const int c = tid & 63, g = tid >> 6;  // column, 16-token group
        float x[16], amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            x[i] = bf2f(tile[16 * g + i][c]);
            amax = fmaxf(amax, fabsf(x[i]));
        }
        const float sc = e4m3_round(amax / 6.0f);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            tile[16 * g + i][c] = (uint16_t)(__float_as_uint(fq_elem_exact(x[i], sc)) >> 16);
        __syncthreads();
    }
    uint16_t* o = a.y + bh * a.D * a.Nout;
    for (int i = tid; i < 64 * 8; i += 256) {
        const int dr = i / 8, pc = i % 8;  // output row d0 + dr, positions pc*8 .. pc*8+7
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w[j] = (uint32_t)tile[pc * 8 + 2 * j][dr] | ((uint32_t)tile[pc * 8 + 2 * j + 1][dr] << 16);
            if (F16) {
                const f32x2 f = {bf_lo(w[j]), bf_hi(w[j])};
                w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
            }
        }
        *(u32x4*)(o + (int64_t)(d0 + dr) * a.Nout + n0 + pc * 8) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// Transposed copy: dst[bh][d][p] = src[bh][tok(p)][d] for a contiguous padded
// [BH][Npad][D] source, with tok(p) = 16 (p / 16) + perm16(p % 16) when PERM
// (operands read by MFMA k-slots in accumulator-row order) and tok(p) = p
// otherwise. With F16 the bf16 values are converted to fp16 (nearest even;
// exact for NVFP4 values). Tile: 64 tokens x 64 columns per block.
template <bool PERM, bool F16>
__global__ __launch_bounds__(256) void transpose_perm_kernel(const uint16_t* __restrict__ src,
                                                             uint16_t* __restrict__ dst,
                                                             int Npad, int D) {
    __shared__ uint16_t tile[64][64 + 2];
    lds_poison(tile);
    const int bh = blockIdx.z;
    const int n0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
    const uint16_t* s = src + (size_t)bh * Npad * D;
    uint16_t* o = dst + (size_t)bh * D * Npad;
    const int tid = threadIdx.x;
    // load 64 x 64: each thread 2 chunks of 8 elements
    for (int i = tid; i < 64 * 8; i += 256) {
        const int r = i / 8, cc = i % 8;
        u32x4 w = *(const u32x4*)(s + (size_t)(n0 + r) * D + d0 + cc * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (F16) {
                const f32x2 f = {bf_lo(w[j]), bf_hi(w[j])};
                w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
            }
            tile[r][cc * 8 + 2 * j] = (uint16_t)(w[j] & 0xFFFFu);
            tile[r][cc * 8 + 2 * j + 1] = (uint16_t)(w[j] >> 16);
        }
    }
    __syncthreads();
    for (int i = tid; i < 64 * 8; i += 256) {
        const int dr = i / 8, pc = i % 8;   // output row d0 + dr, positions pc*8 .. pc*8+7
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int p0 = pc * 8 + 2 * j, p1 = p0 + 1;
            const int t0 = PERM ? (p0 & ~15) + perm16(p0 & 15) : p0;
            const int t1 = PERM ? (p1 & ~15) + perm16(p1 & 15) : p1;
            w[j] = (uint32_t)tile[t0][dr] | ((uint32_t)tile[t1][dr] << 16);
        }
        u32x4 v = {w[0], w[1], w[2], w[3]};
        *(u32x4*)(o + (size_t)(d0 + dr) * Npad + n0 + pc * 8) = v;
    }
}

// Backward preprocess, one 16-lane group per query row:
//   delta[bh][n] = sum_d dO[n][d] * O[n][d]   (fp32)
//   lse2[bh][n]  = LSE[n] * log2(e)
//   dOw[bh][n][:] = dO[n][:]                  (contiguous padded copy)
// Rows n in [Nq, Nq_pad) get zeros.
__global__ __launch_bounds__(256) void bwd_pre_kernel(PreArgs a) {
    const int lanes_per_row = a.D / 8;          // 8 or 16
    const int rows_per_block = 256 / lanes_per_row;
    const int sub = threadIdx.x % lanes_per_row;
    const int64_t row_global = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / lanes_per_row;
    const int64_t total = (int64_t)a.BH * a.Nq_pad;
    const bool active = row_global < total;
    const int64_t bh = active ? row_global / a.Nq_pad : 0;
    const int64_t n = active ? row_global % a.Nq_pad : 0;
    const int64_t b = bh / a.H, h = bh % a.H;
    float acc = 0.0f;
    u32x4 dv = {0u, 0u, 0u, 0u};
    if (active && n < a.Nq) {
        const u32x4 ov = *(const u32x4*)(a.o + b * a.osb + h * a.osh + n * a.osn + sub * 8);
        dv = *(const u32x4*)(a.dout + b * a.dsb + h * a.dsh + n * a.dsn + sub * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc += bf_lo(ov[j]) * bf_lo(dv[j]) + bf_hi(ov[j]) * bf_hi(dv[j]);
    }
    // reduce across the lanes of this row (lanes_per_row is 8 or 16, aligned)
    for (int off = lanes_per_row / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (!active) return;
    *(u32x4*)(a.dOw + (size_t)row_global * a.D + sub * 8) = dv;
    const float lse2 = (n < a.Nq) ? a.lse[bh * a.Nq + n] * kLog2e : 0.0f;
    if (sub == 0) {
        a.delta[row_global] = acc;
        a.lse2[row_global] = lse2;
    }
    if (a.row_max) {
        // dK/dV inputs of the row-max-relative variant: m2 = m log2(e) and
        // dO, Dl scaled by 1/l = exp2(m2 - lse2) (padded rows: zero)
        const float m2 = (n < a.Nq) ? a.row_max[bh * a.Nq + n] * kLog2e : 0.0f;
        const float post = (n < a.Nq) ? __builtin_amdgcn_exp2f(m2 - lse2) : 0.0f;
        u32x4 sv;
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[j] = pack_rne(bf_lo(dv[j]) * post, bf_hi(dv[j]) * post);
        *(u32x4*)(a.dOw_kv + (size_t)row_global * a.D + sub * 8) = sv;
        if (sub == 0) {
            a.delta_kv[row_global] = acc * post;
            a.lse2_kv[row_global] = m2;
        }
    }
}

// ---------------------------------------------------------------------------
// host launchers

static inline int grid_for(int64_t work, int per_block = 256) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g > 65535 * 8) g = 65535 * 8;
    if (g < 1) g = 1;
    return (int)g;
}

hipError_t launch_fq_axis_d(const FqArgs& a, bool quant, hipStream_t st) {
    const int64_t work = (int64_t)a.BH * a.Nout * (a.D / 16);
    if (quant) fq_axis_d_kernel<true><<<grid_for(work), 256, 0, st>>>(a);
    else fq_axis_d_kernel<false><<<grid_for(work), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_fq_axis_n(const FqArgs& a, bool quant, hipStream_t st) {
    constexpr int CW = 2;
    const int64_t work = (int64_t)a.BH * ((a.Nout + 15) / 16) * (a.D / CW);
    if (quant) fq_axis_n_kernel<true, CW><<<grid_for(work), 256, 0, st>>>(a);
    else fq_axis_n_kernel<false, CW><<<grid_for(work), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_fq_n_transpose(const FqArgs& a, bool quant, bool to_f16, hipStream_t st) {
    dim3 grid((unsigned)(a.Nout / 64), (unsigned)(a.D / 64), (unsigned)a.BH);
    if (quant && to_f16) fq_n_transpose_kernel<true, true><<<grid, 256, 0, st>>>(a);
    else if (quant) fq_n_transpose_kernel<true, false><<<grid, 256, 0, st>>>(a);
    else if (to_f16) fq_n_transpose_kernel<false, true><<<grid, 256, 0, st>>>(a);
    else fq_n_transpose_kernel<false, false><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_transpose_perm(const uint16_t* src, uint16_t* dst, int64_t BH, int Npad, int D,
                                 bool perm, bool to_f16, hipStream_t st) {
    dim3 grid(Npad / 64, D / 64, (unsigned)BH);
    if (perm) transpose_perm_kernel<true, false><<<grid, 256, 0, st>>>(src, dst, Npad, D);
    else if (to_f16) transpose_perm_kernel<false, true><<<grid, 256, 0, st>>>(src, dst, Npad, D);
    else transpose_perm_kernel<false, false><<<grid, 256, 0, st>>>(src, dst, Npad, D);
    return hipGetLastError();
}

hipError_t launch_bwd_pre(const PreArgs& a, hipStream_t st) {
    const int rows_per_block = 256 / (a.D / 8);
    const int64_t rows = (int64_t)a.BH * a.Nq_pad;
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    bwd_pre_kernel<<<(unsigned)blocks, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace aq
