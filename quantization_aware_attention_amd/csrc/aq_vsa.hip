// VSA coarse branch and its gated combination with the block-sparse fine
// branch.
//
// FastVideo VSA checkpoint metadata (attention: kind vsa, 128-token cubes,
// coarse precision BF16 without quantization, trained compression gates) and
// the fastvideo-kernel commit message (the gate is scattered into the tile
// buffer with Q, K and V: a per-token tensor). Computed here:
//
//   Qbar, Kbar, Vbar = bf16(block means of the raw Q, K, V) [BH][nb][D]
//   O_c = softmax(sm_scale Qbar Kbar^T) Vbar                   [BH][nbq][D]
//   O   = O_fine + G * O_c[block(t)]
//
// and for the backward, with dO the gradient of O:
//
//   dG    = dO * O_c[block(t)]
//   dO_c  = sum over the block's tokens of G * dO
//   dS    = P (dO_c Vbar^T - rowsum(dO_c O_c)),  P = softmax row
//   dQbar = sm_scale dS Kbar, dKbar = sm_scale dS^T Qbar, dVbar = P^T dO_c
//   dQ, dK, dV += block gradient / block token count, for every token.
//
// The coarse products are tiny (nb x nb x D per head) and run on fp32 vector
// units from the bf16 means; the passes over the token tensors (pooling,
// combination, gate reduction, gradient broadcast) are bound by HBM and move
// 16 bytes per lane per access.
#include "aq_kernels.h"

namespace aq {

namespace {

// Offset of element (bh, t, d) of a strided [B,H,N,D] tensor.
__device__ __forceinline__ int64_t at(int64_t bh, int64_t H, int64_t sb, int64_t sh, int64_t sn,
                                      int64_t t, int d) {
    return (bh / H) * sb + (bh % H) * sh + t * sn + d;
}

// Sum over the 256 threads of a workgroup (result in every thread).
__device__ __forceinline__ float block_sum(float x, float* red) {
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float block_max(float x, float* red) {
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Rows per workgroup of the coarse kernels: each mean row they load serves
// that many dot products.
constexpr int kVsaRows = 4;

// y . x[r] for the kVsaRows fp32 rows x (LDS) and one bf16 (BF) or fp32 row y.
template <int D, bool BF>
__device__ __forceinline__ void dots(const float (*x)[D], const void* y, float* out) {
#pragma unroll
    for (int r = 0; r < kVsaRows; ++r) out[r] = 0.0f;
#pragma unroll 4
    for (int c = 0; c < D / 8; ++c) {
        float v[8];
        if (BF) {
            const u32x4 w = *(const u32x4*)((const uint16_t*)y + 8 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = bf2f(w[e] & 0xffffu);
                v[2 * e + 1] = bf2f(w[e] >> 16);
            }
        } else {
            const float4 a = *(const float4*)((const float*)y + 8 * c);
            const float4 b = *(const float4*)((const float*)y + 8 * c + 4);
            v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z,
            v[7] = b.w;
        }
#pragma unroll
        for (int r = 0; r < kVsaRows; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) out[r] = fmaf(x[r][8 * c + e], v[e], out[r]);
    }
}

// out[r] = sum_j w[r][j] Y[j][d] for column d = threadIdx.x (< D; other
// threads get 0): 256 / D groups of D threads split the rows j.
template <int D, bool BF>
__device__ __forceinline__ void col_sums(const float (*w)[kVsaMaxBlocks], const void* Y, int n,
                                         float (*part)[256], float* out) {
    constexpr int G = 256 / D;
    const int g = threadIdx.x / D, d = threadIdx.x % D;
    float acc[kVsaRows];
#pragma unroll
    for (int r = 0; r < kVsaRows; ++r) acc[r] = 0.0f;
    for (int j = g; j < n; j += G) {
        const float y = BF ? bf2f(((const uint16_t*)Y)[(int64_t)j * D + d]) : ((const float*)Y)[(int64_t)j * D + d];
#pragma unroll
        for (int r = 0; r < kVsaRows; ++r) acc[r] = fmaf(w[r][j], y, acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kVsaRows; ++r) part[r][threadIdx.x] = acc[r];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kVsaRows; ++r) {
        out[r] = 0.0f;
        if (threadIdx.x < D)
            for (int gg = 0; gg < G; ++gg) out[r] += part[r][gg * D + d];
    }
    __syncthreads();
}

// Load kVsaRows rows (row0 .. row0 + kVsaRows - 1 of a [rows][D] array,
// rows >= nrows as zeros) into LDS as fp32.
template <int D, bool BF>
__device__ __forceinline__ void load_rows(float (*dst)[D], const void* src, int64_t row0, int nrows) {
    for (int e = threadIdx.x; e < kVsaRows * D; e += 256) {
        const int r = e / D, d = e % D;
        float x = 0.0f;
        if (r < nrows) x = BF ? bf2f(((const uint16_t*)src)[(row0 + r) * D + d]) : ((const float*)src)[(row0 + r) * D + d];
        dst[r][d] = x;
    }
}

}  // namespace

// Block means of Q, K and V, one workgroup per (block, bh, tensor): thread
// (r, c) sums columns 8 c .. 8 c + 7 of token rows r, r + R, ... in fp64, and
// the R partial sums are added in fp64 too. Sums of bf16 values are exact in
// fp64 for any practical block, so the bf16 rounding of the mean does not
// depend on the summation order.
template <int D>
__global__ __launch_bounds__(256) void vsa_pool_kernel(VsaArgs a) {
    constexpr int C = D / 8, R = 256 / C;
    __shared__ double part[R][D];
    lds_poison(part);
    const int which = blockIdx.z;  // 0 = q, 1 = k, 2 = v
    const int nb = which == 0 ? a.nbq : a.nbk;
    const int j = blockIdx.x;
    if (j >= nb) return;  // the grid covers the larger of nbq and nbk
    const int64_t bh = blockIdx.y;
    const int N = which == 0 ? a.Nq : a.Nk;
    const uint16_t* x = which == 0 ? a.q : (which == 1 ? a.k : a.v);
    const int64_t sb = which == 0 ? a.qsb : (which == 1 ? a.ksb : a.vsb);
    const int64_t sh = which == 0 ? a.qsh : (which == 1 ? a.ksh : a.vsh);
    const int64_t sn = which == 0 ? a.qsn : (which == 1 ? a.ksn : a.vsn);
    const int c = threadIdx.x % C, r = threadIdx.x / C;
    const int t0 = j * a.bt, t1 = min(N, (j + 1) * a.bt);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int t = t0 + r; t < t1; t += R) {
        const u32x4 w = *(const u32x4*)(x + at(bh, a.H, sb, sh, sn, t, 8 * c));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)bf2f(w[e] & 0xffffu);
            acc[2 * e + 1] += (double)bf2f(w[e] >> 16);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r][8 * c + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        double sum = 0.0;
        for (int rr = 0; rr < R; ++rr) sum += part[rr][threadIdx.x];
        uint16_t* out = which == 0 ? a.qbar : (which == 1 ? a.kbar : a.vbar);
        out[(bh * nb + j) * D + threadIdx.x] = bf16_from_double(sum / (double)(t1 - t0));
    }
}

// Coarse attention, one workgroup per kVsaRows query blocks of one bh:
// scores against every key block, softmax in fp32, O_c rows and their LSE.
template <int D>
__global__ __launch_bounds__(256) void vsa_coarse_fwd_kernel(VsaArgs a) {
    __shared__ float qs[kVsaRows][D];
    __shared__ float pw[kVsaRows][kVsaMaxBlocks];
    __shared__ float part[kVsaRows][256];
    __shared__ float red[4];
    lds_poison(qs, pw, part, red);
    const int i0 = blockIdx.x * kVsaRows, nr = min(kVsaRows, a.nbq - i0);
    const int64_t bh = blockIdx.y, row0 = bh * a.nbq + i0;
    load_rows<D, true>(qs, a.qbar, row0, nr);
    __syncthreads();
    const uint16_t* kb = a.kbar + bh * a.nbk * D;
    float mx[kVsaRows];
#pragma unroll
    for (int r = 0; r < kVsaRows; ++r) mx[r] = -INFINITY;
    for (int j = threadIdx.x; j < a.nbk; j += 256) {
        float sv[kVsaRows];
        dots<D, true>(qs, kb + (int64_t)j * D, sv);
#pragma unroll
        for (int r = 0; r < kVsaRows; ++r) {
            pw[r][j] = a.sm_scale * sv[r];
            mx[r] = fmaxf(mx[r], pw[r][j]);
        }
    }
    float lse[kVsaRows];
#pragma unroll
    for (int r = 0; r < kVsaRows; ++r) {
        const float m = block_max(mx[r], red);
        float l = 0.0f;
        for (int j = threadIdx.x; j < a.nbk; j += 256) l += __expf(pw[r][j] - m);
        lse[r] = m + __logf(block_sum(l, red));
    }
    for (int j = threadIdx.x; j < a.nbk; j += 256)
#pragma unroll
        for (int r = 0; r < kVsaRows; ++r) pw[r][j] = __expf(pw[r][j] - lse[r]);
    __syncthreads();
    float o[kVsaRows];
    col_sums<D, true>(pw, a.vbar + bh * a.nbk * D, a.nbk, part, o);
    for (int r = 0; r < nr; ++r) {
        if (threadIdx.x < D) a.oc[(row0 + r) * D + threadIdx.x] = o[r];
        if (threadIdx.x == 0) a.lsec[row0 + r] = lse[r];
    }
}

// O = O_fine + G * O_c[block(t)], 8 columns per thread.
__global__ __launch_bounds__(256) void vsa_combine_kernel(VsaArgs a) {
    const int C = a.D / 8;
    const int64_t total = a.BH * a.Nq * C;
    for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < total;
         gi += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(gi % C);
        const int64_t t = (gi / C) % a.Nq, bh = gi / ((int64_t)C * a.Nq);
        const int64_t off = at(bh, a.H, a.osb, a.osh, a.osn, t, 8 * c);
        const u32x4 f = *(const u32x4*)(a.o_fine + off);
        const u32x4 g = *(const u32x4*)(a.gate + off);
        const float* oc = a.oc + (bh * a.nbq + t / a.bt) * a.D + 8 * c;
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = fmaf(bf2f(g[e] & 0xffffu), oc[2 * e], bf2f(f[e] & 0xffffu));
            const float hi = fmaf(bf2f(g[e] >> 16), oc[2 * e + 1], bf2f(f[e] >> 16));
            r[e] = pack_rne(lo, hi);
        }
        *(u32x4*)(a.o + off) = r;
    }
}

// Per (query block i, bh): dO_c[i] = sum over the block's tokens of G * dO,
// and dG = dO * O_c[i] when requested. Thread (r, c): token rows r, r + R, ...
// of the block, columns 8 c .. 8 c + 7; R = 256 / (D / 8).
template <int D>
__global__ __launch_bounds__(256) void vsa_gate_reduce_kernel(VsaArgs a) {
    constexpr int C = D / 8, R = 256 / C;
    __shared__ float part[R][D];
    lds_poison(part);
    const int i = blockIdx.x;
    const int64_t bh = blockIdx.y, row = bh * a.nbq + i;
    const int c = threadIdx.x % C, r = threadIdx.x / C;
    const int t0 = i * a.bt, t1 = min(a.Nq, (i + 1) * a.bt);
    float oc[8], acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        oc[e] = a.oc[row * D + 8 * c + e];
        acc[e] = 0.0f;
    }
    for (int t = t0 + r; t < t1; t += R) {
        const u32x4 g = *(const u32x4*)(a.gate + at(bh, a.H, a.osb, a.osh, a.osn, t, 8 * c));
        const u32x4 dd = *(const u32x4*)(a.dout + at(bh, a.H, a.dsb, a.dsh, a.dsn, t, 8 * c));
        u32x4 dg;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float d0 = bf2f(dd[e] & 0xffffu), d1 = bf2f(dd[e] >> 16);
            acc[2 * e] = fmaf(bf2f(g[e] & 0xffffu), d0, acc[2 * e]);
            acc[2 * e + 1] = fmaf(bf2f(g[e] >> 16), d1, acc[2 * e + 1]);
            dg[e] = pack_rne(d0 * oc[2 * e], d1 * oc[2 * e + 1]);
        }
        if (a.dgate) *(u32x4*)(a.dgate + at(bh, a.H, a.osb, a.osh, a.osn, t, 8 * c)) = dg;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[r][8 * c + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float s = 0.0f;
        for (int rr = 0; rr < R; ++rr) s += part[rr][threadIdx.x];
        a.doc[row * D + threadIdx.x] = s;
    }
}

// Coarse backward, per kVsaRows query blocks i of one bh: the softmax rows P
// (from the forward's LSE), dS = P (dP - Dc) with Dc = rowsum(dO_c O_c) (kept
// for the key side), and dQbar[i] = sm_scale sum_j dS_ij Kbar_j.
template <int D>
__global__ __launch_bounds__(256) void vsa_coarse_bwd_q_kernel(VsaArgs a) {
    __shared__ float qs[kVsaRows][D], gs[kVsaRows][D];
    __shared__ float dsw[kVsaRows][kVsaMaxBlocks];
    __shared__ float part[kVsaRows][256];
    __shared__ float red[4];
    lds_poison(qs, gs, dsw, part, red);
    const int i0 = blockIdx.x * kVsaRows, nr = min(kVsaRows, a.nbq - i0);
    const int64_t bh = blockIdx.y, row0 = bh * a.nbq + i0;
    load_rows<D, true>(qs, a.qbar, row0, nr);
    load_rows<D, false>(gs, a.doc, row0, nr);
    float dc[kVsaRows], lse[kVsaRows];
#pragma unroll
    for (int r = 0; r < kVsaRows; ++r) {
        float x = 0.0f;
        if (r < nr && threadIdx.x < D)
            x = a.doc[(row0 + r) * D + threadIdx.x] * a.oc[(row0 + r) * D + threadIdx.x];
        dc[r] = block_sum(x, red);
        lse[r] = r < nr ? a.lsec[row0 + r] : 0.0f;
        if (r < nr && threadIdx.x == 0) a.dcc[row0 + r] = dc[r];
    }
    const uint16_t* kb = a.kbar + bh * a.nbk * D;
    const uint16_t* vb = a.vbar + bh * a.nbk * D;
    for (int j = threadIdx.x; j < a.nbk; j += 256) {
        float sv[kVsaRows], pv[kVsaRows];
        dots<D, true>(qs, kb + (int64_t)j * D, sv);
        dots<D, true>(gs, vb + (int64_t)j * D, pv);
#pragma unroll
        for (int r = 0; r < kVsaRows; ++r)
            dsw[r][j] = __expf(a.sm_scale * sv[r] - lse[r]) * (pv[r] - dc[r]);
    }
    __syncthreads();
    float g[kVsaRows];
    col_sums<D, true>(dsw, kb, a.nbk, part, g);
    for (int r = 0; r < nr; ++r)
        if (threadIdx.x < D) a.dqb[(row0 + r) * D + threadIdx.x] = a.sm_scale * g[r];
}

// Coarse backward, per kVsaRows key blocks j of one bh: P_ij and dS_ij
// recomputed for every query block i from contiguous rows (Qbar_i, dO_c[i],
// the LSE and Dc), then dKbar[j] = sm_scale sum_i dS_ij Qbar_i and dVbar[j] =
// sum_i P_ij dO_c[i].
template <int D>
__global__ __launch_bounds__(256) void vsa_coarse_bwd_k_kernel(VsaArgs a) {
    __shared__ float ks[kVsaRows][D], vs[kVsaRows][D];
    __shared__ float ws[kVsaRows][kVsaMaxBlocks], ps[kVsaRows][kVsaMaxBlocks];
    __shared__ float part[kVsaRows][256];
    lds_poison(ks, vs, ws, ps, part);
    const int j0 = blockIdx.x * kVsaRows, nr = min(kVsaRows, a.nbk - j0);
    const int64_t bh = blockIdx.y, row0 = bh * a.nbk + j0;
    load_rows<D, true>(ks, a.kbar, row0, nr);
    load_rows<D, true>(vs, a.vbar, row0, nr);
    __syncthreads();
    const uint16_t* qb = a.qbar + bh * a.nbq * D;
    const float* gb = a.doc + bh * a.nbq * D;
    for (int i = threadIdx.x; i < a.nbq; i += 256) {
        const int64_t qi = bh * a.nbq + i;
        const float lse = a.lsec[qi], dc = a.dcc[qi];
        float sv[kVsaRows], pv[kVsaRows];
        dots<D, true>(ks, qb + (int64_t)i * D, sv);
        dots<D, false>(vs, gb + (int64_t)i * D, pv);
#pragma unroll
        for (int r = 0; r < kVsaRows; ++r) {
            const float p = __expf(a.sm_scale * sv[r] - lse);
            ps[r][i] = p;
            ws[r][i] = p * (pv[r] - dc);
        }
    }
    __syncthreads();
    float gk[kVsaRows], gv[kVsaRows];
    col_sums<D, true>(ws, qb, a.nbq, part, gk);
    col_sums<D, false>(ps, gb, a.nbq, part, gv);
    for (int r = 0; r < nr; ++r)
        if (threadIdx.x < D) {
            a.dkb[(row0 + r) * D + threadIdx.x] = a.sm_scale * gk[r];
            a.dvb[(row0 + r) * D + threadIdx.x] = gv[r];
        }
}

// dQ, dK, dV (bf16, in place) += block gradient / block token count.
__global__ __launch_bounds__(256) void vsa_grad_add_kernel(VsaArgs a) {
    const int C = a.D / 8;
    const int64_t nq = a.BH * a.Nq * C, nk = a.BH * a.Nk * C;
    const int64_t total = nq + 2 * nk;
    for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < total;
         gi += (int64_t)gridDim.x * blockDim.x) {
        const int which = gi < nq ? 0 : (gi < nq + nk ? 1 : 2);
        const int64_t li = which == 0 ? gi : (which == 1 ? gi - nq : gi - nq - nk);
        const int N = which == 0 ? a.Nq : a.Nk;
        const int nb = which == 0 ? a.nbq : a.nbk;
        const int c = (int)(li % C);
        const int64_t t = (li / C) % N, bh = li / ((int64_t)C * N);
        const int blk = (int)(t / a.bt);
        const float inv = 1.0f / (float)(min(N, (blk + 1) * a.bt) - blk * a.bt);
        uint16_t* x = which == 0 ? a.dq : (which == 1 ? a.dk : a.dv);
        const int64_t sb = which == 0 ? a.dqsb : (which == 1 ? a.dksb : a.dvsb);
        const int64_t sh = which == 0 ? a.dqsh : (which == 1 ? a.dksh : a.dvsh);
        const int64_t sn = which == 0 ? a.dqsn : (which == 1 ? a.dksn : a.dvsn);
        const float* gb = (which == 0 ? a.dqb : (which == 1 ? a.dkb : a.dvb)) + (bh * nb + blk) * a.D + 8 * c;
        const int64_t off = at(bh, a.H, sb, sh, sn, t, 8 * c);
        const u32x4 w = *(const u32x4*)(x + off);
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r[e] = pack_rne(fmaf(gb[2 * e], inv, bf2f(w[e] & 0xffffu)), fmaf(gb[2 * e + 1], inv, bf2f(w[e] >> 16)));
        *(u32x4*)(x + off) = r;
    }
}

namespace {
unsigned grid_for(int64_t items) {
    const int64_t b = (items + 255) / 256;
    return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}
}  // namespace

hipError_t launch_vsa_pool(const VsaArgs& a, hipStream_t st) {
    const dim3 g(max(a.nbq, a.nbk), (unsigned)a.BH, 3);
    if (a.D == 128) vsa_pool_kernel<128><<<g, 256, 0, st>>>(a);
    else vsa_pool_kernel<64><<<g, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_vsa_coarse_fwd(const VsaArgs& a, hipStream_t st) {
    const dim3 g((a.nbq + kVsaRows - 1) / kVsaRows, (unsigned)a.BH);
    if (a.D == 128) vsa_coarse_fwd_kernel<128><<<g, 256, 0, st>>>(a);
    else vsa_coarse_fwd_kernel<64><<<g, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_vsa_combine(const VsaArgs& a, hipStream_t st) {
    vsa_combine_kernel<<<grid_for(a.BH * a.Nq * (a.D / 8)), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_vsa_gate_reduce(const VsaArgs& a, hipStream_t st) {
    const dim3 g(a.nbq, (unsigned)a.BH);
    if (a.D == 128) vsa_gate_reduce_kernel<128><<<g, 256, 0, st>>>(a);
    else vsa_gate_reduce_kernel<64><<<g, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_vsa_coarse_bwd(const VsaArgs& a, hipStream_t st) {
    const dim3 gq((a.nbq + kVsaRows - 1) / kVsaRows, (unsigned)a.BH),
        gk((a.nbk + kVsaRows - 1) / kVsaRows, (unsigned)a.BH);
    if (a.D == 128) {
        vsa_coarse_bwd_q_kernel<128><<<gq, 256, 0, st>>>(a);
        vsa_coarse_bwd_k_kernel<128><<<gk, 256, 0, st>>>(a);
    } else {
        vsa_coarse_bwd_q_kernel<64><<<gq, 256, 0, st>>>(a);
        vsa_coarse_bwd_k_kernel<64><<<gk, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_vsa_grad_add(const VsaArgs& a, hipStream_t st) {
    vsa_grad_add_kernel<<<grid_for(a.BH * (a.Nq + 2 * a.Nk) * (a.D / 8)), 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace aq
