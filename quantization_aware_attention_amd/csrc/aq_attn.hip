// Attn-QAT attention on MFMA: two-pass forward and split backward.
//
// What is computed (FastVideo VSA checkpoint metadata, attention.precision:
// NVFP4 fake quantization of Q, K, V and P with BF16 matmuls and no global
// scale; Attn-QAT training guide, FWD_EXACT_M row of the environment table, and
// the fastvideo-kernel commit message on the SM100 route: softmax statistics
// are saved by the forward and P is recomputed from them in the backward):
//
//   S = c0 Qq Kq^T, LSE = ln sum exp(S), P = exp(S - LSE), Pq = FQ_keys(P),
//   O = Pq Vq;   dV = Pq^T dO, dS = P (dO Vq^T - rowsum(dO O)),
//   dQ = c0 dS Kq, dK = c0 dS^T Qq.
//
// Quantizing the normalised P needs the final LSE before any P is formed, so
// the forward runs in two passes over the keys: pass 1 accumulates the row
// statistics, pass 2 recomputes S, quantizes P in registers and multiplies by
// V. Q, K and V arrive already fake-quantized (see aq_prep.hip), contiguous and
// zero-padded to multiples of 128 tokens.
//
// Scores are computed transposed, S^T = K Q^T, so one lane holds one query and
// 16 keys of a 32 x 32 tile: a 16-key P group is 8 registers of lane l plus
// 8 of lane l ^ 32, and its maximum takes one cross-lane swap.
#include "aq_kernels.h"

namespace aq {

__device__ __forceinline__ uint16_t bf16_rne1(float x) {
    const uint32_t u = __float_as_uint(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Key index (within a 32-key block) of accumulator register r for lane half hh.
__device__ __forceinline__ int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// Tile staging through registers. A tile is R rows of W bf16 (16-byte
// chunks); each of the 256 threads owns R * W / 8 / 256 chunks. Loads for the
// next tile are issued before the current tile is computed on, so global
// latency overlaps the MFMA work; the register copy is written to LDS after
// the next barrier.
template <int R, int W>
struct TileRegs {
    static constexpr int N = R * W / 8 / 256;
    static_assert(R * W / 8 % 256 == 0, "tile must split evenly over 256 threads");
    u32x4 v[N];
};

// Load rows [0, R) of a row-major matrix with leading dimension ld (elements).
template <int R, int W>
__device__ __forceinline__ void tile_load(TileRegs<R, W>& t, const uint16_t* g, int ld, int tid) {
#pragma unroll
    for (int j = 0; j < TileRegs<R, W>::N; ++j) {
        const int i = tid + 256 * j;
        const int r = i / (W / 8), cc = i % (W / 8);
        t.v[j] = *(const u32x4*)(g + (size_t)r * ld + cc * 8);
    }
}

// Write the tile to LDS with row pitch P (elements).
template <int R, int W, int P>
__device__ __forceinline__ void tile_store(uint16_t* lds, const TileRegs<R, W>& t, int tid) {
#pragma unroll
    for (int j = 0; j < TileRegs<R, W>::N; ++j) {
        const int i = tid + 256 * j;
        const int r = i / (W / 8), cc = i % (W / 8);
        *(u32x4*)(lds + r * P + cc * 8) = t.v[j];
    }
}

// Store a transposed C tile (rows = head dim d, columns = token) as bf16 rows
// of a [token][d] output: lane holds token `tok`, registers hold d.
template <int D>
__device__ __forceinline__ void store_rows_T(uint16_t* out_row, const f32x16* acc, float scale,
                                             int hh) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            u32x2 w;
            w[0] = pack_rne(acc[db][4 * rr + 0] * scale, acc[db][4 * rr + 1] * scale);
            w[1] = pack_rne(acc[db][4 * rr + 2] * scale, acc[db][4 * rr + 3] * scale);
            *(u32x2*)(out_row + db * 32 + rr * 8 + hh * 4) = w;
        }
    }
}

// ---------------------------------------------------------------------------
// Forward pass 1: LSE per query row.
template <int D>
__global__ __launch_bounds__(256) void fwd_lse_kernel(AttnArgs a) {
    constexpr int BN = 64, KP = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int bh = blockIdx.y, qblk = blockIdx.x;
    const int q0 = qblk * 128 + wave * 32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
    u32x4 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = *(const u32x4*)(Qb + (size_t)(q0 + l32) * D + c * 16 + hh * 8);
    const int32_t* kvi = a.kv_idx ? a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk : nullptr;
    const int n_iter = kvi ? a.topk * 2 : a.Nk_pad / BN;
    auto tile_at = [&](int it) { return kvi ? kvi[it >> 1] * 128 + (it & 1) * BN : it * BN; };
    float m = kNegBig, l = 0.0f;
    TileRegs<BN, D> rk;
    tile_load(rk, Kb + (size_t)tile_at(0) * D, D, tid);
    for (int it = 0; it < n_iter; ++it) {
        const int kt = tile_at(it);
        __syncthreads();
        tile_store<BN, D, KP>(sK, rk, tid);
        __syncthreads();
        if (it + 1 < n_iter) tile_load(rk, Kb + (size_t)tile_at(it + 1) * D, D, tid);
        const bool tail = kt + BN > a.Nk;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 acc = {};
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const u32x4 kf = *(const u32x4*)(sK + (kb * 32 + l32) * KP + c * 16 + hh * 8);
                acc = mfma(kf, qf[c], acc);
            }
            if (tail) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kt + kb * 32 + acc_row(r, hh) >= a.Nk) acc[r] = -INFINITY;
            }
            float mx = m;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
            const float mc = mx * a.c;
            float sum = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[r], a.c, -mc));
            l = l * __builtin_amdgcn_exp2f((m - mx) * a.c) + sum;
            m = mx;
        }
    }
    const float mp = partner_lane(m), lp = partner_lane(l);
    const float mt = fmaxf(m, mp);
    const float lt = l * __builtin_amdgcn_exp2f((m - mt) * a.c) +
                     lp * __builtin_amdgcn_exp2f((mp - mt) * a.c);
    const int q = q0 + l32;
    if (hh == 0 && q < a.Nq) a.lse_out[(size_t)bh * a.Nq + q] = (mt * a.c + log2f(lt)) * kLn2;
}

// ---------------------------------------------------------------------------
// Forward pass 2: O = FQ(P) Vq with P = exp(S - LSE).
template <int D, bool QP>
__global__ __launch_bounds__(256) void fwd_out_kernel(AttnArgs a) {
    constexpr int BN = 64, KP = D + 8, VP = BN + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t sV[D * VP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int bh = blockIdx.y, qblk = blockIdx.x;
    const int q0 = qblk * 128 + wave * 32;
    const int q = q0 + l32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
    const uint16_t* Vtb = a.Vt + (size_t)bh * D * a.Nk_pad;
    u32x4 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = *(const u32x4*)(Qb + (size_t)(q0 + l32) * D + c * 16 + hh * 8);
    const float lse2 = (q < a.Nq) ? a.lse[(size_t)bh * a.Nq + q] * kLog2e : 0.0f;
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    const int32_t* kvi = a.kv_idx ? a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk : nullptr;
    const int n_iter = kvi ? a.topk * 2 : a.Nk_pad / BN;
    auto tile_at = [&](int it) { return kvi ? kvi[it >> 1] * 128 + (it & 1) * BN : it * BN; };
    TileRegs<BN, D> rk;
    TileRegs<D, BN> rv;
    tile_load(rk, Kb + (size_t)tile_at(0) * D, D, tid);
    tile_load(rv, Vtb + tile_at(0), a.Nk_pad, tid);
    for (int it = 0; it < n_iter; ++it) {
        const int kt = tile_at(it);
        __syncthreads();
        tile_store<BN, D, KP>(sK, rk, tid);
        tile_store<D, BN, VP>(sV, rv, tid);
        __syncthreads();
        if (it + 1 < n_iter) {
            const int kn = tile_at(it + 1);
            tile_load(rk, Kb + (size_t)kn * D, D, tid);
            tile_load(rv, Vtb + kn, a.Nk_pad, tid);
        }
        const bool tail = kt + BN > a.Nk;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 acc = {};
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const u32x4 kf = *(const u32x4*)(sK + (kb * 32 + l32) * KP + c * 16 + hh * 8);
                acc = mfma(kf, qf[c], acc);
            }
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], a.c, -lse2));
            if (tail) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kt + kb * 32 + acc_row(r, hh) >= a.Nk) p[r] = 0.0f;
            }
            u32x4 bfr[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                float* pg = p + 8 * g;
                if (QP) {
                    quant_group8_hw(pg);
                    bfr[g] = u32x4{pack_exact(pg[0], pg[1]), pack_exact(pg[2], pg[3]),
                                   pack_exact(pg[4], pg[5]), pack_exact(pg[6], pg[7])};
                } else {
                    bfr[g] = u32x4{pack_rne(pg[0], pg[1]), pack_rne(pg[2], pg[3]),
                                   pack_rne(pg[4], pg[5]), pack_rne(pg[6], pg[7])};
                }
            }
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const u32x4 vf =
                        *(const u32x4*)(sV + (db * 32 + l32) * VP + kb * 32 + g * 16 + hh * 8);
                    o[db] = mfma(vf, bfr[g], o[db]);
                }
            }
        }
    }
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.o + b * a.osb + h * a.osh + (int64_t)q * a.osn, o, 1.0f, hh);
    }
}

// ---------------------------------------------------------------------------
// Backward dQ: grid over 128-query blocks, loop over key tiles.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(AttnArgs a) {
    constexpr int BN = 64, KP = D + 8, VP = BN + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t sV[BN * KP];
    __shared__ __attribute__((aligned(16))) uint16_t sKt[D * VP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int bh = blockIdx.y, qblk = blockIdx.x;
    const int q0 = qblk * 128 + wave * 32;
    const int q = q0 + l32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* dOb = a.dOw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
    const uint16_t* Vb = a.Vw + (size_t)bh * a.Nk_pad * D;
    const uint16_t* Ktb = a.Kt + (size_t)bh * D * a.Nk_pad;
    u32x4 qf[D / 16], df[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        qf[c] = *(const u32x4*)(Qb + (size_t)q * D + c * 16 + hh * 8);
        df[c] = *(const u32x4*)(dOb + (size_t)q * D + c * 16 + hh * 8);
    }
    const float lse2 = a.lse2[(size_t)bh * a.Nq_pad + q];
    const float dl = a.delta[(size_t)bh * a.Nq_pad + q];
    f32x16 dqa[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqa[db] = f32x16{};
    const int32_t* kvi = a.kv_idx ? a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk : nullptr;
    const int n_iter = kvi ? a.topk * 2 : a.Nk_pad / BN;
    auto tile_at = [&](int it) { return kvi ? kvi[it >> 1] * 128 + (it & 1) * BN : it * BN; };
    TileRegs<BN, D> rk, rv;
    TileRegs<D, BN> rkt;
    {
        const int k0 = tile_at(0);
        tile_load(rk, Kb + (size_t)k0 * D, D, tid);
        tile_load(rv, Vb + (size_t)k0 * D, D, tid);
        tile_load(rkt, Ktb + k0, a.Nk_pad, tid);
    }
    for (int it = 0; it < n_iter; ++it) {
        const int kt = tile_at(it);
        __syncthreads();
        tile_store<BN, D, KP>(sK, rk, tid);
        tile_store<BN, D, KP>(sV, rv, tid);
        tile_store<D, BN, VP>(sKt, rkt, tid);
        __syncthreads();
        if (it + 1 < n_iter) {
            const int kn = tile_at(it + 1);
            tile_load(rk, Kb + (size_t)kn * D, D, tid);
            tile_load(rv, Vb + (size_t)kn * D, D, tid);
            tile_load(rkt, Ktb + kn, a.Nk_pad, tid);
        }
        const bool tail = kt + BN > a.Nk;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const u32x4 kf = *(const u32x4*)(sK + (kb * 32 + l32) * KP + c * 16 + hh * 8);
                s = mfma(kf, qf[c], s);
                const u32x4 vf = *(const u32x4*)(sV + (kb * 32 + l32) * KP + c * 16 + hh * 8);
                dp = mfma(vf, df[c], dp);
            }
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[r], a.c, -lse2));
                if (tail && kt + kb * 32 + acc_row(r, hh) >= a.Nk) p = 0.0f;
                ds[r] = p * (dp[r] - dl);
            }
            u32x4 bfr[2];
#pragma unroll
            for (int g = 0; g < 2; ++g)
                bfr[g] = u32x4{pack_rne(ds[8 * g + 0], ds[8 * g + 1]),
                               pack_rne(ds[8 * g + 2], ds[8 * g + 3]),
                               pack_rne(ds[8 * g + 4], ds[8 * g + 5]),
                               pack_rne(ds[8 * g + 6], ds[8 * g + 7])};
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const u32x4 kt_f =
                        *(const u32x4*)(sKt + (db * 32 + l32) * VP + kb * 32 + g * 16 + hh * 8);
                    dqa[db] = mfma(kt_f, bfr[g], dqa[db]);
                }
            }
        }
    }
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.dq + b * a.dqsb + h * a.dqsh + (int64_t)q * a.dqsn, dqa, a.sm_scale, hh);
    }
}

// ---------------------------------------------------------------------------
// Backward dK, dV: grid over 128-key blocks (32 keys per wave), loop over
// 64-query tiles. P^T-layout values are transposed through a per-wave LDS tile
// so that queries become the contraction index.
template <int D, bool QP>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(AttnArgs a) {
    constexpr int BM = 64, KP = D + 8, QTP = BM + 8;
    __shared__ __attribute__((aligned(16))) uint16_t sQ[BM * KP];
    __shared__ __attribute__((aligned(16))) uint16_t sdO[BM * KP];
    __shared__ __attribute__((aligned(16))) uint16_t sQt[D * QTP];
    __shared__ __attribute__((aligned(16))) uint16_t sdOt[D * QTP];
    __shared__ __attribute__((aligned(16))) uint16_t sT[4][2][32 * 32];
    __shared__ float sL[BM], sDl[BM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int bh = blockIdx.y, kblk = blockIdx.x;
    const int k0 = kblk * 128 + wave * 32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* dOb = a.dOw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* Qtb = a.Qt + (size_t)bh * D * a.Nq_pad;
    const uint16_t* dOtb = a.dOt + (size_t)bh * D * a.Nq_pad;
    const float* Lb = a.lse2 + (size_t)bh * a.Nq_pad;
    const float* Db = a.delta + (size_t)bh * a.Nq_pad;
    u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        kf[c] = *(const u32x4*)(a.Kw + ((size_t)bh * a.Nk_pad + k0 + l32) * D + c * 16 + hh * 8);
        vf[c] = *(const u32x4*)(a.Vw + ((size_t)bh * a.Nk_pad + k0 + l32) * D + c * 16 + hh * 8);
    }
    f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dka[db] = f32x16{};
        dva[db] = f32x16{};
    }
    const bool tailK = kblk * 128 + 128 > a.Nk;
    const int32_t* ql = nullptr;
    int n_iter = a.Nq_pad / BM;
    if (a.q_list) {
        ql = a.q_list + ((size_t)bh * a.nbk + kblk) * a.nbq;
        n_iter = 2 * a.q_count[(size_t)bh * a.nbk + kblk];
    }
    // Per-wave 32 x 32 transpose tiles, row = query, 64 bytes per row, 8-byte
    // column chunks XOR-swizzled by (row / 4) % 8 so that both the row writes
    // and the transposing reads are free of bank conflicts.
    uint16_t* Tp = sT[wave][0];
    uint16_t* Td = sT[wave][1];
    const int wsw = (l32 >> 2) & 7;
    const int grp = lane >> 4, i16 = lane & 15;
    auto tile_at = [&](int it) { return ql ? ql[it >> 1] * 128 + (it & 1) * BM : it * BM; };
    TileRegs<BM, D> rq, rdo;
    TileRegs<D, BM> rqt, rdot;
    float rl = 0.0f, rdl = 0.0f;
    auto load_all = [&](int qt) {
        tile_load(rq, Qb + (size_t)qt * D, D, tid);
        tile_load(rdo, dOb + (size_t)qt * D, D, tid);
        tile_load(rqt, Qtb + qt, a.Nq_pad, tid);
        tile_load(rdot, dOtb + qt, a.Nq_pad, tid);
        if (tid < BM) {
            rl = Lb[qt + tid];
            rdl = Db[qt + tid];
        }
    };
    if (n_iter > 0) load_all(tile_at(0));
    for (int it = 0; it < n_iter; ++it) {
        __syncthreads();
        tile_store<BM, D, KP>(sQ, rq, tid);
        tile_store<BM, D, KP>(sdO, rdo, tid);
        tile_store<D, BM, QTP>(sQt, rqt, tid);
        tile_store<D, BM, QTP>(sdOt, rdot, tid);
        if (tid < BM) {
            sL[tid] = rl;
            sDl[tid] = rdl;
        }
        __syncthreads();
        if (it + 1 < n_iter) load_all(tile_at(it + 1));
#pragma unroll
        for (int qb = 0; qb < BM / 32; ++qb) {
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const u32x4 qv = *(const u32x4*)(sQ + (qb * 32 + l32) * KP + c * 16 + hh * 8);
                s = mfma(kf[c], qv, s);
                const u32x4 dv = *(const u32x4*)(sdO + (qb * 32 + l32) * KP + c * 16 + hh * 8);
                dp = mfma(vf[c], dv, dp);
            }
            const float L = sL[qb * 32 + l32];
            const float Dl = sDl[qb * 32 + l32];
            float p[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], a.c, -L));
                if (tailK && k0 + acc_row(r, hh) >= a.Nk) p[r] = 0.0f;
                ds[r] = p[r] * (dp[r] - Dl);
            }
            if (QP) {
                quant_group8_hw(p);
                quant_group8_hw(p + 8);
            }
            // transpose through LDS: write rows (query = l32; keys 8a + 4hh ..
            // + 3 from registers 4a .. 4a + 3), read columns with the
            // transposing load so that lane (key, hh) gets queries 16g + 8hh + j
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int off = l32 * 32 + ((((2 * a4 + hh) ^ wsw)) << 2);
                u32x2 wp, wd;
                if (QP) {
                    wp[0] = pack_exact(p[4 * a4], p[4 * a4 + 1]);
                    wp[1] = pack_exact(p[4 * a4 + 2], p[4 * a4 + 3]);
                } else {
                    wp[0] = pack_rne(p[4 * a4], p[4 * a4 + 1]);
                    wp[1] = pack_rne(p[4 * a4 + 2], p[4 * a4 + 3]);
                }
                wd[0] = pack_rne(ds[4 * a4], ds[4 * a4 + 1]);
                wd[1] = pack_rne(ds[4 * a4 + 2], ds[4 * a4 + 3]);
                *(u32x2*)(Tp + off) = wp;
                *(u32x2*)(Td + off) = wd;
            }
            u32x4 pT[2], dT[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int row = 16 * g + 8 * hh + 4 * half + (i16 >> 2);
                    const int col8 = 4 * (grp & 1) + (i16 & 3);
                    const int off = row * 32 + ((col8 ^ ((row >> 2) & 7)) << 2);
                    const u32x2 vp = lds_read_tr16(Tp + off);
                    const u32x2 vd = lds_read_tr16(Td + off);
                    pT[g][2 * half] = vp[0];
                    pT[g][2 * half + 1] = vp[1];
                    dT[g][2 * half] = vd[0];
                    dT[g][2 * half + 1] = vd[1];
                }
            }
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const int off = (db * 32 + l32) * QTP + qb * 32 + g * 16 + hh * 8;
                    dva[db] = mfma(*(const u32x4*)(sdOt + off), pT[g], dva[db]);
                    dka[db] = mfma(*(const u32x4*)(sQt + off), dT[g], dka[db]);
                }
            }
        }
    }
    const int key = k0 + l32;
    if (key < a.Nk) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.dk + b * a.dksb + h * a.dksh + (int64_t)key * a.dksn, dka, a.sm_scale, hh);
        store_rows_T<D>(a.dv + b * a.dvsb + h * a.dvsh + (int64_t)key * a.dvsn, dva, 1.0f, hh);
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_fwd_lse(const AttnArgs& a, int D, hipStream_t st) {
    dim3 grid(a.Nq_pad / 128, a.BH);
    if (D == 128) fwd_lse_kernel<128><<<grid, 256, 0, st>>>(a);
    else fwd_lse_kernel<64><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_fwd_out(const AttnArgs& a, int D, hipStream_t st) {
    dim3 grid(a.Nq_pad / 128, a.BH);
    if (D == 128) {
        if (a.quant_p) fwd_out_kernel<128, true><<<grid, 256, 0, st>>>(a);
        else fwd_out_kernel<128, false><<<grid, 256, 0, st>>>(a);
    } else {
        if (a.quant_p) fwd_out_kernel<64, true><<<grid, 256, 0, st>>>(a);
        else fwd_out_kernel<64, false><<<grid, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const AttnArgs& a, int D, hipStream_t st) {
    dim3 grid(a.Nq_pad / 128, a.BH);
    if (D == 128) bwd_dq_kernel<128><<<grid, 256, 0, st>>>(a);
    else bwd_dq_kernel<64><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const AttnArgs& a, int D, hipStream_t st) {
    dim3 grid(a.Nk_pad / 128, a.BH);
    if (D == 128) {
        if (a.quant_p) bwd_dkdv_kernel<128, true><<<grid, 256, 0, st>>>(a);
        else bwd_dkdv_kernel<128, false><<<grid, 256, 0, st>>>(a);
    } else {
        if (a.quant_p) bwd_dkdv_kernel<64, true><<<grid, 256, 0, st>>>(a);
        else bwd_dkdv_kernel<64, false><<<grid, 256, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace aq
