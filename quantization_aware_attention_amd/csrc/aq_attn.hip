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
// zero-padded to multiples of 256 tokens.
//
// Scores are computed transposed, S^T = K Q^T, so one lane holds one query and
// 16 keys of a 32 x 32 tile: a 16-key P group is 8 registers of lane l plus
// 8 of lane l ^ 32, and its maximum takes one cross-lane swap.
//
// Tiles stream from HBM into LDS with direct-to-LDS loads (global_load_lds,
// 16 bytes per lane), double-buffered: the loads of tile i + 1 are in flight
// while tile i is multiplied. LDS rows are unpadded; 16-byte chunks are XOR
// swizzled by row so that the MFMA operand reads are free of bank conflicts.
// As on the pages' SM100 route, full key tiles run without bounds masks and a
// separate masked step handles the partial tail tile.
#include "aq_kernels.h"

namespace aq {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// Key index (within a 32-key block) of accumulator register r for lane half hh.
__device__ __forceinline__ int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

// Swizzle of 16-byte chunks for tiles with W bf16 per row: 256-byte rows XOR
// the chunk with row % 16, 128-byte rows with (row / 2) % 8. Sixteen
// consecutive rows read at the same logical chunk then hit 16 distinct bank
// quads.
template <int W>
__device__ __forceinline__ int swz(int row) {
    static_assert(W == 64 || W == 128, "tile width");
    return W == 128 ? (row & 15) : ((row >> 1) & 7);
}

// Element offset of logical 16-byte chunk c of row `row` in a swizzled tile.
template <int W>
__device__ __forceinline__ int toff(int row, int c) {
    return row * W + ((c ^ swz<W>(row)) << 3);
}

// Asynchronous copy of an R x W bf16 tile (row-major source with leading
// dimension ld) into a swizzled LDS tile. Each wave-wide direct-to-LDS load
// fills one contiguous 1 KB block; lane i's 16 bytes land at block + 16 i, so
// each lane fetches the global chunk that the swizzle maps to that slot.
template <int R, int W, int NT>
__device__ __forceinline__ void async_tile(uint16_t* lds, const uint16_t* g, int ld, int tid) {
    constexpr int CH = W / 8;
    constexpr int NB = R * CH / 64;
    constexpr int NW = NT / 64;
    static_assert(NB % NW == 0, "tile must split evenly over the waves");
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int j = 0; j < NB / NW; ++j) {
        const int B = j * NW + wave;
        const int L = B * 64 + lane;
        const int row = L / CH, pch = L % CH;
        const int lch = pch ^ swz<W>(row);
        __builtin_amdgcn_global_load_lds((glb_void_t*)(g + (size_t)row * ld + lch * 8),
                                         (lds_void_t*)(lds + B * 512), 16, 0, 0);
    }
}

// Asynchronous copy of 64 consecutive floats into LDS by one wave.
__device__ __forceinline__ void async_f32x64(float* lds, const float* g, int lane) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)(g + lane), (lds_void_t*)lds, 4, 0, 0);
}

// Wait until this wave's direct-to-LDS loads have landed (vmcnt = 0).
__device__ __forceinline__ void wait_async() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Store a transposed C tile (rows = head dim d, columns = token) as bf16 rows
// of a [token][d] output: lane holds one token, registers hold d.
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

// S^T block (32 keys x 32 queries): keys are rows kr0.. of a swizzled [*, D]
// LDS tile, the queries' B operands are in registers.
template <int D>
__device__ __forceinline__ f32x16 scores_T(const uint16_t* sK, int kr0, const u32x4* qf, int l32,
                                           int hh) {
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        const u32x4 kf = *(const u32x4*)(sK + toff<D>(kr0 + l32, 2 * c + hh));
        acc = mfma(kf, qf[c], acc);
    }
    return acc;
}

// ---------------------------------------------------------------------------
// Forward pass 1: LSE per query row. 4 waves x 32 queries, 64-key tiles.
template <int D>
struct FwdLse {
    static constexpr int BN = 64;
    __device__ static void block(const uint16_t* sK, int kt, int Nk, const u32x4* qf, float c,
                                 float& m, float& l, int l32, int hh, bool tail) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 acc = scores_T<D>(sK, kb * 32, qf, l32, hh);
            if (tail) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kt + kb * 32 + acc_row(r, hh) >= Nk) acc[r] = -INFINITY;
            }
            float mx = m;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
            const float mc = mx * c;
            float sum = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[r], c, -mc));
            l = l * __builtin_amdgcn_exp2f((m - mx) * c) + sum;
            m = mx;
        }
    }
};

template <int D>
__global__ __launch_bounds__(256) void fwd_lse_kernel(AttnArgs a) {
    constexpr int BN = FwdLse<D>::BN;
    __shared__ __attribute__((aligned(1024))) uint16_t sK0[BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sK1[BN * D];
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
    const int n_iter = kvi ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return kvi ? kvi[it >> 1] * 128 + (it & 1) * BN : it * BN; };
    float m = kNegBig, l = 0.0f;
    async_tile<BN, D, 256>(sK0, Kb + (size_t)tile_at(0) * D, D, tid);
    for (int it = 0; it < n_iter; it += 2) {
        {
            const int kt = tile_at(it);
            wait_async();
            __syncthreads();
            if (it + 1 < n_iter) async_tile<BN, D, 256>(sK1, Kb + (size_t)tile_at(it + 1) * D, D, tid);
            FwdLse<D>::block(sK0, kt, a.Nk, qf, a.c, m, l, l32, hh, kt + BN > a.Nk);
        }
        if (it + 1 < n_iter) {
            const int kt = tile_at(it + 1);
            wait_async();
            __syncthreads();
            if (it + 2 < n_iter) async_tile<BN, D, 256>(sK0, Kb + (size_t)tile_at(it + 2) * D, D, tid);
            FwdLse<D>::block(sK1, kt, a.Nk, qf, a.c, m, l, l32, hh, kt + BN > a.Nk);
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
// Forward pass 2: O = FQ(P) Vq with P = exp(S - LSE). 4 waves x 32 queries.
template <int D, bool QP>
struct FwdOut {
    static constexpr int BN = 64;
    __device__ static void block(const uint16_t* sK, const uint16_t* sV, int kt, int Nk,
                                 const u32x4* qf, float c, float lse2, f32x16* o, int l32, int hh,
                                 bool tail) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            const f32x16 acc = scores_T<D>(sK, kb * 32, qf, l32, hh);
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(acc[r], c, -lse2));
            if (tail) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kt + kb * 32 + acc_row(r, hh) >= Nk) p[r] = 0.0f;
            }
            u32x4 bfr[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                float* pg = p + 8 * g;
                if (QP) quant_group8_hw(pg);
                bfr[g] = u32x4{pack_rne(pg[0], pg[1]), pack_rne(pg[2], pg[3]),
                               pack_rne(pg[4], pg[5]), pack_rne(pg[6], pg[7])};
            }
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const u32x4 vf =
                        *(const u32x4*)(sV + toff<BN>(db * 32 + l32, 4 * kb + 2 * g + hh));
                    o[db] = mfma(vf, bfr[g], o[db]);
                }
            }
        }
    }
};

template <int D, bool QP>
__global__ __launch_bounds__(256, 2) void fwd_out_kernel(AttnArgs a) {
    constexpr int BN = FwdOut<D, QP>::BN;
    __shared__ __attribute__((aligned(1024))) uint16_t sK0[BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sK1[BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sV0[D * BN];
    __shared__ __attribute__((aligned(1024))) uint16_t sV1[D * BN];
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
    const int n_iter = kvi ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return kvi ? kvi[it >> 1] * 128 + (it & 1) * BN : it * BN; };
    auto issue = [&](uint16_t* dK, uint16_t* dV, int kt) {
        async_tile<BN, D, 256>(dK, Kb + (size_t)kt * D, D, tid);
        async_tile<D, BN, 256>(dV, Vtb + kt, a.Nk_pad, tid);
    };
    issue(sK0, sV0, tile_at(0));
    for (int it = 0; it < n_iter; it += 2) {
        {
            const int kt = tile_at(it);
            wait_async();
            __syncthreads();
            if (it + 1 < n_iter) issue(sK1, sV1, tile_at(it + 1));
            FwdOut<D, QP>::block(sK0, sV0, kt, a.Nk, qf, a.c, lse2, o, l32, hh, kt + BN > a.Nk);
        }
        if (it + 1 < n_iter) {
            const int kt = tile_at(it + 1);
            wait_async();
            __syncthreads();
            if (it + 2 < n_iter) issue(sK0, sV0, tile_at(it + 2));
            FwdOut<D, QP>::block(sK1, sV1, kt, a.Nk, qf, a.c, lse2, o, l32, hh, kt + BN > a.Nk);
        }
    }
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.o + b * a.osb + h * a.osh + (int64_t)q * a.osn, o, 1.0f, hh);
    }
}

// ---------------------------------------------------------------------------
// Backward dQ: NW waves x 32 queries, loop over 64-key tiles.
template <int D>
struct BwdDq {
    static constexpr int BN = 64;
    __device__ static void block(const uint16_t* sK, const uint16_t* sV, const uint16_t* sKt,
                                 int kt, int Nk, const u32x4* qf, const u32x4* df, float c,
                                 float lse2, float dl, f32x16* dqa, int l32, int hh, bool tail) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int cc = 0; cc < D / 16; ++cc) {
                const int row = kb * 32 + l32;
                const u32x4 kf = *(const u32x4*)(sK + toff<D>(row, 2 * cc + hh));
                s = mfma(kf, qf[cc], s);
                const u32x4 vf = *(const u32x4*)(sV + toff<D>(row, 2 * cc + hh));
                dp = mfma(vf, df[cc], dp);
            }
            float ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
                if (tail && kt + kb * 32 + acc_row(r, hh) >= Nk) p = 0.0f;
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
                    const u32x4 ktf =
                        *(const u32x4*)(sKt + toff<BN>(db * 32 + l32, 4 * kb + 2 * g + hh));
                    dqa[db] = mfma(ktf, bfr[g], dqa[db]);
                }
            }
        }
    }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(AttnArgs a) {
    constexpr int BN = BwdDq<D>::BN, NT = NW * 64;
    __shared__ __attribute__((aligned(1024))) uint16_t sK0[BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sK1[BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sV0[BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sV1[BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sT0[D * BN];
    __shared__ __attribute__((aligned(1024))) uint16_t sT1[D * BN];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int bh = blockIdx.y, qblk = blockIdx.x;
    const int q0 = qblk * (NW * 32) + wave * 32;
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
    // sparse launches use NW = 4 so that a workgroup is one 128-query block
    const int32_t* kvi = a.kv_idx ? a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk : nullptr;
    const int n_iter = kvi ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return kvi ? kvi[it >> 1] * 128 + (it & 1) * BN : it * BN; };
    auto issue = [&](uint16_t* dK, uint16_t* dV, uint16_t* dT, int kt) {
        async_tile<BN, D, NT>(dK, Kb + (size_t)kt * D, D, tid);
        async_tile<BN, D, NT>(dV, Vb + (size_t)kt * D, D, tid);
        async_tile<D, BN, NT>(dT, Ktb + kt, a.Nk_pad, tid);
    };
    issue(sK0, sV0, sT0, tile_at(0));
    for (int it = 0; it < n_iter; it += 2) {
        {
            const int kt = tile_at(it);
            wait_async();
            __syncthreads();
            if (it + 1 < n_iter) issue(sK1, sV1, sT1, tile_at(it + 1));
            BwdDq<D>::block(sK0, sV0, sT0, kt, a.Nk, qf, df, a.c, lse2, dl, dqa, l32, hh,
                            kt + BN > a.Nk);
        }
        if (it + 1 < n_iter) {
            const int kt = tile_at(it + 1);
            wait_async();
            __syncthreads();
            if (it + 2 < n_iter) issue(sK0, sV0, sT0, tile_at(it + 2));
            BwdDq<D>::block(sK1, sV1, sT1, kt, a.Nk, qf, df, a.c, lse2, dl, dqa, l32, hh,
                            kt + BN > a.Nk);
        }
    }
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.dq + b * a.dqsb + h * a.dqsh + (int64_t)q * a.dqsn, dqa, a.sm_scale, hh);
    }
}

// ---------------------------------------------------------------------------
// Backward dK, dV: 4 waves x 32 keys, loop over 64-query tiles. Pq and dS
// (queries on lanes) are transposed through a per-wave LDS tile so that
// queries become the contraction index of dV^T = dO^T Pq and dK^T = Q^T dS.
template <int D, bool QP, bool TAILK>
struct BwdDkdv {
    static constexpr int BM = 64;
    __device__ static void block(const uint16_t* sQ, const uint16_t* sdO, const uint16_t* sQt,
                                 const uint16_t* sdOt, const float* sL, const float* sDl,
                                 uint16_t* Tp, uint16_t* Td, int k0, int Nk, const u32x4* kf,
                                 const u32x4* vf, float c, f32x16* dka, f32x16* dva, int lane) {
        const int l32 = lane & 31, hh = lane >> 5;
        const int wsw = (l32 >> 2) & 7;
        const int grp = lane >> 4, i16 = lane & 15;
#pragma unroll
        for (int qb = 0; qb < BM / 32; ++qb) {
            f32x16 s = {}, dp = {};
            const int row = qb * 32 + l32;
#pragma unroll
            for (int cc = 0; cc < D / 16; ++cc) {
                const u32x4 qv = *(const u32x4*)(sQ + toff<D>(row, 2 * cc + hh));
                s = mfma(kf[cc], qv, s);
                const u32x4 dv = *(const u32x4*)(sdO + toff<D>(row, 2 * cc + hh));
                dp = mfma(vf[cc], dv, dp);
            }
            const float L = sL[row];
            const float Dl = sDl[row];
            float p[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c, -L));
                if (TAILK && k0 + acc_row(r, hh) >= Nk) p[r] = 0.0f;
                ds[r] = p[r] * (dp[r] - Dl);
            }
            if (QP) {
                quant_group8_hw(p);
                quant_group8_hw(p + 8);
            }
            // Transpose through LDS: row = query (l32), keys 8a + 4hh .. + 3
            // from registers 4a .. 4a + 3; 8-byte column chunks XOR-swizzled
            // by (row / 4) % 8 so that these row writes and the transposing
            // column reads are both free of bank conflicts.
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int off = l32 * 32 + (((2 * a4 + hh) ^ wsw) << 2);
                u32x2 wp, wd;
                wp[0] = pack_rne(p[4 * a4], p[4 * a4 + 1]);
                wp[1] = pack_rne(p[4 * a4 + 2], p[4 * a4 + 3]);
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
                    const int trow = 16 * g + 8 * hh + 4 * half + (i16 >> 2);
                    const int col8 = 4 * (grp & 1) + (i16 & 3);
                    const int off = trow * 32 + ((col8 ^ ((trow >> 2) & 7)) << 2);
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
                    const int off = toff<BM>(db * 32 + l32, 4 * qb + 2 * g + hh);
                    dva[db] = mfma(*(const u32x4*)(sdOt + off), pT[g], dva[db]);
                    dka[db] = mfma(*(const u32x4*)(sQt + off), dT[g], dka[db]);
                }
            }
        }
    }
};

// LDS of the dK/dV kernel: double-buffered Q, dO, Q^T, dO^T tiles, the two
// statistics rows, and the per-wave transpose tiles.
template <int D>
struct DkdvLds {
    static constexpr int BM = 64;
    uint16_t *sQ0, *sQ1, *sO0, *sO1, *sQt0, *sQt1, *sOt0, *sOt1, *sT;
    float *sL0, *sL1, *sD0, *sD1;
};

template <int D, bool QP, bool TAILK>
__device__ __forceinline__ void dkdv_loop(const AttnArgs& a, const DkdvLds<D>& S, int bh, int kblk,
                                          f32x16* dka, f32x16* dva) {
    constexpr int BM = BwdDkdv<D, QP, TAILK>::BM;
    uint16_t *sQ0 = S.sQ0, *sQ1 = S.sQ1, *sO0 = S.sO0, *sO1 = S.sO1;
    uint16_t *sQt0 = S.sQt0, *sQt1 = S.sQt1, *sOt0 = S.sOt0, *sOt1 = S.sOt1;
    float *sL0 = S.sL0, *sL1 = S.sL1, *sD0 = S.sD0, *sD1 = S.sD1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
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
    const int32_t* ql = nullptr;
    int n_iter = (a.Nq + BM - 1) / BM;
    if (a.q_list) {
        ql = a.q_list + ((size_t)bh * a.nbk + kblk) * a.nbq;
        n_iter = 2 * a.q_count[(size_t)bh * a.nbk + kblk];
    }
    if (n_iter == 0) return;
    auto tile_at = [&](int it) { return ql ? ql[it >> 1] * 128 + (it & 1) * BM : it * BM; };
    auto issue = [&](uint16_t* dQ, uint16_t* dO, uint16_t* dQt, uint16_t* dOt, float* dL,
                     float* dD, int qt) {
        async_tile<BM, D, 256>(dQ, Qb + (size_t)qt * D, D, tid);
        async_tile<BM, D, 256>(dO, dOb + (size_t)qt * D, D, tid);
        async_tile<D, BM, 256>(dQt, Qtb + qt, a.Nq_pad, tid);
        async_tile<D, BM, 256>(dOt, dOtb + qt, a.Nq_pad, tid);
        if (wave == 0) async_f32x64(dL, Lb + qt, lane);
        if (wave == 1) async_f32x64(dD, Db + qt, lane);
    };
    uint16_t* Tp = S.sT + wave * 2048;
    uint16_t* Td = Tp + 1024;
    issue(sQ0, sO0, sQt0, sOt0, sL0, sD0, tile_at(0));
    for (int it = 0; it < n_iter; it += 2) {
        wait_async();
        __syncthreads();
        if (it + 1 < n_iter) issue(sQ1, sO1, sQt1, sOt1, sL1, sD1, tile_at(it + 1));
        BwdDkdv<D, QP, TAILK>::block(sQ0, sO0, sQt0, sOt0, sL0, sD0, Tp, Td, k0, a.Nk, kf, vf,
                                     a.c, dka, dva, lane);
        if (it + 1 < n_iter) {
            wait_async();
            __syncthreads();
            if (it + 2 < n_iter) issue(sQ0, sO0, sQt0, sOt0, sL0, sD0, tile_at(it + 2));
            BwdDkdv<D, QP, TAILK>::block(sQ1, sO1, sQt1, sOt1, sL1, sD1, Tp, Td, k0, a.Nk, kf,
                                         vf, a.c, dka, dva, lane);
        }
    }
}

template <int D, bool QP>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(AttnArgs a) {
    constexpr int BM = DkdvLds<D>::BM;
    __shared__ __attribute__((aligned(1024))) uint16_t sQ0[BM * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sQ1[BM * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sO0[BM * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sO1[BM * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sQt0[D * BM];
    __shared__ __attribute__((aligned(1024))) uint16_t sQt1[D * BM];
    __shared__ __attribute__((aligned(1024))) uint16_t sOt0[D * BM];
    __shared__ __attribute__((aligned(1024))) uint16_t sOt1[D * BM];
    __shared__ __attribute__((aligned(1024))) uint16_t sT[4 * 2 * 32 * 32];
    __shared__ __attribute__((aligned(256))) float sL0[BM], sL1[BM], sD0[BM], sD1[BM];
    const DkdvLds<D> S{sQ0, sQ1, sO0, sO1, sQt0, sQt1, sOt0, sOt1, sT, sL0, sL1, sD0, sD1};
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hh = lane >> 5, l32 = lane & 31;
    const int bh = blockIdx.y, kblk = blockIdx.x;
    f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        dka[db] = f32x16{};
        dva[db] = f32x16{};
    }
    // keys beyond Nk exist only in the last key block: mask them there only
    if (kblk * 128 + 128 > a.Nk) dkdv_loop<D, QP, true>(a, S, bh, kblk, dka, dva);
    else dkdv_loop<D, QP, false>(a, S, bh, kblk, dka, dva);
    const int key = kblk * 128 + wave * 32 + l32;
    if (key < a.Nk) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.dk + b * a.dksb + h * a.dksh + (int64_t)key * a.dksn, dka, a.sm_scale, hh);
        store_rows_T<D>(a.dv + b * a.dvsb + h * a.dvsh + (int64_t)key * a.dvsn, dva, 1.0f, hh);
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_fwd_lse(const AttnArgs& a, int D, hipStream_t st) {
    dim3 grid(a.kv_idx ? a.nbq : (a.Nq + 127) / 128, a.BH);
    if (D == 128) fwd_lse_kernel<128><<<grid, 256, 0, st>>>(a);
    else fwd_lse_kernel<64><<<grid, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_fwd_out(const AttnArgs& a, int D, hipStream_t st) {
    dim3 grid(a.kv_idx ? a.nbq : (a.Nq + 127) / 128, a.BH);
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
    if (a.kv_idx) {
        dim3 grid(a.nbq, a.BH);
        if (D == 128) bwd_dq_kernel<128, 4><<<grid, 256, 0, st>>>(a);
        else bwd_dq_kernel<64, 4><<<grid, 256, 0, st>>>(a);
    } else {
        dim3 grid((a.Nq + 255) / 256, a.BH);
        if (D == 128) bwd_dq_kernel<128, 8><<<grid, 512, 0, st>>>(a);
        else bwd_dq_kernel<64, 8><<<grid, 512, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const AttnArgs& a, int D, hipStream_t st) {
    dim3 grid((a.Nk + 127) / 128, a.BH);
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
