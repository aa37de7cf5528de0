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
#include <type_traits>

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
// each lane fetches the global chunk that the swizzle maps to that slot. The
// per-lane source offsets depend only on the tile shape, so they are computed
// once; each issue adds them to a wave-uniform tile base.
template <int R, int W, int NT>
struct AsyncTile {
    static constexpr int CH = W / 8, NB = R * CH / 64, NW = NT / 64, NJ = NB / NW;
    static_assert(NB % NW == 0, "tile must split evenly over the waves");
    uint32_t goff[NJ];  // byte offsets of this lane's chunks in the source tile
    int wave;           // wave index (uniform)
    __device__ __forceinline__ void init(int ld, int tid) {
        const int lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int L = (j * NW + wave) * 64 + lane;
            const int row = L / CH, pch = L % CH;
            goff[j] = (uint32_t)(row * ld + ((pch ^ swz<W>(row)) << 3)) * 2u;
        }
    }
    __device__ __forceinline__ void issue(uint16_t* lds, const uint16_t* g) const {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            __builtin_amdgcn_global_load_lds((glb_void_t*)((const char*)g + goff[j]),
                                             (lds_void_t*)(lds + (j * NW + wave) * 512), 16, 0, 0);
    }
};

// Asynchronous copy of 64 consecutive floats into LDS by one wave.
__device__ __forceinline__ void async_f32x64(float* lds, const float* g, int lane) {
    __builtin_amdgcn_global_load_lds((glb_void_t*)(g + lane), (lds_void_t*)lds, 4, 0, 0);
}

// Wait until this wave's direct-to-LDS loads have landed (vmcnt = 0).
__device__ __forceinline__ void wait_async() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Largest block list a sparse workgroup stages in LDS (key blocks per query
// block, or query blocks per key block).
constexpr int kMaxBlockList = 1024;

// Start token of tile `it` in a workgroup's visiting order: consecutive
// T-token tiles (dense), or the 128 / T tiles of each listed 128-token block
// in list order (sparse; the list is staged in LDS).
template <bool SPARSE, int T>
__device__ __forceinline__ int tile_start(const int* lst, int it) {
    constexpr int PER = 128 / T;
    return SPARSE ? lst[it / PER] * 128 + (it % PER) * T : it * T;
}

// Copy a block list of n entries into LDS (all threads, then a barrier).
__device__ __forceinline__ void stage_list(int* lst, const int32_t* g, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) lst[i] = g[i];
    __syncthreads();
}

// Double-buffered tile loop. issue(buf, it) starts the asynchronous copy of
// tile it into buffer buf; body(buf, it, tail) consumes it. Full tiles run the
// unmasked body; a partial last tile (last_partial) runs the masked body once,
// after the loop, so that only one body is live inside the loop.
template <class Issue, class Body>
__device__ __forceinline__ void tile_pipeline(int n_iter, bool last_partial, Issue issue,
                                              Body body) {
    const int n_main = n_iter - (last_partial ? 1 : 0);
    issue(0, 0);
    int it = 0;
    for (; it < n_main; ++it) {
        wait_async();
        __syncthreads();
        if (it + 1 < n_iter) issue((it + 1) & 1, it + 1);
        body(it & 1, it, std::false_type{});
    }
    if (last_partial) {
        wait_async();
        __syncthreads();
        body(it & 1, it, std::true_type{});
    }
}

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
    template <bool tail>
    __device__ static void block(const uint16_t* sK, int kt, int Nk, const u32x4* qf, float c,
                                 float& m, float& l, int l32, int hh) {
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

template <int D, bool SPARSE>
__global__ __launch_bounds__(256) void fwd_lse_kernel(AttnArgs a) {
    constexpr int BN = FwdLse<D>::BN;
    __shared__ __attribute__((aligned(1024))) uint16_t sK[2][BN * D];
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
    __shared__ int lst[SPARSE ? kMaxBlockList : 1];
    if (SPARSE) stage_list(lst, a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk, a.topk);
    const int n_iter = SPARSE ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return tile_start<SPARSE, BN>(lst, it); };
    float m = kNegBig, l = 0.0f;
    AsyncTile<BN, D, 256> tk;
    tk.init(D, tid);
    tile_pipeline(
        n_iter, tile_at(n_iter - 1) + BN > a.Nk,
        [&](int buf, int it) { tk.issue(sK[buf], Kb + (size_t)tile_at(it) * D); },
        [&](int buf, int it, auto tail) {
            FwdLse<D>::template block<decltype(tail)::value>(sK[buf], tile_at(it), a.Nk, qf, a.c,
                                                             m, l, l32, hh);
        });
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
    template <bool tail>
    __device__ static void block(const uint16_t* sK, const uint16_t* sV, int kt, int Nk,
                                 const u32x4* qf, float c, float lse2, f32x16* o, int l32, int hh) {
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

template <int D, bool QP, bool SPARSE>
__global__ __launch_bounds__(256, 2) void fwd_out_kernel(AttnArgs a) {
    constexpr int BN = FwdOut<D, QP>::BN;
    __shared__ __attribute__((aligned(1024))) uint16_t sK[2][BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[2][D * BN];
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
    __shared__ int lst[SPARSE ? kMaxBlockList : 1];
    if (SPARSE) stage_list(lst, a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk, a.topk);
    const int n_iter = SPARSE ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return tile_start<SPARSE, BN>(lst, it); };
    AsyncTile<BN, D, 256> tk;
    AsyncTile<D, BN, 256> tv;
    tk.init(D, tid);
    tv.init(a.Nk_pad, tid);
    tile_pipeline(
        n_iter, tile_at(n_iter - 1) + BN > a.Nk,
        [&](int buf, int it) {
            const int kt = tile_at(it);
            tk.issue(sK[buf], Kb + (size_t)kt * D);
            tv.issue(sV[buf], Vtb + kt);
        },
        [&](int buf, int it, auto tail) {
            FwdOut<D, QP>::template block<decltype(tail)::value>(sK[buf], sV[buf], tile_at(it), a.Nk,
                                                                 qf, a.c, lse2, o, l32, hh);
        });
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
    template <bool tail>
    __device__ static void block(const uint16_t* sK, const uint16_t* sV, const uint16_t* sKt,
                                 int kt, int Nk, const u32x4* qf, const u32x4* df, float c,
                                 float lse2, float dl, f32x16* dqa, int l32, int hh) {
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

template <int D, int NW, bool SPARSE>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(AttnArgs a) {
    constexpr int BN = BwdDq<D>::BN, NT = NW * 64;
    __shared__ __attribute__((aligned(1024))) uint16_t sK[2][BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[2][BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sT[2][D * BN];
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
    static_assert(!SPARSE || NW == 4, "sparse dQ workgroups cover one query block");
    __shared__ int lst[SPARSE ? kMaxBlockList : 1];
    if (SPARSE) stage_list(lst, a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk, a.topk);
    const int n_iter = SPARSE ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return tile_start<SPARSE, BN>(lst, it); };
    AsyncTile<BN, D, NT> tk;
    AsyncTile<D, BN, NT> tt;
    tk.init(D, tid);
    tt.init(a.Nk_pad, tid);
    tile_pipeline(
        n_iter, tile_at(n_iter - 1) + BN > a.Nk,
        [&](int buf, int it) {
            const int kt = tile_at(it);
            tk.issue(sK[buf], Kb + (size_t)kt * D);
            tk.issue(sV[buf], Vb + (size_t)kt * D);
            tt.issue(sT[buf], Ktb + kt);
        },
        [&](int buf, int it, auto tail) {
            BwdDq<D>::template block<decltype(tail)::value>(sK[buf], sV[buf], sT[buf], tile_at(it),
                                                            a.Nk, qf, df, a.c, lse2, dl, dqa, l32,
                                                            hh);
        });
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.dq + b * a.dqsb + h * a.dqsh + (int64_t)q * a.dqsn, dqa, a.sm_scale, hh);
    }
}

// ---------------------------------------------------------------------------
// Backward dK, dV: 4 waves x 32 keys, loop over 64-query tiles. Pq and dS
// (queries on lanes) are transposed through a per-wave LDS tile so that
// queries become the contraction index of dV^T = dO^T Pq and dK^T = Q^T dS.
//
// One wave per SIMD fits (the dK and dV accumulators alone take 128
// registers), so the two 32-query halves of a tile are software-pipelined
// inside the wave: the S/dP products of half 1 run on the matrix cores while
// the vector units turn half 0's S/dP into P, Pq and dS and transpose them,
// and the dV/dK products of half 0 run while half 1 is processed.
// sched_group_barrier lays the two instruction streams out interleaved.

// MFMA issue pattern for a region: N x {1 MFMA, R LDS reads, V VALU}.
template <int N, int R, int V>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (R) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    }
}

template <int D, bool QP, bool TAILK>
struct BwdDkdv {
    static constexpr int BM = 64;

    // S^T and dP^T for the 32 queries of half qb (16 MFMAs).
    __device__ static void sdp(const uint16_t* sQ, const uint16_t* sdO, int qb, const u32x4* kf,
                               const u32x4* vf, f32x16& s, f32x16& dp, int l32, int hh) {
        s = f32x16{};
        dp = f32x16{};
        const int row = qb * 32 + l32;
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
            const u32x4 qv = *(const u32x4*)(sQ + toff<D>(row, 2 * cc + hh));
            s = mfma(kf[cc], qv, s);
            const u32x4 dv = *(const u32x4*)(sdO + toff<D>(row, 2 * cc + hh));
            dp = mfma(vf[cc], dv, dp);
        }
        // the vector units read S and dP next: accumulate them in vector registers
        asm volatile("" : "+v"(s));
        asm volatile("" : "+v"(dp));
    }

    // P, Pq, dS of half qb and their transposes (keys on lanes) as B operands.
    __device__ static void valu(const f32x16& s, const f32x16& dp, const float* sL,
                                const float* sDl, int qb, uint16_t* Tp, uint16_t* Td, int k0,
                                int Nk, float c, u32x4* pT, u32x4* dT, int lane) {
        const int l32 = lane & 31, hh = lane >> 5;
        const int wsw = (l32 >> 2) & 7;
        const int grp = lane >> 4, i16 = lane & 15;
        const int row = qb * 32 + l32;
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
        // Transpose through LDS: row = query (l32), keys 8a + 4hh .. + 3 from
        // registers 4a .. 4a + 3; 8-byte column chunks XOR-swizzled by
        // (row / 4) % 8 so that the row writes and the transposing column
        // reads avoid bank conflicts.
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
    }

    // dV^T += dO^T Pq and dK^T += Q^T dS for half qb (16 MFMAs).
    __device__ static void dvdk(const uint16_t* sQt, const uint16_t* sdOt, int qb,
                                const u32x4* pT, const u32x4* dT, f32x16* dka, f32x16* dva,
                                int l32, int hh) {
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

    __device__ static void block(const uint16_t* sQ, const uint16_t* sdO, const uint16_t* sQt,
                                 const uint16_t* sdOt, const float* sL, const float* sDl,
                                 uint16_t* Tp, uint16_t* Td, int k0, int Nk, const u32x4* kf,
                                 const u32x4* vf, float c, f32x16* dka, f32x16* dva, int lane) {
        const int l32 = lane & 31, hh = lane >> 5;
        f32x16 s0, dp0, s1, dp1;
        u32x4 pT0[2], dT0[2], pT1[2], dT1[2];
        sdp(sQ, sdO, 0, kf, vf, s0, dp0, l32, hh);
        __builtin_amdgcn_sched_barrier(0);
        sdp(sQ, sdO, 1, kf, vf, s1, dp1, l32, hh);
        valu(s0, dp0, sL, sDl, 0, Tp, Td, k0, Nk, c, pT0, dT0, lane);
        interleave_mfma<2 * D / 16, 0, 8>();
        __builtin_amdgcn_sched_barrier(0);
        dvdk(sQt, sdOt, 0, pT0, dT0, dka, dva, l32, hh);
        valu(s1, dp1, sL, sDl, 1, Tp, Td, k0, Nk, c, pT1, dT1, lane);
        interleave_mfma<D / 8, 0, 8>();
        __builtin_amdgcn_sched_barrier(0);
        dvdk(sQt, sdOt, 1, pT1, dT1, dka, dva, l32, hh);
        __builtin_amdgcn_sched_barrier(0);
    }
};

// LDS of the dK/dV kernel: double-buffered Q, dO, Q^T, dO^T tiles, the two
// statistics rows, and the per-wave transpose tiles.
template <int D>
struct DkdvLds {
    static constexpr int BM = 64;
    uint16_t q[2][BM * D], o[2][BM * D], qt[2][D * BM], ot[2][D * BM];
    uint16_t t[4 * 2 * 32 * 32];
    float l[2][BM], d[2][BM];
    int lst[kMaxBlockList];
};

template <int D, bool QP, bool TAILK, bool SPARSE>
__device__ __forceinline__ void dkdv_loop(const AttnArgs& a, DkdvLds<D>& S, int bh, int kblk,
                                          f32x16* dka, f32x16* dva) {
    constexpr int BM = DkdvLds<D>::BM;
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
        // Keep the K/V operands in accumulation registers (MFMA reads its A
        // operand from there) so that the vector registers stay free for the
        // S, dP, P and dS values the vector units work on.
        asm volatile("" : "+a"(kf[c]));
        asm volatile("" : "+a"(vf[c]));
    }
    int n_iter = (a.Nq + BM - 1) / BM;
    if (SPARSE) {
        const int cnt = a.q_count[(size_t)bh * a.nbk + kblk];
        stage_list(S.lst, a.q_list + ((size_t)bh * a.nbk + kblk) * a.nbq, cnt);
        n_iter = 2 * cnt;
    }
    if (n_iter == 0) return;
    auto tile_at = [&](int it) { return tile_start<SPARSE, BM>(S.lst, it); };
    AsyncTile<BM, D, 256> tr;
    AsyncTile<D, BM, 256> tc;
    tr.init(D, tid);
    tc.init(a.Nq_pad, tid);
    auto issue = [&](int buf, int qt) {
        tr.issue(S.q[buf], Qb + (size_t)qt * D);
        tr.issue(S.o[buf], dOb + (size_t)qt * D);
        tc.issue(S.qt[buf], Qtb + qt);
        tc.issue(S.ot[buf], dOtb + qt);
        if (wave == 0) async_f32x64(S.l[buf], Lb + qt, lane);
        if (wave == 1) async_f32x64(S.d[buf], Db + qt, lane);
    };
    uint16_t* Tp = S.t + wave * 2048;
    uint16_t* Td = Tp + 1024;
    issue(0, tile_at(0));
    for (int it = 0; it < n_iter; ++it) {
        const int cur = it & 1;
        wait_async();
        __syncthreads();
        if (it + 1 < n_iter) issue(cur ^ 1, tile_at(it + 1));
        BwdDkdv<D, QP, TAILK>::block(S.q[cur], S.o[cur], S.qt[cur], S.ot[cur], S.l[cur],
                                     S.d[cur], Tp, Td, k0, a.Nk, kf, vf, a.c, dka, dva, lane);
    }
}

template <int D, bool QP, bool SPARSE>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(1024))) DkdvLds<D> S;
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
    if (kblk * 128 + 128 > a.Nk) dkdv_loop<D, QP, true, SPARSE>(a, S, bh, kblk, dka, dva);
    else dkdv_loop<D, QP, false, SPARSE>(a, S, bh, kblk, dka, dva);
    const int key = kblk * 128 + wave * 32 + l32;
    if (key < a.Nk) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.dk + b * a.dksb + h * a.dksh + (int64_t)key * a.dksn, dka, a.sm_scale, hh);
        store_rows_T<D>(a.dv + b * a.dvsb + h * a.dvsh + (int64_t)key * a.dvsn, dva, 1.0f, hh);
    }
}

// ---------------------------------------------------------------------------
template <int D, bool SP>
static void fwd_lse_go(const AttnArgs& a, dim3 g, hipStream_t st) {
    fwd_lse_kernel<D, SP><<<g, 256, 0, st>>>(a);
}

hipError_t launch_fwd_lse(const AttnArgs& a, int D, hipStream_t st) {
    const bool sp = a.kv_idx != nullptr;
    dim3 grid(sp ? a.nbq : (a.Nq + 127) / 128, a.BH);
    if (D == 128) sp ? fwd_lse_go<128, true>(a, grid, st) : fwd_lse_go<128, false>(a, grid, st);
    else sp ? fwd_lse_go<64, true>(a, grid, st) : fwd_lse_go<64, false>(a, grid, st);
    return hipGetLastError();
}

template <int D, bool QP, bool SP>
static void fwd_out_go(const AttnArgs& a, dim3 g, hipStream_t st) {
    fwd_out_kernel<D, QP, SP><<<g, 256, 0, st>>>(a);
}

template <int D>
static void fwd_out_d(const AttnArgs& a, dim3 g, bool sp, hipStream_t st) {
    if (a.quant_p) sp ? fwd_out_go<D, true, true>(a, g, st) : fwd_out_go<D, true, false>(a, g, st);
    else sp ? fwd_out_go<D, false, true>(a, g, st) : fwd_out_go<D, false, false>(a, g, st);
}

hipError_t launch_fwd_out(const AttnArgs& a, int D, hipStream_t st) {
    const bool sp = a.kv_idx != nullptr;
    dim3 grid(sp ? a.nbq : (a.Nq + 127) / 128, a.BH);
    if (D == 128) fwd_out_d<128>(a, grid, sp, st);
    else fwd_out_d<64>(a, grid, sp, st);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const AttnArgs& a, int D, hipStream_t st) {
    if (a.kv_idx) {
        dim3 grid(a.nbq, a.BH);
        if (D == 128) bwd_dq_kernel<128, 4, true><<<grid, 256, 0, st>>>(a);
        else bwd_dq_kernel<64, 4, true><<<grid, 256, 0, st>>>(a);
    } else {
        dim3 grid((a.Nq + 255) / 256, a.BH);
        if (D == 128) bwd_dq_kernel<128, 8, false><<<grid, 512, 0, st>>>(a);
        else bwd_dq_kernel<64, 8, false><<<grid, 512, 0, st>>>(a);
    }
    return hipGetLastError();
}

template <int D, bool QP, bool SP>
static void dkdv_go(const AttnArgs& a, dim3 g, hipStream_t st) {
    bwd_dkdv_kernel<D, QP, SP><<<g, 256, 0, st>>>(a);
}

template <int D>
static void dkdv_d(const AttnArgs& a, dim3 g, bool sp, hipStream_t st) {
    if (a.quant_p) sp ? dkdv_go<D, true, true>(a, g, st) : dkdv_go<D, true, false>(a, g, st);
    else sp ? dkdv_go<D, false, true>(a, g, st) : dkdv_go<D, false, false>(a, g, st);
}

hipError_t launch_bwd_dkdv(const AttnArgs& a, int D, hipStream_t st) {
    dim3 grid((a.Nk + 127) / 128, a.BH);
    const bool sp = a.q_list != nullptr;
    if (D == 128) dkdv_d<128>(a, grid, sp, st);
    else dkdv_d<64>(a, grid, sp, st);
    return hipGetLastError();
}

}  // namespace aq
