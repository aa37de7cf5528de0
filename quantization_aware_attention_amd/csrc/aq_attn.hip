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
// the chunk with row % 16, 128-byte rows with f((row / 2) % 8), where
// f(x) = x ^ ((x & 2) << 1) permutes 0..7. Sixteen consecutive rows read at
// the same logical chunk then hit 16 distinct bank quads; for 128-byte rows
// f also separates rows 4 apart (f(x) and f(x + 2) differ in bit 2), which
// keeps the transposing operand reads of the backward conflict-free.
template <int W>
__device__ __forceinline__ int swz(int row) {
    static_assert(W == 64 || W == 128, "tile width");
    if (W == 128) return row & 15;
    const int x = (row >> 1) & 7;
    return x ^ ((x & 2) << 1);
}

// Element offset of logical 16-byte chunk c of row `row` in a swizzled tile.
template <int W>
__device__ __forceinline__ int toff(int row, int c) {
    return row * W + ((c ^ swz<W>(row)) << 3);
}

// Natural-layout [64][D] query tile (row = query): logical 16-byte chunk c of
// row r sits at chunk c ^ nswz(r). Both reads of the fused backward are then
// free of bank conflicts: 16-byte reads of one chunk in 16 consecutive rows
// (the B operands of S^T and dP^T) and transposing reads that cover 4
// consecutive rows x 4 consecutive chunks per 32 lanes (the A operands of
// dV^T and dK^T).
template <int D>
__device__ __forceinline__ int nswz(int row) {
    static_assert(D == 64 || D == 128, "head dim");
    if (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
    return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int noff(int row, int c) {
    return row * D + ((c ^ nswz<D>(row)) << 3);
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16-byte (and 4-byte) LDS-DMA copies: lane i's global bytes land at LDS
// byte address lds + 16 i (+ 4 i). lds and g are wave-uniform.
__device__ __forceinline__ const void* uniform_ptr(const void* g) {
    const uint64_t v = (uint64_t)g;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(uint32_t lds, const void* g, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(g))
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t lds, const void* g, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(g))
                 : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

// Asynchronous copy of an R x W bf16 tile (row-major source with leading
// dimension ld) into a swizzled LDS tile. Each wave-wide direct-to-LDS load
// fills one contiguous 1 KB block; lane i's 16 bytes land at block + 16 i, so
// each lane fetches the global chunk that the swizzle maps to that slot. The
// per-lane source offsets depend only on the tile shape, so they are computed
// once; each issue adds them to a wave-uniform tile base. The copies are
// issued in inline assembly (dma16): the compiler does not track them, so
// its own LDS waits stay partial, and the kernel waits for the copies itself
// (wait_async) before the barrier that publishes a tile.
// With PERM32, tile row `row` receives source row perm32 of its position in
// its 32-row block (the key order of score tiles, see perm32).
template <int R, int W, int NT, bool PERM32 = false>
struct AsyncTile {
    static constexpr int CH = W / 8, NB = R * CH / 64, NW = NT / 64, NJ = NB / NW;
    static_assert(NB % NW == 0, "tile must split evenly over the waves");
    static_assert(!PERM32 || R % 32 == 0, "permuted tiles hold whole 32-row blocks");
    uint32_t goff[NJ];  // byte offsets of this lane's chunks in the source tile
    int wave;           // wave index (uniform)
    __device__ __forceinline__ void init(int ld, int tid) {
        const int lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int L = (j * NW + wave) * 64 + lane;
            const int row = L / CH, pch = L % CH;
            const int src = PERM32 ? (row & ~31) | perm32(row & 31) : row;
            goff[j] = (uint32_t)(src * ld + ((pch ^ swz<W>(row)) << 3)) * 2u;
        }
    }
    __device__ __forceinline__ void issue(uint16_t* lds, const uint16_t* g) const {
#pragma unroll
        for (int j = 0; j < NJ; ++j) dma16(lds_addr(lds + (j * NW + wave) * 512), g, goff[j]);
    }
};

// Wait until at most N of this wave's vector memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Wait until this wave's direct-to-LDS loads have landed (vmcnt = 0).
__device__ __forceinline__ void wait_async() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Tile index (along gridDim.x) and (batch, head) index of this workgroup for
// dense launches. Workgroups are dealt to the chip's 8 XCDs round-robin by
// linear id, and each XCD has its own L2. Remapping the ids so that XCD x
// runs a contiguous range of the head-major work list keeps the workgroups in
// flight on one XCD within one or two heads, so the K/V (or Q/dO) tiles they
// all stream are fetched into that XCD's L2 once rather than by every XCD.
__device__ __forceinline__ int xcd_index(int L, int n) {
    const int x = L & 7, slot = L >> 3, per = n >> 3, rem = n & 7;
    return x * per + (x < rem ? x : rem) + slot;
}
__device__ __forceinline__ void xcd_work(int& tile, int& bh) {
    const int nx = gridDim.x;
    const int w = xcd_index(blockIdx.x + blockIdx.y * nx, gridDim.x * gridDim.y);
    tile = w % nx;
    bh = w / nx;
}

// Work of one workgroup of a dense launch over nblk blocks of nt tiles each
// that runs in rounds of one workgroup per compute unit. The first nf
// workgroups take one whole block each (head-major, each XCD a contiguous
// range). The F = nblk - nf blocks of the last, partial round are dealt out
// as one run of F nt tiles, `chunk` consecutive tiles per further workgroup
// (stream-K), so that the round's work spreads over every compute unit. A
// chunk (chunk <= nt) covers the end of one block and the start of the next
// at most: up to two segments, whose fp32 partial sums go to slots 2 c and
// 2 c + 1 of chunk c, for a fixup to add.
struct Seg {
    int blk, t0, t1, slot;  // block, tile range [t0, t1), partial slot (-1: whole block)
};
__device__ __forceinline__ int work_segments(int nf, int nblk, int nt, int chunk, Seg* s) {
    const int L = blockIdx.x;
    if (L < nf) {
        s[0] = Seg{xcd_index(L, nf), 0, nt, -1};
        return 1;
    }
    const int c = xcd_index(L - nf, gridDim.x - nf);
    const int total = (nblk - nf) * nt, start = c * chunk, end = min(start + chunk, total);
    const int j = start / nt, e0 = min(end, (j + 1) * nt);
    s[0] = Seg{nf + j, start - j * nt, e0 - j * nt, 2 * c};
    if (end <= e0) return 1;
    s[1] = Seg{nf + j + 1, 0, end - (j + 1) * nt, 2 * c + 1};
    return 2;
}

// Adds the partial sums of last-round block j (0-based within the round) in
// chunk order: rows of 256 x D fp32 per slot; x (8 values at element e) is
// the sum. Chunk c's segment in block j is its second when the chunk starts
// in block j - 1.
template <int D>
__device__ __forceinline__ void sum_slots(const float* part, int j, int nt, int chunk, int e,
                                          f32x4_t& x0, f32x4_t& x1) {
    const int c0 = j * nt / chunk, c1 = ((j + 1) * nt - 1) / chunk;
    x0 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    x1 = x0;
    for (int c = c0; c <= c1; ++c) {
        const int slot = 2 * c + (c * chunk / nt < j ? 1 : 0);
        const float* r = part + (size_t)slot * 256 * D + e;
        x0 += *(const f32x4_t*)r;
        x1 += *(const f32x4_t*)(r + 4);
    }
}

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

// Buffer b (std::integral_constant 0 or 1) of a pair of LDS buffers. The two
// buffers are separate variables and every access names one of them at
// compile time, so the compiler can tell reads of one buffer from the
// direct-to-LDS loads into the other and does not make them wait for those
// loads to land.
template <class B, class T>
__device__ __forceinline__ T* sel(B, T* b0, T* b1) {
    return B::value ? b1 : b0;
}

// Number of trailing tiles of a visiting order that can hold keys >= Nk and
// must run masked: the last tile when it is partial (dense), or both tiles of
// the last listed 128-token block when that block ends past Nk (sparse: the
// list is ascending, so the sequence's partial last block, if selected, comes
// last, and either of its two tiles may be partial or wholly past Nk).
template <bool SPARSE, int T>
__device__ __forceinline__ int masked_tiles(const int32_t* lst, int n_iter, int Nk) {
    constexpr int PER = 128 / T;
    if (n_iter <= 0) return 0;
    if (SPARSE) return (lst[(n_iter - 1) / PER] * 128 + 128 > Nk) ? PER : 0;
    return ((n_iter - 1) * T + T > Nk) ? 1 : 0;
}

// Double-buffered tile loop. issue(buf, it) starts the asynchronous copy of
// tile it into buffer buf; body(buf, it, tail) consumes it; buf is a
// compile-time 0 or 1 (the loop is unrolled by two). Full tiles run the
// unmasked body; the last n_masked tiles (at most two) run the masked body
// after the loop, so that only the unmasked body is live inside the loop. The
// loop covers an even number of tiles, so the masked tiles (one to three:
// an odd leftover full tile runs masked too, which masks nothing) start in
// buffer 0 and their buffers are known at compile time.
template <class Issue, class Body>
__device__ __forceinline__ void tile_pipeline(int n_iter, int n_masked, Issue issue,
                                              Body body) {
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using TAIL = std::true_type;
    const int n_main = (n_iter - n_masked) & ~1;
    issue(B0{}, 0);
    for (int it = 0; it < n_main; it += 2) {
        wait_async();
        __syncthreads();
        issue(B1{}, it + 1);
        body(B0{}, it, std::false_type{});
        wait_async();
        __syncthreads();
        if (it + 2 < n_iter) issue(B0{}, it + 2);
        body(B1{}, it + 1, std::false_type{});
    }
    // tile n_main (if any) is in flight here, the next one is not
    if (n_main < n_iter) {
        wait_async();
        __syncthreads();
        if (n_main + 1 < n_iter) issue(B1{}, n_main + 1);
        body(B0{}, n_main, TAIL{});
    }
    if (n_main + 1 < n_iter) {
        wait_async();
        __syncthreads();
        if (n_main + 2 < n_iter) issue(B0{}, n_main + 2);
        body(B1{}, n_main + 1, TAIL{});
    }
    if (n_main + 2 < n_iter) {
        wait_async();
        __syncthreads();
        body(B0{}, n_main + 2, TAIL{});
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

// As store_rows_T, as fp32 without scaling: row points at this lane's token.
template <int D>
__device__ __forceinline__ void store_rows_f32(float* row, const f32x16* acc, int hh) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            *(f32x4_t*)(row + db * 32 + rr * 8 + hh * 4) =
                f32x4_t{acc[db][4 * rr], acc[db][4 * rr + 1], acc[db][4 * rr + 2], acc[db][4 * rr + 3]};
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

// Issue order for a chain of N MFMAs that each take one operand from LDS:
// PRE reads first, then one MFMA per further read, so every operand is
// requested PRE MFMAs (PRE x 32 cycles) before its use. Ends the scheduling
// region.
template <int N, int PRE>
__device__ __forceinline__ void lds_mfma_chain() {
    __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
    for (int i = 0; i < N - PRE; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PRE, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// As lds_mfma_chain, with V vector instructions issued after each MFMA, so
// that independent vector work fills the matrix core's busy cycles.
constexpr int kValuPerMfma = 8;
template <int N, int PRE, int V>
__device__ __forceinline__ void mfma_valu_chain() {
    __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < N - PRE) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// As mfma_chain_m, with F vector instructions issued after the PRE reads and
// before the first MFMA (vector work that the matrix products of other waves
// can hide, ahead of this wave's own products).
template <int N, int M, int PRE, int F, int V>
__device__ __forceinline__ void mfma_chain_front() {
    constexpr int NR = N / M;
    __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
    if (F > 0) __builtin_amdgcn_sched_group_barrier(0x002, F, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i % M == M - 1 && i / M < NR - PRE) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Issue order for N MFMAs fed by N / M LDS reads (M products per operand):
// PRE reads first, then after every M MFMAs the next read, with V vector
// instructions after each MFMA. Ends the scheduling region.
template <int N, int M, int PRE, int V>
__device__ __forceinline__ void mfma_chain_m() {
    constexpr int NR = N / M;
    __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i % M == M - 1 && i / M < NR - PRE) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// Forward pass 1: LSE per query row. 8 waves x 32 queries, 64-key tiles.
// Each lane keeps a reference m and the sum l of exp2((S - m) c) over its
// keys; LSE log2(e) = m c + log2 l for any m, so m only has to keep the terms
// finite and l's magnitude in range. With LAZY the lane first sums a block
// against its current m and takes a new maximum only when that sum exceeds
// kLazySum (always on its first block, where m c is -1e30 c): no per-element
// maximum in the common case. Without LAZY m is the exact running maximum,
// which the row-max variant stores.
constexpr float kLazySum = 4294967296.0f;  // 2^32: far below fp32 overflow for any row length

template <int D>
struct FwdLse {
    static constexpr int BN = 64;
    template <bool tail, bool LAZY>
    __device__ static void block(const uint16_t* sK, int kt, int Nk, const u32x4* qf, float c,
                                 float& m, float& l, int l32, int hh) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            f32x16 acc = scores_T<D>(sK, kb * 32, qf, l32, hh);
            lds_mfma_chain<D / 16, 4>();  // four operand reads ahead (-1.2% at 31,200 tokens)
            if (tail) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kt + kb * 32 + acc_row(r, hh) >= Nk) acc[r] = -INFINITY;
            }
            if (LAZY) {
                const float mc0 = m * c;
                float s0 = -0.0f;  // -0 + y = y: the first add folds away
#pragma unroll
                for (int r = 0; r < 16; ++r) s0 += __builtin_amdgcn_exp2f(fmaf(acc[r], c, -mc0));
                if (s0 <= kLazySum) {
                    l += s0;
                    continue;
                }
            }
            float mx = m;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = vmax(mx, acc[r]);
            const float mc = mx * c;
            float sum = -0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[r], c, -mc));
            l = l * __builtin_amdgcn_exp2f((m - mx) * c) + sum;
            m = mx;
        }
    }
};

template <int D, int NW, bool SPARSE, bool LAZY>
__global__ __launch_bounds__(NW * 64) void fwd_lse_kernel(AttnArgs a) {
    if (SPARSE && *a.idx_err) return;  // the block index failed its check
    constexpr int BN = FwdLse<D>::BN;
    static_assert(!SPARSE || NW == 4, "sparse workgroups cover one 128-query block");
    __shared__ __attribute__((aligned(1024))) uint16_t sK0[BN * D], sK1[BN * D];
    lds_poison(sK0, sK1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    int qblk = blockIdx.x, bh = blockIdx.y;
    if (!SPARSE) xcd_work(qblk, bh);
    const int q0 = qblk * (NW * 32) + wave * 32;
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
    AsyncTile<BN, D, NW * 64> tk;
    tk.init(D, tid);
    tile_pipeline(
        n_iter, masked_tiles<SPARSE, BN>(lst, n_iter, a.Nk),
        [&](auto b, int it) { tk.issue(sel(b, sK0, sK1), Kb + (size_t)tile_at(it) * D); },
        [&](auto b, int it, auto tail) {
            FwdLse<D>::template block<decltype(tail)::value, LAZY>(sel(b, sK0, sK1), tile_at(it),
                                                                   a.Nk, qf, a.c, m, l, l32, hh);
        });
    const float mp = partner_lane(m), lp = partner_lane(l);
    const float mt = fmaxf(m, mp);
    const float lt = l * __builtin_amdgcn_exp2f((m - mt) * a.c) +
                     lp * __builtin_amdgcn_exp2f((mp - mt) * a.c);
    const int q = q0 + l32;
    if (hh == 0 && q < a.Nq) {
        a.lse_out[(size_t)bh * a.Nq + q] = (mt * a.c + log2f(lt)) * kLn2;
        if (a.row_max_out) a.row_max_out[(size_t)bh * a.Nq + q] = mt * a.sm_scale;
    }
}

// ---------------------------------------------------------------------------
// Forward pass 2: O = FQ(P) Vq with P = exp(S - LSE). 4 waves x 32 queries.
// K tiles are loaded in perm32 row order, so lane half hh of a 32-key score
// block holds keys 16 hh .. 16 hh + 15 for its query: one whole P group.
// With F16 (P and V both quantized) the P V product runs on fp16 operands,
// which hold NVFP4 values exactly, and V^T is stored as fp16.
// Exponent offset of the P quantizer and output factor for query q of head
// bh: the normalised P uses lse2 = LSE log2(e) and factor 1; the
// row-max-relative variant (a.row_max set, P quantized) quantizes
// exp(S - m), i.e. uses m2 = m log2(e), and scales O by 1 / l = exp2(m2 - lse2).
template <bool QP>
__device__ __forceinline__ void p_offset(const AttnArgs& a, int64_t bh, int q, float& off,
                                         float& post) {
    const float lse2 = (q < a.Nq) ? a.lse[bh * a.Nq + q] * kLog2e : 0.0f;
    off = lse2;
    post = 1.0f;
    if (QP && a.row_max && q < a.Nq) {
        const float m2 = a.row_max[bh * a.Nq + q] * kLog2e;
        off = m2;
        post = __builtin_amdgcn_exp2f(m2 - lse2);
    }
}

template <int D, bool QP, bool F16>
struct FwdOut {
    static constexpr int BN = 64;
    static_assert(!F16 || QP, "fp16 P operands are NVFP4 values");

    // P (or its quantization) of one 32-key score block as two B operands
    // (k-slot 8 hh + j of operand g is key 16 hh + 8 g + j).
    template <bool tail>
    __device__ static void probs(f32x16 acc, int k0, int Nk, float c, float lse2, int hh,
                                 u32x4* bfr) {
        if (tail) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (k0 + 16 * hh + r >= Nk) acc[r] = -INFINITY;
        }
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = acc[r];
        if (QP) {
            quant_p_group16<F16>(x, c, lse2, bfr);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = __builtin_amdgcn_exp2f(fmaf(x[r], c, -lse2));
#pragma unroll
            for (int g = 0; g < 2; ++g)
                bfr[g] = u32x4{pack_rne(x[8 * g], x[8 * g + 1]), pack_rne(x[8 * g + 2], x[8 * g + 3]),
                               pack_rne(x[8 * g + 4], x[8 * g + 5]),
                               pack_rne(x[8 * g + 6], x[8 * g + 7])};
        }
    }

    // O^T += V^T P^T for key block kb (D / 16 MFMAs, one LDS read each).
    __device__ static void pv(const uint16_t* sV, int kb, const u32x4* bfr, f32x16* o, int l32,
                              int hh) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const u32x4 vf = *(const u32x4*)(sV + toff<BN>(db * 32 + l32, 4 * kb + 2 * hh + g));
                o[db] = F16 ? mfma_f16(vf, bfr[g], o[db]) : mfma(vf, bfr[g], o[db]);
            }
        }
    }

    // Two 32-key blocks, software-pipelined so that the vector work on one
    // block (exp, quantization, packing) is issued between the matrix
    // products of the other:
    //   S0 | S1 + P(S0) | PV0 + P(S1) | PV1.
    template <bool tail>
    __device__ static void block(const uint16_t* sK, const uint16_t* sV, int kt, int Nk,
                                 const u32x4* qf, float c, float lse2, f32x16* o, int l32, int hh) {
        const f32x16 s0 = scores_T<D>(sK, 0, qf, l32, hh);
        lds_mfma_chain<D / 16, 4>();
        const f32x16 s1 = scores_T<D>(sK, 32, qf, l32, hh);
        u32x4 b0[2], b1[2];
        probs<tail>(s0, kt, Nk, c, lse2, hh, b0);
        mfma_valu_chain<D / 16, 4, kValuPerMfma>();
        pv(sV, 0, b0, o, l32, hh);
        probs<tail>(s1, kt + 32, Nk, c, lse2, hh, b1);
        mfma_valu_chain<D / 16, 4, kValuPerMfma>();
        pv(sV, 1, b1, o, l32, hh);
        lds_mfma_chain<D / 16, 4>();
    }
};

template <int D, bool QP, bool F16, int NW, bool SPARSE>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void fwd_out_kernel(AttnArgs a) {
    if (SPARSE && *a.idx_err) return;  // the block index failed its check
    using F = FwdOut<D, QP, F16>;
    constexpr int BN = F::BN;
    static_assert(!SPARSE || NW == 4, "sparse workgroups cover one 128-query block");
    struct Buf {
        uint16_t k[BN * D];
        uint16_t v[D * BN];
    };
    __shared__ __attribute__((aligned(1024))) Buf s0, s1;
    lds_poison(s0, s1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    int qblk = blockIdx.x, bh = blockIdx.y;
    if (!SPARSE) xcd_work(qblk, bh);
    const int q0 = qblk * (NW * 32) + wave * 32;
    const int q = q0 + l32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
    const uint16_t* Vtb = a.Vt + (size_t)bh * D * a.Nk_pad;
    u32x4 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = *(const u32x4*)(Qb + (size_t)(q0 + l32) * D + c * 16 + hh * 8);
    float lse2, post;
    p_offset<QP>(a, bh, q, lse2, post);
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    __shared__ int lst[SPARSE ? kMaxBlockList : 1];
    if (SPARSE) stage_list(lst, a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk, a.topk);
    const int n_iter = SPARSE ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return tile_start<SPARSE, BN>(lst, it); };
    AsyncTile<BN, D, NW * 64, true> tk;
    AsyncTile<D, BN, NW * 64> tv;
    tk.init(D, tid);
    tv.init(a.Nk_pad, tid);
    tile_pipeline(
        n_iter, masked_tiles<SPARSE, BN>(lst, n_iter, a.Nk),
        [&](auto b, int it) {
            const int kt = tile_at(it);
            tk.issue(sel(b, &s0, &s1)->k, Kb + (size_t)kt * D);
            tv.issue(sel(b, &s0, &s1)->v, Vtb + kt);
        },
        [&](auto b, int it, auto tail) {
            F::template block<decltype(tail)::value>(sel(b, &s0, &s1)->k, sel(b, &s0, &s1)->v,
                                                     tile_at(it), a.Nk, qf, a.c, lse2, o, l32, hh);
        });
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.o + b * a.osb + h * a.osh + (int64_t)q * a.osn, o, post, hh);
    }
}

// ---------------------------------------------------------------------------
// Forward pass 2 with the additive straight-through output: besides
// O = Pq Vq it forms O_ste = P Vq with the unquantized P, whose row sums
// against dO are the backward delta of the pure straight-through reading
// (the caller passes O_ste as the backward's o). One wave per 32 queries as in
// fwd_out_kernel; each V^T operand read feeds both products. P V runs on bf16
// operands here (P is not an NVFP4 value).
template <int D, bool QP>
struct FwdOutSte {
    static constexpr int BN = 64;
    // Pq and P of one 32-key score block, each as two B operands
    template <bool tail>
    __device__ __forceinline__ static void probs(f32x16 acc, int k0, int Nk, float c, float off, int hh, u32x4* bq,
                                 u32x4* bp) {
        float x[16], r[16], sp = 1.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            x[j] = acc[j];
            if (tail && k0 + 16 * hh + j >= Nk) x[j] = -INFINITY;
        }
        if (QP) {
            quant_p_group16_bwd(x, c, off, bq, r, sp);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) r[j] = __builtin_amdgcn_exp2f(fmaf(x[j], c, -off));
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const float* e = r + 8 * g;
            bp[g] = u32x4{pack_rne(e[0] * sp, e[1] * sp), pack_rne(e[2] * sp, e[3] * sp),
                          pack_rne(e[4] * sp, e[5] * sp), pack_rne(e[6] * sp, e[7] * sp)};
            if (!QP) bq[g] = bp[g];
        }
    }
    __device__ __forceinline__ static void pv2(const uint16_t* sV, int kb, const u32x4* bq, const u32x4* bp,
                               f32x16* o, f32x16* os, int l32, int hh) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const u32x4 vf = *(const u32x4*)(sV + toff<BN>(db * 32 + l32, 4 * kb + 2 * hh + g));
                o[db] = mfma(vf, bq[g], o[db]);
                if (QP) os[db] = mfma(vf, bp[g], os[db]);
            }
        }
    }
    // one 32-key block at a time: two output accumulators leave no room for
    // the two-block software pipeline of FwdOut
    template <bool tail>
    __device__ __forceinline__ static void block(const uint16_t* sK, const uint16_t* sV, int kt,
                                                 int Nk, const u32x4* qf, float c, float off,
                                                 f32x16* o, f32x16* os, int l32, int hh) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            const f32x16 sc = scores_T<D>(sK, kb * 32, qf, l32, hh);
            u32x4 bq[2], bp[2];
            probs<tail>(sc, kt + kb * 32, Nk, c, off, hh, bq, bp);
            pv2(sV, kb, bq, bp, o, os, l32, hh);
        }
    }
};

template <int D, bool QP, int NW, bool SPARSE>
__global__ __launch_bounds__(NW * 64) void fwd_out_ste_kernel(AttnArgs a) {
    if (SPARSE && *a.idx_err) return;  // the block index failed its check
    using F = FwdOutSte<D, QP>;
    constexpr int BN = F::BN;
    static_assert(!SPARSE || NW == 4, "sparse workgroups cover one 128-query block");
    struct Buf {
        uint16_t k[BN * D];
        uint16_t v[D * BN];
    };
    __shared__ __attribute__((aligned(1024))) Buf s0, s1;
    lds_poison(s0, s1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    int qblk = blockIdx.x, bh = blockIdx.y;
    if (!SPARSE) xcd_work(qblk, bh);
    const int q0 = qblk * (NW * 32) + wave * 32;
    const int q = q0 + l32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
    const uint16_t* Vtb = a.Vt + (size_t)bh * D * a.Nk_pad;
    u32x4 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = *(const u32x4*)(Qb + (size_t)(q0 + l32) * D + c * 16 + hh * 8);
    float off, post;
    p_offset<QP>(a, bh, q, off, post);
    f32x16 o[D / 32], os[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = os[db] = f32x16{};
    __shared__ int lst[SPARSE ? kMaxBlockList : 1];
    if (SPARSE) stage_list(lst, a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk, a.topk);
    const int n_iter = SPARSE ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return tile_start<SPARSE, BN>(lst, it); };
    AsyncTile<BN, D, NW * 64, true> tk;
    AsyncTile<D, BN, NW * 64> tv;
    tk.init(D, tid);
    tv.init(a.Nk_pad, tid);
    tile_pipeline(
        n_iter, masked_tiles<SPARSE, BN>(lst, n_iter, a.Nk),
        [&](auto b, int it) {
            const int kt = tile_at(it);
            tk.issue(sel(b, &s0, &s1)->k, Kb + (size_t)kt * D);
            tv.issue(sel(b, &s0, &s1)->v, Vtb + kt);
        },
        [&](auto b, int it, auto tail) {
            F::template block<decltype(tail)::value>(sel(b, &s0, &s1)->k, sel(b, &s0, &s1)->v,
                                                     tile_at(it), a.Nk, qf, a.c, off, o, os, l32,
                                                     hh);
        });
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H, at = b * a.osb + h * a.osh + (int64_t)q * a.osn;
        store_rows_T<D>(a.o + at, o, post, hh);
        // without P quantization Pq = P and the two outputs are the same
        store_rows_T<D>(a.o_ste + at, QP ? os : o, post, hh);
    }
}

// ---------------------------------------------------------------------------
// Single-pass forward for problems whose P is not quantized. Without a P
// quantizer nothing needs the final LSE before P V, so O, LSE and the row
// maxima come from one sweep over the keys with an online softmax. The running
// maximum m (shared by the two lanes of a query row) moves only when a block's
// maximum exceeds it by more than 2^kLazyLog2 in P. Then P = 2^((S - m) c)
// stays below 2^kLazyLog2, the fp32 sums keep their full relative precision,
// and the O accumulators are rescaled only on the rare blocks that move m.
// Tiles and operand layouts are those of the straight-through forward: waves
// of 32 queries, K in perm32 order, V^T in token order.
constexpr float kLazyLog2 = 8.0f;
template <int D, int NW, bool SPARSE>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void fwd_single_kernel(AttnArgs a) {
    if (SPARSE && *a.idx_err) return;  // the block index failed its check
    using F = FwdOutSte<D, false>;
    constexpr int BN = F::BN;
    static_assert(!SPARSE || NW == 4, "sparse workgroups cover one 128-query block");
    struct Buf {
        uint16_t k[BN * D];
        uint16_t v[D * BN];
    };
    __shared__ __attribute__((aligned(1024))) Buf s0, s1;
    lds_poison(s0, s1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    int qblk = blockIdx.x, bh = blockIdx.y;
    if (!SPARSE) xcd_work(qblk, bh);
    const int q0 = qblk * (NW * 32) + wave * 32;
    const int q = q0 + l32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
    const uint16_t* Vtb = a.Vt + (size_t)bh * D * a.Nk_pad;
    u32x4 qf[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qf[c] = *(const u32x4*)(Qb + (size_t)(q0 + l32) * D + c * 16 + hh * 8);
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m = -INFINITY, mt = -INFINITY, l = 0.0f;
    const float tau = kLazyLog2 / a.c;  // the lazy threshold in units of raw scores
    __shared__ int lst[SPARSE ? kMaxBlockList : 1];
    if (SPARSE) stage_list(lst, a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk, a.topk);
    const int n_iter = SPARSE ? a.topk * 2 : (a.Nk + BN - 1) / BN;
    auto tile_at = [&](int it) { return tile_start<SPARSE, BN>(lst, it); };
    AsyncTile<BN, D, NW * 64, true> tk;
    AsyncTile<D, BN, NW * 64> tv;
    tk.init(D, tid);
    tv.init(a.Nk_pad, tid);
    tile_pipeline(
        n_iter, masked_tiles<SPARSE, BN>(lst, n_iter, a.Nk),
        [&](auto b, int it) {
            const int kt = tile_at(it);
            tk.issue(sel(b, &s0, &s1)->k, Kb + (size_t)kt * D);
            tv.issue(sel(b, &s0, &s1)->v, Vtb + kt);
        },
        [&](auto b, int it, auto tail) {
            constexpr bool TL = decltype(tail)::value;
            const uint16_t* K = sel(b, &s0, &s1)->k;
            const uint16_t* V = sel(b, &s0, &s1)->v;
            const int kt = tile_at(it);
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                const f32x16 sc = scores_T<D>(K, kb * 32, qf, l32, hh);
                float x[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    x[j] = sc[j];
                    if (TL && kt + kb * 32 + 16 * hh + j >= a.Nk) x[j] = -INFINITY;
                }
                float bm = x[0];
#pragma unroll
                for (int j = 1; j < 16; ++j) bm = vmax(bm, x[j]);
                bm = fmaxf(bm, partner_lane(bm));
                mt = fmaxf(mt, bm);
                const bool up = bm > m + tau;
                if (__any(up)) {
                    const float mn = up ? bm : m;
                    const float al = __builtin_amdgcn_exp2f((m - mn) * a.c);
                    l *= al;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[db][r] *= al;
                    m = mn;
                }
                const float mc = m * a.c;
                float r[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    r[j] = __builtin_amdgcn_exp2f(fmaf(x[j], a.c, -mc));
                    l += r[j];
                }
                u32x4 bp[2];
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    bp[g] = u32x4{pack_rne(r[8 * g], r[8 * g + 1]), pack_rne(r[8 * g + 2], r[8 * g + 3]),
                                  pack_rne(r[8 * g + 4], r[8 * g + 5]), pack_rne(r[8 * g + 6], r[8 * g + 7])};
                F::pv2(V, kb, bp, bp, o, o, l32, hh);
            }
        });
    const float lt = l + partner_lane(l);
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H, at = b * a.osb + h * a.osh + (int64_t)q * a.osn;
        store_rows_T<D>(a.o + at, o, 1.0f / lt, hh);
        // without P quantization the straight-through output is O itself
        if (a.o_ste) store_rows_T<D>(a.o_ste + at, o, 1.0f / lt, hh);
        if (hh == 0) {
            a.lse_out[(size_t)bh * a.Nq + q] = (m * a.c + log2f(lt)) * kLn2;
            if (a.row_max_out) a.row_max_out[(size_t)bh * a.Nq + q] = mt * a.sm_scale;
        }
    }
}

// ---------------------------------------------------------------------------
// Backward dQ: NW waves x 32 QB queries, loop over 64-key tiles. A wave
// keeps the Q and dO B operands of its QB 32-query blocks in registers; each
// K, V or K^T operand read from LDS feeds QB products.
template <int D, int QB>
struct BwdDq {
    static constexpr int BN = 64;

    // S^T and dP^T of 32-key block kb for the wave's query blocks.
    __device__ static void sdp(const uint16_t* sK, const uint16_t* sV, int kb, const u32x4 (*qf)[D / 16],
                               const u32x4 (*df)[D / 16], f32x16* s, f32x16* dp, int l32, int hh) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb] = dp[qb] = f32x16{};
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
            const int row = kb * 32 + l32;
            const u32x4 ka = *(const u32x4*)(sK + toff<D>(row, 2 * cc + hh));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb] = mfma(ka, qf[qb][cc], s[qb]);
            const u32x4 va = *(const u32x4*)(sV + toff<D>(row, 2 * cc + hh));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) dp[qb] = mfma(va, df[qb][cc], dp[qb]);
        }
    }

    // dS = P (dP - Dl) of one block as two bf16 B operands.
    template <bool tail>
    __device__ static void dsop(const f32x16& s, const f32x16& dp, int k0, int Nk, float c,
                                float lse2, float dl, int hh, u32x4* bfr) {
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
            if (tail && k0 + acc_row(r, hh) >= Nk) p = 0.0f;
            ds[r] = p * (dp[r] - dl);
        }
#pragma unroll
        for (int g = 0; g < 2; ++g)
            bfr[g] = u32x4{pack_rne(ds[8 * g + 0], ds[8 * g + 1]), pack_rne(ds[8 * g + 2], ds[8 * g + 3]),
                           pack_rne(ds[8 * g + 4], ds[8 * g + 5]), pack_rne(ds[8 * g + 6], ds[8 * g + 7])};
    }

    // dQ^T += Kt dS^T for block kb.
    __device__ static void dq(const uint16_t* sKt, int kb, const u32x4 (*bfr)[2], f32x16 (*dqa)[D / 32],
                              int l32, int hh) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const u32x4 ktf = *(const u32x4*)(sKt + toff<BN>(db * 32 + l32, 4 * kb + 2 * g + hh));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) dqa[qb][db] = mfma(ktf, bfr[qb][g], dqa[qb][db]);
            }
        }
    }

    // Two 32-key blocks, software-pipelined so that the vector work of one
    // (exp, dS, packing) is issued between the matrix products of the other:
    //   S/dP 0 | S/dP 1 + dS 0 | dQ 0 + dS 1 | dQ 1.
    template <bool tail>
    __device__ static void block(const uint16_t* sK, const uint16_t* sV, const uint16_t* sKt,
                                 int kt, int Nk, const u32x4 (*qf)[D / 16], const u32x4 (*df)[D / 16],
                                 float c, const float* lse2, const float* dl, f32x16 (*dqa)[D / 32],
                                 int l32, int hh) {
        f32x16 s0[QB], dp0[QB], s1[QB], dp1[QB];
        u32x4 b0[QB][2], b1[QB][2];
        sdp(sK, sV, 0, qf, df, s0, dp0, l32, hh);
        mfma_chain_m<QB * D / 8, QB, 4, 0>();
        sdp(sK, sV, 1, qf, df, s1, dp1, l32, hh);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) dsop<tail>(s0[qb], dp0[qb], kt, Nk, c, lse2[qb], dl[qb], hh, b0[qb]);
        mfma_chain_m<QB * D / 8, QB, 4, 5 / QB>();
        dq(sKt, 0, b0, dqa, l32, hh);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            dsop<tail>(s1[qb], dp1[qb], kt + 32, Nk, c, lse2[qb], dl[qb], hh, b1[qb]);
        mfma_chain_m<QB * D / 16, QB, 4, kValuPerMfma>();
        dq(sKt, 1, b1, dqa, l32, hh);
        mfma_chain_m<QB * D / 16, QB, 4, 0>();
    }
};

template <int D, int NW, int QB, bool SPARSE>
__global__ __launch_bounds__(NW * 64) void bwd_dq_kernel(AttnArgs a) {
    if (SPARSE && *a.idx_err) return;  // the block index failed its check
    using DQ = BwdDq<D, QB>;
    constexpr int BN = DQ::BN, NT = NW * 64;
    struct Buf {
        uint16_t k[BN * D];
        uint16_t v[BN * D];
        uint16_t kt[D * BN];
    };
    __shared__ __attribute__((aligned(1024))) Buf s0, s1;
    lds_poison(s0, s1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    constexpr int QW = NW * 32 * QB;  // queries per workgroup
    // sparse launches use NW = 4, QB = 1 so that a workgroup is one 128-query block
    static_assert(!SPARSE || (NW == 4 && QB == 1), "sparse dQ workgroups cover one query block");
    __shared__ int lst[SPARSE ? kMaxBlockList : 1];
    AsyncTile<BN, D, NT> tk;
    AsyncTile<D, BN, NT> tt;
    tk.init(D, tid);
    tt.init(a.Nk_pad, tid);
    // one query block qblk of head bh over key tiles [t0, t1); slot >= 0:
    // fp32 partial sums to that slot instead of dQ
    auto segment = [&](int qblk, int bh, int t0, int t1, int slot) {
        const int q0 = qblk * QW + wave * 32 * QB;
        const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
        const uint16_t* dOb = a.dOw + (size_t)bh * a.Nq_pad * D;
        const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
        const uint16_t* Vb = a.Vw + (size_t)bh * a.Nk_pad * D;
        const uint16_t* Ktb = a.Kt + (size_t)bh * D * a.Nk_pad;
        u32x4 qf[QB][D / 16], df[QB][D / 16];
        float lse2[QB], dl[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int q = q0 + qb * 32 + l32;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                qf[qb][c] = *(const u32x4*)(Qb + (size_t)q * D + c * 16 + hh * 8);
                df[qb][c] = *(const u32x4*)(dOb + (size_t)q * D + c * 16 + hh * 8);
            }
            lse2[qb] = a.lse2[(size_t)bh * a.Nq_pad + q];
            dl[qb] = a.delta[(size_t)bh * a.Nq_pad + q];
        }
        f32x16 dqa[QB][D / 32];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int db = 0; db < D / 32; ++db) dqa[qb][db] = f32x16{};
        if (SPARSE) stage_list(lst, a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk, a.topk);
        const int n_iter = t1 - t0;
        auto tile_at = [&](int it) { return tile_start<SPARSE, BN>(lst, t0 + it); };
        // dense: only a range that ends with the last key tile holds keys >= Nk
        const int n_masked = SPARSE ? masked_tiles<SPARSE, BN>(lst, n_iter, a.Nk)
                                    : (n_iter > 0 && t1 * BN > a.Nk ? 1 : 0);
        tile_pipeline(
            n_iter, n_masked,
            [&](auto b, int it) {
                const int kt = tile_at(it);
                Buf* t = sel(b, &s0, &s1);
                tk.issue(t->k, Kb + (size_t)kt * D);
                tk.issue(t->v, Vb + (size_t)kt * D);
                tt.issue(t->kt, Ktb + kt);
            },
            [&](auto b, int it, auto tail) {
                Buf* t = sel(b, &s0, &s1);
                DQ::template block<decltype(tail)::value>(t->k, t->v, t->kt, tile_at(it), a.Nk, qf,
                                                          df, a.c, lse2, dl, dqa, l32, hh);
            });
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int q = q0 + qb * 32 + l32;
            if (slot >= 0) {
                store_rows_f32<D>(a.dq_part + ((size_t)slot * QW + (q - qblk * QW)) * D, dqa[qb], hh);
            } else if (q < a.Nq) {
                const int64_t b = bh / a.H, h = bh % a.H;
                store_rows_T<D>(a.dq + b * a.dqsb + h * a.dqsh + (int64_t)q * a.dqsn, dqa[qb],
                                a.sm_scale, hh);
            }
        }
    };
    if (SPARSE) {
        segment(blockIdx.x, blockIdx.y, 0, a.topk * 2, -1);
        return;
    }
    // dense: whole query blocks, or up to two segments of the last round
    // (work_segments); the fixup adds the partial sums
    static_assert(SPARSE || QW == 256, "dense dQ partial slots hold 256 queries");
    const int nqb = (a.Nq + QW - 1) / QW, nt = (a.Nk + BN - 1) / BN;
    Seg sg[2];
    const int ns = work_segments(a.dq_full, a.BH * nqb, nt, a.dq_chunk, sg);
    segment(sg[0].blk % nqb, sg[0].blk / nqb, sg[0].t0, sg[0].t1, sg[0].slot);
    if (ns > 1) {
        __syncthreads();  // every wave is done with the tile buffers
        segment(sg[1].blk % nqb, sg[1].blk / nqb, sg[1].t0, sg[1].t1, sg[1].slot);
    }
}

// Sums the partial sums of every last-round query block of a dense dQ
// launch that splits its last round (in chunk order) and writes the block's
// dQ (times sm_scale) as bf16. One workgroup per block.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_fixup_kernel(AttnArgs a) {
    constexpr int QW = 256;
    const int j = blockIdx.x, w = a.dq_full + j;
    const int nqb = (a.Nq + QW - 1) / QW, nt = (a.Nk + 63) / 64;
    const int bh = w / nqb, qblk = w % nqb;
    const int64_t b = bh / a.H, h = bh % a.H;
    // 8 consecutive d values per thread and pass
    for (int e = threadIdx.x * 8; e < QW * D; e += 256 * 8) {
        const int q = qblk * QW + e / D, d = e % D;
        if (q >= a.Nq) continue;
        f32x4_t x0, x1;
        sum_slots<D>(a.dq_part, j, nt, a.dq_chunk, e, x0, x1);
        const float f = a.sm_scale;
        u32x4 v;
        v[0] = pack_rne(x0[0] * f, x0[1] * f);
        v[1] = pack_rne(x0[2] * f, x0[3] * f);
        v[2] = pack_rne(x1[0] * f, x1[1] * f);
        v[3] = pack_rne(x1[2] * f, x1[3] * f);
        *(u32x4*)(a.dq + b * a.dqsb + h * a.dqsh + (int64_t)q * a.dqsn + d) = v;
    }
}

// ---------------------------------------------------------------------------
// Backward dQ, block-sparse: one 128-query block (4 waves of 32 queries) per
// workgroup, over the 64-key tiles of its selected key blocks. K tiles are
// kept in the natural layout (nswz) and the dQ product reads its K^T operands
// from them with transposing reads, so no K^T tile is staged: 32 KB per tile
// stage. The launch bound holds the kernel to 256 registers per lane (at
// d = 128 a few values spill), so that two workgroups (two waves per SIMD)
// share a CU.
// K^T operand of dQ^T += K^T dS^T for d-block db and key group g of a 32-key
// block: lane (hh, r) holds d = 32 db + r of keys 16 g + 4 hh + 0..3 and
// 16 g + 8 + 4 hh + 0..3, the accumulator-row order of the dS operand; two
// transposing reads of 4 consecutive key rows each (t = 0, 1).
template <int D>
__device__ __forceinline__ int ktr_lane(int db, int t, int lane) {
    const int G = lane >> 4, i = lane & 15;
    const int hh = G >> 1, j = i >> 2, q = i & 3;
    const int d = 32 * db + 16 * (G & 1) + 4 * q;
    return noff<D>(8 * t + 4 * hh + j, d >> 3) + (d & 7);
}

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_sparse_kernel(AttnArgs a) {
    if (*a.idx_err) return;  // the block index failed its check
    using DQ = BwdDq<D, 1>;
    constexpr int BN = 64, NT = 256, NW = 4;
    struct Buf {
        uint16_t k[BN * D];  // natural layout (nswz)
        uint16_t v[BN * D];  // toff<D>
    };
    __shared__ __attribute__((aligned(1024))) Buf s0, s1;
    lds_poison(s0, s1);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int bh = blockIdx.y, qblk = blockIdx.x;
    const int q = qblk * 128 + wave * 32 + l32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* dOb = a.dOw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
    const uint16_t* Vb = a.Vw + (size_t)bh * a.Nk_pad * D;
    u32x4 qf[1][D / 16], df[1][D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        qf[0][c] = *(const u32x4*)(Qb + (size_t)q * D + c * 16 + hh * 8);
        df[0][c] = *(const u32x4*)(dOb + (size_t)q * D + c * 16 + hh * 8);
    }
    const float lse2[1] = {a.lse2[(size_t)bh * a.Nq_pad + q]};
    const float dl[1] = {a.delta[(size_t)bh * a.Nq_pad + q]};
    f32x16 dqa[1][D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqa[0][db] = f32x16{};
    // the block list is read from global memory (uniform loads): staging it
    // in LDS would push the workgroup past the 64 KB that lets two share a CU
    const int32_t* lst = a.kv_idx + ((size_t)bh * a.nbq + qblk) * a.topk;
    const int n_iter = a.topk * 2;
    auto tile_at = [&](int it) { return lst[it >> 1] * 128 + (it & 1) * BN; };
    // K tile copies: 1 KB blocks b = j NW + wave hold RB rows of CR chunks;
    // lane i fills slot 16 i with logical chunk (i % CR) ^ nswz(row)
    constexpr int CR = D / 8, RB = 64 / CR, NKB = BN * D * 2 / 1024 / NW;
    uint32_t koff[NKB];
#pragma unroll
    for (int j = 0; j < NKB; ++j) {
        const int row = (j * NW + wave) * RB + lane / CR;
        koff[j] = (uint32_t)(row * D + (((lane % CR) ^ nswz<D>(row)) << 3)) * 2u;
    }
    AsyncTile<BN, D, NT> tv;
    tv.init(D, tid);
    int lo[D / 32][2];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int t = 0; t < 2; ++t) lo[db][t] = ktr_lane<D>(db, t, lane);
    // S^T and dP^T of 32-key block kb (K rows read from the natural tile)
    auto sdp = [&](const uint16_t* sK, const uint16_t* sV, int kb, f32x16& s, f32x16& dp) {
        s = dp = f32x16{};
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
            const int row = kb * 32 + l32;
            const u32x4 ka = *(const u32x4*)(sK + noff<D>(row, 2 * cc + hh));
            s = mfma(ka, qf[0][cc], s);
            const u32x4 va = *(const u32x4*)(sV + toff<D>(row, 2 * cc + hh));
            dp = mfma(va, df[0][cc], dp);
        }
    };
    // dQ^T += K^T dS^T of block kb, K^T operands by transposing reads
    auto dqp = [&](const uint16_t* sK, int kb, const u32x4* bfr) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const uint16_t* base = sK + (32 * kb + 16 * g) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const u32x2 r0 = lds_read_tr16(base + lo[db][0]);
                const u32x2 r1 = lds_read_tr16(base + lo[db][1]);
                dqa[0][db] = mfma(u32x4{r0[0], r0[1], r1[0], r1[1]}, bfr[g], dqa[0][db]);
            }
        }
    };
    tile_pipeline(
        n_iter, masked_tiles<true, BN>(lst, n_iter, a.Nk),
        [&](auto b, int it) {
            const int kt = tile_at(it);
            Buf* t = sel(b, &s0, &s1);
#pragma unroll
            for (int j = 0; j < NKB; ++j)
                dma16(lds_addr(t->k + (j * NW + wave) * 512), Kb + (size_t)kt * D, koff[j]);
            tv.issue(t->v, Vb + (size_t)kt * D);
        },
        [&](auto b, int it, auto tail) {
            constexpr bool TL = decltype(tail)::value;
            const Buf* t = sel(b, &s0, &s1);
            const int kt = tile_at(it);
            // S/dP 0 | S/dP 1 + dS 0 | dQ 0 + dS 1 | dQ 1
            f32x16 s0_, dp0, s1_, dp1;
            u32x4 b0[1][2], b1[1][2];
            sdp(t->k, t->v, 0, s0_, dp0);
            mfma_chain_m<D / 8, 1, 4, 0>();
            sdp(t->k, t->v, 1, s1_, dp1);
            DQ::template dsop<TL>(s0_, dp0, kt, a.Nk, a.c, lse2[0], dl[0], hh, b0[0]);
            mfma_chain_m<D / 8, 1, 4, 5>();
            dqp(t->k, 0, b0[0]);
            DQ::template dsop<TL>(s1_, dp1, kt + 32, a.Nk, a.c, lse2[0], dl[0], hh, b1[0]);
            __builtin_amdgcn_sched_barrier(0);
            dqp(t->k, 1, b1[0]);
            __builtin_amdgcn_sched_barrier(0);
        });
    if (q < a.Nq) {
        const int64_t b = bh / a.H, h = bh % a.H;
        store_rows_T<D>(a.dq + b * a.dqsb + h * a.dqsh + (int64_t)q * a.dqsn, dqa[0], a.sm_scale, hh);
    }
}

// ---------------------------------------------------------------------------
// Backward helpers. Scores are computed with keys on the accumulator rows
// (S^T = K Q^T, perm32 key order: lane half hh holds keys 16 hh + r), the
// layout in which P's 16-key groups are quantized, so P, Pq and dS have
// queries on lanes; a per-wave LDS transpose turns them into B operands with
// queries as the contraction index of dV^T = dO^T Pq and dK^T = Q^T dS.
//
// Transpose of a 32 x 32 score tile packed as bf16 pairs (w[g] holds keys
// 16 hh + 8 g .. + 7 of query l32) through LDS: transpose_write stores it
// with row = query (64 bytes per row, two 16-byte writes per lane; 16-byte
// chunk c of row q sits at c ^ (((q >> 1) ^ (q >> 3)) & 3)); transpose_read
// returns two B operands with keys on lanes and queries 16 g + 8 hh + j on the
// k-slots. The swizzle keeps both sides free of bank conflicts: 16-byte
// writes go through the banks eight lanes (128 bytes) at a time, and the rows
// of eight consecutive queries, 64 bytes apart, then fall on eight different
// 16-byte bank groups; the transposing reads (32 lanes, 256 bytes at a time)
// touch 32 different 8-byte bank pairs. (Measured with the access patterns in
// isolation: the earlier swizzle c ^ ((q >> 2) & 3) left the writes 2-way
// conflicted.)
__device__ __forceinline__ int xoff(int q, int c) { return q * 32 + ((c ^ (((q >> 1) ^ (q >> 3)) & 3)) << 3); }
__device__ __forceinline__ void transpose_write(const u32x4* w, uint16_t* T, int lane) {
    const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int g = 0; g < 2; ++g) *(u32x4*)(T + xoff(l32, 2 * hh + g)) = w[g];
}
__device__ __forceinline__ void transpose_read(const uint16_t* T, u32x4* out, int lane) {
    const int hh = lane >> 5, G = lane >> 4, i16 = lane & 15;
    const int j = i16 >> 2, q = i16 & 3;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // lane 4 j + q of the group reads query j of these 4 and keys
            // 16 (G % 2) + 4 q .. + 3; every lane receives its key's column
            const int row = 16 * g + 8 * hh + 4 * t + j;
            const u32x2 r = lds_read_tr16(T + xoff(row, 2 * (G & 1) + (q >> 1)) + 4 * (q & 1));
            out[g][2 * t] = r[0];
            out[g][2 * t + 1] = r[1];
        }
    }
}

// Per-lane K (and V) A-operand fragments of this wave's 32 keys (row l32 of
// the score tile holds key k0 + perm32(l32) with PERM32).
template <int D, bool PERM32 = false>
__device__ __forceinline__ void load_key_frags(const uint16_t* X, int bh, int Nk_pad, int k0, int l32,
                                               int hh, u32x4* f) {
    const int row = k0 + (PERM32 ? perm32(l32) : l32);
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        f[c] = *(const u32x4*)(X + ((size_t)bh * Nk_pad + row) * D + c * 16 + hh * 8);
}

// Query-tile visiting order of a key workgroup: every 64-query tile (dense) or
// the tiles of the query blocks that selected this key block (sparse, staged).
template <bool SPARSE>
__device__ __forceinline__ int query_tiles(const AttnArgs& a, int bh, int kblk, int* lst) {
    if (!SPARSE) return (a.Nq + 63) / 64;
    const int cnt = a.q_count[(size_t)bh * a.nbk + kblk];
    stage_list(lst, a.q_list + ((size_t)bh * a.nbk + kblk) * a.nbq, cnt);
    return 2 * cnt;
}

// ---------------------------------------------------------------------------
// Backward dK and dV in one kernel. A workgroup owns 128 keys and runs 8
// waves, two per SIMD: producer wave w (waves 0..3) and consumer wave w + 4
// share the same 32 keys (perm32 order, so that a lane's score registers
// hold one whole P group) and the same SIMD.
//   producer: S^T = K Q^T and dP^T = V dO^T (K and V fragments in
//             registers); P = exp(S - LSE), Pq = FQ(P), dS = P (dP - Dl);
//             Pq and dS written transposed (bf16) to an LDS exchange slot
//   consumer: dV^T += dO^T Pq and dK^T += Q^T dS, B operands read from the
//             exchange slot (dV^T and dK^T in registers)
// Each role issues 16 of the 32 products per 32-query sub-block; the
// producer also carries all the vector work, which the hardware overlaps
// with the consumer's products on the shared SIMD. S is computed once.
//
// Query tiles are staged in natural layout (Qq and dO rows, swizzled) with
// the row statistics. The producer reads its B operands with plain 16-byte
// reads, all issued before its first product; the consumer reads its A
// operands (columns of Qq and dO) with transposing reads at the end of the
// previous step, while it waits at the barrier, so that the slower
// transposing reads stay off the producer's path. Tiles live in a ring of
// three buffers. The producer runs one 32-query sub-block ahead of the consumer:
// step u computes sub-block u in the producer and sub-block u - 1 in the
// consumer, through a double-buffered exchange with a single barrier per
// step. Tile t is read in steps 2t .. 2t + 2; its buffer is refilled with
// tile t + 3 right after step 2t + 2, three steps before use. The tile loads
// are LDS-DMA instructions issued in inline assembly, which keeps them out of
// the compiler's wait-count tracking: the kernel waits for them itself, and
// only where a tile is first needed.
template <int D>
struct KVTile {
    static constexpr int BM = 64;
    uint16_t q[BM * D];  // Qq rows, natural layout (noff)
    uint16_t o[BM * D];  // dO rows, natural layout (noff)
    float st[2 * BM];    // LSE * log2(e) for the BM queries, then Dl
};


// B operand of S^T = K Q^T (or dP^T = V dO^T) for d-chunk cc of 32-query
// sub-block sb: lane (hh, c) holds d = 16 cc + 8 hh .. + 7 of query 32 sb + c.
template <int D>
__device__ __forceinline__ u32x4 bop_nat(const uint16_t* t, int sb, int cc, int l32, int hh) {
    return *(const u32x4*)(t + noff<D>(sb * 32 + l32, 2 * cc + hh));
}

// A operand of X^T += A^T B (rows of A^T = d) for d-block db and query group g
// of sub-block sb, read transposed from the natural tile: lane (hh, r) holds
// d = 32 db + r of queries 32 sb + 16 g + 8 hh .. + 7. Each transposing read
// covers 4 queries: in a 16-lane group, lane 4 j + q points at query j and
// d columns 4 q .. 4 q + 3, and every lane receives the column of the d equal
// to its index in the group. The swizzle depends on the row only through
// row % 16, so the per-lane part of the address depends on db and on which
// 4 of the 8 queries are read (aop_lane); sb and g add whole rows.
template <int D>
__device__ __forceinline__ int aop_lane(int db, int t, int lane) {
    const int G = lane >> 4, i = lane & 15;
    const int hh = G >> 1, j = i >> 2, q = i & 3;
    const int d = 32 * db + 16 * (G & 1) + 4 * q;
    return noff<D>(8 * hh + 4 * t + j, d >> 3) + (d & 7);
}
template <int D>
__device__ __forceinline__ u32x4 aop_tr(const uint16_t* t, int sb, int g, const int* lo) {
    const uint16_t* b = t + (32 * sb + 16 * g) * D;
    const u32x2 r0 = lds_read_tr16(b + lo[0]);
    const u32x2 r1 = lds_read_tr16(b + lo[1]);
    return u32x4{r0[0], r0[1], r1[0], r1[1]};
}

template <int D, bool QP, bool SPARSE>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(AttnArgs a) {
    if (SPARSE && *a.idx_err) return;  // the block index failed its check
    using Tile = KVTile<D>;
    constexpr int BM = Tile::BM, KW = 128;
    // loads per wave per tile: Qq and dO rows (BM * D * 2 bytes each, in 1 KB
    // DMA blocks over 8 waves) and one 64-byte slice of the statistics
    constexpr int NJ = 2 * D * BM * 2 / 1024 / 8;
    constexpr int NL = NJ + 1;
    static_assert(2 * D * BM * 2 % 8192 == 0, "tile splits into whole DMA blocks per wave");
    __shared__ __attribute__((aligned(1024))) Tile ring[3];
    // exchange slots per step parity and wave pair: transposed Pq, then dS
    __shared__ __attribute__((aligned(1024))) uint16_t sX[2][4][2 * 32 * 32];
    lds_poison(ring, sX);
    __shared__ int lst[SPARSE ? kMaxBlockList : 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave & 3;
    const bool producer = wave < 4;  // wave-uniform
    const int l32 = lane & 31, hh = lane >> 5;
    // Dense launches: the first a.dkdv_full workgroups take one whole key
    // block each (kb = bh * nbk + kblk, head-major; each XCD a contiguous
    // range); the remaining key blocks are split into a.dkdv_parts parts along
    // the queries, one workgroup per part, written as fp32 partial sums that
    // bwd_dkdv_fixup_kernel adds. The split makes the last round of
    // workgroups as full as possible (the host picks the part count). Sparse
    // launches: one key block per workgroup, the blocks of every head
    // heaviest first (blockIdx.y is the rank of the block's selection count).
    int kblk, bh, t0 = 0, n, side = -1;
    if (SPARSE) {
        bh = blockIdx.x;
        kblk = a.kv_order[(size_t)bh * a.nbk + blockIdx.y];
        n = query_tiles<SPARSE>(a, bh, kblk, lst);
    } else {
        const int nt = (a.Nq + BM - 1) / BM, L = blockIdx.x, nf = a.dkdv_full;
        int kb;
        if (L < nf) {
            kb = xcd_index(L, nf);
            n = nt;
        } else {
            const int w = xcd_index(L - nf, gridDim.x - nf), P = a.dkdv_parts;
            side = w;  // partial slot
            kb = nf + w / P;
            const int part = w % P;
            t0 = nt * part / P;
            n = nt * (part + 1) / P - t0;
        }
        bh = kb / a.nbk;
        kblk = kb % a.nbk;
    }
    const int k0 = kblk * KW + pair * 32;
    const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
    const uint16_t* dOb = a.dOw + (size_t)bh * a.Nq_pad * D;
    // statistics slice of this wave: waves 0..3 LSE2, 4..7 Dl, 16 queries each
    const float* Sb = (wave < 4 ? a.lse2 : a.delta) + (size_t)bh * a.Nq_pad + pair * 16;
    const bool tailk = kblk * KW + KW > a.Nk;
    // Per-lane source offsets of this wave's DMA blocks in a [BM][D] tile:
    // block b = j * 8 + wave covers tile rows RB b .. RB b + RB - 1 (RB rows of
    // CR 16-byte chunks make 1 KB); lane i fills LDS slot 16 i of the block,
    // which holds logical chunk (i % CR) ^ nswz(row) of row RB b + i / CR.
    constexpr int CR = D / 8, RB = 64 / CR;
    uint32_t goff[NJ / 2];
#pragma unroll
    for (int j = 0; j < NJ / 2; ++j) {
        const int row = (j * 8 + wave) * RB + lane / CR;
        goff[j] = (uint32_t)(row * D + (((lane % CR) ^ nswz<D>(row)) << 3)) * 2u;
    }
    auto issue = [&](int t) {
        Tile* T = ring + t % 3;
        const int qt = tile_start<SPARSE, BM>(lst, t0 + t);
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
            const uint32_t blk = (uint32_t)((j * 8 + wave) * 512);  // elements
            dma16(lds_addr(T->q + blk), Qb + (size_t)qt * D, goff[j]);
            dma16(lds_addr(T->o + blk), dOb + (size_t)qt * D, goff[j]);
        }
        if (lane < 16) dma4(lds_addr(T->st + wave * 16), Sb + qt, 4u * (uint32_t)lane);
    };
    // Both roles execute the same barriers (one per step). A key block that
    // no query block selected (sparse) has no steps. With UNROLL the step
    // loop is unrolled by two and body(u, odd) sees the parity of u at
    // compile time (std::bool_constant); otherwise odd is a plain bool.
    auto steps = [&](auto body, auto unroll) {
        if (n == 0) return;
        issue(0);
        if (n > 1) issue(1);
        if (n > 1) wait_vm<NL>();
        else wait_vm<0>();
        auto one = [&](int u, auto odd) {
            // before barrier u (odd u): tile (u + 1) / 2, the newest one
            // issued, must be resident, as the producer reads its first
            // operands during step u; after the barrier tile (u - 1) / 2 + 2
            // refills the buffer freed by step u - 1. The producer's exchange
            // writes must have landed before the barrier; the consumer's
            // operand reads of the next sub-block may still be in flight
            // (their tile is not refilled before they are used), so only the
            // producer waits for its LDS operations here.
            if (odd) wait_vm<0>();
            if (producer) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            if (odd && (u - 1) / 2 + 2 < n) issue((u - 1) / 2 + 2);
            body(u, odd);
        };
        if constexpr (decltype(unroll)::value) {
            for (int u = 0; u <= 2 * n; u += 2) {
                one(u, std::false_type{});
                if (u < 2 * n) one(u + 1, std::true_type{});
            }
        } else {
            for (int u = 0; u <= 2 * n; ++u) one(u, (u & 1) != 0);
        }
    };
    if (producer) {
        u32x4 fk[D / 16], fv[D / 16];
        load_key_frags<D, true>(a.Kw, bh, a.Nk_pad, k0, l32, hh, fk);
        load_key_frags<D, true>(a.Vw, bh, a.Nk_pad, k0, l32, hh, fv);
        // let the fragments land before any tile copy is issued: the copies
        // are invisible to the compiler, whose waits for these loads would
        // otherwise also wait for the copies in flight
        wait_vm<0>();
        // B operands of sub-block v (Qq and dO rows of its 32 queries)
        u32x4 bq[D / 16], bo[D / 16];
        auto fetch = [&](int v) {
            const Tile* T = ring + (v >> 1) % 3;
#pragma unroll
            for (int cc = 0; cc < D / 16; ++cc) {
                bq[cc] = bop_nat<D>(T->q, v & 1, cc, l32, hh);
                bo[cc] = bop_nat<D>(T->o, v & 1, cc, l32, hh);
            }
        };
        // S^T and dP^T of even (A) and odd (B) sub-blocks
        f32x16 sdA, dpA, sdB, dpB;
        auto products = [&](f32x16& sd, f32x16& dp) {
            sd = dp = f32x16{};
#pragma unroll
            for (int cc = 0; cc < D / 16; ++cc) {
                sd = mfma(fk[cc], bq[cc], sd);
                dp = mfma(fv[cc], bo[cc], dp);
            }
        };
        // Step u: the vector work of sub-block u (whose S^T and dP^T are
        // ready) with the products of sub-block u + 1 interleaved, so that
        // this wave's own products fill the matrix unit during its vector
        // work. At u = 2 n - 1 the products read a stale buffer and are
        // discarded. The loop is unrolled by two so that the two score sets
        // alternate without copies.
        auto body = [&](int u, auto odd, auto tail) {
            constexpr bool ODD = decltype(odd)::value;
            constexpr bool TK = decltype(tail)::value;
            if (u >= 2 * n) return;
            f32x16& sd = ODD ? sdB : sdA;
            f32x16& dp = ODD ? dpB : dpA;
            const Tile* T = ring + (u >> 1) % 3;
            constexpr int sb = ODD ? 1 : 0;
            if (!ODD && u == 0) {
                fetch(0);
                products(sd, dp);
            }
            const float L = T->st[sb * 32 + l32], Dl = T->st[BM + sb * 32 + l32];
            __builtin_amdgcn_sched_barrier(0);
            fetch(u + 1);
            float x[16], r[16], sp = 1.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                x[j] = sd[j];
                if (TK && k0 + 16 * hh + j >= a.Nk) x[j] = -INFINITY;
            }
            u32x4 pw[2], dw[2];
            if (QP) {
                quant_p_group16_bwd(x, a.c, L, pw, r, sp);
            } else {
#pragma unroll
                for (int j = 0; j < 16; ++j) r[j] = __builtin_amdgcn_exp2f(fmaf(x[j], a.c, -L));
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    pw[g] = u32x4{pack_rne(r[8 * g], r[8 * g + 1]), pack_rne(r[8 * g + 2], r[8 * g + 3]),
                                  pack_rne(r[8 * g + 4], r[8 * g + 5]),
                                  pack_rne(r[8 * g + 6], r[8 * g + 7])};
            }
            // dS = P (dP - Dl) with P = r s': r (dP s' - Dl s')
            const float sdl = sp * Dl;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                uint32_t w[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int j = 8 * g + 2 * k;
                    w[k] = pack_rne(r[j] * fmaf(dp[j], sp, -sdl), r[j + 1] * fmaf(dp[j + 1], sp, -sdl));
                }
                dw[g] = u32x4{w[0], w[1], w[2], w[3]};
            }
            products(ODD ? sdA : sdB, ODD ? dpA : dpB);
            // issue order: the operand reads, most of the vector work (96
            // instructions) while they land and while the consumer's products
            // of this step hold the matrix unit, then the products with 4
            // vector instructions after each. Front-loading the vector work
            // keeps this wave's products out of the consumer's burst at the
            // start of the step (measured: 5.61 -> 5.34 ms at 6 heads x
            // 31,200 tokens against one product per 8 after 24).
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 16), 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 96, 0);
#pragma unroll
            for (int i = 0; i < 2 * (D / 16); ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            uint16_t* X = sX[sb][pair];
            transpose_write(pw, X, lane);
            transpose_write(dw, X + 32 * 32, lane);
        };
        // keys beyond Nk exist only in the last key workgroup: mask them there
        // only (they would enter the maxima of the last P groups)
        if (tailk) steps([&](int u, auto odd) { body(u, odd, std::true_type{}); }, std::true_type{});
        else steps([&](int u, auto odd) { body(u, odd, std::false_type{}); }, std::true_type{});
    } else {
        f32x16 dva[D / 32], dka[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dva[db] = dka[db] = f32x16{};
        // A operands (dO^T and Q^T rows) of the next sub-block, read at the
        // end of the previous step, while this wave waits for the barrier
        // (the tile is resident: the producer passed a barrier with it)
        u32x4 ao[D / 32][2], aq[D / 32][2];
        int alo[D / 32][2];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int t = 0; t < 2; ++t) alo[db][t] = aop_lane<D>(db, t, lane);
        auto prefetch = [&](int v) {
            const Tile* T = ring + (v >> 1) % 3;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    ao[db][g] = aop_tr<D>(T->o, v & 1, g, alo[db]);
                    aq[db][g] = aop_tr<D>(T->q, v & 1, g, alo[db]);
                }
        };
        steps([&](int u, bool odd) {
            if (u == 0) {
                prefetch(0);
                return;
            }
            const uint16_t* X = sX[odd ? 0 : 1][pair];
            u32x4 pT[2], dT[2];
            transpose_read(X, pT, lane);
            transpose_read(X + 32 * 32, dT, lane);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    dva[db] = mfma(ao[db][g], pT[g], dva[db]);
                    dka[db] = mfma(aq[db][g], dT[g], dka[db]);
                }
            __builtin_amdgcn_sched_barrier(0);
            if (u < 2 * n) prefetch(u);
        }, std::false_type{});
        const int key = k0 + l32;
        if (side >= 0) {
            // fp32 partial sums [dK, dV][128 keys][D] of part slot `side`
            float* ps = a.dkdv_part + (size_t)side * 2 * KW * D;
            store_rows_f32<D>(ps + (size_t)(pair * 32 + l32) * D, dka, hh);
            store_rows_f32<D>(ps + (size_t)(KW + pair * 32 + l32) * D, dva, hh);
        } else if (key < a.Nk) {
            const int64_t b = bh / a.H, h = bh % a.H;
            store_rows_T<D>(a.dv + b * a.dvsb + h * a.dvsh + (int64_t)key * a.dvsn, dva, 1.0f, hh);
            store_rows_T<D>(a.dk + b * a.dksb + h * a.dksh + (int64_t)key * a.dksn, dka, a.sm_scale,
                            hh);
        }
    }
}

// Sums the fp32 parts of every split key block of a dense dK/dV launch (in a
// fixed order, part 0 first) and writes the block's dK (times sm_scale) and
// dV as bf16. One workgroup per split block.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_fixup_kernel(AttnArgs a) {
    constexpr int KW = 128;
    const int P = a.dkdv_parts, kb = a.dkdv_full + blockIdx.x;
    const int bh = kb / a.nbk, kblk = kb % a.nbk;
    const int64_t b = bh / a.H, h = bh % a.H;
    const float* p0 = a.dkdv_part + (size_t)blockIdx.x * P * 2 * KW * D;
    // 8 consecutive d values per thread and pass
    for (int e = threadIdx.x * 8; e < 2 * KW * D; e += 256 * 8) {
        const int which = e / (KW * D), key = (e / D) % KW, d = e % D;
        const int tok = kblk * KW + key;
        if (tok >= a.Nk) continue;
        f32x4_t x0 = *(const f32x4_t*)(p0 + e), x1 = *(const f32x4_t*)(p0 + e + 4);
        for (int part = 1; part < P; ++part) {
            const float* q = p0 + (size_t)part * 2 * KW * D + e;
            x0 += *(const f32x4_t*)q;
            x1 += *(const f32x4_t*)(q + 4);
        }
        const float f = which == 0 ? a.sm_scale : 1.0f;
        u32x4 w;
        w[0] = pack_rne(x0[0] * f, x0[1] * f);
        w[1] = pack_rne(x0[2] * f, x0[3] * f);
        w[2] = pack_rne(x1[0] * f, x1[1] * f);
        w[3] = pack_rne(x1[2] * f, x1[3] * f);
        uint16_t* dst = which == 0 ? a.dk + b * a.dksb + h * a.dksh + (int64_t)tok * a.dksn
                                   : a.dv + b * a.dvsb + h * a.dvsh + (int64_t)tok * a.dvsn;
        *(u32x4*)(dst + d) = w;
    }
}

// ---------------------------------------------------------------------------
// Dense forward pass 2 with producer/consumer wave pairs. A workgroup owns
// 256 queries and runs 16 waves, four per SIMD: producer wave w (waves 0..7)
// and consumer wave w + 8 share 32 queries and a SIMD.
//   producer: S^T = K Q^T (Q fragments in registers), P = exp(S - LSE) and
//             its quantization, packed as the B operands of P V and written
//             to an LDS exchange slot (no transpose: the accumulator rows are
//             the keys, the contraction index of P V)
//   consumer: O^T += V^T Pq^T from the exchange slot (O^T in registers)
// Each takes 8 of the 16 products per 32-key block; the producer also
// carries the vector work. Step t computes key tile t in the producers and
// key tile t - 1 in the consumers, so K tiles run one tile ahead of V^T
// tiles; both are double-buffered, the exchange by step parity, with one
// barrier per 64-key step. Tile copies are LDS-DMA in inline assembly,
// issued right after the barrier that frees their buffer and waited for at
// the next barrier.
template <int D, bool QP, bool F16>
__global__ __launch_bounds__(1024) void fwd_out_pc_kernel(AttnArgs a) {
    using F = FwdOut<D, QP, F16>;
    constexpr int BN = F::BN, NP = 8;
    constexpr int KBLK = BN * D * 2 / 1024, VBLK = D * BN * 2 / 1024;  // 1 KB DMA blocks per tile
    __shared__ __attribute__((aligned(1024))) uint16_t sK[2][BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[2][D * BN];
    // exchange: [parity][pair][32-key block][chunk j][lane][4 dwords]
    __shared__ __attribute__((aligned(1024))) uint32_t sX[2][NP][2][2][64 * 4];
    lds_poison(sK, sV, sX);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave & 7;
    const bool producer = wave < 8;
    const int l32 = lane & 31, hh = lane >> 5;
    // A one-dimensional grid: whole query blocks, or up to two segments of
    // the last round's key tiles (work_segments), whose fp32 partial sums
    // fwd_out_fixup_kernel adds.
    const int nt = (a.Nk + BN - 1) / BN, nqb = (a.Nq + 255) / 256;
    const bool last_partial = nt * BN > a.Nk;
    Seg sg[2];
    const int ns = work_segments(a.fo_full, a.BH * nqb, nt, a.fo_chunk, sg);
    // this wave's DMA blocks: block `wave` of the K tile (rows 4 b .. 4 b + 3
    // for D = 128, each 16 chunks; perm32 source rows) and of the V^T tile
    // (rows 8 b .. 8 b + 7, 8 chunks each); lane i fills slot 16 i
    uint32_t koff = 0, voff = 0;
    {
        constexpr int CH = D / 8;  // 16-byte chunks per K row
        const int kr = wave * (64 / CH) + lane / CH, kc = lane % CH;
        const int src = (kr & ~31) | perm32(kr & 31);
        koff = (uint32_t)(src * D + ((kc ^ swz<D>(kr)) << 3)) * 2u;
        const int vr = wave * 8 + (lane >> 3), vc = lane & 7;
        voff = (uint32_t)(vr * a.Nk_pad + ((vc ^ swz<BN>(vr)) << 3)) * 2u;
    }
    auto segment = [&](const Seg& sgi) {
        const int qblk = sgi.blk % nqb, bh = sgi.blk / nqb;
        const int t0 = sgi.t0, t1 = sgi.t1, slot = sgi.slot;
        const int q0 = qblk * 256 + pair * 32;
        const int q = q0 + l32;
        const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
        const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
        const uint16_t* Vtb = a.Vt + (size_t)bh * D * a.Nk_pad;
        auto issue_k = [&](int t) {
            if (wave < KBLK) dma16(lds_addr(sK[t & 1] + wave * 512), Kb + (size_t)t * BN * D, koff);
        };
        auto issue_v = [&](int t) {
            if (wave < VBLK) dma16(lds_addr(sV[t & 1] + wave * 512), Vtb + t * BN, voff);
        };
        if (producer) {
            u32x4 qf[D / 16];
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                qf[c] = *(const u32x4*)(Qb + (size_t)q * D + c * 16 + hh * 8);
            float lse2, post;
            p_offset<QP>(a, bh, q, lse2, post);
            // let these loads land before any tile copy is issued (the copies
            // are invisible to the compiler's wait counts)
            wait_vm<0>();
            issue_k(t0);
            wait_vm<0>();
            __syncthreads();
            for (int t = t0; t <= t1; ++t) {
                if (t > t0) {
                    wait_vm<0>();
                    __syncthreads();
                }
                if (t + 1 < t1) issue_k(t + 1);
                if (t < t1) issue_v(t);
                if (t >= t1) continue;
                const uint16_t* K = sK[t & 1];
                uint32_t* X = &sX[t & 1][pair][0][0][0];
                auto run = [&](auto tail) {
                    constexpr bool TL = decltype(tail)::value;
                    const f32x16 s0 = scores_T<D>(K, 0, qf, l32, hh);
                    lds_mfma_chain<D / 16, 4>();
                    const f32x16 s1 = scores_T<D>(K, 32, qf, l32, hh);
                    u32x4 b0[2], b1[2];
                    F::template probs<TL>(s0, t * BN, a.Nk, a.c, lse2, hh, b0);
                    // the vector work of block 0 ahead of block 1's products
                    // (2.46 -> 2.40 ms at 6 heads x 31,200 tokens against one
                    // product per 8 vector instructions)
                    mfma_chain_front<D / 16, 1, 4, 64, 0>();
                    F::template probs<TL>(s1, t * BN + 32, a.Nk, a.c, lse2, hh, b1);
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        *(u32x4*)(X + ((0 * 2 + g) * 64 + lane) * 4) = b0[g];
                        *(u32x4*)(X + ((1 * 2 + g) * 64 + lane) * 4) = b1[g];
                    }
                };
                if (last_partial && t == nt - 1) run(std::true_type{});
                else run(std::false_type{});
            }
        } else {
            f32x16 o[D / 32];
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
            issue_k(t0);
            wait_vm<0>();
            __syncthreads();
            for (int t = t0; t <= t1; ++t) {
                if (t > t0) {
                    wait_vm<0>();
                    __syncthreads();
                }
                if (t + 1 < t1) issue_k(t + 1);
                if (t < t1) issue_v(t);
                if (t == t0) continue;
                const uint16_t* V = sV[(t - 1) & 1];
                const uint32_t* X = &sX[(t - 1) & 1][pair][0][0][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    u32x4 bfr[2];
#pragma unroll
                    for (int g = 0; g < 2; ++g)
                        bfr[g] = *(const u32x4*)(X + ((kb * 2 + g) * 64 + lane) * 4);
                    F::pv(V, kb, bfr, o, l32, hh);
                }
                lds_mfma_chain<D / 8, 4>();
            }
            if (slot >= 0) {
                store_rows_f32<D>(a.fo_part + ((size_t)slot * 256 + pair * 32 + l32) * D, o, hh);
            } else if (q < a.Nq) {
                float off, post;
                p_offset<QP>(a, bh, q, off, post);
                const int64_t b = bh / a.H, h = bh % a.H;
                store_rows_T<D>(a.o + b * a.osb + h * a.osh + (int64_t)q * a.osn, o, post, hh);
            }
        }
    };
    segment(sg[0]);
    if (ns > 1) {
        __syncthreads();  // every wave is done with the tile buffers
        segment(sg[1]);
    }
}

// Sums the partial sums of every last-round query block of a dense forward
// pass 2 that splits its last round (in chunk order) and writes the block's
// O (times the row's output factor) as bf16. One workgroup per block.
template <int D, bool QP>
__global__ __launch_bounds__(256) void fwd_out_fixup_kernel(AttnArgs a) {
    constexpr int QW = 256;
    const int j = blockIdx.x, w = a.fo_full + j;
    const int nqb = (a.Nq + QW - 1) / QW, nt = (a.Nk + 63) / 64;
    const int bh = w / nqb, qblk = w % nqb;
    const int64_t b = bh / a.H, h = bh % a.H;
    // 8 consecutive d values per thread and pass
    for (int e = threadIdx.x * 8; e < QW * D; e += 256 * 8) {
        const int q = qblk * QW + e / D, d = e % D;
        if (q >= a.Nq) continue;
        f32x4_t x0, x1;
        sum_slots<D>(a.fo_part, j, nt, a.fo_chunk, e, x0, x1);
        float off, f;
        p_offset<QP>(a, bh, q, off, f);
        u32x4 v;
        v[0] = pack_rne(x0[0] * f, x0[1] * f);
        v[1] = pack_rne(x0[2] * f, x0[3] * f);
        v[2] = pack_rne(x1[0] * f, x1[1] * f);
        v[3] = pack_rne(x1[2] * f, x1[3] * f);
        *(u32x4*)(a.o + b * a.osb + h * a.osh + (int64_t)q * a.osn + d) = v;
    }
}

// ---------------------------------------------------------------------------
// Dense forward pass 2 with the additive straight-through output, with
// producer/consumer wave pairs (a workgroup runs four pairs, 128 queries,
// eight waves, two per SIMD):
//   producer:  S^T = K Q^T, P = exp(S - LSE) and Pq = FQ(P), both packed as
//              bf16 B operands of the P V products and written to an LDS
//              exchange slot (16 products per 64-key step);
//   consumer:  O^T += V^T Pq^T and O_ste^T += V^T P^T, each V^T operand read
//              once for both (32 products per step).
// As in fwd_out_pc_kernel the producers run one key tile ahead of the
// consumers (K tiles one tile ahead of V^T tiles, both double-buffered, the
// exchange by step parity, one barrier per step). V^T is bf16 here (P is not
// an NVFP4 value). A three-role form (one consumer per output, twelve waves)
// measured the same within 1%.
template <int D>
__global__ __launch_bounds__(512) void fwd_out_ste_pc_kernel(AttnArgs a) {
    using F = FwdOutSte<D, true>;
    constexpr int BN = F::BN, NT = 4, NWV = 8;
    constexpr int KBLK = BN * D * 2 / 1024, VBLK = D * BN * 2 / 1024;  // 1 KB DMA blocks per tile
    __shared__ __attribute__((aligned(1024))) uint16_t sK[2][BN * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[2][D * BN];
    // exchange: [parity][pair][Pq, P][32-key block][chunk g][lane][4 dwords]
    __shared__ __attribute__((aligned(1024))) uint32_t sX[2][NT][2][2][2][64 * 4];
    lds_poison(sK, sV, sX);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave & 3, role = wave >> 2;  // 0 producer, 1 consumer
    const int l32 = lane & 31, hh = lane >> 5;
    // A one-dimensional grid: whole 128-query blocks, or up to two segments
    // of the last round's key tiles (work_segments), whose fp32 partial sums
    // of O and O_ste fwd_out_ste_fixup_kernel adds.
    const int nt = (a.Nk + BN - 1) / BN, nqb = (a.Nq + NT * 32 - 1) / (NT * 32);
    const bool last_partial = nt * BN > a.Nk;
    Seg sg[2];
    const int ns = work_segments(a.fo_full, a.BH * nqb, nt, a.fo_chunk, sg);
    // this wave's DMA blocks: blocks wave, wave + 8, ... of each tile (where
    // they exist); K rows in perm32 order, lane i fills slot 16 i
    constexpr int NJ = (KBLK + NWV - 1) / NWV;
    static_assert(KBLK == VBLK, "tiles of equal size");
    uint32_t koff[NJ], voff[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int blk = wave + j * NWV;
        constexpr int CH = D / 8;  // 16-byte chunks per K row
        const int kr = blk * (64 / CH) + lane / CH, kc = lane % CH;
        const int src = (kr & ~31) | perm32(kr & 31);
        koff[j] = (uint32_t)(src * D + ((kc ^ swz<D>(kr)) << 3)) * 2u;
        const int vr = blk * 8 + (lane >> 3), vc = lane & 7;
        voff[j] = (uint32_t)(vr * a.Nk_pad + ((vc ^ swz<BN>(vr)) << 3)) * 2u;
    }
    auto segment = [&](const Seg& sgi) {
        const int qblk = sgi.blk % nqb, bh = sgi.blk / nqb;
        const int t0 = sgi.t0, t1 = sgi.t1, slot = sgi.slot;
        const int q = qblk * (NT * 32) + pair * 32 + l32;
        const uint16_t* Qb = a.Qw + (size_t)bh * a.Nq_pad * D;
        const uint16_t* Kb = a.Kw + (size_t)bh * a.Nk_pad * D;
        const uint16_t* Vtb = a.Vt + (size_t)bh * D * a.Nk_pad;
        auto issue_k = [&](int t) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                if (wave + j * NWV < KBLK)
                    dma16(lds_addr(sK[t & 1] + (wave + j * NWV) * 512), Kb + (size_t)t * BN * D, koff[j]);
        };
        auto issue_v = [&](int t) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                if (wave + j * NWV < VBLK)
                    dma16(lds_addr(sV[t & 1] + (wave + j * NWV) * 512), Vtb + t * BN, voff[j]);
        };
        if (role == 0) {
            u32x4 qf[D / 16];
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                qf[c] = *(const u32x4*)(Qb + (size_t)q * D + c * 16 + hh * 8);
            float off, post;
            p_offset<true>(a, bh, q, off, post);
            // let these loads land before any tile copy is issued (the copies
            // are invisible to the compiler's wait counts)
            wait_vm<0>();
            issue_k(t0);
            wait_vm<0>();
            __syncthreads();
            for (int t = t0; t <= t1; ++t) {
                if (t > t0) {
                    wait_vm<0>();
                    __syncthreads();
                }
                if (t + 1 < t1) issue_k(t + 1);
                if (t < t1) issue_v(t);
                if (t >= t1) continue;
                const uint16_t* K = sK[t & 1];
                uint32_t* X = &sX[t & 1][pair][0][0][0][0];
                auto run = [&](auto tail) {
                    constexpr bool TL = decltype(tail)::value;
                    const f32x16 s0 = scores_T<D>(K, 0, qf, l32, hh);
                    lds_mfma_chain<D / 16, 4>();
                    const f32x16 s1 = scores_T<D>(K, 32, qf, l32, hh);
                    u32x4 q0[2], p0[2], q1[2], p1[2];
                    F::template probs<TL>(s0, t * BN, a.Nk, a.c, off, hh, q0, p0);
                    mfma_chain_front<D / 16, 1, 4, 64, 0>();
                    F::template probs<TL>(s1, t * BN + 32, a.Nk, a.c, off, hh, q1, p1);
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        *(u32x4*)(X + ((0 * 4 + 0 * 2 + g) * 64 + lane) * 4) = q0[g];
                        *(u32x4*)(X + ((0 * 4 + 1 * 2 + g) * 64 + lane) * 4) = q1[g];
                        *(u32x4*)(X + ((1 * 4 + 0 * 2 + g) * 64 + lane) * 4) = p0[g];
                        *(u32x4*)(X + ((1 * 4 + 1 * 2 + g) * 64 + lane) * 4) = p1[g];
                    }
                };
                if (last_partial && t == nt - 1) run(std::true_type{});
                else run(std::false_type{});
            }
        } else {
            f32x16 o[D / 32], os[D / 32];
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] = os[db] = f32x16{};
            issue_k(t0);
            wait_vm<0>();
            __syncthreads();
            for (int t = t0; t <= t1; ++t) {
                if (t > t0) {
                    wait_vm<0>();
                    __syncthreads();
                }
                if (t + 1 < t1) issue_k(t + 1);
                if (t < t1) issue_v(t);
                if (t == t0) continue;
                const uint16_t* V = sV[(t - 1) & 1];
                const uint32_t* X = &sX[(t - 1) & 1][pair][0][0][0][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    u32x4 bq[2], bp[2];
#pragma unroll
                    for (int g = 0; g < 2; ++g) {
                        bq[g] = *(const u32x4*)(X + ((0 * 4 + kb * 2 + g) * 64 + lane) * 4);
                        bp[g] = *(const u32x4*)(X + ((1 * 4 + kb * 2 + g) * 64 + lane) * 4);
                    }
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                        for (int g = 0; g < 2; ++g) {
                            const u32x4 vf =
                                *(const u32x4*)(V + toff<BN>(db * 32 + l32, 4 * kb + 2 * hh + g));
                            o[db] = mfma(vf, bq[g], o[db]);
                            os[db] = mfma(vf, bp[g], os[db]);
                        }
                    }
                }
                mfma_chain_m<D / 4, 2, 4, 0>();
            }
            if (slot >= 0) {  // slot: [O, O_ste][128 queries][D]
                float* dst = a.fo_part + ((size_t)slot * 256 + pair * 32 + l32) * D;
                store_rows_f32<D>(dst, o, hh);
                store_rows_f32<D>(dst + 128 * D, os, hh);
            } else if (q < a.Nq) {
                float off, post;
                p_offset<true>(a, bh, q, off, post);
                const int64_t b = bh / a.H, h = bh % a.H;
                store_rows_T<D>(a.o + b * a.osb + h * a.osh + (int64_t)q * a.osn, o, post, hh);
                store_rows_T<D>(a.o_ste + b * a.osb + h * a.osh + (int64_t)q * a.osn, os, post, hh);
            }
        }
    };
    segment(sg[0]);
    if (ns > 1) {
        __syncthreads();  // every wave is done with the tile buffers
        segment(sg[1]);
    }
}

// Sums the partial sums of every last-round query block of a dense forward
// pass 2 with O_ste that splits its last round (in chunk order) and writes
// the block's O and O_ste (times the row's output factor) as bf16. One
// workgroup per 128-query block; a slot holds [O, O_ste][128 queries][D].
template <int D>
__global__ __launch_bounds__(256) void fwd_out_ste_fixup_kernel(AttnArgs a) {
    constexpr int QW = 128;
    const int j = blockIdx.x, w = a.fo_full + j;
    const int nqb = (a.Nq + QW - 1) / QW, nt = (a.Nk + 63) / 64;
    const int bh = w / nqb, qblk = w % nqb;
    const int64_t b = bh / a.H, h = bh % a.H;
    // 8 consecutive d values per thread and pass
    for (int e = threadIdx.x * 8; e < 2 * QW * D; e += 256 * 8) {
        const int which = e / (QW * D), q = qblk * QW + (e / D) % QW, d = e % D;
        if (q >= a.Nq) continue;
        f32x4_t x0, x1;
        sum_slots<D>(a.fo_part, j, nt, a.fo_chunk, e, x0, x1);
        float off, f;
        p_offset<true>(a, bh, q, off, f);
        u32x4 v;
        v[0] = pack_rne(x0[0] * f, x0[1] * f);
        v[1] = pack_rne(x0[2] * f, x0[3] * f);
        v[2] = pack_rne(x1[0] * f, x1[1] * f);
        v[3] = pack_rne(x1[2] * f, x1[3] * f);
        *(u32x4*)((which ? a.o_ste : a.o) + b * a.osb + h * a.osh + (int64_t)q * a.osn + d) = v;
    }
}

// ---------------------------------------------------------------------------
// Dense forward workgroups are 8 waves (256 queries), so that each K/V tile
// brought into LDS serves 256 queries; sparse ones are one 128-query block
// (4 waves).
constexpr int kFwdDenseWaves = 8;

template <int D, bool LAZY>
static void fwd_lse_d(const AttnArgs& a, bool sp, hipStream_t st) {
    if (sp) {
        fwd_lse_kernel<D, 4, true, LAZY><<<dim3(a.nbq, a.BH), 256, 0, st>>>(a);
    } else {
        constexpr int NW = kFwdDenseWaves;
        fwd_lse_kernel<D, NW, false, LAZY>
            <<<dim3((a.Nq + NW * 32 - 1) / (NW * 32), a.BH), NW * 64, 0, st>>>(a);
    }
}

// The lazy reference maximum is not the row maximum: the row-max variant,
// which stores it, runs the exact running maximum.
hipError_t launch_fwd_lse(const AttnArgs& a, int D, hipStream_t st) {
    const bool sp = a.kv_idx != nullptr;
    const bool lazy = a.row_max_out == nullptr;
    if (D == 128) lazy ? fwd_lse_d<128, true>(a, sp, st) : fwd_lse_d<128, false>(a, sp, st);
    else lazy ? fwd_lse_d<64, true>(a, sp, st) : fwd_lse_d<64, false>(a, sp, st);
    return hipGetLastError();
}

template <int D, bool QP, bool F16>
static void fwd_out_go(const AttnArgs& a, bool sp, hipStream_t st) {
    if (sp) {
        fwd_out_kernel<D, QP, F16, 4, true><<<dim3(a.nbq, a.BH), 256, 0, st>>>(a);
    } else {
        // one workgroup per whole query block, then a.fo_chunks workgroups
        // sharing the last round's blocks; the fixup finishes those blocks
        const int split = a.BH * ((a.Nq + 255) / 256) - a.fo_full;
        fwd_out_pc_kernel<D, QP, F16><<<a.fo_full + (a.fo_chunk ? a.fo_chunks : 0), 1024, 0, st>>>(a);
        if (a.fo_chunk) fwd_out_fixup_kernel<D, QP><<<split, 256, 0, st>>>(a);
    }
}

template <int D, bool QP>
static void fwd_out_ste_go(const AttnArgs& a, bool sp, hipStream_t st) {
    // sparse: four waves of 32 queries, one per SIMD, each forming S, P, Pq
    // and both products (the two output accumulators and the quantizer need
    // more than the 256 registers of two waves per SIMD); dense: producer /
    // consumer pairs, 128 queries per workgroup
    if (sp) {
        fwd_out_ste_kernel<D, QP, 4, true><<<dim3(a.nbq, a.BH), 256, 0, st>>>(a);
    } else {
        // one workgroup per whole 128-query block, then a.fo_chunks
        // workgroups sharing the last round's blocks; the fixup finishes them
        const int split = a.BH * ((a.Nq + 127) / 128) - a.fo_full;
        fwd_out_ste_pc_kernel<D><<<a.fo_full + (a.fo_chunk ? a.fo_chunks : 0), 512, 0, st>>>(a);
        if (a.fo_chunk) fwd_out_ste_fixup_kernel<D><<<split, 256, 0, st>>>(a);
    }
}

// Pass 2 runs only when P is quantized (otherwise the single-pass forward
// runs instead of both passes).
template <int D>
static void fwd_out_d(const AttnArgs& a, bool sp, hipStream_t st) {
    if (a.o_ste) {  // V^T is bf16 then (pv_f16 off)
        fwd_out_ste_go<D, true>(a, sp, st);
        return;
    }
    if (a.pv_f16) fwd_out_go<D, true, true>(a, sp, st);
    else fwd_out_go<D, true, false>(a, sp, st);
}

hipError_t launch_fwd_out(const AttnArgs& a, int D, hipStream_t st) {
    const bool sp = a.kv_idx != nullptr;
    if (D == 128) fwd_out_d<128>(a, sp, st);
    else fwd_out_d<64>(a, sp, st);
    return hipGetLastError();
}

template <int D>
static void fwd_single_d(const AttnArgs& a, bool sp, hipStream_t st) {
    if (sp) {
        fwd_single_kernel<D, 4, true><<<dim3(a.nbq, a.BH), 256, 0, st>>>(a);
    } else {
        constexpr int NW = kFwdDenseWaves;
        fwd_single_kernel<D, NW, false><<<dim3((a.Nq + NW * 32 - 1) / (NW * 32), a.BH), NW * 64, 0,
                                          st>>>(a);
    }
}

hipError_t launch_fwd_single(const AttnArgs& a, int D, hipStream_t st) {
    const bool sp = a.kv_idx != nullptr;
    if (D == 128) fwd_single_d<128>(a, sp, st);
    else fwd_single_d<64>(a, sp, st);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const AttnArgs& a, int D, hipStream_t st) {
    if (a.kv_idx) {
        dim3 grid(a.nbq, a.BH);
        if (D == 128) bwd_dq_sparse_kernel<128><<<grid, 256, 0, st>>>(a);
        else bwd_dq_sparse_kernel<64><<<grid, 256, 0, st>>>(a);
    } else {
        // one workgroup per whole query block, then a.dq_chunks workgroups
        // sharing the last round's blocks; the fixup finishes those blocks
        const int split = a.BH * ((a.Nq + 255) / 256) - a.dq_full;
        const int grid = a.dq_full + (a.dq_chunk ? a.dq_chunks : 0);
        if (D == 128) bwd_dq_kernel<128, 8, 1, false><<<grid, 512, 0, st>>>(a);
        else bwd_dq_kernel<64, 8, 1, false><<<grid, 512, 0, st>>>(a);
        if (a.dq_chunk) {
            if (D == 128) bwd_dq_fixup_kernel<128><<<split, 256, 0, st>>>(a);
            else bwd_dq_fixup_kernel<64><<<split, 256, 0, st>>>(a);
        }
    }
    return hipGetLastError();
}

// Dense: one workgroup per whole key block and one per part of a split one;
// the split blocks are finished by the fixup.
template <int D>
static void dkdv_d(const AttnArgs& a, bool sp, hipStream_t st) {
    if (sp) {
        const dim3 g(a.BH, a.nbk);
        if (a.quant_p) bwd_dkdv_kernel<D, true, true><<<g, 512, 0, st>>>(a);
        else bwd_dkdv_kernel<D, false, true><<<g, 512, 0, st>>>(a);
    } else {
        const int split = a.BH * a.nbk - a.dkdv_full;
        const int g = a.dkdv_full + split * a.dkdv_parts;
        if (a.quant_p) bwd_dkdv_kernel<D, true, false><<<g, 512, 0, st>>>(a);
        else bwd_dkdv_kernel<D, false, false><<<g, 512, 0, st>>>(a);
        if (a.dkdv_parts > 1) bwd_dkdv_fixup_kernel<D><<<split, 256, 0, st>>>(a);
    }
}

hipError_t launch_bwd_dkdv(const AttnArgs& a, int D, hipStream_t st) {
    const bool sp = a.q_list != nullptr;
    if (D == 128) dkdv_d<128>(a, sp, st);
    else dkdv_d<64>(a, sp, st);
    return hipGetLastError();
}


}  // namespace aq
