// VSA-style coarse block selection for block-sparse fine attention.
//
// FastVideo VSA checkpoint metadata, attention object: 128-token cubes
// (cube_shape [4, 4, 8]), coarse precision BF16 without quantization, and
// effective_topk = max(1, min(ceil((1 - sparsity) * num_blocks), num_blocks)).
// The pooled block means and block scores are rounded to bf16 from exactly
// accumulated values (fp64 sums of bf16 inputs), so every selection decision
// is independent of summation order. Ties go to the lower key-block index;
// each row of the result lists its blocks in ascending order.
#include "aq_kernels.h"

namespace aq {

// Block means, one workgroup per (block, bh, tensor: 0 = q, 1 = k): thread
// (r, c) sums columns 8 c .. 8 c + 7 of token rows r, r + R, ... in fp64 and
// the R partial sums are added in fp64 (exact, so order-independent).
template <int D>
__global__ __launch_bounds__(256) void block_pool_kernel(SelectArgs a) {
    constexpr int C = D / 8, R = 256 / C;
    __shared__ double part[R][D];
    const bool isq = blockIdx.z == 0;
    const int nb = isq ? a.nbq : a.nbk;
    const int j = blockIdx.x;
    if (j >= nb) return;  // the grid covers the larger of nbq and nbk
    const int64_t bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
    const int N = isq ? a.Nq : a.Nk;
    const uint16_t* base = isq ? a.q + b * a.qsb + h * a.qsh : a.k + b * a.ksb + h * a.ksh;
    const int64_t sn = isq ? a.qsn : a.ksn;
    const int c = threadIdx.x % C, r = threadIdx.x / C;
    const int t0 = j * a.bt, t1 = min(N, (j + 1) * a.bt);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int t = t0 + r; t < t1; t += R) {
        const u32x4 w = *(const u32x4*)(base + (int64_t)t * sn + 8 * c);
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
        uint16_t* out = isq ? a.qbar : a.kbar;
        out[(bh * nb + j) * D + threadIdx.x] = bf16_from_double(sum / (double)(t1 - t0));
    }
}

// One block per (bh, query block): bf16 scores against every key block, then
// the top-k by (score desc, index asc), written in ascending index order.
__global__ __launch_bounds__(256) void block_topk_kernel(SelectArgs a) {
    __shared__ float sc[1024];
    __shared__ int sel[1024];
    const int64_t row = blockIdx.x;  // bh * nbq + i
    const int64_t bh = row / a.nbq;
    const uint16_t* qb = a.qbar + row * a.D;
    for (int j = threadIdx.x; j < a.nbk; j += blockDim.x) {
        const uint16_t* kb = a.kbar + (bh * a.nbk + j) * a.D;
        double acc = 0.0;  // the products are exact; the sum runs in column order
        for (int c = 0; c < a.D / 8; ++c) {
            const u32x4 x = *(const u32x4*)(qb + 8 * c);
            const u32x4 y = *(const u32x4*)(kb + 8 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc += (double)bf2f(x[e] & 0xffffu) * (double)bf2f(y[e] & 0xffffu);
                acc += (double)bf2f(x[e] >> 16) * (double)bf2f(y[e] >> 16);
            }
        }
        sc[j] = bf2f(bf16_from_double(acc));
    }
    __syncthreads();
    for (int j = threadIdx.x; j < a.nbk; j += blockDim.x) {
        const float sj = sc[j];
        int rank = 0;
        for (int jj = 0; jj < a.nbk; ++jj) {
            const float s2 = sc[jj];
            rank += (s2 > sj || (s2 == sj && jj < j)) ? 1 : 0;
        }
        sel[j] = rank < a.topk ? 1 : 0;
    }
    __syncthreads();
    int32_t* out = a.idx + row * a.topk;
    for (int j = threadIdx.x; j < a.nbk; j += blockDim.x) {
        if (!sel[j]) continue;
        int pos = 0;
        for (int jj = 0; jj < j; ++jj) pos += sel[jj];
        out[pos] = j;
    }
}

// Reverse index: for each key block, the ascending list of query blocks that
// selected it. One workgroup per (bh, key block j): thread t checks query
// blocks t, t + 256, ... (binary search of j in the ascending row), and a
// ballot and prefix count place the selecting ones in ascending order.
__global__ __launch_bounds__(256) void reverse_index_kernel(const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ q_list,
                                                            int32_t* __restrict__ q_count,
                                                            int64_t BH, int nbq, int nbk, int topk,
                                                            const int32_t* __restrict__ idx_err) {
    __shared__ int wsum[4];
    if (*idx_err) return;
    const int j = blockIdx.x;
    const int64_t bh = blockIdx.y, gi = bh * nbk + j;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int32_t* lst = q_list + gi * nbq;
    int total = 0;
    for (int base = 0; base < nbq; base += 256) {
        const int i = base + threadIdx.x;
        bool f = false;
        if (i < nbq) {
            const int32_t* r = idx + (bh * nbq + i) * topk;
            int lo = 0, hi = topk;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (r[mid] < j) lo = mid + 1;
                else hi = mid;
            }
            f = lo < topk && r[lo] == j;
        }
        const unsigned long long b = __ballot(f);
        const int before = __popcll(b & ((1ull << lane) - 1ull));
        if (lane == 0) wsum[w] = __popcll(b);
        __syncthreads();
        int off = total;
        for (int ww = 0; ww < w; ++ww) off += wsum[ww];
        if (f) lst[off + before] = i;
        total += wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
    if (threadIdx.x == 0) q_count[gi] = total;
}

// Key blocks of each head ordered by descending selection count (ties to
// the lower index): one workgroup per head, each thread ranks its blocks.
__global__ __launch_bounds__(256) void block_order_kernel(const int32_t* __restrict__ q_count,
                                                          int32_t* __restrict__ order, int nbk,
                                                          const int32_t* __restrict__ idx_err) {
    if (*idx_err) return;
    const int64_t bh = blockIdx.x;
    const int32_t* c = q_count + bh * nbk;
    for (int j = threadIdx.x; j < nbk; j += 256) {
        const int cj = c[j];
        int rank = 0;
        for (int jj = 0; jj < nbk; ++jj) {
            const int cc = c[jj];
            rank += (cc > cj || (cc == cj && jj < j)) ? 1 : 0;
        }
        order[bh * nbk + rank] = j;
    }
}

// Check of a caller's block index (int32 [rows][topk]): every entry in
// [0, nbk) and every row strictly ascending. Each workgroup checks a
// grid-stride share of the rows (one thread per row) and writes whether any of
// them broke a rule to part[blockIdx.x] (after a barrier that ORs its threads'
// findings); a one-workgroup pass then ORs the parts into flag (1 if the index
// is bad, else 0). No word is updated by more than one thread, so no clearing
// and no atomics are needed. The sparse attention kernels read the flag and
// skip their work when it is set (their loads would otherwise follow the bad
// entries out of the operand buffers).
__global__ __launch_bounds__(256) void check_index_kernel(const int32_t* __restrict__ idx,
                                                          int64_t rows, int topk, int nbk,
                                                          int32_t* __restrict__ part) {
    int bad = 0;
    for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < rows;
         r += (int64_t)gridDim.x * 256) {
        const int32_t* row = idx + r * topk;
        int prev = -1;
        for (int e = 0; e < topk; ++e) {
            const int v = row[e];
            bad |= (v <= prev || v >= nbk) ? 1 : 0;
            prev = v;
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) part[blockIdx.x] = bad ? 1 : 0;
}

__global__ __launch_bounds__(64) void check_index_reduce_kernel(const int32_t* __restrict__ part,
                                                                int nparts,
                                                                int32_t* __restrict__ flag) {
    const int bad = (int)threadIdx.x < nparts ? part[threadIdx.x] : 0;
    const bool any = __any(bad != 0);
    if (threadIdx.x == 0) *flag = any ? 1 : 0;
}

// When the index check failed, every output of the call is overwritten with
// NaN (bf16 0x7FC0 in the strided token tensors, fp32 NaN in the statistics),
// so that a caller who does not read the flag cannot take stale memory for a
// result. A set flag is rare; the common path reads it and returns.
__global__ __launch_bounds__(256) void poison_outputs_kernel(PoisonArgs a) {
    if (*a.flag == 0) return;
    const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x, nth = (int64_t)gridDim.x * 256;
    for (int i = 0; i < a.nt; ++i) {
        const int64_t rows = a.BH * a.N[i];
        for (int64_t r = tid; r < rows; r += nth) {
            const int64_t bh = r / a.N[i], n = r % a.N[i], b = bh / a.H, h = bh % a.H;
            uint16_t* row = a.t[i] + b * a.sb[i] + h * a.sh[i] + n * a.sn[i];
            for (int d = 0; d < a.D; ++d) row[d] = 0x7FC0;
        }
    }
    for (int i = 0; i < a.nf; ++i)
        for (int64_t j = tid; j < a.fn[i]; j += nth) a.f[i][j] = __builtin_nanf("");
}

hipError_t launch_check_index(const int32_t* idx, int64_t rows, int topk, int nbk, int32_t* flag,
                              hipStream_t st) {
    // the parts follow the flag word: at most 63 workgroups (the flag region
    // holds 64 words)
    int64_t g = (rows + 255) / 256;
    if (g > 63) g = 63;
    check_index_kernel<<<(unsigned)g, 256, 0, st>>>(idx, rows, topk, nbk, flag + 1);
    check_index_reduce_kernel<<<1, 64, 0, st>>>(flag + 1, (int)g, flag);
    return hipGetLastError();
}

hipError_t launch_poison_outputs(const PoisonArgs& a, hipStream_t st) {
    poison_outputs_kernel<<<256, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_block_pool(const SelectArgs& a, hipStream_t st) {
    const dim3 g(max(a.nbq, a.nbk), (unsigned)a.BH, 2);
    if (a.D == 128) block_pool_kernel<128><<<g, 256, 0, st>>>(a);
    else block_pool_kernel<64><<<g, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_block_topk(const SelectArgs& a, hipStream_t st) {
    block_topk_kernel<<<(unsigned)(a.BH * a.nbq), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_reverse_index(const int32_t* idx, int32_t* q_list, int32_t* q_count, int64_t BH,
                                int nbq, int nbk, int topk, int32_t* kv_order,
                                const int32_t* idx_err, hipStream_t st) {
    reverse_index_kernel<<<dim3(nbk, (unsigned)BH), 256, 0, st>>>(idx, q_list, q_count, BH, nbq,
                                                                 nbk, topk, idx_err);
    block_order_kernel<<<(unsigned)BH, 256, 0, st>>>(q_count, kv_order, nbk, idx_err);
    return hipGetLastError();
}

}  // namespace aq
