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

// One thread per (bh, block, column): mean over the block's tokens.
__global__ __launch_bounds__(256) void block_pool_kernel(SelectArgs a) {
    const int64_t total_q = a.BH * a.nbq * a.D;
    const int64_t total = total_q + a.BH * a.nbk * a.D;
    for (int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; gi < total;
         gi += (int64_t)gridDim.x * blockDim.x) {
        const bool isq = gi < total_q;
        const int64_t li = isq ? gi : gi - total_q;
        const int nb = isq ? a.nbq : a.nbk;
        const int N = isq ? a.Nq : a.Nk;
        const int d = (int)(li % a.D);
        const int j = (int)((li / a.D) % nb);
        const int64_t bh = li / ((int64_t)a.D * nb);
        const int64_t b = bh / a.H, h = bh % a.H;
        const uint16_t* base = isq ? a.q + b * a.qsb + h * a.qsh : a.k + b * a.ksb + h * a.ksh;
        const int64_t sn = isq ? a.qsn : a.ksn;
        const int t0 = j * a.bt, t1 = min(N, (j + 1) * a.bt);
        double sum = 0.0;
        for (int t = t0; t < t1; ++t) sum += (double)bf2f(base[(int64_t)t * sn + d]);
        const uint16_t m = bf16_from_double(sum / (double)(t1 - t0));
        uint16_t* out = isq ? a.qbar : a.kbar;
        out[(bh * nb + j) * a.D + d] = m;
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
        double acc = 0.0;
        for (int d = 0; d < a.D; ++d) acc += (double)bf2f(qb[d]) * (double)bf2f(kb[d]);
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
                                                            int64_t BH, int nbq, int nbk, int topk) {
    __shared__ int wsum[4];
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

hipError_t launch_block_pool(const SelectArgs& a, hipStream_t st) {
    const int64_t total = a.BH * (int64_t)(a.nbq + a.nbk) * a.D;
    int64_t g = (total + 255) / 256;
    if (g > 65535) g = 65535;
    block_pool_kernel<<<(unsigned)g, 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_block_topk(const SelectArgs& a, hipStream_t st) {
    block_topk_kernel<<<(unsigned)(a.BH * a.nbq), 256, 0, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_reverse_index(const int32_t* idx, int32_t* q_list, int32_t* q_count, int64_t BH,
                                int nbq, int nbk, int topk, hipStream_t st) {
    reverse_index_kernel<<<dim3(nbk, (unsigned)BH), 256, 0, st>>>(idx, q_list, q_count, BH, nbq,
                                                                 nbk, topk);
    return hipGetLastError();
}

}  // namespace aq
