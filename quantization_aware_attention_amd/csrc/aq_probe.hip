// Machine probes for the benchmark (not part of the attention library):
// the dense BF16 matrix-core rate and the shader clock under that load.
//
// Every wave keeps two independent 32x32x16 BF16 MFMA accumulation chains
// busy for `iters` rounds, four waves per SIMD: in a sweep over one to four
// waves per SIMD and one to four chains per wave this shape sustained the
// highest rate (2.36 PFLOP/s; four chains per wave ran ~15% slower, one wave
// with one chain ~35% slower). Lane 0 of workgroup 0 stamps the shader cycle counter
// (s_memtime) and the fixed 100 MHz wall counter (s_memrealtime) before and
// after its loop, so the ratio of the two gives the clock the chip ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink,
                                                        unsigned long long* stamps) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((lane + i) & 7);
        b[i] = (__bf16)(float)((lane * 3 + i) & 7);
    }
    f32x16 c0 = {}, c1 = {};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c1, 0, 0, 0);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        stamps[0] = t0;
        stamps[1] = t1;
        stamps[2] = r0;
        stamps[3] = r1;
    }
}

}  // namespace

extern "C" {

// Dense BF16 MFMA rate over `blocks` workgroups of four waves, each wave
// running 2 x iters products of 32 x 32 x 16 (32,768 FLOPs each). sink
// (device, blocks x 256 floats) and stamps (device, 4 x uint64) are the
// caller's. Reports the FLOPs per second from HIP events around the launch,
// and the shader clock in MHz from workgroup 0's counters. Returns a
// hipError_t value (0 on success).
int aq_probe_mfma_peak(int blocks, int iters, float* sink, unsigned long long* stamps,
                       double* tflops, double* clock_mhz, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    hipEvent_t e0, e1;
    hipError_t e;
    if ((e = hipEventCreate(&e0)) != hipSuccess) return (int)e;
    if ((e = hipEventCreate(&e1)) != hipSuccess) return (int)e;
    hipEventRecord(e0, st);
    mfma_peak_kernel<<<blocks, 256, 0, st>>>(iters, sink, stamps);
    if ((e = hipGetLastError()) != hipSuccess) return (int)e;
    hipEventRecord(e1, st);
    if ((e = hipEventSynchronize(e1)) != hipSuccess) return (int)e;
    float ms = 0.0f;
    hipEventElapsedTime(&ms, e0, e1);
    unsigned long long h[4];
    if ((e = hipMemcpy(h, stamps, sizeof h, hipMemcpyDeviceToHost)) != hipSuccess) return (int)e;
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    const double flops = (double)blocks * 4.0 * 2.0 * (double)iters * 32768.0;
    *tflops = flops / (ms * 1e-3) / 1e12;
    *clock_mhz = (h[3] > h[2]) ? (double)(h[1] - h[0]) / (double)(h[3] - h[2]) * 100.0 : 0.0;
    return 0;
}

}  // extern "C"
