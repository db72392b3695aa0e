// Measurement probe (not part of libgdn): the dense bf16 MFMA rate this GPU
// sustains with v_mfma_f32_16x16x32_bf16, the instruction the chunk loop is
// built on.  Every wave keeps eight independent accumulator chains so that
// issue, not the dependent-result latency, limits it; the grid puts several
// waves on every SIMD of every CU.  The result of each lane is stored so that
// nothing is optimised away.  The bench divides the launch's flops by its
// duration (HIP events) and reports that beside the published peak.
#include <hip/hip_runtime.h>

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ void __launch_bounds__(256) probe_mfma_bf16_kernel(float *out, int iters) {
    const int t = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (bf16)(0.001f * (float)((t + e) & 7));
        b[e] = (bf16)(0.001f * (float)((t * 3 + e) & 7));
    }
    f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
    // one block of eight independent accumulating MFMAs per iteration, each
    // chain writing its accumulator in place (written as one asm block: the
    // compiler's own code for this loop shuffled the accumulators between
    // registers with dozens of moves per iteration)
    for (int i = 0; i < iters; ++i) {
        asm volatile(
            "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
            "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
            "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
            "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
            "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
            "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
            "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
            "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
            : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3), "+v"(c4), "+v"(c5), "+v"(c6), "+v"(c7)
            : "v"(a), "v"(b));
    }
    // let the last products land before their results are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
    const f32x4 s4 = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
    out[(size_t)blockIdx.x * blockDim.x + t] = s4[0] + s4[1] + s4[2] + s4[3];
}

extern "C" {

// Launches blocks x 256 threads, each wave running iters x 8 MFMAs of 16 x 16 x 32
// (16384 flops each).  out: blocks * 256 floats of device memory.  Returns the
// hipError_t of the launch.
int probe_mfma_bf16(float *out, int blocks, int iters, void *stream) {
    hipLaunchKernelGGL(probe_mfma_bf16_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return (int)hipGetLastError();
}

// Flops one probe_mfma_bf16 launch performs.
double probe_mfma_bf16_flops(int blocks, int iters) {
    return (double)blocks * 4.0 /* waves */ * (double)iters * kChains * 16.0 * 16.0 * 32.0 * 2.0;
}

}  // extern "C"
