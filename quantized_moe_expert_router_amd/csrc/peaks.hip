// peaks.hip -- measured peaks of one MI355X (gfx950) for the benchmark's
// roofline: a dense bf16 MFMA loop and a streaming HBM read.  Measurement
// support only (libmoeq_peaks.so); the MoE path does not use it.
//
// moeq_peak_mfma_bf16: every wave runs back-to-back MFMAs on register operands
// into 8 independent accumulators (no memory traffic in the loop), so the
// matrix cores are the only busy unit.  shape 0: v_mfma_f32_16x16x32_bf16
// (16384 flops), shape 1: v_mfma_f32_32x32x16_bf16 (32768 flops).
//
// moeq_peak_read: each block reads a contiguous slice of the buffer with
// 16-byte loads, 8 in flight per lane, and reduces it to one word per thread
// (written, so the loads are not removed).
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

template <int SHAPE>
__global__ __launch_bounds__(1024) void mfma_peak_kernel(int iters, float *out) {
    // operands depend on the lane, so nothing folds; values stay small
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((threadIdx.x + i) & 3);
        b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 3);
    }
    if constexpr (SHAPE == 0) {
        f32x4 acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
        }
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    } else {
        f32x16 acc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[j], 0, 0, 0);
        }
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[j][r];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    }
}

__global__ __launch_bounds__(256) void read_peak_kernel(const u32x4 *__restrict__ buf,
                                                        size_t n_vec, uint32_t *out) {
    const size_t per_block = (n_vec + gridDim.x - 1) / gridDim.x;
    const size_t beg = (size_t)blockIdx.x * per_block;
    const size_t end = beg + per_block < n_vec ? beg + per_block : n_vec;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = beg + threadIdx.x;
    for (; i + 7 * 256 < end; i += 8 * 256) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = buf[i + u * 256];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
    for (; i < end; i += 256) acc ^= buf[i];
    out[blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// blocks x (64 * waves) threads, `iters` loop trips of 8 MFMAs per wave;
// out: device float [blocks * 64 * waves].  Returns a hipError_t code.
int moeq_peak_mfma_bf16(int blocks, int waves, int iters, int shape, float *out, void *stream) {
    if (blocks < 1 || waves < 1 || waves > 16 || iters < 1 || !out) return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (shape == 0)
        hipLaunchKernelGGL(mfma_peak_kernel<0>, dim3(blocks), dim3(64 * waves), 0, s, iters, out);
    else
        hipLaunchKernelGGL(mfma_peak_kernel<1>, dim3(blocks), dim3(64 * waves), 0, s, iters, out);
    return (int)hipGetLastError();
}

// Streaming read of `bytes` (a multiple of 16) at `buf` by `blocks` blocks of
// 256 threads; out: device uint32 [blocks * 256].
int moeq_peak_read(const void *buf, size_t bytes, int blocks, uint32_t *out, void *stream) {
    if (!buf || !out || bytes % 16 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(read_peak_kernel, dim3(blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4 *>(buf),
                       bytes / 16, out);
    return (int)hipGetLastError();
}

}  // extern "C"
