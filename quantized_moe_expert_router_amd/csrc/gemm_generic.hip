// gemm_generic.hip -- reference-structured grouped projections on fp32 VALU.
//
// Used for fp32 activations and as the general path for shapes the MFMA
// kernels do not take.  Each block owns one expert and 64 output columns; its
// 256 threads are 64 columns x 4 row groups; rows are processed 16 at a time
// with the activations staged in LDS as fp32.  Every coefficient is decoded
// from the packed words and rounded to its storage type before use, exactly as
// defined (frozen_awq.rs FrozenAwqOps; native.rs ExpertLayout::Native).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

constexpr int kCols = 64;
constexpr int kRowChunk = 16;
constexpr int kKTile = 64;

// AWQ coefficient (code - zero) * scale rounded to the scale dtype, for row k
// (input feature) and column n (output feature) of expert e.
template <int SD>
__device__ __forceinline__ float awq_coeff(const PackedOperand &w, int e, int k, int n) {
    const int words = w.N >> 3;
    const int G = w.K / w.g;
    const uint32_t word = (uint32_t)w.qw[((size_t)e * w.K + k) * words + (n >> 3)];
    const uint32_t zw = (uint32_t)w.qz[((size_t)e * G + k / w.g) * words + (n >> 3)];
    const int sh = 4 * nibble_of_column(n & 7);
    const int code = (int)((word >> sh) & 0xFu), zero = (int)((zw >> sh) & 0xFu);
    const float s = load_f<SD>(w.scales, ((size_t)e * G + k / w.g) * w.N + n);
    return round_to<SD>((float)(code - zero) * s);  // product exact in fp32 for f16/bf16 s
}

// MXFP4 coefficient of bank row r, input feature c: E2M1 * 2^(scale-127), exact.
__device__ __forceinline__ float mxfp4_coeff(const PackedOperand &w, int e, int r, int c) {
    const int nb = w.K >> 5;
    const size_t blk = ((size_t)e * w.N + r) * nb + (c >> 5);
    const uint8_t byte = reinterpret_cast<const uint8_t *>(w.qw)[blk * 16 + ((c & 31) >> 1)];
    const unsigned nib = (c & 1) ? (byte >> 4) : (byte & 0xFu);
    return e2m1_value(nib) * e8m0_value(reinterpret_cast<const uint8_t *>(w.scales)[blk]);
}

template <int SD>
__device__ __forceinline__ float bias_value(const PackedOperand &w, int e, int n) {
    if (!w.bias) return 0.0f;
    if (w.format == MOEQ_FMT_MXFP4_BANK) return load_f<MOEQ_BF16>(w.bias, (size_t)e * w.N + n);
    return load_f<SD>(w.bias, (size_t)e * w.N + n);
}

__device__ __forceinline__ float swiglu(float g, float u, float clamp, float glo, float alpha,
                                        float off) {
    if (clamp > 0.0f) {
        g = fminf(fmaxf(g, glo), clamp);
        u = fminf(fmaxf(u, -clamp), clamp);
    }
    return g * (1.0f / (1.0f + expf(-alpha * g))) * (u + off);
}

template <int ACT, int SD, int MODE>
__global__ __launch_bounds__(256) void proj_generic_kernel(ProjProblem p) {
    constexpr bool two_in = MODE == PROJ_INPUT_VJP2;
    __shared__ float xs[kRowChunk][kKTile + 1];
    __shared__ float xs2[two_in ? kRowChunk : 1][kKTile + 1];
    const int e = blockIdx.y;
    int r0 = 0, r1 = p.rows;
    if (p.offsets) {
        r0 = p.offsets[e];
        r1 = p.offsets[e + 1];
    }
    if (r1 <= r0) return;  // untouched expert: no weight bytes read
    const int tid = threadIdx.x, cl = tid & (kCols - 1), rg = tid >> 6;
    const int col = blockIdx.x * kCols + cl;
    const bool col_ok = col < p.Nout;
    const bool two = (MODE == PROJ_SWIGLU || MODE == PROJ_BANK_SWIGLU || MODE == PROJ_INPUT_VJP2);

    for (int rc = r0; rc < r1; rc += kRowChunk) {
        float acc0[4] = {0.f, 0.f, 0.f, 0.f}, acc1[4] = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < p.Kred; k0 += kKTile) {
            __syncthreads();
            for (int i = tid; i < kRowChunk * kKTile; i += blockDim.x) {
                const int rr = i / kKTile, kk = i % kKTile;
                const int row = rc + rr, kx = k0 + kk;
                xs[rr][kk] = (row < r1 && kx < p.Kred) ? load_f<ACT>(p.in, (size_t)row * p.Kred + kx)
                                                      : 0.0f;
                if (two_in)
                    xs2[rr][kk] = (row < r1 && kx < p.Kred)
                                      ? load_f<ACT>(p.in2, (size_t)row * p.Kred + kx)
                                      : 0.0f;
            }
            __syncthreads();
            if (!col_ok) continue;
            const int kmax = min(kKTile, p.Kred - k0);
            for (int kk = 0; kk < kmax; ++kk) {
                const int kx = k0 + kk;
                float c0, c1 = 0.0f;
                if (MODE == PROJ_PLAIN) {
                    c0 = p.w0.format == MOEQ_FMT_AWQ ? awq_coeff<SD>(p.w0, e, kx, col)
                                                     : mxfp4_coeff(p.w0, e, col, kx);
                } else if (MODE == PROJ_SWIGLU) {
                    c0 = awq_coeff<SD>(p.w0, e, kx, col);
                    c1 = awq_coeff<SD>(p.w1, e, kx, col);
                } else if (MODE == PROJ_BANK_SWIGLU) {
                    c0 = mxfp4_coeff(p.w0, e, 2 * col, kx);
                    c1 = mxfp4_coeff(p.w0, e, 2 * col + 1, kx);
                } else if (MODE == PROJ_INPUT_VJP2) {  // output column = input feature
                    c0 = awq_coeff<SD>(p.w0, e, col, kx);
                    c1 = awq_coeff<SD>(p.w1, e, col, kx);
                } else {  // PROJ_INPUT_VJP: output column = input feature of W
                    c0 = awq_coeff<SD>(p.w0, e, col, kx);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float xv = xs[rg + 4 * i][kk];
                    acc0[i] = __builtin_fmaf(xv, c0, acc0[i]);
                    if (two_in)
                        acc1[i] = __builtin_fmaf(xs2[rg + 4 * i][kk], c1, acc1[i]);
                    else if (two)
                        acc1[i] = __builtin_fmaf(xv, c1, acc1[i]);
                }
            }
        }
        if (!col_ok) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rc + rg + 4 * i;
            if (row >= r1) continue;
            float v;
            if (MODE == PROJ_PLAIN) {
                v = acc0[i] + bias_value<SD>(p.w0, e, col);
            } else if (MODE == PROJ_SWIGLU) {
                const float g = round_to<ACT>(acc0[i] + bias_value<SD>(p.w0, e, col));
                const float u = round_to<ACT>(acc1[i] + bias_value<SD>(p.w1, e, col));
                v = swiglu(g, u, p.clamp, p.gate_lo, p.alpha, p.up_offset);
            } else if (MODE == PROJ_BANK_SWIGLU) {
                const float g = round_to<ACT>(acc0[i] + bias_value<SD>(p.w0, e, 2 * col));
                const float u = round_to<ACT>(acc1[i] + bias_value<SD>(p.w0, e, 2 * col + 1));
                v = swiglu(g, u, p.clamp, p.gate_lo, p.alpha, p.up_offset);
            } else if (MODE == PROJ_INPUT_VJP2) {
                v = acc0[i] + acc1[i];  // gate part, then up part
            } else {
                v = acc0[i];
            }
            store_f<ACT>(p.out, (size_t)row * p.Nout + col, v);
        }
    }
}

template <int ACT, int SD>
hipError_t launch_mode(const ProjProblem &p, hipStream_t s) {
    dim3 grid((p.Nout + kCols - 1) / kCols, p.offsets ? p.E : 1), block(256);
    switch (p.mode) {
    case PROJ_PLAIN:
        hipLaunchKernelGGL((proj_generic_kernel<ACT, SD, PROJ_PLAIN>), grid, block, 0, s, p);
        break;
    case PROJ_SWIGLU:
        hipLaunchKernelGGL((proj_generic_kernel<ACT, SD, PROJ_SWIGLU>), grid, block, 0, s, p);
        break;
    case PROJ_BANK_SWIGLU:
        hipLaunchKernelGGL((proj_generic_kernel<ACT, SD, PROJ_BANK_SWIGLU>), grid, block, 0, s,
                           p);
        break;
    case PROJ_INPUT_VJP2:
        hipLaunchKernelGGL((proj_generic_kernel<ACT, SD, PROJ_INPUT_VJP2>), grid, block, 0, s,
                           p);
        break;
    default:
        hipLaunchKernelGGL((proj_generic_kernel<ACT, SD, PROJ_INPUT_VJP>), grid, block, 0, s, p);
        break;
    }
    return hipGetLastError();
}

template <int ACT>
hipError_t launch_act(const ProjProblem &p, hipStream_t s) {
    switch (p.w0.sdt) {
    case MOEQ_F32: return launch_mode<ACT, MOEQ_F32>(p, s);
    case MOEQ_F16: return launch_mode<ACT, MOEQ_F16>(p, s);
    default: return launch_mode<ACT, MOEQ_BF16>(p, s);
    }
}

}  // namespace

hipError_t launch_proj_generic(const ProjProblem &p, hipStream_t s) {
    if (p.rows == 0 || p.Nout == 0) return hipSuccess;
    switch (p.act) {
    case MOEQ_F32: return launch_act<MOEQ_F32>(p, s);
    case MOEQ_F16: return launch_act<MOEQ_F16>(p, s);
    default: return launch_act<MOEQ_BF16>(p, s);
    }
}

}  // namespace moeq
