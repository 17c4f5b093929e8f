// backward.hip -- the combine VJP and the fixed-selection router-logit VJP.
//
// moe_exchange.rs (ruda-tensor 0.21.38): MoeDispatchOps::moe_combine_backward
// forms only the derivatives a MoeCombineSelection requests (expert rows and /
// or the FP32 continuous weights); MoeDispatchOps::moe_dispatch_weights_backward
// is the source-logit VJP of the FP32 weights with the discrete selection held
// fixed.  The COPY VJP (moe_dispatch_backward) shares the combine kernel and
// lives beside it in route.hip.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// ------------------------------------------------------------------ combine VJP
// One block per token t, threads over columns in 16-byte vectors (VEC
// elements).  For each slot j with sorted row p = slot_pos[t, j]:
//   grad_y[p, c] = round_act(fl32(w[t, j] * grad[t, c]))      (the fma's partial in y)
//   grad_w[t, j] = round_fp32(sum_c grad[t, c] * y[p, c])     (products and sum in fp64)
// The fp64 partials are reduced across the wave with xor shuffles and across
// waves through LDS in a fixed order, so the result does not vary from run to
// run.  The y rows of all slots are loaded before the first product.
template <int ACT, int KM, bool VEC_OK>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const void *__restrict__ y, const float *__restrict__ weights,
    const int32_t *__restrict__ slot_pos, const void *__restrict__ grad, int k, int K,
    void *__restrict__ grad_y, float *__restrict__ grad_w) {
    typedef typename Storage<ACT>::T S;
    constexpr int VEC = VEC_OK ? 16 / (int)sizeof(S) : 1;
    typedef S sv __attribute__((ext_vector_type(VEC)));
    constexpr int kWaves = 256 / kWave;
    __shared__ int pos_s[KM];
    __shared__ float w_s[KM];
    __shared__ double red_s[kWaves][KM];
    const int t = blockIdx.x;
    if ((int)threadIdx.x < k) {
        pos_s[threadIdx.x] = slot_pos[(size_t)t * k + threadIdx.x];
        w_s[threadIdx.x] = weights[(size_t)t * k + threadIdx.x];
    }
    __syncthreads();
    const S *ys = static_cast<const S *>(y);
    const S *gs = static_cast<const S *>(grad);
    S *dys = static_cast<S *>(grad_y);
    double part[KM];
#pragma unroll
    for (int a = 0; a < KM; ++a) part[a] = 0.0;
    for (int c = threadIdx.x * VEC; c < K; c += blockDim.x * VEC) {
        const sv g = *reinterpret_cast<const sv *>(gs + (size_t)t * K + c);
        if (grad_w) {
            sv yv[KM];  // slots past k reload slot k - 1 (no branch around a load)
#pragma unroll
            for (int a = 0; a < KM; ++a)
                yv[a] = *reinterpret_cast<const sv *>(ys + (size_t)pos_s[min(a, k - 1)] * K + c);
#pragma unroll
            for (int a = 0; a < KM; ++a) {
                double acc = part[a];
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc += (double)(float)g[v] * (double)(float)yv[a][v];
                part[a] = acc;
            }
        }
        if (grad_y) {
            for (int a = 0; a < k; ++a) {
                const float w = w_s[a];
                sv o;
#pragma unroll
                for (int v = 0; v < VEC; ++v) o[v] = (S)(w * (float)g[v]);
                *reinterpret_cast<sv *>(dys + (size_t)pos_s[a] * K + c) = o;
            }
        }
    }
    if (!grad_w) return;
    const int wave = threadIdx.x / kWave, nwaves = (blockDim.x + kWave - 1) / kWave;
#pragma unroll
    for (int a = 0; a < KM; ++a) {
        if (a < k) {
            const double s = wave_sum(part[a]);
            if (lane_id() == 0) red_s[wave][a] = s;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < k) {
        double s = 0.0;
        for (int w = 0; w < nwaves; ++w) s += red_s[w][threadIdx.x];
        grad_w[(size_t)t * k + threadIdx.x] = (float)s;
    }
}

// ------------------------------------------------------------------ logit VJP
// One wave per token.  Lane j < k holds slot j; the weighted sum
// sum_i w_i dw_i is formed by every lane in slot order from lane broadcasts,
// in fp64 (each product of two fp32 values is exact in fp64), then
// dlogit_j = round_fp32(w_j * (dw_j - sum)).  Each lane then writes the
// columns e = lane, lane + 64, ... of the token's row: the value of the slot
// that selected e, else 0 (selected IDs of a token are distinct).
template <int KM>
__global__ __launch_bounds__(256) void weights_backward_kernel(
    const uint32_t *__restrict__ selected, const float *__restrict__ weights,
    const float *__restrict__ grad_w, int T, int E, int k, float *__restrict__ grad_logits) {
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();
    const int j = min(lane, k - 1);
    const float w = weights[(size_t)t * k + j];
    const float dw = grad_w[(size_t)t * k + j];
    const int sel = (int)selected[(size_t)t * k + j];
    double sum = 0.0;
    for (int i = 0; i < k; ++i) {
        const float wi = __shfl(w, i, kWave), dwi = __shfl(dw, i, kWave);
        sum += (double)wi * (double)dwi;
    }
    const float val = (float)((double)w * ((double)dw - sum));
    int sel_j[KM];
    float val_j[KM];
#pragma unroll
    for (int a = 0; a < KM; ++a) {
        sel_j[a] = a < k ? __shfl(sel, a, kWave) : -1;
        val_j[a] = __shfl(val, a < k ? a : 0, kWave);
    }
    float *row = grad_logits + (size_t)t * E;
    for (int e = lane; e < E; e += kWave) {
        float v = 0.0f;
#pragma unroll
        for (int a = 0; a < KM; ++a) v = sel_j[a] == e ? val_j[a] : v;
        row[e] = v;
    }
}

// ------------------------------------------------------------------ SwiGLU VJP
// Elementwise, in place: G becomes dG and U becomes dU, from dh and the
// storage-rounded G, U of the recomputed gate/up projections:
//   dG = dh (u' + off) (s + alpha g' s (1 - s)),  dU = dh g' s,  s = sigmoid(alpha g'),
// g', u' the values clamped to [-clamp, clamp] when clamp > 0; a clamped value
// passes the derivative on the closed interval and blocks it outside.  fp32
// arithmetic, one rounding to the activation type per output.  For bf16 the
// hardware exp and reciprocal (about one fp32 ulp each) stay far inside that
// rounding; fp32 activations use the accurate library exp.
template <int ACT>
__global__ __launch_bounds__(256) void swiglu_vjp_kernel(void *__restrict__ G, void *__restrict__ U,
                                                         const void *__restrict__ dh, size_t n,
                                                         float clamp, float glo, float alpha,
                                                         float off) {
    typedef typename Storage<ACT>::T S;
    constexpr int VEC = 16 / sizeof(S);
    typedef S sv __attribute__((ext_vector_type(VEC)));
    const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * VEC;
    if (i >= n) return;
    sv *gp = reinterpret_cast<sv *>(static_cast<S *>(G) + i);
    sv *up = reinterpret_cast<sv *>(static_cast<S *>(U) + i);
    const sv gv = *gp, uv = *up;
    const sv dv = *reinterpret_cast<const sv *>(static_cast<const S *>(dh) + i);
    sv og, ou;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        float g = (float)gv[v], u = (float)uv[v];
        const float d = (float)dv[v];
        float gpass = 1.0f, upass = 1.0f;
        if (clamp > 0.0f) {
            gpass = (g >= glo && g <= clamp) ? 1.0f : 0.0f;
            upass = (u >= -clamp && u <= clamp) ? 1.0f : 0.0f;
            g = fminf(fmaxf(g, glo), clamp);
            u = fminf(fmaxf(u, -clamp), clamp);
        }
        const float sg = ACT == MOEQ_F32 ? 1.0f / (1.0f + expf(-alpha * g))
                                         : __builtin_amdgcn_rcpf(1.0f + __expf(-alpha * g));
        og[v] = (S)(gpass * d * (u + off) * (sg + alpha * g * sg * (1.0f - sg)));
        ou[v] = (S)(upass * d * g * sg);
    }
    *gp = og;
    *up = ou;
}

}  // namespace

hipError_t launch_swiglu_vjp(void *G, void *U, const void *dh, int act, size_t n, float clamp,
                             float gate_lo, float alpha, float up_offset, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t vec = act == MOEQ_F32 ? 4 : 8;  // n % 8 == 0: whole vectors
    const size_t threads = n / vec;
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (act == MOEQ_F32)
        hipLaunchKernelGGL((swiglu_vjp_kernel<MOEQ_F32>), grid, block, 0, s, G, U, dh, n, clamp,
                           gate_lo, alpha, up_offset);
    else if (act == MOEQ_BF16)
        hipLaunchKernelGGL((swiglu_vjp_kernel<MOEQ_BF16>), grid, block, 0, s, G, U, dh, n, clamp,
                           gate_lo, alpha, up_offset);
    else
        hipLaunchKernelGGL((swiglu_vjp_kernel<MOEQ_F16>), grid, block, 0, s, G, U, dh, n, clamp,
                           gate_lo, alpha, up_offset);
    return hipGetLastError();
}

hipError_t launch_combine_backward(const void *y, int act, const float *weights,
                                   const int32_t *slot_pos, const void *grad, int T, int k, int K,
                                   void *grad_y, float *grad_weights, hipStream_t s) {
    if (T == 0 || (!grad_y && !grad_weights)) return hipSuccess;
    const int vec = act == MOEQ_F32 ? 4 : 8;
    const bool vec_ok = ((uintptr_t)y | (uintptr_t)grad | (uintptr_t)grad_y) % 16 == 0 &&
                        K % vec == 0;
    int threads = vec_ok ? K / vec : K;
    threads = threads >= 256 ? 256 : ((threads + 63) / 64) * 64;
#define MOEQ_CB(DT, KM)                                                                         \
    do {                                                                                        \
        if (vec_ok)                                                                             \
            hipLaunchKernelGGL((combine_backward_kernel<DT, KM, true>), dim3(T), dim3(threads), \
                               0, s, y, weights, slot_pos, grad, k, K, grad_y, grad_weights);   \
        else                                                                                    \
            hipLaunchKernelGGL((combine_backward_kernel<DT, KM, false>), dim3(T),               \
                               dim3(threads), 0, s, y, weights, slot_pos, grad, k, K, grad_y,   \
                               grad_weights);                                                   \
    } while (0)
#define MOEQ_CB_K(DT)          \
    if (k <= 8)                \
        MOEQ_CB(DT, 8);        \
    else if (k <= 16)          \
        MOEQ_CB(DT, 16);       \
    else                       \
        MOEQ_CB(DT, kMaxTopK)
    if (act == MOEQ_F32)
        MOEQ_CB_K(MOEQ_F32);
    else if (act == MOEQ_BF16)
        MOEQ_CB_K(MOEQ_BF16);
    else
        MOEQ_CB_K(MOEQ_F16);
#undef MOEQ_CB_K
#undef MOEQ_CB
    return hipGetLastError();
}

hipError_t launch_weights_backward(const uint32_t *selected, const float *weights,
                                   const float *grad_weights, int T, int E, int k,
                                   float *grad_logits, hipStream_t s) {
    if (T == 0) return hipSuccess;
    constexpr int kTokensPerBlock = 4;
    const dim3 grid((T + kTokensPerBlock - 1) / kTokensPerBlock), block(kTokensPerBlock * kWave);
    if (k <= 8)
        hipLaunchKernelGGL((weights_backward_kernel<8>), grid, block, 0, s, selected, weights,
                           grad_weights, T, E, k, grad_logits);
    else if (k <= 16)
        hipLaunchKernelGGL((weights_backward_kernel<16>), grid, block, 0, s, selected, weights,
                           grad_weights, T, E, k, grad_logits);
    else
        hipLaunchKernelGGL((weights_backward_kernel<kMaxTopK>), grid, block, 0, s, selected,
                           weights, grad_weights, T, E, k, grad_logits);
    return hipGetLastError();
}

}  // namespace moeq
