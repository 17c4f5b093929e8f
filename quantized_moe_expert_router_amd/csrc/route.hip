// route.hip -- router top-k + FP32 softmax, stable COPY dispatch, combine.
//
// moe_exchange.rs (ruda-tensor 0.21.38), MoeDispatchOps::moe_dispatch: per
// token a discrete top-k selection with FP32 continuous weights, then expert-
// sorted copies of the source rows; MoeDispatchOps::moe_combine: the ascending
// expert-ID combine.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace moeq {

// ------------------------------------------------------------------ router
// One wave per token.  Lane l holds the scores of experts l, l+64, ...
// Selection: k rounds of a wave-wide argmax over the untaken experts, ordered
// by (score descending, expert ID ascending).  Slot j keeps the j-th winner.
// Weights: softmax over the k selected scores in double, rounded to fp32.
struct Cand {
    float v;
    int e;  // kNone when the lane has no candidate
};
constexpr int kNone = 0x7fffffff;

__device__ __forceinline__ bool better(const Cand &a, const Cand &b) {
    if (a.e == kNone) return false;
    if (b.e == kNone) return true;
    return a.v > b.v || (a.v == b.v && a.e < b.e);
}

template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ logits,
                                                          const float *__restrict__ bias,
                                                          int T, int E, int k,
                                                          uint32_t *__restrict__ selected,
                                                          float *__restrict__ weights) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    if (t >= T) return;  // uniform per wave
    const float *row = logits + (size_t)t * E;
    float s[EPL];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E) {
            float v = row[e];
            if (bias) v = v + bias[e];  // one IEEE fp32 add
            s[i] = v;
        } else {
            s[i] = 0.0f;
            taken |= 1u << i;
        }
    }
    int my_sel = 0;
    float my_score = 0.0f;
    for (int j = 0; j < k; ++j) {
        Cand c{0.0f, kNone};
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (!((taken >> i) & 1u)) {
                Cand d{s[i], lane + kWave * i};
                if (better(d, c)) c = d;
            }
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            Cand o{__shfl_xor(c.v, off), __shfl_xor(c.e, off)};
            if (better(o, c)) c = o;
        }
        // every lane now holds the same winner
        if ((c.e & (kWave - 1)) == lane) taken |= 1u << (c.e / kWave);
        if (lane == j) {
            my_sel = c.e;
            my_score = c.v;
        }
    }
    const double m = (double)__shfl(my_score, 0);
    const double ex = exp((double)my_score - m);
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += __shfl(ex, j);  // slot order, same in all lanes
    if (lane < k) {
        selected[(size_t)t * k + lane] = (uint32_t)my_sel;
        weights[(size_t)t * k + lane] = (float)(ex / den);
    }
}

hipError_t launch_router(const float *logits, const float *bias, int T, int E, int k,
                         uint32_t *selected, float *weights, hipStream_t s) {
    const int waves_per_block = 4;
    dim3 grid((T + waves_per_block - 1) / waves_per_block), block(waves_per_block * kWave);
    const int epl = (E + kWave - 1) / kWave;
#define MOEQ_ROUTER(N)                                                                  \
    if (epl <= N) {                                                                     \
        hipLaunchKernelGGL(router_topk_kernel<N>, grid, block, 0, s, logits, bias, T, E, \
                           k, selected, weights);                                       \
        return hipGetLastError();                                                       \
    }
    MOEQ_ROUTER(1)
    MOEQ_ROUTER(2)
    MOEQ_ROUTER(4)
    MOEQ_ROUTER(8)
    MOEQ_ROUTER(16)
    MOEQ_ROUTER(32)
#undef MOEQ_ROUTER
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ dispatch
// Stable counting sort of the T*k assignments by expert.
//  1. block_hist: per block of kTokenBlock tokens, the count of each expert.
//  2. block_scan: expert_offsets = exclusive scan of the totals; block_base[b][e]
//     = first sorted row of expert e for token block b.
//  3. block_scatter: one wave walks its block 64 tokens at a time; the rank of
//     a token among the chunk's tokens that chose the same expert is the
//     popcount of the lower lanes in that expert's 64-bit chunk mask.
__global__ __launch_bounds__(256) void block_hist_kernel(const uint32_t *__restrict__ selected,
                                                         int T, int k, int E,
                                                         int32_t *__restrict__ block_base) {
    extern __shared__ int cnt[];
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const long a0 = (long)b * kTokenBlock * k;
    const long a1 = min((long)(b + 1) * kTokenBlock, (long)T) * k;
    for (long a = a0 + threadIdx.x; a < a1; a += blockDim.x) atomicAdd(&cnt[selected[a]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) block_base[(size_t)b * E + e] = cnt[e];
}

// Exclusive scan of v over the 1024 threads of a block (16 waves).
__device__ int block_exclusive_scan_1024(int v, int *wave_tot) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wave_tot[w] = incl;
    __syncthreads();
    if (w == 0) {
        int t = lane < 16 ? wave_tot[lane] : 0;
        int ti = t;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            int o = __shfl_up(ti, off);
            if (lane >= off) ti += o;
        }
        if (lane < 16) wave_tot[lane] = ti - t;  // exclusive wave offsets
    }
    __syncthreads();
    return wave_tot[w] + incl - v;
}

__global__ __launch_bounds__(1024) void block_scan_kernel(int32_t *__restrict__ block_base,
                                                          int nblocks, int E, int A,
                                                          int32_t *__restrict__ offsets) {
    __shared__ int wave_tot[16];
    // each thread owns experts 2*tid, 2*tid+1 (E <= 2048)
    int tot[2] = {0, 0};
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * (int)threadIdx.x + q;
        if (e < E) {
            int run = 0;
            for (int b = 0; b < nblocks; ++b) {
                const int c = block_base[(size_t)b * E + e];
                block_base[(size_t)b * E + e] = run;
                run += c;
            }
            tot[q] = run;
        }
    }
    const int excl = block_exclusive_scan_1024(tot[0] + tot[1], wave_tot);
    const int starts[2] = {excl, excl + tot[0]};
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * (int)threadIdx.x + q;
        if (e < E) {
            offsets[e] = starts[q];
            for (int b = 0; b < nblocks; ++b) block_base[(size_t)b * E + e] += starts[q];
        }
    }
    if (threadIdx.x == 0) offsets[E] = A;
}

__global__ __launch_bounds__(64) void block_scatter_kernel(
    const uint32_t *__restrict__ selected, int T, int k, int E,
    const int32_t *__restrict__ block_base, int32_t *__restrict__ slot_pos,
    int32_t *__restrict__ row_src, uint32_t *__restrict__ row_experts) {
    extern __shared__ unsigned long long smem_u64[];
    unsigned long long *mask = smem_u64;              // [E]
    int *cnt = reinterpret_cast<int *>(mask + E);     // [E]
    const int b = blockIdx.x, lane = threadIdx.x;
    for (int e = lane; e < E; e += kWave) {
        cnt[e] = block_base[(size_t)b * E + e];
        mask[e] = 0ull;
    }
    __syncthreads();
    const int t_end = min((b + 1) * kTokenBlock, T);
    const unsigned long long lower = (1ull << lane) - 1ull;
    for (int t0 = b * kTokenBlock; t0 < t_end; t0 += kWave) {
        const int t = t0 + lane;
        const bool valid = t < t_end;
        if (valid)
            for (int j = 0; j < k; ++j) atomicOr(&mask[selected[(size_t)t * k + j]], 1ull << lane);
        __syncthreads();
        uint32_t lowest = 0;  // bit j: this lane is the first chunk lane of expert sel[t][j]
        if (valid)
            for (int j = 0; j < k; ++j) {
                const uint32_t e = selected[(size_t)t * k + j];
                const unsigned long long m = mask[e];
                const int p = cnt[e] + __popcll(m & lower);
                slot_pos[(size_t)t * k + j] = p;
                row_src[p] = t;
                row_experts[p] = e;
                if ((m & lower) == 0ull) lowest |= 1u << j;
            }
        __syncthreads();
        if (valid)
            for (int j = 0; j < k; ++j)
                if ((lowest >> j) & 1u) {
                    const uint32_t e = selected[(size_t)t * k + j];
                    cnt[e] += __popcll(mask[e]);
                }
        __syncthreads();
        if (valid)
            for (int j = 0; j < k; ++j)
                if ((lowest >> j) & 1u) mask[selected[(size_t)t * k + j]] = 0ull;
        __syncthreads();
    }
}

hipError_t launch_dispatch_index(const uint32_t *selected, int T, int E, int k,
                                 const moeq_route *route, uint32_t *row_experts,
                                 hipStream_t s) {
    const int nb = route->token_blocks;
    hipLaunchKernelGGL(block_hist_kernel, dim3(nb), dim3(256), sizeof(int) * E, s, selected,
                       T, k, E, route->block_base);
    hipLaunchKernelGGL(block_scan_kernel, dim3(1), dim3(1024), 0, s, route->block_base, nb, E,
                       T * k, route->expert_offsets);
    hipLaunchKernelGGL(block_scatter_kernel, dim3(nb), dim3(64),
                       (sizeof(unsigned long long) + sizeof(int)) * E, s, selected, T, k, E,
                       route->block_base, route->slot_pos, route->row_src, row_experts);
    return hipGetLastError();
}

// ------------------------------------------------------------------ row copy
template <typename V>
__global__ __launch_bounds__(256) void copy_rows_kernel(const V *__restrict__ x,
                                                        size_t row_elems, int A,
                                                        const int32_t *__restrict__ row_src,
                                                        V *__restrict__ values) {
    const int p = blockIdx.x;
    const V *src = x + (size_t)row_src[p] * row_elems;
    V *dst = values + (size_t)p * row_elems;
    for (size_t i = (size_t)blockIdx.y * blockDim.x + threadIdx.x; i < row_elems;
         i += (size_t)gridDim.y * blockDim.x)
        dst[i] = src[i];
}

hipError_t launch_copy_rows(const void *x, size_t row_bytes, int A, const int32_t *row_src,
                            void *values, hipStream_t s) {
    if (A == 0 || row_bytes == 0) return hipSuccess;
    const uintptr_t al = (uintptr_t)x | (uintptr_t)values;
    if (row_bytes % 16 == 0 && al % 16 == 0) {
        const size_t n = row_bytes / 16;
        dim3 grid((unsigned)A, (unsigned)min((n + 255) / 256, (size_t)65535));
        hipLaunchKernelGGL(copy_rows_kernel<uint4>, grid, dim3(256), 0, s, (const uint4 *)x, n,
                           A, row_src, (uint4 *)values);
    } else if (row_bytes % 4 == 0 && al % 4 == 0) {
        const size_t n = row_bytes / 4;
        dim3 grid((unsigned)A, (unsigned)min((n + 255) / 256, (size_t)65535));
        hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, grid, dim3(256), 0, s,
                           (const uint32_t *)x, n, A, row_src, (uint32_t *)values);
    } else {
        dim3 grid((unsigned)A, (unsigned)min((row_bytes + 255) / 256, (size_t)65535));
        hipLaunchKernelGGL(copy_rows_kernel<uint8_t>, grid, dim3(256), 0, s,
                           (const uint8_t *)x, row_bytes, A, row_src, (uint8_t *)values);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// One block per token.  The k sorted positions are ranked so that slot a of
// the shared list is the a-th smallest position, i.e. the a-th smallest expert
// ID; every column then runs acc = fma(w, y, acc) in that order.
template <int ACT>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y,
                                                      const float *__restrict__ weights,
                                                      const int32_t *__restrict__ slot_pos,
                                                      int T, int k, int K, void *__restrict__ out) {
    __shared__ int pos_s[kMaxTopK];
    __shared__ float w_s[kMaxTopK];
    const int t = blockIdx.x;
    if ((int)threadIdx.x < k) {
        const int p = slot_pos[(size_t)t * k + threadIdx.x];
        int rank = 0;
        for (int j = 0; j < k; ++j) rank += slot_pos[(size_t)t * k + j] < p;
        pos_s[rank] = p;
        w_s[rank] = weights[(size_t)t * k + threadIdx.x];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < K; c += blockDim.x) {
        float acc = 0.0f;
        for (int a = 0; a < k; ++a)
            acc = __builtin_fmaf(w_s[a], load_f<ACT>(y, (size_t)pos_s[a] * K + c), acc);
        store_f<ACT>(out, (size_t)t * K + c, acc);
    }
}

hipError_t launch_combine(const void *y, int act, const float *weights,
                          const int32_t *slot_pos, int T, int k, int K, void *out,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (act == MOEQ_F32)
        hipLaunchKernelGGL(combine_kernel<MOEQ_F32>, dim3(T), dim3(256), 0, s, y, weights,
                           slot_pos, T, k, K, out);
    else if (act == MOEQ_BF16)
        hipLaunchKernelGGL(combine_kernel<MOEQ_BF16>, dim3(T), dim3(256), 0, s, y, weights,
                           slot_pos, T, k, K, out);
    else
        hipLaunchKernelGGL(combine_kernel<MOEQ_F16>, dim3(T), dim3(256), 0, s, y, weights,
                           slot_pos, T, k, K, out);
    return hipGetLastError();
}

}  // namespace moeq
