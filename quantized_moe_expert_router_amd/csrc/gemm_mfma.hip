// gemm_mfma.hip -- bf16 MFMA grouped dequant-GEMMs for gfx950 (CDNA4).
//
// The AWQ payload (packed_experts.rs AwqExpertPayload; frozen_awq.rs
// FrozenAwqOps) packs eight 4-bit codes of eight consecutive output columns
// into one I32 word; a row of the cube is K-major: word (k, j) holds columns
// 8j..8j+7 of input feature k.  The MFMA B operand wants, per lane, eight
// consecutive k of one column.  A lane that reads the eight words (k..k+7, j)
// therefore holds, for each of the 8 nibble positions, one complete B operand
// for the column that nibble position encodes.  One MFMA per nibble position
// covers 16 word columns (the 16 lanes of a row) -- the output column order is
// permuted only at the store.  No cross-lane shuffles are needed.
//
// Coefficient: (code - zero) * scale, rounded to the scale dtype (the pages'
// definition), formed in fp32 as fma(code, s, -zero*s), exact for bf16/fp16
// scales, then rounded to bf16 for the MFMA (a no-op for bf16 scales).
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Slot sl of a decoded word: bytes 0..3 of (w & 0x0F0F0F0F) are nibbles
// 0,2,4,6 and bytes 0..3 of ((w >> 4) & 0x0F0F0F0F) nibbles 1,3,5,7.  Under the
// AWQ order (nibble i holds column [0 2 4 6 1 3 5 7][i]) slot sl holds column:
__device__ constexpr int kSlotCol[8] = {0, 4, 1, 5, 2, 6, 3, 7};

// AND the compiler cannot fold into later byte extractions, so that each byte
// converts with one v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t and_opaque(uint32_t x, uint32_t m) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
    return r;
}

// The eight 4-bit codes of a word as floats, in slot order.
__device__ __forceinline__ void decode_codes(uint32_t w, float q[8]) {
    const uint32_t lo = and_opaque(w, 0x0F0F0F0Fu);
    const uint32_t hi = and_opaque(w >> 4, 0x0F0F0F0Fu);
    q[0] = (float)(lo & 0xFFu);
    q[1] = (float)((lo >> 8) & 0xFFu);
    q[2] = (float)((lo >> 16) & 0xFFu);
    q[3] = (float)(lo >> 24);
    q[4] = (float)(hi & 0xFFu);
    q[5] = (float)((hi >> 8) & 0xFFu);
    q[6] = (float)((hi >> 16) & 0xFFu);
    q[7] = (float)(hi >> 24);
}

// Per-group dequant constants of one word column, in slot order.
template <int SD>
struct GroupConst {
    float s[8];   // scale
    float zs[8];  // -zero * scale (16-bit scales) | zero (fp32 scales)
};

template <int SD>
__device__ __forceinline__ void load_group(const uint32_t *qz, const void *scales, size_t zidx,
                                           size_t sidx, GroupConst<SD> &gc) {
    const uint32_t zw = qz[zidx];
    float z[8];
    decode_codes(zw, z);
    float sv[8];
    if (SD == MOEQ_F32) {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(scales) + sidx);
        const float4 v0 = p[0], v1 = p[1];
        sv[0] = v0.x; sv[1] = v0.y; sv[2] = v0.z; sv[3] = v0.w;
        sv[4] = v1.x; sv[5] = v1.y; sv[6] = v1.z; sv[7] = v1.w;
    } else {
        typedef typename Storage<SD>::T S;
        typedef S s8 __attribute__((ext_vector_type(8)));
        const s8 v = *reinterpret_cast<const s8 *>(static_cast<const S *>(scales) + sidx);
#pragma unroll
        for (int c = 0; c < 8; ++c) sv[c] = (float)v[c];
    }
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
        gc.s[sl] = sv[kSlotCol[sl]];
        gc.zs[sl] = SD == MOEQ_F32 ? z[sl] : -z[sl] * gc.s[sl];  // exact: 4-bit x 16-bit
    }
}

// Coefficient of slot sl from code q: the scale-dtype value, as fp32.
template <int SD>
__device__ __forceinline__ float coeff(float q, const GroupConst<SD> &gc, int sl) {
    if (SD == MOEQ_F32) return (q - gc.zs[sl]) * gc.s[sl];        // RNE32((q-z)s)
    const float v = __builtin_fmaf(q, gc.s[sl], gc.zs[sl]);         // exact (q-z)s
    return SD == MOEQ_F16 ? (float)(_Float16)v : v;                 // bf16: rounded at pack
}

// Eight words (rows k..k+7 of one word column) -> eight bf16x8 B operands.
template <int SD>
__device__ __forceinline__ void dequant_operands(const uint32_t wd[8], const GroupConst<SD> &gc,
                                                 bf16x8 bop[8]) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float q0[8], q1[8];
        decode_codes(wd[2 * p], q0);
        decode_codes(wd[2 * p + 1], q1);
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            bop[sl][2 * p] = (__bf16)coeff<SD>(q0[sl], gc, sl);
            bop[sl][2 * p + 1] = (__bf16)coeff<SD>(q1[sl], gc, sl);
        }
    }
}

__device__ __forceinline__ float swiglu_f(float g, float u, float clamp, float alpha, float off) {
    if (clamp > 0.0f) {
        g = fminf(fmaxf(g, -clamp), clamp);
        u = fminf(fmaxf(u, -clamp), clamp);
    }
    return g * (1.0f / (1.0f + expf(-alpha * g))) * (u + off);
}

struct StreamArgs {
    const __bf16 *in;         // [A, K] rows sorted by expert
    __bf16 *out;              // [A, Nout]
    const int32_t *offsets;   // [E+1]
    int K, W, strips, g;      // W = N/8 words per weight row, strips = W/16
    const uint32_t *qw[2];
    const uint32_t *qz[2];
    const void *sc[2];
    const void *bias[2];
    float clamp, alpha, up_offset;
};

// ------------------------------------------------------------------ stream
// Weight-streaming kernel for few rows per expert (decode).  Block = one
// expert x one strip of 16 word columns (128 output columns) of each operand
// set (gate and up, or the single down cube).  Its KSPLIT waves split K; each
// wave streams its K range once, decoding into registers, and multiplies it
// against RT x 16 rows.  Partial sums meet in LDS in a fixed order, then wave
// 0 applies bias, storage rounding and SwiGLU and stores.
template <int NSETS, int SD, int KSPLIT, int RT>
__global__ __launch_bounds__(64 * KSPLIT) void awq_stream_kernel(StreamArgs a) {
    constexpr int NACC = NSETS * 8 * RT;
    __shared__ f32x4 red[KSPLIT > 1 ? KSPLIT / 2 : 1][NACC][kWave];
    const int e = blockIdx.x / a.strips, strip = blockIdx.x % a.strips;
    const int r0 = a.offsets[e], r1 = a.offsets[e + 1];
    if (r1 <= r0) return;  // untouched expert: no weight bytes are read
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = lane & 15, grp = lane >> 4;
    const int j = strip * 16 + c;
    const int Kw = a.K / KSPLIT;
    const int kbeg = w * Kw, kend = kbeg + Kw;
    const int G = a.K / a.g;
    const int N = a.W * 8;

    for (int m0 = r0; m0 < r1; m0 += 16 * RT) {
        f32x4 acc[NSETS][8][RT];
#pragma unroll
        for (int s = 0; s < NSETS; ++s)
#pragma unroll
            for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) acc[s][sl][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        GroupConst<SD> gc[NSETS];
        int cur = -1;
        for (int k0 = kbeg; k0 < kend; k0 += 32) {
            const int gi = k0 / a.g;
            if (gi != cur) {
#pragma unroll
                for (int s = 0; s < NSETS; ++s)
                    load_group<SD>(a.qz[s], a.sc[s], ((size_t)e * G + gi) * a.W + j,
                                   ((size_t)e * G + gi) * N + 8 * j, gc[s]);
                cur = gi;
            }
            uint32_t wd[NSETS][8];
            const size_t wrow = ((size_t)e * a.K + k0 + grp * 8) * a.W + j;
#pragma unroll
            for (int s = 0; s < NSETS; ++s)
#pragma unroll
                for (int i = 0; i < 8; ++i) wd[s][i] = a.qw[s][wrow + (size_t)i * a.W];
            bf16x8 av[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int row = m0 + rt * 16 + c;
                if (row < r1)
                    av[rt] = *reinterpret_cast<const bf16x8 *>(a.in + (size_t)row * a.K + k0 +
                                                               grp * 8);
                else
                    av[rt] = bf16x8{};
            }
#pragma unroll
            for (int s = 0; s < NSETS; ++s) {
                bf16x8 bop[8];
                dequant_operands<SD>(wd[s], gc[s], bop);
#pragma unroll
                for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        acc[s][sl][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av[rt], bop[sl], acc[s][sl][rt], 0, 0, 0);
            }
        }
        // fixed-order tree over the K split: w0 = (w0 + w2) + (w1 + w3)
        if (KSPLIT > 1) {
#pragma unroll
            for (int half = KSPLIT / 2; half >= 1; half >>= 1) {
                __syncthreads();
                if (w >= half && w < 2 * half) {
#pragma unroll
                    for (int s = 0; s < NSETS; ++s)
#pragma unroll
                        for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                            for (int rt = 0; rt < RT; ++rt)
                                red[w - half][(s * 8 + sl) * RT + rt][lane] = acc[s][sl][rt];
                }
                __syncthreads();
                if (w < half) {
#pragma unroll
                    for (int s = 0; s < NSETS; ++s)
#pragma unroll
                        for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                            for (int rt = 0; rt < RT; ++rt)
                                acc[s][sl][rt] += red[w][(s * 8 + sl) * RT + rt][lane];
                }
            }
        }
        if (w != 0) continue;
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
            const int col = 8 * j + kSlotCol[sl];
            float b0 = 0.f, b1 = 0.f;
            if (a.bias[0]) b0 = load_f<SD>(a.bias[0], (size_t)e * N + col);
            if (NSETS == 2 && a.bias[1]) b1 = load_f<SD>(a.bias[1], (size_t)e * N + col);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + rt * 16 + grp * 4 + i;
                    if (row >= r1) continue;
                    float v;
                    if (NSETS == 2) {
                        const float g = round_to<MOEQ_BF16>(acc[0][sl][rt][i] + b0);
                        const float u = round_to<MOEQ_BF16>(acc[1][sl][rt][i] + b1);
                        v = swiglu_f(g, u, a.clamp, a.alpha, a.up_offset);
                    } else {
                        v = acc[0][sl][rt][i] + b0;
                    }
                    a.out[(size_t)row * N + col] = (__bf16)v;
                }
        }
    }
}

template <int NSETS, int SD>
hipError_t launch_stream(const StreamArgs &a, int E, int ksplit, int rt, hipStream_t s) {
    dim3 grid(E * a.strips);
#define MOEQ_STREAM(KS, RTT)                                                                  \
    if (ksplit == KS && rt == RTT) {                                                          \
        hipLaunchKernelGGL((awq_stream_kernel<NSETS, SD, KS, RTT>), grid, dim3(64 * KS), 0, s, \
                           a);                                                                \
        return hipGetLastError();                                                             \
    }
    MOEQ_STREAM(4, 1)
    MOEQ_STREAM(4, 2)
    MOEQ_STREAM(2, 1)
    MOEQ_STREAM(2, 2)
    MOEQ_STREAM(1, 1)
    MOEQ_STREAM(1, 2)
#undef MOEQ_STREAM
    return hipErrorInvalidValue;
}

// Host-side choice of the stream kernel for a bf16 AWQ projection.
bool stream_fits(const ProjProblem &p) {
    if (p.act != MOEQ_BF16 || p.w0.format != MOEQ_FMT_AWQ || !p.offsets) return false;
    if (p.w0.N % 128 != 0 || p.w0.K % 32 != 0 || p.w0.g % 32 != 0) return false;
    const double rows_per_expert = (double)p.rows / (double)p.E;
    return rows_per_expert <= 24.0;
}

template <int NSETS>
hipError_t run_stream(const ProjProblem &p, hipStream_t s) {
    StreamArgs a{};
    a.in = static_cast<const __bf16 *>(p.in);
    a.out = static_cast<__bf16 *>(p.out);
    a.offsets = p.offsets;
    a.K = p.w0.K;
    a.W = p.w0.N / 8;
    a.strips = a.W / 16;
    a.g = p.w0.g;
    const PackedOperand *ops[2] = {&p.w0, &p.w1};
    for (int i = 0; i < 2; ++i) {
        a.qw[i] = reinterpret_cast<const uint32_t *>(ops[i]->qw);
        a.qz[i] = reinterpret_cast<const uint32_t *>(ops[i]->qz);
        a.sc[i] = ops[i]->scales;
        a.bias[i] = ops[i]->bias;
    }
    a.clamp = p.clamp;
    a.alpha = p.alpha;
    a.up_offset = p.up_offset;
    // split K four ways when each quarter is whole 32-row steps
    const int ksplit = (a.K % 128 == 0) ? 4 : (a.K % 64 == 0 ? 2 : 1);
    const int rt = ((double)p.rows / (double)p.E) <= 8.0 ? 1 : 2;
    switch (p.w0.sdt) {
    case MOEQ_BF16: return launch_stream<NSETS, MOEQ_BF16>(a, p.E, ksplit, rt, s);
    case MOEQ_F16: return launch_stream<NSETS, MOEQ_F16>(a, p.E, ksplit, rt, s);
    default: return launch_stream<NSETS, MOEQ_F32>(a, p.E, ksplit, rt, s);
    }
}

}  // namespace

hipError_t launch_fast_swiglu(const ProjProblem &p, hipStream_t s, bool *handled) {
    *handled = false;
    if (p.mode != PROJ_SWIGLU || !stream_fits(p)) return hipSuccess;
    *handled = true;
    return run_stream<2>(p, s);
}

hipError_t launch_fast_plain(const ProjProblem &p, hipStream_t s, bool *handled) {
    *handled = false;
    if (p.mode != PROJ_PLAIN || !stream_fits(p)) return hipSuccess;
    *handled = true;
    return run_stream<1>(p, s);
}

}  // namespace moeq
