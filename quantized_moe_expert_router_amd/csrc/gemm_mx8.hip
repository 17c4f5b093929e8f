// gemm_mx8.hip -- the MXFP4 bank on gfx950's block-scaled MFMA, with MXFP8 activations.
//
// libmir-metal clamped_routed/experts/native.rs (ExpertLayout::Native): a bank row
// holds 32 E2M1 weights per 16-byte block with one E8M0 scale per block.  CDNA4's
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies 16 x 128 blocks with per-32-element
// E8M0 scales in hardware, so the bank is read as it is, with no dequantisation;
// the activations go in as OCP MXFP8 (E4M3 elements, one E8M0 scale per 32), which
// is a different rounding of the activations from the bf16 path: an opt-in variant.
//
// Operand layout of the 16x16x128 scaled MFMA, measured on gfx950 (lane l, row or
// column l % 16, lane group q = l / 16):
//   A (fp8): bytes 0..15 are k = 16q..16q+15, bytes 16..31 are k = 64+16q..64+16q+15;
//   B (fp4): 16 bytes = k = 32q..32q+31, even k in the low nibble -- exactly one bank
//            block;
//   scales: the lane's E8M0 byte scales k-block q of its row (A) or column (B);
//   D: row 4q + i, column l % 16.
#include <hip/hip_runtime.h>

#include "awq_dequant.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

using namespace awq;

typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kRows = 128;   // route m-tile
constexpr int kStepK = 128;  // reduction elements per MFMA

// ------------------------------------------------------------------ quantization
// One thread per 32-element block: the shared exponent floor(log2 max|v|) - 8
// (8 = the largest E4M3 exponent) kept in [-127, 127]; elements v / 2^shared,
// saturated to +-448, converted to E4M3 with round-to-nearest-even.  A zero block
// gets scale byte 0.  The scaling by a power of two is exact.
__global__ __launch_bounds__(256) void mx8_quant_kernel(const __bf16 *__restrict__ x, int rows,
                                                        int K, uint8_t *__restrict__ q,
                                                        uint8_t *__restrict__ s) {
    const int nb = K >> 5;
    const long blk = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= (long)rows * nb) return;
    const long r = blk / nb, b = blk - r * nb;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + r * K + b * 32);
    float v[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4 w = src[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * j + 2 * i] = __uint_as_float(w[i] << 16);
            v[8 * j + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int shared = -127;
    if (amax > 0.0f) {
        int e2;
        frexpf(amax, &e2);
        shared = min(max(e2 - 1 - 8, -127), 127);
    }
    s[blk] = (uint8_t)(shared + 127);
    u32x4 out[2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            t[i] = fminf(fmaxf(__builtin_ldexpf(v[4 * j + i], -shared), -448.0f), 448.0f);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], w, true);
        out[j >> 2][j & 3] = (uint32_t)w;
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(q + r * K + b * 32);
    dst[0] = out[0];
    dst[1] = out[1];
}

// ------------------------------------------------------------------ GEMM
struct Mx8Args {
    const uint8_t *q;        // [A, K] E4M3 rows sorted by expert
    const uint8_t *qs;       // [A, K/32] E8M0
    __bf16 *out;             // [A, Nout]
    const int32_t *offsets;
    const int32_t *tile_offsets;
    const int32_t *tile_expert;
    int E, K, R;             // R = bank rows (2I for the gate/up bank)
    int Nout;
    int nblk;                // blocks per m-tile
    const uint8_t *blocks;   // [E, R, K/32, 16]
    const uint8_t *scales;   // [E, R, K/32]
    const __bf16 *bias;      // [E, R]
    float clamp, gate_lo, alpha, up_offset;
};

// LDS slab of one 128-k step: 128 rows x 128 bytes, 16-byte chunks permuted by
// chunk ^ ((row >> 1) & 7) (conflict-free fragment reads of 16 rows x one chunk),
// plus the rows' four scale bytes of the step.
struct Mx8Lds {
    uint8_t A[2][kRows][kStepK];
    uint32_t S[2][kRows];
};

// Block = one 128-row m-tile x CG groups of 64 bank rows; the two waves of a
// column group take one 64-row half of the tile each.
template <bool SWIGLU, int CG>
__global__ __launch_bounds__(128 * CG) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mx8_gemm_kernel(Mx8Args a) {
    constexpr int RT = kRows / 32;  // row tiles per wave
    constexpr int kThreads = 128 * CG;
    __shared__ __attribute__((aligned(16))) Mx8Lds lds;

    // m-tiles in contiguous ranges per XCD (block b runs on XCD b % 8)
    const int mtiles = a.tile_offsets[a.E];
    const int per_xcd = (mtiles + 7) / 8;
    const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int local = idx / a.nblk, nb = idx % a.nblk;
    const int mt = x * per_xcd + local;
    if (local >= per_xcd || mt >= mtiles) return;
    const int e = a.tile_expert[mt];
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kRows;
    const int m1 = min(m0 + kRows, a.offsets[e + 1]);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = wv / CG, cg = wv % CG;
    const int rtn = min((m1 - m0 + 15) >> 4, 4 * (half + 1)) - 4 * half;  // row tiles with rows
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const int n0 = (nb * CG + cg) * 64;           // this wave's 64 bank rows
    const bool active = n0 < a.R;                 // idle waves still stage A and meet barriers
    const int nbk = a.K >> 5;                     // blocks per row
    const int S = (a.K + kStepK - 1) / kStepK;

    // B: bank rows n0 + 16 ct + c, block 4 st + q (past the end: zero data)
    const uint8_t *bexp = a.blocks + (size_t)e * a.R * nbk * 16;
    const uint8_t *sexp = a.scales + (size_t)e * a.R * nbk;
    const int rbase = (active ? n0 : 0) + c;  // bank row of column tile 0
    auto load_b = [&](int st, u32x4 bw[4], int bs[4]) {
        const int kb = 4 * st + q;
        const int kc = min(kb, nbk - 1);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int off = (rbase + 16 * ct) * nbk + kc;
            const u32x4 w = *reinterpret_cast<const u32x4 *>(bexp + (size_t)off * 16);
            bw[ct] = kb < nbk ? w : u32x4{0u, 0u, 0u, 0u};
            bs[ct] = sexp[off];
        }
    };
    // A staging: thread t moves chunks t + kThreads j of the 128 x 8 chunks of a step
    constexpr int kPer = kRows * 8 / kThreads;
    const int tid = threadIdx.x;
    auto load_a = [&](int st, u32x4 ar[kPer], uint32_t &sr) {
        const int k0 = st * kStepK;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int ci = tid + kThreads * j, row = ci >> 3, ch = ci & 7;
            const int rr = min(m0 + row, m1 - 1);  // rows past the tile repeat the last row
            const int k = k0 + 16 * ch;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(a.q + (size_t)rr * a.K + min(k, a.K - 16));
            ar[j] = k < a.K ? v : u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < kRows) {
            const int rr = min(m0 + tid, m1 - 1);
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kb = 4 * st + i;
                w |= (uint32_t)a.qs[(size_t)rr * nbk + min(kb, nbk - 1)] << (8 * i);
            }
            sr = w;
        }
    };
    auto store_a = [&](int buf, const u32x4 ar[kPer], uint32_t sr) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int ci = tid + kThreads * j, row = ci >> 3, ch = ci & 7;
            *reinterpret_cast<u32x4 *>(&lds.A[buf][row][16 * (ch ^ ((row >> 1) & 7))]) = ar[j];
        }
        if (tid < kRows) lds.S[buf][tid] = sr;
    };

    f32x4 acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ar[kPer];
    uint32_t sr = 0;
    u32x4 bw[4], bwn[4];
    int bs[4], bsn[4];
    load_a(0, ar, sr);
    load_b(0, bw, bs);
    store_a(0, ar, sr);
    lds_barrier();
    for (int st = 0; st < S; ++st) {
        const int nx = min(st + 1, S - 1);
        load_a(nx, ar, sr);
        load_b(nx, bwn, bsn);
        const int buf = st & 1;
        v8i B[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
            B[ct] = v8i{(int)bw[ct][0], (int)bw[ct][1], (int)bw[ct][2], (int)bw[ct][3], 0, 0, 0, 0};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt >= rtn) break;  // a partly filled m-tile does only its row tiles
            const int row = (4 * half + rt) * 16 + c;
            const int sw = (row >> 1) & 7;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(&lds.A[buf][row][16 * (q ^ sw)]);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(&lds.A[buf][row][16 * ((4 + q) ^ sw)]);
            const v8i A = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            const int sa = (int)((lds.S[buf][row] >> (8 * q)) & 0xFFu);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
                acc[rt][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    A, B[ct], acc[rt][ct], 0, 4, 0, sa, 0, bs[ct]);
        }
        store_a(buf ^ 1, ar, sr);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            bw[ct] = bwn[ct];
            bs[ct] = bsn[ct];
        }
        lds_barrier();
    }
    if (!active) return;

    // epilogue: D row 4q + i, bank row n0 + 16 ct + c
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int r = n0 + 16 * ct + c;
        const float b = load_f<MOEQ_BF16>(a.bias, (size_t)e * a.R + r);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt >= rtn) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + (4 * half + rt) * 16 + 4 * q + i;
                const float v = acc[rt][ct][i] + b;
                if constexpr (SWIGLU) {
                    // bank row 2f is gate feature f, row 2f + 1 its up: the odd lane's
                    // value joins the even lane's (every lane takes part in the shuffle)
                    const float uv = __shfl_xor(v, 1, kWave);
                    if ((c & 1) == 0 && row < m1) {
                        const float g = round_to<MOEQ_BF16>(v);
                        const float u = round_to<MOEQ_BF16>(uv);
                        a.out[(size_t)row * a.Nout + (r >> 1)] =
                            (__bf16)swiglu_f(g, u, a.clamp, a.gate_lo, a.alpha, a.up_offset);
                    }
                } else {
                    if (row < m1) a.out[(size_t)row * a.Nout + r] = (__bf16)v;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_mx8_quant(const void *x, int rows, int K, uint8_t *q, uint8_t *s,
                            hipStream_t st) {
    const long n = (long)rows * (K >> 5);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(mx8_quant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const __bf16 *>(x), rows, K, q, s);
    return hipGetLastError();
}

// Grouped projection of MXFP8 rows with an MXFP4 bank on the block-scaled MFMA.
// swiglu: interleaved gate/up bank (R = 2 Nout) with the SwiGLU epilogue; else
// a plain bank (R = Nout).  R % 64 == 0.
hipError_t launch_mx8_gemm(const uint8_t *q, const uint8_t *qs, int rows, int K,
                           const PackedOperand &w, const int32_t *offsets,
                           const int32_t *tile_offsets, const int32_t *tile_expert, int E,
                           bool swiglu, int Nout, float clamp, float gate_lo, float alpha,
                           float up_offset, void *out, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    constexpr int CG = 4;
    Mx8Args a{};
    a.q = q;
    a.qs = qs;
    a.out = static_cast<__bf16 *>(out);
    a.offsets = offsets;
    a.tile_offsets = tile_offsets;
    a.tile_expert = tile_expert;
    a.E = E;
    a.K = K;
    a.R = w.N;
    a.Nout = Nout;
    a.nblk = (a.R / 64 + CG - 1) / CG;
    a.blocks = reinterpret_cast<const uint8_t *>(w.qw);
    a.scales = static_cast<const uint8_t *>(w.scales);
    a.bias = static_cast<const __bf16 *>(w.bias);
    a.clamp = clamp;
    a.gate_lo = gate_lo;
    a.alpha = alpha;
    a.up_offset = up_offset;
    const long mtiles = ((long)rows + kRows - 1) / kRows + E;
    const dim3 grid((unsigned)(8 * ((mtiles + 7) / 8) * a.nblk)), block(128 * CG);
    if (swiglu)
        hipLaunchKernelGGL((mx8_gemm_kernel<true, CG>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((mx8_gemm_kernel<false, CG>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace moeq
