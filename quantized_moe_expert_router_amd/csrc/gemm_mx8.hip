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
                                                        uint8_t *__restrict__ s, int sstride) {
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
    s[r * sstride + b] = (uint8_t)(shared + 127);
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
    const uint8_t *qs;       // [A, sstride] E8M0 (K/32 used)
    int sstride;             // scale row stride, a multiple of 16
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

constexpr int kMaxBlocks = 128;  // scale bytes per row held in LDS (K <= 4096)

// LDS: the slab of one 128-k step, 128 rows x 128 bytes with 16-byte chunks
// permuted by chunk ^ ((row >> 1) & 7) (conflict-free fragment reads of 16 rows x
// one chunk), double-buffered; and every scale byte the block uses, staged once:
// the tile rows' activation scales and the block's bank rows' weight scales.
template <int CG>
struct Mx8Lds {
    uint8_t A[2][kRows][kStepK];
    uint8_t SA[kRows][kMaxBlocks];
    // the block's bank rows' scale bytes as one contiguous run, from a 16-byte
    // aligned start (the run begins `shift` bytes in)
    uint8_t SB[64 * CG * kMaxBlocks + 32];
};

// Block = one 128-row m-tile x CG waves of 64 bank rows (one wave per SIMD, the
// 8 x 4 accumulator tiles in AGPRs).  Step st covers k = 128 st .. +127: each
// thread loads its share of the activation slab and each wave its 64 bank rows'
// blocks DEPTH steps ahead into a register ring; the slab of the next step goes to
// the other LDS buffer while this one is used; one LDS-only barrier per step.  The
// scale bytes are staged in LDS once per block with coalesced loads.  The step
// count is padded to a multiple of DEPTH with steps whose data reads as zero, so
// the loop body has no branches and every wait counts exactly.
struct Mx8Stage {
    u32x4 a[4];  // activation chunks (thread's share of the 128 x 128-byte slab)
    u32x4 b[4];  // bank blocks of the wave's four column tiles
    int st;      // the step (loads past the end read clamped addresses; their data
                 // is replaced by zeros where it is used)
};

template <bool SWIGLU, int CG, int DEPTH>
__global__ __launch_bounds__(64 * CG) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mx8_gemm_kernel(Mx8Args a) {
    constexpr int RT = kRows / 16;
    constexpr int kThreads = 64 * CG;
    constexpr int kPer = kRows * 8 / kThreads;  // 16-byte slab chunks per thread
    static_assert(kPer == 4, "stage layout");
    __shared__ __attribute__((aligned(16))) Mx8Lds<CG> lds;

    // m-tiles dealt round-robin to the XCDs (block b runs on XCD b % 8)
    const int mtiles = a.tile_offsets[a.E];
    const int per_xcd = (mtiles + 7) / 8;
    const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int local = idx / a.nblk, nb = idx % a.nblk;
    const int mt = local * 8 + x;  // m-tiles dealt round-robin to the XCDs
    if (local >= per_xcd || mt >= mtiles) return;
    const int e = a.tile_expert[mt];
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kRows;
    const int m1 = min(m0 + kRows, a.offsets[e + 1]);
    const int rtn = (m1 - m0 + 15) >> 4;  // row tiles with rows (block-uniform)

    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const int nblk0 = nb * CG * 64;       // the block's first bank row
    const int n0 = nblk0 + wv * 64;       // this wave's 64 bank rows
    const bool active = n0 < a.R;         // idle waves still stage and meet barriers
    const int nbk = a.K >> 5;             // blocks per bank row
    const int S = (a.K + kStepK - 1) / kStepK;
    const int Spad = (S + DEPTH - 1) / DEPTH * DEPTH;

    const uint8_t *bexp = a.blocks + (size_t)e * a.R * nbk * 16;
    const int rbase = (active ? n0 : 0) + c;
    const int tid = threadIdx.x;

    auto load = [&](int st, Mx8Stage &g) {
        const int k0 = st * kStepK;
        g.st = st;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int ci = tid + kThreads * j, row = ci >> 3, ch = ci & 7;
            const int rr = min(m0 + row, m1 - 1);  // rows past the tile repeat the last row
            const int k = min(k0 + 16 * ch, a.K - 16);
            g.a[j] = *reinterpret_cast<const u32x4 *>(a.q + (size_t)rr * a.K + k);
        }
        const int kc = min(4 * st + q, nbk - 1);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
            g.b[ct] = *reinterpret_cast<const u32x4 *>(
                bexp + ((size_t)(rbase + 16 * ct) * nbk + kc) * 16);
    };
    auto store_slab = [&](int buf, const Mx8Stage &g) {
        const int k0 = g.st * kStepK;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int ci = tid + kThreads * j, row = ci >> 3, ch = ci & 7;
            const u32x4 v = k0 + 16 * ch < a.K ? g.a[j] : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4 *>(&lds.A[buf][row][16 * (ch ^ ((row >> 1) & 7))]) = v;
        }
    };

    f32x4 acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    // every scale byte of the block, once: activation rows (16-byte aligned rows of
    // a.sstride bytes) and the block's bank rows (contiguous, byte loads)
    for (int i = tid; i < kRows * (a.sstride / 16); i += kThreads) {
        const int r = i / (a.sstride / 16), cch = i - r * (a.sstride / 16);
        const int rr = min(m0 + r, m1 - 1);
        const u32x4 v = *reinterpret_cast<const u32x4 *>(a.qs + (size_t)rr * a.sstride + 16 * cch);
        *reinterpret_cast<u32x4 *>(&lds.SA[r][16 * cch]) = v;
    }
    // the bank rows' scales: a 16-byte aligned run of whole chunks (the cube's
    // scale array is 16-byte aligned and a multiple of 16 bytes long)
    const size_t sb0 = ((size_t)e * a.R + nblk0) * nbk;
    const int shift = (int)(sb0 & 15);
    {
        const int nrows = min(64 * CG, a.R - nblk0);
        const int nch = (shift + nrows * nbk + 15) >> 4;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(a.scales + (sb0 - shift));
        for (int i0 = tid; i0 < nch; i0 += 8 * kThreads) {
            u32x4 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = src[min(i0 + j * kThreads, nch - 1)];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = min(i0 + j * kThreads, nch - 1);
                *reinterpret_cast<u32x4 *>(&lds.SB[16 * i]) = v[j];
            }
        }
    }
    // the ring is filled after the staging, in the loop's load order, so the loop
    // entry and its back edge see the same loads in flight
    Mx8Stage ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        load(d, ring[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    store_slab(0, ring[0]);
    __syncthreads();
    for (int s0 = 0; s0 < Spad; s0 += DEPTH) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const int st = s0 + d, buf = st & 1;
            const bool bvalid = 4 * st + q < nbk;
            const int kb = min(4 * st + q, nbk - 1);
            v8i B[4];
            int bsc[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const u32x4 w = bvalid ? ring[d].b[ct] : u32x4{0u, 0u, 0u, 0u};
                B[ct] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
                bsc[ct] = lds.SB[shift + (wv * 64 + 16 * ct + c) * nbk + kb];
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (rt >= rtn) break;  // a partly filled m-tile does only its row tiles
                const int row = rt * 16 + c;
                const int sw = (row >> 1) & 7;
                const u32x4 lo = *reinterpret_cast<const u32x4 *>(&lds.A[buf][row][16 * (q ^ sw)]);
                const u32x4 hi =
                    *reinterpret_cast<const u32x4 *>(&lds.A[buf][row][16 * ((4 + q) ^ sw)]);
                const v8i A = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                const int sa = lds.SA[row][min(4 * st + q, nbk - 1)];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    acc[rt][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        A, B[ct], acc[rt][ct], 0, 4, 0, sa, 0, bsc[ct]);
            }
            // the next step's slab into the other buffer (its loads are DEPTH - 1 old)
            store_slab(buf ^ 1, ring[(d + 1) % DEPTH]);
            load(min(st + DEPTH, Spad - 1), ring[d]);
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
        }
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
                const int row = m0 + rt * 16 + 4 * q + i;
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
                            int sstride, hipStream_t st) {
    const long n = (long)rows * (K >> 5);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(mx8_quant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const __bf16 *>(x), rows, K, q, s, sstride);
    return hipGetLastError();
}

// Grouped projection of MXFP8 rows with an MXFP4 bank on the block-scaled MFMA.
// swiglu: interleaved gate/up bank (R = 2 Nout) with the SwiGLU epilogue; else
// a plain bank (R = Nout).  R % 64 == 0.
hipError_t launch_mx8_gemm(const uint8_t *q, const uint8_t *qs, int sstride, int rows, int K,
                           const PackedOperand &w, const int32_t *offsets,
                           const int32_t *tile_offsets, const int32_t *tile_expert, int E,
                           bool swiglu, int Nout, float clamp, float gate_lo, float alpha,
                           float up_offset, void *out, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    constexpr int CG = 4, DEPTH = 5;
    Mx8Args a{};
    a.q = q;
    a.qs = qs;
    a.sstride = sstride;
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
    const dim3 grid((unsigned)(8 * ((mtiles + 7) / 8) * a.nblk)), block(64 * CG);
    if (swiglu)
        hipLaunchKernelGGL((mx8_gemm_kernel<true, CG, DEPTH>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((mx8_gemm_kernel<false, CG, DEPTH>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace moeq
