// gemm_vjp.hip -- input VJP of the grouped AWQ projections on bf16 MFMA, gfx950.
//
// frozen_awq.rs FrozenAwqOps::frozen_awq_input_backward and packed_experts.rs
// packed_expert_input_backward / packed_swiglu_input_backward: the derivative
// of a packed projection's input is the gradient times the transpose of the
// same rounded coefficients, (code - zero) * scale rounded to the scale dtype,
// with no weight, scale or bias gradients:
//   out[p, k] = sum_n in[p, n] * W_e[k, n]   (+ in2[p, n] * W2_e[k, n] for two cubes)
// where W_e[k, n] is input feature k, output feature n of expert e's cube.
//
// Layout fit.  The AWQ word (k, j) holds the eight consecutive n = 8j..8j+7 of
// row k, and the 16x16x32 bf16 MFMA wants, per lane, eight consecutive
// reduction elements of one output column: one word per lane IS a B operand
// for column k, with its nibbles put in n order by register selection alone.
// The zero word and the eight scales of that word (group k / g) give the
// per-element constants.  A step covers 64 n: lane group q (lanes 16q..16q+15)
// takes words 2q and 2q+1 (n = 16q..16q+15 of the step) and the two MFMA
// sub-steps t use word 2q + t; the A fragments follow the same n assignment.
//
// Each wave owns 64 output columns (four 16-column tiles) and RT 16-row tiles,
// and reuses every decoded B operand for RT MFMAs.
//  RT = 8 (many rows per expert): one block = one 128-row m-tile of the route
//   x CG waves of columns; the 128 x 64 bf16 A slab of a step is staged in a
//   double-buffered LDS tile of 128-byte rows whose 16-byte chunks are permuted
//   by chunk ^ ((row >> 1) & 7), so that the fragment reads of 16 rows x one
//   chunk and the row-wise stores are both free of bank conflicts; one
//   LDS-only barrier per step.
//  RT = 1 (few rows per expert, decode): the block walks its m-tile 16 rows at
//   a time and each wave reads its A fragments straight from memory; weight
//   words, zeros, scales and A run DEPTH steps ahead in registers, so the
//   kernel streams the cubes at HBM rate.
// Blocks deal m-tiles to the eight XCDs in contiguous ranges (block b runs on
// XCD b % 8): the column blocks of an m-tile and the m-tiles of one expert
// share that XCD's L2.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "awq_dequant.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

using namespace awq;

constexpr int kMTile = 128;  // route m-tile rows
constexpr int kStepN = 64;   // reduction elements per step

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Word slot holding natural column i of its eight (inverse of kSlotCol).
__device__ constexpr int kColSlot[8] = {0, 2, 4, 6, 1, 3, 5, 7};

struct VjpArgs {
    const __bf16 *in[2];        // [A, Nred] gradient rows per cube, sorted by expert
    __bf16 *out;                // [A, Kout]
    const int32_t *offsets;     // [E+1]
    const int32_t *tile_offsets;
    const int32_t *tile_expert;
    int E, Kout, Nred, g;       // Kout = cube in_features, Nred = cube out_features
    int nblk;                   // column blocks per m-tile
    const uint32_t *qw[2];
    const uint32_t *qz[2];
    const void *sc[2];
};

// One step of one lane's B-side data: the words of its four column tiles, and
// the zero words and 16 scales of each distinct group (NG) among them.
template <int SD, int NG>
struct StepB {
    static constexpr int kSv = SD == MOEQ_F32 ? 4 : 2;  // 16-byte scale vectors
    u32x2 w[4];
    u32x2 z[NG];
    u32x4 s[NG][kSv];
};

template <int SD, int NG>
__device__ __forceinline__ void load_step_b(const VjpArgs &a, int e, int k0, int q, int c, int st,
                                            StepB<SD, NG> &b) {
    constexpr int sb = SD == MOEQ_F32 ? 4 : 2;
    const int spn = a.Nred / kStepN;
    const int set = st >= spn ? 1 : 0;
    const int n0 = (st - set * spn) * kStepN;
    const int Wn = a.Nred >> 3, G = a.Kout / a.g;
    const int wi = (n0 >> 3) + 2 * q;  // first word of this lane group
    const uint32_t *qw = a.qw[set] + (size_t)e * a.Kout * Wn + wi;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
        b.w[ct] = *reinterpret_cast<const u32x2 *>(qw + (size_t)(k0 + 16 * ct + c) * Wn);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int grp = (k0 + gi * (64 / NG)) / a.g;
        const size_t gr = (size_t)e * G + grp;
        b.z[gi] = *reinterpret_cast<const u32x2 *>(a.qz[set] + gr * Wn + wi);
        const char *sp = static_cast<const char *>(a.sc[set]) +
                         (gr * a.Nred + n0 + 16 * q) * sb;
#pragma unroll
        for (int v = 0; v < StepB<SD, NG>::kSv; ++v)
            b.s[gi][v] = *reinterpret_cast<const u32x4 *>(sp + 16 * v);
    }
}

// The B operands of sub-step t for the four column tiles, in n order.
template <int SD, int NG>
__device__ __forceinline__ void build_b(const StepB<SD, NG> &b, int t, bf16x8 B[4]) {
    GroupConst<SD> gc[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        GroupRaw<SD> r;
        r.zw = b.z[gi][t];
        if (SD == MOEQ_F32) {
            r.s0 = b.s[gi][2 * t];
            r.s1 = b.s[gi][(2 * t + 1) % StepB<SD, NG>::kSv];
        } else {
            r.s0 = b.s[gi][t];
        }
        decode_group<SD>(r, gc[gi]);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const GroupConst<SD> &g = gc[NG == 1 ? 0 : ct / 2];
        float qv[8], cf[8];
        decode_codes(b.w[ct][t], qv);
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) cf[sl] = coeff<SD>(qv[sl], g, sl);
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16(cf[kColSlot[2 * i]], cf[kColSlot[2 * i + 1]]);
        B[ct] = __builtin_bit_cast(bf16x8, v);
    }
}

__device__ __forceinline__ void block_to_tile(const VjpArgs &a, int *mt, int *nb, bool *ok) {
    const int mtiles = a.tile_offsets[a.E];
    const int per_xcd = (mtiles + 7) / 8;
    const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int local = idx / a.nblk;
    *nb = idx % a.nblk;
    *mt = x * per_xcd + local;
    *ok = local < per_xcd && *mt < mtiles;
}

__device__ __forceinline__ void store_tile(const VjpArgs &a, const f32x4 &acc, int row0, int m1,
                                           int col, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = row0 + (lane >> 4) * 4 + i;
        if (row < m1) a.out[(size_t)row * a.Kout + col] = (__bf16)acc[i];
    }
}

// ------------------------------------------------------------------ RT = 8
template <int NSETS, int SD, int NG, int CG>
__global__ __launch_bounds__(64 * CG) __attribute__((amdgpu_waves_per_eu(2, 2)))
void awq_vjp_tile_kernel(VjpArgs a) {
    constexpr int RT = 8;
    constexpr int kThreads = 64 * CG;
    constexpr int kChunks = kMTile * kStepN / 8;        // 16-byte chunks per slab
    constexpr int kPer = kChunks / kThreads;            // per thread
    __shared__ __attribute__((aligned(16))) __bf16 slab[2][kMTile * kStepN];

    int mt, nb;
    bool ok;
    block_to_tile(a, &mt, &nb, &ok);
    if (!ok) return;
    const int e = a.tile_expert[mt];
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kMTile;
    const int m1 = min(m0 + kMTile, a.offsets[e + 1]);
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const int k0 = (nb * CG + wv) * 64;
    const bool active = k0 < a.Kout;  // idle waves still stage A and meet every barrier
    const int kb = active ? k0 : 0;
    const int S = NSETS * a.Nred / kStepN, spn = a.Nred / kStepN;

    // cooperative staging: chunk ci = tid + kThreads * j -> (row ci / 8, chunk ci % 8)
    const int tid = threadIdx.x;
    auto slab_src = [&](int st, int j) -> const u32x4 * {
        const int set = st >= spn ? 1 : 0;
        const int n0 = (st - set * spn) * kStepN;
        const int ci = tid + kThreads * j, row = ci >> 3, ch = ci & 7;
        const int r = min(m0 + row, m1 - 1);  // rows past the tile repeat the last row
        return reinterpret_cast<const u32x4 *>(a.in[set] + (size_t)r * a.Nred + n0 + 8 * ch);
    };
    auto slab_dst = [&](int buf, int j) -> u32x4 * {
        const int ci = tid + kThreads * j, row = ci >> 3, ch = ci & 7;
        return reinterpret_cast<u32x4 *>(&slab[buf][row * kStepN + 8 * (ch ^ ((row >> 1) & 7))]);
    };

    f32x4 acc[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ar[kPer];
    StepB<SD, NG> bcur, bnext;
#pragma unroll
    for (int j = 0; j < kPer; ++j) ar[j] = *slab_src(0, j);
    load_step_b<SD, NG>(a, e, kb, q, c, 0, bcur);
#pragma unroll
    for (int j = 0; j < kPer; ++j) *slab_dst(0, j) = ar[j];
    lds_barrier();

    for (int st = 0; st < S; ++st) {
        const int nx = min(st + 1, S - 1);
#pragma unroll
        for (int j = 0; j < kPer; ++j) ar[j] = *slab_src(nx, j);
        load_step_b<SD, NG>(a, e, kb, q, c, nx, bnext);
        const __bf16 *sl = slab[st & 1];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x8 B[4];
            build_b<SD, NG>(bcur, t, B);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int row = rt * 16 + c, ch = 2 * q + t;
                const bf16x8 A = *reinterpret_cast<const bf16x8 *>(
                    &sl[row * kStepN + 8 * (ch ^ ((row >> 1) & 7))]);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[ct], acc[rt][ct],
                                                                          0, 0, 0);
            }
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) *slab_dst((st + 1) & 1, j) = ar[j];
        bcur = bnext;
        lds_barrier();
    }
    if (!active) return;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) store_tile(a, acc[rt][ct], m0 + rt * 16, m1, k0 + 16 * ct + c, lane);
}

// ------------------------------------------------------------------ RT = 1
template <int SD, int NG>
struct StepAB {
    StepB<SD, NG> b;
    u32x4 a[2];  // A fragments of the two sub-steps
};

template <int NSETS, int SD, int NG, int CG, int DEPTH>
__global__ __launch_bounds__(64 * CG)
void awq_vjp_stream_kernel(VjpArgs a) {
    int mt, nb;
    bool ok;
    block_to_tile(a, &mt, &nb, &ok);
    if (!ok) return;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int k0 = (nb * CG + wv) * 64;
    if (k0 >= a.Kout) return;  // no barriers in this kernel
    const int e = a.tile_expert[mt];
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kMTile;
    const int m1 = min(m0 + kMTile, a.offsets[e + 1]);
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const int S = NSETS * a.Nred / kStepN, spn = a.Nred / kStepN;

    for (int r0 = m0; r0 < m1; r0 += 16) {
        const int arow = min(r0 + c, m1 - 1);  // rows past the tile repeat the last row
        auto load = [&](int st, StepAB<SD, NG> &d) {
            load_step_b<SD, NG>(a, e, k0, q, c, st, d.b);
            const int set = st >= spn ? 1 : 0;
            const int n0 = (st - set * spn) * kStepN;
            const u32x4 *ap =
                reinterpret_cast<const u32x4 *>(a.in[set] + (size_t)arow * a.Nred + n0 + 16 * q);
            d.a[0] = ap[0];
            d.a[1] = ap[1];
        };
        f32x4 acc[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        StepAB<SD, NG> ring[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load(min(d, S - 1), ring[d]);
        for (int s0 = 0; s0 < S; s0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                if (s0 + d < S) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        bf16x8 B[4];
                        build_b<SD, NG>(ring[d].b, t, B);
                        const bf16x8 A = __builtin_bit_cast(bf16x8, ring[d].a[t]);
#pragma unroll
                        for (int ct = 0; ct < 4; ++ct)
                            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[ct], acc[ct],
                                                                              0, 0, 0);
                    }
                }
                load(min(s0 + d + DEPTH, S - 1), ring[d]);
            }
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) store_tile(a, acc[ct], r0, m1, k0 + 16 * ct + c, lane);
    }
}

template <int NSETS, int SD, int NG>
hipError_t launch_nsets(const VjpArgs &a, bool many, int max_tiles, hipStream_t s) {
    constexpr int CG = 4;
    VjpArgs b = a;
    b.nblk = (a.Kout / 64 + CG - 1) / CG;
    const int per_xcd = (max_tiles + 7) / 8;
    const dim3 grid(8 * per_xcd * b.nblk), block(64 * CG);
    if (many)
        hipLaunchKernelGGL((awq_vjp_tile_kernel<NSETS, SD, NG, CG>), grid, block, 0, s, b);
    else
        hipLaunchKernelGGL((awq_vjp_stream_kernel<NSETS, SD, NG, CG, 4>), grid, block, 0, s, b);
    return hipGetLastError();
}

template <int NSETS, int SD>
hipError_t launch_sd(const VjpArgs &a, bool many, int max_tiles, hipStream_t s) {
    return a.g % 64 == 0 ? launch_nsets<NSETS, SD, 1>(a, many, max_tiles, s)
                         : launch_nsets<NSETS, SD, 2>(a, many, max_tiles, s);
}

template <int NSETS>
hipError_t launch_ns(const VjpArgs &a, int sdt, bool many, int max_tiles, hipStream_t s) {
    switch (sdt) {
    case MOEQ_F32: return launch_sd<NSETS, MOEQ_F32>(a, many, max_tiles, s);
    case MOEQ_F16: return launch_sd<NSETS, MOEQ_F16>(a, many, max_tiles, s);
    default: return launch_sd<NSETS, MOEQ_BF16>(a, many, max_tiles, s);
    }
}

}  // namespace

// Shapes this kernel takes: bf16 gradients, AWQ cubes routed through m-tiles,
// 64-column output blocks, whole 64-element reduction steps, groups of 32 or
// multiples of 64, 16-byte aligned rows.
bool vjp_fits(const ProjProblem &p) {
    if (const char *v = getenv("MOEQ_VJP"); v && v[0] == '0') return false;
    if (p.act != MOEQ_BF16 || p.w0.format != MOEQ_FMT_AWQ || !p.offsets || !p.tile_offsets ||
        !p.tile_expert)
        return false;
    if (p.mode != PROJ_INPUT_VJP && p.mode != PROJ_INPUT_VJP2) return false;
    const int Kout = p.Nout, Nred = p.Kred, g = p.w0.g;
    if (Kout % 64 != 0 || Nred % kStepN != 0 || !(g == 32 || g % 64 == 0)) return false;
    if (p.mode == PROJ_INPUT_VJP2 &&
        (p.w1.format != MOEQ_FMT_AWQ || p.w1.sdt != p.w0.sdt || p.w1.g != g || !p.in2))
        return false;
    const uintptr_t al = (uintptr_t)p.in | (uintptr_t)p.in2 | (uintptr_t)p.w0.scales |
                         (uintptr_t)p.w1.scales | (uintptr_t)p.w0.qw | (uintptr_t)p.w1.qw |
                         (uintptr_t)p.w0.qz | (uintptr_t)p.w1.qz;
    return al % 16 == 0;
}

hipError_t launch_vjp(const ProjProblem &p, hipStream_t s) {
    VjpArgs a{};
    const bool two = p.mode == PROJ_INPUT_VJP2;
    a.in[0] = static_cast<const __bf16 *>(p.in);
    a.in[1] = static_cast<const __bf16 *>(two ? p.in2 : p.in);
    a.out = static_cast<__bf16 *>(p.out);
    a.offsets = p.offsets;
    a.tile_offsets = p.tile_offsets;
    a.tile_expert = p.tile_expert;
    a.E = p.E;
    a.Kout = p.Nout;
    a.Nred = p.Kred;
    a.g = p.w0.g;
    const PackedOperand &w1 = two ? p.w1 : p.w0;
    a.qw[0] = reinterpret_cast<const uint32_t *>(p.w0.qw);
    a.qw[1] = reinterpret_cast<const uint32_t *>(w1.qw);
    a.qz[0] = reinterpret_cast<const uint32_t *>(p.w0.qz);
    a.qz[1] = reinterpret_cast<const uint32_t *>(w1.qz);
    a.sc[0] = p.w0.scales;
    a.sc[1] = w1.scales;
    const int max_tiles = (p.rows + kMTile - 1) / kMTile + p.E;
    // many rows per expert on average: the LDS-staged 128-row kernel
    const bool many = (long)p.rows >= 32L * p.E;
    return two ? launch_ns<2>(a, p.w0.sdt, many, max_tiles, s)
               : launch_ns<1>(a, p.w0.sdt, many, max_tiles, s);
}

}  // namespace moeq
