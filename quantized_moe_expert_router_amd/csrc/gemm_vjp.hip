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
//  RT = 8 (more than 8 rows per expert on average): one block = one 128-row
//   m-tile of the route x CG waves of columns, doing only the row tiles that
//   hold rows; the 128 x 64 bf16 A slab of a step is staged in a
//   double-buffered LDS tile of 128-byte rows whose 16-byte chunks are permuted
//   by chunk ^ ((row >> 1) & 7), so that the fragment reads of 16 rows x one
//   chunk and the row-wise stores are both free of bank conflicts; one
//   LDS-only barrier per step.
//  RT = 1 (few rows per expert, decode): a block is 64 columns of one m-tile,
//   its waves split the reduction; it walks the m-tile 16 rows at a time,
//   staging those rows in LDS; weight words, zeros and scales run DEPTH steps
//   of 256 reduction elements ahead in registers, each load reading whole
//   128-byte lines of a weight row.
// Blocks deal m-tiles to the eight XCDs in contiguous ranges (block b runs on
// XCD b % 8): the column blocks of an m-tile and the m-tiles of one expert
// share that XCD's L2.
#include <hip/hip_runtime.h>

#include <cstdio>
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
    const int rtn = (m1 - m0 + 15) >> 4;  // row tiles holding rows (block-uniform)

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
                if (rt >= rtn) break;  // a partly filled m-tile does only its row tiles
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
// Steps of 256 reduction elements: lane group q takes the eight words
// 8q..8q+7 of each of its rows (32 contiguous bytes, so the four lane groups
// read whole 128-byte lines of a weight row) and the eight MFMA sub-steps t
// use word 8q + t.  The block's (at most 16) gradient rows are staged once per
// pass in LDS (16 rows x all reduction elements of both cubes), with 16-byte
// chunks permuted by chunk ^ row so that a fragment read of 16 rows x one chunk
// is free of bank conflicts.
constexpr int kStreamStep = 256;
constexpr size_t kStreamLds = 64 * 1024;  // staged rows: 16 x (reduction of both cubes) bf16

template <int SD, int NG>
struct StreamB {
    static constexpr int kSv = SD == MOEQ_F32 ? 16 : 8;  // 16-byte scale vectors (64 scales)
    u32x4 w[4][2];   // words 8q..8q+7 of each column tile's row
    u32x4 z[NG][2];  // zero words 8q..8q+7
    u32x4 s[NG][kSv];
};

template <int SD, int NG>
__device__ __forceinline__ void load_stream_b(const VjpArgs &a, int e, int k0, int q, int c,
                                              int st, StreamB<SD, NG> &b) {
    constexpr int sb = SD == MOEQ_F32 ? 4 : 2;
    const int spn = a.Nred / kStreamStep;
    const int set = st >= spn ? 1 : 0;
    const int n0 = (st - set * spn) * kStreamStep;
    const int Wn = a.Nred >> 3, G = a.Kout / a.g;
    const int wi = (n0 >> 3) + 8 * q;
    const uint32_t *qw = a.qw[set] + (size_t)e * a.Kout * Wn + wi;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(qw + (size_t)(k0 + 16 * ct + c) * Wn);
        b.w[ct][0] = p[0];
        b.w[ct][1] = p[1];
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const size_t gr = (size_t)e * G + (k0 + gi * (64 / NG)) / a.g;
        const u32x4 *zp = reinterpret_cast<const u32x4 *>(a.qz[set] + gr * Wn + wi);
        b.z[gi][0] = zp[0];
        b.z[gi][1] = zp[1];
        const u32x4 *sp = reinterpret_cast<const u32x4 *>(
            static_cast<const char *>(a.sc[set]) + (gr * a.Nred + n0 + 64 * q) * sb);
#pragma unroll
        for (int v = 0; v < StreamB<SD, NG>::kSv; ++v) b.s[gi][v] = sp[v];
    }
}

// B operands of sub-step t (word 8q + t) for the four column tiles, in n order.
template <int SD, int NG>
__device__ __forceinline__ void build_stream_b(const StreamB<SD, NG> &b, int t, bf16x8 B[4]) {
    GroupConst<SD> gc[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        GroupRaw<SD> r;
        r.zw = b.z[gi][t >> 2][t & 3];
        if (SD == MOEQ_F32) {
            r.s0 = b.s[gi][2 * t];
            r.s1 = b.s[gi][(2 * t + 1) % StreamB<SD, NG>::kSv];
        } else {
            r.s0 = b.s[gi][t];
        }
        decode_group<SD>(r, gc[gi]);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const GroupConst<SD> &g = gc[NG == 1 ? 0 : ct / 2];
        float qv[8], cf[8];
        decode_codes(b.w[ct][t >> 2][t & 3], qv);
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) cf[sl] = coeff<SD>(qv[sl], g, sl);
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack_bf16(cf[kColSlot[2 * i]], cf[kColSlot[2 * i + 1]]);
        B[ct] = __builtin_bit_cast(bf16x8, v);
    }
}

// Block = CG groups of 64 output columns x KS waves each; wave (cg, ks)
// reduces the contiguous step range [ks S / KS, (ks + 1) S / KS), and the KS
// partial sums of a column group meet in LDS (reusing the staging buffer) in
// a fixed order.
template <int NSETS, int SD, int NG, int CG, int KS, int DEPTH>
__global__ __launch_bounds__(64 * CG * KS)
void awq_vjp_stream_kernel(VjpArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char vjp_lds[];
    __bf16 *As = reinterpret_cast<__bf16 *>(vjp_lds);  // [16][NSETS * Nred], chunk-permuted
    f32x4 *red = reinterpret_cast<f32x4 *>(vjp_lds);    // [CG][KS - 1][4][64] after the loop
    int mt, nb;
    bool ok;
    block_to_tile(a, &mt, &nb, &ok);
    if (!ok) return;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cg = wv % CG, ks = wv / CG;
    const int k0 = (nb * CG + cg) * 64;
    const bool active = k0 < a.Kout;  // idle waves still stage rows and meet every barrier
    const int kb = active ? k0 : 0;
    const int e = a.tile_expert[mt];
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kMTile;
    const int m1 = min(m0 + kMTile, a.offsets[e + 1]);
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const int Ntot = NSETS * a.Nred, cpr = Ntot >> 3;  // 16-byte chunks per staged row
    const int S = Ntot / kStreamStep, per = S / KS, sbeg = ks * per;

    for (int r0 = m0; r0 < m1; r0 += 16) {
        f32x4 acc[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        // stage the pass's rows, eight loads in flight per thread (indices past
        // the end repeat the last chunk); fragment reads of rows past the last
        // one read the last row, whose results land in rows that are not stored
        const int nrows = min(16, m1 - r0), arow = min(c, nrows - 1);
        const int total = nrows * cpr;
        for (int i0 = threadIdx.x; i0 < total; i0 += 8 * blockDim.x) {
            u32x4 v[8];
            int at[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = min(i0 + j * (int)blockDim.x, total - 1);
                const int r = i / cpr, ch = i - r * cpr;
                const int row = r0 + r;
                const int n = ch * 8, set = n >= a.Nred ? 1 : 0;
                v[j] = *reinterpret_cast<const u32x4 *>(a.in[set] + (size_t)row * a.Nred +
                                                        (n - set * a.Nred));
                at[j] = r * Ntot + 8 * (ch ^ r);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4 *>(As + at[j]) = v[j];
        }
        // per % DEPTH == 0 (chosen on the host): the loop body has no branches,
        // so the wait before each use counts exactly the DEPTH - 1 younger steps.
        StreamB<SD, NG> ring[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            load_stream_b<SD, NG>(a, e, kb, q, c, sbeg + d, ring[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        for (int s0 = 0; s0 < per; s0 += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int chb = ((sbeg + s0 + d) * kStreamStep >> 3) + 8 * q;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    bf16x8 B[4];
                    build_stream_b<SD, NG>(ring[d], t, B);
                    const bf16x8 A = *reinterpret_cast<const bf16x8 *>(
                        As + (size_t)arow * Ntot + 8 * ((chb + t) ^ arow));
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B[ct], acc[ct], 0,
                                                                          0, 0);
                }
                // past the range: a harmless reload of its last step
                load_stream_b<SD, NG>(a, e, kb, q, c, sbeg + min(s0 + d + DEPTH, per - 1),
                                      ring[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (KS > 1) {
            __syncthreads();  // every wave is done with the staged rows
            if (ks > 0) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    red[((cg * (KS - 1) + ks - 1) * 4 + ct) * 64 + lane] = acc[ct];
            }
            __syncthreads();
            if (ks == 0) {
#pragma unroll
                for (int w = 1; w < KS; ++w)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        acc[ct] += red[((cg * (KS - 1) + w - 1) * 4 + ct) * 64 + lane];
            }
        }
        if (ks == 0 && active) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) store_tile(a, acc[ct], r0, m1, k0 + 16 * ct + c, lane);
        }
        __syncthreads();  // the next pass restages the rows
    }
}

template <int NSETS, int SD, int NG, int CG, int KS>
hipError_t launch_stream_ks(const VjpArgs &a, int per, int per_xcd, size_t lds, hipStream_t s) {
    VjpArgs b = a;
    b.nblk = (a.Kout / 64 + CG - 1) / CG;
    const dim3 grid(8 * per_xcd * b.nblk), block(64 * CG * KS);
    if (per % 2 == 0)
        hipLaunchKernelGGL((awq_vjp_stream_kernel<NSETS, SD, NG, CG, KS, 2>), grid, block, lds, s,
                           b);
    else
        hipLaunchKernelGGL((awq_vjp_stream_kernel<NSETS, SD, NG, CG, KS, 1>), grid, block, lds, s,
                           b);
    return hipGetLastError();
}

template <int NSETS, int SD, int NG>
hipError_t launch_nsets(const VjpArgs &a, bool many, int max_tiles, hipStream_t s) {
    const int per_xcd = (max_tiles + 7) / 8;
    const int S = NSETS * a.Nred / kStreamStep;
    const size_t lds = (size_t)16 * NSETS * a.Nred * 2;
    if (many || a.Nred % kStreamStep != 0 || lds > kStreamLds) {
        constexpr int CG = 4;
        VjpArgs b = a;
        b.nblk = (a.Kout / 64 + CG - 1) / CG;
        const dim3 grid(8 * per_xcd * b.nblk), block(64 * CG);
        hipLaunchKernelGGL((awq_vjp_tile_kernel<NSETS, SD, NG, CG>), grid, block, 0, s, b);
        return hipGetLastError();
    }
    // launch shape: CG column groups x KS reduction slices per block
    int cg = 4, ks = 1;
    if (const char *v = getenv("MOEQ_VJP_SHAPE")) {  // tuning override "CGxKS" (shape only)
        int x = 0, y = 0;
        if (sscanf(v, "%dx%d", &x, &y) == 2 && (x == 1 || x == 2 || x == 4 || x == 8) &&
            (y == 1 || y == 2 || y == 3 || y == 4) && S % y == 0) {
            cg = x;
            ks = y;
        }
    }
    const int per = S / ks;
#define MOEQ_VJP_SHAPE(X, Y) \
    if (cg == X && ks == Y) return launch_stream_ks<NSETS, SD, NG, X, Y>(a, per, per_xcd, lds, s);
    MOEQ_VJP_SHAPE(4, 1)
    MOEQ_VJP_SHAPE(2, 1)
    MOEQ_VJP_SHAPE(1, 1)
    MOEQ_VJP_SHAPE(2, 2)
    MOEQ_VJP_SHAPE(1, 2)
    MOEQ_VJP_SHAPE(1, 3)
    MOEQ_VJP_SHAPE(1, 4)
    MOEQ_VJP_SHAPE(2, 4)
    MOEQ_VJP_SHAPE(4, 2)
    MOEQ_VJP_SHAPE(2, 3)
    MOEQ_VJP_SHAPE(8, 1)
#undef MOEQ_VJP_SHAPE
    return launch_stream_ks<NSETS, SD, NG, 4, 1>(a, S, per_xcd, lds, s);
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
    // more than a few rows per expert on average: the LDS-staged 128-row kernel
    const bool many = (long)p.rows > 8L * p.E;
    return two ? launch_ns<2>(a, p.w0.sdt, many, max_tiles, s)
               : launch_ns<1>(a, p.w0.sdt, many, max_tiles, s);
}

}  // namespace moeq
