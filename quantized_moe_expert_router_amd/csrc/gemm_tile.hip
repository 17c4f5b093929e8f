// gemm_tile.hip -- LDS-tiled bf16 MFMA grouped dequant-GEMM for many rows per
// expert (prefill-shaped batches), gfx950.
//
// packed_experts.rs FrozenPackedExpertOps::packed_swiglu_forward evaluates the
// gate/up/down chain only for the assigned experts; frozen_awq.rs FrozenAwqOps
// fixes the coefficient (code - zero) * scale, rounded to the scale dtype.
//
// Block tile: 128 rows of one expert x 256 LDS columns -- 128 gate + 128 up
// columns (the same logical columns, so SwiGLU pairs them in registers) or
// 256 columns of a single cube.  Per 32-row K step the block
//   * loads the activation tile (128 x 32 bf16) into LDS,
//   * loads 32 x 32 packed words and dequantises them cooperatively, once per
//     block, into an LDS tile laid out column-major in k (one 16-byte MFMA B
//     operand per lane read),
//   * runs 2 x 2 waves of 64 rows x 128 columns: 4 row tiles x 8 column tiles
//     of 16x16x32 bf16 MFMAs per wave, FP32 accumulators.
// Both LDS tiles are double-buffered; the next step's global loads are issued
// before this step's MFMAs, one barrier per step.  Row tiles past the end of
// the expert skip their MFMAs.  Blocks find their (expert, m-tile) through the
// per-expert m-tile prefix the dispatch kernels write; the n-tiles of one
// m-tile run on one XCD so the activation rows are read into one L2.
//
// The same kernel serves the MXFP4 expert bank (native.rs ExpertLayout::Native):
// its rows are output-major with 32 E2M1 elements per 16-byte block, so one
// block of one bank row is exactly one LDS column's 32 k values; gfx950's
// scaled FP4 converter turns it into bf16 (exact: E2M1 x 2^(s-127)).  For the
// interleaved gate/up bank, row 2i is gate feature i and row 2i+1 up feature i.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "awq_dequant.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

using namespace awq;

constexpr int kBM = kTileRows;   // 128 rows per block tile
constexpr int kUnits = 32;       // word-column units per block tile (x 8 columns)
constexpr int kBCols = kUnits * 8;
constexpr int kLdsRow = 32;  // LDS row: 32 bf16 (one K step), 16-byte chunks permuted

// 16-byte chunk position of chunk ch of LDS row `row`: measured on gfx950,
// chunk ^ ((row >> 1) & 3) lets the MFMA fragment reads (16 rows x one chunk
// per 16 lanes) run at the full 256 bytes per clock.
__device__ __forceinline__ int lds_chunk(int row, int ch) { return ch ^ ((row >> 1) & 3); }

struct TileArgs {
    const __bf16 *in;             // [A, K] rows sorted by expert
    __bf16 *out;                  // [A, Nout]
    const int32_t *offsets;       // [E+1]
    const int32_t *tile_offsets;  // [E+1]
    const int32_t *tile_expert;   // [m-tiles]
    int E, K, W, g;               // W = N/8 words per weight row of a cube
    int ntiles;                   // n-tiles (blocks per m-tile)
    int Nout;                     // output row stride (= output columns)
    int R;                        // MXFP4: bank rows (2I for gate/up, H for down)
    const uint32_t *qw[2];
    const uint32_t *qz[2];
    const void *sc[2];
    const void *bias[2];
    float clamp, alpha, up_offset;
    float gate_lo;  // lower clamp bound of the gate
};

template <int FMT, int NSETS, int SD>
__global__ __launch_bounds__(256, 2) void awq_tile_kernel(TileArgs a) {
    constexpr bool MX = FMT == MOEQ_FMT_MXFP4_BANK;
    constexpr int sb = SD == MOEQ_F32 ? 4 : 2;
    __shared__ __attribute__((aligned(16))) __bf16 As[2][kBM][kLdsRow];
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][kBCols][kLdsRow];

    // ---- which tile: the m-tiles are split into eight contiguous ranges, one
    // per XCD (block b runs on XCD b % 8), so consecutive m-tiles of an expert
    // reuse its weights from that XCD's L2; the n-tiles of an m-tile run there
    // back to back and share its rows
    const int mtiles = a.tile_offsets[a.E];
    const int per_xcd = (mtiles + 7) / 8;
    const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int local = idx / a.ntiles, nt = idx % a.ntiles;
    const int mt = x * per_xcd + local;
    if (local >= per_xcd || mt >= mtiles) return;
    const int e = a.tile_expert[mt];
    const int r_end = a.offsets[e + 1];
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kBM;
    const int m1 = min(m0 + kBM, r_end);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;
    const int c = lane & 15, grp = lane >> 4;
    const int K = a.K, W = a.W, N = W * 8, g = a.g, G = K / g;

    // ---- dequant role.  AWQ: word-column unit u, rows 4kq..4kq+3 of each
    // step.  MXFP4: one bank row per thread, its 16-byte block of each step.
    const int u = tid & (kUnits - 1), kq = tid >> 5;
    const int set = (!MX && NSETS == 2) ? (u >> 4) : 0;
    const int j = NSETS == 2 ? nt * 16 + (u & 15) : nt * kUnits + u;
    const uint32_t *qw = nullptr, *qz = nullptr;
    const char *scb = nullptr;
    const uint8_t *mxb = nullptr, *mxs = nullptr;
    int mxcol = 0;
    bool mxon = false;
    if constexpr (MX) {
        const int brow = nt * 256 + tid;  // bank row
        mxon = brow < a.R;
        const size_t rowbase = ((size_t)e * a.R + (mxon ? brow : 0)) * (K / 32);
        mxb = reinterpret_cast<const uint8_t *>(a.qw[0]) + rowbase * 16;
        mxs = static_cast<const uint8_t *>(a.sc[0]) + rowbase;
        mxcol = NSETS == 2 ? (tid & 1) * 128 + (tid >> 1) : tid;  // gate | up halves
    } else {
        qw = a.qw[set] + (size_t)e * K * W + j;
        qz = a.qz[set] + (size_t)e * G * W + j;
        scb = static_cast<const char *>(a.sc[set]) + ((size_t)e * G * N + 8 * j) * sb;
    }
    // ---- activation-tile role: two 16-byte chunks (row, quarter) per thread
    int arow[2], apart[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ch = tid + 256 * h;
        arow[h] = ch >> 2;
        apart[h] = ch & 3;
    }
    const int nsteps = K / 32;

    // one in-flight K step of raw data (two live at a time: steps ks+2, ks+3)
    struct Stage {
        uint32_t wd[4];   // AWQ words
        u32x4 blk;        // MXFP4 block
        uint32_t sbyte;   // MXFP4 E8M0 scale
        u32x4 ar[2];
        GroupRaw<SD> graw;
    };
    Stage st[2];
    GroupConst<SD> gc;
    auto load_step = [&](Stage &S, int ks) {
        if (ks >= nsteps) return;
        const int k0 = ks * 32;
        if constexpr (MX) {
            if (mxon) {
                S.blk = *reinterpret_cast<const u32x4 *>(mxb + (size_t)ks * 16);
                S.sbyte = mxs[ks];
            } else {
                S.blk = u32x4{0u, 0u, 0u, 0u};
                S.sbyte = 127u;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) S.wd[i] = qw[(size_t)(k0 + 4 * kq + i) * W];
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = m0 + arow[h];
            S.ar[h] = row < m1 ? *reinterpret_cast<const u32x4 *>(a.in + (size_t)row * K + k0 +
                                                                   8 * apart[h])
                               : u32x4{0u, 0u, 0u, 0u};
        }
        if (!MX && k0 % g == 0) {
            const int gi = k0 / g;
            S.graw.zw = qz[(size_t)gi * W];
            const u32x4 *sp = reinterpret_cast<const u32x4 *>(scb + (size_t)gi * N * sb);
            S.graw.s0 = sp[0];
            if (SD == MOEQ_F32) S.graw.s1 = sp[1];
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch where it is issued
    };
    // AWQ: LDS column of logical column `col` of word-column unit v is
    // col * 32 + v, so the 32 units' writes of one column spread over the banks.
    auto store_step = [&](const Stage &S, int ks, int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *reinterpret_cast<u32x4 *>(&As[buf][arow[h]][8 * lds_chunk(arow[h], apart[h])]) = S.ar[h];
        if constexpr (MX) {
            // E8M0 scale 2^(s-127) as fp32: s = 0 is the subnormal 2^-127, s = 255 NaN
            const uint32_t sbits = S.sbyte == 255u ? 0x7FC00000u
                                 : S.sbyte ? (S.sbyte << 23) : 0x00400000u;
            const float sc = __uint_as_float(sbits);
#pragma unroll
            for (int d = 0; d < 4; ++d) {  // elements 8d..8d+7: dword d of the block
                typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(S.blk[d], sc, 0);
                const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(S.blk[d], sc, 1);
                const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(S.blk[d], sc, 2);
                const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(S.blk[d], sc, 3);
                u32x4 v;
                v[0] = __builtin_bit_cast(uint32_t, p0);
                v[1] = __builtin_bit_cast(uint32_t, p1);
                v[2] = __builtin_bit_cast(uint32_t, p2);
                v[3] = __builtin_bit_cast(uint32_t, p3);
                *reinterpret_cast<u32x4 *>(&Bs[buf][mxcol][8 * lds_chunk(mxcol, d)]) = v;
            }
        } else {
            if ((ks * 32) % g == 0) decode_group<SD>(S.graw, gc);
            float q[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) decode_codes(S.wd[i], q[i]);
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                uint2 v;
                v.x = pack_bf16(coeff<SD>(q[0][sl], gc, sl), coeff<SD>(q[1][sl], gc, sl));
                v.y = pack_bf16(coeff<SD>(q[2][sl], gc, sl), coeff<SD>(q[3][sl], gc, sl));
                const int L = kSlotCol[sl] * kUnits + u;
                *reinterpret_cast<uint2 *>(&Bs[buf][L][8 * lds_chunk(L, kq >> 1) + 4 * (kq & 1)]) = v;
            }
        }
    };

    // ---- accumulators: 4 row tiles x 8 column tiles per wave
    f32x4 acc[4][8];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wrow0 = m0 + wm * 64;
    int rtn = (m1 - wrow0 + 15) / 16;  // active row tiles of this wave
    rtn = rtn < 0 ? 0 : (rtn > 4 ? 4 : rtn);
    // Column tiles of wave wn: logical columns 4wn..4wn+3 of every word, for the
    // 16 gate units then the 16 up units (tile ct and ct + 4 pair up), or for
    // all 32 units of a single cube.
    // MXFP4 gate/up: LDS columns [0,128) gate features, [128,256) up features;
    // wave wn takes features 64wn..64wn+63 of both halves.  MXFP4 single bank:
    // columns 128wn..128wn+127.
    auto bcol = [&](int ct) {
        if (MX) return NSETS == 2 ? (ct >> 2) * 128 + wn * 64 + (ct & 3) * 16 : wn * 128 + ct * 16;
        return (4 * wn + (ct & 3)) * kUnits + (ct >> 2) * 16;
    };

    auto mfma_step = [&](int buf) {
        if (rtn == 0) return;
        bf16x8 af[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            if (rt < rtn)
                af[rt] = *reinterpret_cast<const bf16x8 *>(
                    &As[buf][wm * 64 + rt * 16 + c][8 * lds_chunk(c, grp)]);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const bf16x8 bf =
                *reinterpret_cast<const bf16x8 *>(&Bs[buf][bcol(ct) + c][8 * lds_chunk(c, grp)]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                if (rt < rtn)
                    acc[rt][ct] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt], bf, acc[rt][ct], 0, 0, 0);
        }
    };

    // Pipeline: step ks computes from LDS buffer ks % 2 while step ks+1 (loaded
    // two iterations ago) is dequantised into the other buffer and steps ks+2,
    // ks+3 are in flight; the loop is unrolled by two so each register stage is
    // a fixed set.
    load_step(st[0], 0);
    load_step(st[1], 1);
    store_step(st[0], 0, 0);
    load_step(st[0], 2);
    lds_barrier();
    for (int ks = 0; ks < nsteps; ks += 2) {
        mfma_step(0);
        if (ks + 1 < nsteps) store_step(st[1], ks + 1, 1);
        load_step(st[1], ks + 3);
        lds_barrier();
        if (ks + 1 >= nsteps) break;
        mfma_step(1);
        if (ks + 2 < nsteps) store_step(st[0], ks + 2, 0);
        load_step(st[0], ks + 4);
        lds_barrier();
    }

    // ---- epilogue: bias, storage rounding, SwiGLU; LDS column -> output column
#pragma unroll
    for (int ct = 0; ct < (NSETS == 2 ? 4 : 8); ++ct) {
        const int L = bcol(ct) + c;  // gate (or single-cube) LDS column
        int n;
        if (MX) {
            n = NSETS == 2 ? nt * 128 + L : nt * 256 + L;
        } else {
            const int uu = L & (kUnits - 1), cc = L / kUnits;
            n = 8 * (NSETS == 2 ? nt * 16 + uu : nt * kUnits + uu) + cc;
        }
        if (MX && n >= a.Nout) continue;  // partial n-tile
        float b0 = 0.f, b1 = 0.f;
        if (MX) {
            const __bf16 *bb = static_cast<const __bf16 *>(a.bias[0]) + (size_t)e * a.R;
            if (NSETS == 2) {
                b0 = (float)bb[2 * n];
                b1 = (float)bb[2 * n + 1];
            } else {
                b0 = (float)bb[n];
            }
        } else {
            if (a.bias[0]) b0 = load_f<SD>(a.bias[0], (size_t)e * N + n);
            if (NSETS == 2 && a.bias[1]) b1 = load_f<SD>(a.bias[1], (size_t)e * N + n);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (rt >= rtn) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wrow0 + rt * 16 + grp * 4 + i;
                if (row >= m1) continue;
                float v;
                if (NSETS == 2) {
                    const float gv = round_to<MOEQ_BF16>(acc[rt][ct][i] + b0);
                    const float uv = round_to<MOEQ_BF16>(acc[rt][ct + 4][i] + b1);
                    v = swiglu_f(gv, uv, a.clamp, a.gate_lo, a.alpha, a.up_offset);
                } else {
                    v = acc[rt][ct][i] + b0;
                }
                a.out[(size_t)row * a.Nout + n] = (__bf16)v;
            }
        }
    }
}

template <int FMT, int NSETS>
hipError_t run_tile(const ProjProblem &p, const int32_t *tile_offsets, const int32_t *tile_expert,
                    hipStream_t s) {
    TileArgs a{};
    a.in = static_cast<const __bf16 *>(p.in);
    a.out = static_cast<__bf16 *>(p.out);
    a.offsets = p.offsets;
    a.tile_offsets = tile_offsets;
    a.tile_expert = tile_expert;
    a.E = p.E;
    a.K = p.w0.K;
    a.W = p.w0.N / 8;
    a.g = p.w0.g;
    a.R = p.w0.N;
    a.Nout = p.Nout;
    if (FMT == MOEQ_FMT_MXFP4_BANK)
        a.ntiles = (a.R + 255) / 256;  // 256 bank rows per block
    else
        a.ntiles = NSETS == 2 ? a.W / 16 : a.W / kUnits;
    const PackedOperand *ops[2] = {&p.w0, &p.w1};
    for (int i = 0; i < 2; ++i) {
        a.qw[i] = reinterpret_cast<const uint32_t *>(ops[i]->qw);
        a.qz[i] = reinterpret_cast<const uint32_t *>(ops[i]->qz);
        a.sc[i] = ops[i]->scales;
        a.bias[i] = ops[i]->bias;
    }
    a.clamp = p.clamp;
    a.gate_lo = p.gate_lo;
    a.alpha = p.alpha;
    a.up_offset = p.up_offset;
    // m-tiles are at most ceil(A / 128) + E; blocks past the last tile exit
    const long mtiles = ((long)p.rows + kBM - 1) / kBM + p.E;
    const long blocks = ((mtiles + 7) / 8) * 8 * a.ntiles;
    if (FMT == MOEQ_FMT_MXFP4_BANK) {
        hipLaunchKernelGGL((awq_tile_kernel<FMT, NSETS, MOEQ_BF16>), dim3((unsigned)blocks),
                           dim3(256), 0, s, a);
        return hipGetLastError();
    }
    switch (p.w0.sdt) {
    case MOEQ_BF16:
        hipLaunchKernelGGL((awq_tile_kernel<FMT, NSETS, MOEQ_BF16>), dim3((unsigned)blocks),
                           dim3(256), 0, s, a);
        break;
    case MOEQ_F16:
        hipLaunchKernelGGL((awq_tile_kernel<FMT, NSETS, MOEQ_F16>), dim3((unsigned)blocks),
                           dim3(256), 0, s, a);
        break;
    default:
        hipLaunchKernelGGL((awq_tile_kernel<FMT, NSETS, MOEQ_F32>), dim3((unsigned)blocks),
                           dim3(256), 0, s, a);
        break;
    }
    return hipGetLastError();
}

}  // namespace

// Tiled path: bf16 activations; AWQ with full 256-column tiles and whole
// 32-row steps, or an MXFP4 bank (any row count, K a multiple of 32).
bool tile_fits(const ProjProblem &p) {
    if (p.act != MOEQ_BF16 || !p.offsets) return false;
    if (p.w0.format == MOEQ_FMT_MXFP4_BANK)
        return (p.mode == PROJ_BANK_SWIGLU || p.mode == PROJ_PLAIN) && p.w0.K % 32 == 0;
    if (p.w0.format != MOEQ_FMT_AWQ || p.w0.K % 32 != 0 || p.w0.g % 32 != 0) return false;
    const int W = p.w0.N / 8;
    if (p.mode == PROJ_SWIGLU) return W % 16 == 0;
    if (p.mode == PROJ_PLAIN) return W % kUnits == 0;
    return false;
}

hipError_t launch_tile(const ProjProblem &p, const int32_t *tile_offsets,
                       const int32_t *tile_expert, hipStream_t s) {
    if (p.w0.format == MOEQ_FMT_MXFP4_BANK)
        return p.mode == PROJ_BANK_SWIGLU
                   ? run_tile<MOEQ_FMT_MXFP4_BANK, 2>(p, tile_offsets, tile_expert, s)
                   : run_tile<MOEQ_FMT_MXFP4_BANK, 1>(p, tile_offsets, tile_expert, s);
    return p.mode == PROJ_SWIGLU ? run_tile<MOEQ_FMT_AWQ, 2>(p, tile_offsets, tile_expert, s)
                                 : run_tile<MOEQ_FMT_AWQ, 1>(p, tile_offsets, tile_expert, s);
}

}  // namespace moeq
