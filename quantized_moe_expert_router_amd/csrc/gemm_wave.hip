// gemm_wave.hip -- register-decoded bf16 MFMA grouped dequant-GEMM for many
// rows per expert (prefill-shaped batches), gfx950.
//
// packed_experts.rs FrozenPackedExpertOps::packed_swiglu_forward evaluates the
// gate/up/down chain for the assigned experts only; frozen_awq.rs FrozenAwqOps
// fixes each coefficient as (code - zero) * scale rounded to the scale dtype.
//
// Each wave owns 128 rows of one expert (eight 16-row MFMA tiles) and decodes
// its B operands in registers, in the layout of the weight-streaming kernel:
// lane (c, grp) reads the eight words (k0 + 8 grp + i, j) of word column j,
// and nibble slot sl of those words is one complete 16x16x32 B operand for
// output column 8 j + kSlotCol[sl].  A wave takes one nibble plane of the
// words -- the low nibbles (slots 0-3) or the high nibbles (slots 4-7) -- so
// one decoded operand feeds eight MFMAs and the accumulators are 4 x 8 fp32
// tiles (128 registers).  Two waves run per SIMD: one wave's dequant VALU
// work runs while the other's MFMAs occupy the matrix core.
//
// The eight waves of a block share the A tile (128 rows x 32 k per step): all
// 512 threads load it DEPTH steps ahead into registers and store it into a
// double-buffered LDS tile of 64-byte rows whose 16-byte chunks are permuted by
// chunk ^ ((row >> 1) & 3) -- measured on gfx950, that makes the MFMA fragment
// reads (16 rows x one chunk per 16 lanes) run at the full 256 bytes per clock,
// twice the rate of padded rows; one LDS-only barrier per step keeps the
// global prefetch in flight across it.
//
// Wave roles.  Single cube: (column group, plane).  gate/up: (column group,
// plane, cube); the gate and up waves of one (group, plane) cover the same
// logical columns, every operand address stays wave-uniform (buffer resources,
// scalar offsets), and at the end the up wave leaves its storage-rounded U
// tile in LDS in its accumulator layout for the gate wave.
//
// Blocks: one m-tile (128 rows of one expert) x the column groups of its
// waves.  The m-tiles are split into eight contiguous ranges, one per XCD
// (block b runs on XCD b % 8), so consecutive m-tiles of an expert reuse its
// weights from that XCD's L2, and the column blocks of an m-tile share its
// rows there.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <type_traits>

#include "awq_dequant.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

using namespace awq;

constexpr int kWaveRows = 128;  // rows per wave task = one m-tile
constexpr int kWaves = 8;       // waves per block (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kRT = kWaveRows / 16;

struct WaveArgs {
    const __bf16 *in;  // [A, K] rows sorted by expert
    __bf16 *out;       // [A, Nout]
    const int32_t *offsets;
    const int32_t *tile_offsets;
    const int32_t *tile_expert;
    int E, K, W, g;
    int groups;  // 128-column groups (16 word columns)
    int nblk;    // blocks per m-tile
    int min_rows;  // > 0: experts with at most this many rows are left to another kernel
    int Nout;
    const uint32_t *qw[2];
    const uint32_t *qz[2];
    const void *sc[2];
    const void *bias[2];
    float clamp, alpha, up_offset;
    float gate_lo;  // lower clamp bound of the gate
    const __bf16 *dh;  // backward epilogue: [A, Nout] derivative of h (NULL: forward)
    __bf16 *out2;      // backward epilogue: dU (out holds dG)
    int vec_out;       // 1: out 16-byte aligned and Nout % 8 == 0 (one-cube 16-byte stores)
};

// After the main loop: gate/up -- every wave's storage-rounded tile (G or U),
// [wave][slot, row tile][lane] (the backward epilogue: the up waves' U tiles);
// one cube -- the halves of the plane waves' tiles that they swap.
template <int NSETS>
struct WaveLds {
    __bf16 A[2][kWaveRows][32];                                 // A tile, double-buffered
    uint2 U[NSETS == 2 ? kWaves : kWaves / 2][4 * kRT][64];
};

template <int NSETS, int SD, int SPG, int DEPTH, bool BWD>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void awq_wave_kernel(WaveArgs a) {
    constexpr int RT = kRT;
    constexpr int sb = SD == MOEQ_F32 ? 4 : 2;
    static_assert(SPG % DEPTH == 0, "ring must tile a group");
    __shared__ __attribute__((aligned(16))) WaveLds<NSETS> lds;

    // ---- block -> (m-tile, column block); contiguous m-tile ranges per XCD
    const int mtiles = a.tile_offsets[a.E];
    const int per_xcd = (mtiles + 7) / 8;
    const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int local = idx / a.nblk, nb = idx % a.nblk;
    const int mt = x * per_xcd + local;
    if (local >= per_xcd || mt >= mtiles) return;

    // ---- wave role (wave-uniform)
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int set = NSETS == 2 ? (wv & 1) : 0;
    const int plane = NSETS == 2 ? ((wv >> 1) & 1) : (wv & 1);
    const int cg = NSETS == 2 ? nb * (kWaves / 4) + (wv >> 2) : nb * (kWaves / 2) + (wv >> 1);
    const bool active = cg < a.groups;  // inactive waves still load A and meet every barrier
    const int e = a.tile_expert[mt];
    if (a.offsets[e + 1] - a.offsets[e] <= a.min_rows) return;  // a light expert: streamed
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kWaveRows;
    const int m1 = min(m0 + kWaveRows, a.offsets[e + 1]);

    const int lane = threadIdx.x & 63;
    const int c = lane & 15, grp = lane >> 4;
    const int j = cg * 16 + c;  // word column
    const int K = a.K, W = a.W, N = W * 8, g = a.g, G = K / g;

    const __amdgpu_buffer_rsrc_t rw =
        buffer_rsrc(a.qw[set] + (size_t)e * K * W, (size_t)K * W * 4);
    const __amdgpu_buffer_rsrc_t rz =
        buffer_rsrc(a.qz[set] + (size_t)e * G * W, (size_t)G * W * 4);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
        static_cast<const char *>(a.sc[set]) + (size_t)e * G * N * sb, (size_t)G * N * sb);
    const int voff_w = active ? (grp * 8 * W + j) * 4 : 0x40000000;  // inactive: zeros
    const int voff_z = j * 4, voff_s = 8 * j * sb;

    // cooperative A loads: thread t loads row t / 4, k chunk t % 4 (8 bf16) of
    // each step; rows past the end read zeros
    const int tid = threadIdx.x;
    const int arow = tid >> 2, achk = tid & 3;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.in, (size_t)m1 * K * 2);
    const int voff_a = m0 + arow < m1 ? ((m0 + arow) * K + 8 * achk) * 2 : 0x7fffffff;

    f32x4 acc[4][RT];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[s4][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    {
        uint32_t wd[DEPTH][8];
        u32x4 ar[DEPTH];
        auto issue_words = [&](int d, int kk) {
            const int so = min(kk, K - 32) * W * 4;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wd[d][i] = __builtin_amdgcn_raw_buffer_load_b32(rw, voff_w, so + i * W * 4, 0);
        };
        auto issue_rows = [&](int d, int kk) {
            ar[d] = __builtin_amdgcn_raw_buffer_load_b128(ra, voff_a, min(kk, K - 32) * 2, 0);
        };
        auto store_rows = [&](int d, int buf) {
            *reinterpret_cast<u32x4 *>(&lds.A[buf][arow][8 * (achk ^ ((arow >> 1) & 3))]) = ar[d];
        };
        GroupRaw<SD> graw;
        GroupConst<SD> gc;
        // step s: A fragments from lds.A[s & 1]; words from ring slot d = s % DEPTH
        auto step = [&](int s, int d) {
            const int buf = s & 1;
            uint32_t pl[8];  // this wave's nibble plane of the eight words
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pl[i] = and_opaque(plane ? (wd[d][i] >> 4) : wd[d][i], 0x0F0F0F0Fu);
            issue_words(d, 32 * (s + DEPTH));  // the words are dead: refill this slot
            // next step's A tile into the other buffer, then refill its slot
            const int dn = (d + 1) % DEPTH;
            store_rows(dn, buf ^ 1);
            issue_rows(dn, 32 * (s + 1 + DEPTH));
            // the four B operands of the step first, then the row tiles one by
            // one, each A fragment read from LDS just before its four MFMAs: a
            // few fragments live at a time instead of eight keeps the kernel
            // within two waves' registers (no spill, so no wait on the whole
            // load ring for a spill reload)
            bf16x8 bop[4];
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                f32x2 qv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    qv[i] = pr ? __builtin_amdgcn_cvt_pk_f32_fp8(pl[i], true)
                               : __builtin_amdgcn_cvt_pk_f32_fp8(pl[i], false);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int s4 = 2 * pr + h;  // slot 4 * plane + s4
                    u32x4 op;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        op[p] = pack_bf16(coeff<SD>(qv[2 * p][h], gc, s4),
                                          coeff<SD>(qv[2 * p + 1][h], gc, s4));
                    bop[s4] = __builtin_bit_cast(bf16x8, op);
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const bf16x8 af = *reinterpret_cast<const bf16x8 *>(
                    &lds.A[buf][rt * 16 + c][8 * (grp ^ ((c >> 1) & 3))]);
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4)
                    acc[s4][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bop[s4],
                                                                          acc[s4][rt], 0, 0, 0);
            }
            lds_barrier();
        };

        // group constants of this wave's four slots (GroupConst slots 0-3)
        auto decode_plane = [&] {
            GroupConst<SD> full;
            decode_group<SD>(graw, full);
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                gc.s[s4] = plane ? full.s[4 + s4] : full.s[s4];
                gc.zs[s4] = plane ? full.zs[4 + s4] : full.zs[s4];
            }
        };

        load_group_raw<SD>(rz, rs, voff_z, voff_s, 0, W, N, graw);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            issue_words(d, 32 * d);
            issue_rows(d, 32 * d);
        }
        store_rows(0, 0);
        issue_rows(0, 32 * DEPTH);
        lds_barrier();
        for (int gi = 0; gi < G; ++gi) {
            decode_plane();
#pragma unroll
            for (int t = 0; t < SPG; ++t) {
                if (t == SPG - DEPTH || (DEPTH >= SPG && t == 0)) {
                    // next group's constants, decoded at least one step from now
                    load_group_raw<SD>(rz, rs, voff_z, voff_s, gi + 1 < G ? gi + 1 : gi, W, N,
                                       graw);
                }
                step(gi * SPG + t, t % DEPTH);
            }
        }
    }

    // ---- epilogue: bias, storage rounding, SwiGLU.  Lane (c, grp) holds, for
    // slot s4 and row tile rt, rows 16 rt + 4 grp + i of column
    // 8 j + kSlotCol[4 plane + s4]: columns 8 j + 2 plane + {0, 1} come from
    // slots (0, 2) and columns 8 j + 4 + 2 plane + {0, 1} from slots (1, 3).
    const int col0 = 8 * j + 2 * plane;
    float bias_v[4];  // by slot
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
        const int col = 8 * j + kSlotCol[4 * plane + s4];
        bias_v[s4] = (active && a.bias[set]) ? load_f<SD>(a.bias[set], (size_t)e * N + col) : 0.0f;
    }
    const int rtn = (m1 - m0 + 15) >> 4;  // row tiles holding rows
    if constexpr (NSETS == 2) {
        if (a.vec_out) {
            // Every wave leaves its tile, bias added and rounded to storage (G or
            // U), in LDS.  Wave (column group, plane p, set s) then finishes row
            // tiles 2(2p + s) and 2(2p + s) + 1 for all eight columns of its
            // lanes' word columns, and stores each row's eight as one 16 bytes
            // (backward: reads dh and stores dG and dU the same way).
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const f32x4 v = acc[s4][rt];
                    const float b = bias_v[s4];
                    lds.U[wv][s4 * RT + rt][lane] =
                        uint2{pack_bf16(v[0] + b, v[1] + b), pack_bf16(v[2] + b, v[3] + b)};
                }
            __syncthreads();
            if (!active) return;
            const int w0 = wv & ~3;  // wave (column group, plane 0, gate)
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int rt = 2 * (wv & 3) + r2;
                if (rt >= rtn) continue;
                float gq[8][4], uq[8][4];  // [column of the word column][row i]
#pragma unroll
                for (int col = 0; col < 8; ++col) {
                    // column col sits in slot sl = 2 (col & 3) + (col >> 2) of the
                    // words: nibble plane sl >> 2, plane slot sl & 3
                    const int sl = 2 * (col & 3) + (col >> 2);
                    const int pw = w0 + 2 * (sl >> 2), s4 = sl & 3;
                    const uint2 gg = lds.U[pw][s4 * RT + rt][lane];
                    const uint2 uu = lds.U[pw + 1][s4 * RT + rt][lane];
                    gq[col][0] = __uint_as_float(gg.x << 16);
                    gq[col][1] = __uint_as_float(gg.x & 0xFFFF0000u);
                    gq[col][2] = __uint_as_float(gg.y << 16);
                    gq[col][3] = __uint_as_float(gg.y & 0xFFFF0000u);
                    uq[col][0] = __uint_as_float(uu.x << 16);
                    uq[col][1] = __uint_as_float(uu.x & 0xFFFF0000u);
                    uq[col][2] = __uint_as_float(uu.y << 16);
                    uq[col][3] = __uint_as_float(uu.y & 0xFFFF0000u);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + rt * 16 + grp * 4 + i;
                    if (row >= m1) continue;
                    const size_t at = (size_t)row * a.Nout + 8 * j;
                    if constexpr (BWD) {
                        const u32x4 dw = *reinterpret_cast<const u32x4 *>(a.dh + at);
                        float dg[8], du[8];
#pragma unroll
                        for (int col = 0; col < 8; ++col) {
                            const uint32_t pr2 = dw[col >> 1];
                            const float dv = __uint_as_float((col & 1) ? (pr2 & 0xFFFF0000u)
                                                                       : (pr2 << 16));
                            swiglu_vjp_f(gq[col][i], uq[col][i], dv, a.clamp, a.gate_lo, a.alpha,
                                         a.up_offset, &dg[col], &du[col]);
                        }
                        *reinterpret_cast<u32x4 *>(a.out + at) =
                            u32x4{pack_bf16(dg[0], dg[1]), pack_bf16(dg[2], dg[3]),
                                  pack_bf16(dg[4], dg[5]), pack_bf16(dg[6], dg[7])};
                        *reinterpret_cast<u32x4 *>(a.out2 + at) =
                            u32x4{pack_bf16(du[0], du[1]), pack_bf16(du[2], du[3]),
                                  pack_bf16(du[4], du[5]), pack_bf16(du[6], du[7])};
                    } else {
                        float h[8];
#pragma unroll
                        for (int col = 0; col < 8; ++col)
                            h[col] = swiglu_f(gq[col][i], uq[col][i], a.clamp, a.gate_lo, a.alpha,
                                              a.up_offset);
                        *reinterpret_cast<u32x4 *>(a.out + at) =
                            u32x4{pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3]),
                                  pack_bf16(h[4], h[5]), pack_bf16(h[6], h[7])};
                    }
                }
            }
            return;
        }
    }
    if constexpr (NSETS == 2) {
        const int pair = wv >> 1;  // (column group, plane)
        // backward: the gate waves fetch their dh pairs before the U hand-off
        // (rows past the tile reread the last row; those results are not stored)
        uint32_t dpre[BWD ? RT : 1][4][2];
        if constexpr (BWD) {
            if (active && set == 0) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = min(m0 + rt * 16 + grp * 4 + i, m1 - 1);
                        const uint32_t *dp =
                            reinterpret_cast<const uint32_t *>(a.dh + (size_t)row * a.Nout + col0);
                        dpre[rt][i][0] = dp[0];
                        dpre[rt][i][1] = dp[2];
                    }
            }
        }
        if (active && set == 1) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (rt >= rtn) continue;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const f32x4 v = acc[s4][rt];
                    const float b = bias_v[s4];
                    lds.U[pair][s4 * RT + rt][lane] =
                        uint2{pack_bf16(v[0] + b, v[1] + b), pack_bf16(v[2] + b, v[3] + b)};
                }
            }
        }
        __syncthreads();
        if (!active || set == 1) return;
        if constexpr (BWD) {
            // backward: dG into out, dU into out2, at the rounded G, U.  The dh pair
            // at col0 holds slots (0, 2), the pair at col0 + 4 slots (1, 3).
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (rt >= rtn) continue;
                float gvv[4][4], uvv[4][4];  // [slot][row i]
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const uint2 u = lds.U[pair][s4 * RT + rt][lane];
                    uvv[s4][0] = __uint_as_float(u.x << 16);
                    uvv[s4][1] = __uint_as_float(u.x & 0xFFFF0000u);
                    uvv[s4][2] = __uint_as_float(u.y << 16);
                    uvv[s4][3] = __uint_as_float(u.y & 0xFFFF0000u);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        gvv[s4][i] = round_to<MOEQ_BF16>(acc[s4][rt][i] + bias_v[s4]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + rt * 16 + grp * 4 + i;
                    if (row >= m1) continue;
                    const size_t at = (size_t)row * a.Nout + col0;
                    const uint32_t d02 = dpre[rt][i][0], d13 = dpre[rt][i][1];
                    const float dv[4] = {__uint_as_float(d02 << 16), __uint_as_float(d13 << 16),
                                         __uint_as_float(d02 & 0xFFFF0000u),
                                         __uint_as_float(d13 & 0xFFFF0000u)};
                    float dg[4], du[4];
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4)
                        swiglu_vjp_f(gvv[s4][i], uvv[s4][i], dv[s4], a.clamp, a.gate_lo, a.alpha,
                                     a.up_offset, &dg[s4], &du[s4]);
                    uint32_t *o = reinterpret_cast<uint32_t *>(a.out + at);
                    uint32_t *o2 = reinterpret_cast<uint32_t *>(a.out2 + at);
                    o[0] = pack_bf16(dg[0], dg[2]);
                    o[2] = pack_bf16(dg[1], dg[3]);
                    o2[0] = pack_bf16(du[0], du[2]);
                    o2[2] = pack_bf16(du[1], du[3]);
                }
            }
            return;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt >= rtn) continue;
            float hv[4][4];  // [row i][slot]
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const uint2 u = lds.U[pair][s4 * RT + rt][lane];
                const float uv[4] = {__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gv = round_to<MOEQ_BF16>(acc[s4][rt][i] + bias_v[s4]);
                    hv[i][s4] = swiglu_f(gv, uv[i], a.clamp, a.gate_lo, a.alpha, a.up_offset);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + rt * 16 + grp * 4 + i;
                if (row >= m1) continue;
                uint32_t *o = reinterpret_cast<uint32_t *>(a.out + (size_t)row * a.Nout + col0);
                o[0] = pack_bf16(hv[i][0], hv[i][2]);
                o[2] = pack_bf16(hv[i][1], hv[i][3]);
            }
        }
    } else if (a.vec_out) {
        // The two plane waves of a column group hold columns {0,1,4,5} and
        // {2,3,6,7} of each word column's eight.  Each sends the other the
        // rows of half its row tiles (plane 0 keeps tiles 0-3, plane 1 tiles
        // 4-7) through LDS, then stores whole 16-byte chunks of its rows.
        const int pr = wv >> 1;  // column group within the block
        auto pack_row = [&](int rt_, int i) {  // {cols 2p,2p+1 ; cols 4+2p,5+2p}
            float v[4];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) v[s4] = acc[s4][rt_][i] + bias_v[s4];
            return uint2{pack_bf16(v[0], v[2]), pack_bf16(v[1], v[3])};
        };
        auto swap_store = [&](auto plane_tag) {
            constexpr int PL = decltype(plane_tag)::value;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lds.U[pr][PL * 16 + r4 * 4 + i][lane] = pack_row(PL ? r4 : 4 + r4, i);
            __syncthreads();
            if (!active) return;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int rt = PL ? 4 + r4 : r4;
                if (rt >= rtn) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + rt * 16 + grp * 4 + i;
                    if (row >= m1) continue;
                    const uint2 own = pack_row(rt, i);
                    const uint2 oth = lds.U[pr][(1 - PL) * 16 + r4 * 4 + i][lane];
                    const u32x4 pk = PL ? u32x4{oth.x, own.x, oth.y, own.y}
                                        : u32x4{own.x, oth.x, own.y, oth.y};
                    *reinterpret_cast<u32x4 *>(a.out + (size_t)row * a.Nout + 8 * j) = pk;
                }
            }
        };
        if (plane)
            swap_store(std::integral_constant<int, 1>{});
        else
            swap_store(std::integral_constant<int, 0>{});
    } else {
        if (!active) return;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt >= rtn) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + rt * 16 + grp * 4 + i;
                if (row >= m1) continue;
                float v[4];
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) v[s4] = acc[s4][rt][i] + bias_v[s4];
                uint32_t *o = reinterpret_cast<uint32_t *>(a.out + (size_t)row * a.Nout + col0);
                o[0] = pack_bf16(v[0], v[2]);
                o[2] = pack_bf16(v[1], v[3]);
            }
        }
    }
}

template <int NSETS, int SD>
hipError_t run_wave(const ProjProblem &p, hipStream_t s) {
    WaveArgs a{};
    a.in = static_cast<const __bf16 *>(p.in);
    a.out = static_cast<__bf16 *>(p.out);
    a.offsets = p.offsets;
    a.tile_offsets = p.tile_offsets;
    a.min_rows = p.split_rows;
    a.tile_expert = p.tile_expert;
    a.E = p.E;
    a.K = p.w0.K;
    a.W = p.w0.N / 8;
    a.g = p.w0.g;
    a.Nout = p.Nout;
    a.groups = a.W / 16;  // 16 word columns per wave
    const int per_blk = NSETS == 2 ? kWaves / 4 : kWaves / 2;  // column groups per block
    a.nblk = (a.groups + per_blk - 1) / per_blk;
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
    a.dh = static_cast<const __bf16 *>(p.in2);
    a.out2 = static_cast<__bf16 *>(p.out2);
    a.vec_out = (((uintptr_t)p.out | (uintptr_t)p.out2 | (uintptr_t)p.in2) % 16) == 0 &&
                p.Nout % 8 == 0;
    // m-tiles are at most ceil(A / 128) + E; blocks past the last tile exit
    const long mtiles = ((long)p.rows + kWaveRows - 1) / kWaveRows + p.E;
    const long blocks = 8 * ((mtiles + 7) / 8) * a.nblk;
    const int spg = a.g / 32;
    // the backward epilogue is a separate instantiation: the forward kernel stays as it is
    const bool bwd = NSETS == 2 && a.dh;
    if (spg == 4) {
        if (bwd)
            hipLaunchKernelGGL((awq_wave_kernel<NSETS, SD, 4, 2, NSETS == 2>),
                               dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((awq_wave_kernel<NSETS, SD, 4, 2, false>), dim3((unsigned)blocks),
                               dim3(kThreads), 0, s, a);
    } else {
        if (bwd)
            hipLaunchKernelGGL((awq_wave_kernel<NSETS, SD, 2, 2, NSETS == 2>),
                               dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
        else
            hipLaunchKernelGGL((awq_wave_kernel<NSETS, SD, 2, 2, false>), dim3((unsigned)blocks),
                               dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace

// Register-decoded path: bf16 activations, AWQ with 16-bit scales, group 64
// or 128, whole 128-column groups.
bool wave_fits(const ProjProblem &p) {
    if (const char *v = getenv("MOEQ_WAVE")) {  // tuning override: 0 disables
        if (atoi(v) == 0) return false;
    }
    if (p.act != MOEQ_BF16 || p.w0.format != MOEQ_FMT_AWQ || !p.offsets || !p.tile_offsets)
        return false;
    if (p.w0.g != 64 && p.w0.g != 128) return false;
    if (p.w0.sdt == MOEQ_F32) return false;  // fp32 scales: the warp-specialised kernel is faster
    if (p.w0.K % p.w0.g != 0) return false;
    if ((size_t)p.rows * p.w0.K * 2 >= ((size_t)1 << 31)) return false;  // 32-bit row offsets
    if (p.mode != PROJ_SWIGLU && p.mode != PROJ_PLAIN) return false;
    return (p.w0.N / 8) % 16 == 0;
}

hipError_t launch_wave(const ProjProblem &p, hipStream_t s) {
    const bool two = p.mode == PROJ_SWIGLU;
    switch (p.w0.sdt) {
    case MOEQ_BF16: return two ? run_wave<2, MOEQ_BF16>(p, s) : run_wave<1, MOEQ_BF16>(p, s);
    case MOEQ_F16: return two ? run_wave<2, MOEQ_F16>(p, s) : run_wave<1, MOEQ_F16>(p, s);
    default: return two ? run_wave<2, MOEQ_F32>(p, s) : run_wave<1, MOEQ_F32>(p, s);
    }
}

}  // namespace moeq
