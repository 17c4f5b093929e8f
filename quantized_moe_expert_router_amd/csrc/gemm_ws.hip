// gemm_ws.hip -- warp-specialised bf16 MFMA grouped dequant-GEMM for many rows
// per expert (prefill-shaped batches), gfx950.
//
// packed_experts.rs FrozenPackedExpertOps::packed_swiglu_forward evaluates the
// gate/up/down chain for the assigned experts only; frozen_awq.rs FrozenAwqOps
// fixes each coefficient as (code - zero) * scale rounded to the scale dtype.
//
// Measured on gfx950: one wave issuing independent MFMAs reaches only about
// half of a SIMD's matrix rate; two waves issuing MFMAs together reach it, and
// a third wave's VALU work co-executes with them.  So a block has 12 waves,
// three per SIMD:
//   * 8 consumer waves (2 x 4) only read fragments from LDS and issue MFMAs;
//   * 4 producer waves load the A tile (128 rows x 32 k) and the packed words
//     of the block's 64 word columns three K steps ahead into a register
//     ring, store the A tile and decode the words -- (code - zero) * scale
//     rounded to the scale dtype, as bf16 -- into the other half of
//     double-buffered LDS tiles.  One barrier per 32-row K step.
//     Every step issues the same loads unconditionally (the group constants
//     are reloaded each step into a staging copy, past-the-end steps load
//     clamped data nobody reads), so the compiler's wait counts stay exact
//     across the loop and the ring stays in flight.
// Block tile: one 128-row m-tile x 64 word columns (512 logical columns): for
// gate/up 32 word columns of each cube (256 logical columns, paired for
// SwiGLU in the consumers' registers), for one cube 64 word columns.
//
// LDS rows are 64 bytes (32 k of one A row or one B column) with their 16-byte
// chunks at chunk ^ ((row >> 1) & 3): measured conflict-free for the
// fragment reads.  B column of (cube, word column wc, slot sl) is
// cube * 256 + sl * 32 + wc (gate/up) or sl * 64 + wc (one cube): a 16-column
// MFMA tile is 16 consecutive word columns of one nibble slot.
//
// Blocks: m-tiles dealt round-robin to the eight XCDs (block b runs on XCD
// b % 8), so a heavy expert's m-tiles spread over all of them.  Contiguous
// ranges per XCD (an expert's m-tiles sharing one L2) were 5% slower on the
// many-expert workload, where a few experts hold most rows.  The m-tiles are
// taken in the route's scheduling order: every full tile first, the partial
// ones (light experts, ragged ends) after, so the longest blocks start first
// and the short ones fill in behind them.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <type_traits>

#include "awq_dequant.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

using namespace awq;

constexpr int kRows = 128;           // m-tile rows
constexpr int kCons = 8;             // consumer waves (2 row halves x 4 column quarters)
constexpr int kProd = 4;             // producer waves
constexpr int kThreads = 64 * (kCons + kProd);
constexpr int kWc = 64;              // word columns per block
constexpr int kBCols = kWc * 8;      // LDS B columns per stage
constexpr int kDepth = 3;            // register ring of A rows and packed words (steps)

struct WsArgs {
    const __bf16 *in;  // [A, K] rows sorted by expert
    __bf16 *out;       // [A, Nout]
    const int32_t *offsets;
    const int32_t *tile_offsets;
    const int32_t *tile_expert;
    const int32_t *tile_order;  // nullable: m-tiles in scheduling order (full ones first)
    int E, K, W, g;
    int nblk;  // blocks per m-tile
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
    int vec_out;       // 1: out 16-byte aligned and Nout % 8 == 0 (staged 16-byte stores)
};

__device__ __forceinline__ int lds_chunk(int row, int ch) { return ch ^ ((row >> 1) & 3); }

template <int NSETS, int SD>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(3, 3)))
void awq_ws_kernel(WsArgs a) {
    constexpr int sb = SD == MOEQ_F32 ? 4 : 2;
    // double-buffered A and B tiles (64-byte rows, permuted chunks)
    __shared__ __attribute__((aligned(16))) __bf16 As[2][kRows][32];     // 16 KiB
    __shared__ __attribute__((aligned(16))) __bf16 Bs[2][kBCols][32];    // 64 KiB

    // ---- block -> (m-tile, column block); m-tile mt runs on XCD mt % 8
    const int mtiles = a.tile_offsets[a.E];
    const int per_xcd = (mtiles + 7) / 8;
    const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int local = idx / a.nblk, nb = idx % a.nblk;
    const int slot = local * 8 + x;
    if (local >= per_xcd || slot >= mtiles) return;
    // full m-tiles start first, partial ones after (longest first)
    const int mt = a.tile_order ? a.tile_order[slot] : slot;
    const int e = a.tile_expert[mt];
    if (a.offsets[e + 1] - a.offsets[e] <= a.min_rows) return;  // a light expert: streamed
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kRows;
    const int m1 = min(m0 + kRows, a.offsets[e + 1]);
    const int K = a.K, W = a.W, N = W * 8, g = a.g, G = K / g;
    const int nsteps = K / 32;

    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, grp = lane >> 4;

    if (wv >= kCons) {
        // =================================================== producer waves
        const int pw = wv - kCons, pt = pw * 64 + lane;  // producer thread 0..255
        // words: thread (cube, wc, kq) decodes the eight words k = 8 kq .. 8 kq + 7
        // of word column wc; gate/up: waves 0,1 gate, 2,3 up (32 word columns)
        const int cube = NSETS == 2 ? (pw >> 1) : 0;
        const int wc = NSETS == 2 ? (lane & 31) : lane;
        const int kq = NSETS == 2 ? ((pw & 1) * 2 + (lane >> 5)) : pw;
        const int jcol = nb * (NSETS == 2 ? kWc / 2 : kWc) + wc;  // word column in the cube
        const bool on = jcol < W;
        const __amdgpu_buffer_rsrc_t rz =
            buffer_rsrc(a.qz[cube] + (size_t)e * G * W, (size_t)G * W * 4);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
            static_cast<const char *>(a.sc[cube]) + (size_t)e * G * N * sb, (size_t)G * N * sb);
        const int voff_z = on ? jcol * 4 : 0x40000000;
        const int voff_s = on ? 8 * jcol * sb : 0x40000000;
        const __amdgpu_buffer_rsrc_t rw =
            buffer_rsrc(a.qw[cube] + (size_t)e * K * W, (size_t)K * W * 4);
        const int voff_w = on ? (kq * 8 * W + jcol) * 4 : 0x40000000;
        // A tile: chunks pt and pt + 256 of 512 (row u / 4, k chunk u % 4)
        const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.in, (size_t)m1 * K * 2);
        int voff_a[2], arow[2], achk[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int u = pt + 256 * h;
            arow[h] = u >> 2;
            achk[h] = u & 3;
            const int row = m0 + arow[h];
            voff_a[h] = row < m1 ? (row * K + 8 * achk[h]) * 2 : 0x7fffffff;
        }
        uint32_t wd[kDepth][8];
        u32x4 ar[kDepth][2];
        GroupRaw<SD> gr[kDepth];  // constants of the step's group
        // A rows, words and group constants of step q into ring slot d
        auto issue = [&](int d, int q) {
            const int ks = min(q, nsteps - 1);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wd[d][i] = __builtin_amdgcn_raw_buffer_load_b32(rw, voff_w, (ks * 32 + i) * W * 4, 0);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                ar[d][h] = __builtin_amdgcn_raw_buffer_load_b128(ra, voff_a[h], ks * 64, 0);
            load_group_raw<SD>(rz, rs, voff_z, voff_s, ks * 32 / g, W, N, gr[d]);
        };
        GroupConst<SD> gc;
        // Step q from ring slot d into LDS buffer q & 1, then refill slot d
        // with step q + kDepth.
        auto produce = [&](int q, auto d_tag) {
            constexpr int d = decltype(d_tag)::value;
            const int buf = q & 1;
            if ((q * 32) % g == 0) decode_group<SD>(gr[d], gc);  // a group starts
#pragma unroll
            for (int h = 0; h < 2; ++h)
                *reinterpret_cast<u32x4 *>(&As[buf][arow[h]][8 * lds_chunk(arow[h], achk[h])]) =
                    ar[d][h];
            uint32_t lo[8], hi[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lo[i] = and_opaque(wd[d][i], 0x0F0F0F0Fu);
                hi[i] = and_opaque(wd[d][i] >> 4, 0x0F0F0F0Fu);
            }
            issue(d, q + kDepth);
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                f32x2 qv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t v = pr < 2 ? lo[i] : hi[i];
                    qv[i] = (pr & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(v, true)
                                     : __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int sl = 2 * pr + hh;
                    u32x4 op;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        op[p] = pack_bf16(coeff<SD>(qv[2 * p][hh], gc, sl),
                                          coeff<SD>(qv[2 * p + 1][hh], gc, sl));
                    const int col = NSETS == 2 ? cube * 256 + sl * 32 + wc : sl * 64 + wc;
                    *reinterpret_cast<u32x4 *>(&Bs[buf][col][8 * lds_chunk(col, kq)]) = op;
                }
            }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;

        // the scheduler must not sink these loads past the first refill: the
        // compiler's wait counts on the loop entry would then assume slot 2
        // was loaded last and wait for it on every trip
        issue(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue(1, 1);
        __builtin_amdgcn_sched_barrier(0);
        issue(2, 2);
        __builtin_amdgcn_sched_barrier(0);
        // step q is produced in iteration q - 1 (step 0 before the loop); the
        // consumers run step q in iteration q.  Steps past the end decode
        // clamped data into a buffer nobody reads, keeping every iteration's
        // loads the same.
        produce(0, I0{});
        lds_barrier();
        int q = 1;
        for (; q + 2 <= nsteps; q += 3) {
            produce(q, I1{});
            lds_barrier();
            produce(q + 1, I2{});
            lds_barrier();
            produce(q + 2, I0{});
            lds_barrier();
        }
        // tail: iterations q - 1 .. nsteps - 1 (at most two), slots 1 then 2
        if (q <= nsteps) {
            produce(q, I1{});
            lds_barrier();
            ++q;
        }
        if (q <= nsteps) {
            produce(q, I2{});
            lds_barrier();
        }
    }

    // ======================================================= consumer waves
    // (the producer waves pass through to the epilogue's barriers)
    const int wm = (wv >> 2) & 1, wn = wv & 3;  // 64-row half, column quarter
    // column tiles: gate/up -- tile t < 4 gate, t + 4 the up tile of the same
    // logical columns (slot 2 wn + (t >> 1), word columns (t & 1) * 16 + c);
    // one cube -- slot 2 wn + (t >> 2), word columns (t & 3) * 16 + c
    auto tcol = [&](int t) {
        if (NSETS == 2) {
            const int tt = t & 3;
            return (t >> 2) * 256 + (2 * wn + (tt >> 1)) * 32 + (tt & 1) * 16;
        }
        return (2 * wn + (t >> 2)) * 64 + (t & 3) * 16;
    };
    const int rbase = m0 + wm * 64;
    const int rtn = max(0, min(4, (m1 - rbase + 15) >> 4));  // live row tiles (wave-uniform)

    f32x4 acc[4][8];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto consume = [&](auto rl_tag) {
        constexpr int RL = decltype(rl_tag)::value;
        lds_barrier();  // A tile and B tile of step 0 in place
        for (int s = 0; s < nsteps; ++s) {
            const int buf = s & 1;
            if constexpr (RL > 0) {
                bf16x8 af[RL];
#pragma unroll
                for (int rt = 0; rt < RL; ++rt) {
                    const int row = wm * 64 + rt * 16 + c;
                    af[rt] = *reinterpret_cast<const bf16x8 *>(
                        &As[buf][row][8 * lds_chunk(row, grp)]);
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int col = tcol(t) + c;
                    const bf16x8 bf =
                        *reinterpret_cast<const bf16x8 *>(&Bs[buf][col][8 * lds_chunk(col, grp)]);
#pragma unroll
                    for (int rt = 0; rt < RL; ++rt)
                        acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[rt], bf, acc[rt][t],
                                                                             0, 0, 0);
                }
            }
            lds_barrier();
        }
    };
    if (wv < kCons) switch (rtn) {
    case 4: consume(std::integral_constant<int, 4>{}); break;
    case 3: consume(std::integral_constant<int, 3>{}); break;
    case 2: consume(std::integral_constant<int, 2>{}); break;
    case 1: consume(std::integral_constant<int, 1>{}); break;
    default: consume(std::integral_constant<int, 0>{}); break;
    }

    // ---- epilogue: lane (c, grp) holds, for row tile rt and column tile t,
    // rows rbase + 16 rt + 4 grp + i of the logical column of tile t, lane c
    const int jb = nb * (NSETS == 2 ? kWc / 2 : kWc);  // first word column of the block
    if (a.vec_out && !(NSETS == 2 && a.dh)) {
        // The block's outputs go through LDS (the B tiles are free now) and
        // all twelve waves store whole 16-byte chunks of each row: a block row
        // is 256 h columns (gate/up) or 512 outputs, contiguous in out.
        // gate/up takes one pass over the 128 rows, one cube a pass per
        // 64-row half.
        constexpr int COLS = NSETS == 2 ? kWc * 4 : kWc * 8;
        constexpr int PROWS = NSETS == 2 ? kRows : kRows / 2;
        constexpr int CH = COLS / 8;
        static_assert(PROWS * COLS <= 2 * kBCols * 32, "staging fits in the B tiles");
        __bf16 *st = &Bs[0][0][0];
        __syncthreads();  // every wave is done with the tiles
#pragma unroll
        for (int pass = 0; pass < kRows / PROWS; ++pass) {
            if (wv < kCons && (NSETS == 2 || wm == pass)) {
#pragma unroll
                for (int t = 0; t < (NSETS == 2 ? 4 : 8); ++t) {
                    const int col = tcol(t);
                    int sl, wcol;
                    if (NSETS == 2) {
                        sl = (col & 255) >> 5;
                        wcol = (col & 31) + c;
                    } else {
                        sl = col >> 6;
                        wcol = (col & 63) + c;
                    }
                    const int n = 8 * wcol + kSlotCol[sl];  // block-local output column
                    const bool on = jb + wcol < W;
                    const size_t nb_ = (size_t)e * N + 8 * jb + n;
                    const float b0 = (on && a.bias[0]) ? load_f<SD>(a.bias[0], nb_) : 0.0f;
                    const float b1 = (NSETS == 2 && on && a.bias[1]) ? load_f<SD>(a.bias[1], nb_)
                                                                     : 0.0f;
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt) {
                        if (rt >= rtn) continue;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int rl = (NSETS == 2 ? wm * 64 : 0) + rt * 16 + grp * 4 + i;
                            float v;
                            if (NSETS == 2) {
                                const float gv = round_to<MOEQ_BF16>(acc[rt][t][i] + b0);
                                const float uv = round_to<MOEQ_BF16>(acc[rt][t + 4][i] + b1);
                                v = swiglu_f(gv, uv, a.clamp, a.gate_lo, a.alpha, a.up_offset);
                            } else {
                                v = acc[rt][t][i] + b0;
                            }
                            st[rl * COLS + n] = (__bf16)v;
                        }
                    }
                }
            }
            __syncthreads();
            for (int u = threadIdx.x; u < PROWS * CH; u += kThreads) {
                const int rl = u / CH, ch = u - rl * CH;
                const int row = m0 + pass * PROWS + rl, col = 8 * jb + 8 * ch;
                if (row < m1 && col < a.Nout)
                    *reinterpret_cast<u32x4 *>(a.out + (size_t)row * a.Nout + col) =
                        *reinterpret_cast<const u32x4 *>(st + rl * COLS + 8 * ch);
            }
            if (pass + 1 < kRows / PROWS) __syncthreads();
        }
        return;
    }
    if (wv >= kCons) return;
#pragma unroll
    for (int t = 0; t < (NSETS == 2 ? 4 : 8); ++t) {
        const int col = tcol(t);
        int sl, wcol;
        if (NSETS == 2) {
            sl = (col & 255) >> 5;
            wcol = jb + (col & 31) + c;
        } else {
            sl = col >> 6;
            wcol = jb + (col & 63) + c;
        }
        if (wcol >= W) continue;
        const int n = 8 * wcol + kSlotCol[sl];
        const float b0 = a.bias[0] ? load_f<SD>(a.bias[0], (size_t)e * N + n) : 0.0f;
        const float b1 = (NSETS == 2 && a.bias[1]) ? load_f<SD>(a.bias[1], (size_t)e * N + n) : 0.0f;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (rt >= rtn) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = rbase + rt * 16 + grp * 4 + i;
                if (row >= m1) continue;
                float v;
                if (NSETS == 2) {
                    const float gv = round_to<MOEQ_BF16>(acc[rt][t][i] + b0);
                    const float uv = round_to<MOEQ_BF16>(acc[rt][t + 4][i] + b1);
                    if (a.dh) {  // backward: dG, dU at the rounded G, U
                        const size_t at = (size_t)row * a.Nout + n;
                        float dg, du;
                        swiglu_vjp_f(gv, uv, (float)a.dh[at], a.clamp, a.gate_lo, a.alpha, a.up_offset,
                                     &dg, &du);
                        a.out[at] = (__bf16)dg;
                        a.out2[at] = (__bf16)du;
                        continue;
                    }
                    v = swiglu_f(gv, uv, a.clamp, a.gate_lo, a.alpha, a.up_offset);
                } else {
                    v = acc[rt][t][i] + b0;
                }
                a.out[(size_t)row * a.Nout + n] = (__bf16)v;
            }
        }
    }
}

template <int NSETS, int SD>
hipError_t run_ws(const ProjProblem &p, hipStream_t s) {
    WsArgs a{};
    a.in = static_cast<const __bf16 *>(p.in);
    a.out = static_cast<__bf16 *>(p.out);
    a.offsets = p.offsets;
    a.tile_offsets = p.tile_offsets;
    a.tile_expert = p.tile_expert;
    a.tile_order = p.tile_order;
    a.min_rows = p.split_rows;
    a.E = p.E;
    a.K = p.w0.K;
    a.W = p.w0.N / 8;
    a.g = p.w0.g;
    a.Nout = p.Nout;
    const int per_blk = NSETS == 2 ? kWc / 2 : kWc;  // word columns of one cube per block
    a.nblk = (a.W + per_blk - 1) / per_blk;
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
    a.vec_out = ((uintptr_t)p.out % 16) == 0 && p.Nout % 8 == 0;
    const long mtiles = ((long)p.rows + kRows - 1) / kRows + p.E;
    const long blocks = 8 * ((mtiles + 7) / 8) * a.nblk;
    hipLaunchKernelGGL((awq_ws_kernel<NSETS, SD>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       a);
    return hipGetLastError();
}

}  // namespace

// Warp-specialised path: bf16 activations, AWQ, K and group multiples of 32,
// whole word columns in groups of 8 (partial column blocks are masked).
bool ws_fits(const ProjProblem &p) {
    if (const char *v = getenv("MOEQ_WS")) {  // tuning override: 0 disables
        if (atoi(v) == 0) return false;
    }
    if (p.act != MOEQ_BF16 || p.w0.format != MOEQ_FMT_AWQ || !p.offsets || !p.tile_offsets)
        return false;
    if (p.mode != PROJ_SWIGLU && p.mode != PROJ_PLAIN) return false;
    if (p.w0.K % 32 != 0 || p.w0.g % 32 != 0 || p.w0.K % p.w0.g != 0) return false;
    if ((size_t)p.rows * p.w0.K * 2 >= ((size_t)1 << 31)) return false;  // 32-bit row offsets
    return (p.w0.N / 8) % 16 == 0;
}

hipError_t launch_ws(const ProjProblem &p, hipStream_t s) {
    const bool two = p.mode == PROJ_SWIGLU;
    switch (p.w0.sdt) {
    case MOEQ_BF16: return two ? run_ws<2, MOEQ_BF16>(p, s) : run_ws<1, MOEQ_BF16>(p, s);
    case MOEQ_F16: return two ? run_ws<2, MOEQ_F16>(p, s) : run_ws<1, MOEQ_F16>(p, s);
    default: return two ? run_ws<2, MOEQ_F32>(p, s) : run_ws<1, MOEQ_F32>(p, s);
    }
}

}  // namespace moeq
