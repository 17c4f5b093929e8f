// gemm_mfma.hip -- bf16 MFMA grouped dequant-GEMMs for gfx950 (CDNA4).
//
// The AWQ payload (packed_experts.rs AwqExpertPayload; frozen_awq.rs
// FrozenAwqOps) packs eight 4-bit codes of eight consecutive output columns
// into one I32 word; a cube is K-major: word (k, j) holds columns 8j..8j+7 of
// input feature k.  The MFMA B operand wants, per lane, eight consecutive k of
// one column.  A lane that reads the eight words (k..k+7, j) therefore holds,
// for each of the 8 nibble positions, one complete B operand for the column
// that nibble position encodes.  One 16x16x32 MFMA per nibble position covers
// 16 word columns (the 16 lanes of a row); output columns are permuted only at
// the store, and no cross-lane shuffles are needed.
//
// Coefficient: (code - zero) * scale, rounded to the scale dtype (the pages'
// definition).  Codes become floats exactly through the fp8 E4M3 converter
// (a byte b < 16 encodes b * 2^-9), then fma(code', s * 2^9, -zero * s) gives
// the exact product for bf16/fp16 scales; the pack to bf16 rounds once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "awq_dequant.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace moeq {

bool tile_fits(const ProjProblem &p);
hipError_t launch_tile(const ProjProblem &p, const int32_t *tile_offsets,
                       const int32_t *tile_expert, hipStream_t s);
bool wave_fits(const ProjProblem &p);
hipError_t launch_wave(const ProjProblem &p, hipStream_t s);
bool ws_fits(const ProjProblem &p);
hipError_t launch_ws(const ProjProblem &p, hipStream_t s);
bool mx_fits(const ProjProblem &p);
hipError_t launch_mx(const ProjProblem &p, hipStream_t s);

namespace {

using namespace awq;

struct StreamArgs {
    const __bf16 *in;         // [A, K] rows sorted by expert
    __bf16 *out;              // [A, N]
    const int32_t *offsets;   // [E+1]
    int K, W, g;              // W = N/8 words per weight row
    int parts;                // column parts per expert (blocks per expert)
    int E;                    // experts
    int xcd_pairs;            // 1: the parts of an expert share an XCD (see kernel)
    int max_rows;             // > 0: experts with more rows are left to an m-tile kernel
    int vec_out;              // 1: out (and out2, dh) 16-byte aligned: one vector per row of 8 columns
    const uint32_t *qw[2];
    const uint32_t *qz[2];
    const void *sc[2];
    const void *bias[2];
    float clamp, alpha, up_offset;
    float gate_lo;  // lower clamp bound of the gate
    const __bf16 *dh;  // backward epilogue: [A, N] derivative of h (NULL: forward)
    __bf16 *out2;      // backward epilogue: dU (out holds dG)
};

// ------------------------------------------------------------------ stream
// Weight-streaming kernel for few rows per expert (decode).
//
// Block = one expert x one column part of SPW strips (a strip = 16 word
// columns = 128 output columns).  Its waves are NSETS x SPW x KSPLIT: wave
// (set, strip, q) streams one strip of one cube (gate or up, or the single
// down cube) over K slice q.  The waves of a block advance in lockstep (a
// barrier per 128 rows, and per 32-row step for the pipelined gate/up
// variant), so the CU reads each row block of its part as one contiguous
// piece -- one wave per strip would leave every row split over several XCDs
// and halve the achieved bandwidth.
//
// Per wave and 32-row step: eight buffer loads of one word per lane (row
// offsets are scalar), nibble planes, codes through the fp8 converter, one fma
// per coefficient, one pack per pair, 8 MFMAs per 16-row tile.  Steps run
// DEPTH ahead; the K slices meet in LDS in a fixed order; the up results join
// the gate results in LDS for the bias / storage rounding / SwiGLU epilogue.
template <int RT>
constexpr int stream_waves() { return RT == 1 ? 3 : 2; }

template <int NSETS, int SPW, int KSPLIT>
constexpr int stream_lds_bufs() {
    constexpr int tree = NSETS * SPW * (KSPLIT / 2);
    constexpr int join = NSETS == 2 ? SPW : 0;
    return tree > join ? tree : (join > 0 ? join : 1);
}

template <int NSETS, int SD, int SPW, int KSPLIT, int RT, int DEPTH, int SPG, bool BWD>
__global__ __launch_bounds__(64 * NSETS * SPW * KSPLIT)
__attribute__((amdgpu_waves_per_eu(stream_waves<RT>(), stream_waves<RT>())))
void awq_stream_kernel(StreamArgs a) {
    constexpr int NACC = 8 * RT;
    constexpr int sb = SD == MOEQ_F32 ? 4 : 2;
    // LDS: partial sums of the K tree, then the up results for the epilogue
    __shared__ f32x4 red[stream_lds_bufs<NSETS, SPW, KSPLIT>()][NACC][kWave];

    // Blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b % 8).
    // With xcd_pairs, block b = 8 * (P * n + part) + x holds expert 8n + x,
    // part `part`: the P parts of an expert run on one XCD, launched together,
    // so its L2 sees whole rows.
    int e, part;
    if (a.xcd_pairs) {
        const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
        e = (idx / a.parts) * 8 + x;
        part = idx % a.parts;
        if (e >= a.E) return;
    } else {
        e = blockIdx.x / a.parts;
        part = blockIdx.x % a.parts;
    }
    const int r0 = a.offsets[e], r1 = a.offsets[e + 1];
    if (r1 <= r0) return;  // untouched expert: no weight bytes are read
    if (a.max_rows > 0 && r1 - r0 > a.max_rows) return;  // a heavy expert: m-tile kernel
    // wave roles as scalars: keeps every K offset (buffer soffset) in SGPRs
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = wv % KSPLIT, unit = wv / KSPLIT;  // unit = (set, strip)
    const int strip = unit % SPW, set = unit / SPW;
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, grp = lane >> 4;
    const int j = (part * SPW + strip) * 16 + c;  // this lane's word column
    const int K = a.K, W = a.W, N = W * 8, g = a.g, G = K / g;
    const int Kw = K / KSPLIT;
    const int kbeg = q * Kw, kend = kbeg + Kw;

    const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(a.qw[set] + (size_t)e * K * W, (size_t)K * W * 4);
    const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(a.qz[set] + (size_t)e * G * W, (size_t)G * W * 4);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
        static_cast<const char *>(a.sc[set]) + (size_t)e * G * N * sb, (size_t)G * N * sb);
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.in, (size_t)r1 * K * 2);
    const int voff_w = (grp * 8 * W + j) * 4;
    const int voff_z = j * 4, voff_s = 8 * j * sb;

    for (int m0 = r0; m0 < r1; m0 += 16 * RT) {
        int voff_a[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int row = m0 + rt * 16 + c;
            voff_a[rt] = row < r1 ? (row * K + grp * 8) * 2 : 0x7fffffff;  // past end: zeros
        }
        f32x4 acc[8][RT];
#pragma unroll
        for (int sl = 0; sl < 8; ++sl)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[sl][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

        GroupRaw<SD> graw;
        GroupConst<SD> gc;
        // One 32-row step: nibble planes of the eight words, then (refill hook:
        // the words are dead from here) codes, coefficients, packs and MFMAs.
        auto step = [&](const uint32_t wd[8], const bf16x8 av[RT], auto &&refill_words) {
            uint32_t lo[8], hi[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lo[i] = and_opaque(wd[i], 0x0F0F0F0Fu);
                hi[i] = and_opaque(wd[i] >> 4, 0x0F0F0F0Fu);
            }
            refill_words();
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {  // slot pair (2pr, 2pr+1)
                f32x2 qv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t v = pr < 2 ? lo[i] : hi[i];
                    qv[i] = (pr & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(v, true)
                                     : __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int sl = 2 * pr + h;
                    u32x4 op;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        op[p] = pack_bf16(coeff<SD>(qv[2 * p][h], gc, sl),
                                          coeff<SD>(qv[2 * p + 1][h], gc, sl));
                    const bf16x8 bop = __builtin_bit_cast(bf16x8, op);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        acc[sl][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rt], bop,
                                                                              acc[sl][rt], 0, 0, 0);
                }
            }
        };

        if constexpr (SPG > 0) {
            // Branch-free pipeline: groups of SPG steps, steps unrolled, DEPTH
            // steps in flight in a fixed register ring (slot t % DEPTH).  Loads
            // past the wave's K range re-read its last step (clamped, in range,
            // never consumed), so every load is issued unconditionally and the
            // wait counts stay exact.  Each issue is pinned by a scheduling
            // barrier: the scheduler would otherwise sink the prefetch next to
            // its use.
            static_assert(SPG % DEPTH == 0 && SPG >= DEPTH, "ring must tile a group");
            uint32_t wd[DEPTH][8];
            bf16x8 av[DEPTH][RT];
            auto issue_words = [&](int st, int kk) {
                const int kc = kk < kend ? kk : kend - 32;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    wd[st][i] = __builtin_amdgcn_raw_buffer_load_b32(rw, voff_w, (kc + i) * W * 4, 0);
                __builtin_amdgcn_sched_barrier(0);
            };
            auto issue_rows = [&](int st, int kk) {
                const int kc = kk < kend ? kk : kend - 32;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    av[st][rt] = __builtin_bit_cast(
                        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra, voff_a[rt], kc * 2, 0));
                __builtin_amdgcn_sched_barrier(0);
            };
            const int gbeg = kbeg / g, gend = kend / g;
            load_group_raw<SD>(rz, rs, voff_z, voff_s, gbeg, W, N, graw);
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                issue_words(d, kbeg + 32 * d);
                issue_rows(d, kbeg + 32 * d);
            }
            for (int gi = gbeg; gi < gend; ++gi) {
                lockstep_barrier();  // the block reads one row block at a time
                decode_group<SD>(graw, gc);
#pragma unroll
                for (int t = 0; t < SPG; ++t) {
                    const int d = t % DEPTH;
                    const int kn = gi * g + 32 * (t + DEPTH);
                    if (t == SPG - DEPTH) {
                        // next group's constants, decoded DEPTH steps from now
                        load_group_raw<SD>(rz, rs, voff_z, voff_s, gi + 1 < gend ? gi + 1 : gi,
                                           W, N, graw);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    // gate/up: lockstep per 32-row step, so the CU keeps reading one
                    // row block at a time (once per 128-row group was 4% slower;
                    // the down projection is faster with one per group)
                    if (NSETS == 2 && t > 0) lockstep_barrier();
                    step(wd[d], av[d], [&] { issue_words(d, kn); });
                    issue_rows(d, kn);
                }
            }
        } else {
            // General K ranges and group sizes: one step in flight, a lockstep
            // barrier every 4 steps (every wave runs the same number of steps).
            uint32_t wd[8], wn[8];
            bf16x8 av[RT], an[RT];
            load_group_raw<SD>(rz, rs, voff_z, voff_s, kbeg / g, W, N, graw);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wd[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, voff_w, (kbeg + i) * W * 4, 0);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                av[rt] = __builtin_bit_cast(
                    bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra, voff_a[rt], kbeg * 2, 0));
            int it = 0;
            for (int k0 = kbeg; k0 < kend; k0 += 32, ++it) {
                if ((it & 3) == 0) lockstep_barrier();
                if (k0 == kbeg || k0 % g == 0) decode_group<SD>(graw, gc);
                const int kn = k0 + 32;
                if (kn < kend) {
                    if (kn % g == 0) load_group_raw<SD>(rz, rs, voff_z, voff_s, kn / g, W, N, graw);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        wn[i] = __builtin_amdgcn_raw_buffer_load_b32(rw, voff_w, (kn + i) * W * 4, 0);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        an[rt] = __builtin_bit_cast(
                            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ra, voff_a[rt], kn * 2, 0));
                }
                step(wd, av, [] {});
                if (kn < kend) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) wd[i] = wn[i];
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) av[rt] = an[rt];
                }
            }
        }

        // fixed-order tree over the K slices of each (set, strip):
        // q0 = (q0 + q2) + (q1 + q3)
        if constexpr (KSPLIT > 1) {
#pragma unroll
            for (int half = KSPLIT / 2; half >= 1; half >>= 1) {
                __syncthreads();
                if (q >= half && q < 2 * half) {
                    const int b = unit * (KSPLIT / 2) + (q - half);
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) red[b][sl * RT + rt][lane] = acc[sl][rt];
                }
                __syncthreads();
                if (q < half) {
                    const int b = unit * (KSPLIT / 2) + q;
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) acc[sl][rt] += red[b][sl * RT + rt][lane];
                }
            }
        }
        if constexpr (NSETS == 2) {
            // up results (set 1) join the gate results (set 0) of the same strip
            __syncthreads();
            if (q == 0 && set == 1) {
#pragma unroll
                for (int sl = 0; sl < 8; ++sl)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) red[strip][sl * RT + rt][lane] = acc[sl][rt];
            }
            __syncthreads();
        }
        if (q == 0 && set == 0) {
            float b0[8], b1[8];  // by slot
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                const int col = 8 * j + kSlotCol[sl];
                b0[sl] = a.bias[0] ? load_f<SD>(a.bias[0], (size_t)e * N + col) : 0.f;
                b1[sl] = (NSETS == 2 && a.bias[1]) ? load_f<SD>(a.bias[1], (size_t)e * N + col)
                                                   : 0.f;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 up4[8];
#pragma unroll
                for (int sl = 0; sl < 8; ++sl)
                    up4[sl] = NSETS == 2 ? red[strip][sl * RT + rt][lane] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + rt * 16 + grp * 4 + i;
                    if (row >= r1) continue;
                    const size_t base = (size_t)row * N + 8 * j;
                    if constexpr (BWD) {
                        // backward: dG, dU at the rounded G, U; dh read, dG and dU
                        // written as one 16-byte vector per row when aligned
                        float dv[8];  // by slot
                        if (a.vec_out) {
                            const u32x4 w = *reinterpret_cast<const u32x4 *>(a.dh + base);
#pragma unroll
                            for (int sl = 0; sl < 8; ++sl) {
                                const int c = kSlotCol[sl];
                                const uint32_t pair = w[c >> 1];
                                dv[sl] = __uint_as_float((c & 1) ? (pair & 0xFFFF0000u) : (pair << 16));
                            }
                        } else {
#pragma unroll
                            for (int sl = 0; sl < 8; ++sl) dv[sl] = (float)a.dh[base + kSlotCol[sl]];
                        }
                        float dg[8], du[8];
#pragma unroll
                        for (int sl = 0; sl < 8; ++sl) {
                            const float gv = round_to<MOEQ_BF16>(acc[sl][rt][i] + b0[sl]);
                            const float uv = round_to<MOEQ_BF16>(up4[sl][i] + b1[sl]);
                            swiglu_vjp_f(gv, uv, dv[sl], a.clamp, a.gate_lo, a.alpha, a.up_offset,
                                         &dg[sl], &du[sl]);
                        }
                        if (a.vec_out) {
                            u32x4 pg, pu;
                            pg[0] = pack_bf16(dg[0], dg[2]);
                            pg[1] = pack_bf16(dg[4], dg[6]);
                            pg[2] = pack_bf16(dg[1], dg[3]);
                            pg[3] = pack_bf16(dg[5], dg[7]);
                            pu[0] = pack_bf16(du[0], du[2]);
                            pu[1] = pack_bf16(du[4], du[6]);
                            pu[2] = pack_bf16(du[1], du[3]);
                            pu[3] = pack_bf16(du[5], du[7]);
                            *reinterpret_cast<u32x4 *>(a.out + base) = pg;
                            *reinterpret_cast<u32x4 *>(a.out2 + base) = pu;
                        } else {
#pragma unroll
                            for (int sl = 0; sl < 8; ++sl) {
                                a.out[base + kSlotCol[sl]] = (__bf16)dg[sl];
                                a.out2[base + kSlotCol[sl]] = (__bf16)du[sl];
                            }
                        }
                        continue;
                    }
                    float v[8];  // by slot
#pragma unroll
                    for (int sl = 0; sl < 8; ++sl) {
                        if (NSETS == 2) {
                            const float gv = round_to<MOEQ_BF16>(acc[sl][rt][i] + b0[sl]);
                            const float uv = round_to<MOEQ_BF16>(up4[sl][i] + b1[sl]);
                            v[sl] = swiglu_f(gv, uv, a.clamp, a.gate_lo, a.alpha, a.up_offset);
                        } else {
                            v[sl] = acc[sl][rt][i] + b0[sl];
                        }
                    }
                    {
                        // the lane's 8 columns 8 j .. 8 j + 7 are slots 0 2 4 6 1 3 5 7
                        __bf16 *o = a.out + base;
                        if (a.vec_out) {
                            u32x4 pk;
                            pk[0] = pack_bf16(v[0], v[2]);
                            pk[1] = pack_bf16(v[4], v[6]);
                            pk[2] = pack_bf16(v[1], v[3]);
                            pk[3] = pack_bf16(v[5], v[7]);
                            *reinterpret_cast<u32x4 *>(o) = pk;
                        } else {
#pragma unroll
                            for (int sl = 0; sl < 8; ++sl) o[kSlotCol[sl]] = (__bf16)v[sl];
                        }
                    }
                }
            }
        }
    }
}

template <int NSETS, int SD, int SPW, bool BWD>
hipError_t launch_stream(const StreamArgs &a, int E, int ksplit, int rt, int depth,
                         hipStream_t s) {
    dim3 grid(a.xcd_pairs ? ((E + 7) / 8) * 8 * a.parts : E * a.parts);
#define MOEQ_STREAM(KS, RTT, D, SP)                                                          \
    if (ksplit == KS && rt == RTT && depth == D) {                                           \
        hipLaunchKernelGGL((awq_stream_kernel<NSETS, SD, SPW, KS, RTT, D, SP, BWD>), grid,   \
                           dim3(64 * NSETS * SPW * KS), 0, s, a);                            \
        return hipGetLastError();                                                            \
    }
    if constexpr (NSETS * SPW * 2 <= 12) {
        MOEQ_STREAM(2, 1, 4, 4)
        MOEQ_STREAM(2, 1, 2, 4)
        MOEQ_STREAM(2, 1, 1, 0)
    }
    if constexpr (NSETS * SPW * 2 <= 8) {  // two row tiles: at most two waves per SIMD
        MOEQ_STREAM(2, 2, 2, 4)
    }
    MOEQ_STREAM(1, 1, 4, 4)
    MOEQ_STREAM(1, 1, 2, 4)
    MOEQ_STREAM(1, 1, 1, 0)
    if constexpr (NSETS * SPW <= 8) {
        MOEQ_STREAM(1, 2, 2, 4)
    }
    MOEQ_STREAM(1, 2, 1, 0)
#undef MOEQ_STREAM
    return hipErrorInvalidValue;
}

template <int NSETS, int SPW, bool BWD>
hipError_t stream_by_sdt_b(const StreamArgs &a, int sdt, int E, int ksplit, int rt, int depth,
                           hipStream_t s) {
    switch (sdt) {
    case MOEQ_BF16: return launch_stream<NSETS, MOEQ_BF16, SPW, BWD>(a, E, ksplit, rt, depth, s);
    case MOEQ_F16: return launch_stream<NSETS, MOEQ_F16, SPW, BWD>(a, E, ksplit, rt, depth, s);
    default: return launch_stream<NSETS, MOEQ_F32, SPW, BWD>(a, E, ksplit, rt, depth, s);
    }
}

// the backward epilogue is a separate instantiation: the forward kernels stay as they are
template <int NSETS, int SPW>
hipError_t stream_by_sdt(const StreamArgs &a, int sdt, int E, int ksplit, int rt, int depth,
                         hipStream_t s) {
    if constexpr (NSETS == 2)
        if (a.dh) return stream_by_sdt_b<NSETS, SPW, true>(a, sdt, E, ksplit, rt, depth, s);
    return stream_by_sdt_b<NSETS, SPW, false>(a, sdt, E, ksplit, rt, depth, s);
}

// Host-side choice of the stream kernel for a bf16 AWQ projection.
bool stream_fits(const ProjProblem &p) {
    if (p.act != MOEQ_BF16 || p.w0.format != MOEQ_FMT_AWQ || !p.offsets) return false;
    if (p.w0.N % 128 != 0 || p.w0.K % 32 != 0 || p.w0.g % 32 != 0) return false;
    if ((size_t)p.rows * p.w0.K * 2 >= ((size_t)1 << 31)) return false;
    const double rows_per_expert = (double)p.rows / (double)p.E;
    double limit = 8.0;
    if (const char *v = getenv("MOEQ_STREAM_MAX_ROWS")) limit = atof(v);  // tuning override
    return rows_per_expert <= limit;
}

// max_rows > 0: the light-expert half of a split launch -- only experts with
// 1..max_rows rows (at most 32: one pass of two 16-row tiles), the rest left to
// an m-tile kernel.
// Skewed routing with few rows per expert on average (more than the stream
// kernel's 8, at most 64): experts with at most kSplitRows rows stream their
// weights, the heavier ones run on an m-tile kernel that skips the light ones.
// A light expert's m-tile costs an m-tile kernel nearly as much as a full one
// (its per-step decode and barriers do not shrink with the rows), so on the
// many-expert workload the light experts' blocks took most of the call.
constexpr int kSplitRows = 32;

int split_rows() {
    if (const char *v = getenv("MOEQ_SPLIT_ROWS")) {  // tuning override: 16 or 32
        const int x = atoi(v);
        if (x == 16 || x == 32) return x;
    }
    return kSplitRows;
}

bool split_fits(const ProjProblem &p) {
    if (const char *v = getenv("MOEQ_SPLIT")) {  // tuning override: 0 disables
        if (atoi(v) == 0) return false;
    }
    if (p.act != MOEQ_BF16 || p.w0.format != MOEQ_FMT_AWQ || !p.offsets || !p.tile_offsets)
        return false;
    if (p.w0.N % 128 != 0 || p.w0.K % 32 != 0 || p.w0.g % 32 != 0) return false;
    if ((size_t)p.rows * p.w0.K * 2 >= ((size_t)1 << 31)) return false;
    const double rows_per_expert = (double)p.rows / (double)p.E;
    return rows_per_expert > 8.0 && rows_per_expert <= 64.0;
}

template <int NSETS>
hipError_t run_stream(const ProjProblem &p, hipStream_t s, int max_rows = 0) {
    StreamArgs a{};
    a.max_rows = max_rows;
    a.in = static_cast<const __bf16 *>(p.in);
    a.out = static_cast<__bf16 *>(p.out);
    a.offsets = p.offsets;
    a.K = p.w0.K;
    a.W = p.w0.N / 8;
    a.g = p.w0.g;
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
    const int strips = a.W / 16;
    // rows: one 16-row tile unless experts average more than 8 rows (or, split,
    // may hold more than 16)
    const int rt = max_rows > 0 ? (max_rows > 16 ? 2 : 1)
                                : (((double)p.rows / (double)p.E) <= 8.0 ? 1 : 2);
    // columns: a block's part is as wide as possible while E * parts still
    // covers the 256 CUs; two operand sets take 3-strip parts, one set 8
    int spw;
    if (NSETS == 2)
        spw = strips % 3 == 0 ? 3 : (strips % 2 == 0 ? 2 : 1);
    else
        spw = strips % 8 == 0 ? 8 : (strips % 4 == 0 ? 4 : (strips % 2 == 0 ? 2 : 1));
    // split launches (light experts only, fp32 scales on the many-expert workload
    // measured): one-strip parts, so the blocks spread over more CUs
    if (max_rows > 0 && NSETS == 2) spw = 1;
    if (const char *v = getenv("MOEQ_STREAM_SPW")) {  // tuning override (launch shape only)
        const int x = atoi(v);
        if ((x == 1 || x == 2 || x == 3 || x == 4 || x == 8) && strips % x == 0) spw = x;
    }
    // K split: two ways when the block stays within 12 waves (3 per SIMD, all
    // unspilled) and each half is whole groups
    int ksplit = (NSETS * spw * 2 <= 12 && (a.K / a.g) % 2 == 0) ? 2 : 1;
    if (rt == 2 && (max_rows == 0 || NSETS * spw * 2 > 8)) ksplit = 1;
    if (rt == 2 && NSETS * spw > 8) return hipErrorInvalidValue;  // not instantiated
    if (const char *v = getenv("MOEQ_STREAM_KSPLIT")) {
        const int x = atoi(v);
        if ((x == 1 || x == 2) && NSETS * spw * x <= (rt == 1 ? 12 : 8) && a.K % (32 * x) == 0)
            ksplit = x;
    }
    // the pipelined variant needs 128-row groups and group-aligned K slices
    int depth = ((rt == 1 || max_rows > 0) && a.g == 128 && (a.K / ksplit) % a.g == 0) ? 2 : 1;
    if (const char *v = getenv("MOEQ_STREAM_DEPTH")) {
        const int x = atoi(v);
        if (x == 1 || (depth > 1 && (x == 2 || x == 4))) depth = x;
    }
    // two row tiles exist at depths 1 and 2, and split over K only at depth 2
    // (group sizes other than 128 run unpipelined, hence unsplit)
    if (rt == 2) {
        if (depth == 4) depth = 2;
        if (ksplit == 2 && (depth != 2 || NSETS * spw * 2 > 8)) ksplit = 1;
    }
    a.parts = strips / spw;
    a.E = p.E;
    a.vec_out = (((uintptr_t)p.out | (uintptr_t)p.out2 | (uintptr_t)p.in2) % 16) == 0;
    a.xcd_pairs = 1;
    if (const char *v = getenv("MOEQ_STREAM_XCD")) a.xcd_pairs = atoi(v) != 0;
#define MOEQ_SPW(X) \
    case X: return stream_by_sdt<NSETS, X>(a, p.w0.sdt, p.E, ksplit, rt, depth, s);
    switch (spw) {
        MOEQ_SPW(1)
        MOEQ_SPW(2)
        MOEQ_SPW(3)
        MOEQ_SPW(4)
        MOEQ_SPW(8)
    default: return hipErrorInvalidValue;
    }
#undef MOEQ_SPW
}

// Second stream of a split launch, so that the light experts' streaming kernel
// runs beside the heavy experts' m-tile kernel instead of before it (each is
// latency-bound and leaves most of the chip idle on its own).  One stream and
// two events per host thread and device, created on first use outside graph
// capture and kept until the process ends (not destroyed at exit: the runtime
// may be gone by then).  Without them the two launches run one after the other
// on the caller's stream.
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool failed = false;
};

SideStream *side_stream(hipStream_t s, bool two_sets) {
    // tuning override: 0 serialises, 1 forks both calls, 2 only single-cube ones,
    // 3 only gate/up ones
    int policy = 1;
    if (const char *v = getenv("MOEQ_SPLIT_FORK")) policy = atoi(v);
    if (policy == 0 || (policy == 2 && two_sets) || (policy == 3 && !two_sets)) return nullptr;
    constexpr int kMaxDev = 64;
    thread_local SideStream sides[kMaxDev];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return nullptr;
    }
    SideStream &sd = sides[dev];
    if (sd.failed) return nullptr;
    if (!sd.stream) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
            (void)hipGetLastError();
            return nullptr;  // no stream creation under capture; create on a later call
        }
        if (hipStreamCreateWithFlags(&sd.stream, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&sd.join, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            sd.failed = true;
            return nullptr;
        }
    }
    return &sd;
}

// light(stream) and heavy(stream) write disjoint rows (each skips the other's
// experts) and read the same inputs: fork the light one onto the side stream,
// launch the heavy one on s, and join, so that later work on s waits for both.
template <class Light, class Heavy>
hipError_t fork_join(hipStream_t s, bool two_sets, Light light, Heavy heavy) {
    SideStream *sd = side_stream(s, two_sets);
    if (!sd) {
        const hipError_t err = light(s);
        return err != hipSuccess ? err : heavy(s);
    }
    // the heavy kernel is queued first, so its long-running blocks take CUs before
    // the light kernel's many short ones (measured: 0.2975 ms per many-expert step
    // against 0.3036 light first and 0.3228 serialised)
    bool heavy_first = true;
    if (const char *v = getenv("MOEQ_SPLIT_ORDER")) heavy_first = atoi(v) != 0;  // tuning
    hipError_t err = hipEventRecord(sd->fork, s);
    if (err != hipSuccess) return err;
    hipError_t eh = heavy_first ? heavy(s) : hipSuccess;
    err = hipStreamWaitEvent(sd->stream, sd->fork, 0);
    if (err != hipSuccess) return err;
    hipError_t el = light(sd->stream);
    // the join is recorded whatever the launches returned, so a capture stays joined
    hipError_t ej = hipEventRecord(sd->join, sd->stream);
    if (!heavy_first) eh = heavy(s);
    hipError_t ew = hipStreamWaitEvent(s, sd->join, 0);
    for (hipError_t e : {el, eh, ej, ew})
        if (e != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace

// Few rows per expert: the weight-streaming kernel; many: the register-decoded
// wave kernel, then the warp-specialised one (fp32 scales), then the LDS-tiled one.
hipError_t launch_fast_swiglu(const ProjProblem &p, hipStream_t s, bool *handled) {
    *handled = false;
    if (p.mode == PROJ_BANK_SWIGLU) {
        if (mx_fits(p)) {
            *handled = true;
            return launch_mx(p, s);
        }
        if (p.tile_offsets && tile_fits(p)) {
            *handled = true;
            return launch_tile(p, p.tile_offsets, p.tile_expert, s);
        }
        return hipSuccess;
    }
    if (p.mode != PROJ_SWIGLU) return hipSuccess;
    if (stream_fits(p)) {
        *handled = true;
        return run_stream<2>(p, s);
    }
    if (split_fits(p)) {
        ProjProblem heavy = p;
        heavy.split_rows = split_rows();
        const bool wave = wave_fits(heavy);
        if (wave || ws_fits(heavy)) {
            *handled = true;
            return fork_join(
                s, true, [&](hipStream_t st) { return run_stream<2>(p, st, split_rows()); },
                [&](hipStream_t st) { return wave ? launch_wave(heavy, st) : launch_ws(heavy, st); });
        }
    }
    if (wave_fits(p)) {
        *handled = true;
        return launch_wave(p, s);
    }
    if (ws_fits(p)) {
        *handled = true;
        return launch_ws(p, s);
    }
    if (p.in2) return hipSuccess;  // the backward epilogue lives in the three kernels above
    if (p.tile_offsets && tile_fits(p)) {
        *handled = true;
        return launch_tile(p, p.tile_offsets, p.tile_expert, s);
    }
    return hipSuccess;
}

hipError_t launch_fast_plain(const ProjProblem &p, hipStream_t s, bool *handled) {
    *handled = false;
    if (p.mode != PROJ_PLAIN) return hipSuccess;
    if (mx_fits(p)) {
        *handled = true;
        return launch_mx(p, s);
    }
    if (stream_fits(p)) {
        *handled = true;
        return run_stream<1>(p, s);
    }
    if (split_fits(p)) {
        ProjProblem heavy = p;
        heavy.split_rows = split_rows();
        const bool wave = wave_fits(heavy);
        if (wave || ws_fits(heavy)) {
            *handled = true;
            return fork_join(
                s, false, [&](hipStream_t st) { return run_stream<1>(p, st, split_rows()); },
                [&](hipStream_t st) { return wave ? launch_wave(heavy, st) : launch_ws(heavy, st); });
        }
    }
    if (wave_fits(p)) {
        *handled = true;
        return launch_wave(p, s);
    }
    if (ws_fits(p)) {
        *handled = true;
        return launch_ws(p, s);
    }
    if (p.tile_offsets && tile_fits(p)) {
        *handled = true;
        return launch_tile(p, p.tile_offsets, p.tile_expert, s);
    }
    return hipSuccess;
}

}  // namespace moeq
