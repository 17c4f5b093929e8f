// gemm_mx.hip -- register-decoded bf16 MFMA grouped GEMM over MXFP4 expert
// banks, gfx950.
//
// native.rs ExpertLayout::Native: a bank row is one output feature, K split in
// 32-element blocks of 16 bytes (two E2M1 codes per byte, even element in the
// low nibble) with one E8M0 scale byte per block; the fused gate/up bank
// interleaves gate feature i (row 2i) and up feature i (row 2i + 1), and the
// bias is a bf16 vector per bank row.  Each coefficient is E2M1 x 2^(s-127),
// exact in bf16; gfx950's v_cvt_scalef32_pk_bf16_fp4 produces two of them per
// instruction.
//
// Wave tile: up to 128 rows of one expert (live 16-row tiles only) x 3 column
// tiles of 16 bank rows.  One K super-step covers 4 blocks (128 k): lane
// (c, grp) loads the whole 16-byte block kb0 + grp of bank row n0 + c, and
// MFMA sub-step s uses its dword s, i.e. k = 32 (kb0 + grp) + 8 s + 0..7.  The
// A fragments follow the same k order, read from an LDS tile of the
// super-step's 128 k that the block's eight waves load cooperatively.  One
// block (16 B) per lane per column tile per super-step feeds 4 x RL MFMAs with
// four conversions per sub-step: the matrix core, not the decode, bounds it.
//
// gate/up: MFMA columns c (even) and c + 1 hold gate and up of feature
// (n0 + c) / 2; a DPP swap of adjacent lanes pairs them for SwiGLU.
//
// Blocks: one m-tile (128 rows of one expert) x 8 waves x 48 bank rows.  The
// m-tiles are dealt round-robin to the eight XCDs (block b runs on XCD b % 8;
// contiguous ranges per XCD were 0.6% slower); the column blocks of an m-tile
// run on one XCD and share its rows in L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "awq_dequant.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace moeq {

namespace {

using namespace awq;

constexpr int kRows = 128;        // rows per m-tile
constexpr int kWaves = 8;         // waves per block (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kCT = 3;            // 16-row column tiles per wave
constexpr int kSS = 128;          // k per super-step (4 blocks)
constexpr int kArow = kSS;        // LDS A row: 128 bf16, 16-byte chunks permuted

// 16-byte chunk position of chunk ch of LDS A row `row`: measured on gfx950,
// this permutation lets the fragment reads (16 rows x one chunk per 16 lanes)
// run at the full 256 bytes per clock.
__device__ __forceinline__ int a_chunk(int row, int ch) {
    return ch ^ ((row >> 1) & 3) ^ ((row & 1) << 3);
}

struct MxArgs {
    const __bf16 *in;  // [A, K] rows sorted by expert
    __bf16 *out;       // [A, Nout]
    const int32_t *offsets;
    const int32_t *tile_offsets;
    const int32_t *tile_expert;
    const uint8_t *blocks;  // [E, R, K/32, 16]
    const uint8_t *scales;  // [E, R, K/32]
    const __bf16 *bias;     // [E, R]
    int E, K, R, Nout;
    int nblk;  // blocks per m-tile
    float clamp, alpha, up_offset;
    float gate_lo;  // lower clamp bound of the gate
    int vec_out;    // 1: out 16-byte aligned and Nout % 8 == 0 (staged 16-byte stores)
};

__device__ __forceinline__ float e8m0_scale(uint32_t b) {
    return __uint_as_float(b == 255u ? 0x7FC00000u : b ? (b << 23) : 0x00400000u);
}

template <int MODE>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
void mx_wave_kernel(MxArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 As[2][kRows][kArow];  // 64 KB

    // ---- block -> (m-tile, column block); m-tile mt runs on XCD mt % 8
    const int mtiles = a.tile_offsets[a.E];
    const int per_xcd = (mtiles + 7) / 8;
    const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int local = idx / a.nblk, nb = idx % a.nblk;
    const int mt = local * 8 + x;  // m-tiles dealt round-robin to the XCDs
    if (local >= per_xcd || mt >= mtiles) return;
    const int e = a.tile_expert[mt];
    const int m0 = a.offsets[e] + (mt - a.tile_offsets[e]) * kRows;
    const int m1 = min(m0 + kRows, a.offsets[e + 1]);
    const int K = a.K, R = a.R, nbk = K / 32;
    const int nss = (nbk + 3) / 4;  // super-steps (the last may hold fewer blocks)

    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, grp = lane >> 4;
    const int n0 = (nb * kWaves + wv) * kCT * 16;  // first bank row of this wave

    // B operand sources: bank row n0 + 16 ct + c, block 4 ss + grp
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(a.blocks + (size_t)e * R * nbk * 16, (size_t)R * nbk * 16);
    const __amdgpu_buffer_rsrc_t rsc = buffer_rsrc(a.scales + (size_t)e * R * nbk, (size_t)R * nbk);
    int voff_b[kCT];  // scale byte offset = voff_b / 16
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
        const int r = n0 + ct * 16 + c;
        voff_b[ct] = r < R ? (r * nbk + grp) * 16 : 0x40000000;
    }

    // cooperative A loads: 128 rows x 16 chunks of 8 k per super-step, 4 per
    // thread (chunk u = tid + 512 h: row u / 16, k chunk u % 16)
    const int tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.in, (size_t)m1 * K * 2);
    int voff_a[4], arow[4], achk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int u = tid + kThreads * h;
        arow[h] = u >> 4;
        achk[h] = u & 15;
        const int row = m0 + arow[h];
        voff_a[h] = row < m1 ? (row * K + 8 * achk[h]) * 2 : -1;
    }
    const int rtn = (m1 - m0 + 15) >> 4;

    f32x4 acc[kCT][8];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) acc[ct][rt] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto main_loop = [&](auto rl_tag) {
        constexpr int RL = decltype(rl_tag)::value;
        constexpr int DB = 3;  // B ring depth (super-steps in flight)
        u32x4 bw[DB][kCT];
        uint32_t sw[DB][kCT];
        u32x4 ar[4];
        auto issue_b = [&](int d, int ss) {
            const int so = min(ss, nss - 1) * 64;  // 4 blocks of 16 bytes
#pragma unroll
            for (int ct = 0; ct < kCT; ++ct) {
                // blocks past the end of the row read as zero
                const int vo = 4 * ss + grp < nbk ? voff_b[ct] : 0x40000000;
                const int vs = vo >> 4;
                bw[d][ct] = __builtin_amdgcn_raw_buffer_load_b128(rb, vo, so, 0);
                sw[d][ct] = __builtin_amdgcn_raw_buffer_load_b8(rsc, vs, so / 16, 0);
            }
        };
        auto issue_a = [&](int ss) {
            const int k0 = min(ss, nss - 1) * kSS;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                // rows past the end and k past K read zeros (the scalar offset
                // stays wave-uniform)
                const bool on = voff_a[h] >= 0 && k0 + 8 * achk[h] < K;
                ar[h] = __builtin_amdgcn_raw_buffer_load_b128(ra, on ? voff_a[h] : 0x7fffffff,
                                                              k0 * 2, 0);
            }
        };
        auto store_a = [&](int buf) {
#pragma unroll
            for (int h = 0; h < 4; ++h)
                *reinterpret_cast<u32x4 *>(&As[buf][arow[h]][8 * a_chunk(arow[h], achk[h])]) = ar[h];
        };
        auto step = [&](int ss, int d) {
            const int buf = ss & 1;
            float sc[kCT];
#pragma unroll
            for (int ct = 0; ct < kCT; ++ct) sc[ct] = e8m0_scale(sw[d][ct] & 0xFFu);
            // next super-step's A tile into the other buffer; the loads stay
            // in program order (A tile, then the block refill at the end)
            store_a(buf ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            issue_a(ss + 2);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                // row tiles in groups of at most four: fewer live A fragments
                auto rows = [&](auto h0_tag, auto hw_tag) {
                    constexpr int H0 = decltype(h0_tag)::value, HW = decltype(hw_tag)::value;
                    bf16x8 af[HW];
#pragma unroll
                    for (int r = 0; r < HW; ++r)
                        af[r] = *reinterpret_cast<const bf16x8 *>(
                            &As[buf][(H0 + r) * 16 + c][8 * a_chunk(c, 4 * grp + s)]);
#pragma unroll
                    for (int ct = 0; ct < kCT; ++ct) {
                        const uint32_t w = bw[d][ct][s];
                        u32x4 op;
                        op[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc[ct], 0));
                        op[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc[ct], 1));
                        op[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc[ct], 2));
                        op[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc[ct], 3));
                        const bf16x8 bop = __builtin_bit_cast(bf16x8, op);
#pragma unroll
                        for (int r = 0; r < HW; ++r)
                            acc[ct][H0 + r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                af[r], bop, acc[ct][H0 + r], 0, 0, 0);
                    }
                };
                using I0 = std::integral_constant<int, 0>;
                using I2 = std::integral_constant<int, 2>;
                using I4 = std::integral_constant<int, 4>;
                if constexpr (RL <= 4) {
                    rows(I0{}, std::integral_constant<int, RL>{});
                } else {
                    rows(I0{}, I4{});
                    if constexpr (RL == 6) rows(I4{}, I2{});
                    else rows(I4{}, I4{});
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            issue_b(d, ss + DB);  // this slot's blocks are consumed: refill it
            __builtin_amdgcn_sched_barrier(0);
            lds_barrier();
        };

        // Prologue in the loop's own load order -- a step issues the A tile
        // two super-steps ahead, then refills its block slot -- so that on the
        // loop entry the next A tile is again followed by one slot's block
        // loads; scheduling barriers keep the compiler's wait counts exact
        // (otherwise the first step of every trip drains the whole ring).
        issue_b(0, 0);
        issue_b(1, 1);
        issue_a(0);
        store_a(0);
        __builtin_amdgcn_sched_barrier(0);
        issue_a(1);
        __builtin_amdgcn_sched_barrier(0);
        issue_b(2, 2);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        // ring slot of super-step ss is ss % DB: unrolled by DB, then the tail
        static_assert(DB == 3, "unrolled for a ring of three");
        int ss = 0;
        for (; ss + 2 < nss; ss += 3) {
            step(ss, 0);
            step(ss + 1, 1);
            step(ss + 2, 2);
        }
        if (ss < nss) step(ss, 0);
        if (ss + 1 < nss) step(ss + 1, 1);
    };
    if (rtn > 6)
        main_loop(std::integral_constant<int, 8>{});
    else if (rtn > 4)
        main_loop(std::integral_constant<int, 6>{});
    else if (rtn > 2)
        main_loop(std::integral_constant<int, 4>{});
    else
        main_loop(std::integral_constant<int, 2>{});

    // ---- epilogue.  Lane (c, grp) holds, for column tile ct and row tile rt,
    // rows 16 rt + 4 grp + i of bank row n0 + 16 ct + c.
    const __bf16 *bias = a.bias + (size_t)e * R;
    if (a.vec_out) {
        // The block's outputs go through LDS (the A tiles are free now) and
        // leave as whole 16-byte chunks of each row: a block row is 192 h
        // features (gate/up) or 384 outputs, contiguous in out.  gate/up takes
        // one pass over the 128 rows, one bank two passes of 64 rows.
        constexpr bool SW = MODE == PROJ_BANK_SWIGLU;
        constexpr int COLS = SW ? kWaves * kCT * 8 : kWaves * kCT * 16;
        constexpr int PROWS = SW ? kRows : kRows / 2;
        constexpr int CH = COLS / 8;  // 16-byte chunks per staged row
        static_assert(PROWS * COLS <= 2 * kRows * kArow, "staging fits in the A tiles");
        __bf16 *st = &As[0][0][0];
        const int col0 = nb * kWaves * kCT * (SW ? 8 : 16);  // first output column of the block
        const int wcol = wv * kCT * 16;                     // first bank row of the wave, block-local
        __syncthreads();  // every wave is done with the A tiles
#pragma unroll
        for (int pass = 0; pass < kRows / PROWS; ++pass) {
#pragma unroll
            for (int ct = 0; ct < kCT; ++ct) {
                const int r = n0 + ct * 16 + c;
                const float b = r < R ? (float)bias[r] : 0.0f;
#pragma unroll
                for (int rt = pass * (PROWS / 16); rt < (pass + 1) * (PROWS / 16); ++rt) {
                    if (rt >= rtn) continue;
                    const int rl = rt * 16 + grp * 4 - pass * PROWS;  // staged row of i = 0
                    if constexpr (SW) {
                        const bool gate_lane = (c & 1) == 0;
                        float own[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) own[i] = round_to<MOEQ_BF16>(acc[ct][rt][i] + b);
                        const float s0 = gate_lane ? own[2] : own[0];
                        const float s1 = gate_lane ? own[3] : own[1];
                        const float p0 = __int_as_float(
                            __builtin_amdgcn_mov_dpp(__float_as_int(s0), 0xB1, 0xF, 0xF, false));
                        const float p1 = __int_as_float(
                            __builtin_amdgcn_mov_dpp(__float_as_int(s1), 0xB1, 0xF, 0xF, false));
                        const int f = (wcol + ct * 16 + c) >> 1;  // block-local feature
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const float mine = gate_lane ? own[q] : own[2 + q];
                            const float other = q == 0 ? p0 : p1;
                            const float gv = gate_lane ? mine : other;
                            const float uv = gate_lane ? other : mine;
                            st[(rl + (gate_lane ? q : 2 + q)) * COLS + f] =
                                (__bf16)swiglu_f(gv, uv, a.clamp, a.gate_lo, a.alpha, a.up_offset);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            st[(rl + i) * COLS + wcol + ct * 16 + c] = (__bf16)(acc[ct][rt][i] + b);
                    }
                }
            }
            __syncthreads();
            for (int u = threadIdx.x; u < PROWS * CH; u += kThreads) {
                const int rl = u / CH, ch = u - rl * CH;
                const int row = m0 + pass * PROWS + rl, col = col0 + 8 * ch;
                if (row < m1 && col < a.Nout)
                    *reinterpret_cast<u32x4 *>(a.out + (size_t)row * a.Nout + col) =
                        *reinterpret_cast<const u32x4 *>(st + rl * COLS + 8 * ch);
            }
            if (pass + 1 < kRows / PROWS) __syncthreads();
        }
        return;
    }
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
        const int r = n0 + ct * 16 + c;
        const float b = r < R ? (float)bias[r] : 0.0f;
        if constexpr (MODE == PROJ_BANK_SWIGLU) {
            const bool gate_lane = (c & 1) == 0;
            const int f = r >> 1;  // feature of the pair
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                if (rt >= rtn) continue;
                float own[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) own[i] = round_to<MOEQ_BF16>(acc[ct][rt][i] + b);
                // gate lanes finish rows 0,1 of their quad, up lanes rows 2,3
                const float s0 = gate_lane ? own[2] : own[0];
                const float s1 = gate_lane ? own[3] : own[1];
                const float p0 = __int_as_float(
                    __builtin_amdgcn_mov_dpp(__float_as_int(s0), 0xB1, 0xF, 0xF, false));
                const float p1 = __int_as_float(
                    __builtin_amdgcn_mov_dpp(__float_as_int(s1), 0xB1, 0xF, 0xF, false));
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float mine = gate_lane ? own[q] : own[2 + q];
                    const float other = q == 0 ? p0 : p1;
                    const float gv = gate_lane ? mine : other;
                    const float uv = gate_lane ? other : mine;
                    const int row = m0 + rt * 16 + grp * 4 + (gate_lane ? q : 2 + q);
                    if (row < m1 && r < R)
                        a.out[(size_t)row * a.Nout + f] =
                            (__bf16)swiglu_f(gv, uv, a.clamp, a.gate_lo, a.alpha, a.up_offset);
                }
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                if (rt >= rtn) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + rt * 16 + grp * 4 + i;
                    if (row < m1 && r < R)
                        a.out[(size_t)row * a.Nout + r] = (__bf16)(acc[ct][rt][i] + b);
                }
            }
        }
    }
}

}  // namespace

// MXFP4 banks with bf16 activations, K a multiple of 32.
bool mx_fits(const ProjProblem &p) {
    if (const char *v = getenv("MOEQ_MX")) {  // tuning override: 0 disables
        if (atoi(v) == 0) return false;
    }
    if (p.act != MOEQ_BF16 || p.w0.format != MOEQ_FMT_MXFP4_BANK || !p.offsets || !p.tile_offsets)
        return false;
    if (p.mode != PROJ_BANK_SWIGLU && p.mode != PROJ_PLAIN) return false;
    if (p.w0.K % 32 != 0) return false;
    if ((size_t)p.rows * p.w0.K * 2 >= ((size_t)1 << 31)) return false;  // 32-bit row offsets
    if ((size_t)p.w0.N * p.w0.K / 2 >= ((size_t)1 << 30)) return false;  // 32-bit bank offsets
    return true;
}

hipError_t launch_mx(const ProjProblem &p, hipStream_t s) {
    MxArgs a{};
    a.in = static_cast<const __bf16 *>(p.in);
    a.out = static_cast<__bf16 *>(p.out);
    a.offsets = p.offsets;
    a.tile_offsets = p.tile_offsets;
    a.tile_expert = p.tile_expert;
    a.blocks = reinterpret_cast<const uint8_t *>(p.w0.qw);
    a.scales = static_cast<const uint8_t *>(p.w0.scales);
    a.bias = static_cast<const __bf16 *>(p.w0.bias);
    a.E = p.E;
    a.K = p.w0.K;
    a.R = p.w0.N;
    a.Nout = p.Nout;
    a.clamp = p.clamp;
    a.gate_lo = p.gate_lo;
    a.alpha = p.alpha;
    a.up_offset = p.up_offset;
    a.vec_out = ((uintptr_t)p.out % 16) == 0 && p.Nout % 8 == 0;
    const int rows_per_block = kWaves * kCT * 16;
    a.nblk = (a.R + rows_per_block - 1) / rows_per_block;
    const long mtiles = ((long)p.rows + kRows - 1) / kRows + p.E;
    const long blocks = 8 * ((mtiles + 7) / 8) * a.nblk;
    if (p.mode == PROJ_BANK_SWIGLU)
        hipLaunchKernelGGL((mx_wave_kernel<PROJ_BANK_SWIGLU>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((mx_wave_kernel<PROJ_PLAIN>), dim3((unsigned)blocks), dim3(kThreads),
                           0, s, a);
    return hipGetLastError();
}

}  // namespace moeq
