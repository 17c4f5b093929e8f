// route.hip -- router top-k + FP32 softmax, stable COPY dispatch, combine.
//
// moe_exchange.rs (ruda-tensor 0.21.38), MoeDispatchOps::moe_dispatch: per
// token a discrete top-k selection with FP32 continuous weights, then expert-
// sorted copies of the source rows; MoeDispatchOps::moe_combine: the ascending
// expert-ID combine.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "internal.hpp"

namespace moeq {

// ------------------------------------------------------------------ router
// Selection key: one 64-bit integer per (score, expert) whose unsigned order is
// the selection order -- score descending, then expert ID ascending.  High
// word: the score's bits made order-preserving (-0 is first turned into +0,
// since equal scores tie); low word: the inverted expert ID.  Key 0 marks an
// expert that is already taken or absent.  Scores are finite (no NaN).
__device__ __forceinline__ uint64_t sel_key(float score, int e) {
    uint32_t u = __float_as_uint(score + 0.0f);          // -0 + 0 = +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);      // monotone in the float order
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)e;
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)~(uint32_t)key; }
__device__ __forceinline__ float key_score(uint64_t key) {
    uint32_t u = (uint32_t)(key >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_key(uint64_t v) {
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Max key over the 16 lanes of a DPP row: four rotations (row_ror 8, 4, 2, 1)
// leave the row maximum in every lane of the row.
__device__ __forceinline__ uint64_t row16_max(uint64_t k) {
    k = umax64(k, dpp_key<0x128>(k));
    k = umax64(k, dpp_key<0x124>(k));
    k = umax64(k, dpp_key<0x122>(k));
    k = umax64(k, dpp_key<0x121>(k));
    return k;
}

// Sorts a lane's keys in descending order (bitonic network, N a power of two).
template <int N>
__device__ __forceinline__ void sort_keys_desc(uint64_t (&a)[N]) {
#pragma unroll
    for (int size = 2; size <= N; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ stride;
                if (l > i) {
                    const bool desc = (i & size) == 0;  // direction of this bitonic run
                    const uint64_t x = a[i], y = a[l];
                    const bool sw = desc ? x < y : x > y;
                    a[i] = sw ? y : x;
                    a[l] = sw ? x : y;
                }
            }
}

// Per-lane select by a wave lane mask, as one v_cndmask per 32-bit half.  The
// pop below is a chain of these; written as C selects, the compiler rewrote
// the chain into a compare-heavy state machine of twice the length.
__device__ __forceinline__ uint64_t select_by_mask(uint64_t lanes, uint64_t if_set,
                                                   uint64_t if_clear) {
    uint32_t lo, hi;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3"
        : "=v"(lo)
        : "v"((uint32_t)if_clear), "v"((uint32_t)if_set), "s"(lanes));
    asm("v_cndmask_b32_e64 %0, %1, %2, %3"
        : "=v"(hi)
        : "v"((uint32_t)(if_clear >> 32)), "v"((uint32_t)(if_set >> 32)), "s"(lanes));
    return ((uint64_t)hi << 32) | lo;
}

// Routes token t with the LANES lanes of the calling group (16: a DPP row; 64:
// the whole wave, rows joined by two cross-row shuffles).  Lane r holds the
// scores of experts r, r+LANES, ...; each of the k rounds takes the group-wide
// maximum key, and its owner lane clears it.  Lane j < k receives slot j: its
// expert and its weight, the softmax over the k selected scores evaluated in
// double in slot order and rounded once to fp32.
// The lane's logits and expert biases, loaded with clamped indices (no branch
// around a load), so the lane waits once.
template <int EPL>
struct RouteRaw {
    float v[EPL], b[EPL];
};

// LBF16: bf16 logits, widened exactly to fp32 (the bits moved to the high half).
template <int LANES, int EPL, bool LBF16>
__device__ __forceinline__ void route_load(const void *__restrict__ logits,
                                           const float *__restrict__ bias, int t, int E, int r,
                                           RouteRaw<EPL> &raw) {
    if constexpr (LBF16) {
        const uint16_t *row = static_cast<const uint16_t *>(logits) + (size_t)t * E;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            raw.v[i] = __uint_as_float((uint32_t)row[min(r + LANES * i, E - 1)] << 16);
    } else {
        const float *row = static_cast<const float *>(logits) + (size_t)t * E;
#pragma unroll
        for (int i = 0; i < EPL; ++i) raw.v[i] = row[min(r + LANES * i, E - 1)];
    }
    if (bias) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) raw.b[i] = bias[min(r + LANES * i, E - 1)];
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) raw.b[i] = 0.0f;  // unused: no add without a bias
    }
}

template <int LANES, int EPL, bool SORTED = (EPL <= 16)>
__device__ __forceinline__ void route_select(const RouteRaw<EPL> &raw, bool has_bias, int E,
                                             int k, int r, int group_base_lane, int *sel_out,
                                             float *w_out) {
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = has_bias ? raw.v[i] + raw.b[i] : raw.v[i];  // one fp32 add
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = r + LANES * i;
        key[i] = e < E ? sel_key(v[i], e) : 0;
    }
    uint64_t mine = 0;
    if constexpr (SORTED) {
        // sorted lane lists: each round compares the heads only, and the lane
        // that owns the maximum pops it (keys are unique, so exactly one lane)
        sort_keys_desc<EPL>(key);
        for (int j = 0; j < k; ++j) {
            uint64_t best = row16_max(key[0]);
            if (LANES == 64) {
                best = umax64(best, __shfl_xor(best, 16));
                best = umax64(best, __shfl_xor(best, 32));
            }
            const uint64_t win = __builtin_amdgcn_ballot_w64(key[0] == best);
#pragma unroll
            for (int i = 0; i + 1 < EPL; ++i) key[i] = select_by_mask(win, key[i + 1], key[i]);
            key[EPL - 1] = select_by_mask(win, 0, key[EPL - 1]);
            mine = r == j ? best : mine;
        }
    } else {
        for (int j = 0; j < k; ++j) {
            uint64_t best = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) best = umax64(best, key[i]);
            best = row16_max(best);
            if (LANES == 64) {
                best = umax64(best, __shfl_xor(best, 16));
                best = umax64(best, __shfl_xor(best, 32));
            }
#pragma unroll
            for (int i = 0; i < EPL; ++i) key[i] = key[i] == best ? 0 : key[i];  // taken
            mine = r == j ? best : mine;
        }
    }
    const float my_score = key_score(mine);
    const double m = (double)__shfl(my_score, group_base_lane);
    const double ex = exp((double)my_score - m);
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += __shfl(ex, group_base_lane + j);  // slot order
    *sel_out = key_expert(mine);
    *w_out = (float)(ex / den);
}

template <int LANES, int EPL, bool LBF16>
__device__ __forceinline__ void route_token(const void *__restrict__ logits,
                                            const float *__restrict__ bias, int t, int E, int k,
                                            int r, int group_base_lane, int *sel_out,
                                            float *w_out) {
    RouteRaw<EPL> raw;
    route_load<LANES, EPL, LBF16>(logits, bias, t, E, r, raw);
    route_select<LANES, EPL>(raw, bias != nullptr, E, k, r, group_base_lane, sel_out, w_out);
}

template <int LANES, int EPL, bool LBF16>
__global__ __launch_bounds__(256) void router_kernel(const void *__restrict__ logits,
                                                     const float *__restrict__ bias, int T, int E,
                                                     int k, uint32_t *__restrict__ selected,
                                                     float *__restrict__ weights) {
    const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) / LANES);
    const int r = threadIdx.x % LANES;
    if (t >= T) return;  // uniform per group
    int sel;
    float w;
    route_token<LANES, EPL, LBF16>(logits, bias, t, E, k, r,
                                   (int)(threadIdx.x & 63) & ~(LANES - 1), &sel, &w);
    if (r < k) {
        selected[(size_t)t * k + r] = (uint32_t)sel;
        weights[(size_t)t * k + r] = w;
    }
}

hipError_t launch_router(const void *logits, bool logits_bf16, const float *bias, int T, int E,
                         int k, uint32_t *selected, float *weights, hipStream_t s) {
    // 16 lanes per token while a lane holds at most 16 experts, else 64
#define MOEQ_ROUTER(L, N)                                                                \
    if (L * N >= E && k <= L) {                                                          \
        dim3 grid((unsigned)(((size_t)T * L + 255) / 256)), block(256);                  \
        if (logits_bf16)                                                                 \
            hipLaunchKernelGGL((router_kernel<L, N, true>), grid, block, 0, s, logits, bias, \
                               T, E, k, selected, weights);                              \
        else                                                                             \
            hipLaunchKernelGGL((router_kernel<L, N, false>), grid, block, 0, s, logits, bias, \
                               T, E, k, selected, weights);                              \
        return hipGetLastError();                                                        \
    }
    MOEQ_ROUTER(16, 2)
    MOEQ_ROUTER(16, 8)
    MOEQ_ROUTER(16, 16)
    MOEQ_ROUTER(64, 8)
    MOEQ_ROUTER(64, 16)
    MOEQ_ROUTER(64, 32)
#undef MOEQ_ROUTER
    return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ two-launch dispatch
// Dispatch in two launches while the per-expert token bitmasks fit in LDS
// (E * ceil(T/64) <= 8192 words, T <= 4096): the router kernel, then
// index_rows_kernel.  Block b of the latter owns tokens [b*tpb, (b+1)*tpb).  It
// reads all T*k selections (L2-resident), sets bit t of word t/64 of expert e's
// mask for each, counts each expert's rows from the masks and scans them with
// one wave (no block-wide barrier inside the scan).  The rank of its own
// assignment (t, e) among expert e's rows is then the popcount of the mask
// words below t, one wave per assignment; the block writes the route entries of
// its own tokens (block 0 also the offsets and m-tile lists) and copies their
// rows.  The index work is repeated in every block, but it is a few us of LDS
// traffic, and it replaces three launches of the multi-pass path below.
// (Routing in that same launch, as one earlier design did for small batches,
// kept each CU's VALU busy for about 5 us at decode: every block would route
// every token.)
//
// The copy runs over source vectors: x is [T][vecs] 16-byte vectors, and
// vector (t, i) goes to row slot_pos[t, j] of every slot j.  A thread's first
// kIdxPre vectors are loaded before the selections, so their latency overlaps
// the index work.
constexpr int kIdxWords = 8192;      // mask words in LDS (64 KB)
constexpr int kIdxMaxTokens = 16;    // tokens owned per block: T <= 256 * 16
constexpr int kIdxThreads = 1024;
constexpr int kIdxPre = 4;
constexpr int kIdxMaxAssign = 16384;  // T * k
typedef uint32_t vec4u __attribute__((ext_vector_type(4)));  // kept in registers

// Exclusive scans over experts by one wave (lane l owns a contiguous run of
// experts): rows (off_s, offsets), m-tiles of the tiled projections
// (tile_offsets, tile_expert) and their scheduling order (tile_order: every
// full m-tile in m-tile order, then the partial ones).
__device__ void scan_experts_wave(const int32_t *hist_s, int E, int A, bool write_route,
                                  int32_t *off_s, int32_t *__restrict__ offsets,
                                  int32_t *__restrict__ tile_offsets,
                                  int32_t *__restrict__ tile_expert,
                                  int32_t *__restrict__ tile_order) {
    const int lane = threadIdx.x & (kWave - 1);
    const int per = (E + kWave - 1) / kWave;
    const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
    int sc = 0, st = 0, sf = 0, sp = 0;
    for (int e = e0; e < e1; ++e) {
        const int c = hist_s[e], nt = (c + kTileRows - 1) / kTileRows, nf = c / kTileRows;
        sc += c;
        st += nt;
        sf += nf;
        sp += nt - nf;
    }
    int ic = sc, it = st, iff = sf, ip = sp;  // inclusive over lanes
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int a0 = __shfl_up(ic, o), a1 = __shfl_up(it, o);
        const int a2 = __shfl_up(iff, o), a3 = __shfl_up(ip, o);
        if (lane >= o) {
            ic += a0;
            it += a1;
            iff += a2;
            ip += a3;
        }
    }
    const int ftotal = __shfl(iff, kWave - 1);
    int ec = ic - sc, et = it - st, ef = iff - sf, ep = ip - sp;
    for (int e = e0; e < e1; ++e) {
        const int c = hist_s[e], nt = (c + kTileRows - 1) / kTileRows, nf = c / kTileRows;
        off_s[e] = ec;
        if (write_route) {
            offsets[e] = ec;
            tile_offsets[e] = et;
            for (int t = 0; t < nt; ++t) tile_expert[et + t] = e;
            for (int t = 0; t < nf; ++t) tile_order[ef + t] = et + t;
            if (nt > nf) tile_order[ftotal + ep] = et + nf;
        }
        ec += c;
        et += nt;
        ef += nf;
        ep += nt - nf;
    }
    if (lane == kWave - 1) {
        off_s[E] = A;
        if (write_route) {
            offsets[E] = A;
            tile_offsets[E] = it;
        }
    }
}

__global__ __launch_bounds__(kIdxThreads) void index_rows_kernel(
    const vec4u *__restrict__ x, int vecs, const uint32_t *__restrict__ selected, int T, int E,
    int k, int tpb, vec4u *__restrict__ values, uint32_t *__restrict__ row_experts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ row_src, int32_t *__restrict__ slot_pos,
    int32_t *__restrict__ tile_offsets, int32_t *__restrict__ tile_expert) {
    __shared__ unsigned long long mask_s[kIdxWords];
    __shared__ int32_t hist_s[kMaxExperts];
    __shared__ int32_t off_s[kMaxExperts + 1];
    __shared__ int32_t pos_s[kIdxMaxTokens * kMaxTopK];
    const int tid = threadIdx.x, A = T * k, MW = (T + 63) / 64;
    const int t0 = blockIdx.x * tpb, t1 = min(t0 + tpb, T);
    const long v0 = (long)t0 * vecs, nv = (long)(t1 - t0) * vecs;
    vec4u pre[kIdxPre];
#pragma unroll
    for (int u = 0; u < kIdxPre; ++u) pre[u] = x[v0 + min((long)u * kIdxThreads + tid, nv - 1)];

    for (int i = tid; i < E * MW; i += kIdxThreads) mask_s[i] = 0ull;
    for (int e = tid; e < E; e += kIdxThreads) hist_s[e] = 0;
    __syncthreads();
    // 1. per-expert token bitmasks (a token selects an expert at most once)
    for (int a = tid; a < A; a += kIdxThreads) {
        const int e = (int)selected[a], t = a / k;
        atomicOr(&mask_s[e * MW + (t >> 6)], 1ull << (t & 63));
    }
    __syncthreads();
    // 2. rows per expert, then the scans
    for (int i = tid; i < E * MW; i += kIdxThreads) {
        const int c = __popcll(mask_s[i]);
        if (c) atomicAdd(&hist_s[i / MW], c);
    }
    __syncthreads();
    if (tid < kWave)
        scan_experts_wave(hist_s, E, A, blockIdx.x == 0, off_s, offsets, tile_offsets,
                          tile_expert, tile_expert + tile_cap(A, E));
    __syncthreads();
    // 3. stable positions of the block's own assignments: the rank of token t
    //    among the tokens of expert e, one wave per assignment
    const int wv = tid / kWave, lane = tid & (kWave - 1);
    const int na = (t1 - t0) * k;
    for (int q = wv; q < na; q += kIdxThreads / kWave) {
        const int a = t0 * k + q, t = a / k;
        const int e = (int)selected[a];
        const int tw = t >> 6;
        int c = 0;
        if (lane < tw)
            c = __popcll(mask_s[e * MW + lane]);
        else if (lane == tw)
            c = __popcll(mask_s[e * MW + lane] & ((1ull << (t & 63)) - 1ull));
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) c += __shfl_xor(c, o);
        if (lane == 0) {
            const int p = off_s[e] + c;
            pos_s[q] = p;
            slot_pos[a] = p;
            row_src[p] = t;
            row_experts[p] = (uint32_t)e;
        }
    }
    __syncthreads();
    // 4. row copies: each source vector is stored to the rows of the token's k
    //    slots (for a fixed slot, consecutive threads write consecutive vectors)
#pragma unroll
    for (int u = 0; u < kIdxPre; ++u) {
        const long pr = (long)u * kIdxThreads + tid;
        if (pr < nv) {
            const int tl = (int)(pr / vecs), i = (int)(pr - (long)tl * vecs);
            for (int j = 0; j < k; ++j) values[(size_t)pos_s[tl * k + j] * vecs + i] = pre[u];
        }
    }
    for (long pr = (long)kIdxPre * kIdxThreads + tid; pr < nv; pr += kIdxThreads) {
        const vec4u v = x[v0 + pr];
        const int tl = (int)(pr / vecs), i = (int)(pr - (long)tl * vecs);
        for (int j = 0; j < k; ++j) values[(size_t)pos_s[tl * k + j] * vecs + i] = v;
    }
}

int index_rows_tpb(int T) { return T <= 256 ? 1 : (T + 255) / 256; }

bool index_rows_fits(int T, int E, int k, size_t row_bytes, const void *x, const void *values) {
    if (T < 1 || T > 256 * kIdxMaxTokens || E < 1 || E > kMaxExperts || k < 1 || k > kMaxTopK)
        return false;
    if ((long)E * ((T + 63) / 64) > kIdxWords) return false;
    // every block reads all T*k selections: at prefill size (32768) that and the
    // copy of 16 tokens per block, one block per CU, took 55 us against 46 us for
    // the multi-pass path
    if ((long)T * k > kIdxMaxAssign) return false;
    if (index_rows_tpb(T) * k > kIdxMaxTokens * kMaxTopK) return false;
    return row_bytes >= 16 && row_bytes % 16 == 0 && row_bytes < ((size_t)1 << 30) &&
           ((uintptr_t)x | (uintptr_t)values) % 16 == 0;
}

hipError_t launch_index_rows(const void *x, size_t row_bytes, const uint32_t *selected, int T,
                             int E, int k, void *values, uint32_t *row_experts,
                             const moeq_route *route, hipStream_t s) {
    const int tpb = index_rows_tpb(T);
    const int blocks = (T + tpb - 1) / tpb;
    hipLaunchKernelGGL(index_rows_kernel, dim3(blocks), dim3(kIdxThreads), 0, s,
                       (const vec4u *)x, (int)(row_bytes / 16), selected, T, E, k, tpb,
                       (vec4u *)values, row_experts, route->expert_offsets, route->row_src,
                       route->slot_pos, route->tile_offsets, route->tile_expert);
    return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch
// Stable counting sort of the T*k assignments by expert.
//  1. block_hist: per block of kTokenBlock tokens, the count of each expert.
//  2. block_scan: expert_offsets = exclusive scan of the totals; block_base[b][e]
//     = first sorted row of expert e for token block b.
//  3. block_scatter: the rank of a token among the block's tokens that chose
//     the same expert is a popcount over per-wave 64-bit token masks.
__global__ __launch_bounds__(256) void block_hist_kernel(const uint32_t *__restrict__ selected,
                                                         int T, int k, int E,
                                                         int32_t *__restrict__ block_base) {
    extern __shared__ int cnt[];
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    const long a0 = (long)b * kTokenBlock * k;
    const long a1 = min((long)(b + 1) * kTokenBlock, (long)T) * k;
    for (long a = a0 + threadIdx.x; a < a1; a += blockDim.x) atomicAdd(&cnt[selected[a]], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) block_base[(size_t)b * E + e] = cnt[e];
}

// Exclusive scan of v over the 1024 threads of a block (16 waves).
__device__ int block_exclusive_scan_1024(int v, int *wave_tot) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wave_tot[w] = incl;
    __syncthreads();
    if (w == 0) {
        int t = lane < 16 ? wave_tot[lane] : 0;
        int ti = t;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            int o = __shfl_up(ti, off);
            if (lane >= off) ti += o;
        }
        if (lane < 16) wave_tot[lane] = ti - t;  // exclusive wave offsets
    }
    __syncthreads();
    return wave_tot[w] + incl - v;
}

__global__ __launch_bounds__(1024) void block_scan_kernel(int32_t *__restrict__ block_base,
                                                          int nblocks, int E, int A,
                                                          int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ tile_offsets,
                                                          int32_t *__restrict__ tile_expert) {
    __shared__ int wave_tot[16];
    constexpr int kBatch = 8;  // independent loads in flight per thread
    // each thread owns experts 2*tid, 2*tid+1 (E <= 2048); pass 1: totals
    int tot[2] = {0, 0};
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * (int)threadIdx.x + q;
        if (e < E) {
            for (int b0 = 0; b0 < nblocks; b0 += kBatch) {
                int c[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    c[i] = b0 + i < nblocks ? block_base[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
                for (int i = 0; i < kBatch; ++i) tot[q] += c[i];
            }
        }
    }
    const int excl = block_exclusive_scan_1024(tot[0] + tot[1], wave_tot);
    const int starts[2] = {excl, excl + tot[0]};
    // pass 2: block_base[b][e] = first sorted row of expert e for token block b
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * (int)threadIdx.x + q;
        if (e < E) {
            offsets[e] = starts[q];
            int run = starts[q];
            for (int b0 = 0; b0 < nblocks; b0 += kBatch) {
                int c[kBatch];
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
                    c[i] = b0 + i < nblocks ? block_base[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    if (b0 + i < nblocks) block_base[(size_t)(b0 + i) * E + e] = run;
                    run += c[i];
                }
            }
        }
    }
    if (threadIdx.x == 0) offsets[E] = A;
    // m-tiles of kTileRows rows per expert, as a prefix over experts
    __syncthreads();
    const int nt0 = (tot[0] + kTileRows - 1) / kTileRows, nt1 = (tot[1] + kTileRows - 1) / kTileRows;
    const int texcl = block_exclusive_scan_1024(nt0 + nt1, wave_tot);
    // scheduling order: every full m-tile (m-tile order), then the partial ones
    const int nf0 = tot[0] / kTileRows, nf1 = tot[1] / kTileRows;
    const int np0 = nt0 - nf0, np1 = nt1 - nf1;
    __syncthreads();
    const int fexcl = block_exclusive_scan_1024(nf0 + nf1, wave_tot);
    __syncthreads();
    __shared__ int ftotal_s;
    if (threadIdx.x == blockDim.x - 1) ftotal_s = fexcl + nf0 + nf1;
    const int pexcl = block_exclusive_scan_1024(np0 + np1, wave_tot);
    __syncthreads();
    const int ftotal = ftotal_s;
    int32_t *tile_order = tile_expert + tile_cap(A, E);
    for (int q = 0; q < 2; ++q) {
        const int e = 2 * (int)threadIdx.x + q;
        const int first = q == 0 ? texcl : texcl + nt0, n = q == 0 ? nt0 : nt1;
        const int nf = q == 0 ? nf0 : nf1, np = q == 0 ? np0 : np1;
        const int fpos = q == 0 ? fexcl : fexcl + nf0, ppos = q == 0 ? pexcl : pexcl + np0;
        if (e < E) {
            tile_offsets[e] = first;
            for (int t = 0; t < n; ++t) tile_expert[first + t] = e;
            for (int t = 0; t < nf; ++t) tile_order[fpos + t] = first + t;
            if (np) tile_order[ftotal + ppos] = first + nf;
        }
        if (e == E - 1) tile_offsets[E] = first + n;
    }
}

// Wave w of the block ranks tokens 64w .. 64w + 63 of the token block: the rank
// of token t among the block's tokens that chose expert e is the popcount of
// the chosen-e masks of the earlier waves plus that of the lower lanes of its
// own wave.  Two barriers per block.
constexpr int kScatterWaves = kTokenBlock / 64;
__global__ __launch_bounds__(kTokenBlock) void block_scatter_kernel(
    const uint32_t *__restrict__ selected, int T, int k, int E,
    const int32_t *__restrict__ block_base, int32_t *__restrict__ slot_pos,
    int32_t *__restrict__ row_src, uint32_t *__restrict__ row_experts) {
    extern __shared__ unsigned long long smem_u64[];
    unsigned long long *mask = smem_u64;  // [kScatterWaves][E]
    const int b = blockIdx.x, w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    for (int i = threadIdx.x; i < kScatterWaves * E; i += blockDim.x) mask[i] = 0ull;
    __syncthreads();
    const int t = b * kTokenBlock + (int)threadIdx.x;
    const bool valid = t < T;
    if (valid)
        for (int j = 0; j < k; ++j)
            atomicOr(&mask[w * E + selected[(size_t)t * k + j]], 1ull << lane);
    __syncthreads();
    if (valid) {
        const unsigned long long lower = (1ull << lane) - 1ull;
        for (int j = 0; j < k; ++j) {
            const uint32_t e = selected[(size_t)t * k + j];
            int p = block_base[(size_t)b * E + e] + __popcll(mask[w * E + e] & lower);
            for (int v = 0; v < w; ++v) p += __popcll(mask[v * E + e]);
            slot_pos[(size_t)t * k + j] = p;
            row_src[p] = t;
            row_experts[p] = e;
        }
    }
}

hipError_t launch_dispatch_index(const uint32_t *selected, int T, int E, int k,
                                 const moeq_route *route, uint32_t *row_experts,
                                 hipStream_t s) {
    const int nb = route->token_blocks;
    hipLaunchKernelGGL(block_hist_kernel, dim3(nb), dim3(256), sizeof(int) * E, s, selected,
                       T, k, E, route->block_base);
    hipLaunchKernelGGL(block_scan_kernel, dim3(1), dim3(1024), 0, s, route->block_base, nb, E,
                       T * k, route->expert_offsets, route->tile_offsets, route->tile_expert);
    hipLaunchKernelGGL(block_scatter_kernel, dim3(nb), dim3(kTokenBlock),
                       sizeof(unsigned long long) * kScatterWaves * E, s, selected, T, k, E,
                       route->block_base, route->slot_pos, route->row_src, row_experts);
    return hipGetLastError();
}

// ------------------------------------------------------------------ unsorted rows
// Local expert index of each incoming row (IDs validated on the host).
__global__ __launch_bounds__(256) void local_ids_kernel(const uint32_t *__restrict__ gid, int rows,
                                                        uint32_t start,
                                                        uint32_t *__restrict__ local) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < rows) local[t] = gid[t] - start;
}

hipError_t launch_local_ids(const uint32_t *gid, int rows, int start, uint32_t *local,
                            hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(local_ids_kernel, dim3((rows + 255) / 256), dim3(256), 0, s, gid, rows,
                       (uint32_t)start, local);
    return hipGetLastError();
}

// Row map of a single cube over all rows: offsets {0, rows}, 128-row m-tiles.
__global__ __launch_bounds__(256) void single_tiles_kernel(int rows, int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ tile_offsets,
                                                           int32_t *__restrict__ tile_expert) {
    const int nt = (rows + kTileRows - 1) / kTileRows;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0) {
        offsets[0] = 0;
        offsets[1] = rows;
        tile_offsets[0] = 0;
        tile_offsets[1] = nt;
    }
    if (i < nt) {
        tile_expert[i] = 0;
        tile_expert[tile_cap(rows, 1) + i] = i;  // scheduling order: the m-tiles in order
    }
}

hipError_t launch_single_tiles(int rows, int32_t *offsets, int32_t *tile_offsets,
                               int32_t *tile_expert, hipStream_t s) {
    const int nt = (rows + kTileRows - 1) / kTileRows;
    hipLaunchKernelGGL(single_tiles_kernel, dim3((nt + 255) / 256 + 1), dim3(256), 0, s, rows,
                       offsets, tile_offsets, tile_expert);
    return hipGetLastError();
}

// ------------------------------------------------------------------ row copy
template <typename V>
__global__ __launch_bounds__(256) void copy_rows_kernel(const V *__restrict__ x,
                                                        size_t row_elems, int A,
                                                        const int32_t *__restrict__ row_src,
                                                        V *__restrict__ values) {
    const int p = blockIdx.x;
    const V *src = x + (size_t)row_src[p] * row_elems;
    V *dst = values + (size_t)p * row_elems;
    for (size_t i = (size_t)blockIdx.y * blockDim.x + threadIdx.x; i < row_elems;
         i += (size_t)gridDim.y * blockDim.x)
        dst[i] = src[i];
}

hipError_t launch_copy_rows(const void *x, size_t row_bytes, int A, const int32_t *row_src,
                            void *values, hipStream_t s) {
    if (A == 0 || row_bytes == 0) return hipSuccess;
    const uintptr_t al = (uintptr_t)x | (uintptr_t)values;
    if (row_bytes % 16 == 0 && al % 16 == 0) {
        const size_t n = row_bytes / 16;
        dim3 grid((unsigned)A, (unsigned)min((n + 255) / 256, (size_t)65535));
        hipLaunchKernelGGL(copy_rows_kernel<uint4>, grid, dim3(256), 0, s, (const uint4 *)x, n,
                           A, row_src, (uint4 *)values);
    } else if (row_bytes % 4 == 0 && al % 4 == 0) {
        const size_t n = row_bytes / 4;
        dim3 grid((unsigned)A, (unsigned)min((n + 255) / 256, (size_t)65535));
        hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, grid, dim3(256), 0, s,
                           (const uint32_t *)x, n, A, row_src, (uint32_t *)values);
    } else {
        dim3 grid((unsigned)A, (unsigned)min((row_bytes + 255) / 256, (size_t)65535));
        hipLaunchKernelGGL(copy_rows_kernel<uint8_t>, grid, dim3(256), 0, s,
                           (const uint8_t *)x, row_bytes, A, row_src, (uint8_t *)values);
    }
    return hipGetLastError();
}

// Source-major COPY dispatch for large batches: x is [T][vecs] 16-byte
// vectors, and vector (t, i) goes to row slot_pos[t, j] of each slot j.  A
// block covers kScatterU * 256 consecutive source vectors; each thread loads
// its kScatterU vectors at once (clamped, no branch around a load) while the
// block stages the slot positions of its tokens in LDS, then stores every
// vector k times (for a fixed slot, consecutive threads write consecutive
// vectors).  Each source row is read once instead of once per slot.
constexpr int kScatterU = 4;
constexpr int kScatterMinVecs = 16;  // at most 65 tokens per block
constexpr int kScatterTokens = (256 * kScatterU) / kScatterMinVecs + 1;

__global__ __launch_bounds__(256) void scatter_rows_kernel(const vec4u *__restrict__ x, int vecs,
                                                           int T, int k,
                                                           const int32_t *__restrict__ slot_pos,
                                                           vec4u *__restrict__ values) {
    __shared__ int32_t pos_s[kScatterTokens * kMaxTopK];
    const long n = (long)T * vecs;
    const long b0 = (long)blockIdx.x * (256 * kScatterU);
    const long b1 = min(b0 + 256 * kScatterU, n);
    const int t_lo = (int)(b0 / vecs), t_hi = (int)((b1 - 1) / vecs);
    vec4u v[kScatterU];
#pragma unroll
    for (int u = 0; u < kScatterU; ++u)
        v[u] = x[min(b0 + u * 256 + (long)threadIdx.x, n - 1)];
    const int cnt = (t_hi - t_lo + 1) * k;
    for (int i = threadIdx.x; i < cnt; i += 256) pos_s[i] = slot_pos[(size_t)t_lo * k + i];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kScatterU; ++u) {
        const long pr = b0 + u * 256 + (long)threadIdx.x;
        if (pr < n) {
            const int t = (int)(pr / vecs), i = (int)(pr - (long)t * vecs);
            const int32_t *pt = pos_s + (t - t_lo) * k;
            for (int j = 0; j < k; ++j) values[(size_t)pt[j] * vecs + i] = v[u];
        }
    }
}

bool scatter_rows_fits(size_t row_bytes, int k, const void *x, const void *values) {
    return row_bytes % 16 == 0 && row_bytes / 16 >= (size_t)kScatterMinVecs &&
           row_bytes / 16 < ((size_t)1 << 30) && k >= 1 && k <= kMaxTopK &&
           ((uintptr_t)x | (uintptr_t)values) % 16 == 0;
}

hipError_t launch_scatter_rows(const void *x, size_t row_bytes, int T, int k,
                               const int32_t *slot_pos, void *values, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int vecs = (int)(row_bytes / 16);
    const long n = (long)T * vecs;
    const long blocks = (n + 256 * kScatterU - 1) / (256 * kScatterU);
    if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const vec4u *)x, vecs, T, k, slot_pos, (vec4u *)values);
    return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// One block per token.  The k sorted positions are ranked so that slot a of
// the shared list is the a-th smallest position, i.e. the a-th smallest expert
// ID; every column then runs acc = fma(w, y, acc) in that order.  Each thread
// owns VEC consecutive columns and moves them as one 16-byte vector; its row
// loads are all issued before the first fma (KM >= k bounds them at compile
// time).  WEIGHTED = false is the COPY VJP (moe_exchange.rs
// MoeDispatchOps::moe_dispatch_backward): w = 1, so fma(1, y, acc) is the plain
// fp32 sum acc + y in the same ascending order, and `weights` is not read.
template <int ACT, int KM, bool WEIGHTED>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ y,
                                                      const float *__restrict__ weights,
                                                      const int32_t *__restrict__ slot_pos,
                                                      int T, int k, int K, bool vec_ok,
                                                      void *__restrict__ out) {
    typedef typename Storage<ACT>::T S;
    constexpr int VEC = 16 / sizeof(S);
    typedef S sv __attribute__((ext_vector_type(VEC)));
    __shared__ int raw_s[KM];
    __shared__ float wraw_s[KM];
    __shared__ int pos_s[KM];
    __shared__ float w_s[KM];
    const int t = blockIdx.x;
    if ((int)threadIdx.x < k) {
        raw_s[threadIdx.x] = slot_pos[(size_t)t * k + threadIdx.x];
        wraw_s[threadIdx.x] = WEIGHTED ? weights[(size_t)t * k + threadIdx.x] : 1.0f;
    }
    __syncthreads();
    if ((int)threadIdx.x < k) {
        const int p = raw_s[threadIdx.x];
        int rank = 0;
        for (int j = 0; j < k; ++j) rank += raw_s[j] < p;
        pos_s[rank] = p;
        w_s[rank] = wraw_s[threadIdx.x];
    }
    __syncthreads();
    const S *ys = static_cast<const S *>(y);
    S *os = static_cast<S *>(out);
    if (vec_ok) {
        for (int c = threadIdx.x * VEC; c < K; c += blockDim.x * VEC) {
            sv yv[KM];  // slots past k reload slot k - 1 (no branch around a load)
#pragma unroll
            for (int a = 0; a < KM; ++a)
                yv[a] = *reinterpret_cast<const sv *>(ys + (size_t)pos_s[min(a, k - 1)] * K + c);
            float acc[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
#pragma unroll
            for (int a = 0; a < KM; ++a) {
                if (a < k) {
                    const float w = w_s[a];
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[v] = __builtin_fmaf(w, (float)yv[a][v], acc[v]);
                }
            }
            sv o;
#pragma unroll
            for (int v = 0; v < VEC; ++v) o[v] = (S)acc[v];
            *reinterpret_cast<sv *>(os + (size_t)t * K + c) = o;
        }
    } else {
        for (int c = threadIdx.x; c < K; c += blockDim.x) {
            float acc = 0.0f;
            for (int a = 0; a < k; ++a)
                acc = __builtin_fmaf(w_s[a], (float)ys[(size_t)pos_s[a] * K + c], acc);
            os[(size_t)t * K + c] = (S)acc;
        }
    }
}

hipError_t launch_combine(const void *y, int act, const float *weights,
                          const int32_t *slot_pos, int T, int k, int K, void *out,
                          hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int vec = act == MOEQ_F32 ? 4 : 8;
    const bool vec_ok = ((uintptr_t)y | (uintptr_t)out) % 16 == 0 && K % vec == 0;
    int threads = vec_ok ? K / vec : K;
    threads = threads >= 256 ? 256 : ((threads + 63) / 64) * 64;
#define MOEQ_COMBINE(DT, KM)                                                                 \
    hipLaunchKernelGGL((combine_kernel<DT, KM, true>), dim3(T), dim3(threads), 0, s, y, weights, \
                       slot_pos, T, k, K, vec_ok, out)
#define MOEQ_COMBINE_K(DT)            \
    if (k <= 8)                       \
        MOEQ_COMBINE(DT, 8);          \
    else if (k <= 16)                 \
        MOEQ_COMBINE(DT, 16);         \
    else                              \
        MOEQ_COMBINE(DT, kMaxTopK)
    if (act == MOEQ_F32)
        MOEQ_COMBINE_K(MOEQ_F32);
    else if (act == MOEQ_BF16)
        MOEQ_COMBINE_K(MOEQ_BF16);
    else
        MOEQ_COMBINE_K(MOEQ_F16);
#undef MOEQ_COMBINE_K
#undef MOEQ_COMBINE
    return hipGetLastError();
}

hipError_t launch_dispatch_backward(const void *grad, int act, const int32_t *slot_pos, int T,
                                    int k, int K, void *grad_x, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int vec = act == MOEQ_F32 ? 4 : 8;
    const bool vec_ok = ((uintptr_t)grad | (uintptr_t)grad_x) % 16 == 0 && K % vec == 0;
    int threads = vec_ok ? K / vec : K;
    threads = threads >= 256 ? 256 : ((threads + 63) / 64) * 64;
#define MOEQ_COPY_VJP(DT, KM)                                                                 \
    hipLaunchKernelGGL((combine_kernel<DT, KM, false>), dim3(T), dim3(threads), 0, s, grad,     \
                       nullptr, slot_pos, T, k, K, vec_ok, grad_x)
#define MOEQ_COPY_VJP_K(DT)           \
    if (k <= 8)                       \
        MOEQ_COPY_VJP(DT, 8);         \
    else if (k <= 16)                 \
        MOEQ_COPY_VJP(DT, 16);        \
    else                              \
        MOEQ_COPY_VJP(DT, kMaxTopK)
    if (act == MOEQ_F32)
        MOEQ_COPY_VJP_K(MOEQ_F32);
    else if (act == MOEQ_BF16)
        MOEQ_COPY_VJP_K(MOEQ_BF16);
    else
        MOEQ_COPY_VJP_K(MOEQ_F16);
#undef MOEQ_COPY_VJP_K
#undef MOEQ_COPY_VJP
    return hipGetLastError();
}

}  // namespace moeq
