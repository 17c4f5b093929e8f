// api.cpp -- the C-ABI of libmoeq: host-side validation, then kernel launches.
//
// Every entry point checks its arguments completely before it enqueues
// anything; a failed check returns a negative moeq_status, records the reason
// for moeq_last_error() and leaves all outputs untouched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "internal.hpp"
#include "moeq.h"

namespace moeq {
hipError_t launch_fast_swiglu(const ProjProblem &p, hipStream_t s, bool *handled);
hipError_t launch_fast_plain(const ProjProblem &p, hipStream_t s, bool *handled);
}  // namespace moeq

using namespace moeq;

namespace {

thread_local char g_last_error[512] = "";

moeq_status fail(moeq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

moeq_status device_status(hipError_t err, const char *what) {
    if (err == hipSuccess) return MOEQ_OK;
    return fail(MOEQ_EDEVICE, "%s: %s", what, hipGetErrorString(err));
}

bool valid_dtype(int d) { return d == MOEQ_F32 || d == MOEQ_F16 || d == MOEQ_BF16; }
size_t dtype_bytes(int d) { return d == MOEQ_F32 ? 4 : 2; }

// a * b with overflow detection (native.rs validate: ShapeOverflow)
bool mul_ok(size_t a, size_t b, size_t *out) {
    if (a != 0 && b > SIZE_MAX / a) return false;
    *out = a * b;
    return true;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
    size_t off_offsets, off_row_src, off_slot_pos, off_block_base, off_tiles, off_tile_expert,
        total;
    int blocks;
};

bool route_layout(int32_t T, int32_t E, int32_t k, Layout *L) {
    if (T < 0 || E < 1 || k < 1 || k > E) return false;
    size_t A;
    if (!mul_ok((size_t)T, (size_t)k, &A) || A > (size_t)INT32_MAX) return false;
    L->blocks = (int)((T + kTokenBlock - 1) / kTokenBlock);
    size_t bb;
    if (!mul_ok((size_t)L->blocks, (size_t)E, &bb)) return false;
    size_t o = 0;
    L->off_offsets = o;
    o += align256(sizeof(int32_t) * ((size_t)E + 1));
    L->off_row_src = o;
    o += align256(sizeof(int32_t) * (A ? A : 1));
    L->off_slot_pos = o;
    o += align256(sizeof(int32_t) * (A ? A : 1));
    L->off_block_base = o;
    o += align256(sizeof(int32_t) * (bb ? bb : 1));
    L->off_tiles = o;
    o += align256(sizeof(int32_t) * ((size_t)E + 1));
    L->off_tile_expert = o;  // tile_expert then tile_order, tile_cap(A, E) each
    o += align256(sizeof(int32_t) * 2 * (size_t)tile_cap((long)A, E));
    L->total = o;
    return true;
}

moeq_status check_route(const moeq_route *r) {
    if (!r) return fail(MOEQ_EINVAL, "route is NULL");
    if (r->magic != kRouteMagic || !r->expert_offsets || !r->row_src || !r->slot_pos ||
        !r->block_base || !r->tile_offsets || !r->tile_expert)
        return fail(MOEQ_EINVAL, "route was not bound by moeq_route_bind");
    Layout L;
    if (!route_layout(r->T, r->E, r->top_k, &L) || L.blocks != r->token_blocks)
        return fail(MOEQ_EINVAL, "route shape (T=%d, E=%d, top_k=%d) is invalid", r->T, r->E,
                    r->top_k);
    return MOEQ_OK;
}

// Validate one expert cube against the route and the expected geometry.
// want_K / want_N < 0: not constrained.
moeq_status check_experts(const moeq_experts *w, const char *name, int route_E, int want_K,
                          int want_N, bool want_interleaved) {
    if (!w) return fail(MOEQ_EINVAL, "%s descriptor is NULL", name);
    if (w->experts < 1 || w->in_features < 1 || w->out_features < 1 || w->group_size < 1 ||
        w->expert_start < 0)
        return fail(MOEQ_EINVAL, "%s: sizes must be positive", name);
    if (route_E >= 0 && (w->expert_start != 0 || w->experts != route_E))
        return fail(MOEQ_ERANGE,
                    "%s: resident experts [%d, %d) must cover the routed IDs [0, %d)", name,
                    w->expert_start, w->expert_start + w->experts, route_E);
    if (want_K >= 0 && w->in_features != want_K)
        return fail(MOEQ_ESHAPE, "%s: in_features %d, expected %d", name, w->in_features, want_K);
    if (want_N >= 0 && w->out_features != want_N)
        return fail(MOEQ_ESHAPE, "%s: out_features %d, expected %d", name, w->out_features,
                    want_N);
    if (!w->qweight || !w->scales) return fail(MOEQ_EINVAL, "%s: NULL payload pointer", name);
    size_t n;
    // coefficient count must be a size some device could hold (2^48 codes)
    if (!mul_ok((size_t)w->experts, (size_t)w->in_features, &n) ||
        !mul_ok(n, (size_t)w->out_features, &n) || n > ((size_t)1 << 48))
        return fail(MOEQ_ESHAPE, "%s: size overflow", name);
    if (w->format == MOEQ_FMT_AWQ) {
        if (w->out_features % 8 != 0)
            return fail(MOEQ_ESHAPE, "%s: out_features %d not divisible by 8", name,
                        w->out_features);
        if (w->in_features % w->group_size != 0)
            return fail(MOEQ_ESHAPE, "%s: in_features %d not a whole number of groups of %d",
                        name, w->in_features, w->group_size);
        if (!w->qzeros) return fail(MOEQ_EINVAL, "%s: NULL qzeros", name);
        if (!valid_dtype(w->scale_dtype))
            return fail(MOEQ_EDTYPE, "%s: unknown scale dtype %d", name, (int)w->scale_dtype);
        if (w->group_size % 32 != 0)
            return fail(MOEQ_EUNSUPPORTED, "%s: group size %d (kernels take multiples of 32)",
                        name, w->group_size);
        if (w->interleaved_gate_up)
            return fail(MOEQ_EUNSUPPORTED, "%s: interleaved gate/up applies to MXFP4 banks",
                        name);
    } else if (w->format == MOEQ_FMT_MXFP4_BANK) {
        if (w->in_features % 32 != 0)
            return fail(MOEQ_ESHAPE, "%s: in_features %d not a whole number of 32-blocks", name,
                        w->in_features);
        if (w->group_size != 32)
            return fail(MOEQ_ESHAPE, "%s: MXFP4 block is 32, got group %d", name, w->group_size);
        if (w->qzeros) return fail(MOEQ_EINVAL, "%s: MXFP4 bank has no zero words", name);
        if (!w->bias) return fail(MOEQ_EINVAL, "%s: requires MXFP4 scales and BF16 bias", name);
        if ((w->interleaved_gate_up != 0) != want_interleaved)
            return fail(MOEQ_ESHAPE, want_interleaved
                                         ? "%s: requires an interleaved gate/up expert bank"
                                         : "%s: matrix-bank layout differs from routed role",
                        name);
    } else {
        return fail(MOEQ_EDTYPE, "%s: unknown format %d", name, (int)w->format);
    }
    return MOEQ_OK;
}

// Workspace of the unsorted-row calls: a route for (rows, experts, top_k 1), the local
// expert IDs, the sorted rows' expert IDs, and the sorted input and output rows.
struct UnsortedLayout {
    size_t route, local, rex, xs, ys, total;
};

bool unsorted_layout(int32_t rows, int32_t experts, int32_t K, int32_t N, int act,
                     UnsortedLayout *L) {
    Layout r;
    if (rows < 0 || K < 1 || N < 1 || !valid_dtype(act) || !route_layout(rows, experts, 1, &r))
        return false;
    size_t row_bytes;
    if (!mul_ok((size_t)(K > N ? K : N), dtype_bytes(act), &row_bytes)) return false;
    size_t tile;
    if (!mul_ok((size_t)(rows ? rows : 1), row_bytes, &tile)) return false;
    size_t o = 0;
    L->route = o;
    o += align256(r.total);
    L->local = o;
    o += align256(sizeof(uint32_t) * (size_t)(rows ? rows : 1));
    L->rex = o;
    o += align256(sizeof(uint32_t) * (size_t)(rows ? rows : 1));
    L->xs = o;
    o += align256(tile);
    L->ys = o;
    o += align256(tile);
    L->total = o;
    return true;
}

// Lower clamp bound of the gate: -clamp, or -inf for the one-sided variant.
float gate_lower(const moeq_swiglu &fn) {
    return fn.gate_one_sided ? -__builtin_inff() : -fn.clamp;
}

PackedOperand operand_of(const moeq_experts *w) {
    PackedOperand o;
    o.format = w->format;
    o.sdt = w->scale_dtype;
    o.qw = static_cast<const int32_t *>(w->qweight);
    o.qz = static_cast<const int32_t *>(w->qzeros);
    o.scales = w->scales;
    o.bias = w->bias;
    o.K = w->in_features;
    o.N = w->out_features;
    o.g = w->group_size;
    return o;
}

}  // namespace

namespace moeq {
moeq_status report_error(moeq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}
}  // namespace moeq

extern "C" {

const char *moeq_status_string(moeq_status s) {
    switch (s) {
    case MOEQ_OK: return "ok";
    case MOEQ_EINVAL: return "invalid argument";
    case MOEQ_ESHAPE: return "shape mismatch";
    case MOEQ_EDTYPE: return "dtype mismatch";
    case MOEQ_ERANGE: return "expert range";
    case MOEQ_EWORKSPACE: return "workspace";
    case MOEQ_EUNSUPPORTED: return "unsupported (no dense fallback)";
    case MOEQ_EDEVICE: return "device error";
    }
    return "unknown status";
}

const char *moeq_last_error(void) { return g_last_error; }

size_t moeq_route_workspace_bytes(int32_t T, int32_t E, int32_t top_k) {
    Layout L;
    return route_layout(T, E, top_k, &L) ? L.total : 0;
}

moeq_status moeq_route_bind(moeq_route *route, void *workspace, size_t bytes, int32_t T,
                            int32_t E, int32_t top_k) {
    if (!route || !workspace) return fail(MOEQ_EINVAL, "route or workspace is NULL");
    Layout L;
    if (!route_layout(T, E, top_k, &L))
        return fail(MOEQ_EINVAL, "invalid route shape T=%d E=%d top_k=%d", T, E, top_k);
    if ((uintptr_t)workspace % 256 != 0)
        return fail(MOEQ_EWORKSPACE, "workspace must be 256-byte aligned");
    if (bytes < L.total)
        return fail(MOEQ_EWORKSPACE, "workspace has %zu bytes, needs %zu", bytes, L.total);
    char *base = static_cast<char *>(workspace);
    memset(route, 0, sizeof *route);
    route->T = T;
    route->E = E;
    route->top_k = top_k;
    route->token_blocks = L.blocks;
    route->workspace = workspace;
    route->workspace_bytes = bytes;
    route->expert_offsets = reinterpret_cast<int32_t *>(base + L.off_offsets);
    route->row_src = reinterpret_cast<int32_t *>(base + L.off_row_src);
    route->slot_pos = reinterpret_cast<int32_t *>(base + L.off_slot_pos);
    route->block_base = reinterpret_cast<int32_t *>(base + L.off_block_base);
    route->tile_offsets = reinterpret_cast<int32_t *>(base + L.off_tiles);
    route->tile_expert = reinterpret_cast<int32_t *>(base + L.off_tile_expert);
    route->magic = kRouteMagic;
    return MOEQ_OK;
}

moeq_status moe_dispatch(const void *x, moeq_dtype act, int32_t T, int32_t K,
                         const void *logits, moeq_dtype logit_dtype, int32_t E,
                         const float *expert_bias, int32_t top_k, void *values, float *weights,
                         uint32_t *selected, uint32_t *row_experts, moeq_route *route,
                         void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (route->T != T || route->E != E || route->top_k != top_k)
        return fail(MOEQ_ESHAPE, "route bound for (T=%d, E=%d, top_k=%d), called with (%d, %d, %d)",
                    route->T, route->E, route->top_k, T, E, top_k);
    if (K < 1) return fail(MOEQ_EINVAL, "K must be positive");
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if (logit_dtype != MOEQ_F32 && logit_dtype != MOEQ_BF16)
        return fail(MOEQ_EDTYPE, "router logits are fp32 or bf16, got dtype %d", (int)logit_dtype);
    const bool lbf16 = logit_dtype == MOEQ_BF16;
    if (E > kMaxExperts || top_k > kMaxTopK)
        return fail(MOEQ_EUNSUPPORTED, "router implements E <= %d and top_k <= %d", kMaxExperts,
                    kMaxTopK);
    size_t row_bytes;
    if (!mul_ok((size_t)K, dtype_bytes(act), &row_bytes))
        return fail(MOEQ_ESHAPE, "size overflow");
    if (T == 0) return MOEQ_OK;
    if (!x || !logits || !values || !weights || !selected || !row_experts)
        return fail(MOEQ_EINVAL, "NULL tensor pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = device_status(launch_router(logits, lbf16, expert_bias, T, E, top_k, selected,
                                          weights, s),
                            "router")) != MOEQ_OK)
        return st;
    if (index_rows_fits(T, E, top_k, row_bytes, x, values))  // one more launch
        return device_status(launch_index_rows(x, row_bytes, selected, T, E, top_k, values,
                                               row_experts, route, s),
                             "dispatch");
    if ((st = device_status(launch_dispatch_index(selected, T, E, top_k, route, row_experts, s),
                            "dispatch index")) != MOEQ_OK)
        return st;
    if (scatter_rows_fits(row_bytes, top_k, x, values))  // each source row read once
        return device_status(launch_scatter_rows(x, row_bytes, T, top_k, route->slot_pos, values, s),
                             "row scatter");
    return device_status(launch_copy_rows(x, row_bytes, T * top_k, route->row_src, values, s),
                         "row copy");
}

moeq_status moe_dispatch_counts(const moeq_route *route, const int64_t *expert_prefix,
                                int32_t R, int64_t *counts, void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (R < 0 || !expert_prefix || (R > 0 && !counts))
        return fail(MOEQ_EINVAL, "bad prefix arguments");
    for (int32_t r = 0; r <= R; ++r) {
        if (expert_prefix[r] < 0 || expert_prefix[r] > route->E)
            return fail(MOEQ_ERANGE, "prefix[%d] = %lld outside [0, %d]", r,
                        (long long)expert_prefix[r], route->E);
        if (r > 0 && expert_prefix[r] < expert_prefix[r - 1])
            return fail(MOEQ_ERANGE, "prefix is not non-decreasing at %d", r);
    }
    if (R == 0) return MOEQ_OK;
    std::vector<int32_t> off((size_t)route->E + 1, 0);
    if (route->T > 0) {
        hipStream_t s = static_cast<hipStream_t>(stream);
        if ((st = device_status(hipMemcpyAsync(off.data(), route->expert_offsets,
                                               sizeof(int32_t) * off.size(),
                                               hipMemcpyDeviceToHost, s),
                                "offset copy")) != MOEQ_OK)
            return st;
        if ((st = device_status(hipStreamSynchronize(s), "stream sync")) != MOEQ_OK) return st;
    }
    for (int32_t r = 0; r < R; ++r)
        counts[r] = (int64_t)off[expert_prefix[r + 1]] - (int64_t)off[expert_prefix[r]];
    return MOEQ_OK;
}

moeq_status awq_grouped_swiglu(const moeq_route *route, const void *values, moeq_dtype act,
                               const moeq_experts *gate, const moeq_experts *up,
                               moeq_swiglu fn, void *h, void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if (!gate) return fail(MOEQ_EINVAL, "gate descriptor is NULL");
    const bool bank = gate->format == MOEQ_FMT_MXFP4_BANK;
    if ((st = check_experts(gate, "gate", route->E, -1, -1, bank)) != MOEQ_OK) return st;
    int I;
    if (bank) {
        if (up) return fail(MOEQ_EINVAL, "an interleaved gate/up bank takes no up descriptor");
        if (gate->out_features % 2 != 0)
            return fail(MOEQ_ESHAPE, "gate/up bank rows %d are not 2*I", gate->out_features);
        I = gate->out_features / 2;
    } else {
        if ((st = check_experts(up, "up", route->E, gate->in_features, gate->out_features,
                                false)) != MOEQ_OK)
            return st;
        if (up->format != MOEQ_FMT_AWQ)
            return fail(MOEQ_EDTYPE, "gate and up must share one format");
        if (up->scale_dtype != gate->scale_dtype || up->group_size != gate->group_size)
            return fail(MOEQ_EDTYPE, "gate and up must share scale dtype and group size");
        if ((up->bias == nullptr) != (gate->bias == nullptr))
            return fail(MOEQ_EINVAL, "gate and up must both have or both lack a bias");
        I = gate->out_features;
    }
    if (!(fn.clamp >= 0.0f) || !(fn.alpha == fn.alpha) || !(fn.up_offset == fn.up_offset) ||
        (fn.gate_one_sided != 0 && fn.gate_one_sided != 1))
        return fail(MOEQ_EINVAL, "bad SwiGLU parameters");
    const int A = route->T * route->top_k;
    if (A == 0) return MOEQ_OK;
    if (!values || !h) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    ProjProblem p{};
    p.in = values;
    p.out = h;
    p.offsets = route->expert_offsets;
    p.tile_offsets = route->tile_offsets;
    p.tile_expert = route->tile_expert;
    p.tile_order = route->tile_expert + tile_cap((long)route->T * route->top_k, route->E);
    p.rows = A;
    p.E = route->E;
    p.act = act;
    p.Kred = gate->in_features;
    p.Nout = I;
    p.w0 = operand_of(gate);
    p.w1 = bank ? p.w0 : operand_of(up);
    p.mode = bank ? PROJ_BANK_SWIGLU : PROJ_SWIGLU;
    p.clamp = fn.clamp;
    p.gate_lo = gate_lower(fn);
    p.alpha = fn.alpha;
    p.up_offset = fn.up_offset;
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool handled = false;
    hipError_t err = launch_fast_swiglu(p, s, &handled);
    if (!handled) err = launch_proj_generic(p, s);
    return device_status(err, "gate/up projection");
}

moeq_status awq_grouped_down(const moeq_route *route, const void *h, moeq_dtype act,
                             const moeq_experts *down, void *y, void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if ((st = check_experts(down, "down", route->E, -1, -1, false)) != MOEQ_OK) return st;
    const int A = route->T * route->top_k;
    if (A == 0) return MOEQ_OK;
    if (!h || !y) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    ProjProblem p{};
    p.in = h;
    p.out = y;
    p.offsets = route->expert_offsets;
    p.tile_offsets = route->tile_offsets;
    p.tile_expert = route->tile_expert;
    p.tile_order = route->tile_expert + tile_cap((long)route->T * route->top_k, route->E);
    p.rows = A;
    p.E = route->E;
    p.act = act;
    p.Kred = down->in_features;
    p.Nout = down->out_features;
    p.w0 = operand_of(down);
    p.w1 = p.w0;
    p.mode = PROJ_PLAIN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool handled = false;
    hipError_t err = launch_fast_plain(p, s, &handled);
    if (!handled) err = launch_proj_generic(p, s);
    return device_status(err, "down projection");
}

moeq_status moe_combine(const moeq_route *route, const void *y, moeq_dtype act, int32_t K,
                        const float *weights, void *out, void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if (K < 1) return fail(MOEQ_EINVAL, "K must be positive");
    if (route->top_k > kMaxTopK)
        return fail(MOEQ_EUNSUPPORTED, "combine implements top_k <= %d", kMaxTopK);
    if (route->T == 0) return MOEQ_OK;
    if (!y || !weights || !out) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    return device_status(launch_combine(y, act, weights, route->slot_pos, route->T, route->top_k,
                                        K, out, static_cast<hipStream_t>(stream)),
                         "combine");
}

moeq_status awq_input_backward(const moeq_route *route, const void *grad, moeq_dtype gdt,
                               int32_t rows, const moeq_experts *w, void *grad_in,
                               void *stream) {
    moeq_status st;
    if (route) {
        if ((st = check_route(route)) != MOEQ_OK) return st;
        if (rows != route->T * route->top_k)
            return fail(MOEQ_ESHAPE, "rows %d != routed rows %d", rows, route->T * route->top_k);
        if ((st = check_experts(w, "weights", route->E, -1, -1, false)) != MOEQ_OK) return st;
    } else {
        if (rows < 0) return fail(MOEQ_EINVAL, "rows must be >= 0");
        if ((st = check_experts(w, "weights", -1, -1, -1, false)) != MOEQ_OK) return st;
        if (w->experts != 1)
            return fail(MOEQ_ERANGE, "without a route the cube must hold one expert, has %d",
                        w->experts);
    }
    if (w->format != MOEQ_FMT_AWQ)
        return fail(MOEQ_EUNSUPPORTED, "input VJP is implemented for AWQ cubes");
    if (!valid_dtype(gdt)) return fail(MOEQ_EDTYPE, "unknown gradient dtype %d", (int)gdt);
    if (rows == 0) return MOEQ_OK;
    if (!grad || !grad_in) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    ProjProblem p{};
    p.in = grad;
    p.out = grad_in;
    p.offsets = route ? route->expert_offsets : nullptr;
    p.tile_offsets = route ? route->tile_offsets : nullptr;
    p.tile_expert = route ? route->tile_expert : nullptr;
    p.tile_order = route ? route->tile_expert + tile_cap((long)route->T * route->top_k, route->E)
                         : nullptr;
    p.rows = rows;
    p.E = route ? route->E : 1;
    p.act = gdt;
    p.Kred = w->out_features;
    p.Nout = w->in_features;
    p.w0 = operand_of(w);
    p.w1 = p.w0;
    p.mode = PROJ_INPUT_VJP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return device_status(vjp_fits(p) ? launch_vjp(p, s) : launch_proj_generic(p, s),
                         "input VJP");
}

// ---------------------------------------------------------------- backward path

moeq_status moe_combine_backward(const moeq_route *route, const void *y, moeq_dtype act,
                                 int32_t K, const float *weights, const void *grad,
                                 void *grad_y, float *grad_weights, void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if (K < 1) return fail(MOEQ_EINVAL, "K must be positive");
    if (route->top_k > kMaxTopK)
        return fail(MOEQ_EUNSUPPORTED, "combine VJP implements top_k <= %d", kMaxTopK);
    if (route->T == 0 || (!grad_y && !grad_weights)) return MOEQ_OK;
    if (!grad || !weights || !y)
        return fail(MOEQ_EINVAL, "NULL tensor pointer");
    return device_status(launch_combine_backward(y, act, weights, route->slot_pos, grad, route->T,
                                                 route->top_k, K, grad_y, grad_weights,
                                                 static_cast<hipStream_t>(stream)),
                         "combine backward");
}

moeq_status moe_dispatch_backward(const moeq_route *route, const void *grad, moeq_dtype act,
                                  int32_t K, void *grad_x, void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if (K < 1) return fail(MOEQ_EINVAL, "K must be positive");
    if (route->top_k > kMaxTopK)
        return fail(MOEQ_EUNSUPPORTED, "COPY VJP implements top_k <= %d", kMaxTopK);
    if (route->T == 0) return MOEQ_OK;
    if (!grad || !grad_x) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    return device_status(launch_dispatch_backward(grad, act, route->slot_pos, route->T,
                                                  route->top_k, K, grad_x,
                                                  static_cast<hipStream_t>(stream)),
                         "dispatch backward");
}

moeq_status moe_dispatch_weights_backward(const moeq_route *route, const uint32_t *selected,
                                          const float *weights, const float *grad_weights,
                                          float *grad_logits, void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (route->top_k > kMaxTopK)
        return fail(MOEQ_EUNSUPPORTED, "logit VJP implements top_k <= %d", kMaxTopK);
    if (route->T == 0) return MOEQ_OK;
    if (!selected || !weights || !grad_weights || !grad_logits)
        return fail(MOEQ_EINVAL, "NULL tensor pointer");
    return device_status(launch_weights_backward(selected, weights, grad_weights, route->T,
                                                 route->E, route->top_k, grad_logits,
                                                 static_cast<hipStream_t>(stream)),
                         "weights backward");
}

size_t awq_swiglu_input_backward_workspace_bytes(int32_t rows, int32_t I, moeq_dtype act) {
    if (rows < 0 || I < 1 || !valid_dtype(act)) return 0;
    size_t n;
    if (!mul_ok((size_t)rows, (size_t)I, &n) || !mul_ok(n, dtype_bytes(act), &n)) return 0;
    return 3 * align256(n ? n : 1);
}

moeq_status awq_swiglu_input_backward(const moeq_route *route, const void *values,
                                      moeq_dtype act, const moeq_experts *gate,
                                      const moeq_experts *up, const moeq_experts *down,
                                      moeq_swiglu fn, const void *grad, void *grad_values,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if ((st = check_experts(gate, "gate", route->E, -1, -1, false)) != MOEQ_OK) return st;
    const int K = gate->in_features, I = gate->out_features;
    if ((st = check_experts(up, "up", route->E, K, I, false)) != MOEQ_OK) return st;
    if ((st = check_experts(down, "down", route->E, I, K, false)) != MOEQ_OK) return st;
    if (gate->format != MOEQ_FMT_AWQ || up->format != MOEQ_FMT_AWQ ||
        down->format != MOEQ_FMT_AWQ)
        return fail(MOEQ_EUNSUPPORTED, "the chain VJP is implemented for AWQ cubes");
    if (up->scale_dtype != gate->scale_dtype || up->group_size != gate->group_size)
        return fail(MOEQ_EDTYPE, "gate and up must share scale dtype and group size");
    if ((up->bias == nullptr) != (gate->bias == nullptr))
        return fail(MOEQ_EINVAL, "gate and up must both have or both lack a bias");
    if (!(fn.clamp >= 0.0f) || !(fn.alpha == fn.alpha) || !(fn.up_offset == fn.up_offset) ||
        (fn.gate_one_sided != 0 && fn.gate_one_sided != 1))
        return fail(MOEQ_EINVAL, "bad SwiGLU parameters");
    const int A = route->T * route->top_k;
    const size_t need = awq_swiglu_input_backward_workspace_bytes(A, I, act);
    if (need == 0) return fail(MOEQ_ESHAPE, "size overflow");
    if (A == 0) return MOEQ_OK;
    if (!values || !grad || !grad_values) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    if (!workspace) return fail(MOEQ_EINVAL, "workspace is NULL");
    if ((uintptr_t)workspace % 256 != 0)
        return fail(MOEQ_EWORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(MOEQ_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    char *dh = static_cast<char *>(workspace);  // [A, I] each
    char *gg = dh + need / 3;                   // G, then dG
    char *uu = gg + need / 3;                   // U, then dU
    hipStream_t s = static_cast<hipStream_t>(stream);
    ProjProblem p{};
    p.offsets = route->expert_offsets;
    p.tile_offsets = route->tile_offsets;
    p.tile_expert = route->tile_expert;
    p.tile_order = route->tile_expert + tile_cap((long)route->T * route->top_k, route->E);
    p.rows = A;
    p.E = route->E;
    p.act = act;
    // dh = grad . Wd^T
    ProjProblem q = p;
    q.in = grad;
    q.out = dh;
    q.Kred = K;
    q.Nout = I;
    q.w0 = q.w1 = operand_of(down);
    q.mode = PROJ_INPUT_VJP;
    if ((st = device_status(vjp_fits(q) ? launch_vjp(q, s) : launch_proj_generic(q, s),
                            "down input VJP")) != MOEQ_OK)
        return st;
    // G and U recomputed as in the forward (bias added, rounded to act), with the
    // SwiGLU VJP in the gate/up kernel's epilogue: dG, dU straight from dh
    q = p;
    q.in = values;
    q.in2 = dh;
    q.out = gg;
    q.out2 = uu;
    q.Kred = K;
    q.Nout = I;
    q.w0 = operand_of(gate);
    q.w1 = operand_of(up);
    q.mode = PROJ_SWIGLU;
    q.clamp = fn.clamp;
    q.gate_lo = gate_lower(fn);
    q.alpha = fn.alpha;
    q.up_offset = fn.up_offset;
    bool fused = false;
    if ((st = device_status(launch_fast_swiglu(q, s, &fused), "gate/up backward epilogue")) !=
        MOEQ_OK)
        return st;
    // otherwise: G and U by two plain projections, then the SwiGLU VJP in place
    for (int c = 0; c < 2 && !fused; ++c) {
        q = p;
        q.in = values;
        q.out = c == 0 ? gg : uu;
        q.Kred = K;
        q.Nout = I;
        q.w0 = q.w1 = operand_of(c == 0 ? gate : up);
        q.mode = PROJ_PLAIN;
        bool handled = false;
        hipError_t err = launch_fast_plain(q, s, &handled);
        if (!handled) err = launch_proj_generic(q, s);
        if ((st = device_status(err, "gate/up recompute")) != MOEQ_OK) return st;
    }
    if (!fused &&
        (st = device_status(launch_swiglu_vjp(gg, uu, dh, act, (size_t)A * I, fn.clamp,
                                              gate_lower(fn), fn.alpha, fn.up_offset, s),
                            "SwiGLU VJP")) != MOEQ_OK)
        return st;
    // grad_values = dG . Wg^T + dU . Wu^T
    q = p;
    q.in = gg;
    q.in2 = uu;
    q.out = grad_values;
    q.Kred = I;
    q.Nout = K;
    q.w0 = operand_of(gate);
    q.w1 = operand_of(up);
    q.mode = PROJ_INPUT_VJP2;
    return device_status(vjp_fits(q) ? launch_vjp(q, s) : launch_proj_generic(q, s),
                         "gate/up input VJP");
}

// ---------------------------------------------------------------- MXFP8 activations

size_t mx8_workspace_bytes(int32_t rows, int32_t K) {
    if (rows < 0 || K < 32 || K % 32 != 0) return 0;
    size_t n;
    if (!mul_ok((size_t)rows, (size_t)K, &n)) return 0;
    // codes, then scale rows padded to 16 bytes
    const size_t sstride = ((size_t)K / 32 + 15) / 16 * 16;
    return align256(n ? n : 1) + align256((size_t)(rows ? rows : 1) * sstride);
}

moeq_status mx8_quantize(const void *x, moeq_dtype act, int32_t rows, int32_t K, uint8_t *q,
                         uint8_t *s, void *stream) {
    if (act != MOEQ_BF16) return fail(MOEQ_EUNSUPPORTED, "MXFP8 quantization takes bf16 rows");
    if (rows < 0 || K < 32 || K % 32 != 0)
        return fail(MOEQ_ESHAPE, "rows >= 0 and K a positive multiple of 32 (K = %d)", K);
    if (rows == 0) return MOEQ_OK;
    if (!x || !q || !s) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    if ((uintptr_t)x % 16 != 0 || (uintptr_t)q % 16 != 0)
        return fail(MOEQ_EINVAL, "rows must be 16-byte aligned");
    return device_status(
        launch_mx8_quant(x, rows, K, q, s, K / 32, static_cast<hipStream_t>(stream)),
        "MXFP8 quantization");
}

namespace {

moeq_status mx8_check(const moeq_route *route, const void *in, moeq_dtype act,
                      const moeq_experts *w, bool swiglu, void *workspace, size_t bytes) {
    moeq_status st = check_route(route);
    if (st != MOEQ_OK) return st;
    if (!w) return fail(MOEQ_EINVAL, "bank descriptor is NULL");
    if (w->format != MOEQ_FMT_MXFP4_BANK)
        return fail(MOEQ_EUNSUPPORTED, "the block-scaled MFMA path takes MXFP4 banks");
    if ((st = check_experts(w, swiglu ? "gate/up bank" : "down bank", route->E, -1, -1,
                            swiglu)) != MOEQ_OK)
        return st;
    if (act != MOEQ_BF16) return fail(MOEQ_EUNSUPPORTED, "MXFP8 activations come from bf16 rows");
    if (w->out_features % 64 != 0)
        return fail(MOEQ_EUNSUPPORTED, "bank rows %d are not a multiple of 64", w->out_features);
    if (w->in_features > 4096)
        return fail(MOEQ_EUNSUPPORTED, "in_features %d above 4096", w->in_features);
    if ((uintptr_t)w->scales % 16 != 0 || (uintptr_t)w->qweight % 16 != 0)
        return fail(MOEQ_EINVAL, "bank blocks and scales must be 16-byte aligned");
    const int A = route->T * route->top_k;
    if (A == 0) return MOEQ_OK;
    if (!in) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    if (!workspace) return fail(MOEQ_EINVAL, "workspace is NULL");
    if ((uintptr_t)workspace % 256 != 0)
        return fail(MOEQ_EWORKSPACE, "workspace must be 256-byte aligned");
    const size_t need = mx8_workspace_bytes(A, w->in_features);
    if (bytes < need) return fail(MOEQ_EWORKSPACE, "workspace has %zu bytes, needs %zu", bytes, need);
    return MOEQ_OK;
}

moeq_status mx8_run(const moeq_route *route, const void *in, const moeq_experts *w, bool swiglu,
                    moeq_swiglu fn, void *out, void *workspace, hipStream_t s) {
    const int A = route->T * route->top_k, K = w->in_features;
    uint8_t *q = static_cast<uint8_t *>(workspace);
    uint8_t *qs = q + align256((size_t)A * K);
    const int sstride = (K / 32 + 15) / 16 * 16;
    moeq_status st;
    if ((st = device_status(launch_mx8_quant(in, A, K, q, qs, sstride, s),
                            "MXFP8 quantization")) != MOEQ_OK)
        return st;
    return device_status(launch_mx8_gemm(q, qs, sstride, A, K, operand_of(w),
                                         route->expert_offsets,
                                         route->tile_offsets, route->tile_expert, route->E,
                                         swiglu, swiglu ? w->out_features / 2 : w->out_features,
                                         fn.clamp, gate_lower(fn), fn.alpha, fn.up_offset, out,
                                         s),
                         "block-scaled projection");
}

}  // namespace

moeq_status mx8_grouped_swiglu(const moeq_route *route, const void *values, moeq_dtype act,
                               const moeq_experts *gate_up, moeq_swiglu fn, void *h,
                               void *workspace, size_t workspace_bytes, void *stream) {
    moeq_status st = mx8_check(route, values, act, gate_up, true, workspace, workspace_bytes);
    if (st != MOEQ_OK) return st;
    if (!(fn.clamp >= 0.0f) || !(fn.alpha == fn.alpha) || !(fn.up_offset == fn.up_offset) ||
        (fn.gate_one_sided != 0 && fn.gate_one_sided != 1))
        return fail(MOEQ_EINVAL, "bad SwiGLU parameters");
    if (route->T == 0) return MOEQ_OK;
    if (!h) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    return mx8_run(route, values, gate_up, true, fn, h, workspace,
                   static_cast<hipStream_t>(stream));
}

moeq_status mx8_grouped_down(const moeq_route *route, const void *h, moeq_dtype act,
                             const moeq_experts *down, void *y, void *workspace,
                             size_t workspace_bytes, void *stream) {
    moeq_status st = mx8_check(route, h, act, down, false, workspace, workspace_bytes);
    if (st != MOEQ_OK) return st;
    if (route->T == 0) return MOEQ_OK;
    if (!y) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    return mx8_run(route, h, down, false, moeq_swiglu{0.0f, 1.0f, 0.0f, 0}, y, workspace,
                   static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- unsorted rows

size_t awq_expert_workspace_bytes(int32_t rows, int32_t experts, int32_t K, int32_t N,
                                  moeq_dtype act) {
    UnsortedLayout L;
    return unsorted_layout(rows, experts, K, N, act, &L) ? L.total : 0;
}

namespace {

// Shared by awq_expert_forward and awq_expert_input_backward: validation of the
// IDs on the host, then the local stable sort by expert (route of top_k 1) and the
// gather of the incoming rows into expert order.
moeq_status unsorted_prepare(const void *in, int act, int32_t rows, int32_t in_cols,
                             const uint32_t *global_ids, const moeq_experts *w, int32_t K,
                             int32_t N, void *workspace, size_t workspace_bytes, hipStream_t s,
                             moeq_route *route, UnsortedLayout *L) {
    moeq_status st;
    if (!unsorted_layout(rows, w->experts, K, N, act, L))
        return fail(MOEQ_ESHAPE, "invalid sizes or size overflow");
    if (!workspace) return fail(MOEQ_EINVAL, "workspace is NULL");
    if ((uintptr_t)workspace % 256 != 0)
        return fail(MOEQ_EWORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < L->total)
        return fail(MOEQ_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                    L->total);
    if (!in || !global_ids) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    // the pages return an error for an ID outside the resident range: check on the host
    std::vector<uint32_t> ids((size_t)rows);
    if ((st = device_status(hipMemcpyAsync(ids.data(), global_ids, sizeof(uint32_t) * ids.size(),
                                           hipMemcpyDeviceToHost, s),
                            "ID copy")) != MOEQ_OK)
        return st;
    if ((st = device_status(hipStreamSynchronize(s), "stream sync")) != MOEQ_OK) return st;
    const uint64_t lo = (uint64_t)w->expert_start, hi = lo + (uint64_t)w->experts;
    for (int32_t t = 0; t < rows; ++t)
        if (ids[t] < lo || ids[t] >= hi)
            return fail(MOEQ_ERANGE, "global_ids[%d] = %u outside the resident experts [%llu, %llu)",
                        t, ids[t], (unsigned long long)lo, (unsigned long long)hi);
    char *base = static_cast<char *>(workspace);
    if ((st = moeq_route_bind(route, base + L->route, workspace_bytes - L->route, rows,
                              w->experts, 1)) != MOEQ_OK)
        return st;
    uint32_t *local = reinterpret_cast<uint32_t *>(base + L->local);
    uint32_t *rex = reinterpret_cast<uint32_t *>(base + L->rex);
    if ((st = device_status(launch_local_ids(global_ids, rows, w->expert_start, local, s),
                            "local IDs")) != MOEQ_OK)
        return st;
    if ((st = device_status(launch_dispatch_index(local, rows, w->experts, 1, route, rex, s),
                            "local sort")) != MOEQ_OK)
        return st;
    return device_status(launch_copy_rows(in, (size_t)in_cols * dtype_bytes(act), rows,
                                          route->row_src, base + L->xs, s),
                         "row gather");
}

}  // namespace

moeq_status awq_expert_forward(const void *x, moeq_dtype act, int32_t rows,
                               const uint32_t *global_ids, const moeq_experts *w, void *y,
                               void *workspace, size_t workspace_bytes, void *stream) {
    moeq_status st;
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if (rows < 0) return fail(MOEQ_EINVAL, "rows must be >= 0");
    if ((st = check_experts(w, "weights", -1, -1, -1, false)) != MOEQ_OK) return st;
    if (w->experts > kMaxExperts)
        return fail(MOEQ_EUNSUPPORTED, "the local sort implements up to %d experts", kMaxExperts);
    const int K = w->in_features, N = w->out_features;
    if (rows == 0) return MOEQ_OK;
    if (!y) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    moeq_route route;
    UnsortedLayout L;
    if ((st = unsorted_prepare(x, act, rows, K, global_ids, w, K, N, workspace, workspace_bytes,
                               s, &route, &L)) != MOEQ_OK)
        return st;
    char *base = static_cast<char *>(workspace);
    ProjProblem p{};
    p.in = base + L.xs;
    p.out = base + L.ys;
    p.offsets = route.expert_offsets;
    p.tile_offsets = route.tile_offsets;
    p.tile_expert = route.tile_expert;
    p.tile_order = route.tile_expert + tile_cap((long)route.T * route.top_k, route.E);
    p.rows = rows;
    p.E = w->experts;
    p.act = act;
    p.Kred = K;
    p.Nout = N;
    p.w0 = p.w1 = operand_of(w);
    p.mode = PROJ_PLAIN;
    bool handled = false;
    hipError_t err = launch_fast_plain(p, s, &handled);
    if (!handled) err = launch_proj_generic(p, s);
    if ((st = device_status(err, "projection")) != MOEQ_OK) return st;
    // inverse permutation: incoming row t is sorted row slot_pos[t]
    return device_status(launch_copy_rows(base + L.ys, (size_t)N * dtype_bytes(act), rows,
                                          route.slot_pos, y, s),
                         "row restore");
}

moeq_status awq_expert_input_backward(const void *grad, moeq_dtype gdt, int32_t rows,
                                      const uint32_t *global_ids, const moeq_experts *w,
                                      void *grad_in, void *workspace, size_t workspace_bytes,
                                      void *stream) {
    moeq_status st;
    if (!valid_dtype(gdt)) return fail(MOEQ_EDTYPE, "unknown gradient dtype %d", (int)gdt);
    if (rows < 0) return fail(MOEQ_EINVAL, "rows must be >= 0");
    if ((st = check_experts(w, "weights", -1, -1, -1, false)) != MOEQ_OK) return st;
    if (w->format != MOEQ_FMT_AWQ)
        return fail(MOEQ_EUNSUPPORTED, "input VJP is implemented for AWQ cubes");
    if (w->experts > kMaxExperts)
        return fail(MOEQ_EUNSUPPORTED, "the local sort implements up to %d experts", kMaxExperts);
    const int K = w->in_features, N = w->out_features;
    if (rows == 0) return MOEQ_OK;
    if (!grad_in) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    moeq_route route;
    UnsortedLayout L;
    if ((st = unsorted_prepare(grad, gdt, rows, N, global_ids, w, K, N, workspace,
                               workspace_bytes, s, &route, &L)) != MOEQ_OK)
        return st;
    char *base = static_cast<char *>(workspace);
    ProjProblem p{};
    p.in = base + L.xs;
    p.out = base + L.ys;
    p.offsets = route.expert_offsets;
    p.tile_offsets = route.tile_offsets;
    p.tile_expert = route.tile_expert;
    p.tile_order = route.tile_expert + tile_cap((long)route.T * route.top_k, route.E);
    p.rows = rows;
    p.E = w->experts;
    p.act = gdt;
    p.Kred = N;
    p.Nout = K;
    p.w0 = p.w1 = operand_of(w);
    p.mode = PROJ_INPUT_VJP;
    if ((st = device_status(vjp_fits(p) ? launch_vjp(p, s) : launch_proj_generic(p, s),
                            "input VJP")) != MOEQ_OK)
        return st;
    return device_status(launch_copy_rows(base + L.ys, (size_t)K * dtype_bytes(gdt), rows,
                                          route.slot_pos, grad_in, s),
                         "row restore");
}

size_t frozen_awq_workspace_bytes(int32_t rows) {
    if (rows < 0) return 0;
    // offsets [2], m-tile prefix [2], expert of each m-tile
    return align256(2 * sizeof(int32_t)) * 2 +
           align256(sizeof(int32_t) * 2 * (size_t)tile_cap(rows, 1));
}

moeq_status frozen_awq_forward(const void *x, moeq_dtype act, int32_t rows,
                               const moeq_experts *w, void *y, void *workspace,
                               size_t workspace_bytes, void *stream) {
    moeq_status st;
    if (!valid_dtype(act)) return fail(MOEQ_EDTYPE, "unknown activation dtype %d", (int)act);
    if (rows < 0) return fail(MOEQ_EINVAL, "rows must be >= 0");
    if ((st = check_experts(w, "weights", -1, -1, -1, false)) != MOEQ_OK) return st;
    if (w->experts != 1)
        return fail(MOEQ_ERANGE, "a single frozen projection holds one expert, has %d",
                    w->experts);
    if (rows == 0) return MOEQ_OK;
    if (!x || !y) return fail(MOEQ_EINVAL, "NULL tensor pointer");
    const size_t need = frozen_awq_workspace_bytes(rows);
    if (!workspace) return fail(MOEQ_EINVAL, "workspace is NULL");
    if ((uintptr_t)workspace % 256 != 0)
        return fail(MOEQ_EWORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(MOEQ_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    char *base = static_cast<char *>(workspace);
    int32_t *offsets = reinterpret_cast<int32_t *>(base);
    int32_t *tile_offsets = reinterpret_cast<int32_t *>(base + align256(2 * sizeof(int32_t)));
    int32_t *tile_expert = reinterpret_cast<int32_t *>(base + 2 * align256(2 * sizeof(int32_t)));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((st = device_status(launch_single_tiles(rows, offsets, tile_offsets, tile_expert, s),
                            "row map")) != MOEQ_OK)
        return st;
    ProjProblem p{};
    p.in = x;
    p.out = y;
    p.offsets = offsets;
    p.tile_offsets = tile_offsets;
    p.tile_expert = tile_expert;
    p.tile_order = tile_expert + tile_cap(rows, 1);
    p.rows = rows;
    p.E = 1;
    p.act = act;
    p.Kred = w->in_features;
    p.Nout = w->out_features;
    p.w0 = p.w1 = operand_of(w);
    p.mode = PROJ_PLAIN;
    bool handled = false;
    hipError_t err = launch_fast_plain(p, s, &handled);
    if (!handled) err = launch_proj_generic(p, s);
    return device_status(err, "frozen projection");
}

}  // extern "C"
