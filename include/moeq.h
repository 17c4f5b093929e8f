/*
 * moeq.h -- C-ABI of libmoeq.so: the routed mixture-of-experts expert FFN over
 * frozen packed 4-bit expert weights, on one AMD Instinct MI355X (gfx950).
 *
 * The forward path is five calls on one stream:
 *   moe_dispatch         router top-k + FP32 softmax weights + COPY dispatch
 *   awq_grouped_swiglu   grouped gate/up projections dequantised in registers,
 *                        storage-rounded SwiGLU
 *   awq_grouped_down     grouped down projection
 *   moe_combine          ascending expert-ID weighted combine back to tokens
 * plus moe_dispatch_counts (range counts on the host) and awq_input_backward
 * (input VJP through the same rounded coefficients).
 *
 * The first-order backward path runs the forward calls' VJPs in reverse:
 *   moe_combine_backward           expert-row and FP32 weight derivatives
 *   awq_swiglu_input_backward      input VJP through down, SwiGLU and gate/up
 *   moe_dispatch_backward          COPY VJP back to the source tokens
 *   moe_dispatch_weights_backward  fixed-selection router-logit VJP
 *
 * Rows in any order (the expert-parallel receive side, and single projections):
 *   awq_expert_forward, awq_expert_input_backward, frozen_awq_forward
 *
 * Sources (the pages the operations are defined on):
 *   ruda-tensor 0.21.38 src/moe_exchange.rs    -- MoeDispatched, MoeDispatchOps
 *   ruda-tensor 0.21.34 src/packed_experts.rs  -- AwqExpertOptions,
 *       AwqExpertPayload, PackedExpertPayload, PackedExpertAutodiffError,
 *       FrozenPackedExpertOps
 *   ruda-tensor 0.21.33 src/frozen_awq.rs      -- FrozenAwqError, FrozenAwqOps
 *   libmir-metal 0.3.0 src/engine/clamped_routed/experts/native.rs
 *       -- ExpertLayout::Native, native_layout / companions / validate
 *
 * Conventions for every call:
 *  - All tensor arguments are device pointers to contiguous row-major memory
 *    owned by the caller.  The library allocates no device memory, frees
 *    nothing, and does not synchronise, except moe_dispatch_counts, which
 *    returns host values, and awq_expert_forward / awq_expert_input_backward,
 *    which validate their expert IDs on the host; these synchronise `stream`.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All kernels of a
 *    call are enqueued on it; the call returns once they are enqueued.
 *  - Arguments are validated on the host before anything is enqueued.  On a
 *    validation error the call returns a negative status, enqueues nothing and
 *    leaves every output untouched; moeq_last_error() then names the check.
 *  - A launch failure returns MOEQ_EDEVICE (the pages' Native(E) error).
 *  - There is never a dense fallback or a requantisation (frozen_awq.rs,
 *    FrozenAwqError::Native): a shape or dtype the kernels do not implement
 *    returns MOEQ_EUNSUPPORTED.
 *  - Calls on one stream are ordered; calls that share output buffers on
 *    different streams race.
 *  - Activation and gradient storage (`act`, `gdt`) is F32, F16 or BF16 unless a
 *    call says otherwise (frozen_awq.rs: the input storage may differ from the
 *    scales').  The MFMA kernels take BF16 rows; F32 and F16 rows run on the
 *    fp32 VALU kernels with the same rounding points.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOEQ_OK = 0,
    MOEQ_EINVAL = -1,        /* NULL pointer, negative size, unbound route      */
    MOEQ_ESHAPE = -2,        /* inconsistent or non-divisible shapes, overflow  */
    MOEQ_EDTYPE = -3,        /* unknown or mismatched storage type              */
    MOEQ_ERANGE = -4,        /* expert range / prefix outside the routed IDs   */
    MOEQ_EWORKSPACE = -5,    /* route workspace too small or misaligned         */
    MOEQ_EUNSUPPORTED = -6,  /* valid input the kernels do not implement        */
    MOEQ_EDEVICE = -7        /* HIP launch or copy failure                      */
} moeq_status;

/* The *_RANGE_ enumerators below are not valid values.  They give each enum the
 * whole int32 range, so that an unknown value from a caller is still a value of
 * the type (in C++ a value outside an enum's range is undefined), which the
 * validation then rejects with MOEQ_EDTYPE or MOEQ_EINVAL. */
typedef enum {
    MOEQ_F32 = 0, MOEQ_F16 = 1, MOEQ_BF16 = 2,
    MOEQ_DTYPE_RANGE_MIN_ = -2147483647 - 1, MOEQ_DTYPE_RANGE_MAX_ = 2147483647
} moeq_dtype;

/* Packed payload tag (packed_experts.rs PackedExpertPayload): AWQ I32 words,
 * or an MXFP4 expert bank (native.rs ExpertLayout::Native). */
typedef enum {
    MOEQ_FMT_AWQ = 0, MOEQ_FMT_MXFP4_BANK = 1,
    MOEQ_FMT_RANGE_MIN_ = -2147483647 - 1, MOEQ_FMT_RANGE_MAX_ = 2147483647
} moeq_format;

/*
 * Route state: the "private native row mappings" of moe_exchange.rs
 * (MoeDispatchOps::MoeDispatchState), produced only by moe_dispatch and read by
 * the grouped projections, the counts and the combine.  A host struct holding
 * device pointers into one caller-owned workspace (moeq_route_bind).
 */
typedef struct moeq_route {
    int32_t T, E, top_k;       /* routed shape; every consumer checks it        */
    int32_t token_blocks;      /* internal: token blocks of the stable scatter  */
    void *workspace;           /* device, caller-owned                           */
    size_t workspace_bytes;
    int32_t *expert_offsets;   /* [E+1] first sorted row of each expert; [E]=A  */
    int32_t *row_src;          /* [A]   source token of sorted row p            */
    int32_t *slot_pos;         /* [T*top_k] sorted row of assignment (t, j)     */
    int32_t *block_base;       /* internal [token_blocks*E]                      */
    int32_t *tile_offsets;     /* internal [E+1] prefix of ceil(rows_e / 128)    */
    int32_t *tile_expert;      /* internal [2*(ceil(A/128)+E)]: expert of each     */
                               /* m-tile, then the m-tiles in scheduling order  */
    uint32_t magic;            /* set by moeq_route_bind                         */
} moeq_route;

/* Bytes of device workspace a route of this shape needs (0 on invalid sizes). */
size_t moeq_route_workspace_bytes(int32_t T, int32_t E, int32_t top_k);

/* Lay a route out in `workspace` (device memory, >= the bytes above, 256-byte
 * aligned).  Host only; enqueues nothing.  Errors: EINVAL (NULL, sizes < 0 or
 * top_k outside [1, E]), EWORKSPACE (too small / misaligned). */
moeq_status moeq_route_bind(moeq_route *route, void *workspace, size_t bytes,
                            int32_t T, int32_t E, int32_t top_k);

/*
 * Expert cube descriptor: AwqExpertOptions + AwqExpertPayload
 * (packed_experts.rs), or an MXFP4 bank (native.rs ExpertLayout::Native).
 *
 * AWQ:   qweight int32 [E, K, N/8] (eight 4-bit codes per word, AWQ nibble
 *        order: nibble i holds column 0 2 4 6 1 3 5 7 [i] of its group of 8),
 *        qzeros  int32 [E, K/g, N/8] (same order), scales [E, K/g, N] in
 *        scale_dtype (F32/F16/BF16), bias [E, N] in scale_dtype or NULL.
 *        coefficient(k, n) = (code - zero) * scale rounded once to scale_dtype
 *        (frozen_awq.rs FrozenAwqOps doc comment).
 *        K = in_features, N = out_features (N % 8 == 0), g = group_size
 *        (K % g == 0; the kernels implement g % 32 == 0).
 * MXFP4: qweight uint8 blocks [E, N, K/32, 16] (row = output feature, 32
 *        E2M1 elements per 16 bytes, even element in the low nibble),
 *        scales uint8 E8M0 [E, N, K/32], bias bf16 [E, N] (required, as the
 *        bank layout has one), qzeros NULL, scale_dtype ignored,
 *        group_size 32.  A gate/up bank has N = 2*I and interleaved_gate_up = 1
 *        (row 2i = gate feature i, row 2i+1 = up feature i); a down bank has
 *        interleaved_gate_up = 0 (native.rs native_layout / companions).
 * experts / expert_start: the resident cubes cover global IDs
 *        [expert_start, expert_start + experts); on one GPU this must be the
 *        route's full range [0, E) (else ERANGE: no unchecked imported offsets).
 */
typedef struct moeq_experts {
    moeq_format format;
    int32_t experts;
    int32_t expert_start;
    int32_t in_features;
    int32_t out_features;
    int32_t group_size;
    const void *qweight;
    const void *qzeros;
    const void *scales;
    moeq_dtype scale_dtype;
    const void *bias;
    int32_t interleaved_gate_up;
} moeq_experts;

/* SwiGLU parameters: h = g' * sigmoid(alpha * g') * (u' + up_offset) with
 * g', u' clamped to [-clamp, clamp] when clamp > 0.  Plain SwiGLU is
 * {0, 1, 0, 0}; the clamped routed variant of native.rs's engine is
 * {7, 1, 0, 0}.  gate_one_sided = 1 clamps the gate from above only,
 * g' = min(g, clamp) (u' unchanged): with {7, 1.702, 1, 1} it is the form some
 * MXFP4 models use.  A clamped value passes the derivative on its closed
 * interval (the backward path) and blocks it outside. */
typedef struct moeq_swiglu {
    float clamp;
    float alpha;
    float up_offset;
    int32_t gate_one_sided;  /* 0 or 1 */
} moeq_swiglu;

/*
 * moe_dispatch -- moe_exchange.rs MoeDispatchOps::moe_dispatch / MoeDispatched.
 *   x        [T, K] act (F32, F16 or BF16)     input rows
 *   logits   [T, E] logit_dtype (F32 or BF16)   router logits; bf16 logits are
 *                                               widened exactly to fp32 first
 *   expert_bias [E] fp32 or NULL                added to the logits (one fp32
 *                                               add) before selection and softmax
 * Outputs (A = T * top_k):
 *   values      [A, K] act   expert-sorted bit copies of the source rows
 *   weights     [T, top_k] fp32  softmax over the selected scores
 *   selected    [T, top_k] u32   expert IDs, descending score, ties -> lower ID
 *   row_experts [A] u32      expert ID of each sorted row (non-decreasing)
 *   route        bound to (T, E, top_k); receives the row mappings
 * The sort is stable: the rows of one expert keep ascending token order.
 * Implemented for E <= 2048, top_k <= 32 (else EUNSUPPORTED).  T = 0: no-op.
 */
moeq_status moe_dispatch(const void *x, moeq_dtype act, int32_t T, int32_t K,
                         const void *logits, moeq_dtype logit_dtype, int32_t E,
                         const float *expert_bias, int32_t top_k, void *values, float *weights,
                         uint32_t *selected, uint32_t *row_experts, moeq_route *route,
                         void *stream);

/*
 * moe_dispatch_static -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): moe_dispatch with the route's row mappings in a fixed device
 * array of the library instead of a caller workspace.  Same arguments, outputs,
 * validation and kernels as moe_dispatch, except that `route` need not be
 * bound: on success the call binds it to the array of the current device (the
 * device of `stream`); on an error it leaves `route` untouched.
 * Limit: moeq_route_workspace_bytes(T, E, top_k) <= MOEQ_STATIC_ROUTE_BYTES
 * (4 MiB, e.g. T * top_k up to about 400k assignments at E = 512), else
 * EWORKSPACE.  The array is one per GPU, held until the process ends, and
 * shared by every call on that GPU: each call overwrites the row mappings of
 * the previous one.  A route from this call therefore serves the calls that
 * consume it (grouped projections, counts, combine, backward calls) when they
 * are ordered before the next moe_dispatch_static on that GPU, e.g. enqueued on
 * the same stream before it; calls that overlap on one GPU (other streams or
 * threads without ordering) race.  Allocates and frees nothing; the first call
 * on a device looks the array's address up once (hipGetSymbolAddress).
 */
#define MOEQ_STATIC_ROUTE_BYTES (4u << 20)

moeq_status moe_dispatch_static(const void *x, moeq_dtype act, int32_t T, int32_t K,
                                const void *logits, moeq_dtype logit_dtype, int32_t E,
                                const float *expert_bias, int32_t top_k, void *values,
                                float *weights, uint32_t *selected, uint32_t *row_experts,
                                moeq_route *route, void *stream);

/*
 * moe_dispatch_counts -- moe_exchange.rs MoeDispatchOps::moe_dispatch_counts:
 * rows per caller-declared contiguous range of global expert IDs, read from
 * the expert offsets only.  expert_prefix: host int64 [R+1], non-decreasing,
 * within [0, E] (else ERANGE); counts: host int64 [R],
 * counts[r] = rows routed to experts [prefix[r], prefix[r+1]).
 * Copies E+1 offsets to the host and synchronises `stream`.
 */
moeq_status moe_dispatch_counts(const moeq_route *route, const int64_t *expert_prefix,
                                int32_t R, int64_t *counts, void *stream);

/*
 * awq_grouped_swiglu -- packed_experts.rs FrozenPackedExpertOps::
 * packed_swiglu_forward, gate/up half: for the rows of each expert e,
 *   G = values . Wg_e (+ bg_e), U = values . Wu_e (+ bu_e),
 *   rounded to act, then h = round_act(SwiGLU(G, U)).
 *   values [A, K] act (from moe_dispatch), h [A, I] act.
 * AWQ: gate and up are two descriptors of equal shape [E, K, I/8].
 * MXFP4: gate is an interleaved gate/up bank (N = 2I), up must be NULL.
 * Only experts with rows are read (untouched experts cost no bytes).
 */
moeq_status awq_grouped_swiglu(const moeq_route *route, const void *values,
                               moeq_dtype act, const moeq_experts *gate,
                               const moeq_experts *up, moeq_swiglu fn, void *h,
                               void *stream);

/*
 * awq_grouped_down -- the down projection of packed_swiglu_forward:
 *   y = round_act(h . Wd_e (+ bd_e)),  h [A, I] act, y [A, K] act.
 * AWQ down: [E, I, K/8] words; MXFP4: a non-interleaved bank [E, K, I/32, 16].
 */
moeq_status awq_grouped_down(const moeq_route *route, const void *h, moeq_dtype act,
                             const moeq_experts *down, void *y, void *stream);

/*
 * moe_combine -- moe_exchange.rs MoeDispatchOps::moe_combine: ascending
 * expert-ID combine after the rows returned to their source:
 *   out[t, :] = round_act( fp32 sum, in ascending expert ID, of
 *               weights[t, j] * y[slot_pos[t, j], :] )
 * written as acc = fma(w, y, acc) from acc = 0.
 *   y [A, K] act, weights [T, top_k] fp32, out [T, K] act.
 */
moeq_status moe_combine(const moeq_route *route, const void *y, moeq_dtype act,
                        int32_t K, const float *weights, void *out, void *stream);

/*
 * awq_input_backward -- frozen_awq.rs FrozenAwqOps::frozen_awq_input_backward
 * and packed_experts.rs packed_expert_input_backward: the transpose of the
 * same rounded packed coefficients, no weight / scale / bias gradients:
 *   grad_in[p, :] = round_gdt( grad[p, :] . W_e^T )
 *   grad [rows, N] gdt, grad_in [rows, K] gdt.
 * route != NULL: rows must equal the route's A and row p uses the expert of
 * sorted row p.  route == NULL: the single frozen projection; w must hold one
 * expert and every row uses it.  AWQ only.
 */
moeq_status awq_input_backward(const moeq_route *route, const void *grad,
                               moeq_dtype gdt, int32_t rows, const moeq_experts *w,
                               void *grad_in, void *stream);

/*
 * moe_combine_backward -- moe_exchange.rs MoeDispatchOps::moe_combine_backward
 * with a MoeCombineSelection: only the requested derivatives are formed.
 *   y [A, K] act (the rows the forward combined), weights [T, top_k] fp32,
 *   grad [T, K] act (derivative of the combine output).
 *   grad_y [A, K] act or NULL:
 *       grad_y[slot_pos[t, j], :] = round_act(fl32(weights[t, j] * grad[t, :]))
 *   grad_weights [T, top_k] fp32 or NULL:
 *       grad_weights[t, j] = round_fp32(sum over c of grad[t, c] * y[slot_pos[t, j], c]),
 *       products and sum in fp64 (one rounding).
 * Both NULL: nothing to do (returns OK).  T = 0: no-op.
 */
moeq_status moe_combine_backward(const moeq_route *route, const void *y, moeq_dtype act,
                                 int32_t K, const float *weights, const void *grad,
                                 void *grad_y, float *grad_weights, void *stream);

/*
 * moe_dispatch_backward -- moe_exchange.rs MoeDispatchOps::moe_dispatch_backward:
 * the COPY VJP.  Each token sums the derivatives of its top_k expert-sorted
 * copies, without multiplying the routing weights again:
 *   grad_x[t, :] = round_act( fp32 sum, in ascending expert ID, of
 *                  grad[slot_pos[t, j], :] )  from 0.
 *   grad [A, K] act, grad_x [T, K] act.
 */
moeq_status moe_dispatch_backward(const moeq_route *route, const void *grad, moeq_dtype act,
                                  int32_t K, void *grad_x, void *stream);

/*
 * moe_dispatch_weights_backward -- moe_exchange.rs MoeDispatchOps::
 * moe_dispatch_weights_backward: the source-logit VJP of the FP32 weights with
 * the discrete selection held fixed.  With w the softmax over the selected
 * scores,
 *   grad_logits[t, selected[t, j]] = round_fp32( w_j * (dw_j - sum_i w_i dw_i) )
 * evaluated in fp64 (the sum in slot order); every unselected logit gets 0.
 *   selected [T, top_k] u32 and weights [T, top_k] fp32 from moe_dispatch,
 *   grad_weights [T, top_k] fp32, grad_logits [T, E] fp32 (fully written).
 * The derivative of an added expert bias is the column sum of grad_logits.
 */
moeq_status moe_dispatch_weights_backward(const moeq_route *route, const uint32_t *selected,
                                          const float *weights, const float *grad_weights,
                                          float *grad_logits, void *stream);

/*
 * awq_swiglu_input_backward -- packed_experts.rs FrozenPackedExpertOps::
 * packed_swiglu_input_backward: the first-order input VJP through the selected
 * packed chain gate/up -> SwiGLU -> down, no weight / scale / bias gradients
 * (PackedExpertAutodiffError: metadata frozen, first order only).
 *   dh = round_act(grad . Wd_e^T)                      (as awq_input_backward)
 *   G, U recomputed as in awq_grouped_swiglu (rounded to act), then
 *   dG = round_act(dh * (u' + up_offset) * (s + alpha g' s (1 - s))),
 *   dU = round_act(dh * g' * s),  s = sigmoid(alpha g'),
 *   with g', u' the clamped G, U; a clamped value passes the derivative on
 *   [-clamp, clamp] and blocks it outside;
 *   grad_values = round_act(dG . Wg_e^T + dU . Wu_e^T).
 * values [A, K] act (the forward's dispatched rows), grad [A, K] act (the
 * derivative of the down output), grad_values [A, K] act.  gate / up / down:
 * the forward's AWQ cubes (MXFP4 banks return EUNSUPPORTED).
 * workspace: device, >= awq_swiglu_input_backward_workspace_bytes(A, I, act)
 * bytes, 256-byte aligned, caller-owned; it holds dh, G / dG and U / dU
 * ([A, I] act each) between the call's kernels and may be reused once the
 * stream has passed them.
 */
size_t awq_swiglu_input_backward_workspace_bytes(int32_t rows, int32_t I, moeq_dtype act);

moeq_status awq_swiglu_input_backward(const moeq_route *route, const void *values,
                                      moeq_dtype act, const moeq_experts *gate,
                                      const moeq_experts *up, const moeq_experts *down,
                                      moeq_swiglu fn, const void *grad, void *grad_values,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * awq_expert_forward -- packed_experts.rs FrozenPackedExpertOps::
 * packed_expert_forward: rows in any order, each with its global expert ID;
 * only the experts that occur are evaluated and the output keeps the incoming
 * row order:
 *   y[t, :] = round_act( x[t, :] . W_{id[t]} (+ b_{id[t]}) )
 * It is also the receive side of moe_exchange.rs MoeReceivedOps::
 * moe_received_forward: a local sort by global ID, the grouped expert kernels,
 * and the inverse permutation.
 *   x [rows, K] act, global_ids [rows] u32 (device), y [rows, N] act.
 *   w: an AWQ cube or a non-interleaved MXFP4 bank; IDs must lie in
 *      [expert_start, expert_start + experts), else ERANGE.  Experts that no
 *      row names are never read (empty owners are allowed).
 * The IDs are validated on the host: the call copies them and synchronises
 * `stream` before it enqueues the sort, the gather, the projection and the
 * restore.  workspace: device, 256-byte aligned, caller-owned,
 * >= awq_expert_workspace_bytes(rows, experts, K, N, act).  Implemented for
 * experts <= 2048 (else EUNSUPPORTED).  rows = 0: no-op.
 */
size_t awq_expert_workspace_bytes(int32_t rows, int32_t experts, int32_t in_features,
                                  int32_t out_features, moeq_dtype act);

moeq_status awq_expert_forward(const void *x, moeq_dtype act, int32_t rows,
                               const uint32_t *global_ids, const moeq_experts *w, void *y,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * awq_expert_input_backward -- packed_experts.rs FrozenPackedExpertOps::
 * packed_expert_input_backward for awq_expert_forward: the transpose of the same
 * rounded coefficients, rows in the incoming order:
 *   grad_in[t, :] = round_gdt( grad[t, :] . W_{id[t]}^T )
 *   grad [rows, N] gdt, grad_in [rows, K] gdt; AWQ only.
 * Same IDs, validation, synchronisation and workspace as awq_expert_forward.
 */
moeq_status awq_expert_input_backward(const void *grad, moeq_dtype gdt, int32_t rows,
                                      const uint32_t *global_ids, const moeq_experts *w,
                                      void *grad_in, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * frozen_awq_forward -- frozen_awq.rs FrozenAwqOps::frozen_awq_forward: one packed
 * projection over all rows, y = round_act(x . W (+ b)).  w holds one expert
 * (experts == 1, else ERANGE): AWQ words [1, K, N/8] or a non-interleaved MXFP4
 * bank.  x [rows, K] act, y [rows, N] act.  workspace: device, 256-byte aligned,
 * >= frozen_awq_workspace_bytes(rows) (the kernels' row map).  Its input VJP is
 * awq_input_backward with route NULL.
 */
size_t frozen_awq_workspace_bytes(int32_t rows);

moeq_status frozen_awq_forward(const void *x, moeq_dtype act, int32_t rows,
                               const moeq_experts *w, void *y, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * Block-scaled MFMA path of the MXFP4 bank (an opt-in variant: the activations
 * are rounded differently from the bf16 path).  native.rs ExpertLayout::Native
 * banks are read as they are by gfx950's v_mfma_scale_f32_16x16x128_f8f6f4; the
 * activation rows are first quantized to OCP MXFP8: per 32-element block a
 * shared E8M0 exponent floor(log2 max|v|) - 8 (kept in [-127, 127]; a zero block
 * gets byte 0), elements v / 2^shared saturated to +-448 and rounded to the
 * nearest E4M3 value, ties to even.  Products are exact, accumulation fp32.
 *
 * mx8_quantize: x [rows, K] bf16 (16-byte aligned, K % 32 == 0) -> q [rows, K] E4M3
 *   codes, s [rows, K/32] E8M0 bytes.
 * mx8_grouped_swiglu: as awq_grouped_swiglu over an interleaved gate/up bank,
 *   with MXFP8 values: h = round_bf16(SwiGLU(round_bf16(G), round_bf16(U))).
 * mx8_grouped_down: as awq_grouped_down over a plain bank, with MXFP8 h.
 * Both take bf16 activations and a workspace (device, 256-byte aligned) of at
 * least mx8_workspace_bytes(A, in_features) for the quantized rows; bank rows
 * must be a multiple of 64 (else EUNSUPPORTED).
 */
size_t mx8_workspace_bytes(int32_t rows, int32_t K);

moeq_status mx8_quantize(const void *x, moeq_dtype act, int32_t rows, int32_t K, uint8_t *q,
                         uint8_t *s, void *stream);

moeq_status mx8_grouped_swiglu(const moeq_route *route, const void *values, moeq_dtype act,
                               const moeq_experts *gate_up, moeq_swiglu fn, void *h,
                               void *workspace, size_t workspace_bytes, void *stream);

moeq_status mx8_grouped_down(const moeq_route *route, const void *h, moeq_dtype act,
                             const moeq_experts *down, void *y, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Static text for a status code. */
const char *moeq_status_string(moeq_status status);

/* Text of the last validation or device error raised on the calling thread. */
const char *moeq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOEQ_H */
