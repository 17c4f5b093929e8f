// internal.hpp -- launcher declarations shared by the host API and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moeq.h"

namespace moeq {

constexpr uint32_t kRouteMagic = 0x6d6f6571u;  // "moeq"
constexpr int kTokenBlock = 256;              // tokens per block of the stable scatter
constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 2048;
constexpr int kTileRows = 128;                // rows per m-tile of the tiled projections

// Most m-tiles of kTileRows rows that A rows in E experts can form.  A route's
// tile list holds tile_expert[cap] followed by tile_order[cap]: the m-tiles
// with every full tile (in m-tile order) before the partial ones, the order in
// which the warp-specialised kernel schedules them (longest first).
__host__ __device__ inline int tile_cap(long A, int E) {
    return (int)((A + kTileRows - 1) / kTileRows) + E;
}

// One packed projection operand as the kernels see it (validated on the host).
struct PackedOperand {
    int format;          // moeq_format
    int sdt;             // scale dtype (AWQ)
    const int32_t *qw;   // AWQ words  | MXFP4 block bytes (as int32 for alignment)
    const int32_t *qz;   // AWQ zeros  | NULL
    const void *scales;  // AWQ scales | MXFP4 E8M0 bytes
    const void *bias;    // nullable
    int K;               // reduction length of the forward projection (in_features)
    int N;               // out_features of the cube
    int g;               // AWQ group
};

// Projection problem: rows of `in` grouped by expert through `offsets`
// (offsets == NULL: `rows` rows, all expert 0).
struct ProjProblem {
    const void *in;
    void *out;
    const void *in2;     // second input: dU (INPUT_VJP2) | dh (SWIGLU backward epilogue)
    void *out2;          // dU of the SWIGLU backward epilogue (out then holds dG)
    const int32_t *offsets;
    const int32_t *tile_offsets;  // [E+1] m-tile prefix (route), nullable
    const int32_t *tile_expert;   // expert of each m-tile (route), nullable
    const int32_t *tile_order;    // m-tiles, full ones first (route), nullable
    int rows;            // total rows (A)
    int E;               // experts in the grid
    int act;             // activation / gradient storage
    int Kred;            // reduction length
    int Nout;            // output columns
    PackedOperand w0;    // gate (or the only operand)
    PackedOperand w1;    // up (AWQ gate/up only)
    int mode;            // see ProjMode
    float clamp, alpha, up_offset;
    float gate_lo;       // lower clamp bound of the gate: -clamp, or -inf (one-sided variant)
    int split_rows;      // > 0: experts with at most this many rows go to the weight-streaming
                         // kernel, the m-tile kernels skip them (set by the kernel choice)
};

enum ProjMode {
    PROJ_PLAIN = 0,      // out = in . W (+ b)
    PROJ_SWIGLU = 1,     // out = SwiGLU(in . Wg (+ bg), in . Wu (+ bu)), AWQ; with
                         // in2 = dh: out = dG, out2 = dU of the SwiGLU at those G, U
    PROJ_BANK_SWIGLU = 2,// MXFP4 interleaved gate/up bank + SwiGLU
    PROJ_INPUT_VJP = 3,  // out = in . W^T, AWQ (no bias)
    PROJ_INPUT_VJP2 = 4, // out = in . Wg^T + in2 . Wu^T, AWQ
};

// Record a validation or device error for moeq_last_error() and return `st`.
moeq_status report_error(moeq_status st, const char *fmt, ...);

hipError_t launch_router(const void *logits, bool logits_bf16, const float *bias, int T, int E,
                         int k, uint32_t *selected, float *weights, hipStream_t s);
bool index_rows_fits(int T, int E, int k, size_t row_bytes, const void *x, const void *values);
// after launch_router: the stable order, the route and the row copies in one launch
hipError_t launch_index_rows(const void *x, size_t row_bytes, const uint32_t *selected, int T,
                             int E, int k, void *values, uint32_t *row_experts,
                             const moeq_route *route, hipStream_t s);
hipError_t launch_dispatch_index(const uint32_t *selected, int T, int E, int k,
                                 const moeq_route *route, uint32_t *row_experts,
                                 hipStream_t s);
bool scatter_rows_fits(size_t row_bytes, int k, const void *x, const void *values);
hipError_t launch_scatter_rows(const void *x, size_t row_bytes, int T, int k,
                               const int32_t *slot_pos, void *values, hipStream_t s);
hipError_t launch_copy_rows(const void *x, size_t row_bytes, int A, const int32_t *row_src,
                            void *values, hipStream_t s);
hipError_t launch_local_ids(const uint32_t *gid, int rows, int start, uint32_t *local,
                            hipStream_t s);
hipError_t launch_single_tiles(int rows, int32_t *offsets, int32_t *tile_offsets,
                               int32_t *tile_expert, hipStream_t s);
hipError_t launch_combine(const void *y, int act, const float *weights,
                          const int32_t *slot_pos, int T, int k, int K, void *out,
                          hipStream_t s);
hipError_t launch_proj_generic(const ProjProblem &p, hipStream_t s);

// backward path
hipError_t launch_dispatch_backward(const void *grad, int act, const int32_t *slot_pos, int T,
                                    int k, int K, void *grad_x, hipStream_t s);
hipError_t launch_combine_backward(const void *y, int act, const float *weights,
                                   const int32_t *slot_pos, const void *grad, int T, int k, int K,
                                   void *grad_y, float *grad_weights, hipStream_t s);
hipError_t launch_swiglu_vjp(void *G, void *U, const void *dh, int act, size_t n, float clamp,
                             float gate_lo, float alpha, float up_offset, hipStream_t s);
hipError_t launch_mx8_quant(const void *x, int rows, int K, uint8_t *q, uint8_t *s,
                            int sstride, hipStream_t st);
hipError_t launch_mx8_gemm(const uint8_t *q, const uint8_t *qs, int sstride, int rows, int K,
                           const PackedOperand &w, const int32_t *offsets,
                           const int32_t *tile_offsets, const int32_t *tile_expert, int E,
                           bool swiglu, int Nout, float clamp, float gate_lo, float alpha,
                           float up_offset, void *out, hipStream_t s);
bool vjp_fits(const ProjProblem &p);
hipError_t launch_vjp(const ProjProblem &p, hipStream_t s);
hipError_t launch_weights_backward(const uint32_t *selected, const float *weights,
                                   const float *grad_weights, int T, int E, int k,
                                   float *grad_logits, hipStream_t s);

}  // namespace moeq
