/*
 * moe_oracle.h -- plain CPU oracle for the routed MoE expert FFN over frozen
 * packed 4-bit experts.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the HIP path.  Only
 * the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code, header, table or helper with the HIP library and
 * includes nothing from it.
 *
 * Every function is the plain definition written out: scalar loops, double
 * accumulation, one rounding to the storage type where the pages place one.
 * The sources it follows are cited per function in moe_oracle.c:
 *   - ruda-tensor 0.21.38, src/moe_exchange.rs   (MoeDispatched, MoeDispatchOps)
 *   - ruda-tensor 0.21.34, src/packed_experts.rs (AwqExpertOptions,
 *     AwqExpertPayload, FrozenPackedExpertOps)
 *   - ruda-tensor 0.21.33, src/frozen_awq.rs     (FrozenAwqOps doc comment)
 *   - libmir-metal 0.3.0, src/engine/clamped_routed/experts/native.rs
 *     (ExpertLayout::Native companion shapes in `validate`)
 *
 * Parity status of each function is listed in the header comment of
 * moe_oracle.c ("pinned by" / "parity unpinned").
 *
 * Storage type codes (shared by every function): 0 = fp32, 1 = fp16, 2 = bf16.
 * fp16 and bf16 buffers are passed as uint16_t bit patterns.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* scalar helpers, exported so the tests can pin them directly */
double orc_load(const void *buf, int dtype, size_t i);
void orc_store(void *buf, int dtype, size_t i, double v);
uint16_t orc_round_f16(double v);
uint16_t orc_round_bf16(double v);
double orc_f16_value(uint16_t bits);
double orc_bf16_value(uint16_t bits);

/* router: selected [T,k] u32, weights [T,k] f32 */
void orc_route(int T, int E, int k, const float *logits, const float *bias,
               uint32_t *selected, float *weights);

/* dispatch index: offsets [E+1], row_src [A], slot_pos [T*k], row_experts [A] */
void orc_dispatch_index(int T, int E, int k, const uint32_t *selected,
                        int32_t *offsets, int32_t *row_src, int32_t *slot_pos,
                        uint32_t *row_experts);

/* COPY dispatch of whole rows (bit copy) */
void orc_copy_rows(int A, size_t row_bytes, const void *x, const int32_t *row_src,
                   void *values);

/* counts per caller range; returns 0 or -1 on an invalid prefix */
int orc_counts(int E, const int32_t *offsets, int R, const int64_t *prefix,
               int64_t *counts);

/* AWQ coefficient W[e,k,n] as a double (already rounded to the scale dtype) */
double orc_awq_coeff(int K, int N, int g, const int32_t *qweight,
                     const int32_t *qzeros, const void *scales, int sdt,
                     int e, int k, int n);

/* dense dequantised cube W [E,K,N] in double */
void orc_awq_dequant(int E, int K, int N, int g, const int32_t *qweight,
                     const int32_t *qzeros, const void *scales, int sdt,
                     double *W);

/* grouped projection out[p,:] = round_adt(in[p,:] . W_{row_experts[p]} + b).
 * row_experts may be NULL: then every row uses expert 0.
 * out_exact (nullable) receives the unrounded double result. */
void orc_awq_project(int A, int K, int N, const void *in, int adt,
                     const uint32_t *row_experts, int E, int g,
                     const int32_t *qweight, const int32_t *qzeros,
                     const void *scales, int sdt, const void *bias,
                     void *out, double *out_exact);

/* storage-rounded SwiGLU on n elements */
void orc_swiglu(size_t n, const void *G, const void *U, int adt, double clamp,
                double alpha, double up_offset, int gate_one_sided, void *h);

/* ascending expert-ID combine: out [T,K] */
void orc_combine(int T, int k, int K, const void *y, int adt,
                 const float *weights, const int32_t *slot_pos, void *out);

/* COPY VJP: dx[t,:] = sum of the gradient rows that copied token t */
void orc_copy_vjp(int T, int k, int K, const double *dvalues,
                  const int32_t *slot_pos, double *dx);

/* input VJP: grad_in[p,:] = round_gdt(grad[p,:] . W_e^T) */
void orc_awq_input_backward(int A, int K, int N, const void *grad, int gdt,
                            const uint32_t *row_experts, int E, int g,
                            const int32_t *qweight, const int32_t *qzeros,
                            const void *scales, int sdt, void *grad_in);

/* backward path (first order) */
/* COPY VJP in the combine's arithmetic: dx[t,:] = round_adt(fp32 sum of the
 * token's gradient rows in ascending sorted position) */
void orc_dispatch_backward(int T, int k, int K, const void *dvalues, int adt,
                           const int32_t *slot_pos, void *dx);
/* fixed-selection logit VJP of the softmax weights: dlogits [T,E] f32 */
void orc_dispatch_weights_backward(int T, int E, int k, const uint32_t *selected,
                                   const float *weights, const float *dweights,
                                   float *dlogits);
/* combine VJP: dy [A,K] adt and dweights [T,k] f32, each nullable */
void orc_combine_backward(int T, int k, int K, const void *y, int adt,
                          const float *weights, const int32_t *slot_pos,
                          const void *dout, void *dy, float *dweights);
/* SwiGLU VJP at the forward's G, U: dG, dU [n] adt */
void orc_swiglu_backward(size_t n, const void *G, const void *U, const void *dh, int adt,
                         double clamp, double alpha, double up_offset, int gate_one_sided,
                         void *dG, void *dU);
/* input VJP of the gate/up + SwiGLU part: dvalues [A,K] adt from dh [A,I] adt */
void orc_awq_swiglu_input_backward(int A, int K, int I, const void *values, int adt,
                                   const uint32_t *row_experts, int E, int g,
                                   const int32_t *gqw, const int32_t *gqz, const void *gs,
                                   const int32_t *uqw, const int32_t *uqz, const void *us,
                                   int sdt, const void *gbias, const void *ubias,
                                   double clamp, double alpha, double up_offset,
                                   int gate_one_sided, const void *dh, void *dvalues);

/* MXFP4 bank */
double orc_e2m1_value(int nibble);
double orc_e8m0_value(int byte);
/* W [E,R,C] (R output rows, C = input features) from blocks [E,R,C/32,16] */
void orc_mxfp4_dequant(int E, int R, int C, const uint8_t *blocks,
                       const uint8_t *scales, double *W);
/* out[p,r] = round_adt(in[p,:] . W_e[r,:] + bias_bf16[e,r]) */
void orc_mxfp4_project(int A, int C, int R, const void *in, int adt,
                       const uint32_t *row_experts, int E, const uint8_t *blocks,
                       const uint8_t *scales, const uint16_t *bias_bf16, void *out);
/* MXFP8 activations: E4M3 element value; OCP MX quantization of 32-blocks;
 * projection of the quantized rows with an MXFP4 bank */
double orc_e4m3_value(int byte);
void orc_mxfp8_quantize(int rows, int K, const void *x, int adt, uint8_t *q, uint8_t *s);
void orc_mx8_project(int A, int C, int R, const uint8_t *q, const uint8_t *s,
                     const uint32_t *row_experts, int E, const uint8_t *blocks,
                     const uint8_t *scales, const uint16_t *bias_bf16, int adt, void *out);

/* Whole forward path, logits -> out, for the CPU baseline and end-to-end tests.
 * fmt 0 = AWQ (gate/up/down descriptors), fmt 1 = MXFP4 interleaved bank.
 * Intermediates are allocated internally.  Returns 0. */
typedef struct {
    int fmt;            /* 0 AWQ, 1 MXFP4 bank */
    int T, H, I, E, k, group;
    int adt, sdt;
    const void *x;      /* [T,H] adt */
    const float *logits;/* [T,E] */
    const float *router_bias; /* [E] or NULL */
    /* AWQ */
    const int32_t *gate_qw, *gate_qz, *up_qw, *up_qz, *down_qw, *down_qz;
    const void *gate_s, *up_s, *down_s;
    const void *gate_b, *up_b, *down_b; /* nullable, scale dtype */
    /* MXFP4 */
    const uint8_t *gu_blocks, *gu_scales, *dn_blocks, *dn_scales;
    const uint16_t *gu_bias, *dn_bias;
    double clamp, alpha, up_offset;
    int gate_one_sided; /* 0: g and u clamped to [-c, c]; 1: g clamped from above only */
    void *out;          /* [T,H] adt */
    /* optional intermediates for inspection (nullable) */
    uint32_t *selected; float *weights; int32_t *offsets, *row_src, *slot_pos;
    uint32_t *row_experts; void *values; void *h; void *y;
} orc_moe_args;
int orc_moe_forward(const orc_moe_args *a);

#ifdef __cplusplus
}
#endif
#endif
