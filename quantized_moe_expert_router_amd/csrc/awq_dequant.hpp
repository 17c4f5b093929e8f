// awq_dequant.hpp -- device helpers shared by the AWQ MFMA kernels: nibble
// decode, per-group constants, coefficient formation, bf16 packing, SwiGLU and
// raw buffer resources.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moeq {
namespace awq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Slot sl of a word: bytes 0..3 of (w & 0x0F0F0F0F) are nibbles 0,2,4,6 and
// bytes 0..3 of ((w >> 4) & 0x0F0F0F0F) nibbles 1,3,5,7.  Under the AWQ order
// (nibble i holds column [0 2 4 6 1 3 5 7][i]) slot sl holds column:
__device__ constexpr int kSlotCol[8] = {0, 4, 1, 5, 2, 6, 3, 7};

// Byte b < 16 read as OCP fp8 E4M3 is b * 2^-9 (exponent-0 subnormals continue
// linearly into exponent 1); scales are pre-multiplied by 2^9 to compensate.
constexpr float kCodeUnit = 512.0f;

// AND the compiler cannot fold into later byte extractions.
__device__ __forceinline__ uint32_t and_opaque(uint32_t x, uint32_t m) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
    return r;
}

// The eight 4-bit codes of a word, in slot order, as code * 2^-9.
__device__ __forceinline__ void decode_codes(uint32_t w, float q[8]) {
    const uint32_t lo = and_opaque(w, 0x0F0F0F0Fu);
    const uint32_t hi = and_opaque(w >> 4, 0x0F0F0F0Fu);
    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
    const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    q[0] = a[0]; q[1] = a[1]; q[2] = b[0]; q[3] = b[1];
    q[4] = c[0]; q[5] = c[1]; q[6] = d[0]; q[7] = d[1];
}

// Per-group dequant constants of one word column, in slot order.
template <int SD>
struct GroupConst {
    float s[8];   // scale * 2^9
    float zs[8];  // -zero * scale (rounded to fp32 for fp32 scales)
};

// Coefficient of slot sl from q = code * 2^-9, as the scale-dtype value in fp32.
// 16-bit scales: the fma is the exact (code - zero) * scale.  fp32 scales: the
// MFMA operand is bf16 anyway, so the one-op code * scale - RN(zero * scale)
// (within one fp32 ulp of RNE32((code - zero) * scale)) goes to the bf16 pack.
template <int SD>
__device__ __forceinline__ float coeff(float q, const GroupConst<SD> &gc, int sl) {
    const float v = __builtin_fmaf(q, gc.s[sl], gc.zs[sl]);
    return SD == MOEQ_F16 ? (float)(_Float16)v : v;                 // bf16: rounded at pack
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});  // v_cvt_pk_bf16_f32
}

// SwiGLU for bf16 outputs: the hardware exp and reciprocal (about one fp32 ulp
// each) stay far inside the bf16 rounding of h.
// glo: the gate's lower clamp bound (-clamp, or -inf for the one-sided variant).
__device__ __forceinline__ float swiglu_f(float g, float u, float clamp, float glo, float alpha,
                                          float off) {
    if (clamp > 0.0f) {
        g = fminf(fmaxf(g, glo), clamp);
        u = fminf(fmaxf(u, -clamp), clamp);
    }
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-alpha * g)) * (u + off);
}

// Derivatives of h = g' sigmoid(alpha g') (u' + off) for the backward epilogues
// (bf16 outputs; hardware exp and reciprocal as in swiglu_f): g', u' clamped
// when clamp > 0, a clamped value passing the derivative on the closed interval
// and blocking it outside.
__device__ __forceinline__ void swiglu_vjp_f(float g, float u, float d, float clamp, float glo,
                                             float alpha, float off, float *dg, float *du) {
    float gpass = 1.0f, upass = 1.0f;
    if (clamp > 0.0f) {
        gpass = (g >= glo && g <= clamp) ? 1.0f : 0.0f;
        upass = (u >= -clamp && u <= clamp) ? 1.0f : 0.0f;
        g = fminf(fmaxf(g, glo), clamp);
        u = fminf(fmaxf(u, -clamp), clamp);
    }
    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-alpha * g));
    *dg = gpass * d * (u + off) * (sg + alpha * g * sg * (1.0f - sg));
    *du = upass * d * g * sg;
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// only.  __syncthreads() also waits for every global load in flight
// (vmcnt(0)), which would drain the prefetch ring at each barrier.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Barrier that only aligns the waves of a block (no memory hand-off): nothing
// in flight is waited for.
__device__ __forceinline__ void lockstep_barrier() { __builtin_amdgcn_s_barrier(); }

constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 buffer descriptor, 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)(uint32_t)bytes,
                                             kRawBufferWord3);
}

// Raw per-group words of one operand: the zero word and 8 scales.
template <int SD>
struct GroupRaw {
    uint32_t zw;
    u32x4 s0, s1;  // s1 only for fp32 scales
};

template <int SD>
__device__ __forceinline__ void load_group_raw(__amdgpu_buffer_rsrc_t rz, __amdgpu_buffer_rsrc_t rs,
                                               int voff_z, int voff_s, int gi, int W, int N,
                                               GroupRaw<SD> &r) {
    constexpr int sb = SD == MOEQ_F32 ? 4 : 2;
    r.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, voff_z, gi * W * 4, 0);
    r.s0 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_s, gi * N * sb, 0);
    if (SD == MOEQ_F32) r.s1 = __builtin_amdgcn_raw_buffer_load_b128(rs, voff_s + 16, gi * N * sb, 0);
}

template <int SD>
__device__ __forceinline__ void decode_group(const GroupRaw<SD> &r, GroupConst<SD> &gc) {
    float z[8], sv[8];
    decode_codes(r.zw, z);  // zero * 2^-9
    if (SD == MOEQ_F32) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            sv[c] = __uint_as_float(r.s0[c]);
            sv[4 + c] = __uint_as_float(r.s1[c]);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t v = r.s0[c];
            if (SD == MOEQ_BF16) {
                sv[2 * c] = __uint_as_float(v << 16);
                sv[2 * c + 1] = __uint_as_float(v & 0xFFFF0000u);
            } else {
                sv[2 * c] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
                sv[2 * c + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
            }
        }
    }
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
        const float sc = sv[kSlotCol[sl]];
        gc.s[sl] = sc * kCodeUnit;                                          // exact
        gc.zs[sl] = -(z[sl] * kCodeUnit) * sc;  // 16-bit scales: exact (4 x 16 bits)
    }
}

}  // namespace awq
}  // namespace moeq
