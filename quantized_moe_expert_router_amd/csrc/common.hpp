// common.hpp -- device helpers shared by the gfx950 kernels of libmoeq.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moeq.h"

namespace moeq {

constexpr int kWave = 64;

// ---------------------------------------------------------------- storage
// Storage codes match moeq_dtype: 0 fp32, 1 fp16, 2 bf16.
template <int DT> struct Storage;
template <> struct Storage<MOEQ_F32> { using T = float; };
template <> struct Storage<MOEQ_F16> { using T = _Float16; };
template <> struct Storage<MOEQ_BF16> { using T = __bf16; };

template <int DT>
__device__ __forceinline__ float load_f(const void *p, size_t i) {
    return (float)static_cast<const typename Storage<DT>::T *>(p)[i];
}

// Conversions to fp16 / bf16 round to nearest, ties to even.
template <int DT>
__device__ __forceinline__ void store_f(void *p, size_t i, float v) {
    static_cast<typename Storage<DT>::T *>(p)[i] = (typename Storage<DT>::T)v;
}

// Round an fp32 value to the storage type and widen it back (exact widening).
template <int DT>
__device__ __forceinline__ float round_to(float v) {
    return (float)(typename Storage<DT>::T)v;
}

// ---------------------------------------------------------------- AWQ words
// Nibble position holding logical column c of a group of eight: the AWQ pack
// order stores column [0 2 4 6 1 3 5 7][i] in nibble i, so column c sits in
// nibble kNibbleOfColumn[c].
__device__ __forceinline__ int nibble_of_column(int c) {
    // [0,4,1,5,2,6,3,7][c] as a bit trick: even c -> c/2, odd c -> 4 + c/2
    return (c >> 1) + ((c & 1) << 2);
}

// Column of its group held by nibble i (inverse of nibble_of_column).
__device__ __forceinline__ int column_of_nibble(int i) {
    return ((i & 3) << 1) + (i >> 2);
}

// ---------------------------------------------------------------- MXFP4
// OCP MX E2M1 element value (sign, 2-bit exponent with bias 1, 1-bit mantissa).
__device__ __forceinline__ float e2m1_value(unsigned nib) {
    const unsigned ex = (nib >> 1) & 3u, man = nib & 1u;
    const float mag = ex == 0 ? 0.5f * (float)man
                              : __builtin_ldexpf(1.0f + 0.5f * (float)man, (int)ex - 1);
    return (nib & 8u) ? -mag : mag;
}

// E8M0 shared scale 2^(byte - 127) (byte 255 is not generated; treated as 2^128).
__device__ __forceinline__ float e8m0_value(unsigned byte) {
    return byte == 255u ? __builtin_nanf("") : __builtin_ldexpf(1.0f, (int)byte - 127);
}

// ---------------------------------------------------------------- waves
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

}  // namespace moeq
