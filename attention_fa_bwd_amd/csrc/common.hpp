// common.hpp -- element types and small device helpers shared by the kernels
// of libfa_bwd.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// bfloat16 is carried as its 16-bit pattern in memory; e16_t is any 16-bit
// element (bf16 or fp16) as its bit pattern, for code that only moves bits.
typedef uint16_t bf16_t;
typedef uint16_t e16_t;
// IEEE half precision, as the compiler's native type.
typedef _Float16 f16_t;

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

struct Shape {
    int B, H, N, d;
    long long rows() const { return (long long)B * H * N; }
    long long elems() const { return rows() * d; }
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(f16_t x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float((uint32_t)x << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t bf16_rne(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(bf16_t, h);
}

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    typedef float f32x2_v __attribute__((ext_vector_type(2)));
    f32x2_v v = {a, b};
    bf16x2_v h = __builtin_convertvector(v, bf16x2_v);
    return __builtin_bit_cast(uint32_t, h);
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return bf16_rne(f); }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float f) { return (f16_t)f; }

// Two fp32 -> packed fp16x2 (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
    typedef float f32x2_v __attribute__((ext_vector_type(2)));
    f32x2_v v = {a, b};
    f16x2_v h = __builtin_convertvector(v, f16x2_v);
    return __builtin_bit_cast(uint32_t, h);
}

// Unpack a 16-byte vector into VEC floats.
__device__ __forceinline__ void unpack16(const uint4& u, float* f /*[8]*/, bf16_t) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack16(const uint4& u, float* f /*[8]*/, f16_t) {
    typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
    const f16x8_v h = __builtin_bit_cast(f16x8_v, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}
__device__ __forceinline__ void unpack16(const uint4& u, float* f /*[4]*/, float) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
}

}  // namespace fa
