// preprocess.hip -- the two HBM-bound steps around the main backward kernel.
//
// preprocess: D_i = sum_k O_ik dO_ik in fp32 (FA2 chapter 16, sec 16.1: the
//   identity D_i = dO_i . O_i; sec 16.8 item 1: computed once before the main
//   loop).  dq_accum needs no clearing: the query-outer dQ pass writes every
//   element of it.
// convert:    dQ = scale * dq_accum, cast to the element type (sec 16.3: the
//   separate kernel that applies the softmax scale to the fp32 buffer).
//
// Both stream their operands once with 16-byte accesses; a row of d elements
// is handled by d / VEC consecutive lanes whose partial dot products are
// combined with cross-lane shuffles.
#include "launch.hpp"

namespace fa {

template <typename T, int D>
__global__ __launch_bounds__(256) void preprocess_kernel(const T* __restrict__ O,
                                                         const T* __restrict__ dO,
                                                         float* __restrict__ Dout,
                                                         long long rows) {
    constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte access
    constexpr int TPR = D / VEC;         // lanes per row
    constexpr int RPB = 256 / TPR;       // rows per block and sweep
    static_assert(TPR >= 1 && TPR <= 64 && (TPR & (TPR - 1)) == 0, "bad row split");
    const int sub = threadIdx.x % TPR;
    for (long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR; row < rows;
         row += (long long)gridDim.x * RPB) {
        const long long off = row * D + sub * VEC;
        const uint4 uo = *reinterpret_cast<const uint4*>(O + off);
        const uint4 ug = *reinterpret_cast<const uint4*>(dO + off);
        float fo[VEC], fg[VEC];
        unpack16(uo, fo, T());
        unpack16(ug, fg, T());
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc = fmaf(fo[i], fg[i], acc);
#pragma unroll
        for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
        if (sub == 0) Dout[row] = acc;
    }
}

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ src,
                                                      T* __restrict__ dst, long long n4,
                                                      float scale) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4;
         i += (long long)gridDim.x * 256) {
        const float4 v = reinterpret_cast<const float4*>(src)[i];
        if constexpr (sizeof(T) == 4) {
            reinterpret_cast<float4*>(dst)[i] =
                make_float4(v.x * scale, v.y * scale, v.z * scale, v.w * scale);
        } else {
            uint2 p;
            if constexpr (__is_same(T, f16_t)) {
                p.x = pack_f16x2(v.x * scale, v.y * scale);
                p.y = pack_f16x2(v.z * scale, v.w * scale);
            } else {
                p.x = pack_bf16x2(v.x * scale, v.y * scale);
                p.y = pack_bf16x2(v.z * scale, v.w * scale);
            }
            reinterpret_cast<uint2*>(dst)[i] = p;
        }
    }
}

static unsigned grid_for(long long work, long long per_block) {
    long long g = (work + per_block - 1) / per_block;
    const long long cap = 256LL * 64;  // enough waves to saturate HBM; grid-stride beyond
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (unsigned)g;
}

template <typename T, int D>
static hipError_t pre_t(const void* O, const void* dO, float* Dv, Shape s, hipStream_t st) {
    constexpr int RPB = 256 / (D / (16 / (int)sizeof(T)));
    hipLaunchKernelGGL((preprocess_kernel<T, D>), dim3(grid_for(s.rows(), RPB)), dim3(256), 0,
                       st, (const T*)O, (const T*)dO, Dv, s.rows());
    return hipGetLastError();
}

template <typename T>
static hipError_t pre_d(const void* O, const void* dO, float* Dv, Shape s, hipStream_t st) {
    switch (s.d) {
        case 16: return pre_t<T, 16>(O, dO, Dv, s, st);
        case 32: return pre_t<T, 32>(O, dO, Dv, s, st);
        case 64: return pre_t<T, 64>(O, dO, Dv, s, st);
        case 128: return pre_t<T, 128>(O, dO, Dv, s, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_preprocess(int dtype, const void* O, const void* dO, float* D, Shape s,
                             hipStream_t st) {
    return dtype == DT_BF16  ? pre_d<bf16_t>(O, dO, D, s, st)
           : dtype == DT_F16 ? pre_d<f16_t>(O, dO, D, s, st)
                             : pre_d<float>(O, dO, D, s, st);
}

hipError_t launch_convert_dq(int dtype, const float* dq_accum, void* dQ, Shape s, float scale,
                             hipStream_t st) {
    const long long n4 = s.elems() / 4;
    const unsigned g = grid_for(n4, 256);
    if (dtype == DT_BF16)
        hipLaunchKernelGGL((convert_kernel<bf16_t>), dim3(g), dim3(256), 0, st, dq_accum,
                           (bf16_t*)dQ, n4, scale);
    else if (dtype == DT_F16)
        hipLaunchKernelGGL((convert_kernel<f16_t>), dim3(g), dim3(256), 0, st, dq_accum,
                           (f16_t*)dQ, n4, scale);
    else
        hipLaunchKernelGGL((convert_kernel<float>), dim3(g), dim3(256), 0, st, dq_accum,
                           (float*)dQ, n4, scale);
    return hipGetLastError();
}

}  // namespace fa
