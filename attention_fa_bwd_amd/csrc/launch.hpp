// launch.hpp -- internal launcher interface between the C ABI (api.hip) and the
// kernel translation units.  Each launcher assumes validated arguments and
// returns the hipError_t of its launch.
#pragma once

#include "common.hpp"

namespace fa {

// Resident workgroups per CU of kernel k launched with `threads` threads (the
// occupancy query; 1 where the query fails).
int resident_per_cu(const void* k, int threads);

// Workgroups of a persistent grid over `items` work items: as many as the
// current device holds at once (its CU count times per_cu), at most `items`;
// 0 where the device cannot be queried.
int persistent_grid(long long items, int per_cu);

hipError_t launch_preprocess(int dtype, const void* O, const void* dO, float* D, Shape s,
                             hipStream_t st);

hipError_t launch_convert_dq(int dtype, const float* dq_accum, void* dQ, Shape s,
                             float scale, hipStream_t st);

hipError_t launch_fwd(int dtype, const void* Q, const void* K, const void* V, void* O,
                      float* L, Shape s, float scale, bool causal, hipStream_t st);

// Matrix-core forward, bf16 or fp16 (dtype), head dim 64 or 128.
hipError_t launch_fwd_mfma(int dtype, const void* Q, const void* K, const void* V, void* O,
                           float* L, Shape s, float scale, bool causal, hipStream_t st);

// L alone, by the same two forward kernels without V and O.
hipError_t launch_lse(int dtype, const void* Q, const void* K, float* L, Shape s, float scale,
                      bool causal, hipStream_t st);
hipError_t launch_lse_mfma(int dtype, const void* Q, const void* K, float* L, Shape s,
                           float scale, bool causal, hipStream_t st);

// Vector-ALU backward (fp32 FMA), every dtype and head dim: key-outer dK/dV
// pass and query-outer dQ pass (dq_accum rows written once, unscaled).
hipError_t launch_bwd_dkdv_simt(int dtype, const void* Q, const void* K, const void* V,
                                const void* dO, const float* L, const float* D, void* dK,
                                void* dV, Shape s, float scale, bool causal, hipStream_t st);
hipError_t launch_bwd_dq_simt(int dtype, const void* Q, const void* K, const void* V,
                              const void* dO, const float* L, const float* D, float* dq_accum,
                              Shape s, float scale, bool causal, hipStream_t st);
// Both vector-ALU passes in one launch (fa_bwd).
hipError_t launch_bwd_fused_simt(int dtype, const void* Q, const void* K, const void* V,
                                 const void* dO, const float* L, const float* D, float* dq_accum,
                                 void* dK, void* dV, Shape s, float scale, bool causal,
                                 hipStream_t st);
// The same dQ pass writing dQ = scale * dq_accum in the element type directly.
hipError_t launch_bwd_dq_simt_direct(int dtype, const void* Q, const void* K, const void* V,
                                     const void* dO, const float* L, const float* D, void* dQ,
                                     Shape s, float scale, bool causal, hipStream_t st);

// Matrix-core backward, bf16 or fp16 (dtype), head dim 64 or 128: key-outer
// dK/dV pass and query-outer dQ pass (dq_accum rows written once, unscaled).
hipError_t launch_bwd_dkdv_mfma(int dtype, const void* Q, const void* K, const void* V,
                                const void* dO, const float* L, const float* D, void* dK,
                                void* dV, Shape s, float scale, bool causal, hipStream_t st);
// Both matrix-core passes in one launch (fa_bwd): dQ-pass work items first,
// then dK/dV-pass work items, in one grid.
hipError_t launch_bwd_fused_mfma(int dtype, const void* Q, const void* K, const void* V,
                                 const void* dO, const float* L, const float* D, float* dq_accum,
                                 void* dK, void* dV, Shape s, float scale, bool causal,
                                 hipStream_t st);
hipError_t launch_bwd_dq_mfma(int dtype, const void* Q, const void* K, const void* V,
                              const void* dO, const float* L, const float* D, float* dq_accum,
                              Shape s, float scale, bool causal, hipStream_t st);
// The same dQ pass writing dQ = scale * dq_accum in the element type directly.
hipError_t launch_bwd_dq_mfma_direct(int dtype, const void* Q, const void* K, const void* V,
                                     const void* dO, const float* L, const float* D, void* dQ,
                                     Shape s, float scale, bool causal, hipStream_t st);

}  // namespace fa
