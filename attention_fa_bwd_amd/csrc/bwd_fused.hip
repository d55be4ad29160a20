// bwd_fused.hip -- fa_bwd's two matrix-core passes in one launch.
//
// Given D, the query-outer dQ pass (bwd_dq.hpp) and the key-outer dK/dV pass
// (bwd_dkdv.hpp) read the same inputs and write disjoint outputs, so nothing
// orders them (FA2 chapter 16 sec 16.3: dQ by a separate kernel instead of
// atomics).  One persistent grid runs the work items of both: each workgroup
// takes its scheduled dQ-pass items, back to back, and then its dK/dV-pass
// items, each computed exactly as in its own kernel (same code and per-item
// order, so the results are bitwise those of fa_bwd_dq followed by
// fa_bwd_dkdv).  The schedule deals each XCD an eighth of either kind and
// spreads both kinds over all workgroups (a dQ-pass item carries 1.5 times the
// work of a dK/dV item at the same N), so neither pass leaves a tail of idle
// CUs, a small problem runs both passes side by side instead of one after the
// other, and the second launch is saved.
#include "bwd_dkdv.hpp"
#include "bwd_dq.hpp"
#include "launch.hpp"

namespace fa {
namespace {

using namespace mf;

static_assert(dqp::NWAVE == dkvp::NWAVE, "one workgroup shape for both passes");

template <int DH>
constexpr int fused_lds() {
    return dqp::Plan<DH>::LDS_BYTES > dkvp::Plan<DH>::LDS_BYTES ? dqp::Plan<DH>::LDS_BYTES
                                                                 : dkvp::Plan<DH>::LDS_BYTES;
}

template <typename E, int DH, bool CAUSAL>
__global__ __launch_bounds__(dqp::NWAVE * 64) void bwd_fused_kernel(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    const e16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    float* __restrict__ dqa, e16_t* __restrict__ dK, e16_t* __restrict__ dV, int N, int nqb,
    int nkb, int nq, int nk, float scale) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem[fused_lds<DH>()];
    const Schedule sch(nq, nk, gridDim.x, blockIdx.x);
    dqp::dq_run<E, DH, CAUSAL, false>(Q, K, V, dO, Lg, Dg, dqa, N, nqb, scale, sch, Run(sch, 0),
                                      nq, smem);
    // every LDS read of the dQ-pass items precedes their last barrier
    dkvp::dkdv_run<E, DH, CAUSAL>(Q, K, V, dO, Lg, Dg, dK, dV, N, nkb, scale, sch, Run(sch, 1), nk,
                                  smem);
}

template <typename E, int DH, bool CAUSAL>
hipError_t launch_fused_k(const void* Q, const void* K, const void* V, const void* dO,
                          const float* L, const float* Dv, float* dqa, void* dK, void* dV, Shape s,
                          float scale, int nqb, int nkb, int nq, int nk, hipStream_t st) {
    static const int per_cu = resident_per_cu(
        reinterpret_cast<const void*>(&bwd_fused_kernel<E, DH, CAUSAL>), dqp::NWAVE * 64);
    const int G = persistent_grid((long long)nq + nk, per_cu);
    if (G <= 0) return hipErrorInvalidDevice;
    hipLaunchKernelGGL((bwd_fused_kernel<E, DH, CAUSAL>), dim3(G), dim3(dqp::NWAVE * 64), 0, st,
                       (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (const e16_t*)dO, L, Dv,
                       dqa, (e16_t*)dK, (e16_t*)dV, s.N, nqb, nkb, nq, nk, scale);
    return hipGetLastError();
}

template <typename E, int DH>
hipError_t launch_fused(const void* Q, const void* K, const void* V, const void* dO,
                        const float* L, const float* Dv, float* dqa, void* dK, void* dV, Shape s,
                        float scale, bool causal, hipStream_t st) {
    const int nqb = (s.N + dqp::BQ - 1) / dqp::BQ;
    const int nkb = (s.N + dkvp::BC - 1) / dkvp::BC;
    const long long nq = (long long)nqb * s.H * s.B, nk = (long long)nkb * s.H * s.B;
    if (nq + nk > 0x7fffffffLL) return hipErrorInvalidValue;
    return causal ? launch_fused_k<E, DH, true>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, nqb,
                                                 nkb, (int)nq, (int)nk, st)
                  : launch_fused_k<E, DH, false>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, nqb,
                                                  nkb, (int)nq, (int)nk, st);
}

template <typename E>
hipError_t launch_fused_e(const void* Q, const void* K, const void* V, const void* dO,
                          const float* L, const float* Dv, float* dqa, void* dK, void* dV,
                          Shape s, float scale, bool causal, hipStream_t st) {
    return s.d == 64
               ? launch_fused<E, 64>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st)
               : launch_fused<E, 128>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
}

}  // namespace

hipError_t launch_bwd_fused_mfma(int dtype, const void* Q, const void* K, const void* V,
                                 const void* dO, const float* L, const float* Dv, float* dqa,
                                 void* dK, void* dV, Shape s, float scale, bool causal,
                                 hipStream_t st) {
    if (s.d != 64 && s.d != 128) return hipErrorInvalidValue;
    return dtype == DT_F16
               ? launch_fused_e<F16E>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st)
               : launch_fused_e<Bf16E>(Q, K, V, dO, L, Dv, dqa, dK, dV, s, scale, causal, st);
}

}  // namespace fa
