// fwd_mfma.hip -- attention forward on gfx950 matrix cores, bf16 and fp16, head dims 64
// and 128: O and the logsumexp L (supporting step: they feed the backward).
//
// Query blocks outer, key blocks inner, online softmax per query
// (1point3acres post "手扒了FlashAttention": running max m, denominator l and
// accumulator a; per key block the accumulator and denominator are rebased
// to the new maximum before the block's terms are added; finally O = a / l
// and L = m + log l, which FA2 chapter 16 sec 16.4 stores for the backward).
// The rebase is lazy: the maximum the terms are taken against only moves
// when the block maximum exceeds it by more than 2^8 (in exp2 units), so most
// blocks skip rescaling the accumulator; every term stays below 2^8 and the
// quotient a / l is unchanged.  Under the causal mask the key loop stops at
// the diagonal (FA2 chapter 16 sec 16.8 item 2).
//
// gfx950 mapping: 8 waves, two per SIMD; wave w owns queries [32 w, +32) of
// the workgroup's 256 (its Q^T B-operand fragments stay in registers).  Key
// blocks of 64 run in phases, one barrier each; in phase j a wave forms
// S^T = K Q^T of block j (key on rows, query on lanes: a query's maximum,
// denominator and rescale factor are per-lane values) while, in between those
// products, it adds O^T += V^T P^T of block j - 1: P^T straight from registers
// (accumulator layout, contraction index permuted), V^T through
// ds_read_b64_tr_b16.  Then it turns S^T into P^T for the next phase.  All
// waves copy parts of key block j + 2 of K and V into LDS (direct-to-LDS
// loads); K rotates through three buffers, V through four (112 KiB at
// d = 128, 56 KiB at d = 64).  Key rows
// at or beyond N are staged as copies of row N - 1 and masked; query rows at
// or beyond N are not stored.
//
// Without O (WITH_O false) the same kernel is the pass that recomputes L
// when the forward did not store it (FA2 chapter 16 sec 16.4: the backward
// then has to run the online softmax once more, a full sweep over K): no V
// copies, no O^T products, only the running maximum and denominator.
#include "launch.hpp"
#include "mfma_common.hpp"

namespace fa {
namespace {

using namespace mf;

constexpr int BQ = 256;                  // queries per workgroup
constexpr int BK = 64;                   // keys per block
constexpr int NWAVE = 8;
constexpr int SD = 2;                    // blocks copied ahead
constexpr int NKB = SD + 1;              // K buffers: blocks j .. j + SD
constexpr int NVB = SD + 2;              // V buffers: blocks j - 1 .. j + SD

// LDS plan for head dim DH
template <int DH>
struct Plan {
    static constexpr int ROWB = 2 * DH;           // bytes per 16-bit row
    static constexpr int NI = DH / 16;            // d-chunks of an S^T product's contraction
    static constexpr int DB = DH / 32;            // 32-row blocks of d (O^T accumulators)
    static constexpr int TILE = BK * ROWB;        // one K or V block
    static constexpr int OFF_K = 0;
    static constexpr int OFF_V = NKB * TILE;
    static constexpr int LDS_BYTES = OFF_V + NVB * TILE;
    static_assert(LDS_BYTES <= 112 * 1024, "LDS plan");
};
constexpr float kLazy = 8.f;             // rebase threshold, log2 units
constexpr float kLn2 = 0.6931471805599453f;

template <typename E, int DH, bool CAUSAL, bool WITH_O>
__global__ __launch_bounds__(NWAVE * 64) void fwd_mfma_kernel(
    const e16_t* __restrict__ Q, const e16_t* __restrict__ K, const e16_t* __restrict__ V,
    e16_t* __restrict__ O, float* __restrict__ Lg, int N, int nqb, float scale) {
    using PL = Plan<DH>;
    constexpr int NI = PL::NI, DB = PL::DB;
    constexpr int NSTEP = 2 * NI;  // S^T products per block (= O^T products, 4 DB)
    static_assert(NSTEP == 4 * DB, "one O^T product per S^T product");
    // without O only the K buffers are used (48 KiB at d = 128): two
    // workgroups fit a CU
    __shared__ __attribute__((aligned(1024))) unsigned char smem[WITH_O ? PL::LDS_BYTES : PL::OFF_V];

    const int work = xcd_work_item(blockIdx.x, gridDim.x);
    int head = work / nqb, qblk = work % nqb;
    if (CAUSAL) {  // heaviest (last) query blocks first
        heavy_first_work(work, gridDim.x, nqb, head, qblk);
        qblk = nqb - 1 - qblk;
    }
    const int q0 = qblk * BQ;
    const long long hoff = (long long)head * N * DH;
    const e16_t* Kh = K + hoff;
    const e16_t* Vh = V + hoff;

    const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, h = l >> 5, n = l & 31;
    const int q = q0 + 32 * wave + n;  // this lane's query
    const int kend = CAUSAL ? min(N, q0 + BQ) : N;
    const int nblk = (kend + BK - 1) / BK;
    const int full = CAUSAL ? min(q0 / BK, N / BK) : N / BK;  // blocks needing no mask
    const float sc = scale * kLog2e;

#pragma unroll
    for (int b = 0; b < SD; ++b) {
        if (b < nblk) {
            stage_rows<BK, NWAVE, DH>(smem + PL::OFF_K + b * PL::TILE, Kh, b * BK, N, wave, l);
            if (WITH_O)
                stage_rows<BK, NWAVE, DH>(smem + PL::OFF_V + b * PL::TILE, Vh, b * BK, N, wave, l);
        }
    }
    const int qc = q < N ? q : N - 1;  // clamped: finite data, row not stored
    v16x8_t qt[NI];
#pragma unroll
    for (int dk = 0; dk < NI; ++dk)
        qt[dk] = as_v16x8(*reinterpret_cast<const uint4*>(Q + hoff + (long long)qc * DH + 16 * dk + 8 * h));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // per-lane operand offsets: S^T A operand (K row n, d-chunk i, this half);
    // V^T A operand (transposing reads of key rows 4 h + (l % 16) / 4 and + 8,
    // d-block db) -- key rows 32 + ... and 16 t + ... share their swizzle
    int so[NI], ob0[DB], ob1[DB];
#pragma unroll
    for (int i = 0; i < NI; ++i) so[i] = tile_off<PL::ROWB>(n, 32 * i + 16 * h);
    {
        const int g2 = (l >> 4) & 1, x = 4 * h + ((l & 15) >> 2);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int colb = 64 * db + 32 * g2 + 8 * (l & 3);
            ob0[db] = tile_off<PL::ROWB>(x, colb);
            ob1[db] = tile_off<PL::ROWB>(x + 8, colb);
        }
    }
    using Copier = TileCopier<BK, NWAVE, DH>;
    const Copier cp(wave, l);
    const uint32_t lds0 = lds_addr(smem);

    f32x16_t acc[DB];  // O^T of d-block db: lane = query, rows 32 db + 8 (r / 4) + 4 h + r % 4
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i] = f32x16_t{};
    v16x8_t pb[4];   // P^T of the previous block, 16-key step t = 2 mb + hh
    float mu = -1e30f, lsum = 0.f;

    // with O the last phase only adds block nblk - 1's O^T products
    const int jend = WITH_O ? nblk : nblk - 1;
    for (int j = 0; j <= jend; ++j) {
        // copies of block j + SD; past the last block the buffers they fill
        // are read by no one, and they are issued all the same (rows clamped
        // into range) to keep the loop free of branches around them
        {
            const int kn = (j + SD) * BK;
            const uint32_t lk = lds0 + PL::OFF_K + ((j + SD) % NKB) * PL::TILE;
            const uint32_t lv = lds0 + PL::OFF_V + ((j + SD) % NVB) * PL::TILE;
#pragma unroll
            for (int s = 0; s < cp.SLICES; ++s) {
                cp.copy(s, Kh, kn, N, lk);
                if (WITH_O) cp.copy(s, Vh, kn, N, lv);
            }
        }
        const bool mf = j < nblk, pv = WITH_O && j >= 1;
        const unsigned char* sK = smem + PL::OFF_K + (j % NKB) * PL::TILE;
        const unsigned char* sV = smem + PL::OFF_V + ((j + NVB - 1) % NVB) * PL::TILE;
        f32x16_t S0 = f32x16_t{}, S1 = f32x16_t{};
        // NSTEP steps: S^T product i (key half i / NI, d-chunk i % NI) and O^T
        // product i (16-key step i / DB, d-block i % DB); operands two / one
        // steps ahead
        v16x8_t ak[3], av[2];
        auto kop = [&](int i) { return lds_b128(sK + so[i % NI] + 32 * PL::ROWB * (i / NI)); };
        auto vop = [&](int i) {
            const int t = i / DB, db = i % DB;
            return tr16_pair(sV + ob0[db] + 16 * PL::ROWB * t, sV + ob1[db] + 16 * PL::ROWB * t);
        };
        if (mf) {
            ak[0] = kop(0);
            ak[1] = kop(1);
        }
        if (pv) av[0] = vop(0);
#pragma unroll
        for (int i = 0; i < NSTEP; ++i) {
            if (mf) {
                if (i + 2 < NSTEP) ak[(i + 2) % 3] = kop(i + 2);
                if (i < NI)
                    S0 = E::mma(ak[i % 3], qt[i], S0);
                else
                    S1 = E::mma(ak[i % 3], qt[i - NI], S1);
            }
            if (pv) {
                if (i + 1 < NSTEP) av[(i + 1) & 1] = vop(i + 1);
                acc[i % DB] = E::mma(av[i & 1], pb[i / DB], acc[i % DB]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (mf) {
            // raw scores, masked where needed; the block maximum is taken on
            // them and scaled once (the scale is positive, so the maximum of
            // the scaled scores is the scaled maximum, exactly)
            float s2[32];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s2[r] = S0[r];
                s2[16 + r] = S1[r];
            }
            if (j >= full) {
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const int key = j * BK + 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * h + (e & 3);
                    if (key >= N || (CAUSAL && key > q)) s2[e] = -INFINITY;
                }
            }
            // block maximum as four interleaved chains (exact in any order)
            float m4[4] = {s2[0], s2[1], s2[2], s2[3]};
#pragma unroll
            for (int e = 4; e < 32; ++e) m4[e & 3] = fmaxf(m4[e & 3], s2[e]);
            float bm = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * sc;
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const bool rebase = bm > mu + kLazy;
            if (__ballot(rebase)) {
                const float alpha = rebase ? __builtin_amdgcn_exp2f(mu - bm) : 1.f;
                mu = rebase ? bm : mu;
                lsum *= alpha;
                if (WITH_O)
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
            }
            // terms grouped by operation (the scaling and the subtraction of
            // the running maximum are one fused multiply-add), the
            // denominator summed in four interleaved partial sums, so that no
            // result feeds the very next instruction
            float p[32];
#pragma unroll
            for (int e = 0; e < 32; ++e) p[e] = __builtin_fmaf(s2[e], sc, -mu);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 32; ++e) p[e] = __builtin_amdgcn_exp2f(p[e]);
            __builtin_amdgcn_sched_barrier(0);
            float l4[4] = {p[0], p[1], p[2], p[3]};
#pragma unroll
            for (int e = 4; e < 32; ++e) l4[e & 3] += p[e];
            lsum += (l4[0] + l4[1]) + (l4[2] + l4[3]);
            if (WITH_O)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    pb[t] = as_v16x8(make_uint4(E::pack2(p[8 * t], p[8 * t + 1]),
                                             E::pack2(p[8 * t + 2], p[8 * t + 3]),
                                             E::pack2(p[8 * t + 4], p[8 * t + 5]),
                                             E::pack2(p[8 * t + 6], p[8 * t + 7])));
        }
        // block j + 1's copies (issued one phase ago) must have landed; this
        // phase's (SLICES per tensor) may stay in flight
        if (j < jend)
            __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0((WITH_O ? 2 : 1) * Copier::SLICES));
        else
            __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    if (q < N) {
        if (WITH_O) {
            const float inv = 1.f / ltot;
            e16_t* orow = O + hoff + (long long)q * DH;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int r = 4 * a4;
                    uint2 v;
                    v.x = E::pack2(acc[db][r] * inv, acc[db][r + 1] * inv);
                    v.y = E::pack2(acc[db][r + 2] * inv, acc[db][r + 3] * inv);
                    *reinterpret_cast<uint2*>(orow + 32 * db + 8 * a4 + 4 * h) = v;
                }
        }
        if (h == 0) Lg[(long long)head * N + q] = (mu + __builtin_log2f(ltot)) * kLn2;
    }
}

template <typename E, int DH, bool WITH_O>
hipError_t launch_fwd_mfma(const void* Q, const void* K, const void* V, void* O, float* L,
                           Shape s, float scale, bool causal, hipStream_t st) {
    const int nqb = (s.N + BQ - 1) / BQ;
    const long long nwork = (long long)nqb * s.H * s.B;
    if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)nwork);
    if (causal)
        hipLaunchKernelGGL((fwd_mfma_kernel<E, DH, true, WITH_O>), grid, dim3(NWAVE * 64), 0, st,
                           (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (e16_t*)O, L, s.N,
                           nqb, scale);
    else
        hipLaunchKernelGGL((fwd_mfma_kernel<E, DH, false, WITH_O>), grid, dim3(NWAVE * 64), 0, st,
                           (const e16_t*)Q, (const e16_t*)K, (const e16_t*)V, (e16_t*)O, L, s.N,
                           nqb, scale);
    return hipGetLastError();
}

template <bool WITH_O>
hipError_t launch_fwd_any(int dtype, const void* Q, const void* K, const void* V, void* O,
                          float* L, Shape s, float scale, bool causal, hipStream_t st) {
    if (s.d != 64 && s.d != 128) return hipErrorInvalidValue;
    if (dtype == DT_F16)
        return s.d == 64 ? launch_fwd_mfma<F16E, 64, WITH_O>(Q, K, V, O, L, s, scale, causal, st)
                         : launch_fwd_mfma<F16E, 128, WITH_O>(Q, K, V, O, L, s, scale, causal, st);
    return s.d == 64 ? launch_fwd_mfma<Bf16E, 64, WITH_O>(Q, K, V, O, L, s, scale, causal, st)
                     : launch_fwd_mfma<Bf16E, 128, WITH_O>(Q, K, V, O, L, s, scale, causal, st);
}

}  // namespace

hipError_t launch_fwd_mfma(int dtype, const void* Q, const void* K, const void* V, void* O,
                           float* L, Shape s, float scale, bool causal, hipStream_t st) {
    return launch_fwd_any<true>(dtype, Q, K, V, O, L, s, scale, causal, st);
}

// L alone (no O); V is never read, K stands in for it.
hipError_t launch_lse_mfma(int dtype, const void* Q, const void* K, float* L, Shape s,
                           float scale, bool causal, hipStream_t st) {
    return launch_fwd_any<false>(dtype, Q, K, K, nullptr, L, s, scale, causal, st);
}

}  // namespace fa
