// bwd_mfma.hip -- FA2 backward main kernel on CDNA4 bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16), head dim 128.
//
// Method (FA2 chapter 16): one workgroup per (key block of 128 keys, head,
// batch) -- the sec 16.6 grid -- with key blocks outer and query tiles inner
// (sec 16.2).  Per query tile of 64 rows it recomputes S = scale Q K^T and
// P = exp(S - L) (sec 16.4), forms dP = dO V^T and dS = P (dP - D) with D from
// the preprocess (sec 16.1, sec 16.8 item 1), accumulates dV += P^T dO and
// dK += dS^T Q in registers for the whole loop, and adds the unscaled dS K
// into the fp32 dq_accum buffer with atomics (sec 16.3).  dK is scaled at
// write-out (sec 16.6).  Under the causal mask the query loop starts at the
// key block's first key, so tiles above the diagonal are never visited
// (sec 16.8 item 2); diagonal tiles are masked element by element.
//
// gfx950 mapping (4 waves, one per SIMD):
//   * wave w owns keys [32w, 32w+32) of the block.  Its K^T and V^T operand
//     fragments (B operands of S = Q K^T and dP = dO V^T) and the K fragment
//     for its 32-column slice of d (B operand of dQ = dS K) stay in VGPRs for
//     the whole query loop; dV^T and dK^T (32 d x 32 keys x 4 d-blocks each)
//     accumulate in registers.
//   * Q and dO tiles are double-buffered in LDS with an XOR swizzle of 16-byte
//     chunks; the next tile's global loads are issued before the current
//     tile's matrix work.
//   * S and dP come out of the matrix core with the key on the lane, so P and
//     dS feed dV^T = dO^T P and dK^T = Q^T dS straight from registers; the
//     transposed A operands dO^T and Q^T come from the row-major LDS tiles
//     through ds_read_b64_tr_b16.
//   * dS^T goes to LDS ([key][query], bf16) so every wave can form dQ for its
//     own 32 columns of d over all 128 keys; its A operand is again a
//     transposing LDS read.  dQ partials go to dq_accum with no-return fp32
//     atomics, one per (key block, query tile) pair.
//   * P = exp2(S * scale * log2(e) - L * log2(e)) with L pre-multiplied by
//     log2(e) when staged; rows beyond N get L = +inf (P = 0).
//   * Workgroups are numbered so that consecutive work items -- the key blocks
//     of one head, heaviest first under the causal mask -- land on the same
//     XCD and share its L2 for the Q, dO and dq_accum traffic of that head.
#include "launch.hpp"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b,
                                                 const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
    return __builtin_bit_cast(bf16x8_t, u);
}

// Two transposing 8-byte LDS reads combined into one 8-element operand.
__device__ __forceinline__ bf16x8_t tr16_pair(const unsigned char* p0, const unsigned char* p1) {
    i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4_t, p0));
    i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4_t, p1));
    i16x8_t v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
}

// 16-byte chunk swizzles (chunk index within a row).
__device__ __forceinline__ int swz_tile(int row) { return row & 15; }       // 256-byte rows
__device__ __forceinline__ int swz_ds(int row) { return ((row & 1) << 2) | ((row >> 1) & 3); }  // 128-byte rows

constexpr int D = 128;     // head dim
constexpr int BC = 128;    // keys per workgroup
constexpr int BR = 64;     // queries per inner tile
constexpr int NTHR = 256;  // 4 waves
constexpr int ROWB = D * 2;                 // bytes per Q/dO/K row
constexpr int TILE = BR * ROWB;             // 16 KiB
constexpr int OFF_Q = 0;                    // 2 buffers
constexpr int OFF_DO = 2 * TILE;            // 2 buffers
constexpr int OFF_DST = 4 * TILE;           // dS^T [BC][BR] bf16 = 16 KiB
constexpr int DST_ROWB = BR * 2;            // 128 bytes
constexpr int OFF_L = OFF_DST + BC * DST_ROWB;  // 2 x BR floats
constexpr int OFF_D = OFF_L + 2 * BR * 4;       // 2 x BR floats
constexpr int LDS_BYTES = OFF_D + 2 * BR * 4;
static_assert(2 * TILE >= BC * ROWB, "K staging must fit in the Q buffers");

struct TileRegs {
    uint4 q[4], g[4];
    float lg;  // L (lanes 0..63) or D (lanes 64..127)
};

// Global -> registers for one query tile: lane t loads 16-byte chunk t%16 of
// rows t/16 + 16 i.  Rows at or beyond N load zeros; their L is +inf.
__device__ __forceinline__ void load_tile(TileRegs& r, const bf16_t* Qh, const bf16_t* dOh,
                                          const float* Lh, const float* Dh, int q0, int N,
                                          int tid) {
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 4) + 16 * i;
        const int q = q0 + row;
        if (q < N) {
            r.q[i] = *reinterpret_cast<const uint4*>(Qh + (long long)q * D + 8 * c);
            r.g[i] = *reinterpret_cast<const uint4*>(dOh + (long long)q * D + 8 * c);
        } else {
            r.q[i] = make_uint4(0, 0, 0, 0);
            r.g[i] = make_uint4(0, 0, 0, 0);
        }
    }
    if (tid < 2 * BR) {
        const int row = tid & (BR - 1);
        const int q = q0 + row;
        if (tid < BR)
            r.lg = q < N ? Lh[q] * kLog2e : INFINITY;
        else
            r.lg = q < N ? Dh[q] : 0.f;
    }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, unsigned char* smem, int buf,
                                           int tid) {
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (tid >> 4) + 16 * i;
        const int off = row * ROWB + ((c ^ swz_tile(row)) << 4);
        *reinterpret_cast<uint4*>(smem + OFF_Q + buf * TILE + off) = r.q[i];
        *reinterpret_cast<uint4*>(smem + OFF_DO + buf * TILE + off) = r.g[i];
    }
    if (tid < 2 * BR) {
        const int row = tid & (BR - 1);
        float* dst = reinterpret_cast<float*>(smem + (tid < BR ? OFF_L : OFF_D) + buf * BR * 4);
        dst[row] = r.lg;
    }
}

template <bool CAUSAL>
__global__ __launch_bounds__(NTHR) void bwd_mfma_d128_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ Lg, const float* __restrict__ Dg,
    float* __restrict__ dqa, bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int N, int nkb,
    float scale) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[LDS_BYTES];

    // work item: consecutive items share an XCD (workgroups are dealt to the
    // 8 XCDs round-robin by workgroup id)
    const int nwork = gridDim.x;
    const int bid = blockIdx.x;
    const int work = (nwork % 8 == 0) ? (bid % 8) * (nwork / 8) + bid / 8 : bid;
    const int head = work / nkb;
    const int kb = work % nkb;
    const int k0 = kb * BC;
    const long long hoff = (long long)head * N * D;
    const bf16_t* Qh = Q + hoff;
    const bf16_t* Kh = K + hoff;
    const bf16_t* Vh = V + hoff;
    const bf16_t* dOh = dO + hoff;
    const float* Lh = Lg + (long long)head * N;
    const float* Dh = Dg + (long long)head * N;
    float* dqh = dqa + hoff;

    const int tid = threadIdx.x;
    const int w = tid >> 6;        // wave
    const int l = tid & 63;        // lane
    const int h = l >> 5;          // half of the wave
    const int n = l & 31;          // lane within half
    const int g2 = (l >> 4) & 1;   // 16-lane group within half
    const int key = k0 + 32 * w + n;  // this lane's key in S / dP / dV / dK

    // ---- K^T, V^T operand fragments: K[key][16 dk + 8 h .. +7]
    bf16x8_t kt[8], vt[8];
#pragma unroll
    for (int dk = 0; dk < 8; ++dk) {
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        if (key < N) {
            a = *reinterpret_cast<const uint4*>(Kh + (long long)key * D + 16 * dk + 8 * h);
            b = *reinterpret_cast<const uint4*>(Vh + (long long)key * D + 16 * dk + 8 * h);
        }
        kt[dk] = as_bf16x8(a);
        vt[dk] = as_bf16x8(b);
    }

    // ---- K fragment for dQ = dS K over this wave's d columns [32 w, 32 w + 32):
    // stage the K block in LDS (row = key), then transpose-read.
    {
        const int c = tid & 15;
#pragma unroll
        for (int i = 0; i < BC / 16; ++i) {
            const int row = (tid >> 4) + 16 * i;
            const int kk = k0 + row;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (kk < N) v = *reinterpret_cast<const uint4*>(Kh + (long long)kk * D + 8 * c);
            *reinterpret_cast<uint4*>(smem + OFF_Q + row * ROWB + ((c ^ swz_tile(row)) << 4)) = v;
        }
    }
    __syncthreads();
    bf16x8_t kd[8];
    {
        const int colb = 64 * w + 32 * g2 + 8 * (l & 3);  // byte column of the 8-byte chunk
        const int chunk = colb >> 4, within = colb & 15;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int r0 = 16 * kk + 8 * h + ((l & 15) >> 2);
            const int r1 = r0 + 4;
            kd[kk] = tr16_pair(smem + OFF_Q + r0 * ROWB + ((chunk ^ swz_tile(r0)) << 4) + within,
                               smem + OFF_Q + r1 * ROWB + ((chunk ^ swz_tile(r1)) << 4) + within);
        }
    }
    __syncthreads();

    f32x16_t accdV[4], accdK[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        accdV[i] = f32x16_t{};
        accdK[i] = f32x16_t{};
    }

    const int q_begin = CAUSAL ? k0 : 0;
    const int ntiles = (N - q_begin + BR - 1) / BR;
    const float sc = scale * kLog2e;

    TileRegs pf;
    load_tile(pf, Qh, dOh, Lh, Dh, q_begin, N, tid);
    store_tile(pf, smem, 0, tid);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        const int q0 = q_begin + it * BR;
        const bool more = it + 1 < ntiles;
        if (more) load_tile(pf, Qh, dOh, Lh, Dh, q0 + BR, N, tid);

        const unsigned char* sQ = smem + OFF_Q + buf * TILE;
        const unsigned char* sdO = smem + OFF_DO + buf * TILE;
        const float* sL = reinterpret_cast<const float*>(smem + OFF_L + buf * BR * 4);
        const float* sD = reinterpret_cast<const float*>(smem + OFF_D + buf * BR * 4);

        // ---- S = Q K^T and dP = dO V^T (query on rows, key on lanes)
        f32x16_t S[2], dP[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            S[qb] = f32x16_t{};
            dP[qb] = f32x16_t{};
            const int row = 32 * qb + n;
#pragma unroll
            for (int dk = 0; dk < 8; ++dk) {
                const int off = row * ROWB + (((2 * dk + h) ^ swz_tile(row)) << 4);
                const bf16x8_t a = as_bf16x8(*reinterpret_cast<const uint4*>(sQ + off));
                const bf16x8_t g = as_bf16x8(*reinterpret_cast<const uint4*>(sdO + off));
                S[qb] = mfma32x32x16(a, kt[dk], S[qb]);
                dP[qb] = mfma32x32x16(g, vt[dk], dP[qb]);
            }
        }

        // ---- P = exp2(S sc - L'), dS = P (dP - D); pack to bf16
        const bool need_mask = (CAUSAL && q0 < k0 + BC) || (k0 + BC > N);
        bf16x8_t Pb[2][2], dSb[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float p[16], ds[16];
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int rq = 32 * qb + 8 * a4 + 4 * h;  // first of 4 consecutive rows
                const f32x4_t Lv = *reinterpret_cast<const f32x4_t*>(sL + rq);
                const f32x4_t Dv = *reinterpret_cast<const f32x4_t*>(sD + rq);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * a4 + e;
                    float x = S[qb][r] * sc - Lv[e];
                    if (need_mask) {
                        const int q = q0 + rq + e;
                        if (key >= N || (CAUSAL && key > q)) x = -INFINITY;
                    }
                    const float pv = __builtin_amdgcn_exp2f(x);
                    p[r] = pv;
                    ds[r] = pv * (dP[qb][r] - Dv[e]);
                }
            }
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                uint4 up, ud;
                up.x = pack_bf16x2(p[8 * hh + 0], p[8 * hh + 1]);
                up.y = pack_bf16x2(p[8 * hh + 2], p[8 * hh + 3]);
                up.z = pack_bf16x2(p[8 * hh + 4], p[8 * hh + 5]);
                up.w = pack_bf16x2(p[8 * hh + 6], p[8 * hh + 7]);
                ud.x = pack_bf16x2(ds[8 * hh + 0], ds[8 * hh + 1]);
                ud.y = pack_bf16x2(ds[8 * hh + 2], ds[8 * hh + 3]);
                ud.z = pack_bf16x2(ds[8 * hh + 4], ds[8 * hh + 5]);
                ud.w = pack_bf16x2(ds[8 * hh + 6], ds[8 * hh + 7]);
                Pb[qb][hh] = as_bf16x8(up);
                dSb[qb][hh] = as_bf16x8(ud);
                // dS^T row = this lane's key, queries 32 qb + 16 hh + {4h..4h+3, 8+4h..8+4h+3}
                const int krow = 32 * w + n;
#pragma unroll
                for (int part = 0; part < 2; ++part) {
                    const int chunk = 4 * qb + 2 * hh + part;
                    uint2 v = part ? make_uint2(ud.z, ud.w) : make_uint2(ud.x, ud.y);
                    *reinterpret_cast<uint2*>(smem + OFF_DST + krow * DST_ROWB +
                                              ((chunk ^ swz_ds(krow)) << 4) + 8 * h) = v;
                }
            }
        }

        // ---- dV^T += dO^T P, dK^T += Q^T dS  (d on rows, key on lanes)
#pragma unroll
        for (int t = 0; t < 4; ++t) {  // 16-query steps
            const int r0 = 16 * t + 4 * h + ((l & 15) >> 2);
            const int r1 = r0 + 8;
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const int colb = 64 * db + 32 * g2 + 8 * (l & 3);
                const int chunk = colb >> 4, within = colb & 15;
                const int o0 = r0 * ROWB + ((chunk ^ swz_tile(r0)) << 4) + within;
                const int o1 = r1 * ROWB + ((chunk ^ swz_tile(r1)) << 4) + within;
                const bf16x8_t aO = tr16_pair(sdO + o0, sdO + o1);
                const bf16x8_t aQ = tr16_pair(sQ + o0, sQ + o1);
                accdV[db] = mfma32x32x16(aO, Pb[t >> 1][t & 1], accdV[db]);
                accdK[db] = mfma32x32x16(aQ, dSb[t >> 1][t & 1], accdK[db]);
            }
        }
        __syncthreads();  // dS^T complete

        // ---- dQ[:, 32w .. 32w+31] = dS K over the 128 keys; atomics into dq_accum
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            f32x16_t acc = f32x16_t{};
            const int colb = 64 * qb + 32 * g2 + 8 * (l & 3);
            const int chunk = colb >> 4, within = colb & 15;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int r0 = 16 * kk + 8 * h + ((l & 15) >> 2);
                const int r1 = r0 + 4;
                const bf16x8_t a = tr16_pair(
                    smem + OFF_DST + r0 * DST_ROWB + ((chunk ^ swz_ds(r0)) << 4) + within,
                    smem + OFF_DST + r1 * DST_ROWB + ((chunk ^ swz_ds(r1)) << 4) + within);
                acc = mfma32x32x16(a, kd[kk], acc);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = q0 + 32 * qb + 8 * (r >> 2) + 4 * h + (r & 3);
                if (q < N) atomicAdd(dqh + (long long)q * D + 32 * w + n, acc[r]);
            }
        }

        if (more) store_tile(pf, smem, buf ^ 1, tid);
        __syncthreads();
    }

    // ---- epilogue: dK = scale dK^T^T, dV = dV^T^T; lane holds key, 4 consecutive d per store
    if (key < N) {
        bf16_t* dKr = dK + hoff + (long long)key * D;
        bf16_t* dVr = dV + hoff + (long long)key * D;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = 32 * db + 8 * a4 + 4 * h;
                const int r = 4 * a4;
                uint2 kv, vv;
                kv.x = pack_bf16x2(accdK[db][r] * scale, accdK[db][r + 1] * scale);
                kv.y = pack_bf16x2(accdK[db][r + 2] * scale, accdK[db][r + 3] * scale);
                vv.x = pack_bf16x2(accdV[db][r], accdV[db][r + 1]);
                vv.y = pack_bf16x2(accdV[db][r + 2], accdV[db][r + 3]);
                *reinterpret_cast<uint2*>(dKr + d0) = kv;
                *reinterpret_cast<uint2*>(dVr + d0) = vv;
            }
        }
    }
}

}  // namespace

// bf16, d = 128 main kernel.  Grid: one workgroup per (key block, head, batch).
hipError_t launch_bwd_mfma_d128(const void* Q, const void* K, const void* V, const void* dO,
                                const float* L, const float* Dv, float* dqa, void* dK, void* dV,
                                Shape s, float scale, bool causal, hipStream_t st) {
    const int nkb = (s.N + BC - 1) / BC;
    const long long nwork = (long long)nkb * s.H * s.B;
    if (nwork > 0x7fffffffLL) return hipErrorInvalidValue;
    dim3 grid((unsigned)nwork);
    if (causal)
        hipLaunchKernelGGL((bwd_mfma_d128_kernel<true>), grid, dim3(NTHR), 0, st, (const bf16_t*)Q,
                           (const bf16_t*)K, (const bf16_t*)V, (const bf16_t*)dO, L, Dv, dqa,
                           (bf16_t*)dK, (bf16_t*)dV, s.N, nkb, scale);
    else
        hipLaunchKernelGGL((bwd_mfma_d128_kernel<false>), grid, dim3(NTHR), 0, st,
                           (const bf16_t*)Q, (const bf16_t*)K, (const bf16_t*)V, (const bf16_t*)dO,
                           L, Dv, dqa, (bf16_t*)dK, (bf16_t*)dV, s.N, nkb, scale);
    return hipGetLastError();
}

}  // namespace fa
