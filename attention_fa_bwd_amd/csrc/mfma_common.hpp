// mfma_common.hpp -- CDNA4 (gfx950) matrix-core helpers shared by the
// matrix-core kernels (key-outer dK/dV pass, query-outer dQ pass, forward),
// head dims 64 and 128.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 and _f16 (the same; checked on
// the hardware):
//   A (32 x 16, M x K): lane l holds row l % 32, k = 8 (l / 32) + 0..7
//   B (16 x 32, K x N): lane l holds column l % 32, k = 8 (l / 32) + 0..7
//   C (32 x 32):        lane l holds column l % 32, row 8 (r / 4) + 4 (l / 32) + r % 4
//                       for accumulator register r = 0..15
// ds_read_b64_tr_b16 (per 16-lane group): output lane i, slot s receives
//   element i % 4 of the 8-byte chunk addressed by lane 4 s + i / 4.
//
// A C-layout accumulator can feed a later MFMA as its B operand (or as its A
// operand, when its columns are the new rows) without any data movement: the
// contraction index is then permuted the same way on both operands.  Register
// r = 8 hh + s of a 32-row accumulator is k-slot s of the 16-row step hh and
// holds row 16 hh + 8 (s / 4) + 4 (l / 32) + s % 4.  The matching operand for
// the other side is gathered with two transposing LDS reads over rows
// {16 hh + 4 (l / 32) + 0..3} and {16 hh + 8 + 4 (l / 32) + 0..3}.
#pragma once

#include "common.hpp"

namespace fa {
namespace mf {

// Eight 16-bit elements: one matrix-core operand per lane.  The vector is
// declared with bf16 elements; fp16 operands are carried in it as bit patterns
// and reinterpreted at the fp16 product.
typedef __bf16 v16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

#define FA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt operand that waits for LDS (and scalar) traffic only: vmcnt and
// expcnt at their maxima, lgkmcnt 0.
constexpr int kLgkmOnly = 0xC07F;
// s_waitcnt operand: at most n (< 16) vector-memory operations outstanding,
// LDS and scalar traffic drained (vmcnt n, expcnt 7, lgkmcnt 0).
constexpr int vmcnt_lgkm0(int n) { return 0x0070 | n; }

__device__ __forceinline__ f32x16_t mfma(const v16x8_t& a, const v16x8_t& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Element types of the matrix-core kernels: the product instruction and the
// fp32 -> element packing (round to nearest even).
struct Bf16E {
    static constexpr int dtype = DT_BF16;
    static __device__ __forceinline__ f32x16_t mma(const v16x8_t& a, const v16x8_t& b,
                                                   const f32x16_t& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
};
struct F16E {
    static constexpr int dtype = DT_F16;
    static __device__ __forceinline__ f32x16_t mma(const v16x8_t& a, const v16x8_t& b,
                                                   const f32x16_t& c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_f16x2(a, b); }
};

__device__ __forceinline__ v16x8_t as_v16x8(const uint4& u) { return __builtin_bit_cast(v16x8_t, u); }

__device__ __forceinline__ v16x8_t lds_b128(const unsigned char* p) {
    return as_v16x8(*reinterpret_cast<const uint4*>(p));
}

// Two transposing 8-byte LDS reads combined into one 8-element operand.
__device__ __forceinline__ v16x8_t tr16_pair(const unsigned char* p0, const unsigned char* p1) {
    i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(i16x4_t, p0));
    i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FA_LDS(i16x4_t, p1));
    return __builtin_bit_cast(v16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 16-byte chunk swizzle of an LDS tile row of ROWB bytes (the head dim DH of
// the matrix-core kernels is 64 or 128: rows of 128 or 256 bytes, 8 or 16
// chunks), XORed into the chunk index.  LDS has 64 banks of 4 bytes (256
// bytes per cycle).  The row-wise operand reads (ds_read_b128: 16 lanes, 16
// consecutive rows, one logical chunk) need the 16 rows on 16 distinct
// 16-byte bank slots; the transposing reads (4 consecutive rows x one 64-byte
// block per 32 lanes) need the 4 rows on 4 distinct 64-byte bank groups.
//   256-byte rows: bits [3:2] of the XOR from row bits [1:0], bits [1:0] from
//                  row bits [3:2].
//   128-byte rows: a row pair fills the 256 bank bytes, so row bit 0 already
//                  separates the halves; bit 2 of the XOR from row bit 1,
//                  bits [1:0] from row bits [3:2].
// Both depend on the row modulo 16 only.
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
    static_assert(ROWB == 256 || ROWB == 128, "rows of 64 or 128 16-bit elements");
    return ROWB == 256 ? (((row & 3) << 2) | ((row >> 2) & 3))
                       : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Byte offset of (row, byte column) in a swizzled tile of ROWB-byte rows.
template <int ROWB>
__device__ __forceinline__ int tile_off(int row, int colb) {
    return row * ROWB + ((((colb >> 4) ^ swz<ROWB>(row)) << 4) | (colb & 15));
}

// One direct-to-LDS copy of 16 bytes per lane: lane i's 16 bytes at src land at
// LDS byte lds + 16 i.  Issued as inline assembly on purpose: for the builtin
// form the compiler cannot tell which LDS bytes the copy writes, so it makes
// the wave's next LDS read wait for every outstanding copy -- which would put
// the full load latency of the next tile in front of the current tile's work.
// Callers order these copies themselves: s_waitcnt vmcnt(0) and a barrier
// before any wave reads the destination.  (M0 must be written one instruction
// ahead of its use by the copy.  The compiler reserves M0 and sets it right
// before each of its own uses, so overwriting it here is safe; it warns about
// the clobber all the same.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Copy rows [r0, r0 + NROWS) of a [N, DH] 16-bit matrix into a swizzled LDS
// tile with direct-to-LDS loads: each wave moves 1 KiB (64 lanes x 16 bytes)
// per instruction, lane i landing at byte 16 i of the wave's slice, so lane i
// fetches the logical chunk that the swizzle places there.  Rows at or beyond
// N are clamped to row N - 1 (finite data; callers make them contribute 0).
// UNTRACKED: issue through lds_copy16 (the caller waits before use).
template <int NROWS, int NWAVES, int DH, bool UNTRACKED = false>
__device__ __forceinline__ void stage_rows(unsigned char* lds_tile, const e16_t* src, int r0,
                                           int N, int wave, int lane) {
    constexpr int ROWB = 2 * DH;
    constexpr int BYTES = NROWS * ROWB;
    constexpr int PER_WAVE = BYTES / NWAVES;
    static_assert(PER_WAVE % 1024 == 0, "tile must split into 1 KiB slices per wave");
#pragma unroll
    for (int j = 0; j < PER_WAVE / 1024; ++j) {
        const int p = wave * PER_WAVE + j * 1024 + lane * 16;
        const int row = p / ROWB;
        const int chunk = ((p % ROWB) >> 4) ^ swz<ROWB>(row);
        int g = r0 + row;
        g = g < N ? g : N - 1;
        const e16_t* gp = src + (long long)g * DH + chunk * 8;
        unsigned char* lp = lds_tile + wave * PER_WAVE + j * 1024;
        if (UNTRACKED)
            lds_copy16(gp, __builtin_amdgcn_readfirstlane(
                               (uint32_t)(uintptr_t)FA_LDS(unsigned char, lp)));
        else
            __builtin_amdgcn_global_load_lds(gp, FA_LDS(void, lp), 16, 0, 0);
    }
}

// The same copy with a scalar base address and a 32-bit per-lane offset.  base
// and lds must be the same in every lane; they are read from the first active
// lane, which states that to the compiler where it cannot prove it (a value
// carried through a loop of one wave role).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16_sbase(const void* base, uint32_t voff, uint32_t lds) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t ua = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t ul = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(reinterpret_cast<const void*>(ua)), "s"(ul)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Copies NROWS-row tiles of [N, DH] 16-bit matrices into swizzled LDS tiles
// with NWAVES waves, one 1 KiB slice (one direct-to-LDS copy) at a time, so
// that the copies of a tile can be spread over the work of a loop iteration.
// The per-lane byte offsets of the slices are computed once; a full tile then
// needs two vector operations per copy.  Rows at or beyond N (a ragged last
// tile) are clamped to row N - 1.  Callers wait (vmcnt(0)) and synchronise
// before any wave reads the tile.
template <int NROWS, int NWAVES, int DH>
struct TileCopier {
    static constexpr int ROWB = 2 * DH;
    static constexpr int PER_WAVE = NROWS * ROWB / NWAVES;
    static constexpr int SLICES = PER_WAVE / 1024;
    static_assert(PER_WAVE % 1024 == 0, "tile must split into 1 KiB slices per wave");
    uint32_t voff[SLICES];  // byte offset of this lane's 16 bytes within the tile's rows
    uint32_t lds_wave;      // LDS byte offset of this wave's first slice within a tile
    int rowj[SLICES];       // tile row of this lane's 16 bytes, slice j

    __device__ __forceinline__ TileCopier(int wave, int lane) {
        lds_wave = (uint32_t)__builtin_amdgcn_readfirstlane(wave * PER_WAVE);
#pragma unroll
        for (int j = 0; j < SLICES; ++j) {
            const int p = wave * PER_WAVE + j * 1024 + lane * 16;
            const int row = p / ROWB;
            const int chunk = ((p % ROWB) >> 4) ^ swz<ROWB>(row);
            rowj[j] = row;
            voff[j] = (uint32_t)(row * ROWB + chunk * 16);
        }
    }
    // Slice j of rows [r0, r0 + NROWS) of src into the LDS tile at byte
    // lds_tile.  Branch-free, so that a copy can sit anywhere in a stretch of
    // products without splitting it into separate blocks: the base row r0 and
    // the lane's row are both clamped into [0, N), which also turns a tile
    // that starts at or beyond N into a harmless copy of row N - 1.
    __device__ __forceinline__ void copy(int j, const e16_t* src, int r0, int N,
                                         uint32_t lds_tile) const {
        const int rb = r0 < N ? r0 : N - 1;
        const int lim = N - 1 - rb;
        const int row = rowj[j] < lim ? rowj[j] : lim;
        lds_copy16_sbase(src + (long long)rb * DH,
                         (uint32_t)(row * ROWB) + (voff[j] & (ROWB - 1)),
                         lds_tile + lds_wave + j * 1024);
    }
};

// Pins the computation of v to this point of the instruction stream: an empty
// volatile statement that takes v in a register and gives it back.  The
// statement keeps its place among other side-effecting operations (LDS
// accesses, sched_barrier), so the arithmetic that produces v cannot drift
// past it.  sched_barrier alone only constrains the final machine scheduler,
// which sees pure arithmetic where instruction selection has already put it.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }

// LDS byte address of a pointer into a __shared__ array (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(uintptr_t)FA_LDS(const unsigned char, p));
}

// Workgroup id -> work item so that consecutive work items share an XCD
// (workgroups are dealt to the 8 XCDs round-robin by id).
__device__ __forceinline__ int xcd_work_item(int bid, int nwork) {
    return (nwork % 8 == 0) ? (bid % 8) * (nwork / 8) + bid / 8 : bid;
}

// Static schedule of a persistent grid: G workgroups (at most one per CU at a
// time) run n0 work items of one kind and then n1 of another (n1 = 0: one
// kind), each workgroup a fixed list of them, so that one item's start can
// overlap the previous item's end and no workgroup launch sits between them.
// When n0, n1 and G all divide by 8, XCD x (workgroup b runs on XCD b % 8)
// takes the x-th eighth of each kind, its share: n0 / 8 positions of kind 0
// followed by n1 / 8 of kind 1, and the share's P = G / 8 workgroups take its
// positions in snake order -- round m gives slot s = b / 8 position m P + s
// for even m, m P + P - 1 - s for odd m -- so that with items sorted heaviest
// first every workgroup gets about the same work.  Otherwise all items form
// one share over all G workgroups.  Positions grow with the round, so each
// workgroup runs its kind-0 items before its kind-1 items.
struct Schedule {
    int slot, slots;     // this workgroup's slot in its share, workgroups per share
    int share0, share1;  // positions of each kind in a share
    int base0, base1;    // first work item of each kind in this workgroup's share

    __device__ __forceinline__ Schedule(int n0, int n1, int G, int b) {
        const bool xcd = n0 % 8 == 0 && n1 % 8 == 0 && G % 8 == 0;
        const int parts = xcd ? 8 : 1, x = xcd ? b % 8 : 0;
        slot = xcd ? b / 8 : b;
        slots = G / parts;
        share0 = n0 / parts;
        share1 = n1 / parts;
        base0 = x * share0;
        base1 = x * share1;
    }
    __device__ __forceinline__ int pos(int m) const {
        return m * slots + ((m & 1) ? slots - 1 - slot : slot);
    }
    // first round whose position is at least v
    __device__ __forceinline__ int first_round(int v) const {
        const int m = v / slots;
        return pos(m) < v ? m + 1 : m;
    }
};

// The rounds [m0, m1) of one kind in a workgroup's list; round m is work item
// base + pos(m) - lo of that kind.
struct Run {
    int m0, m1, base, lo;
    __device__ __forceinline__ Run(const Schedule& s, int kind) {
        lo = kind ? s.share0 : 0;
        m0 = s.first_round(lo);
        m1 = s.first_round(kind ? s.share0 + s.share1 : s.share0);
        base = kind ? s.base1 : s.base0;
    }
    __device__ __forceinline__ int item(const Schedule& s, int m) const {
        return base + s.pos(m) - lo;
    }
};

// Causal work item -> (head, rank of its block by work, 0 the heaviest), the
// heaviest blocks first.  When each XCD's contiguous share of work items
// holds whole pairs of heads, the two heads of a pair alternate (rank 0 of
// head 2p, of head 2p + 1, then rank 1 of each, ...): with several heads per
// share run one after the other, the last head's heavy blocks would start
// after the others' light ones and leave the share's CUs idle at its end.
__device__ __forceinline__ void heavy_first_work(int work, int nwork, int nb, int& head,
                                                 int& rank) {
    const bool pairs = nwork % 8 == 0 && (nwork / 8) % (2 * nb) == 0;
    if (pairs) {
        const int r = work % (2 * nb);
        head = 2 * (work / (2 * nb)) + (r & 1);
        rank = r >> 1;
    } else {
        head = work / nb;
        rank = work % nb;
    }
}

}  // namespace mf
}  // namespace fa
