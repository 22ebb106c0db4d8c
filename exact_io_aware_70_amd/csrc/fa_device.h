// Device-side building blocks shared by the forward and backward kernels (gfx950 only).
//
// MFMA register layouts used throughout (checked on gfx950 by a lane-layout probe):
//   v_mfma_f32_32x32x16_bf16  A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + i], i = 0..7
//                             B (16 x 32): lane l holds B[8 * (l / 32) + i][l % 32]
//                             C (32 x 32): lane l, register r holds
//                                          C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
//   v_mfma_f32_32x32x2_f32    A: A[l % 32][l / 32], B: B[l / 32][l % 32], C as above.
// Only the pairing of A's and B's k index matters for a contraction, so any consistent
// permutation of k between the two operands is allowed; the kernels use that freedom to
// feed an accumulator straight back in as the next product's operand.
//
// ds_read_b64_tr_b16 (gfx950): inside each group of 16 lanes, lane 4e + q supplies the
// address of four consecutive 16-bit values; lane i of the group receives, as element e,
// value (i % 4) of lane 4e + i / 4.  Pointing lane 4e + q at row r0 + e, column c0 + 4q of
// a row-major tile therefore hands lane i the column c0 + i of rows r0..r0+3: a
// transposed 4 x 16 block in one instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for -infinity as the initial running maximum: exp2 of (it - finite)
// is exactly 0 and (it - it) is 0, so no inf - inf = NaN can arise.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Four 16-bit values, transposed across each 16-lane group (see the header comment).
__device__ __forceinline__ i16x4 lds_read_tr16(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p);
}

__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
    i16x8 t = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, t);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Round eight consecutive accumulator values (starting at `first`) to bf16, RNE.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& acc, int first) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)acc[first + i];
    return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (l ^ 32): the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// v_permlane32_swap on (x, x) leaves the lower-half values in every lane of the first
// result and the upper-half values in every lane of the second, so max / sum of the pair is
// the combination over lanes l and l ^ 32, in all 64 lanes, with one cross-lane instruction.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum of the 16 values of an accumulator tile (a max3 tree: 8 VALU operations).
__device__ __forceinline__ float max16(const f32x16& a) {
    const float m0 = fmaxf(fmaxf(a[0], a[1]), a[2]), m1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
    const float m2 = fmaxf(fmaxf(a[6], a[7]), a[8]), m3 = fmaxf(fmaxf(a[9], a[10]), a[11]);
    const float m4 = fmaxf(fmaxf(a[12], a[13]), a[14]);
    return fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), a[15]));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// acc + sum of the eight bf16 values of v (four v_dot2 against (1, 1), fp32 accumulation).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v[2 * i], v[2 * i + 1]}, one, acc, false);
    return acc;
}

// Buffer resource (raw, stride 0) over `bytes` bytes starting at `base`, as four SGPRs.
// Loads through it return 0 for any byte offset at or past `bytes`, so ragged tails need no
// address clamping.  `base` and `bytes` must be uniform across the wave.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));  // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;  // raw buffer, 32-bit data format
    return r;
}

// LDS byte address of a __shared__ location (wave-uniform for the stage bases used here).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p);
}

// 16 bytes per lane from rsrc + voffset straight into LDS: lane l's data lands at byte
// lds_base + 16 l (M0 holds the wave-uniform base; 64 lanes fill 1 KiB).  Issued as inline
// assembly so the compiler does not add its own conservative wait before every LDS read;
// callers order these loads explicitly with wait_vmcnt() and a workgroup barrier.
__device__ __forceinline__ void load_lds_b128(i32x4 rsrc, uint32_t lds_base, uint32_t voffset) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(rsrc), "{m0}"(lds_base) : "memory");
}

// 4 bytes per lane from rsrc + voffset straight into LDS at lds_base + 4 l (see load_lds_b128).
__device__ __forceinline__ void load_lds_b32(i32x4 rsrc, uint32_t lds_base, uint32_t voffset) {
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voffset), "s"(rsrc), "{m0}"(lds_base) : "memory");
}

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 encoding: vmcnt[3:0] and vmcnt[5:4] at bits 15:14; expcnt and lgkmcnt left at their maxima.
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Scheduling hints: within the current basic block, ask the scheduler for N repetitions of
// {DS reads, one MFMA, VALU ops} so the matrix core and the vector ALU work side by side.
enum : int { kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100 };
template <int N, int DS, int VALU>
__device__ __forceinline__ void interleave_mfma() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (DS > 0) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, DS, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        if (VALU > 0) __builtin_amdgcn_sched_group_barrier(kSchedVALU, VALU, 0);
    }
}

// An empty volatile asm that claims to rewrite the operands: everything computing them must
// happen before this point, and nothing is emitted.
template <int A, int B>
__device__ __forceinline__ void pin_regs(bf16x8 (&v)[A][B]) {
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
        for (int b = 0; b < B; ++b) asm volatile("" : "+v"(v[a][b]));
}

// LDS swizzle: row r of a stage stores its logical 16-byte chunk c at slot c ^ swz_row(r).
// gfx950's LDS has 64 four-byte banks (256 bytes per clock).  A 256-byte row (D = 128)
// covers every bank once, so a row's slot is its 16-byte bank group.
//   * Row reads (128-bit, the K / Q operands): 16 lanes fetch one logical chunk from 16
//     consecutive rows, so swz_row must be a permutation on each aligned block of 16 rows.
//   * Transposed reads (ds_read_b64_tr_b16, the V^T / Q^T / dO^T / K^T operands): half a
//     wave fetches four consecutive chunks (an aligned group 4g..4g+3) from each of four
//     consecutive rows.  XOR keeps each row's four chunks inside one aligned group, number
//     g ^ (swz_row(r) / 4), so the four rows need four different values of swz_row(r) / 4.
//   D = 128: swz_row(r) = 4 (r mod 4) + (r / 4 mod 4) meets both: it is a permutation of
//            0..15, and r mod 4 picks the group.  (The earlier (2r mod 8) | (r/4 mod 2) |
//            (r mod 16 >= 8 ? 8 : 0) met only the first and cost every transposed read a
//            two-way conflict, SQ_LDS_BANK_CONFLICT = 2 cycles per read.)
//   D = 64 (128-byte rows, two per 256 bytes): the same idea on row pairs.
template <int D>
__device__ __forceinline__ int swz_row(int r) {
    if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    const int x = (r >> 1) & 7;
    return 2 * (x & 3) + ((x >> 2) & 1);
}

// Element index of (row, col) inside a swizzled stage (col a multiple of 4).
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
    return row * D + (((col >> 3) ^ swz_row<D>(row)) << 3) + (col & 7);
}

// Map a linear workgroup id to a logical one so that consecutive logical ids land on the
// same XCD (workgroups are dealt to the 8 XCDs round-robin); keeps one head's tiles
// inside one L2.
__device__ __forceinline__ int xcd_remap(int b, int g) {
    return (g % 8 == 0) ? (b % 8) * (g / 8) + b / 8 : b;
}

// Work order over a grid of nheads x ntiles workgroups (logical id L, after xcd_order); rank 0
// is a head's heaviest causal tile.  By default one head at a time, heaviest tile first: the
// workgroups in flight on an XCD then share one head's K/V (or Q/dO) stream in L2.
//   * Head counts that do not divide by 8.  The XCD remap hands each XCD a contiguous eighth
//     of this order, which would end inside a head and give one XCD that head's heaviest
//     tiles and the next its lightest (a 3:1 split of the work at one head per two XCDs).
//     Each head is therefore cut into s = 8 / gcd(nheads, 8) parts of equal causal work, so
//     that every XCD gets whole parts: part j takes, from each run of 2s consecutive ranks,
//     the j-th and the (2s-1-j)-th (a heavy tile paired with a light one).  Ranks still
//     fall through each part heaviest first, and an XCD interleaves its parts by rank.
//   * Few tiles per head.  With fewer than kPairTilesBelow tiles per head, one head at a time
//     can leave the last head's heaviest tiles starting after nearly everything else (a
//     list-scheduling model of 64 slots per XCD loses up to a third at 32 tiles per head and
//     nothing at 64 or 128).  Heads then go in groups of G (head_group: the smallest power of
//     two with G x ntiles >= kPairTilesBelow, at most 8) whose tiles are taken rank-major,
//     the heaviest of all G heads first, which removes the tail.  It costs L2 reuse (pairs at
//     N = 8192 raised the forward's HBM bytes from 1.14x to 1.52x the compulsory ones), so it
//     is kept to the short case.  A last, smaller group takes the heads that remain.
// Both results are uniform and returned through readfirstlane: the integer divisions are
// expanded on the VALU, and left in VGPRs they turned every address derived from the head
// into VALU work inside the loops (and cost the 254-VGPR dK/dV kernel a spill).
constexpr int kPairTilesBelow = 64;
__device__ __forceinline__ int head_group(int ntiles) {
    int g = 1;
    while (g * ntiles < kPairTilesBelow && g < 8) g *= 2;
    return g;
}
__device__ __forceinline__ void tile_order(int L, int ntiles, int nheads, int& head, int& rank) {
    int h, r;
    if (ntiles >= kPairTilesBelow) {
        const int s = 8 / min(nheads & -nheads, 8);  // parts per head
        if (s > 1 && ntiles % (2 * s) == 0) {
            // An XCD's eighth holds P whole parts; it walks them rank-major (the i-th tile of
            // each of its parts, then the (i+1)-th), so the heaviest tiles of all its parts
            // start first instead of those of its last part starting last.
            const int per = ntiles / s, P = nheads * s / 8;
            const int x = L / (P * per), loc = L - x * (P * per);
            const int i = loc / P, part = x * P + (loc - i * P);
            h = part / s;
            const int j = part - h * s;
            r = 2 * s * (i >> 1) + ((i & 1) ? 2 * s - 1 - j : j);
        } else {
            h = L / ntiles;
            r = L - h * ntiles;
        }
    } else {
        const int G = head_group(ntiles);
        const int group = L / (G * ntiles), j = L - group * G * ntiles;
        const int gs = min(G, nheads - group * G);  // heads in this group (the last may be short)
        const int i = j / gs;
        h = group * G + (j - i * gs);
        r = i;
    }
    head = __builtin_amdgcn_readfirstlane(h);
    rank = __builtin_amdgcn_readfirstlane(r);
}

// Logical id of workgroup b in a grid of g = nheads x ntiles: the XCD remap, which gives each
// XCD a contiguous eighth of tile_order's sequence.  Head groups (fewer than kPairTilesBelow
// tiles per head) cannot be cut into equal parts that way, so when an eighth is not a whole
// number of groups the ids stay as dispatched, which deals every head's tiles round-robin
// over the XCDs.
__device__ __forceinline__ int xcd_order(int b, int g, int ntiles) {
    if (ntiles >= kPairTilesBelow) return xcd_remap(b, g);
    return g % (8 * head_group(ntiles) * ntiles) == 0 ? xcd_remap(b, g) : b;
}

}  // namespace fa
