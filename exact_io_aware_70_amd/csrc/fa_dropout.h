// Dropout masks for the attention kernels (gfx950): Philox4x32-10 and the lane exchanges
// that give each lane the mask bytes of the scores it holds.
//
// "How FlashAttention Actually Works" -- "The GPU Memory Wall: HBM vs. SRAM" lists dropout
// among the steps of attention that a fused kernel keeps on chip.  The random numbers are Philox4x32-10
// (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011).
// Mask of head bh: one call with counter (j >> 2, i >> 2, bh, offset) and key (seed lo,
// seed hi) covers the 4 x 4 block of (query i, key j); element (i, j) is byte (j & 3) of
// output word (i & 3), kept iff it is >= t = round(256 p).  Kept probabilities are scaled
// by 256 / (256 - t), the reciprocal of the exact keep probability (the kernels fold that
// into their outputs).
//
// Score layouts (32 x 32 MFMA accumulators, half = lane / 32):
//   query per lane (forward, dQ: S^T):  register r of lane (query, half) is key
//       k0 + 8 (r / 4) + 4 half + r % 4 of a 32-key sub-tile;
//   key per lane (dK/dV: S):            register r of lane (key, half) is query
//       q0 + 8 (r / 4) + 4 half + r % 4 of a 32-query sub-tile.
// In both, registers 4g .. 4g + 3 cover one 4-wide group of the other index, and the four
// lanes 4a .. 4a + 3 of a quad share one 4-wide group of their own index.  So lane u of the
// quad computes the call of the quad's block with the group g = u of the other index, and a
// 4 x 4 transpose across the quad hands every lane its bytes of all four calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"  // DropoutArgs

namespace fa {

// Philox4x32-10 of counter (c0, c1, c2, c3), key (k0, k1).
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// DPP quad permutations: lane d of each quad reads lane perm[d].
__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {  // [1, 0, 3, 2]
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {  // [2, 3, 0, 1]
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}

// 4 x 4 transpose across a quad: on entry lane u holds x[0..3] (row u); on exit it holds
// column u, i.e. x[i] = (entry value x[u] of lane i).  u = lane % 4.
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int u) {
    // 2 x 2 blocks first: swap the off-diagonal element of each block with the neighbour.
    const bool odd = u & 1;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint32_t send = odd ? x[2 * c] : x[2 * c + 1];
        const uint32_t recv = quad_swap1(send);
        if (odd) x[2 * c] = recv; else x[2 * c + 1] = recv;
    }
    // then the off-diagonal blocks between lane pairs (u, u ^ 2).
    const bool hi = u & 2;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const uint32_t send = hi ? x[e] : x[2 + e];
        const uint32_t recv = quad_swap2(send);
        if (hi) x[e] = recv; else x[2 + e] = recv;
    }
}

// Transpose the bytes of four words: out[k] byte i = in[i] byte k.
__device__ __forceinline__ void byte_transpose(uint32_t (&w)[4]) {
    uint32_t t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        t[k] = ((w[0] >> (8 * k)) & 0xFFu) | (((w[1] >> (8 * k)) & 0xFFu) << 8) |
               (((w[2] >> (8 * k)) & 0xFFu) << 16) | (((w[3] >> (8 * k)) & 0xFFu) << 24);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = t[k];
}

// Mask bytes of the scores a lane holds for one 32 x 32 sub-tile: on return byte (r % 4) of
// m[r / 4] is the random byte of the lane's register r.
//   QUERY_PER_LANE: lane (query i, half h), keys k0 .. k0 + 31 (k0 a multiple of 32).
//   otherwise:      lane (key j, half h), queries q0 .. q0 + 31.
// `own` is the lane's own index (query or key), `other0` the sub-tile's first index of the
// other kind.
template <bool QUERY_PER_LANE>
__device__ __forceinline__ void dropout_bytes(const DropoutArgs& d, uint32_t bh, int own, int other0, int lane,
                                              uint32_t (&m)[4]) {
    const int u = lane & 3, half = (lane >> 5) & 1;
    const uint32_t own4 = (uint32_t)own >> 2;                       // the quad's block of its own index
    const uint32_t oth4 = ((uint32_t)other0 >> 2) + 2 * u + half;  // group g = u of the other index
    uint32_t c0 = QUERY_PER_LANE ? oth4 : own4;                    // key block
    uint32_t c1 = QUERY_PER_LANE ? own4 : oth4;                    // query block
    uint32_t c2 = bh, c3 = d.offset;
    philox4x32_10(c0, c1, c2, c3, d.k0, d.k1);
    m[0] = c0;
    m[1] = c1;
    m[2] = c2;
    m[3] = c3;
    // m[w] byte b: query (q4 * 4 + w), key (k4 * 4 + b).
    if (!QUERY_PER_LANE) byte_transpose(m);  // now m[b'] byte w: this lane wants b' = key & 3
    quad_transpose(m, u);                    // m[g] = this lane's 4 bytes of group g
}

// Zero the dropped ones of 8 bf16 probabilities: p holds registers 8c .. 8c + 7 of the
// layout above as 4 dwords of two values (dword e: registers 8c + 2e, 8c + 2e + 1), i.e.
// groups 2c (m_lo) and 2c + 1 (m_hi).
__device__ __forceinline__ void dropout_apply_bf16(uint32_t (&p)[4], uint32_t m_lo, uint32_t m_hi, uint32_t thr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t m = e < 2 ? m_lo : m_hi;
        const int sh = (e & 1) ? 16 : 0;
        const uint32_t b0 = (m >> sh) & 0xFFu, b1 = (m >> (sh + 8)) & 0xFFu;
        const uint32_t keep = (b0 >= thr ? 0x0000FFFFu : 0u) | (b1 >= thr ? 0xFFFF0000u : 0u);
        p[e] &= keep;
    }
}

// Dropout factor of register r (the layout above): the keep scale if kept, else 0.
__device__ __forceinline__ float dropout_factor(const uint32_t (&m)[4], int r, const DropoutArgs& d) {
    const uint32_t b = (m[r >> 2] >> (8 * (r & 3))) & 0xFFu;
    return b >= d.thr ? d.inv_keep : 0.f;
}

}  // namespace fa
