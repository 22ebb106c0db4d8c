// FP8 forward (gfx950): tiled attention with online softmax over OCP E4M3 Q, K, V.
//
// The same method as the bf16 forward ("Breaking the Memory Wall: A Deep Dive into
// FlashAttention" -- "The Solution: IO-Awareness & Tiling", items 1-2; the running max /
// running sum merge of "How does FlashAttention optimize memory and speed via tiling?" --
// "Core Technical Innovations", item 2), with both products on the FP8 matrix cores
// (twice the bf16 rate).  "How does FlashAttention optimize memory and speed via tiling?"
// -- "Interview tips" names FP8 support as a FlashAttention-3 addition; the format and the
// scaling here are this library's: E4M3 codes with one float descale per (batch, head) and
// tensor, logits scale * q_descale * k_descale * (Q8 K8^T), probabilities rounded to E4M3
// for the P V product, O written in bf16.
//
// Layout (d = 128): K and V tiles of 64 keys (128-byte rows) stream through a four-stage
// LDS ring filled by buffer loads that write LDS directly; the 16-byte chunks of row r sit
// at slot chunk ^ f(r), f a bit permutation of (r / 2) mod 8, which keeps both the K row
// reads and the transposed V reads free of bank conflicts.
//
// Operand pairing of v_mfma_f32_32x32x64_f8f6f4 (checked by a lane-layout probe): byte b
// of lane l of A multiplies byte b of lane l' of B when l / 32 = l' / 32, with A row l % 32
// and B column l' % 32; C has the 32 x 32 layout of the bf16 MFMA.  So:
//   S^T = K Q^T:  A lane (key, half h) holds K[key][64 dc + 32 h + b], B lane (query, h)
//                 holds Q[query][64 dc + 32 h + b]: two 32-byte halves of the d range.
//   O^T += V^T P^T:  B lane (query, h) byte b = 16 kb + r is the bf16-style S^T register r
//                 of key block kb, i.e. key kappa(h, b) = 32 kb + 8 (r / 4) + 4 h + r % 4;
//                 A lane (d row, h) byte b holds V[kappa(h, b)][d], gathered by
//                 ds_read_b64_tr_b8 (in each 16-lane group, lane 2e + q names row e and
//                 bytes 8q .. 8q + 7 of an 8 x 16 byte tile; lane i receives column i).
//   Row sums: one more MFMA with an all-ones A gives sum_k P8[k][q] in every row, the sum
//                 of exactly the rounded probabilities the P V product uses.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kRescaleSlackFp8 = 8.0f;  // probabilities stay <= 2^8 = 256 < 448

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    // E4M3 x E4M3 (format 0 for both operands), unit block scales (E8M0 127 = 2^0).
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)p);
}

__device__ __forceinline__ i32x8 load_b256_lds(const uint8_t* p0, const uint8_t* p1) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p0), hi = *reinterpret_cast<const u32x4*>(p1);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Chunk swizzle of 128-byte rows: bits (x1, x0, x2) of x = (r / 2) mod 8.  Per parity of r it
// is a permutation of 0..7 over 16 consecutive rows (K row reads), and its upper two bits
// take four distinct values over the rows {b, b+2, b+8, b+10} each transposed read names.
__device__ __forceinline__ int swz8_row(int r) {
    const int x = (r >> 1) & 7;
    return ((x >> 1) & 1) | ((x & 1) << 1) | (x & 4);
}

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 256), amdgpu_waves_per_eu(2, 2))) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const float* __restrict__ QD, const float* __restrict__ KD, const float* __restrict__ VD,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float scale_log2) {
    constexpr int D = 128, NW = 4, BK = 64, NS = 4, NT = NW * 64;
    constexpr int CH = D / 16;          // 16-byte chunks per row
    constexpr int STAGE = BK * D;       // bytes per tensor per stage
    constexpr int LPT = BK * CH / NT;   // LDS-direct loads per thread per tensor per tile
    constexpr int LPS = 2 * LPT;        // ... for K and V together
    constexpr int BM = 32 * NW;         // query rows per workgroup
    constexpr int DB = D / 32;          // 32-row blocks of O^T
    static_assert(LPT >= 1 && BK * CH % NT == 0, "tile / thread mismatch");

    __shared__ __attribute__((aligned(1024))) uint8_t Ks[NS][STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t Vs[NS][STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;

    const int L = xcd_order(blockIdx.x, gridDim.x, nqt);
    int bh, rank;
    tile_order(L, nqt, gridDim.x / nqt, bh, rank);
    const int qt = nqt - 1 - rank;  // heaviest (causal) tiles first
    const int q0 = qt * BM;
    const size_t base = (size_t)bh * N * D;
    const int wq0 = q0 + wave * 32;
    const int myq = wq0 + l32;
    const float sl2 = scale_log2 * QD[bh] * KD[bh];  // log2-domain logit scale of this head
    const float vd = VD[bh];

    // Q^T fragments (B operand of S^T): bytes 64 dc + 32 half .. + 31 of this lane's query row.
    i32x8 qf[2];
    {
        const int row = min(myq, N - 1);
        const uint8_t* qrow = Q + base + (size_t)row * D;
#pragma unroll
        for (int dc = 0; dc < 2; ++dc) qf[dc] = *reinterpret_cast<const i32x8*>(qrow + 64 * dc + 32 * half);
    }
    wait_vmcnt<0>();

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int nt = (kv_end + BK - 1) / BK;
    const int wave_nt = (wq0 >= N) ? 0 : (CAUSAL ? min(nt, (wq0 + 31) / BK + 1) : nt);

    uint32_t voff[LPT];
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int g = j * NT + tid, r = g / CH, c = (g % CH) ^ swz8_row(r);
        voff[j] = (uint32_t)(r * D + c * 16);
    }
    const uint8_t* Kh = K + base;
    const uint8_t* Vh = V + base;
    auto issue = [&](auto st, int t) {
        constexpr int ST = decltype(st)::value;
        const int kv0 = t * BK;
        const uint32_t bytes = (uint32_t)min(max(0, N - kv0), BK) * D;  // one sub-tile: never wraps
        const i32x4 rk = make_rsrc(Kh + (size_t)min(kv0, N) * D, bytes);
        const i32x4 rv = make_rsrc(Vh + (size_t)min(kv0, N) * D, bytes);
#pragma unroll
        for (int j = 0; j < LPT; ++j) {
            load_lds_b128(rk, lds_addr(&Ks[ST][(j * NT + wave * 64) * 16]), voff[j]);
            load_lds_b128(rv, lds_addr(&Vs[ST][(j * NT + wave * 64) * 16]), voff[j]);
        }
    };

    f32x16 oacc[DB], lacc = f32x16{};
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_ref = kNegBig;

    // K row reads: row 32 kb + l32, chunk 4 dc + 2 half + u (kb = 1 adds 32 rows: the swizzle
    // repeats every 16 rows).
    const uint8_t* k_lane[4];
#pragma unroll
    for (int dc = 0; dc < 2; ++dc)
#pragma unroll
        for (int u = 0; u < 2; ++u)
            k_lane[2 * dc + u] = &Ks[0][l32 * D + (((4 * dc + 2 * half + u) ^ swz8_row(l32)) << 4)];
    // Transposed V reads: in 16-lane group g = lane / 16 (half = g / 2), lane 2e + q names row
    // 16 c + r_l, r_l = 8 (e / 4) + 4 half + e % 4, bytes 32 db + 16 (g % 2) + 8 q .. + 7.
    // Chunk c adds 16 c rows.
    const int tr_e = (lane & 15) >> 1;
    const int tr_r = 8 * (tr_e >> 2) + 4 * half + (tr_e & 3);
    const uint8_t* v_lane[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
        v_lane[db] = &Vs[0][tr_r * D + (((2 * db + ((lane >> 4) & 1)) ^ swz8_row(tr_r)) << 4) + 8 * (lane & 1)];
    // E4M3 1.0 in every byte.  Not const: an empty asm after each use keeps it in its eight
    // registers (otherwise the compiler rebuilds them from one register at every tile).
    i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                  0x38383838, 0x38383838, 0x38383838, 0x38383838};

    // S^T of the tile in stage ST: s[kb] covers keys 32 kb .. 32 kb + 31 (lane = query, register
    // r = key 32 kb + 8(r/4) + 4 half + r%4); the two key blocks are independent chains.
    auto scores = [&](auto st, f32x16 (&s)[2]) {
        constexpr int ST = decltype(st)::value;
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int dc = 0; dc < 2; ++dc)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int off = ST * STAGE + 32 * kb * D;
                s[kb] = mfma_fp8(load_b256_lds(k_lane[2 * dc] + off, k_lane[2 * dc + 1] + off), qf[dc], s[kb]);
            }
    };
    auto mask = [&](int t, f32x16 (&s)[2]) {
        const int kv0 = t * BK;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
                if (CAUSAL ? (key > myq) : (key >= N)) s[kb][r] = -INFINITY;
            }
    };
    auto needs_mask = [&](int t) { return CAUSAL ? (t * BK + BK - 1 > wq0) : (t * BK + BK > N); };
    auto raise_ref = [&](f32x16 (&s)[2]) {
        const float mt = max_halves(fmaxf(max16(s[0]), max16(s[1]))) * sl2;
        if (__any(mt > m_ref + kRescaleSlackFp8)) {
            const float mn = fmaxf(m_ref, mt);
            const float alpha = fast_exp2(m_ref - mn);
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            lacc *= alpha;
            m_ref = mn;
        }
    };
    // P(t) = 2^(S * scale - m_ref) rounded to E4M3, packed in S^T register order (byte 16 kb + r).
    auto probs = [&](f32x16 (&s)[2], i32x8& pb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(fmaf(s[kb][r], sl2, -m_ref));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int w = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][4 * j], s[kb][4 * j + 1], pb[4 * kb + j], false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(s[kb][4 * j + 2], s[kb][4 * j + 3], w, true);
                pb[4 * kb + j] = w;
            }
        }
    };
    // O^T += V^T P^T for the tile in stage ST, and the row sums of P through the all-ones A.
    auto pv = [&](auto st, const i32x8& pb) {
        constexpr int ST = decltype(st)::value;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint8_t* p = v_lane[db] + ST * STAGE;
            const i32x2 a0 = lds_read_tr8(p), a1 = lds_read_tr8(p + 16 * D), a2 = lds_read_tr8(p + 32 * D),
                        a3 = lds_read_tr8(p + 48 * D);
            const i32x8 a = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
            oacc[db] = mfma_fp8(a, pb, oacc[db]);
        }
        lacc = mfma_fp8(ones, pb, lacc);
        asm volatile("" : "+v"(ones));
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    static_assert(NS == 4, "the loop below is unrolled over four stages");

    issue(S0{}, 0);
    issue(S1{}, 1);
    issue(S2{}, 2);
    wait_vmcnt<(NS - 2) * LPS>();
    __syncthreads();

    f32x16 sa[2], sb[2];
    if (wave_nt > 0) {
        scores(S0{}, sa);
        if (needs_mask(0)) mask(0, sa);
        raise_ref(sa);
    }

    // P of the current tile, carried across steps: each word's first conversion names the
    // register it overwrites as the preserved half (both halves are rewritten), so no
    // zeroing instruction precedes it.
    i32x8 pb = {};
    // One pipeline step on tile i (stage CUR = i % NS): `cur` holds S(i) (masked, reference
    // raised); leaves S(i+1) in `nxt`.  Every wave runs every step (barriers and loads are
    // collective); the arithmetic stops after the wave's own last tile.  On that last tile
    // S(i+1) is still computed, but every key of it lies past the wave's rows or past N, so
    // the mask clears it and it raises nothing.
    auto step = [&](auto cur_st, int i, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        constexpr int CUR = decltype(cur_st)::value;
        wait_vmcnt<(NS - 3) * LPS>();  // tile i + 1 has landed (this wave's share)
        __syncthreads();               // ... and every wave's; stage (i - 1) % NS is free
        issue(std::integral_constant<int, (CUR + NS - 1) % NS>{}, i + NS - 1);
        if (i >= wave_nt) return;
        probs(cur, pb);
        scores(std::integral_constant<int, (CUR + 1) % NS>{}, nxt);
        // The compiler's MFMA / exponential interleaving (iglp_opt 3) places this region's
        // exponentials, FMAs and conversions among the four S products 2-3% better than fixed
        // {MFMA, 16 VALU} groups.
        __builtin_amdgcn_iglp_opt(3);
        asm volatile("" : "+v"(pb));  // keep the exponentials next to the S products
        if (needs_mask(i + 1)) mask(i + 1, nxt);
        pv(cur_st, pb);
        raise_ref(nxt);
    };
    int i = 0;
    for (; i + 3 < nt; i += 4) {
        step(S0{}, i, sa, sb);
        step(S1{}, i + 1, sb, sa);
        step(S2{}, i + 2, sa, sb);
        step(S3{}, i + 3, sb, sa);
    }
    if (i < nt) step(S0{}, i, sa, sb);
    if (i + 1 < nt) step(S1{}, i + 1, sb, sa);
    if (i + 2 < nt) step(S2{}, i + 2, sa, sb);
    wait_vmcnt<0>();  // no LDS-direct load may still be writing when the workgroup's LDS is freed

    // Epilogue: every row of the ones block holds this query's sum of P8.
    if (myq < N) {
        const float l = lacc[0];
        const float inv = vd / l;
        __bf16* orow = O + base + (size_t)myq * D;  // O [B,H,N,d] bf16: same element index as the codes
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                __bf16 w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[db][4 * g + e] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * half) = __builtin_bit_cast(u32x2, w);
            }
        if (half == 0) LSE[(size_t)bh * N + myq] = m_ref * kLn2 + __logf(l);
    }
}

template <bool CAUSAL>
hipError_t launch_fp8(const Fp8FwdArgs& a, hipStream_t st) {
    const int nqt = (a.N + 127) / 128;
    const long long grid = (long long)nqt * a.B * a.H;
    hipLaunchKernelGGL((fwd_fp8_kernel<CAUSAL>), dim3((unsigned)grid), dim3(256), 0, st,
                       static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                       static_cast<const uint8_t*>(a.v), a.q_descale, a.k_descale, a.v_descale,
                       static_cast<__bf16*>(a.o), a.lse, a.N, nqt, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t st) {
    return a.causal ? launch_fp8<true>(a, st) : launch_fp8<false>(a, st);
}

}  // namespace fa
