// Forward kernels: tiled attention with online softmax (gfx950).
//
// "Breaking the Memory Wall: A Deep Dive into FlashAttention" -- "The Solution:
// IO-Awareness & Tiling": Q, K, V are cut into blocks that fit on chip, a running
// maximum and running sum are kept per query row, earlier partial results are rescaled
// when the maximum grows, and only the final O (plus the per-row normaliser, here the
// logsumexp) is written back.  "How does FlashAttention optimize memory and speed via
// tiling?" -- "Core Technical Innovations", item 2, gives the merge
//     m2 = max(m1, m~),  l2 = e^{m1 - m2} l1 + e^{m~ - m2} l~.
//
// Work split (differs from the pages' K/V-outer loop): each workgroup owns one query
// tile and walks the K/V tiles of its head, so the output accumulators, m and l never
// leave registers.  Each wave owns 32 query rows.  The score tile is computed transposed,
// S^T = K Q^T, so a lane holds 32 scores of ONE query row: the row maximum and row sum
// are in-lane except for one exchange between the two wave halves, and the accumulator
// of S^T is directly the B operand of O^T += V^T P^T.
#include <type_traits>

#include "fa_device.h"
#include "fa_dropout.h"
#include "fa_internal.h"

namespace fa {
namespace {

// Lazy rescaling: the reference maximum m_ref of a row is raised only when a tile's
// maximum exceeds it by more than kRescaleSlack (log2 units), so exponentials stay
// below 2^kRescaleSlack.  The result is the same sum written relative to a different
// reference point (exact in real arithmetic), and most tiles skip the O rescale.
constexpr float kRescaleSlack = 8.0f;

// ------------------------------------------------------------------ bf16, MFMA 32x32x16
// Workgroup: NW waves, each owning QB blocks of 32 query rows (every K/V operand read from
// LDS feeds QB MFMAs).  K/V stream in sub-tiles of 32 keys through an NS-stage
// LDS ring filled by buffer loads that write LDS directly (no register staging).  Rows of
// a stage are stored with their 16-byte chunks XOR-swizzled by swz_row(row) (fa_device.h),
// which keeps both the row-wise K reads and the transposed V reads free of bank conflicts.
//
// Key groups (NG = 2, chosen for grids that do not fill the machine): the workgroup has two
// groups of NW waves over the same query rows; group g walks the sub-tiles 2i + g through a
// ring of its own, and the groups' partial (m, l, O) merge at the end.  The heaviest causal
// tiles, whose walk sets the time of a small grid, then take half as long.
//
// Software pipeline per sub-tile i (one barrier each):
//   exponentials of S(i) on the VALU  ||  S(i+1) = K(i+1) Q^T on the MFMA
//   O^T += V(i)^T P(i)^T on the MFMA   ||  row sums of P(i), row max of S(i+1)
template <int D>
struct FwdTile {
    static constexpr int BK = 32;          // keys per sub-tile
    static constexpr int NS = 4;           // LDS stages
    static constexpr int CPR = D / 8;      // 16-byte chunks per row
    static constexpr int STAGE = BK * D;   // bf16 elements per tensor per stage
};

// Two waves per SIMD at d = 128: the register budget stays within 256 VGPRs, so every MFMA
// keeps its accumulator in ordinary VGPRs and the softmax reads the scores in place.  At
// d = 64 the kernel needs under 128 VGPRs and a 32 KiB ring, so four waves per SIMD (three
// with dropout, whose mask needs more registers) hide more latency.
// DROP: dropout of the probabilities in the P V product (the row sums, hence lse, stay
// undropped; the keep scale is folded into the epilogue).
template <int D, bool DROP>
struct FwdWaves : std::integral_constant<int, D == 64 ? (DROP ? 3 : 4) : 2> {};

template <int D, int NW, int QB, bool CAUSAL, bool DROP, int NG>
__global__ __attribute__((amdgpu_flat_work_group_size(1, NG * NW * 64),
                               amdgpu_waves_per_eu(FwdWaves<D, DROP>::value, FwdWaves<D, DROP>::value))) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float scale_log2, DropoutArgs drop) {
    using T = FwdTile<D>;
    constexpr int BK = T::BK, NS = T::NS, CPR = T::CPR, STAGE = T::STAGE;
    constexpr int RW = 32 * QB;         // query rows per wave
    constexpr int BM = RW * NW;         // query rows per workgroup
    constexpr int NT = NG * NW * 64;    // threads
    constexpr int DC = D / 16;          // k-steps of the S^T product
    constexpr int DB = D / 32;          // 32-row blocks of O^T
    constexpr int LPT = BK * CPR / NT;  // LDS-direct loads per thread per tensor per sub-tile
    constexpr int LPS = 2 * NG * LPT;   // ... for K and V of every group's sub-tile
    static_assert(LPT >= 1 && BK * CPR % NT == 0, "tile / thread mismatch");
    static_assert(NS >= 3 && (NS - 2) * LPS < 64, "pipeline depth");

    static_assert(NG == 1 || NG == 2, "one or two key groups");
    __shared__ __attribute__((aligned(1024))) __bf16 Ks[NG][NS][STAGE];
    __shared__ __attribute__((aligned(1024))) __bf16 Vs[NG][NS][STAGE];

    // The wave index is uniform across the wave; readfirstlane lets the compiler see that, so
    // every per-wave decision below is a scalar branch rather than an exec-masked one.
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    // Key groups: with NG = 2 the waves come in two groups of NW that own the same query rows;
    // group g takes the sub-tiles t = 2i + g, and the two partial results merge at the end.
    const int grp = NG == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave / NW);
    const int wr = NG == 1 ? wave : wave - grp * NW;  // row block of this wave

    const int L = xcd_order(blockIdx.x, gridDim.x, nqt);
    int bh, rank;
    tile_order(L, nqt, gridDim.x / nqt, bh, rank);
    const int qt = nqt - 1 - rank;  // heaviest (causal) tiles first
    const int q0 = qt * BM;
    const size_t base = (size_t)bh * N * D;
    const int wq0 = q0 + wr * RW;        // first query row of this wave

    // Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop.  Rows past N
    // read row N - 1: finite values whose results are never stored.
    bf16x8 qf[QB][DC];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = min(wq0 + 32 * qb + l32, N - 1);
#pragma unroll
        for (int kc = 0; kc < DC; ++kc) qf[qb][kc] = load_bf16x8(Q + base + (size_t)row * D + 16 * kc + 8 * half);
    }
    // Retire the Q loads before the K/V pipeline starts, so every later vmcnt wait counts
    // only the K/V stage loads.
    wait_vmcnt<0>();

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int nt = (kv_end + BK - 1) / BK;
    const int nsteps = (nt + NG - 1) / NG;  // steps of the workgroup; step i takes sub-tile NG i + g
    // Steps this wave computes: causal waves stop at their own last row.
    const int wave_last = (wq0 >= N) ? -1 : (CAUSAL ? min(nt, (wq0 + RW - 1) / BK + 1) : nt) - 1;
    const int wave_nt = wave_last < grp ? 0 : (wave_last - grp) / NG + 1;

    // Per-thread byte offsets of the LDS-direct loads inside one sub-tile (fixed across tiles):
    // LDS chunk g = j * NT + tid holds row g / CPR, logical chunk (g % CPR) ^ swz_row(row).
    uint32_t voff[LPT];
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int g = j * NT + tid, r = g / CPR, c = (g % CPR) ^ swz_row<D>(r);
        voff[j] = (uint32_t)((r * D + c * 8) * 2);
    }
    const __bf16* Kh = K + base;
    const __bf16* Vh = V + base;
    // Enqueue step i's sub-tiles (NG i + g for each group g) into stage ST = i % NS of the
    // groups' rings.  Sub-tiles at or past N read zeros.
    auto issue = [&](auto st, int i) {
        constexpr int ST = decltype(st)::value;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int kv0 = (NG * i + g) * BK;
            // Each resource spans only its own sub-tile (at most BK rows), so the 32-bit byte
            // count cannot wrap however long the sequence is.
            const uint32_t bytes = (uint32_t)min(max(0, N - kv0), BK) * D * 2;
            const i32x4 rk = make_rsrc(Kh + (size_t)min(kv0, N) * D, bytes);
            const i32x4 rv = make_rsrc(Vh + (size_t)min(kv0, N) * D, bytes);
#pragma unroll
            for (int j = 0; j < LPT; ++j) {
                load_lds_b128(rk, lds_addr(&Ks[g][ST][(j * NT + wave * 64) * 8]), voff[j]);
                load_lds_b128(rv, lds_addr(&Vs[g][ST][(j * NT + wave * 64) * 8]), voff[j]);
            }
        }
    };

    f32x16 oacc[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[qb][db] = f32x16{};
    float m_ref[QB], lsum[QB];  // log2-domain reference max; this lane's share of the row sum
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_ref[qb] = kNegBig;
        lsum[qb] = 0.f;
    }

    // LDS read addresses that depend only on the lane (stages and k-steps add immediates).
    // K rows for the A operand of S^T: row l32, chunk 2kc + half (swizzled).
    const __bf16* k_lane[DC];
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) k_lane[kc] = &Ks[grp][0][swz<D>(l32, 16 * kc + 8 * half)];
    // Transposed V reads: rows tr_row and tr_row + 8 (16 cc adds whole rows: the swizzle
    // repeats every 16 rows), column 32 db + tr_col.
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const __bf16* v_lane[2][DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        v_lane[0][db] = &Vs[grp][0][swz<D>(tr_row, 32 * db + tr_col)];
        v_lane[1][db] = &Vs[grp][0][swz<D>(tr_row + 8, 32 * db + tr_col)];
    }

    // S^T of the sub-tile in stage ST for both query blocks: lane = query, register r =
    // key 8(r/4) + 4 half + r%4.
    auto scores = [&](auto st, f32x16 (&s)[QB]) {
        constexpr int ST = decltype(st)::value;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < DC; ++kc) {
            const bf16x8 a = load_bf16x8(k_lane[kc] + ST * STAGE);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb] = mfma_bf16(a, qf[qb][kc], s[qb]);
        }
    };
    // Causal (key > query) or tail (key >= N) mask; only sub-tiles that need it call this.
    auto mask = [&](int i, f32x16 (&s)[QB]) {
        const int kv0 = (NG * i + grp) * BK;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int myq = wq0 + 32 * qb + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kv0 + 8 * (r / 4) + 4 * half + (r % 4);
                if (CAUSAL ? (key > myq) : (key >= N)) s[qb][r] = -INFINITY;
            }
        }
    };
    auto needs_mask = [&](int i) {
        const int kv0 = (NG * i + grp) * BK;
        return CAUSAL ? (kv0 + BK - 1 > wq0) : (kv0 + BK > N);
    };
    static_assert(BK % 32 == 0, "a sub-tile past the wave's rows must be fully masked");
    static_assert(BK % 16 == 0, "stage bases must keep the 16-row swizzle period");
    // Row max of S(t) and the (rare) raise of the reference max: O and l are rescaled by
    // 2^(m_old - m_new) only when some row's max exceeds its reference by more than the slack.
    auto raise_ref = [&](f32x16 (&s)[QB]) {
        float mt[QB];
        bool up = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            mt[qb] = max_halves(max16(s[qb])) * scale_log2;
            up |= mt[qb] > m_ref[qb] + kRescaleSlack;
        }
        if (__any(up)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mn = fmaxf(m_ref[qb], mt[qb]);
                const float alpha = fast_exp2(m_ref[qb] - mn);
                lsum[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[qb][db] *= alpha;
                m_ref[qb] = mn;
            }
        }
    };
    // P(t) = 2^(S * scale * log2 e - m_ref), rounded to bf16 B operands (P^T, keys as in S^T).
    auto probs = [&](f32x16 (&s)[QB], bf16x8 (&pb)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[qb][r] = fast_exp2(fmaf(s[qb][r], scale_log2, -m_ref[qb]));
            pb[qb][0] = to_bf16x8(s[qb], 0);
            pb[qb][1] = to_bf16x8(s[qb], 8);
        }
    };
    // Row sums of the bf16-rounded P(t) (the values the P V product uses), two per v_dot2.
    auto rowsum = [&](const bf16x8 (&pb)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) lsum[qb] = sum_bf16x8(pb[qb][1], sum_bf16x8(pb[qb][0], lsum[qb]));
    };
    // O^T += V^T P^T for the sub-tile in stage ST: for k-step cc the B operand holds keys
    // 16cc + 8(i/4) + 4 half + i%4, and the two transposed reads fetch V^T at exactly those
    // keys (rows 16cc + tr_row and 16cc + tr_row + 8).
    auto pv = [&](auto st, const bf16x8 (&pb)[QB][2]) {
        constexpr int ST = decltype(st)::value;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int off = ST * STAGE + 16 * cc * D;
                const bf16x8 a = join_tr(lds_read_tr16(v_lane[0][db] + off), lds_read_tr16(v_lane[1][db] + off));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma_bf16(a, pb[qb][cc], oacc[qb][db]);
            }
        }
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    static_assert(NS == 4, "the loop below is unrolled over four stages");

    // Prologue: NS - 1 sub-tiles in flight, then S(0).
    issue(S0{}, 0);
    issue(S1{}, 1);
    issue(S2{}, 2);
    wait_vmcnt<(NS - 2) * LPS>();
    __syncthreads();

    f32x16 sa[QB], sb[QB];
    if (wave_nt > 0) {
        scores(S0{}, sa);
        if (needs_mask(0)) mask(0, sa);
        raise_ref(sa);
    }

    // One pipeline step on sub-tile i (stage CUR = i % NS): `cur` holds S(i) (masked,
    // reference raised); leaves S(i+1) in `nxt`.  Every wave runs every step (barriers and
    // loads are collective); the arithmetic is skipped past the wave's own last sub-tile.
    // On that last sub-tile S(i+1) is still computed (its stage holds loaded data or zeros)
    // but every key of it lies past the wave's rows or past N, so the mask clears it and
    // it raises nothing.
    // Region 1: the exponentials of S(i) overlap the MFMAs of S(i+1).  Region 2: the row
    // sums of P(i) and the max of S(i+1) overlap the MFMAs of O += P(i) V(i).
    auto step = [&](auto cur_st, int i, f32x16 (&cur)[QB], f32x16 (&nxt)[QB]) {
        constexpr int CUR = decltype(cur_st)::value;
        wait_vmcnt<(NS - 3) * LPS>();  // sub-tile i + 1 has landed (this wave's share)
        __syncthreads();               // ... and every wave's; stage (i - 1) % NS is free
        issue(std::integral_constant<int, (CUR + NS - 1) % NS>{}, i + NS - 1);
        if (i >= wave_nt) return;
        bf16x8 pb[QB][2];
        probs(cur, pb);
        scores(std::integral_constant<int, (CUR + 1) % NS>{}, nxt);
        // At d = 64 (half the MFMAs per exponential, four waves per SIMD) the compiler's own
        // MFMA / exponential interleaving (iglp_opt 2) is 1-2% faster than fixed groups; at
        // d = 128 every strategy was equal or slower than the {MFMA, 6 VALU} groups.
        if constexpr (D == 64 && !DROP) __builtin_amdgcn_iglp_opt(2);
        else interleave_mfma<DC * QB, 0, 6>();
        pin_regs(pb);  // keep the exponentials in region 1 (they would sink to their use)
        if (needs_mask(i + 1)) mask(i + 1, nxt);
        if constexpr (DROP) {
            bf16x8 pd[QB][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                uint32_t m[4];
                dropout_bytes<true>(drop, (uint32_t)bh, wq0 + 32 * qb + l32, (NG * i + grp) * BK, lane, m);
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    u32x4 w4 = __builtin_bit_cast(u32x4, pb[qb][cc]);
                    uint32_t w[4] = {w4[0], w4[1], w4[2], w4[3]};
                    dropout_apply_bf16(w, m[2 * cc], m[2 * cc + 1], drop.thr);
                    pd[qb][cc] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
                }
            }
            pv(cur_st, pd);
        } else {
            pv(cur_st, pb);
        }
        rowsum(pb);
        raise_ref(nxt);
    };
    int i = 0;
    for (; i + 3 < nsteps; i += 4) {
        step(S0{}, i, sa, sb);
        step(S1{}, i + 1, sb, sa);
        step(S2{}, i + 2, sa, sb);
        step(S3{}, i + 3, sb, sa);
    }
    if (i < nsteps) step(S0{}, i, sa, sb);
    if (i + 1 < nsteps) step(S1{}, i + 1, sb, sa);
    if (i + 2 < nsteps) step(S2{}, i + 2, sa, sb);
    wait_vmcnt<0>();  // no LDS-direct load may still be writing when the workgroup's LDS is freed

    if constexpr (NG == 2) {
        // Merge the two groups' partial results of each row ("How does FlashAttention optimize
        // memory and speed via tiling?", Core Technical Innovations, item 2): with m = max(m0, m1),
        // O = 2^(m0 - m) O0 + 2^(m1 - m) O1 and l likewise.  Group 1 hands its (m, l, O) over
        // through the LDS of the finished rings, laid out [row block][value][lane].
        constexpr int NV = QB * DB * 16 + 2 * QB;  // values per lane
        static_assert(NW * NV * 64 * 4 <= (int)(sizeof(Ks) + sizeof(Vs)), "merge buffer");
        float* xs = reinterpret_cast<float*>(&Ks[0][0][0]) + wr * NV * 64 + lane;
        __syncthreads();  // every wave is done with the rings
        if (grp == 1) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) xs[((qb * DB + db) * 16 + r) * 64] = oacc[qb][db][r];
                xs[(QB * DB * 16 + qb) * 64] = m_ref[qb];
                xs[(QB * DB * 16 + QB + qb) * 64] = lsum[qb];
            }
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float m1 = xs[(QB * DB * 16 + qb) * 64], l1 = xs[(QB * DB * 16 + QB + qb) * 64];
            const float mn = fmaxf(m_ref[qb], m1);
            const float a0 = fast_exp2(m_ref[qb] - mn), a1 = fast_exp2(m1 - mn);
            lsum[qb] = lsum[qb] * a0 + l1 * a1;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    oacc[qb][db][r] = oacc[qb][db][r] * a0 + xs[((qb * DB + db) * 16 + r) * 64] * a1;
            m_ref[qb] = mn;
        }
    }

    // Epilogue: O = acc / l, lse = m_ref ln 2 + ln l.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = sum_halves(lsum[qb]);
        const int myq = wq0 + 32 * qb + l32;
        if (myq < N) {
            const float inv = (DROP ? drop.inv_keep : 1.0f) / l;
            __bf16* orow = O + base + (size_t)myq * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    __bf16 w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[qb][db][4 * g + e] * inv);
                    *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * half) = __builtin_bit_cast(u32x2, w);
                }
            if (half == 0) LSE[(size_t)bh * N + myq] = m_ref[qb] * kLn2 + __logf(l);
        }
    }
}

// ------------------------------------------------------------------ fp32, MFMA 32x32x2
// Same structure with fp32 operands throughout (no reduced precision anywhere).  Single
// LDS buffer; this path serves the small fp32 workloads.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float scale_log2) {
    constexpr int NW = 4, BM = 32 * NW, BN = 64, NT = 256;
    constexpr int KST = D + 1;  // odd stride: column reads across rows hit distinct banks
    constexpr int VST = D + 8;
    constexpr int DB = D / 32;
    __shared__ float Ks[BN * KST];
    __shared__ float Vs[BN * VST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int L = xcd_order(blockIdx.x, gridDim.x, nqt);
    int bh, rank;
    tile_order(L, nqt, gridDim.x / nqt, bh, rank);
    const int q0 = (nqt - 1 - rank) * BM;
    const size_t base = (size_t)bh * N * D;
    const int wq0 = q0 + wave * 32, myq = wq0 + l32;

    float qf[D / 2];
#pragma unroll
    for (int kc = 0; kc < D / 2; ++kc) qf[kc] = (myq < N) ? Q[base + (size_t)myq * D + 2 * kc + half] : 0.f;

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int nt = (kv_end + BN - 1) / BN;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_ref = kNegBig, lsum = 0.f;

    for (int t = 0; t < nt; ++t) {
        const int kv0 = t * BN;
        __syncthreads();
        for (int c = tid; c < BN * D; c += NT) {
            const int r = c / D, col = c % D;
            const bool ok = kv0 + r < N;
            Ks[r * KST + col] = ok ? K[base + (size_t)(kv0 + r) * D + col] : 0.f;
            Vs[r * VST + col] = ok ? V[base + (size_t)(kv0 + r) * D + col] : 0.f;
        }
        __syncthreads();
        const bool active = (wq0 < N) && (!CAUSAL || kv0 <= wq0 + 31);
        if (!active) continue;

        f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kc = 0; kc < D / 2; ++kc)
                s[kb] = mfma_f32(Ks[(32 * kb + l32) * KST + 2 * kc + half], qf[kc], s[kb]);

        const bool need_mask = CAUSAL ? (kv0 + BN - 1 > wq0) : (kv0 + BN > N);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
                    if (CAUSAL ? (key > myq) : (key >= N)) s[kb][r] = -INFINITY;
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = fmaxf(mx, swap_halves(mx));
        const float mt = mx * scale_log2;
        if (__any(mt > m_ref + kRescaleSlack)) {
            const float mn = fmaxf(m_ref, mt);
            const float alpha = fast_exp2(m_ref - mn);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m_ref = mn;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(fmaf(s[kb][r], scale_log2, -m_ref));
                s[kb][r] = p;
                lsum += p;
            }
        // O^T += V^T P^T, one MFMA per accumulator register: lane l's register r is
        // the probability of key 32kb + 8(r/4) + 4(l/32) + r%4, read row-wise from V.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int krow = 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    oacc[db] = mfma_f32(Vs[krow * VST + 32 * db + l32], s[kb][r], oacc[db]);
            }
    }

    lsum += swap_halves(lsum);
    if (myq < N) {
        const float inv = 1.0f / lsum;
        float* orow = O + base + (size_t)myq * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = oacc[db][4 * g + i] * inv;
                *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * half) = w;
            }
        if (half == 0) LSE[(size_t)bh * N + myq] = m_ref * kLn2 + logf(lsum);
    }
}

template <int D, int NW, int QB, bool CAUSAL, int NG>
hipError_t launch_bf16(const FwdArgs& a, hipStream_t st) {
    constexpr int BM = 32 * QB * NW;
    const int nqt = (a.N + BM - 1) / BM;
    const long long grid = (long long)nqt * a.B * a.H;
    if (a.dropout)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, QB, CAUSAL, true, NG>), dim3((unsigned)grid), dim3(NG * NW * 64), 0, st,
                           (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse,
                           a.N, nqt, a.scale * kLog2e, a.drop);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, QB, CAUSAL, false, NG>), dim3((unsigned)grid), dim3(NG * NW * 64), 0, st,
                           (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse,
                           a.N, nqt, a.scale * kLog2e, a.drop);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdArgs& a, hipStream_t st) {
    const int nqt = (a.N + 127) / 128;
    const long long grid = (long long)nqt * a.B * a.H;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(256), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                       a.N, nqt, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
    if (a.dtype == kBF16) {
        if (a.d == 128) {
            // Grids that do not fill the machine twice over: each tile's keys split over two
            // groups of waves, which halves the walk of the heaviest causal tiles.
            const long long tiles = (long long)((a.N + 127) / 128) * a.B * a.H;
            if (tiles <= kSplitTilesAtMost)
                return a.causal ? launch_bf16<128, 4, 1, true, 2>(a, st) : launch_bf16<128, 4, 1, false, 2>(a, st);
            return a.causal ? launch_bf16<128, 4, 1, true, 1>(a, st) : launch_bf16<128, 4, 1, false, 1>(a, st);
        }
        return a.causal ? launch_bf16<64, 4, 1, true, 1>(a, st) : launch_bf16<64, 4, 1, false, 1>(a, st);
    }
    if (a.d == 128) return a.causal ? launch_f32<128, true>(a, st) : launch_f32<128, false>(a, st);
    return a.causal ? launch_f32<64, true>(a, st) : launch_f32<64, false>(a, st);
}

long long fwd_grid_tiles(int N, int dtype) {
    (void)dtype;
    return (N + 127) / 128;  // both paths use 128 query rows per workgroup
}

}  // namespace fa
