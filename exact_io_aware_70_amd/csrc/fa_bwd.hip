// Backward kernels: gradients by recomputation (gfx950).
//
// "How FlashAttention Actually Works" -- "The Backward Pass: Recomputation" and "Breaking
// the Memory Wall: A Deep Dive into FlashAttention" -- "3. Backward Pass Recomputation":
// the probability matrix is never stored; each score tile is rebuilt on chip from Q, K and
// the per-row normaliser kept by the forward pass (here lse), then used at once.
//
// For the loss L = sum(O * dO), with P = exp(scale Q K^T - lse) (the softmax Jacobian
// written out; the pages give no formulas):
//     dV = P^T dO,  dP = dO V^T,  D_i = rowsum(dO * O)_i,  dS = P * (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q.
//
// Two launches on one stream, no atomics (run-to-run bitwise deterministic):
//   1. dQ:     one workgroup per query tile, each wave holding 32 queries, walking the key
//              tiles (recomputes S and dP a second time instead of accumulating dQ with
//              atomics).  Its prologue computes D_i = rowsum(dO * O) of its own rows from the
//              dO fragments it loads anyway, and stores D and lse * log2(e) into the caller's
//              workspace;
//   2. dK/dV:  one workgroup per key tile, each wave holding 32 keys (K, V fragments and
//              the dK^T, dV^T accumulators in registers), walking the query tiles with the
//              D and lse * log2(e) of every query row from the workspace.
#include <type_traits>

#include "fa_device.h"
#include "fa_dropout.h"
#include "fa_internal.h"

namespace fa {
namespace {

// ------------------------------------------------------------------ bf16 dK / dV
// Workgroup: NW waves, each holding 32 keys (K^T and V^T fragments as MFMA B operands and
// the dK^T, dV^T accumulators in registers).  Query sub-tiles of 32 rows (Q, dO, lse, D)
// stream through an NS-stage LDS ring filled by loads that write LDS directly; Q and dO
// rows are XOR-swizzled exactly like the forward's K/V stages, so the row reads (A operands
// of S and dP) and the transposed reads (dO^T, Q^T for dV and dK) are conflict-free.
// S = Q K^T and dP = dO V^T come out with lane = key, register = query, so P and dS feed
// the B operands of dV^T += dO^T P and dK^T += Q^T dS without any shuffle.
// Query rows past N load as zeros with lse = D = 0: their P is 1 but multiplies zero dO
// rows, and their dS = P (0 - 0) = 0, so they contribute nothing.
// DROP: dropout (dV takes the dropped P; dS = P (Z dP - D) with Z the keep factor; the
// keep scale of dV is applied at the store).
// NG = 2 (grids of at most kSplitTilesAtMost key tiles): two groups of NW waves per key tile
// take alternate query sub-tiles through rings of their own, so the heaviest key tiles' walk
// halves; group 1's dK, dV partials join group 0's through the LDS at the end.
// Occupancy: two waves per SIMD at d = 128 (254 of 256 VGPRs); three at d = 64 without
// dropout, where the kernel fits the 168-VGPR budget without spilling.
template <int D, bool DROP>
struct DkdvWaves : std::integral_constant<int, D == 64 && !DROP ? 3 : 2> {};

template <int D, int NW, bool CAUSAL, bool DROP, int NG>
__global__ __attribute__((amdgpu_flat_work_group_size(1, NG * NW * 64),
                               amdgpu_waves_per_eu(DkdvWaves<D, DROP>::value, DkdvWaves<D, DROP>::value))) void dkdv_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Delta,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int N, int nkt, float scale, float scale_log2,
    DropoutArgs drop) {
    constexpr int BQ = 32;              // query rows per sub-tile
    constexpr int NS = 4;               // LDS stages
    constexpr int STAGE = BQ * D;       // bf16 elements per tensor per stage
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int NT = NG * NW * 64;
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int LPT = BQ * CPR / NT;  // LDS-direct 16-byte loads per thread per tensor per sub-tile
    constexpr int LPS = NG * (2 * LPT + 2);  // per step and group: Q, dO, then lse and D (4 bytes per lane)
    static_assert(LPT >= 1 && BQ * CPR % NT == 0, "tile / thread mismatch");
    static_assert((NS - 2) * LPS < 64, "pipeline depth");

    static_assert(NG == 1 || NG == 2, "one or two query groups");
    __shared__ __attribute__((aligned(1024))) __bf16 Qs[NG][NS][STAGE];
    __shared__ __attribute__((aligned(1024))) __bf16 dOs[NG][NS][STAGE];
    // lse and D rows of each stage; each 64-lane 4-byte load fills one 64-float row (lanes
    // past the sub-tile read zeros into the unused upper half).
    __shared__ __attribute__((aligned(256))) float LDs[NG][NS][2][64];  // lse2 | D
    // With dropout the mask needs registers the kernel does not have (at d = 128 two K
    // fragments were spilled to scratch, and each reload's vmcnt(0) also waited on the ring's
    // prefetches): the K fragments of the last KSP k-steps live in LDS instead, each lane's own
    // 16 bytes, read back per use.  12 KiB more per workgroup keeps two workgroups per CU.
    // The two-group form needs a few registers for its group index and loop bounds: two K
    // fragments move to LDS there too.
    constexpr int KSP = DROP ? 3 : (NG == 2 ? 2 : 0);
    __shared__ __attribute__((aligned(16))) bf16x8 Ksp[KSP ? NG * NW : 1][KSP ? KSP : 1][64];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    // Query groups (NG = 2): two groups of NW waves own the same keys; group g takes every
    // other query sub-tile of the ring, and the two partial dK, dV add up at the end.
    const int grp = NG == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave / NW);
    const int wr = NG == 1 ? wave : wave - grp * NW;
    const int L = xcd_order(blockIdx.x, gridDim.x, nkt);
    int bh, kt;                          // causal: low key tiles see the most queries
    tile_order(L, nkt, gridDim.x / nkt, bh, kt);  // scalar results: this kernel has no VGPR to spare
    const int k0 = kt * 32 * NW, kw0 = k0 + 32 * wr, mykey = kw0 + l32;
    const size_t base = (size_t)bh * N * D, rbase = (size_t)bh * N;

    // K^T and V^T fragments (B operands): row mykey (clamped; results past N are not stored).
    bf16x8 kf[DC], vf[DC];
    {
        const int row = min(mykey, N - 1);
#pragma unroll
        for (int kc = 0; kc < DC; ++kc) {
            kf[kc] = load_bf16x8(K + base + (size_t)row * D + 16 * kc + 8 * half);
            vf[kc] = load_bf16x8(V + base + (size_t)row * D + 16 * kc + 8 * half);
        }
    }
    wait_vmcnt<0>();
    if constexpr (KSP > 0) {
#pragma unroll
        for (int j = 0; j < KSP; ++j) Ksp[wave][j][lane] = kf[DC - KSP + j];
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    const int t_begin = CAUSAL ? k0 / BQ : 0;   // first query sub-tile any key here can see
    const int nsub = (N + BQ - 1) / BQ - t_begin;  // query sub-tiles of the ring
    const int nsteps = (nsub + NG - 1) / NG;         // step i takes sub-tile NG i + g of the ring
    // The ring walks the query sub-tiles from the last one down to t_begin, so the workgroups
    // of a head, which all start at the last sub-tile, read the same Q / dO sub-tile at about
    // the same time and an XCD fetches it from HBM about once.  Walking up from each one's own
    // diagonal, they read different sub-tiles at a time and rely on L2 holding the head's whole
    // Q / dO: at B=4 H=32 N=8192 that fetched 1.42x the compulsory bytes, against 1.19x now.
    const int t_last = t_begin + nsub - 1;
    auto tile_of = [&](int i, int g) { return NG * i + g < nsub ? t_last - (NG * i + g) : -1; };  // -1: past the end
    const int wave_first = CAUSAL ? kw0 / BQ : 0;
    const bool wave_live = kw0 < N;

    uint32_t voff[LPT];
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int g = j * NT + tid, r = g / CPR, c = (g % CPR) ^ swz_row<D>(r);
        voff[j] = (uint32_t)((r * D + c * 8) * 2);
    }
    // Sub-tile t of the query range into stage ST.  Rows at or past N read zeros.  Every
    // wave writes the (identical) lse / D rows, so each wave issues the same loads.
    auto issue = [&](auto st, int i) {
        constexpr int ST = decltype(st)::value;
        // One group: nothing is loaded past the end of the walk, so the ring's last NS
        // sub-tiles are still in their stages when the loop ends (the diagonal pass reads them
        // there).  Two groups keep loading zeros past the end, which keeps their waits fixed.
        if (NG == 1 && i >= nsub) return;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int t = tile_of(i, g);
            const int q0 = t < 0 ? N : t * BQ;  // past the end: zero rows, the loads read zeros
            // Each resource spans only this sub-tile (at most BQ rows): the 32-bit byte count
            // cannot wrap however long the sequence is.
            const uint32_t rows = (uint32_t)min(max(0, N - q0), BQ);
            const i32x4 rq = make_rsrc(Q + base + (size_t)min(q0, N) * D, rows * D * 2);
            const i32x4 ro = make_rsrc(dO + base + (size_t)min(q0, N) * D, rows * D * 2);
#pragma unroll
            for (int j = 0; j < LPT; ++j) {
                load_lds_b128(rq, lds_addr(&Qs[g][ST][(j * NT + wave * 64) * 8]), voff[j]);
                load_lds_b128(ro, lds_addr(&dOs[g][ST][(j * NT + wave * 64) * 8]), voff[j]);
            }
            const i32x4 rl = make_rsrc(LSE2 + rbase + min(q0, N), rows * 4);
            const i32x4 rd = make_rsrc(Delta + rbase + min(q0, N), rows * 4);
            load_lds_b32(rl, lds_addr(&LDs[g][ST][0][0]), (uint32_t)(lane * 4));
            load_lds_b32(rd, lds_addr(&LDs[g][ST][1][0]), (uint32_t)(lane * 4));
        }
    };

    // LDS read addresses that depend only on the lane.
    const __bf16* r_lane[DC];  // Q / dO rows (A operands of S and dP): row l32, chunk 2kc + half
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) r_lane[kc] = &Qs[grp][0][swz<D>(l32, 16 * kc + 8 * half)];
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const __bf16* t_lane[2][DB];  // transposed reads (dO^T, Q^T): rows tr_row, tr_row + 8
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        t_lane[0][db] = &Qs[grp][0][swz<D>(tr_row, 32 * db + tr_col)];
        t_lane[1][db] = &Qs[grp][0][swz<D>(tr_row + 8, 32 * db + tr_col)];
    }
    constexpr int DO_OFF = (int)(sizeof(Qs) / sizeof(__bf16));  // dOs follows Qs in the same layout

    // The arithmetic of one query sub-tile whose rows start at stage offset `so` (elements);
    // MASKED applies the causal mask of the wave's own diagonal sub-tile (query rows
    // kw0 .. kw0 + 31: key l32 > query 8(r/4) + 4 half + r%4).
    auto body = [&](auto masked, int so, int ls, int qs0) {
        constexpr bool MASKED = decltype(masked)::value;
        uint32_t dm[4];
        if constexpr (DROP) dropout_bytes<false>(drop, (uint32_t)bh, mykey, qs0, lane, dm);
        // S = Q K^T and dP = dO V^T: lane = key, register r = query 8(r/4) + 4 half + r%4.
        f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
        for (int kc = 0; kc < DC; ++kc) {
            const bf16x8 kop = (kc >= DC - KSP) ? Ksp[wave][max(kc - (DC - KSP), 0)][lane] : kf[kc];
            sacc = mfma_bf16(load_bf16x8(r_lane[kc] + so), kop, sacc);
            pacc = mfma_bf16(load_bf16x8(r_lane[kc] + so + DO_OFF), vf[kc], pacc);
        }
        // P first: the dV products need only P, so the scheduler can run them on the MFMA
        // while the VALU forms dS = P (dP - D); the dK products follow.  (Pinning P before the
        // dV products, or a scheduling hint here, pushes the kernel past 256 VGPRs.)
        f32x4 d4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(&LDs[grp][ls][0][8 * g + 4 * half]);
            d4[g] = *reinterpret_cast<const f32x4*>(&LDs[grp][ls][1][8 * g + 4 * half]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float p = fast_exp2(fmaf(sacc[4 * g + e], scale_log2, -l4[e]));
                if (MASKED && l32 > 8 * g + 4 * half + e) p = 0.f;
                sacc[4 * g + e] = p;
            }
        }
        bf16x8 pb[2] = {to_bf16x8(sacc, 0), to_bf16x8(sacc, 8)};
        if constexpr (DROP) {
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                u32x4 w4 = __builtin_bit_cast(u32x4, pb[cc]);
                uint32_t w[4] = {w4[0], w4[1], w4[2], w4[3]};
                dropout_apply_bf16(w, dm[2 * cc], dm[2 * cc + 1], drop.thr);
                pb[cc] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
            }
        }
        // dV^T += dO^T P, dK^T += Q^T dS: for k-step cc the B operands hold queries
        // 16cc + 8(i/4) + 4 half + i%4; the transposed reads fetch rows 16cc + tr_row (+8).
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int off = so + 16 * cc * D;
                const bf16x8 a_do = join_tr(lds_read_tr16(t_lane[0][db] + off + DO_OFF),
                                            lds_read_tr16(t_lane[1][db] + off + DO_OFF));
                dv[db] = mfma_bf16(a_do, pb[cc], dv[db]);
            }
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = sacc[4 * g + e];
                if constexpr (DROP)
                    pacc[4 * g + e] = p * (pacc[4 * g + e] * dropout_factor(dm, 4 * g + e, drop) - d4[g][e]);
                else
                    pacc[4 * g + e] = p * (pacc[4 * g + e] - d4[g][e]);
            }
        const bf16x8 sb[2] = {to_bf16x8(pacc, 0), to_bf16x8(pacc, 8)};
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int off = so + 16 * cc * D;
                const bf16x8 a_q = join_tr(lds_read_tr16(t_lane[0][db] + off), lds_read_tr16(t_lane[1][db] + off));
                dk[db] = mfma_bf16(a_q, sb[cc], dk[db]);
            }
    };

    // Causal: the ring pass covers the sub-tiles strictly after each wave's diagonal one, so
    // its body needs no mask; the diagonal sub-tile is done once at the end (below).
    auto step = [&](auto st, int i) {
        constexpr int ST = decltype(st)::value;
        // Sub-tile i has landed (this wave's share) once at most the loads of the next NS - 2
        // steps are outstanding; near the end of a one-group walk fewer of those exist.
        static_assert(NS - 2 == 2, "the waits below assume two steps of loads in flight");
        if (NG == 2 || i + 2 < nsteps) wait_vmcnt<2 * LPS>();
        else if (i + 1 < nsteps) wait_vmcnt<LPS>();
        else wait_vmcnt<0>();
        __syncthreads();  // ... and every wave's; stage (i - 1) % NS is free
        issue(std::integral_constant<int, (ST + NS - 1) % NS>{}, i + NS - 1);
        const int t = tile_of(i, grp);
        if (!wave_live || (CAUSAL ? t <= wave_first : false)) return;
        body(std::false_type{}, ST * STAGE, ST, t * BQ);
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    static_assert(NS == 4, "the loop below is unrolled over four stages");
    issue(S0{}, 0);
    issue(S1{}, 1);
    issue(S2{}, 2);
    int i = 0;
    for (; i + 3 < nsteps; i += 4) {
        step(S0{}, i);
        step(S1{}, i + 1);
        step(S2{}, i + 2);
        step(S3{}, i + 3);
    }
    if (i < nsteps) step(S0{}, i);
    if (i + 1 < nsteps) step(S1{}, i + 1);
    if (i + 2 < nsteps) step(S2{}, i + 2);
    wait_vmcnt<0>();  // the ring's loads have landed ...

    if constexpr (CAUSAL && NG == 1) {
        // Wave w's diagonal sub-tile is ring position nsub - 1 - w, one of the last NS, which
        // no later load has overwritten: it is read where it is.
        static_assert(NS >= NW, "the last NW sub-tiles of the walk must all still be in the ring");
        if (wave_live) {
            const int st = (nsub - 1 - wr) % NS;
            body(std::true_type{}, st * STAGE, st, kw0);
        }
    }
    if constexpr (CAUSAL && NG == 2) {
        static_assert(NS >= NW, "each wave needs a stage of its own for its diagonal sub-tile");
        __syncthreads();  // ... and every wave is done reading the ring
        if (grp == 0 && wave_live) {
            // The diagonal sub-tile (query rows kw0 .. kw0 + 31) into this wave's own stage;
            // only this wave reads it, so its own vmcnt wait is enough.
            const int q0 = kw0;
            const uint32_t rows = (uint32_t)min(max(0, N - q0), BQ);  // one sub-tile: never wraps
            const i32x4 rq = make_rsrc(Q + base + (size_t)q0 * D, rows * D * 2);
            const i32x4 ro = make_rsrc(dO + base + (size_t)q0 * D, rows * D * 2);
#pragma unroll
            for (int j = 0; j < BQ * CPR / 64; ++j) {
                const int g = j * 64 + lane, r = g / CPR, c = (g % CPR) ^ swz_row<D>(r);
                const uint32_t vo = (uint32_t)((r * D + c * 8) * 2);
                load_lds_b128(rq, lds_addr(&Qs[0][wr][j * 64 * 8]), vo);
                load_lds_b128(ro, lds_addr(&dOs[0][wr][j * 64 * 8]), vo);
            }
            const i32x4 rl = make_rsrc(LSE2 + rbase + q0, rows * 4);
            const i32x4 rd = make_rsrc(Delta + rbase + q0, rows * 4);
            load_lds_b32(rl, lds_addr(&LDs[0][wr][0][0]), (uint32_t)(lane * 4));
            load_lds_b32(rd, lds_addr(&LDs[0][wr][1][0]), (uint32_t)(lane * 4));
            wait_vmcnt<0>();
            body(std::true_type{}, wr * STAGE, wr, kw0);
        }
    }

    if constexpr (NG == 2) {
        // dK and dV are plain sums over queries: group 1's partials join group 0's through the
        // LDS of the finished rings, laid out [key block][value][lane].
        constexpr int NV = 2 * DB * 16;
        static_assert(NW * NV * 64 * 4 <= (int)(sizeof(Qs) + sizeof(dOs)), "merge buffer");
        float* xs = reinterpret_cast<float*>(&Qs[0][0][0]) + wr * NV * 64 + lane;
        __syncthreads();  // group 0 is done with its diagonal stages
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    xs[(db * 16 + r) * 64] = dk[db][r];
                    xs[((DB + db) * 16 + r) * 64] = dv[db][r];
                }
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dk[db][r] += xs[(db * 16 + r) * 64];
                dv[db][r] += xs[((DB + db) * 16 + r) * 64];
            }
    }

    if (mykey < N) {
        __bf16* dkrow = dK + base + (size_t)mykey * D;
        __bf16* dvrow = dV + base + (size_t)mykey * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                __bf16 wk[4], wv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wk[e] = (__bf16)(dk[db][4 * g + e] * scale);
                    wv[e] = (__bf16)(DROP ? dv[db][4 * g + e] * drop.inv_keep : dv[db][4 * g + e]);
                }
                const int col = 32 * db + 8 * g + 4 * half;
                *reinterpret_cast<u32x2*>(dkrow + col) = __builtin_bit_cast(u32x2, wk);
                *reinterpret_cast<u32x2*>(dvrow + col) = __builtin_bit_cast(u32x2, wv);
            }
    }
}

// ------------------------------------------------------------------ bf16 dQ
// Workgroup: NW waves x 32 queries (Q^T and dO^T fragments as B operands, the dQ^T
// accumulator in registers); K/V sub-tiles of 32 keys stream through the same swizzled
// NS-stage LDS ring as the forward.  S^T = K Q^T and dP^T = V dO^T put one query per lane,
// so lse and D are per-lane scalars and dS^T feeds dQ^T += K^T dS^T (K^T by transposed
// reads).  This recomputes S and dP instead of accumulating dQ with atomics.  The prologue
// also loads the O rows of its queries and forms D = rowsum(dO o O) next to the dO
// fragments, storing D and lse log2(e) for the dK/dV kernel (the D step of the backward
// pass, with no launch of its own and no second read of dO).
// Software pipeline: the exponentials and dS of sub-tile i run on the VALU while the MFMAs
// compute S and dP of sub-tile i + 1 (two independent chains), then dQ += K(i)^T dS(i).
// DROP: dropout (dS = P (Z dP - D) with Z the keep factor).
// Occupancy: two waves per SIMD at d = 128; three at d = 64, where the kernel fits 168 VGPRs
// (two with dropout, whose mask would spill at that budget).
// NG = 2 (grids of at most kSplitTilesAtMost query tiles): two groups of NW waves per query
// tile take alternate key sub-tiles, and group 1's partial dQ joins group 0's at the end.
template <int D, bool DROP>
struct DqWaves : std::integral_constant<int, D == 64 && !DROP ? 3 : 2> {};

template <int D, int NW, bool CAUSAL, bool DROP, int NG>
__global__ __attribute__((amdgpu_flat_work_group_size(1, NG * NW * 64),
                               amdgpu_waves_per_eu(DqWaves<D, DROP>::value, DqWaves<D, DROP>::value))) void dq_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const __bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ LSE2, float* __restrict__ Delta, __bf16* __restrict__ dQ, int N, int nqt, float scale,
    float scale_log2, DropoutArgs drop) {
    constexpr int BK = 32, NS = 4, STAGE = BK * D, CPR = D / 8, NT = NG * NW * 64;
    constexpr int BM = 32 * NW, DC = D / 16, DB = D / 32;
    constexpr int LPT = BK * CPR / NT;
    constexpr int LPS = 2 * NG * LPT;
    static_assert(LPT >= 1 && BK * CPR % NT == 0, "tile / thread mismatch");
    static_assert((NS - 2) * LPS < 64, "pipeline depth");

    static_assert(NG == 1 || NG == 2, "one or two key groups");
    __shared__ __attribute__((aligned(1024))) __bf16 Ks[NG][NS][STAGE];
    __shared__ __attribute__((aligned(1024))) __bf16 Vs[NG][NS][STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    // Key groups (NG = 2): two groups of NW waves own the same queries; group g takes the
    // sub-tiles 2i + g, and the two partial dQ add up at the end.
    const int grp = NG == 1 ? 0 : __builtin_amdgcn_readfirstlane(wave / NW);
    const int wr = NG == 1 ? wave : wave - grp * NW;
    const int L = xcd_order(blockIdx.x, gridDim.x, nqt);
    int bh, rank;
    tile_order(L, nqt, gridDim.x / nqt, bh, rank);
    const int q0 = (nqt - 1 - rank) * BM;  // heaviest (causal) tiles first
    const size_t base = (size_t)bh * N * D;
    const int wq0 = q0 + 32 * wr, myq = wq0 + l32;

    bf16x8 qf[DC], of[DC];
    // lse of this lane's query (row N - 1 past the end, so the load needs no select that
    // would wait for it here); lse2 and D are formed once the loads have landed (below).
    const float lse_row = LSE[(size_t)bh * N + min(myq, N - 1)];
    float lse2 = INFINITY;
    bf16x8 ob[DC];   // the O row, for D below
    float del = 0.f;  // D of this lane's query
    {
        const int row = min(myq, N - 1);
#pragma unroll
        for (int kc = 0; kc < DC; ++kc) {
            qf[kc] = load_bf16x8(Q + base + (size_t)row * D + 16 * kc + 8 * half);
            of[kc] = load_bf16x8(dO + base + (size_t)row * D + 16 * kc + 8 * half);
            ob[kc] = load_bf16x8(O + base + (size_t)row * D + 16 * kc + 8 * half);
        }
    }
    // No wait here: these loads and the ring's first stage are in flight together (below).

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int nt = (kv_end + BK - 1) / BK;
    const int nsteps = (nt + NG - 1) / NG;  // step i takes sub-tile NG i + g
    const int wave_last = (wq0 >= N) ? -1 : (CAUSAL ? min(nt, (wq0 + 31) / BK + 1) : nt) - 1;
    const int wave_nt = wave_last < grp ? 0 : (wave_last - grp) / NG + 1;

    uint32_t voff[LPT];
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
        const int g = j * NT + tid, r = g / CPR, c = (g % CPR) ^ swz_row<D>(r);
        voff[j] = (uint32_t)((r * D + c * 8) * 2);
    }
    auto issue = [&](auto st, int i) {
        constexpr int ST = decltype(st)::value;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const int kv0 = (NG * i + g) * BK;
            const uint32_t bytes = (uint32_t)min(max(0, N - kv0), BK) * D * 2;  // one sub-tile: never wraps
            const i32x4 rk = make_rsrc(K + base + (size_t)min(kv0, N) * D, bytes);
            const i32x4 rv = make_rsrc(V + base + (size_t)min(kv0, N) * D, bytes);
#pragma unroll
            for (int j = 0; j < LPT; ++j) {
                load_lds_b128(rk, lds_addr(&Ks[g][ST][(j * NT + wave * 64) * 8]), voff[j]);
                load_lds_b128(rv, lds_addr(&Vs[g][ST][(j * NT + wave * 64) * 8]), voff[j]);
            }
        }
    };

    const __bf16* r_lane[DC];  // K / V rows (A operands of S^T and dP^T)
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) r_lane[kc] = &Ks[grp][0][swz<D>(l32, 16 * kc + 8 * half)];
    constexpr int V_OFF = (int)(sizeof(Ks) / sizeof(__bf16));  // Vs follows Ks in the same layout
    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const __bf16* t_lane[2][DB];  // K^T by transposed reads: rows tr_row, tr_row + 8
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        t_lane[0][db] = &Ks[grp][0][swz<D>(tr_row, 32 * db + tr_col)];
        t_lane[1][db] = &Ks[grp][0][swz<D>(tr_row + 8, 32 * db + tr_col)];
    }

    // S^T and dP^T of the sub-tile in stage ST: two independent accumulator chains.
    auto chains = [&](auto st, f32x16& s, f32x16& dp) {
        constexpr int ST = decltype(st)::value;
        s = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int kc = 0; kc < DC; ++kc) {
            s = mfma_bf16(load_bf16x8(r_lane[kc] + ST * STAGE), qf[kc], s);
            dp = mfma_bf16(load_bf16x8(r_lane[kc] + ST * STAGE + V_OFF), of[kc], dp);
        }
    };
    // Causal (key > query) or tail (key >= N) mask of sub-tile t, as -inf scores (P = 0).
    auto needs_mask = [&](int i) {
        const int kv0 = (NG * i + grp) * BK;
        return CAUSAL ? (kv0 + BK - 1 > wq0) : (kv0 + BK > N);
    };
    auto mask = [&](int i, f32x16& s) {
        const int kv0 = (NG * i + grp) * BK;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 8 * (r / 4) + 4 * half + (r % 4);
            if (CAUSAL ? (key > myq) : (key >= N)) s[r] = -INFINITY;
        }
    };
    // P = 2^(scale log2(e) s - lse2) and dS = P (dP - D) of sub-tile t, as bf16 B operands.
    auto grad_scores = [&](int t, f32x16& s, f32x16& dp, bf16x8 (&sb)[2]) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], scale_log2, -lse2));
        if constexpr (DROP) {
            uint32_t dm[4];
            dropout_bytes<true>(drop, (uint32_t)bh, myq, (NG * t + grp) * BK, lane, dm);
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[r] = s[r] * (dp[r] * dropout_factor(dm, r, drop) - del);
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[r] = s[r] * (dp[r] - del);
        }
        sb[0] = to_bf16x8(dp, 0);
        sb[1] = to_bf16x8(dp, 8);
    };
    // dQ^T += K^T dS^T for the sub-tile in stage ST.
    auto dq_product = [&](auto st, const bf16x8 (&sb)[2]) {
        constexpr int ST = decltype(st)::value;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int off = ST * STAGE + 16 * cc * D;
                const bf16x8 a = join_tr(lds_read_tr16(t_lane[0][db] + off), lds_read_tr16(t_lane[1][db] + off));
                dq[db] = mfma_bf16(a, sb[cc], dq[db]);
            }
    };

    // Software pipeline, as in the forward: step i (stage CUR = i % NS) holds S(i), dP(i)
    // (masked) in `sc`, `dc`; the exponentials and dS of sub-tile i run on the VALU while the
    // MFMAs compute S(i+1), dP(i+1) into `sn`, `dn`; then dQ += K(i)^T dS(i).  On a wave's last
    // sub-tile the chains of sub-tile i + 1 still run (on loaded data or zeros, fully masked)
    // and are never used.
    auto step = [&](auto cur_st, int i, f32x16& sc, f32x16& dc, f32x16& sn, f32x16& dn) {
        constexpr int CUR = decltype(cur_st)::value;
        wait_vmcnt<(NS - 3) * LPS>();  // sub-tile i + 1 has landed (this wave's share)
        __syncthreads();               // ... and every wave's; stage (i - 1) % NS is free
        issue(std::integral_constant<int, (CUR + NS - 1) % NS>{}, i + NS - 1);
        if (i >= wave_nt) return;
        bf16x8 sb[2];
        grad_scores(i, sc, dc, sb);
        chains(std::integral_constant<int, (CUR + 1) % NS>{}, sn, dn);
        // Without dropout the compiler's own single-wave GEMM interleaving (iglp_opt 1), which
        // spreads the LDS reads among the S and dP MFMAs, beats the fixed {MFMA, 4 VALU}
        // groups by 2-3% at d = 128 (equal at d = 64, the same code otherwise); the dropout
        // form keeps the groups, which serve its mask's VALU work better.
        if constexpr (DROP) interleave_mfma<2 * DC, 0, 4>();
        else __builtin_amdgcn_iglp_opt(1);
        asm volatile("" : "+v"(sb[0]), "+v"(sb[1]));  // keep the VALU work in region 1
        dq_product(cur_st, sb);
        if (needs_mask(i + 1)) mask(i + 1, sn);
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    static_assert(NS == 4, "the loop below is unrolled over four stages");
    static_assert((NS - 2) * LPS < 64, "pipeline depth");
    issue(S0{}, 0);
    wait_vmcnt<0>();  // the Q, dO, O fragments, lse and stage 0, loaded together
    issue(S1{}, 1);
    issue(S2{}, 2);
    // Rows past N: lse = +inf makes their P exactly 0 (they are not stored either).
    lse2 = myq < N ? lse_row * kLog2e : INFINITY;
    // D = rowsum(dO o O) of this lane's query: the lane holds columns 16 kc + 8 half .. + 7 of
    // dO and O, the lane l ^ 32 the other half of the row.  D and lse log2(e) of these rows
    // go to the workspace for the dK/dV kernel, which runs next.
    {
        float acc = 0.f;
#pragma unroll
        for (int kc = 0; kc < DC; ++kc)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)of[kc][e], (float)ob[kc][e], acc);
        del = myq < N ? sum_halves(acc) : 0.f;
    }
    if (grp == 0 && half == 0 && myq < N) {
        Delta[(size_t)bh * N + myq] = del;
        LSE2[(size_t)bh * N + myq] = lse2;
    }
    __syncthreads();
    f32x16 sa, da, sbb, dbb;
    if (wave_nt > 0) {
        chains(S0{}, sa, da);
        if (needs_mask(0)) mask(0, sa);
    }
    int i = 0;
    for (; i + 3 < nsteps; i += 4) {
        step(S0{}, i, sa, da, sbb, dbb);
        step(S1{}, i + 1, sbb, dbb, sa, da);
        step(S2{}, i + 2, sa, da, sbb, dbb);
        step(S3{}, i + 3, sbb, dbb, sa, da);
    }
    if (i < nsteps) step(S0{}, i, sa, da, sbb, dbb);
    if (i + 1 < nsteps) step(S1{}, i + 1, sbb, dbb, sa, da);
    if (i + 2 < nsteps) step(S2{}, i + 2, sa, da, sbb, dbb);
    wait_vmcnt<0>();

    if constexpr (NG == 2) {
        // dQ is a plain sum over keys: group 1's partial joins group 0's through the LDS of
        // the finished rings, laid out [row block][value][lane].
        constexpr int NV = DB * 16;
        static_assert(NW * NV * 64 * 4 <= (int)(sizeof(Ks) + sizeof(Vs)), "merge buffer");
        float* xs = reinterpret_cast<float*>(&Ks[0][0][0]) + wr * NV * 64 + lane;
        __syncthreads();  // every wave is done with the rings
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) xs[(db * 16 + r) * 64] = dq[db][r];
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) dq[db][r] += xs[(db * 16 + r) * 64];
    }

    if (myq < N) {
        __bf16* row = dQ + base + (size_t)myq * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                __bf16 w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)(dq[db][4 * g + e] * scale);
                *reinterpret_cast<u32x2*>(row + 32 * db + 8 * g + 4 * half) = __builtin_bit_cast(u32x2, w);
            }
    }
}

// ------------------------------------------------------------------ fp32 dK / dV
// fp32 MFMA 32x32x2 (no reduced precision).  Each wave holds 32 keys; per step 32 query
// rows are staged in LDS.  In fp32 the "transposed" products need no transposed reads:
// one MFMA per accumulator register r uses LDS row q(r) directly.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dK, float* __restrict__ dV, int N, int nkt, float scale, float scale_log2) {
    constexpr int NW = 4, BNK = 32 * NW, BQ = 32, NT = 256;
    constexpr int ST = D + 1, DB = D / 32;
    __shared__ float Qs[BQ * ST], dOs[BQ * ST], lse_s[BQ], del_s[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int L = xcd_order(blockIdx.x, gridDim.x, nkt);
    int bh, kt;
    tile_order(L, nkt, gridDim.x / nkt, bh, kt);
    const int k0 = kt * BNK, kw0 = k0 + wave * 32, mykey = kw0 + l32;
    const size_t base = (size_t)bh * N * D, rbase = (size_t)bh * N;

    float kf[D / 2], vf[D / 2];
#pragma unroll
    for (int kc = 0; kc < D / 2; ++kc) {
        kf[kc] = (mykey < N) ? K[base + (size_t)mykey * D + 2 * kc + half] : 0.f;
        vf[kc] = (mykey < N) ? V[base + (size_t)mykey * D + 2 * kc + half] : 0.f;
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }
    const int q_begin = CAUSAL ? (k0 / BQ) * BQ : 0;
    for (int qs0 = q_begin; qs0 < N; qs0 += BQ) {
        __syncthreads();
        for (int c = tid; c < BQ * D; c += NT) {
            const int r = c / D, col = c % D;
            const bool ok = qs0 + r < N;
            Qs[r * ST + col] = ok ? Q[base + (size_t)(qs0 + r) * D + col] : 0.f;
            dOs[r * ST + col] = ok ? dO[base + (size_t)(qs0 + r) * D + col] : 0.f;
        }
        if (tid < BQ) {
            lse_s[tid] = (qs0 + tid < N) ? LSE[rbase + qs0 + tid] * kLog2e : INFINITY;
            del_s[tid] = (qs0 + tid < N) ? Delta[rbase + qs0 + tid] : 0.f;
        }
        __syncthreads();
        if (kw0 >= N || (CAUSAL && qs0 + 31 < kw0)) continue;
        f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
        for (int kc = 0; kc < D / 2; ++kc) {
            sacc = mfma_f32(Qs[l32 * ST + 2 * kc + half], kf[kc], sacc);
            pacc = mfma_f32(dOs[l32 * ST + 2 * kc + half], vf[kc], pacc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ql = 8 * (r / 4) + 4 * half + (r % 4);
            float p = fast_exp2(fmaf(sacc[r], scale_log2, -lse_s[ql]));
            if (CAUSAL && mykey > qs0 + ql) p = 0.f;
            sacc[r] = p;
            pacc[r] = p * (pacc[r] - del_s[ql]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ql = 8 * (r / 4) + 4 * half + (r % 4);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dv[db] = mfma_f32(dOs[ql * ST + 32 * db + l32], sacc[r], dv[db]);
                dk[db] = mfma_f32(Qs[ql * ST + 32 * db + l32], pacc[r], dk[db]);
            }
        }
    }
    if (mykey < N) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 wk, wv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wk[i] = dk[db][4 * g + i] * scale;
                    wv[i] = dv[db][4 * g + i];
                }
                const size_t off = base + (size_t)mykey * D + 32 * db + 8 * g + 4 * half;
                *reinterpret_cast<f32x4*>(dK + off) = wk;
                *reinterpret_cast<f32x4*>(dV + off) = wv;
            }
    }
}

// ------------------------------------------------------------------ fp32 dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ LSE2, float* __restrict__ Delta, float* __restrict__ dQ, int N, int nqt, float scale,
    float scale_log2) {
    constexpr int NW = 4, BM = 32 * NW, BN = 32, NT = 256;
    constexpr int ST = D + 1, DB = D / 32;
    __shared__ float Ks[BN * ST], Vs[BN * ST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int L = xcd_order(blockIdx.x, gridDim.x, nqt);
    int bh, rank;
    tile_order(L, nqt, gridDim.x / nqt, bh, rank);
    const int q0 = (nqt - 1 - rank) * BM;
    const size_t base = (size_t)bh * N * D;
    const int wq0 = q0 + wave * 32, myq = wq0 + l32;

    float qf[D / 2], of[D / 2];
    float acc = 0.f;  // D = rowsum(dO o O): this lane's columns 2 kc + half, lane l ^ 32 the rest
#pragma unroll
    for (int kc = 0; kc < D / 2; ++kc) {
        qf[kc] = (myq < N) ? Q[base + (size_t)myq * D + 2 * kc + half] : 0.f;
        of[kc] = (myq < N) ? dO[base + (size_t)myq * D + 2 * kc + half] : 0.f;
        acc = fmaf(of[kc], (myq < N) ? O[base + (size_t)myq * D + 2 * kc + half] : 0.f, acc);
    }
    const float lse_l = (myq < N) ? LSE[(size_t)bh * N + myq] * kLog2e : INFINITY;
    const float del_l = (myq < N) ? sum_halves(acc) : 0.f;
    // D for the dK/dV kernel, which runs next; lse log2(e) too, so the workspace holds the same
    // two arrays on both paths (the fp32 dK/dV kernel forms it from lse itself).
    if (half == 0 && myq < N) {
        Delta[(size_t)bh * N + myq] = del_l;
        LSE2[(size_t)bh * N + myq] = lse_l;
    }
    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    for (int kv0 = 0; kv0 < kv_end; kv0 += BN) {
        __syncthreads();
        for (int c = tid; c < BN * D; c += NT) {
            const int r = c / D, col = c % D;
            const bool ok = kv0 + r < N;
            Ks[r * ST + col] = ok ? K[base + (size_t)(kv0 + r) * D + col] : 0.f;
            Vs[r * ST + col] = ok ? V[base + (size_t)(kv0 + r) * D + col] : 0.f;
        }
        __syncthreads();
        if (wq0 >= N || (CAUSAL && kv0 > wq0 + 31)) continue;
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kc = 0; kc < D / 2; ++kc) {
            s = mfma_f32(Ks[l32 * ST + 2 * kc + half], qf[kc], s);
            dp = mfma_f32(Vs[l32 * ST + 2 * kc + half], of[kc], dp);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kl = 8 * (r / 4) + 4 * half + (r % 4), key = kv0 + kl;
            float p = fast_exp2(fmaf(s[r], scale_log2, -lse_l));
            if (CAUSAL ? (key > myq) : (key >= N)) p = 0.f;
            dp[r] = p * (dp[r] - del_l);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kl = 8 * (r / 4) + 4 * half + (r % 4);
#pragma unroll
            for (int db = 0; db < DB; ++db) dq[db] = mfma_f32(Ks[kl * ST + 32 * db + l32], dp[r], dq[db]);
        }
    }
    if (myq < N) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = dq[db][4 * g + i] * scale;
                *reinterpret_cast<f32x4*>(dQ + base + (size_t)myq * D + 32 * db + 8 * g + 4 * half) = w;
            }
    }
}

// Record the caller's timing event `i` (if any) on the stream.
hipError_t mark(const BwdArgs& a, int i, hipStream_t st) {
    return a.events ? hipEventRecord(static_cast<hipEvent_t>(a.events[i]), st) : hipSuccess;
}

// Two launches: dQ first, which also computes D = rowsum(dO o O) and lse log2(e) of its rows
// into the workspace, then dK/dV, which reads them for every query row.
template <int D, bool CAUSAL, bool DROP>
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
    constexpr int NW = 4;
    hipError_t e;
    if ((e = mark(a, 0, st)) != hipSuccess) return e;
    const int nqt = (a.N + 32 * NW - 1) / (32 * NW);
    const long long qtiles = (long long)nqt * a.B * a.H;
    bool split = false;  // two key groups per tile (see dq_bf16_kernel)
    if constexpr (D == 128) {
        split = qtiles <= kSplitTilesAtMost;
        if (split)
            hipLaunchKernelGGL((dq_bf16_kernel<D, NW, CAUSAL, DROP, 2>), dim3((unsigned)qtiles),
                               dim3(2 * NW * 64), 0, st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                               (const __bf16*)a.dout, (const __bf16*)a.o, a.lse, a.lse2, a.delta, (__bf16*)a.dq,
                               a.N, nqt, a.scale, a.scale * kLog2e, a.drop);
    }
    if (!split)
        hipLaunchKernelGGL((dq_bf16_kernel<D, NW, CAUSAL, DROP, 1>), dim3((unsigned)qtiles),
                           dim3(NW * 64), 0, st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                           (const __bf16*)a.dout, (const __bf16*)a.o, a.lse, a.lse2, a.delta, (__bf16*)a.dq, a.N,
                           nqt, a.scale, a.scale * kLog2e, a.drop);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(a, 1, st)) != hipSuccess) return e;
    const int nkt = (a.N + 32 * NW - 1) / (32 * NW);
    const long long ktiles = (long long)nkt * a.B * a.H;
    bool ksplit = false;  // two query groups per key tile (see dkdv_bf16_kernel)
    if constexpr (D == 128) {
        ksplit = ktiles <= kSplitTilesAtMost;
        if (ksplit)
            hipLaunchKernelGGL((dkdv_bf16_kernel<D, NW, CAUSAL, DROP, 2>), dim3((unsigned)ktiles), dim3(2 * NW * 64),
                               0, st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                               (const __bf16*)a.dout, (const float*)a.lse2, (const float*)a.delta, (__bf16*)a.dk,
                               (__bf16*)a.dv, a.N, nkt, a.scale, a.scale * kLog2e, a.drop);
    }
    if (!ksplit)
        hipLaunchKernelGGL((dkdv_bf16_kernel<D, NW, CAUSAL, DROP, 1>), dim3((unsigned)ktiles),
                           dim3(NW * 64), 0, st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                           (const __bf16*)a.dout, (const float*)a.lse2, (const float*)a.delta, (__bf16*)a.dk, (__bf16*)a.dv,
                           a.N, nkt, a.scale, a.scale * kLog2e, a.drop);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(a, 2, st);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t st) {
    hipError_t e;
    if ((e = mark(a, 0, st)) != hipSuccess) return e;
    const int nqt = (a.N + 127) / 128;
    hipLaunchKernelGGL((dq_f32_kernel<D, CAUSAL>), dim3((unsigned)((long long)nqt * a.B * a.H)), dim3(256), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout,
                       (const float*)a.o, a.lse, a.lse2, a.delta, (float*)a.dq, a.N, nqt, a.scale,
                       a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(a, 1, st)) != hipSuccess) return e;
    const int nkt = (a.N + 127) / 128;
    hipLaunchKernelGGL((dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)((long long)nkt * a.B * a.H)), dim3(256), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse,
                       (const float*)a.delta, (float*)a.dk, (float*)a.dv, a.N, nkt, a.scale, a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(a, 2, st);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
    if (a.dtype == kBF16) {
        if (a.dropout) {
            if (a.d == 128)
                return a.causal ? launch_bwd_bf16<128, true, true>(a, st) : launch_bwd_bf16<128, false, true>(a, st);
            return a.causal ? launch_bwd_bf16<64, true, true>(a, st) : launch_bwd_bf16<64, false, true>(a, st);
        }
        if (a.d == 128)
            return a.causal ? launch_bwd_bf16<128, true, false>(a, st) : launch_bwd_bf16<128, false, false>(a, st);
        return a.causal ? launch_bwd_bf16<64, true, false>(a, st) : launch_bwd_bf16<64, false, false>(a, st);
    }
    if (a.d == 128) return a.causal ? launch_bwd_f32<128, true>(a, st) : launch_bwd_f32<128, false>(a, st);
    return a.causal ? launch_bwd_f32<64, true>(a, st) : launch_bwd_f32<64, false>(a, st);
}

}  // namespace fa
