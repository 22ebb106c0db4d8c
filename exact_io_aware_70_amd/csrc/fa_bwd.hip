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
// Three launches on one stream, no atomics (run-to-run bitwise deterministic):
//   1. delta:  D_i = rowsum(dO * O) into the caller's workspace;
//   2. dK/dV:  one workgroup per key tile, each wave holding 32 keys (K, V fragments and
//              the dK^T, dV^T accumulators in registers), walking the query tiles;
//   3. dQ:     one workgroup per query tile, each wave holding 32 queries, walking the key
//              tiles (recomputes S and dP a second time instead of accumulating dQ with
//              atomics).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// ------------------------------------------------------------------ delta = rowsum(dO * O)
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                     float* __restrict__ Delta, long long rows) {
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;         // chunks (threads) per row
    constexpr int RPB = 256 / CPR;       // rows per block
    const int tid = threadIdx.x;
    const long long row = (long long)blockIdx.x * RPB + tid / CPR;
    const int c = tid % CPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + c * EPC);
        const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + c * EPC);
        if constexpr (sizeof(T) == 2) {
            const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = fmaf((float)x[i], (float)y[i], acc);
        } else {
            const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = fmaf(x[i], y[i], acc);
        }
    }
#pragma unroll
    for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && c == 0) Delta[row] = acc;
}

// ------------------------------------------------------------------ bf16 dK / dV
// Workgroup: NW waves x 32 keys.  Per step a 64-row query tile (Q, dO, lse, D) is staged
// in LDS (double-buffered).  S = Q K^T and dP = dO V^T are computed with keys along the
// lanes (C layout: lane = key, registers = queries), so P and dS feed the B operand of
// dV^T += dO^T P and dK^T += Q^T dS directly; dO^T and Q^T come from transposed LDS reads.
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void dkdv_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    __bf16* __restrict__ dK, __bf16* __restrict__ dV, int N, int nkt, float scale, float scale_log2) {
    constexpr int BNK = 32 * NW, BQ = 64, NT = NW * 64;
    constexpr int ST = D + 8;
    constexpr int DC = D / 16, DB = D / 32, CPR = D / 8;
    constexpr int NCH = BQ * CPR / NT;
    static_assert(NCH >= 1 && BQ * CPR % NT == 0, "tile / thread mismatch");

    __shared__ __attribute__((aligned(16))) __bf16 Qs[2][BQ * ST];
    __shared__ __attribute__((aligned(16))) __bf16 dOs[2][BQ * ST];
    __shared__ __attribute__((aligned(16))) float lse_s[2][BQ];
    __shared__ __attribute__((aligned(16))) float del_s[2][BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nkt;
    const int kt = L % nkt;  // causal: low key tiles see the most queries; they go first
    const int k0 = kt * BNK, kw0 = k0 + wave * 32, mykey = kw0 + l32;
    const size_t base = (size_t)bh * N * D;
    const size_t rbase = (size_t)bh * N;

    bf16x8 kf[DC], vf[DC];
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) {
        if (mykey < N) {
            kf[kc] = load_bf16x8(K + base + (size_t)mykey * D + 16 * kc + 8 * half);
            vf[kc] = load_bf16x8(V + base + (size_t)mykey * D + 16 * kc + 8 * half);
        } else {
            kf[kc] = bf16x8{};
            vf[kc] = bf16x8{};
        }
    }
    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dk[db] = f32x16{};
        dv[db] = f32x16{};
    }

    const int q_begin = CAUSAL ? (k0 / BQ) * BQ : 0;
    const int nsteps = (N - q_begin + BQ - 1) / BQ;

    u32x4 qst[NCH], ost[NCH];
    float lse_r = 0.f, del_r = 0.f;
    auto gload = [&](int s) {
        const int qs0 = q_begin + s * BQ;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
            if (qs0 + r < N) {
                qst[i] = *reinterpret_cast<const u32x4*>(Q + base + (size_t)(qs0 + r) * D + cc * 8);
                ost[i] = *reinterpret_cast<const u32x4*>(dO + base + (size_t)(qs0 + r) * D + cc * 8);
            } else {
                qst[i] = u32x4{0, 0, 0, 0};
                ost[i] = u32x4{0, 0, 0, 0};
            }
        }
        if (tid < BQ) {
            // Rows past N: lse = +inf makes their P exactly 0, and D = 0 their dS.
            lse_r = (qs0 + tid < N) ? LSE[rbase + qs0 + tid] * kLog2e : INFINITY;
            del_r = (qs0 + tid < N) ? Delta[rbase + qs0 + tid] : 0.f;
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
            *reinterpret_cast<u32x4*>(&Qs[buf][r * ST + cc * 8]) = qst[i];
            *reinterpret_cast<u32x4*>(&dOs[buf][r * ST + cc * 8]) = ost[i];
        }
        if (tid < BQ) {
            lse_s[buf][tid] = lse_r;
            del_s[buf][tid] = del_r;
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    for (int s = 0; s < nsteps; ++s) {
        const int buf = s & 1, qs0 = q_begin + s * BQ;
        if (s + 1 < nsteps) gload(s + 1);
        if (kw0 < N) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int qb0 = qs0 + 32 * qb;
                if (CAUSAL && qb0 + 31 < kw0) continue;  // every query of the block precedes every key
                f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
                for (int kc = 0; kc < DC; ++kc) {
                    const int off = (32 * qb + l32) * ST + 16 * kc + 8 * half;
                    sacc = mfma_bf16(load_bf16x8(&Qs[buf][off]), kf[kc], sacc);
                    pacc = mfma_bf16(load_bf16x8(&dOs[buf][off]), vf[kc], pacc);
                }
                // lane = key, register r = query 32qb + 8(r/4) + 4half + r%4.
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ql = 32 * qb + 8 * g + 4 * half;
                    const f32x4 lse4 = *reinterpret_cast<const f32x4*>(&lse_s[buf][ql]);
                    const f32x4 del4 = *reinterpret_cast<const f32x4*>(&del_s[buf][ql]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float p = fast_exp2(fmaf(sacc[4 * g + i], scale_log2, -lse4[i]));
                        if (CAUSAL && mykey > qs0 + ql + i) p = 0.f;
                        sacc[4 * g + i] = p;
                        pacc[4 * g + i] = p * (pacc[4 * g + i] - del4[i]);
                    }
                }
                const bf16x8 pb[2] = {to_bf16x8(sacc, 0), to_bf16x8(sacc, 8)};
                const bf16x8 sb[2] = {to_bf16x8(pacc, 0), to_bf16x8(pacc, 8)};
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int row = (32 * qb + 16 * cc + tr_row) * ST + tr_col;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 a_do = join_tr(lds_read_tr16(&dOs[buf][row + 32 * db]),
                                                    lds_read_tr16(&dOs[buf][row + 8 * ST + 32 * db]));
                        dv[db] = mfma_bf16(a_do, pb[cc], dv[db]);
                        const bf16x8 a_q = join_tr(lds_read_tr16(&Qs[buf][row + 32 * db]),
                                                   lds_read_tr16(&Qs[buf][row + 8 * ST + 32 * db]));
                        dk[db] = mfma_bf16(a_q, sb[cc], dk[db]);
                    }
                }
            }
        }
        if (s + 1 < nsteps) lstore(buf ^ 1);
        __syncthreads();
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
                for (int i = 0; i < 4; ++i) {
                    wk[i] = (__bf16)(dk[db][4 * g + i] * scale);
                    wv[i] = (__bf16)dv[db][4 * g + i];
                }
                const int col = 32 * db + 8 * g + 4 * half;
                *reinterpret_cast<u32x2*>(dkrow + col) = __builtin_bit_cast(u32x2, wk);
                *reinterpret_cast<u32x2*>(dvrow + col) = __builtin_bit_cast(u32x2, wv);
            }
    }
}

// ------------------------------------------------------------------ bf16 dQ
// Workgroup: NW waves x 32 queries, K/V tiles of 64 keys double-buffered in LDS.  Like
// the forward: S^T = K Q^T and dP^T = V dO^T put one query per lane, so lse and D are
// per-lane scalars and dS^T feeds dQ^T += K^T dS^T (K^T by transposed LDS reads).
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void dq_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    __bf16* __restrict__ dQ, int N, int nqt, float scale, float scale_log2) {
    constexpr int BM = 32 * NW, BN = 64, NT = NW * 64;
    constexpr int KST = D + 16;  // K is read both row-wise and transposed
    constexpr int VST = D + 8;
    constexpr int DC = D / 16, DB = D / 32, CPR = D / 8;
    constexpr int NCH = BN * CPR / NT;
    static_assert(NCH >= 1 && BN * CPR % NT == 0, "tile / thread mismatch");

    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * KST];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[2][BN * VST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt;
    const int q0 = (nqt - 1 - (L % nqt)) * BM;
    const size_t base = (size_t)bh * N * D;
    const int wq0 = q0 + wave * 32, myq = wq0 + l32;

    bf16x8 qf[DC], of[DC];
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) {
        if (myq < N) {
            qf[kc] = load_bf16x8(Q + base + (size_t)myq * D + 16 * kc + 8 * half);
            of[kc] = load_bf16x8(dO + base + (size_t)myq * D + 16 * kc + 8 * half);
        } else {
            qf[kc] = bf16x8{};
            of[kc] = bf16x8{};
        }
    }
    const float lse_l = (myq < N) ? LSE[(size_t)bh * N + myq] * kLog2e : INFINITY;
    const float del_l = (myq < N) ? Delta[(size_t)bh * N + myq] : 0.f;

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int nt = (kv_end + BN - 1) / BN;

    u32x4 kst[NCH], vst[NCH];
    auto gload = [&](int t) {
        const int kv0 = t * BN;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
            if (kv0 + r < N) {
                kst[i] = *reinterpret_cast<const u32x4*>(K + base + (size_t)(kv0 + r) * D + cc * 8);
                vst[i] = *reinterpret_cast<const u32x4*>(V + base + (size_t)(kv0 + r) * D + cc * 8);
            } else {
                kst[i] = u32x4{0, 0, 0, 0};
                vst[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
            *reinterpret_cast<u32x4*>(&Ks[buf][r * KST + cc * 8]) = kst[i];
            *reinterpret_cast<u32x4*>(&Vs[buf][r * VST + cc * 8]) = vst[i];
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    const int tr_row = 4 * half + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1, kv0 = t * BN;
        if (t + 1 < nt) gload(t + 1);
        const bool active = (wq0 < N) && (!CAUSAL || kv0 <= wq0 + 31);
        if (active) {
            f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int kc = 0; kc < DC; ++kc)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    s[kb] = mfma_bf16(load_bf16x8(&Ks[buf][(32 * kb + l32) * KST + 16 * kc + 8 * half]), qf[kc], s[kb]);
                    dp[kb] = mfma_bf16(load_bf16x8(&Vs[buf][(32 * kb + l32) * VST + 16 * kc + 8 * half]), of[kc], dp[kb]);
                }
            bf16x8 sb[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kv0 + 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
                    float p = fast_exp2(fmaf(s[kb][r], scale_log2, -lse_l));
                    if (CAUSAL ? (key > myq) : (key >= N)) p = 0.f;
                    dp[kb][r] = p * (dp[kb][r] - del_l);
                }
                sb[kb][0] = to_bf16x8(dp[kb], 0);
                sb[kb][1] = to_bf16x8(dp[kb], 8);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const __bf16* krow = &Ks[buf][(32 * kb + 16 * cc + tr_row) * KST + tr_col];
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 a = join_tr(lds_read_tr16(krow + 32 * db), lds_read_tr16(krow + 8 * KST + 32 * db));
                        dq[db] = mfma_bf16(a, sb[kb][cc], dq[db]);
                    }
                }
        }
        if (t + 1 < nt) lstore(buf ^ 1);
        __syncthreads();
    }

    if (myq < N) {
        __bf16* row = dQ + base + (size_t)myq * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                __bf16 w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (__bf16)(dq[db][4 * g + i] * scale);
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
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nkt, kt = L % nkt;
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
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dQ, int N, int nqt, float scale, float scale_log2) {
    constexpr int NW = 4, BM = 32 * NW, BN = 32, NT = 256;
    constexpr int ST = D + 1, DB = D / 32;
    __shared__ float Ks[BN * ST], Vs[BN * ST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt;
    const int q0 = (nqt - 1 - (L % nqt)) * BM;
    const size_t base = (size_t)bh * N * D;
    const int wq0 = q0 + wave * 32, myq = wq0 + l32;

    float qf[D / 2], of[D / 2];
#pragma unroll
    for (int kc = 0; kc < D / 2; ++kc) {
        qf[kc] = (myq < N) ? Q[base + (size_t)myq * D + 2 * kc + half] : 0.f;
        of[kc] = (myq < N) ? dO[base + (size_t)myq * D + 2 * kc + half] : 0.f;
    }
    const float lse_l = (myq < N) ? LSE[(size_t)bh * N + myq] * kLog2e : INFINITY;
    const float del_l = (myq < N) ? Delta[(size_t)bh * N + myq] : 0.f;
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

template <typename T, int D>
hipError_t launch_delta(const BwdArgs& a, hipStream_t st) {
    constexpr int CPR = D / (16 / sizeof(T));
    constexpr int RPB = 256 / CPR;
    const long long rows = (long long)a.B * a.H * a.N;
    const long long grid = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, st, (const T*)a.o, (const T*)a.dout,
                       a.delta, rows);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
    constexpr int NW = 4;
    hipError_t e = launch_delta<__bf16, D>(a, st);
    if (e != hipSuccess) return e;
    const int nkt = (a.N + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((dkdv_bf16_kernel<D, NW, CAUSAL>), dim3((unsigned)((long long)nkt * a.B * a.H)), dim3(NW * 64), 0,
                       st, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                       (const float*)a.delta, (__bf16*)a.dk, (__bf16*)a.dv, a.N, nkt, a.scale, a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int nqt = (a.N + 32 * NW - 1) / (32 * NW);
    hipLaunchKernelGGL((dq_bf16_kernel<D, NW, CAUSAL>), dim3((unsigned)((long long)nqt * a.B * a.H)), dim3(NW * 64), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                       (const float*)a.delta, (__bf16*)a.dq, a.N, nqt, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t st) {
    hipError_t e = launch_delta<float, D>(a, st);
    if (e != hipSuccess) return e;
    const int nkt = (a.N + 127) / 128;
    hipLaunchKernelGGL((dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)((long long)nkt * a.B * a.H)), dim3(256), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse,
                       (const float*)a.delta, (float*)a.dk, (float*)a.dv, a.N, nkt, a.scale, a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int nqt = (a.N + 127) / 128;
    hipLaunchKernelGGL((dq_f32_kernel<D, CAUSAL>), dim3((unsigned)((long long)nqt * a.B * a.H)), dim3(256), 0, st,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse,
                       (const float*)a.delta, (float*)a.dq, a.N, nqt, a.scale, a.scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t st) {
    if (a.dtype == kBF16) {
        if (a.d == 128) return a.causal ? launch_bwd_bf16<128, true>(a, st) : launch_bwd_bf16<128, false>(a, st);
        return a.causal ? launch_bwd_bf16<64, true>(a, st) : launch_bwd_bf16<64, false>(a, st);
    }
    if (a.d == 128) return a.causal ? launch_bwd_f32<128, true>(a, st) : launch_bwd_f32<128, false>(a, st);
    return a.causal ? launch_bwd_f32<64, true>(a, st) : launch_bwd_f32<64, false>(a, st);
}

}  // namespace fa
