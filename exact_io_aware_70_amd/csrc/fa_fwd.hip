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
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// Lazy rescaling: the reference maximum m_ref of a row is raised only when a tile's
// maximum exceeds it by more than kRescaleSlack (log2 units), so exponentials stay
// below 2^kRescaleSlack.  The result is the same sum written relative to a different
// reference point (exact in real arithmetic), and most tiles skip the O rescale.
constexpr float kRescaleSlack = 8.0f;

// ------------------------------------------------------------------ bf16, MFMA 32x32x16
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int nqt, float scale_log2) {
    constexpr int BM = 32 * NW;         // query rows per workgroup
    constexpr int BN = 64;              // keys per K/V tile
    constexpr int NT = NW * 64;         // threads
    constexpr int KST = D + 8;          // K row stride in LDS (16-byte pad: conflict-free b128 reads)
    constexpr int VST = D + 16;         // V row stride in LDS (32-byte pad for transposed reads)
    constexpr int DC = D / 16;          // k-steps of the S^T product
    constexpr int DB = D / 32;          // 32-row blocks of O^T
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int NCH = BN * CPR / NT;  // chunks per thread per tensor per tile
    static_assert(NCH >= 1 && BN * CPR % NT == 0, "tile / thread mismatch");

    __shared__ __attribute__((aligned(16))) __bf16 Ks[2][BN * KST];
    __shared__ __attribute__((aligned(16))) __bf16 Vs[2][BN * VST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int half = lane >> 5, l32 = lane & 31;

    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt;
    const int qt = nqt - 1 - (L % nqt);  // heaviest (causal) tiles first
    const int q0 = qt * BM;
    const size_t base = (size_t)bh * N * D;
    const __bf16* Qh = Q + base;
    const __bf16* Kh = K + base;
    const __bf16* Vh = V + base;

    const int wq0 = q0 + wave * 32;  // first query row of this wave
    const int myq = wq0 + l32;       // this lane's query row

    // Q^T fragment as the B operand of S^T = K Q^T, resident for the whole loop.
    bf16x8 qf[DC];
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) {
        if (myq < N) qf[kc] = load_bf16x8(Qh + (size_t)myq * D + 16 * kc + 8 * half);
        else qf[kc] = bf16x8{};
    }

    const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
    const int nt = (kv_end + BN - 1) / BN;

    u32x4 kst[NCH], vst[NCH];
    auto gload = [&](int t) {
        const int kv0 = t * BN;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + i * NT, r = c / CPR, cc = c % CPR;
            if (kv0 + r < N) {
                kst[i] = *reinterpret_cast<const u32x4*>(Kh + (size_t)(kv0 + r) * D + cc * 8);
                vst[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)(kv0 + r) * D + cc * 8);
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

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_ref = kNegBig;  // log2-domain reference maximum of this row
    float lsum = 0.f;       // this lane's share of the row sum (the other half holds the rest)

    gload(0);
    lstore(0);
    __syncthreads();

    for (int t = 0; t < nt; ++t) {
        const int buf = t & 1, kv0 = t * BN;
        if (t + 1 < nt) gload(t + 1);

        const bool active = (wq0 < N) && (!CAUSAL || kv0 <= wq0 + 31);  // wave-uniform
        if (active) {
            // S^T tile: rows = 64 keys (two 32-blocks), columns = the wave's 32 queries.
            f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int kc = 0; kc < DC; ++kc) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = load_bf16x8(&Ks[buf][(32 * kb + l32) * KST + 16 * kc + 8 * half]);
                    s[kb] = mfma_bf16(a, qf[kc], s[kb]);
                }
            }
            // Masks: causal (key > query) on tiles that reach past the wave's first row,
            // and keys beyond N on the ragged last tile.
            const bool need_mask = CAUSAL ? (kv0 + BN - 1 > wq0) : (kv0 + BN > N);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
                        const bool dead = CAUSAL ? (key > myq) : (key >= N);
                        if (dead) s[kb][r] = -INFINITY;
                    }
            }
            // Row maximum of this tile (log2 domain).
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
            // P~ = exp2(s * scale * log2(e) - m_ref), summed and rounded to bf16 operands.
            bf16x8 pb[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(s[kb][r], scale_log2, -m_ref));
                    s[kb][r] = p;
                    lsum += p;
                }
                pb[kb][0] = to_bf16x8(s[kb], 0);
                pb[kb][1] = to_bf16x8(s[kb], 8);
            }
            // O^T += V^T P^T.  For P^T operand (kb, cc), lane l carries keys
            // 32kb + 16cc + 4(l/32) + {0..3} and the same + 8; the transposed LDS read
            // gives V^T rows d = 32db + l%32 at exactly those keys.
            const int tr_row = 4 * half + ((lane & 15) >> 2);
            const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const __bf16* vrow = &Vs[buf][(32 * kb + 16 * cc + tr_row) * VST + tr_col];
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 a = join_tr(lds_read_tr16(vrow + 32 * db),
                                                 lds_read_tr16(vrow + 8 * VST + 32 * db));
                        oacc[db] = mfma_bf16(a, pb[kb][cc], oacc[db]);
                    }
                }
        }
        if (t + 1 < nt) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: O = acc / l, lse = m_ref * ln 2 + ln l.
    lsum += swap_halves(lsum);
    if (myq < N) {
        const float inv = 1.0f / lsum;
        __bf16* orow = O + base + (size_t)myq * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                __bf16 w[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (__bf16)(oacc[db][4 * g + i] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * half) = __builtin_bit_cast(u32x2, w);
            }
        if (half == 0) LSE[(size_t)bh * N + myq] = m_ref * kLn2 + __logf(lsum);
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
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = L / nqt;
    const int q0 = (nqt - 1 - (L % nqt)) * BM;
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

template <int D, int NW, bool CAUSAL>
hipError_t launch_bf16(const FwdArgs& a, hipStream_t st) {
    constexpr int BM = 32 * NW;
    const int nqt = (a.N + BM - 1) / BM;
    const long long grid = (long long)nqt * a.B * a.H;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, CAUSAL>), dim3((unsigned)grid), dim3(NW * 64), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse,
                       a.N, nqt, a.scale * kLog2e);
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
        if (a.d == 128) return a.causal ? launch_bf16<128, 4, true>(a, st) : launch_bf16<128, 4, false>(a, st);
        return a.causal ? launch_bf16<64, 4, true>(a, st) : launch_bf16<64, 4, false>(a, st);
    }
    if (a.d == 128) return a.causal ? launch_f32<128, true>(a, st) : launch_f32<128, false>(a, st);
    return a.causal ? launch_f32<64, true>(a, st) : launch_f32<64, false>(a, st);
}

long long fwd_grid_tiles(int N, int dtype) {
    (void)dtype;
    return (N + 127) / 128;  // both paths use 128 query rows per workgroup
}

}  // namespace fa
