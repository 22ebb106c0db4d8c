// Standard (materialising) attention on gfx950: the baseline the pages measure FlashAttention
// against, built from the same kind of kernels so both run on one harness.
//
// "How FlashAttention Actually Works" -- "The GPU Memory Wall: HBM vs. SRAM": standard attention
// writes the score matrix Q K^T to HBM, reads it back for the softmax, writes the probability
// matrix, and reads it again to multiply by V.  "Breaking the Memory Wall" -- "The Problem: The
// Memory Wall": those N x N intermediates are what grows quadratically.  The backward pass of
// standard attention reads the stored probability matrix instead of recomputing it ("How
// FlashAttention Actually Works" -- "The Backward Pass: Recomputation" describes the
// alternative).
//
// Forward, three launches per call:
//   1. S = scale Q K^T (masked to -inf) into the caller's P buffer   (N x N written)
//   2. row softmax of that buffer in place, lse per row              (N x N read and written)
//   3. O = P V                                                       (N x N read)
// Backward, five launches:
//   1. dV = P^T dO          (P read)
//   2. dP = dO V^T          (N x N written to the caller's workspace)
//   3. dS = P o (dP - D), D = rowsum(P o dP), in place over dP     (P, dP read; dS written)
//   4. dQ = scale dS K      (dS read)
//   5. dK = scale dS^T Q    (dS read)
//
// The N x N matrices are stored [B, H, N, Np] in bf16, Np = N rounded up to 128: rows are whole
// 16-byte vectors, and the padding columns hold S = -inf, P = 0, dP = 0 and dS = 0.
//
// One MFMA GEMM kernel serves all six products: C = alpha op(A) op(B) per head, 128 x BN
// output tiles, four waves of 64 x BN/2, 32-deep k-steps through a two-stage LDS ring filled
// by loads that write LDS directly.  An operand is "k-major" when its reduction index is the
// contiguous one (Q, K as K^T, dO as the A of dO V^T, P and dS as the A of P V and dS K) and
// "m-major" otherwise (V, dO, K, Q as B operands; P^T, dS^T as A operands); m-major tiles are
// read with ds_read_b64_tr_b16, so no operand is transposed in memory.  Rows of an operand past
// its valid range read zeros through range-checked buffer loads.  A causal product skips the
// k-steps where the triangular operand is zero, and the score and dP products skip the tiles
// above the diagonal, writing -inf (S) or 0 (dP) there.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kStdBM = 128;  // output rows per workgroup
constexpr int kStdBK = 32;   // reduction depth per k-step

// k-range of a causal product: P and dS are zero above the diagonal (key > query).
enum : int {
    kRangeFull = 0,
    kRangeUpToRow = 1,    // A[m][k] = 0 for k > m (P, dS as A, m = query): k < m0 + BM
    kRangeFromRow = 2,    // A[m][k] = 0 for k < m (P^T, dS^T as A, m = key): k >= m0
};
// What the epilogue writes.
enum : int {
    kEpiPlain = 0,   // alpha * acc, rows < M
    kEpiScores = 1,  // S: -inf for col >= n_valid or (causal) col > row; causal tiles above the
                     // diagonal are filled with -inf without being computed
    kEpiZeroAbove = 2,  // dP: causal tiles above the diagonal are filled with 0 (P is 0 there)
};

struct StdGemmArgs {
    const __bf16* A;
    const __bf16* B;
    __bf16* C;
    long long sA, sB, sC;  // per-head strides (elements)
    int lda, ldb, ldc;     // row strides of the stored arrays (elements)
    int a_rows, b_rows;    // valid stored rows of A and B (rows past read as zeros)
    int M;                 // rows of C that are stored
    int ntiles_n;          // column tiles of C (BN columns each)
    int K;                 // reduction length, a multiple of kStdBK
    int n_valid;           // kEpiScores: keys < n_valid are real
    int causal;
    float alpha;
};

// Geometry of one operand tile: R rows of the m (or n) dimension by kStdBK reduction steps.
//   k-major: stored rows are m, LDS tile [R][32] (64-byte rows, four 16-byte chunks); chunk c of
//            row r sits at slot c ^ ((r >> 2) & 3), so the 16 rows a 128-bit read touches at
//            once fall in 16 distinct bank groups.
//   m-major: stored rows are k, LDS tile [32][R] with the attention kernels' swizzle swz<R>,
//            which keeps the transposed reads free of bank conflicts.
template <bool KMAJ, int R>
struct StdOp {
    static constexpr int CPR = KMAJ ? kStdBK / 8 : R / 8;  // 16-byte chunks per stored row
    static constexpr int CHUNKS = R * kStdBK / 8;
    static constexpr int LPT = CHUNKS / 256;                // LDS-direct loads per thread
    static constexpr int ELEMS = R * kStdBK;
    static_assert(LPT >= 1 && CHUNKS % 256 == 0, "tile / thread mismatch");

    // Byte offset, from the tile's first stored element, that thread `tid` loads for its j-th
    // chunk, and the tile's buffer resource (stored rows past `valid` read zeros).
    __device__ static uint32_t voff(int j, int tid, int ld) {
        const int g = j * 256 + tid, row = g / CPR, slot = g % CPR;
        const int c = KMAJ ? (slot ^ ((row >> 2) & 3)) : (slot ^ swz_row<R>(row));
        return (uint32_t)(row * ld * 2 + c * 16);
    }
    __device__ static i32x4 rsrc(const __bf16* base, int valid, int ld) {
        const int rows = KMAJ ? R : kStdBK;
        const int v = max(0, min(valid, rows));
        const uint32_t bytes = v ? (uint32_t)((v - 1) * ld * 2 + (KMAJ ? kStdBK : R) * 2) : 0u;
        return make_rsrc(base, bytes);
    }
    // MFMA operand for `lane`: rows rb .. rb + 31 of the m dimension, reduction elements
    // 16 ks + 8 (lane / 32) + 0..7.
    __device__ static bf16x8 read(const __bf16* tile, int rb, int ks, int lane) {
        const int half = lane >> 5, l32 = lane & 31;
        if constexpr (KMAJ) {
            const int row = rb + l32, c = 2 * ks + half;
            return load_bf16x8(tile + (row * 4 + (c ^ ((row >> 2) & 3))) * 8);
        } else {
            const int row = 16 * ks + 8 * half + ((lane & 15) >> 2);
            const int col = rb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            return join_tr(lds_read_tr16(tile + swz<R>(row, col)), lds_read_tr16(tile + swz<R>(row + 4, col)));
        }
    }
};

template <bool A_KMAJ, bool B_KMAJ, int BN, int RANGE, int EPI>
__device__ __forceinline__ void std_gemm(const StdGemmArgs& a) {
    using OA = StdOp<A_KMAJ, kStdBM>;
    using OB = StdOp<B_KMAJ, BN>;
    constexpr int BM = kStdBM, BK = kStdBK;
    constexpr int WN = BN / 2;        // output columns per wave
    constexpr int NBJ = WN / 32;      // 32-column blocks per wave
    __shared__ __attribute__((aligned(1024))) __bf16 As[2][OA::ELEMS];
    __shared__ __attribute__((aligned(1024))) __bf16 Bs[2][OB::ELEMS];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int ntiles_m = (a.M + BM - 1) / BM;
    const int per_head = ntiles_m * a.ntiles_n;
    const int bh = blockIdx.x / per_head, t = blockIdx.x - bh * per_head;
    const int mt = t / a.ntiles_n, nt = t - mt * a.ntiles_n;
    const int m0 = mt * BM, n0 = nt * BN;
    __bf16* C = a.C + bh * a.sC;

    // Causal score / dP tiles wholly above the diagonal: written, not computed.
    if constexpr (EPI == kEpiScores || EPI == kEpiZeroAbove) {
        if (a.causal && n0 > m0 + BM - 1) {
            const __bf16 fill = (EPI == kEpiScores) ? (__bf16)(-INFINITY) : (__bf16)0.0f;
            // 16 bytes per thread per row pass: BN / 8 threads per row.
            constexpr int TPR = BN / 8, RPP = 256 / TPR;
            bf16x8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = fill;
            for (int r = tid / TPR; r < BM; r += RPP) {
                const int row = m0 + r;
                if (row < a.M)
                    *reinterpret_cast<u32x4*>(C + (size_t)row * a.ldc + n0 + 8 * (tid % TPR)) =
                        __builtin_bit_cast(u32x4, f);
            }
            return;
        }
    }

    int k_begin = 0, k_end = a.K;
    if constexpr (RANGE == kRangeUpToRow) {
        if (a.causal) k_end = min(a.K, (m0 + BM + BK - 1) / BK * BK);
    } else if constexpr (RANGE == kRangeFromRow) {
        if (a.causal) k_begin = m0 / BK * BK;
    }

    const __bf16* A = a.A + bh * a.sA;
    const __bf16* B = a.B + bh * a.sB;
    uint32_t va[OA::LPT], vb[OB::LPT];
#pragma unroll
    for (int j = 0; j < OA::LPT; ++j) va[j] = OA::voff(j, tid, a.lda);
#pragma unroll
    for (int j = 0; j < OB::LPT; ++j) vb[j] = OB::voff(j, tid, a.ldb);

    // Enqueue the k-step starting at k0 into stage st.
    auto issue = [&](int st, int k0) {
        const __bf16* abase = A_KMAJ ? A + (size_t)m0 * a.lda + k0 : A + (size_t)k0 * a.lda + m0;
        const __bf16* bbase = B_KMAJ ? B + (size_t)n0 * a.ldb + k0 : B + (size_t)k0 * a.ldb + n0;
        const i32x4 ra = OA::rsrc(abase, A_KMAJ ? a.a_rows - m0 : a.a_rows - k0, a.lda);
        const i32x4 rb = OB::rsrc(bbase, B_KMAJ ? a.b_rows - n0 : a.b_rows - k0, a.ldb);
#pragma unroll
        for (int j = 0; j < OA::LPT; ++j) load_lds_b128(ra, lds_addr(&As[st][(j * 256 + wave * 64) * 8]), va[j]);
#pragma unroll
        for (int j = 0; j < OB::LPT; ++j) load_lds_b128(rb, lds_addr(&Bs[st][(j * 256 + wave * 64) * 8]), vb[j]);
    };

    f32x16 acc[2][NBJ];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) acc[bi][bj] = f32x16{};

    const int nk = (k_end - k_begin) / BK;
    if (nk > 0) issue(0, k_begin);
    for (int i = 0; i < nk; ++i) {
        const int st = i & 1;
        wait_vmcnt<0>();  // this wave's share of step i has landed ...
        __syncthreads();  // ... and every wave's; every wave is done with stage st ^ 1
        if (i + 1 < nk) issue(st ^ 1, k_begin + (i + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8 ao[2], bo[NBJ];
#pragma unroll
            for (int bi = 0; bi < 2; ++bi) ao[bi] = OA::read(As[st], wm * 64 + 32 * bi, ks, lane);
#pragma unroll
            for (int bj = 0; bj < NBJ; ++bj) bo[bj] = OB::read(Bs[st], wn * WN + 32 * bj, ks, lane);
#pragma unroll
            for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                for (int bj = 0; bj < NBJ; ++bj) acc[bi][bj] = mfma_bf16(ao[bi], bo[bj], acc[bi][bj]);
        }
    }
    wait_vmcnt<0>();  // nothing may still be writing LDS when the workgroup ends

    // Epilogue: lane holds column l32 of each 32 x 32 block, rows 8 (r / 4) + 4 half + r % 4.
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) {
            const int col = n0 + wn * WN + 32 * bj + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 64 + 32 * bi + 8 * (r / 4) + 4 * half + (r % 4);
                float v = acc[bi][bj][r] * a.alpha;
                if constexpr (EPI == kEpiScores)
                    if (col >= a.n_valid || (a.causal && col > row)) v = -INFINITY;
                if (row < a.M) C[(size_t)row * a.ldc + col] = (__bf16)v;
            }
        }
}

// One kernel name per product, so profiles tell them apart.
__global__ __launch_bounds__(256) void std_scores_kernel(StdGemmArgs a) {  // S = scale Q K^T
    std_gemm<true, true, 128, kRangeFull, kEpiScores>(a);
}
__global__ __launch_bounds__(256) void std_dp_kernel(StdGemmArgs a) {  // dP = dO V^T
    std_gemm<true, true, 128, kRangeFull, kEpiZeroAbove>(a);
}
template <int D>
__global__ __launch_bounds__(256) void std_pv_kernel(StdGemmArgs a) {  // O = P V
    std_gemm<true, false, D, kRangeUpToRow, kEpiPlain>(a);
}
template <int D>
__global__ __launch_bounds__(256) void std_dq_kernel(StdGemmArgs a) {  // dQ = scale dS K
    std_gemm<true, false, D, kRangeUpToRow, kEpiPlain>(a);
}
template <int D>
__global__ __launch_bounds__(256) void std_dv_kernel(StdGemmArgs a) {  // dV = P^T dO
    std_gemm<false, false, D, kRangeFromRow, kEpiPlain>(a);
}
template <int D>
__global__ __launch_bounds__(256) void std_dk_kernel(StdGemmArgs a) {  // dK = scale dS^T Q
    std_gemm<false, false, D, kRangeFromRow, kEpiPlain>(a);
}

template <typename Kernel>
hipError_t gemm(Kernel kernel, const StdGemmArgs& g, int heads, hipStream_t st) {
    const long long grid = (long long)heads * ((g.M + kStdBM - 1) / kStdBM) * g.ntiles_n;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), 0, st, g);
    return hipGetLastError();
}

}  // namespace

int std_ld(int N) { return (N + kStdBM - 1) / kStdBM * kStdBM; }

hipError_t launch_std_fwd(const StdArgs& a, hipStream_t st) {
    const int heads = a.B * a.H, N = a.N, d = a.d, Np = std_ld(N);
    const int Kq = (N + kStdBK - 1) / kStdBK * kStdBK;  // keys rounded up to whole k-steps
    hipError_t e;
    // 1. S = scale Q K^T into P's buffer; keys >= N and (causal) key > query get -inf.
    StdGemmArgs s{(const __bf16*)a.q, (const __bf16*)a.k, (__bf16*)a.p, (long long)N * d, (long long)N * d,
                  (long long)N * Np, d, d, Np, N, N, N, Np / kStdBM, d, N, a.causal, a.scale};
    if ((e = gemm(std_scores_kernel, s, heads, st)) != hipSuccess) return e;
    // 2. P = softmax(S) in place, with lse.
    SoftmaxArgs sm{a.p, a.p, a.lse, (long long)heads * N, Np, kBF16};
    if ((e = launch_softmax(sm, st)) != hipSuccess) return e;
    // 3. O = P V.
    StdGemmArgs pv{(const __bf16*)a.p, (const __bf16*)a.v, (__bf16*)a.o, (long long)N * Np, (long long)N * d,
                   (long long)N * d, Np, d, d, N, N, N, 1, Kq, N, a.causal, 1.0f};
    return d == 128 ? gemm(std_pv_kernel<128>, pv, heads, st) : gemm(std_pv_kernel<64>, pv, heads, st);
}

hipError_t launch_std_bwd(const StdArgs& a, hipStream_t st) {
    const int heads = a.B * a.H, N = a.N, d = a.d, Np = std_ld(N);
    const int Kq = (N + kStdBK - 1) / kStdBK * kStdBK;
    const long long sT = (long long)N * d, sP = (long long)N * Np;
    hipError_t e;
    // 1. dV = P^T dO (rows = keys; the reduction runs over queries).
    StdGemmArgs dv{(const __bf16*)a.p, (const __bf16*)a.dout, (__bf16*)a.dv, sP, sT, sT, Np, d, d, N, N, N, 1, Kq,
                   N, a.causal, 1.0f};
    if ((e = d == 128 ? gemm(std_dv_kernel<128>, dv, heads, st) : gemm(std_dv_kernel<64>, dv, heads, st)) !=
        hipSuccess)
        return e;
    // 2. dP = dO V^T into the workspace.
    StdGemmArgs dp{(const __bf16*)a.dout, (const __bf16*)a.v, (__bf16*)a.dp, sT, sT, sP, d, d, Np, N, N, N,
                   Np / kStdBM, d, N, a.causal, 1.0f};
    if ((e = gemm(std_dp_kernel, dp, heads, st)) != hipSuccess) return e;
    // 3. dS = P o (dP - rowsum(P o dP)), in place over dP.
    SoftmaxArgs sg{a.p, a.dp, nullptr, (long long)heads * N, Np, kBF16};
    if ((e = launch_softmax_grad(sg, st)) != hipSuccess) return e;
    // 4. dQ = scale dS K.
    StdGemmArgs dq{(const __bf16*)a.dp, (const __bf16*)a.k, (__bf16*)a.dq, sP, sT, sT, Np, d, d, N, N, N, 1, Kq,
                   N, a.causal, a.scale};
    if ((e = d == 128 ? gemm(std_dq_kernel<128>, dq, heads, st) : gemm(std_dq_kernel<64>, dq, heads, st)) !=
        hipSuccess)
        return e;
    // 5. dK = scale dS^T Q.
    StdGemmArgs dk{(const __bf16*)a.dp, (const __bf16*)a.q, (__bf16*)a.dk, sP, sT, sT, Np, d, d, N, N, N, 1, Kq,
                   N, a.causal, a.scale};
    return d == 128 ? gemm(std_dk_kernel<128>, dk, heads, st) : gemm(std_dk_kernel<64>, dk, heads, st);
}

}  // namespace fa
