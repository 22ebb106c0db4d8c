// Row-wise softmax with its logsumexp (gfx950): the online-softmax primitive on its own.
//
// "How FlashAttention Actually Works" -- "The Secret Weapon: Online Softmax": a row's
// softmax needs its maximum (subtracted before exponentiating, so nothing overflows) and
// the sum of the exponentials, and both can be kept as a running pair over blocks;
// "How does FlashAttention optimize memory and speed via tiling?" -- "Core Technical
// Innovations", item 2, gives the merge of two such pairs,
//     m = max(m1, m2),  l = e^{m1 - m} l1 + e^{m2 - m} l2.
//
// Work split: a team of TEAM lanes (one wave, or a whole 256-thread workgroup) owns one
// row and reads it as 16-byte vectors of the flat [rows, cols] array, lane t taking vectors
// t, t + TEAM, ...; consecutive lanes read consecutive vectors, so every wave load is one
// contiguous KiB.  Rows need not start on a 16-byte boundary: the first and last vectors
// of a row may hold a neighbour's elements, which are masked to -inf on load and never
// stored (those two vectors are stored element by element).
//   - Cached path (the row fits in the team's registers): the row is read once and kept as
//     raw 16-byte words, its maximum and sum reduced over the team, and the outputs
//     written from registers: one HBM read and one write per element.
//   - Streaming path (longer rows): each lane folds its vectors into a running (max, sum)
//     pair chunk by chunk with the merge above, the team merges the lanes' pairs the same
//     way, and a second pass re-reads the row to write the outputs.
// A row with no finite entry (all -inf) has no softmax; its outputs and lse are NaN.  This
// file is built with NaN semantics honoured (unlike the attention kernels) so that holds.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
    static constexpr int VE = 4;  // elements per 16-byte vector
    __device__ static float get(const float* p) { return *p; }
    __device__ static void put(float* p, float v) { *p = v; }
    // Whole-vector casts: per-element bit casts of a u32x4 were compiled into copies of
    // element 0 on this path.
    __device__ static void unpack(u32x4 raw, float (&f)[4]) {
        const f32x4 v = __builtin_bit_cast(f32x4, raw);
        f[0] = v.x;
        f[1] = v.y;
        f[2] = v.z;
        f[3] = v.w;
    }
    __device__ static u32x4 pack(const float (&f)[4]) {
        const f32x4 v = {f[0], f[1], f[2], f[3]};
        return __builtin_bit_cast(u32x4, v);
    }
};
template <>
struct Vec16<__bf16> {
    static constexpr int VE = 8;
    __device__ static float get(const __bf16* p) { return (float)*p; }
    __device__ static void put(__bf16* p, float v) { *p = (__bf16)v; }
    __device__ static void unpack(u32x4 raw, float (&f)[8]) {
        // bf16 -> fp32 is a 16-bit shift of the bit pattern.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = __builtin_bit_cast(float, raw[e] << 16);
            f[2 * e + 1] = __builtin_bit_cast(float, raw[e] & 0xffff0000u);
        }
    }
    __device__ static u32x4 pack(const float (&f)[8]) {
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const __bf16 lo = (__bf16)f[2 * e], hi = (__bf16)f[2 * e + 1];
            r[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        return r;
    }
};

// -inf in each element of a vector, as raw bits.
template <typename T>
__device__ __forceinline__ uint32_t neg_inf_word();
template <>
__device__ __forceinline__ uint32_t neg_inf_word<float>() { return 0xff800000u; }
template <>
__device__ __forceinline__ uint32_t neg_inf_word<__bf16>() { return 0xff80ff80u; }

// One row as seen by its team: flat element range [e0, e1) of an array of `total`
// elements, vectors v0 .. v0 + nv - 1 (vector v covers elements v * VE .. v * VE + VE - 1).
// Vectors are kept as raw 16-byte words (4 registers each) and unpacked to fp32 only while
// a pass works on them; entries outside the row hold the bits of -inf.
template <typename T>
struct Row {
    static constexpr int VE = Vec16<T>::VE;
    static constexpr int EB = 16 / VE * 8;  // bits per element
    long long e0, e1, total, v0;
    int nv;
    __device__ Row(long long r, int cols, long long rows) {
        e0 = r * cols;
        e1 = e0 + cols;
        total = rows * cols;
        v0 = e0 / VE;
        nv = (int)((e1 - 1) / VE - v0 + 1);
    }
    // Replace the bits of element e of a raw vector by those of -inf.
    __device__ static void mask_elem(u32x4& w, int e) {
        if constexpr (VE == 4) {
            w[e] = 0xff800000u;
        } else {
            const int k = e >> 1, sh = (e & 1) * 16;
            w[k] = (w[k] & ~(0xffffu << sh)) | (0xff80u << sh);
        }
    }
    // Vector j of the row, raw, entries outside the row set to -inf.  Whole vectors are read
    // with one 16-byte load; only the array's last vector, which may run past the end of the
    // allocation, is read element by element.
    __device__ u32x4 load(const T* x, int j) const {
        const long long vb = (v0 + j) * VE;
        u32x4 w;
        if (vb + VE <= total) {
            w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + vb));
        } else {
            const uint32_t ni = neg_inf_word<T>();
            w = u32x4{ni, ni, ni, ni};
            const uint16_t* xs = reinterpret_cast<const uint16_t*>(x + vb);
            const uint32_t* xw = reinterpret_cast<const uint32_t*>(x + vb);
#pragma unroll
            for (int e = 0; e < VE; ++e)
                if (vb + e < total) {
                    if constexpr (VE == 4) {
                        w[e] = xw[e];
                    } else {
                        const int k = e >> 1, sh = (e & 1) * 16;
                        w[k] = (w[k] & ~(0xffffu << sh)) | ((uint32_t)xs[e] << sh);
                    }
                }
        }
        if (vb < e0 || vb + VE > e1) {
#pragma unroll
            for (int e = 0; e < VE; ++e)
                if (vb + e < e0 || vb + e >= e1) mask_elem(w, e);
        }
        return w;
    }
    // Store the entries of vector j that belong to the row.
    __device__ void store(T* y, int j, const float (&f)[VE]) const {
        const long long vb = (v0 + j) * VE;
        if (vb >= e0 && vb + VE <= e1) {
            __builtin_nontemporal_store(Vec16<T>::pack(f), reinterpret_cast<u32x4*>(y + vb));
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e)
                if (vb + e >= e0 && vb + e < e1) Vec16<T>::put(y + vb + e, f[e]);
        }
    }
};

// Reductions over a team of TEAM lanes (64: the wave; 256: the workgroup, through LDS).
template <int TEAM>
__device__ __forceinline__ float team_max(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if constexpr (TEAM == 256) {
        const int w = threadIdx.x >> 6;
        __syncthreads();  // earlier readers of red are done
        if ((threadIdx.x & 63) == 0) red[w] = v;
        __syncthreads();
        v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    return v;
}
template <int TEAM>
__device__ __forceinline__ float team_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if constexpr (TEAM == 256) {
        const int w = threadIdx.x >> 6;
        __syncthreads();
        if ((threadIdx.x & 63) == 0) red[w] = v;
        __syncthreads();
        v = (red[0] + red[1]) + (red[2] + red[3]);
    }
    return v;
}

template <typename T>
__device__ __forceinline__ float vmax(u32x4 w, float m) {
    float f[Vec16<T>::VE];
    Vec16<T>::unpack(w, f);
#pragma unroll
    for (int e = 0; e < Vec16<T>::VE; ++e) m = fmaxf(m, f[e]);
    return m;
}
template <typename T>
__device__ __forceinline__ float vsum_exp(u32x4 w, float ms, float s) {
    float f[Vec16<T>::VE];
    Vec16<T>::unpack(w, f);
#pragma unroll
    for (int e = 0; e < Vec16<T>::VE; ++e) s += fast_exp2(fmaf(f[e], kLog2e, -ms));
    return s;
}

// KV raw vectors per lane are held (STREAM = false: the whole row; STREAM = true: one chunk
// at a time).  Each 256-thread workgroup serves 256 / TEAM rows.
template <typename T, int TEAM, int KV, bool STREAM>
// Row r = row0 + blockIdx.x * RPW + ...: the host splits very long row ranges over several
// launches (a dispatch holds fewer than 2^32 work-items).
__global__ __launch_bounds__(256) void softmax_rows_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                           float* __restrict__ lse, long long row0, long long rows,
                                                           int cols) {
    constexpr int VE = Vec16<T>::VE;
    constexpr int RPW = 256 / TEAM;
    __shared__ float red[4];
    const int t = threadIdx.x % TEAM;
    const long long r = row0 + (long long)blockIdx.x * RPW + threadIdx.x / TEAM;
    // A team past the last row leaves at once: with TEAM = 256 that is the whole workgroup,
    // and TEAM = 64 reductions stay inside the wave, so no barrier is left waiting.
    if (r >= rows) return;
    const Row<T> row(r, cols, rows);
    const uint32_t ni = neg_inf_word<T>();

    u32x4 w[KV];
    float m = kNegBig, l = 0.f;
    if constexpr (!STREAM) {
#pragma unroll
        for (int j = 0; j < KV; ++j) {
            const int idx = t + j * TEAM;
            w[j] = idx < row.nv ? row.load(x, idx) : u32x4{ni, ni, ni, ni};
        }
#pragma unroll
        for (int j = 0; j < KV; ++j) m = vmax<T>(w[j], m);
        m = team_max<TEAM>(m, red);
        const float ms = m * kLog2e;
#pragma unroll
        for (int j = 0; j < KV; ++j) l = vsum_exp<T>(w[j], ms, l);
        l = team_sum<TEAM>(l, red);
    } else {
        // Pass 1: this lane's running (max, sum) over its vectors, chunk by chunk.
        for (int c0 = 0; c0 < row.nv; c0 += KV * TEAM) {
#pragma unroll
            for (int j = 0; j < KV; ++j) {
                const int idx = c0 + t + j * TEAM;
                w[j] = idx < row.nv ? row.load(x, idx) : u32x4{ni, ni, ni, ni};
            }
            float cm = kNegBig;
#pragma unroll
            for (int j = 0; j < KV; ++j) cm = vmax<T>(w[j], cm);
            const float mn = fmaxf(m, cm), ms = mn * kLog2e;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < KV; ++j) s = vsum_exp<T>(w[j], ms, s);
            l = l * fast_exp2((m - mn) * kLog2e) + s;
            m = mn;
        }
        // Merge the lanes' pairs.
        const float mt = team_max<TEAM>(m, red);
        l = team_sum<TEAM>(l * fast_exp2((m - mt) * kLog2e), red);
        m = mt;
    }

    // l = 0 only when the row has no finite entry: its softmax is 0 / 0.
    const bool empty = !(l > 0.f);
    const float inv = empty ? __builtin_nanf("") : 1.0f / l;
    if (lse && t == 0) lse[r] = empty ? __builtin_nanf("") : m + __logf(l);
    const float ms = m * kLog2e;

    // Write the normalised row (the streaming path re-reads it first).
    for (int c0 = 0; c0 < (STREAM ? row.nv : 1); c0 += KV * TEAM) {
        if constexpr (STREAM) {
#pragma unroll
            for (int j = 0; j < KV; ++j) {
                const int idx = c0 + t + j * TEAM;
                if (idx < row.nv) w[j] = row.load(x, idx);
            }
        }
#pragma unroll
        for (int j = 0; j < KV; ++j) {
            const int idx = c0 + t + j * TEAM;
            if (idx < row.nv) {
                float f[VE];
                Vec16<T>::unpack(w[j], f);
#pragma unroll
                for (int e = 0; e < VE; ++e) f[e] = fast_exp2(fmaf(f[e], kLog2e, -ms)) * inv;
                row.store(y, idx, f);
            }
        }
    }
}

// Backward of the row softmax (the standard-attention baseline's dS step): with P = softmax
// rows in x and the upstream gradient dP in y, D = rowsum(P o dP) and y <- P o (dP - D), in
// place.  Same team layout as the forward kernel: rows that fit (STREAM = false) are read once
// into registers; longer rows are read twice (D, then the outputs).
template <typename T, int TEAM, int KV, bool STREAM>
__global__ __launch_bounds__(256) void softmax_grad_rows_kernel(const T* __restrict__ p, T* __restrict__ g,
                                                                long long row0, long long rows, int cols) {
    constexpr int VE = Vec16<T>::VE;
    constexpr int RPW = 256 / TEAM;
    __shared__ float red[4];
    const int t = threadIdx.x % TEAM;
    const long long r = row0 + (long long)blockIdx.x * RPW + threadIdx.x / TEAM;
    if (r >= rows) return;
    const Row<T> row(r, cols, rows);

    // D over this lane's vectors (entries outside the row read as -inf in P and are skipped).
    auto dot = [&](u32x4 wp, u32x4 wg, float acc) {
        float fp[VE], fg[VE];
        Vec16<T>::unpack(wp, fp);
        Vec16<T>::unpack(wg, fg);
#pragma unroll
        for (int e = 0; e < VE; ++e)
            if (fp[e] != -INFINITY) acc = fmaf(fp[e], fg[e], acc);
        return acc;
    };
    auto out = [&](u32x4 wp, u32x4 wg, float dd, float (&f)[VE]) {
        float fp[VE], fg[VE];
        Vec16<T>::unpack(wp, fp);
        Vec16<T>::unpack(wg, fg);
#pragma unroll
        for (int e = 0; e < VE; ++e) f[e] = fp[e] * (fg[e] - dd);
    };
    u32x4 wp[KV], wg[KV];
    float dsum = 0.f;
    for (int c0 = 0; c0 < (STREAM ? row.nv : 1); c0 += KV * TEAM) {
#pragma unroll
        for (int j = 0; j < KV; ++j) {
            const int idx = c0 + t + j * TEAM;
            if (idx < row.nv) {
                wp[j] = row.load(p, idx);
                wg[j] = row.load(g, idx);
                dsum = dot(wp[j], wg[j], dsum);
            }
        }
    }
    const float dd = team_sum<TEAM>(dsum, red);
    for (int c0 = 0; c0 < (STREAM ? row.nv : 1); c0 += KV * TEAM) {
#pragma unroll
        for (int j = 0; j < KV; ++j) {
            const int idx = c0 + t + j * TEAM;
            if (idx < row.nv) {
                if constexpr (STREAM) {
                    wp[j] = row.load(p, idx);
                    wg[j] = row.load(g, idx);
                }
                float f[VE];
                out(wp[j], wg[j], dd, f);
                row.store(g, idx, f);
            }
        }
    }
}

// Launch shape by row length: short rows get one wave each (four rows per workgroup, no
// barriers); longer rows a whole workgroup holding as few vectors per lane as the row needs
// (fewer registers, more workgroups per CU, more bytes in flight); rows past 2048 vectors
// stream.  Measured on the 65536 x 8192 bf16 workload: 5 vectors per lane beat 8 (5.8 vs
// 5.2 TB/s), and non-temporal loads and stores (the data is touched once) add 6%.
template <typename T, int TEAM, int KV, bool STREAM>
hipError_t launch_shape(const SoftmaxArgs& a, hipStream_t st) {
    constexpr int RPW = 256 / TEAM;
    constexpr long long kMaxGrid = 1LL << 22;  // workgroups per launch (2^30 work-items)
    for (long long r0 = 0; r0 < a.rows; r0 += kMaxGrid * RPW) {
        const long long grid = min((a.rows - r0 + RPW - 1) / RPW, kMaxGrid);
        hipLaunchKernelGGL((softmax_rows_kernel<T, TEAM, KV, STREAM>), dim3((unsigned)grid), dim3(256), 0, st,
                           static_cast<const T*>(a.x), static_cast<T*>(a.y), a.lse, r0, a.rows, a.cols);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t launch_softmax_t(const SoftmaxArgs& a, hipStream_t st) {
    const long long nv_max = a.cols / Vec16<T>::VE + 2;  // vectors a row can touch
    if (nv_max <= 64 * 4) return launch_shape<T, 64, 4, false>(a, st);
    if (nv_max <= 256 * 2) return launch_shape<T, 256, 2, false>(a, st);
    if (nv_max <= 256 * 3) return launch_shape<T, 256, 3, false>(a, st);
    if (nv_max <= 256 * 5) return launch_shape<T, 256, 5, false>(a, st);
    if (nv_max <= 256 * 8) return launch_shape<T, 256, 8, false>(a, st);
    return launch_shape<T, 256, 8, true>(a, st);
}

}  // namespace

hipError_t launch_softmax(const SoftmaxArgs& a, hipStream_t st) {
    return a.dtype == kBF16 ? launch_softmax_t<__bf16>(a, st) : launch_softmax_t<float>(a, st);
}

namespace {
template <typename T, int TEAM, int KV, bool STREAM>
hipError_t launch_grad_shape(const SoftmaxArgs& a, hipStream_t st) {
    constexpr int RPW = 256 / TEAM;
    constexpr long long kMaxGrid = 1LL << 22;
    for (long long r0 = 0; r0 < a.rows; r0 += kMaxGrid * RPW) {
        const long long grid = min((a.rows - r0 + RPW - 1) / RPW, kMaxGrid);
        hipLaunchKernelGGL((softmax_grad_rows_kernel<T, TEAM, KV, STREAM>), dim3((unsigned)grid), dim3(256), 0, st,
                           static_cast<const T*>(a.x), static_cast<T*>(a.y), r0, a.rows, a.cols);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}
}  // namespace

hipError_t launch_softmax_grad(const SoftmaxArgs& a, hipStream_t st) {
    using T = __bf16;
    const long long nv_max = a.cols / Vec16<T>::VE + 2;
    if (nv_max <= 64 * 4) return launch_grad_shape<T, 64, 4, false>(a, st);
    if (nv_max <= 256 * 2) return launch_grad_shape<T, 256, 2, false>(a, st);
    if (nv_max <= 256 * 4) return launch_grad_shape<T, 256, 4, false>(a, st);
    if (nv_max <= 256 * 8) return launch_grad_shape<T, 256, 8, false>(a, st);
    return launch_grad_shape<T, 256, 8, true>(a, st);
}

}  // namespace fa
