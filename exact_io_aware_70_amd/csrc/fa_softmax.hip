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
//   - Cached path (the row fits in the team's registers): the row is read once, its
//     maximum and sum reduced over the team, and the outputs written from registers: one
//     HBM read and one write per element.
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

// One row as seen by its team: flat element range [e0, e1) of an array of `total`
// elements, vectors v0 .. v0 + nv - 1 (vector v covers elements v * VE .. v * VE + VE - 1).
template <typename T>
struct Row {
    static constexpr int VE = Vec16<T>::VE;
    long long e0, e1, total, v0;
    int nv;
    __device__ Row(long long r, int cols, long long rows) {
        e0 = r * cols;
        e1 = e0 + cols;
        total = rows * cols;
        v0 = e0 / VE;
        nv = (int)((e1 - 1) / VE - v0 + 1);
    }
    // Vector j of the row as floats, entries outside the row set to -inf.  Whole vectors are
    // read with one 16-byte load; only the array's last vector, which may run past the end
    // of the allocation, is read element by element.
    __device__ void load(const T* x, int j, float (&f)[VE]) const {
        const long long vb = (v0 + j) * VE;
        if (vb + VE <= total) {
            Vec16<T>::unpack(*reinterpret_cast<const u32x4*>(x + vb), f);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) f[e] = (vb + e < total) ? Vec16<T>::get(x + vb + e) : -INFINITY;
        }
        if (vb < e0 || vb + VE > e1) {
#pragma unroll
            for (int e = 0; e < VE; ++e)
                if (vb + e < e0 || vb + e >= e1) f[e] = -INFINITY;
        }
    }
    // Store the entries of vector j that belong to the row.
    __device__ void store(T* y, int j, const float (&f)[VE]) const {
        const long long vb = (v0 + j) * VE;
        if (vb >= e0 && vb + VE <= e1) {
            *reinterpret_cast<u32x4*>(y + vb) = Vec16<T>::pack(f);
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

// KV vectors per lane are cached (STREAM = false: the whole row; STREAM = true: one chunk
// at a time).  Each 256-thread workgroup serves 256 / TEAM rows.
template <typename T, int TEAM, int KV, bool STREAM>
__global__ __launch_bounds__(256) void softmax_rows_kernel(const T* __restrict__ x, T* __restrict__ y,
                                                           float* __restrict__ lse, long long rows, int cols) {
    constexpr int VE = Vec16<T>::VE;
    constexpr int RPW = 256 / TEAM;
    __shared__ float red[4];
    const int t = threadIdx.x % TEAM;
    const long long r = (long long)blockIdx.x * RPW + threadIdx.x / TEAM;
    // A team past the last row leaves at once: with TEAM = 256 that is the whole workgroup,
    // and TEAM = 64 reductions stay inside the wave, so no barrier is left waiting.
    if (r >= rows) return;
    const Row<T> row(r, cols, rows);

    float f[KV][VE];
    float m = kNegBig, l = 0.f;
    if constexpr (!STREAM) {
#pragma unroll
        for (int j = 0; j < KV; ++j) {
            const int idx = t + j * TEAM;
            if (idx < row.nv) {
                row.load(x, idx, f[j]);
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) f[j][e] = -INFINITY;
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) m = fmaxf(m, f[j][e]);
        }
        m = team_max<TEAM>(m, red);
        const float ms = m * kLog2e;
#pragma unroll
        for (int j = 0; j < KV; ++j)
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                f[j][e] = fast_exp2(fmaf(f[j][e], kLog2e, -ms));
                l += f[j][e];
            }
        l = team_sum<TEAM>(l, red);
    } else {
        // Pass 1: this lane's running (max, sum) over its vectors, chunk by chunk.
        for (int c0 = 0; c0 < row.nv; c0 += KV * TEAM) {
            float cm = kNegBig;
#pragma unroll
            for (int j = 0; j < KV; ++j) {
                const int idx = c0 + t + j * TEAM;
                if (idx < row.nv) {
                    row.load(x, idx, f[j]);
                } else {
#pragma unroll
                    for (int e = 0; e < VE; ++e) f[j][e] = -INFINITY;
                }
#pragma unroll
                for (int e = 0; e < VE; ++e) cm = fmaxf(cm, f[j][e]);
            }
            const float mn = fmaxf(m, cm), ms = mn * kLog2e;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < KV; ++j)
#pragma unroll
                for (int e = 0; e < VE; ++e) s += fast_exp2(fmaf(f[j][e], kLog2e, -ms));
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

    if constexpr (!STREAM) {
#pragma unroll
        for (int j = 0; j < KV; ++j) {
            const int idx = t + j * TEAM;
            if (idx < row.nv) {
#pragma unroll
                for (int e = 0; e < VE; ++e) f[j][e] *= inv;
                row.store(y, idx, f[j]);
            }
        }
    } else {
        // Pass 2: re-read and write the normalised row.
        const float ms = m * kLog2e;
        for (int c0 = 0; c0 < row.nv; c0 += KV * TEAM) {
#pragma unroll
            for (int j = 0; j < KV; ++j) {
                const int idx = c0 + t + j * TEAM;
                if (idx < row.nv) row.load(x, idx, f[j]);
            }
#pragma unroll
            for (int j = 0; j < KV; ++j) {
                const int idx = c0 + t + j * TEAM;
                if (idx < row.nv) {
#pragma unroll
                    for (int e = 0; e < VE; ++e) f[j][e] = fast_exp2(fmaf(f[j][e], kLog2e, -ms)) * inv;
                    row.store(y, idx, f[j]);
                }
            }
        }
    }
}

template <typename T>
hipError_t launch_softmax_t(const SoftmaxArgs& a, hipStream_t st) {
    constexpr int VE = Vec16<T>::VE;
    const long long nv_max = a.cols / VE + 2;  // vectors a row can touch
    const T* x = static_cast<const T*>(a.x);
    T* y = static_cast<T*>(a.y);
    if (nv_max <= 64 * 4) {
        const long long grid = (a.rows + 3) / 4;
        hipLaunchKernelGGL((softmax_rows_kernel<T, 64, 4, false>), dim3((unsigned)grid), dim3(256), 0, st, x, y,
                           a.lse, a.rows, a.cols);
    } else if (nv_max <= 256 * 8) {
        hipLaunchKernelGGL((softmax_rows_kernel<T, 256, 8, false>), dim3((unsigned)a.rows), dim3(256), 0, st, x, y,
                           a.lse, a.rows, a.cols);
    } else {
        hipLaunchKernelGGL((softmax_rows_kernel<T, 256, 8, true>), dim3((unsigned)a.rows), dim3(256), 0, st, x, y,
                           a.lse, a.rows, a.cols);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_softmax(const SoftmaxArgs& a, hipStream_t st) {
    return a.dtype == kBF16 ? launch_softmax_t<__bf16>(a, st) : launch_softmax_t<float>(a, st);
}

}  // namespace fa
