// Host-side interface between the C ABI (fa_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// Grids of at most this many 128-row tiles (one round of two workgroups per CU) run the bf16
// d = 128 kernels with two groups of waves per tile, each taking every other sub-tile of the
// tile's walk; the groups' partial results merge on chip.  Measured: 17-25% faster from 64 to
// 512 tiles, slower from 640 up, where the grid already fills the machine.
constexpr long long kSplitTilesAtMost = 512;

// Dropout of the probabilities (see fa_dropout.h): Philox key, counter word 3, 8-bit keep
// threshold (keep iff byte >= thr) and the keep scale 256 / (256 - thr).
struct DropoutArgs {
    uint32_t k0, k1;
    uint32_t offset;
    uint32_t thr;
    float inv_keep;
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, N, d;
    float scale;
    int causal;
    int dtype;
    int dropout;       // nonzero: apply `drop`
    DropoutArgs drop;
};

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    int B, H, N, d;
    float scale;
    int causal;
    int dtype;
    float* delta;  // workspace: D_i = rowsum(dout * o), float [B, H, N]
    float* lse2;   // workspace: lse * log2(e), float [B, H, N]
    void* const* events;  // optional: hipEvent_t recorded before each launch and after the last
    int dropout;          // nonzero: apply `drop`
    DropoutArgs drop;
};

struct Fp8FwdArgs {
    const void* q;  // E4M3 codes [B, H, N, d]
    const void* k;
    const void* v;
    const float* q_descale;  // [B, H]
    const float* k_descale;
    const float* v_descale;
    void* o;  // bf16 [B, H, N, d]
    float* lse;
    int B, H, N, d;
    float scale;
    int causal;
};

struct SoftmaxArgs {
    const void* x;
    void* y;
    float* lse;  // may be null
    long long rows;
    int cols;
    int dtype;
};

// Standard (materialising) attention, bf16: p (and dp) are [B, H, N, std_ld(N)] matrices.
struct StdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;  // backward input
    void* o;           // forward output
    void* p;           // forward: written (scores, then probabilities); backward: read
    void* dp;          // backward: dP, then dS in place
    float* lse;        // forward output
    void* dq;          // backward outputs
    void* dk;
    void* dv;
    int B, H, N, d;
    float scale;
    int causal;
};

// Enqueue the forward / backward / row-softmax kernels on `st`; return hipGetLastError()
// of the launches.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t st);
hipError_t launch_softmax(const SoftmaxArgs& a, hipStream_t st);
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, hipStream_t st);
// y <- P o (y - rowsum(P o y)) for P = x (bf16 only; lse unused).
hipError_t launch_softmax_grad(const SoftmaxArgs& a, hipStream_t st);
hipError_t launch_std_fwd(const StdArgs& a, hipStream_t st);
hipError_t launch_std_bwd(const StdArgs& a, hipStream_t st);
// Row stride (elements) of the standard path's N x N matrices: N rounded up to 128.
int std_ld(int N);

// Device address, on the device of `stream` (the current device for a NULL stream), of the
// library's static backward scratch (fa_noalloc.hip), looked up once per device.
hipError_t scratch_address(hipStream_t stream, void** out);

// Query tiles per (batch, head) of the forward grid.
long long fwd_grid_tiles(int N, int dtype);

}  // namespace fa
