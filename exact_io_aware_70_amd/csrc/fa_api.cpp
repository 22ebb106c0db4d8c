// C ABI of libfa.so: argument validation, workspace sizing and dispatch to the kernel
// launchers.  Validation touches no HIP API, so every error path below can be exercised
// on a machine without a GPU; nothing is enqueued unless all checks pass.
#include "../../include/fa.h"

#include <stdint.h>

#include <cmath>

#include "fa_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxN = FA_MAX_N;
constexpr long long kMaxTiles = FA_MAX_TILES;  // B * H * ceil(N / 64)

// Checks shared by the forward and backward entry points.
int check_common(int B, int H, int N, int d, float scale, int dtype) {
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (!(scale > 0.0f) || !std::isfinite(scale)) return FA_ERR_UNSUPPORTED;
    // Row and key indices stay far from int overflow (the kernels form N + 128 and the like).
    if (N > kMaxN) return FA_ERR_SHAPE;
    // The attention kernels launch one 256-thread workgroup per (batch, head, tile of at least
    // 64 rows); a dispatch holds fewer than 2^32 work-items, so fewer than 2^24 workgroups.
    const long long tiles = (long long)B * H * (((long long)N + 63) / 64);
    if (tiles > kMaxTiles) return FA_ERR_SHAPE;
    return FA_OK;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    const int st = check_common(B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal ? 1 : 0, dtype};
    const hipError_t e = fa::launch_fwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d, int dtype) {
    if (check_common(B, H, N, d, 1.0f, dtype) != FA_OK) return 0;
    // D_i = rowsum(dout * o) and lse * log2(e): one float each per (batch, head, row).
    return 2 * round_up((size_t)B * H * N * sizeof(float), 256);
}

// Pointer, size and alignment checks of the backward entry points (workspace aside).
static int bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                     int dtype) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
    const int st = check_common(B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    return FA_OK;
}

static int bwd_common(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                      int causal, int dtype, void* workspace, size_t workspace_bytes, void* stream,
                      void* const* events) {
    const int st = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, H, N, d, dtype) || !aligned(workspace, 256))
        return FA_ERR_WORKSPACE;
    float* delta = static_cast<float*>(workspace);
    float* lse2 = delta + round_up((size_t)B * H * N * sizeof(float), 256) / sizeof(float);
    fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal ? 1 : 0, dtype, delta, lse2, events};
    const hipError_t e = fa::launch_bwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
           void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, workspace,
                      workspace_bytes, stream, nullptr);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                   void* stream) {
    const int st = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    const size_t need = fa_bwd_workspace_size(B, H, N, d, dtype);
    if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
    void* ws = nullptr;
    if (fa::scratch_address(static_cast<hipStream_t>(stream), &ws) != hipSuccess) return FA_ERR_HIP;
    return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, ws,
                      FA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int fa_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    if (!events) return FA_ERR_NULL;
    for (int i = 0; i <= FA_BWD_LAUNCHES; ++i)
        if (!events[i]) return FA_ERR_NULL;
    return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, workspace,
                      workspace_bytes, stream, events);
}

// Dropout parameters: p in [0, 1); threshold t = round(256 p); key from the 64-bit seed.
// An element is kept with probability (256 - t) / 256 exactly, so kept values are scaled by
// 256 / (256 - t), which makes the expected keep factor exactly 1 (0 when t = 256: nothing
// is kept).
static bool make_dropout(float p, unsigned long long seed, unsigned offset, fa::DropoutArgs* d) {
    if (!(p >= 0.0f && p < 1.0f)) return false;
    const double t = std::floor(256.0 * (double)p + 0.5);
    d->k0 = (uint32_t)(seed & 0xffffffffull);
    d->k1 = (uint32_t)(seed >> 32);
    d->offset = offset;
    d->thr = (uint32_t)(t < 0.0 ? 0.0 : (t > 256.0 ? 256.0 : t));
    d->inv_keep = d->thr < 256 ? 256.0f / (float)(256 - d->thr) : 0.0f;
    return true;
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, int dtype, float dropout_p, unsigned long long seed, unsigned offset,
                   void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    const int st = check_common(B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    fa::DropoutArgs dr{};
    if (dtype != FA_BF16 || !make_dropout(dropout_p, seed, offset, &dr)) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal ? 1 : 0, dtype, dropout_p > 0.0f ? 1 : 0, dr};
    const hipError_t e = fa::launch_fwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                   float dropout_p, unsigned long long seed, unsigned offset, void* workspace,
                   size_t workspace_bytes, void* stream, void* const* events) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
    const int st = check_common(B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    fa::DropoutArgs dr{};
    if (dtype != FA_BF16 || !make_dropout(dropout_p, seed, offset, &dr)) return FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, H, N, d, dtype) || !aligned(workspace, 256))
        return FA_ERR_WORKSPACE;
    if (events)
        for (int i = 0; i <= FA_BWD_LAUNCHES; ++i)
            if (!events[i]) return FA_ERR_NULL;
    float* delta = static_cast<float*>(workspace);
    float* lse2 = delta + round_up((size_t)B * H * N * sizeof(float), 256) / sizeof(float);
    fa::BwdArgs a{q,     k,    v,   o,     dout,  lse,   dq,  dk,    dv,    B,      H,
                  N,     d,    scale, causal ? 1 : 0, dtype, delta, lse2, events, dropout_p > 0.0f ? 1 : 0, dr};
    const hipError_t e = fa::launch_bwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_descale, const float* k_descale,
               const float* v_descale, void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
               void* stream) {
    if (!q8 || !k8 || !v8 || !q_descale || !k_descale || !v_descale || !o || !lse) return FA_ERR_NULL;
    const int st = check_common(B, H, N, d, scale, FA_BF16);
    if (st != FA_OK) return st;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
        !aligned(q_descale, 4) || !aligned(k_descale, 4) || !aligned(v_descale, 4))
        return FA_ERR_ALIGN;
    fa::Fp8FwdArgs a{q8, k8, v8, q_descale, k_descale, v_descale, o, lse, B, H, N, d, scale, causal ? 1 : 0};
    const hipError_t e = fa::launch_fwd_fp8(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_softmax_rows(const void* x, void* y, float* lse, long long rows, int cols, int dtype, void* stream) {
    if (!x || !y) return FA_ERR_NULL;
    // One workgroup per row at most: keep the 1-D grid in range.
    if (rows < 1 || cols < 1 || rows > 0x7fffffffLL) return FA_ERR_SHAPE;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(y, 16) || (lse && !aligned(lse, 4))) return FA_ERR_ALIGN;
    fa::SoftmaxArgs a{x, y, lse, rows, cols, dtype};
    const hipError_t e = fa::launch_softmax(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_std_ld(int N) { return N < 1 || N > FA_STD_MAX_N ? 0 : fa::std_ld(N); }

size_t fa_std_matrix_bytes(int B, int H, int N) {
    if (B < 1 || H < 1 || N < 1 || N > FA_STD_MAX_N) return 0;
    return (size_t)B * H * N * fa::std_ld(N) * 2;
}

// Checks shared by the standard-attention entry points.
static int std_check(int B, int H, int N, int d, float scale, int dtype) {
    const int st = check_common(B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (N > FA_STD_MAX_N) return FA_ERR_SHAPE;
    return FA_OK;
}

int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* p, int B, int H, int N,
               int d, float scale, int causal, int dtype, void* stream) {
    if (!q || !k || !v || !o || !lse || !p) return FA_ERR_NULL;
    const int st = std_check(B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(p, 16) ||
        !aligned(lse, 4))
        return FA_ERR_ALIGN;
    fa::StdArgs a{q, k, v, nullptr, o, p, nullptr, lse, nullptr, nullptr, nullptr, B, H, N, d, scale,
                  causal ? 1 : 0};
    const hipError_t e = fa::launch_std_fwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_std_bwd(const void* q, const void* k, const void* v, const void* dout, const void* p, void* dq, void* dk,
               void* dv, void* dp, int B, int H, int N, int d, float scale, int causal, int dtype, void* stream) {
    if (!q || !k || !v || !dout || !p || !dq || !dk || !dv || !dp) return FA_ERR_NULL;
    const int st = std_check(B, H, N, d, scale, dtype);
    if (st != FA_OK) return st;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) || !aligned(p, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dp, 16))
        return FA_ERR_ALIGN;
    fa::StdArgs a{q, k, v, dout, nullptr, const_cast<void*>(p), dp, nullptr, dq, dk, dv, B, H, N, d, scale,
                  causal ? 1 : 0};
    const hipError_t e = fa::launch_std_bwd(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK: success";
        case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE: sizes must be >= 1, N <= 2^30 and B*H*ceil(N/64) < 2^24";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: d must be 64 or 128, dtype FA_F32 or FA_BF16, scale finite and > 0 (dropout: bf16, 0 <= p < 1; FP8: d = 128)";
        case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointers must be 16-byte aligned (lse 4-byte)";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing, misaligned or smaller than fa_bwd_workspace_size()";
        case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected a kernel launch";
        case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: fa_bwd_noalloc needs more than its static scratch (FA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown fa_status code";
    }
}

int fa_version(void) { return FA_VERSION; }

}  // extern "C"
