/*
 * fa.h -- exact IO-aware self-attention for AMD MI355X (gfx950): the C ABI of libfa.so.
 *
 * Computes O = softmax(scale * Q K^T) V per (batch, head) without ever writing the
 * N x N score or probability matrix to HBM: the forward pass walks key/value tiles
 * with an online (running max, running sum) softmax and keeps only the per-row
 * logsumexp; the backward pass recomputes each score tile from Q, K and that
 * logsumexp instead of reading a stored probability matrix.
 *
 * Sources (page title -- section):
 *   "Breaking the Memory Wall: A Deep Dive into FlashAttention" -- "The Problem: The
 *     Memory Wall" (P = softmax(Q K^T / sqrt(d))), "The Solution: IO-Awareness &
 *     Tiling" items 1-3 (tiling, incremental softmax, backward recomputation from the
 *     saved normalisation factors);
 *   "How does FlashAttention optimize memory and speed via tiling?" -- "Core Technical
 *     Innovations in FlashAttention" (the running max / running sum merge);
 *   "How FlashAttention Actually Works" -- "The Backward Pass: Recomputation".
 *
 * Conventions shared by every entry point
 *   - Tensors q, k, v, o, dout, dq, dk, dv are DEVICE pointers to contiguous
 *     [B, H, N, d] arrays, d fastest, all of element type `dtype`
 *     (FA_F32: IEEE float; FA_BF16: bfloat16 stored as 16-bit words).
 *   - lse is a DEVICE pointer to float [B, H, N]: the natural-log logsumexp of row i
 *     of scale * Q K^T (over its visible keys).
 *   - scale multiplies the logits and is used as given (callers pass 1/sqrt(d)).
 *   - causal != 0 masks key j > query i (square, diagonal visible).
 *   - stream is a hipStream_t (NULL = the default stream).  All work is enqueued on
 *     it in order; no call waits for the GPU, allocates or frees memory, or keeps
 *     state between calls.  The caller owns every buffer.
 *   - Arithmetic: bf16 inputs are multiplied on bf16 MFMA with fp32 accumulation;
 *     probabilities and dS are rounded to bf16 before their products; outputs are
 *     rounded to the input dtype (round to nearest even).  The fp32 path uses fp32
 *     MFMA throughout.
 *   - Supported: B, H, N >= 1; N <= FA_MAX_N (2^30); d in {64, 128};
 *     B*H*ceil(N/64) <= FA_MAX_TILES (2^24 - 1: every attention launch has at most 256
 *     threads per 64 rows, and a dispatch holds fewer than 2^32 work-items).  Sizes outside this return FA_ERR_SHAPE.  Inside it no index or byte
 *     count wraps: tensor offsets are 64-bit, and each range-checked tile load spans only
 *     its own tile.
 *   (fa_softmax_rows, below, has conventions of its own.)
 *   - Errors: arguments are validated before anything is enqueued; on failure a
 *     negative fa_status is returned and nothing runs.  A failed kernel launch returns
 *     FA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *     synchronisation, as for any HIP work.
 *   - Aliasing: outputs must not overlap inputs or each other (not checked).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_VERSION 100 /* 1.0.0 */

#define FA_MAX_N (1 << 30)               /* largest sequence length accepted */
#define FA_MAX_TILES ((1LL << 24) - 1)   /* largest B * H * ceil(N / 64) accepted */

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,        /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,       /* a size < 1, N > FA_MAX_N, or B*H*ceil(N/64) > FA_MAX_TILES */
    FA_ERR_UNSUPPORTED = -3, /* d not in {64, 128} or unknown dtype */
    FA_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned (lse: 4-byte) */
    FA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than fa_bwd_workspace_size() */
    FA_ERR_HIP = -6,         /* the HIP runtime rejected a launch */
    FA_ERR_SCRATCH = -7      /* fa_bwd_noalloc: the sizes need more than the static scratch */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/*
 * Forward pass.  Writes o [B,H,N,d] (dtype) and lse [B,H,N] (float).
 * "Breaking the Memory Wall" -- "The Solution: IO-Awareness & Tiling", items 1-2:
 * K/V tiles are streamed past each query tile, the running max m and running sum l
 * are merged per tile, the unnormalised output is rescaled by e^{m_old - m_new},
 * and O = acc / l, lse = m + ln l at the end.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (>= 256; 0 if the sizes are
 * invalid).  Only the size matters; the contents need no initialisation.  Plumbing: no
 * page defines it.  The workspace holds D_i = rowsum(dout * o) and lse * log2(e), one float
 * each per (batch, head, row), each array rounded up to 256 bytes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d, int dtype);

/*
 * Backward pass for the loss L = sum(O * dout): writes dq, dk, dv [B,H,N,d] (dtype).
 * q, k, v are the forward inputs; o and lse are what fa_fwd wrote for them; dout is
 * dL/dO.  Score tiles are recomputed from q, k and lse ("How FlashAttention Actually
 * Works" -- "The Backward Pass: Recomputation"; "Breaking the Memory Wall" -- item 3).
 * With P = exp(scale q k^T - lse), dP = dout v^T, D_i = rowsum(dout * o)_i and
 * dS = P * (dP - D):  dv = P^T dout,  dq = scale dS k,  dk = scale dS^T q.
 * workspace: device memory of at least fa_bwd_workspace_size() bytes, 256-byte aligned,
 * owned by the caller, not shared with a concurrent call.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The same arguments, checks, kernels and
 * results as fa_bwd, without the workspace: it lives in a static device array of
 * FA_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  The call allocates and
 * frees nothing; its first call on a device looks up that device's copy of the array.
 * Sizes whose fa_bwd_workspace_size() exceeds FA_NOALLOC_SCRATCH_BYTES (B*H*N above about
 * 2^21 rows) return FA_ERR_SCRATCH before anything is enqueued.  All calls on one GPU share
 * its array: calls that overlap on one GPU (concurrent streams, threads) race.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/* Number of kernel launches one fa_bwd call makes: dQ, which also forms D = rowsum(dout * o)
 * and lse * log2(e) into the workspace, then dK/dV. */
#define FA_BWD_LAUNCHES 2

/*
 * fa_bwd with per-launch timing, for profilers and benchmarks: the same arguments, checks
 * and work as fa_bwd, plus `events`, an array of FA_BWD_LAUNCHES + 1 hipEvent_t handles
 * created (and later destroyed) by the caller.  events[i] is recorded on `stream` right
 * before launch i (0: dQ with D, 1: dK/dV) and events[FA_BWD_LAUNCHES] after the last, so
 * hipEventElapsedTime(events[i], events[i + 1]) is the duration of launch i.  A NULL array
 * or NULL handle returns FA_ERR_NULL before anything is enqueued; a failed record returns
 * FA_ERR_HIP.  Same passages as fa_bwd ("How FlashAttention Actually Works" -- "The
 * Backward Pass: Recomputation").
 */
int fa_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, float scale, int causal, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/*
 * Forward and backward passes with dropout on the probabilities ("How FlashAttention
 * Actually Works" -- "The GPU Memory Wall: HBM vs. SRAM": dropout is one of the steps of
 * attention that a fused kernel keeps on chip).  The same arguments and behaviour as fa_fwd / fa_bwd (fa_bwd_timed when
 * `events` is non-NULL), plus:
 *   dropout_p in [0, 1) (FA_ERR_UNSUPPORTED otherwise; p = 0 is plain attention);
 *   seed, offset: the random stream.  Mask of head bh = b * H + h: Philox4x32-10 (Salmon,
 *     Moraes, Dror, Shaw, SC 2011) with counter (j >> 2, i >> 2, bh, offset) and key (seed
 *     mod 2^32, seed >> 32); element (query i, key j) reads byte (j & 3) of output word
 *     (i & 3) and is kept iff that byte >= round(256 dropout_p).
 * An element is kept with probability (256 - t) / 256, t = round(256 dropout_p), and kept
 * values are scaled by 256 / (256 - t) (0 if t = 256), so the keep factor Z has mean 1.
 * O = (P o Z) V; lse is the logsumexp of the undropped scores.  The
 * backward pass regenerates the same mask from (seed, offset): dV = (P o Z)^T dout,
 * dS = P o (Z o (dout V^T) - D).  Pass the forward's seed and offset to the backward.
 * bf16 only (FA_ERR_UNSUPPORTED for FA_F32).
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, int dtype, float dropout_p, unsigned long long seed, unsigned offset,
                   void* stream);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                   float dropout_p, unsigned long long seed, unsigned offset, void* workspace,
                   size_t workspace_bytes, void* stream, void* const* events);

/*
 * FP8 forward pass: the same tiled online-softmax forward as fa_fwd over OCP E4M3 inputs,
 * with both products on the FP8 matrix cores ("Breaking the Memory Wall" -- "The
 * Solution: IO-Awareness & Tiling", items 1-2; "How does FlashAttention optimize memory
 * and speed via tiling?" -- "Interview tips" names FP8 support as a FlashAttention-3
 * addition).
 *   q8, k8, v8: DEVICE pointers to E4M3 codes (1 byte each) [B, H, N, d], 16-byte aligned;
 *     the value of a code of head (b, h) is decode(code) * X_descale[b * H + h].
 *   q_descale, k_descale, v_descale: DEVICE pointers to float [B, H].
 *   o: DEVICE pointer to bf16 [B, H, N, d]; lse: float [B, H, N], the natural-log logsumexp
 *     of scale * (descaled Q) (descaled K)^T over the visible keys.
 * Arithmetic: Q8 K8^T on E4M3 MFMA with fp32 accumulation, times scale * q_descale *
 * k_descale; probabilities exp(s - m) (m a running reference within 8 log2 units of the row
 * maximum, so they stay <= 256) rounded to E4M3 (nearest even) for the P V product and for
 * the row sum; O = (P8 V8) * v_descale / sum(P8), rounded to bf16.
 * Supported: d = 128 only (FA_ERR_UNSUPPORTED otherwise); other conventions as fa_fwd.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_descale, const float* k_descale,
               const float* v_descale, void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
               void* stream);

/*
 * Row-wise softmax of a [rows, cols] array and the logsumexp of each row: the online
 * softmax on its own ("How FlashAttention Actually Works" -- "The Secret Weapon: Online
 * Softmax": subtract the row maximum before exponentiating, keep a running maximum and
 * sum; "How does FlashAttention optimize memory and speed via tiling?" -- "Core Technical
 * Innovations", item 2: the merge of two (max, sum) pairs).
 *   y[r, c] = exp(x[r, c] - m_r) / l_r,  lse[r] = m_r + ln l_r,
 *   m_r = max_c x[r, c],  l_r = sum_c exp(x[r, c] - m_r).
 * x, y: DEVICE pointers to contiguous row-major [rows, cols] arrays of element type `dtype`
 * (FA_F32 or FA_BF16), 16-byte aligned; rows need not start on 16-byte boundaries.  y may
 * equal x (in place); no other overlap is allowed.  lse: DEVICE pointer to float [rows]
 * (4-byte aligned), or NULL to skip it.  -inf entries are allowed and give exact zeros; a
 * row whose entries are all -inf has no softmax and gets NaN outputs and a NaN lse.  x
 * must hold no NaN or +inf.  Arithmetic in fp32; y is rounded to `dtype` (nearest even).
 * A row that fits on chip (up to 16368 bf16 or 8184 fp32 values) is read from HBM once;
 * longer rows are read twice (an online pass, then the normalising pass).
 * Errors: FA_ERR_NULL (x or y NULL), FA_ERR_SHAPE (rows or cols < 1, rows > 2^31 - 1),
 * FA_ERR_UNSUPPORTED (dtype), FA_ERR_ALIGN; nothing is enqueued on failure.  Enqueued on
 * `stream`; no allocation, no synchronisation.
 */
int fa_softmax_rows(const void* x, void* y, float* lse, long long rows, int cols, int dtype, void* stream);

/*
 * Standard (materialising) attention: the baseline the pages compare FlashAttention with,
 * on the same device and harness.  "How FlashAttention Actually Works" -- "The GPU Memory
 * Wall: HBM vs. SRAM": standard attention writes Q K^T to HBM, reads it back for the softmax,
 * writes the probability matrix, and reads it again to multiply by V; its backward pass reads
 * the stored probabilities ("The Backward Pass: Recomputation" describes the alternative).
 * bf16 only (FA_ERR_UNSUPPORTED otherwise), d in {64, 128}, N <= FA_STD_MAX_N.
 *
 * The N x N matrices are bf16 [B, H, N, ld] with ld = fa_std_ld(N) (N rounded up to 128;
 * the padding columns hold 0 in P and dS); fa_std_matrix_bytes() is the size of one.
 *
 * fa_std_fwd: writes S = scale q k^T (-inf where masked) into p, turns it into P = softmax(S)
 *   in place (lse per row), then o = P v.  p is an output the backward pass reads.
 * fa_std_bwd: from the forward's p: dv = P^T dout; dP = dout v^T into `dp` (caller-owned, of
 *   fa_std_matrix_bytes()); dS = P o (dP - rowsum(P o dP)) in place; dq = scale dS k;
 *   dk = scale dS^T q.
 * Layout, dtype, stream, ownership and error conventions as fa_fwd / fa_bwd; p and dp must be
 * 16-byte aligned.  Nothing is allocated; all work is enqueued on `stream`.
 */
#define FA_STD_MAX_N 65536
int fa_std_ld(int N);
size_t fa_std_matrix_bytes(int B, int H, int N);
int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* p,
               int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);
int fa_std_bwd(const void* q, const void* k, const void* v, const void* dout, const void* p,
               void* dq, void* dk, void* dv, void* dp, int B, int H, int N, int d, float scale,
               int causal, int dtype, void* stream);

/* A static, never-NULL description of a status code (unknown codes included).  Plumbing:
 * no page defines it. */
const char* fa_status_string(int status);

/* FA_VERSION of the built library.  Plumbing: no page defines it. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
