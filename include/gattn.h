/*
 * gattn — causal multi-head scaled dot-product self-attention for MI355X (gfx950).
 *
 * What is computed (per batch b and head h, independently: heads run in
 * parallel, "Let's build GPT" summary page, timestamp 1:22:27):
 *
 *   S[i][j] = scale * sum_d Q[i][d] * K[j][d]     affinity of query i with key j
 *                                                 (1:04:00-1:06:16); scale is
 *                                                 normally 1/sqrt(hs) (1:17:18)
 *   S[i][j] = -inf for j > i                      lower-triangular tril mask, the
 *                                                 diagonal kept (48:54, 55:20)
 *   P[i][:] = softmax(S[i][:])                    each row sums to one (51:04)
 *   O[i][:] = sum_j P[i][j] * V[j][:]             the value is what gets passed on
 *                                                 (1:10:15)
 *   lse[i]  = ln sum_{j<=i} exp(S[i][j])          natural log, float32
 *
 * The backward (the pages only say the model is trained by backprop) is the
 * chain rule of the above: with D[i] = sum_d dO[i][d] * O[i][d],
 * dS[i][j] = P[i][j] * (dO[i].V[j] - D[i]),
 *   dV[j] = sum_{i>=j} P[i][j] dO[i],  dQ[i] = scale * sum_{j<=i} dS[i][j] K[j],
 *   dK[j] = scale * sum_{i>=j} dS[i][j] Q[i].
 *
 * Layout: the plain entry points take every tensor contiguous (B, H, T, hs),
 * row-major, hs innermost; the *_strided entry points take element strides
 * {batch, head, row} for each group of tensors (hs always contiguous), so the
 * fused projection output (B, T, 3C) and a (B, T, C) output are used in place.
 * lse and D are always contiguous (B, H, T) float32.  The T x T mask is never
 * materialised.
 *
 * Dtypes: q, k, v, o, dO, dq, dk, dv all have `dtype`; lse is always float32.
 *   GATTN_BF16: hs in {32, 64}; MFMA kernels, bf16 inputs/outputs, float32
 *               accumulation, every float32 -> bf16 conversion rounds to
 *               nearest even.  The backward's dS products (dq = scale dS k,
 *               dk = scale dS^T q) take fp16 operands: dS keeps 11
 *               significant bits instead of bf16's 8, and q and k are
 *               converted to fp16, exactly for magnitudes in
 *               [2^-14, 65504] (smaller ones keep 2^-24 absolute precision,
 *               larger ones become inf); |dS| must stay below 65504.
 *   GATTN_F16 : IEEE binary16 (the pages' other half-precision option), same
 *               kernels and rules as GATTN_BF16 with the fp16 MFMA; the
 *               softmax weights stay <= 256 and are stored to fp16 only as
 *               MFMA operands, so no intermediate overflows; outputs whose
 *               magnitude exceeds 65504 become inf, as any fp16 store does.
 *   GATTN_F32 : any hs in [1, 128]; float32 throughout (deterministic).
 *
 * Ownership: every pointer is a device pointer owned by the caller.  The
 * library allocates nothing and keeps no state; calls are re-entrant.  Work is
 * enqueued on `stream` (0 = the null stream) and the call returns without
 * waiting; buffers must stay alive until that stream has finished it.
 * Outputs (o, lse, dq, dk, dv, workspace) are overwritten, never accumulated,
 * and must not alias any input.
 *
 * Errors: every function returns a gattn_status.  All argument checks run
 * before any HIP call, so an invalid call enqueues nothing.  INVALID_ARG: a
 * required pointer is NULL or not 16-byte aligned, B, H or T < 1, hs < 1,
 * scale not finite or <= 0, B*H*T*hs >= 2^31, dtype unknown, or, for bf16
 * and fp16, (T + 256) * hs * 2 >= 2^31 (one slice's rows, plus the tile
 * boundary past T, addressed with 32-bit byte offsets).
 * UNSUPPORTED: bf16 or fp16 with hs not in {32, 64}, or f32 with hs > 128.
 * WORKSPACE: workspace NULL, not 256-byte aligned, or smaller than
 * gattn_bwd_workspace_bytes().
 * HIP: a kernel launch failed (the HIP error is not cleared from the caller's
 * view beyond what hipLaunchKernel itself reports).
 */
#ifndef GATTN_H
#define GATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GATTN_F32 = 0, GATTN_BF16 = 1, GATTN_F16 = 2 } gattn_dtype;

typedef enum {
  GATTN_OK = 0,
  GATTN_ERR_INVALID_ARG = 1,
  GATTN_ERR_UNSUPPORTED = 2,
  GATTN_ERR_WORKSPACE = 3,
  GATTN_ERR_HIP = 4
} gattn_status;

/*
 * Forward: o = softmax(mask_causal(scale * q k^T)) v, and lse.
 * Passages: tril mask and -inf fill (48:54, 55:20), row softmax (51:04),
 * query.key affinity scaled by 1/sqrt(head size) (1:06:16, 1:17:18), weighted
 * sum of values (1:10:15), one head per (b, h) (1:22:27).
 *   q, k, v : inputs, (B, H, T, hs), `dtype`.
 *   o       : output, (B, H, T, hs), `dtype`.
 *   lse     : output, (B, H, T) float32, natural log; may be NULL when no
 *             backward will follow (inference).
 *   scale   : multiplier of q.k (> 0, finite), normally 1/sqrt(hs).
 */
int gattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int T, int hs, float scale, int dtype, hipStream_t stream);

/*
 * Forward on strided tensors: as gattn_fwd, with element (b, h, t, d) of q, k
 * and v at b*s[0] + h*s[1] + t*s[2] + d for s = qkv_strides (one stride set
 * shared by q, k and v, each from its own base pointer), and of o for
 * s = o_strides; lse stays contiguous (B, H, T).  A NULL stride pointer means
 * the contiguous layout {H*T*hs, T*hs, hs}.  Example, the attention of a GPT
 * block with C = H*hs: qkv_strides = {T*3C, hs, 3C} with q = qkv, k = qkv + C,
 * v = qkv + 2C (elements) reads the (B, T, 3C) output of the fused projection
 * directly, and o_strides = {T*C, hs, C} writes o as (B, T, C).
 * Extra INVALID_ARG cases: a stride < 0, a row stride < hs (rows overlap), a
 * stride whose byte size is not a multiple of 16, or (T + 256) rows of one
 * slice spanning 2^31 bytes or more.  The caller is responsible for o not
 * overlapping itself across heads or batches (any layout of distinct rows is
 * accepted) and for o not aliasing q, k or v.
 */
int gattn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int T, int hs, float scale, int dtype,
                      const int64_t* qkv_strides, const int64_t* o_strides, hipStream_t stream);

/*
 * Forward of the newest Tq tokens against Tk >= Tq keys: decoding with the
 * keys and values of earlier tokens kept.  Query i is the token at position
 * Tk - Tq + i of the key sequence and sees keys j <= Tk - Tq + i (the tril
 * mask, 48:54 / 55:20, aligned on the newest token).  The pages' generate
 * recomputes the whole forward for every new token instead ("nanoGPT" notes,
 * section 5: no key/value cache); the rows computed here are the last Tq rows
 * of that forward.  Tq = Tk is the causal forward.
 *   q, o    : (B, H, Tq, hs), `dtype`, strides q_strides / o_strides.
 *   k, v    : (B, H, Tk, hs), `dtype`, one stride set kv_strides: e.g. the
 *             first Tk rows of a (B, H, Tmax, hs) cache, {H*Tmax*hs, Tmax*hs, hs}.
 *   lse     : (B, H, Tq) float32, contiguous, may be NULL.
 *   strides : as in gattn_fwd_strided (NULL = contiguous for that length).
 *   workspace: at least gattn_fwd_decode_workspace_bytes() bytes, 256-byte
 *             aligned, overwritten (partial results of the key splits); may be
 *             NULL when that size is 0 (float32, or a single split).
 * The 16-bit path reads every kept key and value from HBM once, split over
 * the wavefronts of a workgroup (merged through LDS) and, when the heads
 * alone would leave the GPU idle, over several workgroups whose partial
 * results a second kernel merges (that case needs the workspace).  Tq = 1
 * runs a vector-ALU kernel, Tq > 1 the MFMA kernel; float32 runs one
 * wavefront per query.  INVALID_ARG also for Tq < 1 or Tk < Tq; WORKSPACE for
 * a missing, misaligned or short workspace when one is needed.
 */
int gattn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Tq, int Tk, int hs, float scale, int dtype,
                     const int64_t* q_strides, const int64_t* kv_strides,
                     const int64_t* o_strides, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Workspace bytes gattn_fwd_decode needs (0 for float32 and for arguments it
 * would reject). */
size_t gattn_fwd_decode_workspace_bytes(int B, int H, int Tq, int Tk, int hs, int dtype);

/*
 * Bytes of device workspace the backward needs: D = rowsum(dO * o) and
 * lse * log2(e), each float32 (B, H, T) starting on a 256-byte boundary.
 * Returns 0 for arguments gattn_bwd would reject.
 */
size_t gattn_bwd_workspace_bytes(int B, int H, int T, int hs, int dtype);

/*
 * Backward: dq, dk, dv of L = sum(dO * o) for the forward above (chain rule;
 * the pages state only that training runs a backward pass).  The row term
 * D[i] is the exact sum_j P[i][j] dP[i][j] (= dO[i] . o[i] before o was
 * rounded to `dtype`): the dQ pass starts from dO . o of the stored o and
 * corrects it, and dq, by the float32 row sums of dS.
 *   q, k, v, o, dO : inputs (B, H, T, hs), `dtype`; o is what gattn_fwd wrote.
 *   lse            : input (B, H, T) float32, what gattn_fwd wrote (required).
 *   dq, dk, dv     : outputs (B, H, T, hs), `dtype`.
 *   workspace      : caller-owned device memory of at least
 *                    gattn_bwd_workspace_bytes() bytes, 256-byte aligned; the
 *                    library overwrites it (it needs no clearing).
 * Equivalent to gattn_bwd_dq then gattn_bwd_dkdv on `stream`.  Every output
 * is deterministic (no atomics).
 */
int gattn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* dq, void* dk, void* dv,
              int B, int H, int T, int hs, float scale, int dtype,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): as gattn_bwd, with the row terms kept in a static
 * device array of the library (gattn_bwd_noalloc_max_bytes() bytes, 8 MiB, one
 * copy per GPU, held until the process ends) instead of a caller workspace.
 * Calls at most gattn_bwd_workspace_bytes() <= that size: B*H*T up to about
 * one million rows (WORKSPACE otherwise, before any HIP call).  The first call
 * on a device looks up the array's device address (hipGetSymbolAddress) with
 * that device current; the stream must belong to the current device.  Every
 * call on a GPU shares its array: calls that overlap on one GPU (different
 * streams, or host threads without ordering) race and give wrong results;
 * calls ordered on one stream do not.  Results equal gattn_bwd's bit for bit.
 */
int gattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int H, int T, int hs, float scale, int dtype, hipStream_t stream);

/* Bytes of the static device array gattn_bwd_noalloc uses. */
size_t gattn_bwd_noalloc_max_bytes(void);

/*
 * Backward on strided tensors: as gattn_bwd, with q, k, v addressed by
 * qkv_strides, o and dO by o_strides, and dq, dk, dv by grad_strides (same
 * convention and checks as gattn_fwd_strided; NULL = contiguous).  For a GPT
 * block: o_strides = {T*C, hs, C} reads o and the incoming gradient dO as
 * (B, T, C), and grad_strides = {T*3C, hs, 3C} with dq = dqkv, dk = dqkv + C,
 * dv = dqkv + 2C writes the gradient of the fused projection output directly.
 * The workspace is the same as gattn_bwd's.
 */
int gattn_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int H, int T, int hs, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, const int64_t* qkv_strides,
                      const int64_t* o_strides, const int64_t* grad_strides,
                      hipStream_t stream);

/*
 * Backward, row terms only: D[i] = sum_d dO[i][d] * o[i][d] from the stored o
 * (the row term of dS = P (dP - D), off by up to half an ulp of each o
 * element; gattn_bwd_dq writes it exactly) and lse[i] * log2(e), float32,
 * into the workspace.  For callers that run gattn_bwd_dkdv without
 * gattn_bwd_dq first.
 */
int gattn_bwd_preprocess(const void* o, const void* dO, const float* lse, int B, int H, int T,
                         int hs, int dtype, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Backward, dq = scale * dS k, with P recomputed from q, k and lse (exactly 0
 * above the diagonal) and dS = P (dO v^T - D).  Also leaves the row terms in
 * the workspace, D exact (see gattn_bwd).
 */
int gattn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                 const float* lse, void* dq, int B, int H, int T, int hs, float scale, int dtype,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward, dk = scale * dS^T q and dv = P^T dO, recomputing P and dS as
 * gattn_bwd_dq does from the row terms already in the workspace (written by
 * gattn_bwd_dq, exact, or gattn_bwd_preprocess earlier on the stream).
 * gattn_bwd_dq then gattn_bwd_dkdv equals gattn_bwd bit for bit.
 */
int gattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, void* dk,
                   void* dv, int B, int H, int T, int hs, float scale, int dtype, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * Attention dropout.  The RobGPT page ("GPT da zero", parameter table) trains
 * with dropout 0.1; the GPT-2 124M configuration ("Model Architecture
 * Nanogpt", Workflow 2) uses 0.0.  Dropout acts on the attention weights after
 * the row softmax and before the value sum, with kept weights scaled by
 * 1/(1 - p):
 *   O[i][:] = sum_j P[i][j] * Z[i][j] * V[j][:],   Z = keep / (1 - p_eff),
 * lse is that of the softmax before dropout, and the backward is
 *   dV = (P*Z)^T dO,   dS = P * (Z * (dO V^T) - D),   D[i] = dO[i] . O[i],
 *   dQ = scale dS K,   dK = scale dS^T Q.
 * Mask: t = floor(p * 65536 + 0.5) (p as given, in double precision; the
 * effective probability is p_eff = t / 65536).  For slice (b, h), query i,
 * key j, the Philox-4x32-10 generator (Salmon, Moraes, Dror, Shaw, SC 2011)
 * with counter (i, j >> 3, b*H + h, offset) and key (seed mod 2^32,
 * seed >> 32) gives four 32-bit words; u(i, j) is the (j & 1)-th 16-bit half
 * (low half first) of word (j & 7) >> 1, and keep(i, j) = u(i, j) >= t.  The
 * same (seed, offset) draws the same mask in the forward, the backward and
 * gattn_dropout_mask; give each layer and step its own (seed, offset).
 * The 16-bit kernels draw each decision once per training step when the
 * caller keeps them: the forward stores the decisions it draws as bits in a
 * keep buffer (like lse, saved for the backward), and the backward reads
 * them.  Without a keep buffer the backward draws them once itself (in its
 * dQ pass) and keeps them in its workspace for its dK/dV pass.  The float32
 * path always draws them where needed.  Either way the decisions, and so the
 * results, are the same.
 *
 * Keep buffer layout (bf16 and fp16): per (b, h) slice, ng x ng blocks of 8
 * bytes, ng = ceil(T / 8); block (I, G) at byte (((b*H + h) * ng + I) * ng + G)
 * * 8 holds the decisions of queries 8I .. 8I+7 (byte e: query 8I + e) and
 * keys 8G .. 8G+7 (bit r: key 8G + r, 1 = kept).  Only blocks with some key
 * <= some query are written.
 *
 * gattn_dropout_keep_bytes: size of the keep buffer, B*H*ng*ng*8 rounded up
 * to 256; 0 for B, H or T < 1, T > 131064, or more than 2^40 bytes.
 */
size_t gattn_dropout_keep_bytes(int B, int H, int T);

/*
 * gattn_fwd_dropout: as gattn_fwd_strided (strides NULL = contiguous) with
 * dropout of probability p.  p = 0 (t = 0) runs exactly gattn_fwd_strided.
 * keep: NULL, or a device buffer of gattn_dropout_keep_bytes() bytes, 16-byte
 * aligned, into which the bf16 and fp16 kernels store the keep decisions
 * (layout above; nothing is written for float32 or t = 0).
 * INVALID_ARG also for p not finite, p < 0, p >= 1, or t > 65535, and for a
 * keep buffer that is misaligned or whose shape has no keep size.
 */
int gattn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int T, int hs, float scale, int dtype, float p,
                      uint64_t seed, uint32_t offset, void* keep, const int64_t* qkv_strides,
                      const int64_t* o_strides, hipStream_t stream);

/*
 * gattn_bwd_dropout_workspace_bytes: workspace bytes gattn_bwd_dropout needs
 * without a keep buffer for this shape and p: gattn_bwd_workspace_bytes()
 * plus, for bf16 and fp16 with p rounding to a nonzero threshold,
 * gattn_dropout_keep_bytes() (the backward keeps the decisions it draws
 * there).  0 for arguments gattn_bwd_dropout rejects as INVALID_ARG or
 * UNSUPPORTED (bad shape or p; 16-bit with dropout and T > 131064).
 */
size_t gattn_bwd_dropout_workspace_bytes(int B, int H, int T, int hs, int dtype, float p);

/*
 * gattn_bwd_dropout: the backward of gattn_fwd_dropout with the same p, seed
 * and offset (o and lse as that forward wrote them); arguments and strides
 * as gattn_bwd_strided.  keep: NULL, or the keep buffer that forward filled
 * (same shape, p, seed and offset; read only, bf16 and fp16; ignored for
 * float32 and t = 0).  workspace: 256-byte aligned, contents need no
 * initialisation, at least gattn_bwd_workspace_bytes() bytes with a keep
 * buffer and gattn_bwd_dropout_workspace_bytes() bytes without
 * (GATTN_ERR_WORKSPACE if smaller).  p = 0 runs exactly gattn_bwd_strided.
 * INVALID_ARG also for p as in gattn_fwd_dropout, a misaligned keep buffer
 * and, for bf16 and fp16 with dropout, T > 131064.
 */
int gattn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int hs,
                      float scale, int dtype, float p, uint64_t seed, uint32_t offset,
                      const void* keep, void* workspace, size_t workspace_bytes,
                      const int64_t* qkv_strides, const int64_t* o_strides,
                      const int64_t* grad_strides, hipStream_t stream);

/*
 * gattn_dropout_mask: the keep decisions of the mask above as bytes
 * (1 = kept, 0 = dropped), keep[((b*H + h) * T + i) * T + j] for every i, j < T
 * (above the causal diagonal too), from the same generator code the kernels
 * use.  keep: device buffer of B*H*T*T bytes (no alignment needed).
 * INVALID_ARG for keep NULL, B, H or T < 1, B*H*T*T >= 2^40, or p as in
 * gattn_fwd_dropout.
 */
int gattn_dropout_mask(uint8_t* keep, int B, int H, int T, float p, uint64_t seed,
                       uint32_t offset, hipStream_t stream);

/*
 * Diagnostic, not part of attention: `blocks` workgroups of 4 wavefronts each
 * run `iters` rounds of 8 independent bf16 MFMAs (32x32x16, 32768 FLOP each)
 * on register operands, with no memory traffic, and write one float per
 * wavefront to sink (device buffer of 4*blocks floats).  Timing it gives the
 * achievable bf16 MFMA rate at the current clock: FLOP = blocks * 4 * iters *
 * 8 * 32768.  INVALID_ARG for sink NULL, blocks < 1 or iters < 1.
 */
int gattn_probe_mfma_bf16(float* sink, int blocks, int iters, hipStream_t stream);

/*
 * Diagnostic, not part of attention: what vector-ALU work costs beside the
 * matrix core.  `blocks` workgroups of 8 wavefronts, one per CU (96 KB of LDS
 * each keeps a second one off; two wavefronts per SIMD: wavefronts 0-3 and
 * 4-7 each span the CU's four SIMDs) run register-only loops chosen by
 * `roles`: bit 0, wavefronts 0-3 run mfma_iters rounds of 4 independent bf16
 * MFMAs (32x32x16); bit 1, wavefronts 0-3 run valu_iters rounds of 16
 * independent wave64 instructions of `kind` (0 v_fma_f32, 1 v_mul_f32,
 * 2 v_exp_f32); bits 2 and 3, the same for wavefronts 4-7.  Each wavefront
 * writes one float to sink (device buffer of 8*blocks floats).  Timing
 * launches of different roles gives the cost of a vector instruction in MFMA
 * cycles, with one or two issuing wavefronts per SIMD, and how much of it
 * runs beside another wavefront's MFMAs.  INVALID_ARG for sink NULL,
 * blocks < 1, a negative count, kind outside 0..2 or roles outside 1..15.
 */
int gattn_probe_issue(float* sink, int blocks, int mfma_iters, int valu_iters, int kind,
                      int roles, hipStream_t stream);

/* Static, human-readable name of a gattn_status value. */
const char* gattn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GATTN_H */
