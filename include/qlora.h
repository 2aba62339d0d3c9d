/*
 * qlora.h -- C ABI of libqlora, the gfx950 (MI355X) QLoRA adapted linear.
 *
 * The layer (page "LoRA and QLoRA fine-tuning: mechanics, and when not to
 * fine-tune", section "The update LoRA is allowed to learn", and the forward
 * equation in "What QLoRA freezes, and in how many bits"):
 *
 *     Y = X w~^T + s (X A^T) B^T,      s = alpha / r
 *
 * where W0 (d x k, frozen) is stored as 4-bit NormalFloat in blocks of 64
 * with double-quantised block constants, and w~ is its dequantisation to
 * bf16.  A (r x k) and B (d x r) are the trainable low-rank adapters.
 *
 * Conventions shared by every call
 *   - Every pointer argument except the nf4 descriptor, status strings and
 *     the host table of qlora_nf4_levels is a DEVICE pointer.  The caller
 *     owns every buffer, including workspaces; the library allocates no
 *     device memory.
 *   - Matrices are dense row-major.  bf16 values are passed as their 16-bit
 *     patterns (uint16_t).  X is M x k, Y and dY are M x d (one token per
 *     row).
 *   - Device pointers must be 16-byte aligned (QLORA_ERR_ALIGN otherwise).
 *   - 16 <= d, d % 16 == 0, 64 <= k, k % 64 == 0, 0 <= M; every matrix
 *     (M*k, M*d, d*k) must have fewer than 2^31 elements (QLORA_ERR_SHAPE
 *     otherwise).  k % 64 comes from the storage format (a block of 64 lies
 *     inside one row); d % 16 keeps every bf16 row 32-byte aligned.
 *   - 0 <= r <= 64 (QLORA_ERR_RANK).  r == 0 selects the frozen path only:
 *     A, B and alpha are then ignored and may be NULL / anything.
 *   - alpha must be finite (QLORA_ERR_ALPHA).  s is computed as
 *     fl32(alpha / r).
 *   - M == 0 is a no-op returning QLORA_OK.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error nothing is written and nothing is launched.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL means the default stream).  Launch failures are reported
 *     as QLORA_ERR_HIP; faults inside kernels surface at the caller's next
 *     synchronisation, as with any HIP call.
 *   - Outputs are overwritten, never accumulated into.  Outputs must not
 *     overlap inputs (QLORA_ERR_ALIAS), except where a call says so.
 *   - Calls are re-entrant.  Two calls that share a workspace must not run
 *     concurrently.
 *   - No C++ exception crosses this interface.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum qlora_status {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,      /* a required pointer is NULL                    */
  QLORA_ERR_SHAPE = 2,     /* d, k or M out of range, k%64 or d%16 != 0    */
  QLORA_ERR_RANK = 3,      /* r < 0 or r > 64                               */
  QLORA_ERR_ALIGN = 4,     /* a device pointer is not 16-byte aligned       */
  QLORA_ERR_WORKSPACE = 5, /* workspace NULL or smaller than required       */
  QLORA_ERR_ALPHA = 6,     /* alpha is not finite                           */
  QLORA_ERR_ALIAS = 7,     /* an output overlaps an input                   */
  QLORA_ERR_HIP = 8        /* a HIP runtime call or kernel launch failed    */
};

#define QLORA_NF4_BLOCK 64   /* weights per first-level block constant      */
#define QLORA_DQ_GROUP 256   /* block constants per second-level constant   */
#define QLORA_MAX_RANK 64

/*
 * NF4 storage of a frozen d x k weight (page "LoRA and QLoRA fine-tuning:
 * mechanics, ...", paragraphs "4-bit NormalFloat" and "Double quantisation").
 * All four buffers are device memory owned by the caller.
 *
 *   codes        d*k/2 bytes.  The row-major flattening of W0 is cut into
 *                n_b = d*k/64 blocks of 64 consecutive weights (a block lies
 *                inside one row).  Codes are packed per aligned group of 8
 *                consecutive elements into 4 bytes: byte j (j = 0..3) holds
 *                element j in its low nibble and element j+4 in its high
 *                nibble (so a 32-bit word decodes to 8 consecutive bf16 with
 *                byte permutes only).  Code i means the i-th NF4 level in
 *                ascending order (code 7 = 0).
 *   absmax_q     n_b bytes: block constant a_b - mu, divided by its group's
 *                absmax_scale and rounded (nearest-even, saturating) to OCP
 *                FP8 E4M3FN.
 *   absmax_scale ceil(n_b/256) floats: per group of 256 consecutive blocks,
 *                max |a_b - mu| / 448.
 *   absmax_mean  1 float: mu, the mean of all block absmax values.
 *
 * Decode: a^_b = fl32(fl32(e4m3(absmax_q[b]) * absmax_scale[b/256]) + mu);
 *         w~   = bf16_rne(fl32(level[code] * a^_b)).
 */
typedef struct qlora_nf4 {
  int64_t d;
  int64_t k;
  uint8_t *codes;
  uint8_t *absmax_q;
  float *absmax_scale;
  float *absmax_mean;
} qlora_nf4_t;

/* Human-readable name of a status code (static storage). */
const char *qlora_status_string(int status);

/* Library version, (major << 16) | minor. */
int qlora_version(void);

/*
 * The 16 NF4 levels the library uses, ascending, written to a HOST array.
 * Built once per process from standard-normal quantiles (Wichura's AS241
 * inverse normal in double precision) and rounded to fp32; see the
 * "4-bit NormalFloat" paragraph of page "LoRA and QLoRA fine-tuning:
 * mechanics, ...".  Pure host computation; needs no GPU.
 */
int qlora_nf4_levels(float *levels_out16);

/* Byte sizes of the four NF4 buffers of a d x k weight (any pointer may be
 * NULL).  Returns QLORA_ERR_SHAPE for an invalid shape. */
int qlora_nf4_sizes(int64_t d, int64_t k, size_t *codes_bytes,
                    size_t *absmax_q_bytes, size_t *absmax_scale_bytes,
                    size_t *absmax_mean_bytes);

/*
 * nf4_quantize -- blockwise NF4 quantisation with double-quantised absmax
 * (page "LoRA and QLoRA fine-tuning: mechanics, ...", paragraphs
 * "4-bit NormalFloat" and "Double quantisation").
 *
 *   W0    device, d x k fp32 row-major (read only).
 *   out   host descriptor; out->d and out->k must equal d and k; its four
 *         device buffers are written (sizes from qlora_nf4_sizes).
 *   ws    device workspace of at least qlora_quantize_workspace_bytes(d, k).
 *
 * Steps: absmax a_b of each block of 64; codes = nearest NF4 level of
 * fl32(w / a_b) (ties to the lower code; all-zero blocks code to 7);
 * mu = fl32(S / n_b) with S the float64 sum of all a_b taken sequentially
 * inside each group of 256 and then sequentially over groups; per group
 * c1 = fl32(max|fl32(a - mu)| / 448) and c2 = e4m3(fl32(fl32(a - mu) / c1))
 * (c2 = 0 when c1 == 0).  The result is deterministic and bit-exact with
 * that definition.  Non-finite weights give unspecified codes.
 */
size_t qlora_quantize_workspace_bytes(int64_t d, int64_t k);
int nf4_quantize(const float *W0, int64_t d, int64_t k, const qlora_nf4_t *out,
                 void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_forward -- Y = X w~^T + s (X A^T) B^T in bf16 with fp32 accumulation
 * (page "LoRA and QLoRA fine-tuning: mechanics, ...": the forward equation of
 * "What QLoRA freezes"; page "Fine-Tuning on a Budget", diagram of
 * "The LoRA hypothesis").
 *
 *   X       device, M x k bf16.
 *   W0      host descriptor of the NF4 weight (d x k).
 *   A, B    device, r x k and d x r bf16 (ignored when r == 0).
 *   Y       device, M x d bf16, written.
 *   T_save  optional device buffer of qlora_tsave_bytes(M, r) bytes:
 *           receives T^T, the transpose of the LoRA down-projection
 *           T = X A^T rounded to bf16 (r rows, row stride roundup(M, 64)
 *           elements; the padding is left unspecified), for reuse by
 *           qlora_backward.  May be NULL.  Ignored when r == 0.
 *   ws      device workspace, at least qlora_forward_workspace_bytes(M,d,k,r).
 *
 * T is rounded to bf16 before the up-projection (the pages compute the
 * adapter product in BF16).  Y must not overlap X, A, B or T_save.
 */
size_t qlora_tsave_bytes(int64_t M, int32_t r);
size_t qlora_forward_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t r);
int qlora_forward(const uint16_t *X, int64_t M, const qlora_nf4_t *W0,
                  const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                  uint16_t *Y, uint16_t *T_save, void *ws, size_t ws_bytes,
                  void *stream);

/*
 * qlora_backward -- gradients of the adapted linear for an upstream
 * gradient dY (M x d).  W0 is frozen and gets no gradient; the input
 * gradient flows through the dequantised base (page "LoRA and QLoRA
 * fine-tuning: mechanics, ...", "What QLoRA freezes": the adapters are the
 * only trained weights, and the input gradient is formed with the bf16
 * expansion of the frozen base).
 *
 *   U  = dY B                          (M x r, rounded to bf16)
 *   dX = dY w~ + s U A                 (M x k bf16; skipped if dX == NULL)
 *   dA = s U^T X                       (r x k bf16)
 *   dB = s dY^T T,   T = X A^T         (d x r bf16)
 *
 *   T_saved  optional: the r x M buffer written by qlora_forward's T_save
 *            for the same X and A.  When NULL, T is recomputed from X.
 *   ws       device workspace, at least qlora_backward_workspace_bytes.
 *
 * When r == 0 only dX is produced (dA, dB may be NULL).  dA and dB are
 * reduced over tokens in a fixed order: results are deterministic.
 */
size_t qlora_backward_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t r);
int qlora_backward(const uint16_t *dY, const uint16_t *X, int64_t M,
                   const qlora_nf4_t *W0, const uint16_t *A, const uint16_t *B,
                   int32_t r, float alpha, const uint16_t *T_saved,
                   uint16_t *dX, uint16_t *dA, uint16_t *dB, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * qlora_backward_noalloc -- qlora_backward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or training
 * loops, and harnesses that forbid hipMalloc.  Same arguments and results
 * as qlora_backward, without the workspace: the library uses instead one
 * static device array of QLORA_NOALLOC_SCRATCH_BYTES on each GPU it runs on
 * (reserved when its device code is loaded on that GPU, held until the
 * process ends; its device address is looked up once per GPU, on the first
 * call with a stream of that GPU).  The call itself allocates nothing.
 *
 * Returns QLORA_ERR_WORKSPACE when qlora_backward_workspace_bytes(M, d, k, r)
 * exceeds QLORA_NOALLOC_SCRATCH_BYTES (e.g. 4096 tokens at 8192 x 22016 with
 * r = 64 need 5.7 MiB; 128 tokens at 4096 x 11008 with r = 16, 27.4 MiB).
 * All calls on one GPU share that GPU's array and the array keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * on one GPU -- on different streams, or from different host threads --
 * race on it and give undefined results.
 */
#define QLORA_NOALLOC_SCRATCH_BYTES (32u << 20)
int qlora_backward_noalloc(const uint16_t *dY, const uint16_t *X, int64_t M,
                           const qlora_nf4_t *W0, const uint16_t *A, const uint16_t *B,
                           int32_t r, float alpha, const uint16_t *T_saved,
                           uint16_t *dX, uint16_t *dA, uint16_t *dB, void *stream);

/*
 * qlora_forward_sections, qlora_backward_sections -- nsec adapted linears
 * that read the same input (a layer's q, k and v projections, or gate and
 * up: page "LoRA vs QLoRA: Parameter-Efficient Fine-Tuning Explained", the
 * target modules of the run configuration; page "LoRA and QLoRA
 * fine-tuning: mechanics, ...", the per-projection matrix W of "The update
 * LoRA is allowed to learn") computed as one GEMM over their row-stacked
 * NF4 weights, each projection keeping its own adapter.  For section p
 * (output features p*d/nsec .. (p+1)*d/nsec - 1):
 *
 *   Y_p  = X w~_p^T + s (X A_p^T) B_p^T
 *   dX   = sum_p dY_p w~_p + s U_p A_p,   U_p = dY_p B_p
 *   dA_p = s U_p^T X,   dB_p = s dY_p^T T_p,   T_p = X A_p^T
 *
 * which is what nsec separate calls of qlora_forward / qlora_backward
 * compute (up to fp32 summation order; dX sums the sections' products in
 * one accumulator).  One pass over X (or dY) serves every section.
 *
 *   W0     d x k descriptor whose rows stack nsec weights quantised one by
 *          one (nf4_quantize into consecutive slices of one set of buffers:
 *          codes, absmax_q and absmax_scale of section p start at its first
 *          row), with absmax_mean pointing to nsec floats, the sections'
 *          means in order.  A section's slices form a valid single-weight
 *          descriptor of its own (merge and unmerge work per section).
 *   A      (nsec*r) x k: A_0 .. A_{nsec-1} stacked.   dA likewise.
 *   B      d x r: B_0 .. B_{nsec-1} stacked by rows.  dB likewise.
 *   T_save / T_saved   qlora_tsave_bytes(M, nsec*r) bytes (nsec*r rows).
 *   ws     qlora_forward_workspace_bytes(M, d, k, nsec*r) and
 *          qlora_backward_workspace_bytes(M, d, k, nsec*r) bytes.
 *
 * Requires 1 <= nsec <= 4 and d % nsec == 0; for nsec > 1 also
 * (d/nsec) % 256 == 0 (QLORA_ERR_SHAPE otherwise) and r % 16 == 0 with
 * r <= 64 (QLORA_ERR_RANK), so up to 256 ranks in all.  r == 0 runs the
 * base GEMM with the per-section means.  nsec == 1 is qlora_forward /
 * qlora_backward.  The size queries (qlora_tsave_bytes and the two
 * workspace queries) accept the total rank nsec*r up to 256 for this.
 */
int qlora_forward_sections(const uint16_t *X, int64_t M, const qlora_nf4_t *W0,
                           int32_t nsec, const uint16_t *A, const uint16_t *B,
                           int32_t r, float alpha, uint16_t *Y, uint16_t *T_save,
                           void *ws, size_t ws_bytes, void *stream);
int qlora_backward_sections(const uint16_t *dY, const uint16_t *X, int64_t M,
                            const qlora_nf4_t *W0, int32_t nsec, const uint16_t *A,
                            const uint16_t *B, int32_t r, float alpha,
                            const uint16_t *T_saved, uint16_t *dX, uint16_t *dA,
                            uint16_t *dB, void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_forward_dropout, qlora_backward_dropout -- the adapted linear with
 * LoRA dropout on the adapter path's input (page "LoRA vs QLoRA:
 * Parameter-Efficient Fine-Tuning Explained", run configuration: a
 * dropout rate of 5 to 10 % on the adapters, as a regulariser).  The
 * random draw is the caller's: keep is an M x k byte mask (nonzero =
 * kept), p the dropout probability, and the adapter path reads
 *
 *   Xd = bf16(x * fl32(1 / (1 - p)))  where keep != 0,  0 elsewhere
 *
 *   Y  = X w~^T + s (Xd A^T) B^T              (frozen path on X itself)
 *   dX = dY w~ + s (U A) * keep / (1 - p),    U = dY B
 *   dA = s U^T Xd,   dB = s dY^T T,   T = Xd A^T
 *
 * The backward must get the forward's mask and p.  keep is 16-byte
 * aligned (QLORA_ERR_ALIGN), p in [0, 1) (QLORA_ERR_ALPHA otherwise);
 * both are ignored when r == 0.  Xd_save (optional, M x k bf16, 16-byte
 * aligned) receives Xd; passing it back as Xd_saved spares the backward
 * its own pass over X and the mask (like T_save / T_saved).  Workspaces:
 * qlora_forward_dropout_workspace_bytes / qlora_backward_dropout_...
 * (they add the M x k bf16 Xd).  With p == 0 and nothing dropped the
 * results equal qlora_forward / qlora_backward.
 */
size_t qlora_forward_dropout_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t r);
size_t qlora_backward_dropout_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t r);
int qlora_forward_dropout(const uint16_t *X, int64_t M, const qlora_nf4_t *W0,
                          const uint16_t *A, const uint16_t *B, int32_t r, float alpha,
                          const uint8_t *keep, float p, uint16_t *Y, uint16_t *T_save,
                          uint16_t *Xd_save, void *ws, size_t ws_bytes, void *stream);
int qlora_backward_dropout(const uint16_t *dY, const uint16_t *X, int64_t M,
                           const qlora_nf4_t *W0, const uint16_t *A, const uint16_t *B,
                           int32_t r, float alpha, const uint8_t *keep, float p,
                           const uint16_t *T_saved, const uint16_t *Xd_saved, uint16_t *dX,
                           uint16_t *dA, uint16_t *dB, void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_forward_multi -- one frozen base serving several adapters in one
 * batch, each token with its own (page "LoRA and QLoRA fine-tuning:
 * mechanics, ...", "What to choose and why": a batch that mixes tasks keeps
 * the adapters unmerged and picks one per example; page "Fine-Tuning on a
 * Budget": one frozen base plus a stack of small adapters swapped per
 * request; page "LoRA and QLoRA Explained": the shared base with a
 * separate adapter per task, picked at inference time).  For token m with
 * a = idx[m]:
 *
 *   Y[m] = X[m] w~^T + s (X[m] A_a^T) B_a^T    if 0 <= a < nad
 *   Y[m] = X[m] w~^T                            otherwise (no adapter)
 *
 *   A     (nad*r) x k: A_0 .. A_{nad-1} stacked.
 *   B     nad blocks of d x r: B_a starts at B + a*d*r.
 *   idx   device, M int32 adapter indices.
 *   ws    qlora_forward_multi_workspace_bytes(M, d, k, nad, r) bytes.
 *
 * Made for decode-shaped batches: tokens are taken 128 at a time (64 when
 * k % 256 != 0) through the split-K decode kernels, each group computing
 * X A_a^T for all nad
 * adapters inside the weight stream (r*nad*k*2 more bytes per group) and
 * picking each token's in the last step (with nad = 1 and every index 0
 * this is qlora_forward bit for bit at M <= 64).
 * 1 <= nad <= 64 (QLORA_ERR_RANK), 0 <= r <= 64; r == 0 ignores A, B, idx.
 */
size_t qlora_forward_multi_workspace_bytes(int64_t M, int64_t d, int64_t k, int32_t nad,
                                           int32_t r);
int qlora_forward_multi(const uint16_t *X, int64_t M, const qlora_nf4_t *W0, int32_t nad,
                        const uint16_t *A, const uint16_t *B, const int32_t *idx, int32_t r,
                        float alpha, uint16_t *Y, void *ws, size_t ws_bytes, void *stream);

/*
 * qlora_adam_step -- one Adam step on n adapter parameters (A and B, in one
 * buffer or one call each) with an fp32 master copy (page "Fine-Tuning on a
 * Budget", "Why full fine-tuning costs so much": a trained parameter keeps
 * a 16-bit weight, a 32-bit master copy and Adam's two 32-bit moments; page
 * "LoRA and QLoRA fine-tuning: mechanics, ...": only the adapter carries
 * optimiser state, and QLoRA pages that state to host memory).  Elementwise,
 * in fp32 with every operation rounded:
 *
 *   m = b1 m + (1 - b1) g,   v = b2 v + (1 - b2) g^2
 *   W = W - lr ( (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps) + wd W )
 *   P = bf16(W)
 *
 *   P      device, n bf16: the copy forward/backward read (written).
 *   W, m, v  n fp32 each, updated in place.  They may be in any memory the
 *          GPU addresses: device memory, or host-pinned / managed memory for
 *          paged state (the caller allocates; the library never does).
 *   G      n bf16 gradients (dA or dB as qlora_backward wrote them).
 *   step   1 for the first step (bias corrections); wd = 0 is plain Adam.
 *
 * All pointers 16-byte aligned (QLORA_ERR_ALIGN) and disjoint
 * (QLORA_ERR_ALIAS); lr, wd >= 0 finite, b1, b2 in [0, 1), eps > 0,
 * step >= 1 (QLORA_ERR_ALPHA otherwise).
 */
int qlora_adam_step(uint16_t *P, float *W, const uint16_t *G, float *m, float *v, int64_t n,
                    float lr, float beta1, float beta2, float eps, float weight_decay,
                    int64_t step, void *stream);

/*
 * lora_merge -- deploy-time merge W = bf16_rne(w~ + s B A), d x k bf16
 * (page "LoRA and QLoRA fine-tuning: mechanics, ...", "The update LoRA is
 * allowed to learn": merged layer has the shape and latency of a plain one;
 * page "Fine-Tuning on a Budget", "What actually goes wrong": merge into the
 * 16-bit weights, not the quantised ones).  r == 0 writes w~ itself.
 * The product s B A is accumulated in fp32 and added to w~ before one
 * rounding.
 */
int lora_merge(const qlora_nf4_t *W0, const uint16_t *A, const uint16_t *B,
               int32_t r, float alpha, uint16_t *W, void *stream);

/*
 * lora_unmerge -- task switch: W0_out = bf16_rne(W - s B A) for a d x k
 * bf16 W (page "LoRA and QLoRA fine-tuning: mechanics, ...": switch tasks by
 * subtracting BA and adding B'A').  W0_out may equal W (in place); any other
 * overlap is QLORA_ERR_ALIAS.  r == 0 copies W.
 */
int lora_unmerge(const uint16_t *W, int64_t d, int64_t k, const uint16_t *A,
                 const uint16_t *B, int32_t r, float alpha, uint16_t *W0_out,
                 void *stream);

/*
 * Per-kernel timing (a profiling aid for benchmarks; off by default).
 * While enabled, every kernel this library launches is bracketed by two HIP
 * events recorded on the stream it runs on.  qlora_timing_collect() waits for
 * the brackets recorded so far and adds their elapsed times to per-kernel
 * totals, which qlora_timing_query() returns by kernel name (for example
 * "fwd_rich", "fwd_decode", "dx", "lora_proj", "token_reduce", "merge").
 * Process-wide state guarded by a mutex; events are created on demand and
 * reused (no device memory is allocated).  Returns QLORA_ERR_HIP if an event
 * call failed.
 */
int qlora_timing_enable(int on);
int qlora_timing_collect(void);
int qlora_timing_query(const char *kernel, double *total_ms, int64_t *launches);
int qlora_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
