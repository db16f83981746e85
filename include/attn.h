/*
 * attn.h -- C ABI of the MI355X (gfx950) fused attention library.
 *
 * One operation: scaled-dot-product attention over [B, H, S, D] tensors,
 *   S_ij  = scale * sum_d Q_id K_jd        (key j visible from query i;
 *                                          causal: visible iff j <= i)
 *   LSE_i = ln sum_{j visible} exp(S_ij)
 *   O_i   = sum_j exp(S_ij - LSE_i) V_j
 * forward (O and LSE saved) and backward (dQ, dK, dV for a loss whose
 * gradient with respect to O is dO).  "Meganeura: Portable GPU Training and
 * Inference through Vulkan and Metal" (arXiv 2608.01563) treats attention as
 * one graph node with a local derivative rule (Section 3.1) and lowers it to
 * tiled attention forward, dQ and fused dK+dV kernels (Section 3.3); this
 * library provides those three kernels for one GPU.
 *
 * Conventions shared by every entry point:
 *  - Pointers named q, k, v, o, dout, dq, dk, dv, lse, workspace are DEVICE
 *    pointers owned by the caller.  The library never allocates or frees
 *    device memory and keeps no pointer after the call returns; its only
 *    state is two host-side caches keyed by device and shape (resident
 *    workgroups per kernel, the static work schedule), filled on first use
 *    under a lock, so calls from several host threads are safe.
 *  - Layout: [batch, heads, seq, head_dim] contiguous row-major for Q, K, V,
 *    O, dO, dQ, dK, dV; LSE is [batch, heads, seq] float32.  Query and key
 *    length are both `seq` (self-attention).
 *  - Element type per `dtype` (attn_dtype_t): ATTN_F32 = IEEE float32 for
 *    every tensor (strict f32: f32 MFMA operands, f32 accumulation); ATTN_BF16
 *    = bfloat16 storage for Q, K, V, O, dO, dQ, dK, dV, with bf16 MFMA
 *    operands (the softmax probabilities and dS rounded to nearest-even
 *    bf16) and f32 accumulation, softmax statistics and LSE.  These are the
 *    two arithmetic contracts of the pages' Section 4.2 (strict f32 versus a
 *    reduced-input matrix path), here with bf16 in place of f16.
 *    ATTN_F32_BF16FWD (float32 tensors, bf16-rounded forward operands,
 *    strict f32 backward) is the pages' practical mixed contract.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    and the call returns; outputs are valid once the caller synchronises
 *    the stream.  Faults inside a kernel surface at that synchronisation.
 *  - Outputs are overwritten (=, never +=), must not alias inputs or each
 *    other, and inputs are never written.
 *  - Validation happens before anything is enqueued: on any error nothing
 *    is launched and the error code is returned.
 *      ATTN_ERR_INVALID_ARG  null pointer, batch/heads/seq <= 0, causal not
 *                            0 or 1, scale not a finite positive number (a
 *                            softmax temperature; the kernels take row
 *                            maxima of the unscaled scores, which are the
 *                            maxima of the scaled ones only for scale > 0), a
 *                            pointer not 16-byte aligned, or sizes whose
 *                            element count overflows a 32-bit signed index
 *      ATTN_ERR_UNSUPPORTED  head_dim not in {32, 64, 128}, or unknown dtype
 *      ATTN_ERR_WORKSPACE    workspace smaller than attn_bwd_workspace_size()
 *      ATTN_ERR_HIP          the HIP runtime reported a launch error
 */
#ifndef ATTN_MI355X_ATTN_H
#define ATTN_MI355X_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,
  ATTN_ERR_UNSUPPORTED = 2,
  ATTN_ERR_WORKSPACE = 3,
  ATTN_ERR_HIP = 4
} attn_status_t;

typedef enum {
  ATTN_F32 = 0,         /* strict float32 contract */
  ATTN_BF16 = 1,        /* bf16 storage and MFMA operands, f32 accumulation */
  ATTN_F32_BF16FWD = 2, /* float32 storage; the forward rounds its MFMA
                           operands (Q, K, V, P) to bf16 and accumulates and
                           stores in f32; every backward entry point treats
                           it as ATTN_F32 (strict) */
  ATTN_DTYPE_INT_RANGE_ = 0x7fffffff  /* not a dtype: makes every int value a
                           valid attn_dtype_t in C++, so that an unknown code
                           from a caller is rejected (ATTN_ERR_UNSUPPORTED)
                           rather than being undefined behaviour */
} attn_dtype_t;

/*
 * Forward pass (tiled attention forward; pages' Section 3.3).
 *   in : q, k, v   [B,H,S,D] dtype
 *   out: o         [B,H,S,D] dtype   softmax(scale * Q K^T, masked) V
 *        lse       [B,H,S]   float32 natural-log row normaliser, scale
 *                                    included; the backward reads it.  NULL
 *                                    skips it: an inference-only forward
 *                                    that keeps no statistics for a
 *                                    backward (the inference timing of the
 *                                    pages' Section 4.3).
 * ATTN_F32_BF16FWD is the pages' practical contract (Section 4.2: forward
 * matrix and attention inputs rounded locally to reduced precision, f32
 * accumulation and stores, backward kept f32): tensors as ATTN_F32, MFMA
 * operands rounded to bf16 inside the kernel.
 * One kernel launch.
 */
attn_status_t attn_fwd(attn_dtype_t dtype,
                       const void* q, const void* k, const void* v,
                       void* o, float* lse,
                       int batch, int heads, int seq, int head_dim,
                       int causal, float scale, void* stream);

/*
 * Forward with a key split, for few long heads (the minimal-latency long
 * context of the pages' Section 4.3): when the longest query tile of a head
 * walks far more key tiles than a balanced share of the GPU, each such query
 * tile's keys are cut into chunks processed as separate work items whose
 * partial (O, row maximum, row sum) go to the workspace and are merged in
 * chunk order by a second kernel (deterministic).  Self-attention, [B,H,S,D]
 * layout, the arguments and errors of attn_fwd plus:
 *   workspace   NULL, or DEVICE memory, 16-byte aligned, contents ignored;
 *               the split is used iff workspace_bytes >=
 *               attn_fwd_workspace_size(), else the call is attn_fwd.
 * attn_fwd_workspace_size returns 0 for shapes that are not split (enough
 * work items already) or rejected, else
 *   chunks * B*H * ceil(S/64)*64 * (head_dim + 2) * 4 bytes (rounded up to 256).
 * O and LSE equal attn_fwd's up to the summation order of the chunks.
 */
size_t attn_fwd_workspace_size(attn_dtype_t dtype, int batch, int heads, int seq,
                               int head_dim, int causal);
attn_status_t attn_fwd_ws(attn_dtype_t dtype,
                          const void* q, const void* k, const void* v,
                          void* o, float* lse, void* workspace, size_t workspace_bytes,
                          int batch, int heads, int seq, int head_dim,
                          int causal, float scale, void* stream);

/*
 * Workspace of the backward, in bytes (pure host functions; 0 for arguments
 * attn_bwd would reject).  The pages' runtime plans its buffers statically
 * and allocates nothing while a step runs (Section 3.5, static execution and
 * memory planning); here the caller owns every scratch byte, sized by these
 * functions from the shape alone.  The workspace holds, in this order:
 *   1. for every query row, D_i = sum_d dO_id O_id and LSE_i * log2(e) (two
 *      [B,H,S] float32 vectors, rounded up to 256 bytes): the minimum;
 *   2. dS transposed, [B*H][Sp][Sp] with Sp = ceil(S/128)*128, in the
 *      element type, which lets dQ be computed as one GEMM dS K instead of
 *      recomputing the scores (the dS path);
 *   3. only for shapes with few (key tile, head) pairs -- fewer than 512
 *      with float32 tensors, 256 with bf16 (64-key tiles), e.g. many queries
 *      over few keys, or few long heads -- float32 partial sums of dK and dV
 *      over chunks of the queries, [2][C][B*H][S][D] with C chunks chosen
 *      from the shape alone (each chunk is then its own work item and the
 *      chunks are added up in a fixed order, so results stay deterministic).
 *   attn_bwd_workspace_size      recommended size: 1 + 2 + 3 while part 2
 *                                (which grows as S^2) is at most 256 MiB,
 *                                the last-level cache; beyond it 1 + 3, so
 *                                the recommended size stays O(S) for long
 *                                sequences (the dS path was measured 20-30%
 *                                faster in f32 and 5-15% in bf16 there, so a
 *                                caller with memory to spare may still give
 *                                1 + 2 + 3 bytes)
 *   attn_bwd_workspace_size_min  minimum size: 1 (dQ recomputes P and dP)
 * The backward takes the dS path iff workspace_bytes >= the size of 1 + 2,
 * and the query-chunk split iff the partials fit as well (after 2 on the dS
 * path, else after 1).
 */
size_t attn_bwd_workspace_size(attn_dtype_t dtype, int batch, int heads,
                               int seq, int head_dim, int causal);
size_t attn_bwd_workspace_size_min(attn_dtype_t dtype, int batch, int heads,
                                   int seq, int head_dim, int causal);

/*
 * Backward pass (the pages' attention derivative: dQ kernel and fused dK+dV
 * kernel, Section 3.3; profiled in Section 7.3): attn_bwd_prep, then
 * attn_bwd_dkdv, then attn_bwd_dq, enqueued on `stream` -- except that bf16
 * on the dS path (no padded keys, strided layout or RoPE) runs no prep: its
 * dK+dV kernel forms D and LSE*log2(e) of each query tile from O, dO and
 * the LSE itself (workspace part 1 is then left unused).
 *   in : q, k, v, o, dout  [B,H,S,D] dtype  (o = the forward's output)
 *        lse               [B,H,S]   float32 (the forward's LSE)
 *   out: dq, dk, dv        [B,H,S,D] dtype  gradients of the loss
 *   workspace              >= attn_bwd_workspace_size_min() bytes of device
 *                          memory, 16-byte aligned; contents on entry are
 *                          ignored and left undefined.
 * Deterministic: no atomics; every output element is written by exactly one
 * thread in a fixed order, so repeated calls give bitwise identical results.
 */
attn_status_t attn_bwd(attn_dtype_t dtype,
                       const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse,
                       void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes,
                       int batch, int heads, int seq, int head_dim,
                       int causal, float scale, void* stream);

/*
 * Allocation-free backward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): attn_bwd without the workspace arguments.  Its workspace is a
 * device array inside the library, ATTN_BWD_NOALLOC_MAX_BYTES (128 MiB) per
 * GPU, reserved when the library's device code is loaded on that GPU and
 * held until the process ends; the call itself allocates and frees nothing.
 * It uses the largest layout of attn_bwd_workspace_size() that fits the
 * array (the dS path whenever the minimum plus dS^T fits: up to 127 heads
 * of S = 512 in float32, 254 in bf16), so its results are bitwise those of
 * attn_bwd given a workspace of that size.
 * Errors as attn_bwd, and ATTN_ERR_WORKSPACE when even the minimum workspace
 * (2 * batch * heads * seq float32, rounded up to 256 bytes) exceeds the
 * array, i.e. when batch * heads * seq > 16,777,216.
 * Every call on one GPU uses that GPU's one array: calls that can overlap in
 * time on the same GPU (several streams, several host threads) race and give
 * undefined results, so serialise them (one stream).  Nothing in the array
 * has to start at zero: every workspace value a call uses is written earlier
 * in the same call.
 */
#define ATTN_BWD_NOALLOC_MAX_BYTES ((size_t)128 << 20)
attn_status_t attn_bwd_noalloc(attn_dtype_t dtype,
                               const void* q, const void* k, const void* v,
                               const void* o, const void* dout, const float* lse,
                               void* dq, void* dk, void* dv,
                               int batch, int heads, int seq, int head_dim,
                               int causal, float scale, void* stream);

/*
 * Backward stage 1 alone: D_i = sum_d dO_id O_id and LSE_i * log2(e) into
 * the workspace (memory-bound, one pass over O and dO).
 */
attn_status_t attn_bwd_prep(attn_dtype_t dtype,
                            const void* o, const void* dout, const float* lse,
                            void* workspace, size_t workspace_bytes,
                            int batch, int heads, int seq, int head_dim,
                            void* stream);

/*
 * Backward stage 2 alone (the pages' fused dK+dV kernel): per key row,
 * dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i P_ij (dP_ij - D_i) Q_i,
 * with P recomputed from the workspace's LSE*log2(e) and D (stage 1 must have
 * run first, in stream order).  With the recommended workspace it also
 * stores dS for stage 3.
 */
attn_status_t attn_bwd_dkdv(attn_dtype_t dtype,
                            const void* q, const void* k, const void* v,
                            const void* dout, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes,
                            int batch, int heads, int seq, int head_dim,
                            int causal, float scale, void* stream);

/*
 * Backward stage 3 alone (the pages' dQ kernel): dQ_i = scale * sum_j dS_ij K_j,
 * as a GEMM over the stored dS with the recommended workspace (stage 2 must
 * have run first with the same workspace), else recomputing P and dP per key
 * tile from the workspace's LSE*log2(e) and D (stage 1 must have run).
 */
attn_status_t attn_bwd_dq(attn_dtype_t dtype,
                          const void* q, const void* k, const void* v,
                          const void* dout, void* dq,
                          const void* workspace, size_t workspace_bytes,
                          int batch, int heads, int seq, int head_dim,
                          int causal, float scale, void* stream);

/*
 * Cross-attention and padded keys (the pages' text cross-attention of the
 * diffusion workload and the one-token minimal-latency query, Sections 10
 * and 4.3): the forward and backward above with separate query and key
 * lengths and optional per-batch key counts.
 *   q, o, dout, dq  [B,H,seq_q,D] dtype      lse  [B,H,seq_q] float32
 *   k, v, dk, dv    [B,H,seq_k,D] dtype
 *   kv_len          NULL (every key valid) or a DEVICE array of `batch`
 *                   int32, 4-byte aligned: batch b has L_b = kv_len[b] valid
 *                   keys (values are clamped to [0, seq_k] on the device;
 *                   rows of k and v at or past L_b are never read).
 * Key j is visible from query i iff j < L_b and, when causal,
 * j <= i + L_b - seq_q: the causal diagonal is aligned with the end of the
 * valid keys (with seq_q = seq_k = L_b this is the self-attention rule
 * j <= i, and a one-token query sees every valid key).  A query row with no
 * visible key gets O = 0 and LSE = -inf, and contributes no gradient; dK and
 * dV rows at or past L_b are written as zeros.  The workspace sizes follow
 * from (seq_q, seq_k): D and LSE*log2(e) per query row, for the dS path
 * dS transposed, [B*H][ceil(seq_k/128)*128][ceil(seq_q/128)*128], and for
 * the query-chunk split the dK, dV partials [2][C][B*H][seq_k][D] float32
 * (the 77-key text cross-attention over 4096 queries is such a shape), in
 * the order and with the rules of attn_bwd_workspace_size.  Errors as
 * for attn_fwd / attn_bwd (seq_q, seq_k <= 0 or a misaligned kv_len:
 * ATTN_ERR_INVALID_ARG).
 */
attn_status_t attn_fwd_cross(attn_dtype_t dtype,
                             const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             int batch, int heads, int seq_q, int seq_k, int head_dim,
                             const int* kv_len, int causal, float scale, void* stream);
size_t attn_bwd_cross_workspace_size(attn_dtype_t dtype, int batch, int heads,
                                     int seq_q, int seq_k, int head_dim, int causal);
size_t attn_bwd_cross_workspace_size_min(attn_dtype_t dtype, int batch, int heads,
                                         int seq_q, int seq_k, int head_dim, int causal);
attn_status_t attn_bwd_cross(attn_dtype_t dtype,
                             const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes,
                             int batch, int heads, int seq_q, int seq_k, int head_dim,
                             const int* kv_len, int causal, float scale, void* stream);

/*
 * Strided layouts (the pages' packed projection forms, Section 3.2): the
 * cross-attention forward and backward above, with every tensor given as a
 * base pointer plus element strides (batch, head, row) of its [B,H,S,D]
 * indexing; the head dimension is contiguous.
 *   strides  HOST array of int64: attn_fwd_strided 12 values, (batch, head,
 *            row) for q, k, v, o in that order; attn_bwd_strided 24 values,
 *            for q, k, v, o, dout, dq, dk, dv.
 * Examples: [B,H,S,D] row-major {H*S*D, S*D, D}; [B,S,H,D] {S*H*D, D, H*D};
 * Q, K, V of a packed [B,S,3,H,D] projection at element offsets 0, H*D,
 * 2*H*D with {S*3*H*D, D, 3*H*D}; one K, V head shared by all query heads
 * (multi-query attention) with head stride 0 on k and v.  lse stays
 * [B,H,seq_q] float32 and the workspace keeps its layout and sizes
 * (attn_bwd_cross_workspace_size).  Strides are non-negative multiples of
 * 8 elements below 2^31, row strides at most 2^24; input rows may overlap (a shared
 * head), output rows (o, dq, dk, dv) may not (checked: sorted by stride,
 * each stride covers the span of the dimensions below it).  Pointers as
 * for attn_fwd_cross / attn_bwd_cross.  Errors as there, and
 * ATTN_ERR_INVALID_ARG for a null, misaligned or overlapping stride set.
 */
attn_status_t attn_fwd_strided(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                               void* o, float* lse, int batch, int heads, int seq_q, int seq_k,
                               int head_dim, const int* kv_len, const long long* strides,
                               int causal, float scale, void* stream);
attn_status_t attn_bwd_strided(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                               const void* o, const void* dout, const float* lse, void* dq,
                               void* dk, void* dv, void* workspace, size_t workspace_bytes,
                               int batch, int heads, int seq_q, int seq_k, int head_dim,
                               const int* kv_len, const long long* strides, int causal,
                               float scale, void* stream);

/*
 * Rotary position embedding and row-layout change, one memory-bound pass
 * (the pages' axial RoPE in front of attention, Section 5.2, and their
 * packed projection forms, Section 3.2).  For every (b, h, s) < (batch,
 * heads, seq) it reads row s of head h of batch b of src and writes row
 * (b, h, s) of dst, each row head_dim contiguous elements at
 *   b*strides[0] + h*strides[1] + s*strides[2]      (elements, not bytes).
 * [B,H,S,D] row-major is strides {H*S*D, S*D, D}; [B,S,H,D] is
 * {S*H*D, D, H*D}; a packed [B,S,3,H,D] projection holds Q, K, V at element
 * offsets 0, H*D, 2*H*D (src = base + offset) with strides {S*3*H*D, D, 3*H*D}.
 *   cos_table, sin_table  NULL (a plain copy) or DEVICE float32 tables
 *                          [table_rows][head_dim/2]; row s uses table row
 *                          pos_offset + s, which must be < table_rows
 *   transpose = 0: y_i = x_i c - x_{i+D/2} s, y_{i+D/2} = x_{i+D/2} c + x_i s
 *               (pair (i, i + D/2) turned by the angle of cosine c, sine s:
 *               the rotate-half RoPE; 1-D and axial positions differ only
 *               in the tables);
 *   transpose = 1: the transposed rotation (angle negated), which maps the
 *               gradient with respect to the rotated rows back to the rows.
 * dtype: ATTN_F32 and ATTN_F32_BF16FWD (float32 tensors, arithmetic in
 * float32) or ATTN_BF16 (bf16 tensors, rotation in float32, one rounding to
 * bf16 per output).  src and dst are 16-byte aligned device pointers; strides
 * are non-negative multiples of 8 elements.  The rows written must not
 * overlap each other; dst may equal src with the same strides (in place).
 * Errors: ATTN_ERR_INVALID_ARG (null or misaligned pointers, bad strides,
 * only one table, a table too short, transpose not 0/1, sizes <= 0),
 * ATTN_ERR_UNSUPPORTED (dtype, head_dim), ATTN_ERR_HIP (launch failure).
 */
attn_status_t attn_rope_copy(attn_dtype_t dtype, const void* src, const long long* src_strides,
                             void* dst, const long long* dst_strides, const float* cos_table,
                             const float* sin_table, int table_rows, int pos_offset, int batch,
                             int heads, int seq, int head_dim, int transpose, void* stream);

/*
 * Attention with RoPE on Q and K, fused into the kernels (axial RoPE in front
 * of the attention, Section 5.2, on the packed projection forms of Section
 * 3.2): self-attention (seq_q = seq_k = seq) on strided Q, K, V, O, with
 * query and key i turned by the angles of table row pos_offset + i -- the
 * result of attn_rope_copy (transpose = 0) on Q and K, then
 * attn_fwd_strided / attn_bwd_strided on the turned rows, then the
 * transposed rotation of dQ and dK -- with no pass of its own:
 *   attn_fwd_rope turns the Q and K tiles inside the forward kernel as they
 *     arrive in on-chip memory, and stores every turned Q and K row once
 *     into qk_rot;
 *   attn_bwd_rope reads the turned Q and K from qk_rot and applies the
 *     transposed rotation to dQ and dK in the kernels that store them, in
 *     float32 before the one rounding to the storage type.
 *   strides    HOST int64 (batch, head, row) strides as for
 *              attn_fwd_strided: attn_fwd_rope 12 values for q, k, v, o;
 *              attn_bwd_rope 18 values for v, o, dout, dq, dk, dv.
 *   qk_rot     DEVICE buffer of 2*batch*heads*seq*head_dim elements of the
 *              tensors' storage type (float32, or bf16 for ATTN_BF16),
 *              16-byte aligned, owned by the caller: turned Q at element 0,
 *              turned K at element batch*heads*seq*head_dim, each
 *              [B,H,S,D] row-major (heads*seq*head_dim < 2^31).  Written by
 *              attn_fwd_rope, read by attn_bwd_rope; it must not overlap
 *              any other argument.
 *   cos_table, sin_table  DEVICE float32 [table_rows][head_dim/2], 16-byte
 *              aligned (row p: the cosines and sines of the angles of
 *              position p; 1-D and axial RoPE differ only in these tables);
 *              pos_offset >= 0 and pos_offset + seq <= table_rows.
 * Every other argument, the workspace (attn_bwd_workspace_size of the same
 * shape) and the dtypes are as for attn_fwd_strided / attn_bwd_strided
 * (ATTN_F32_BF16FWD: the forward's operands, turned in float32, are
 * rounded to bf16 as they enter the MFMA).  Turned values are rounded
 * exactly as attn_rope_copy rounds them, so the turned Q and K in qk_rot
 * equal attn_rope_copy's output.  Errors as for the strided entry points,
 * and ATTN_ERR_INVALID_ARG for missing or misaligned tables, a table too
 * short, or a null or misaligned qk_rot.  Calls that overlap on one stream
 * order as usual; nothing is allocated.
 */
attn_status_t attn_fwd_rope(attn_dtype_t dtype, const void* q, const void* k, const void* v,
                            void* o, float* lse, void* qk_rot, int batch, int heads, int seq,
                            int head_dim, const long long* strides, const float* cos_table,
                            const float* sin_table, int table_rows, int pos_offset, int causal,
                            float scale, void* stream);
attn_status_t attn_bwd_rope(attn_dtype_t dtype, const void* qk_rot, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            void* workspace, size_t workspace_bytes, int batch, int heads, int seq,
                            int head_dim, const long long* strides, const float* cos_table,
                            const float* sin_table, int table_rows, int pos_offset, int causal,
                            float scale, void* stream);

/* Static, human-readable name of a status code. */
const char* attn_status_string(attn_status_t status);

/* Library version string ("<major>.<minor>.<patch>"). */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_ATTN_H */
