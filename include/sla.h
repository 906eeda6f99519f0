/*
 * sla.h - C interface of the MI355X (gfx950) sparse + linear attention: the
 * forward, its 8-bit sparse branch, the SoftTop-k weights and the backward.
 *
 * The library computes, for attention inputs Q, K, V of shape [B, H, N, d]:
 *
 *   1. a block mask: Q and K are cut into blocks of bq and bk tokens and
 *      mean-pooled per block; the pooled vectors (optionally passed through
 *      two router matrices) give block logits S_ij = q_i . k_j / sqrt(d) and a
 *      row softmax P; each query block keeps the union of its Top-k blocks
 *      (k = ceil(k_frac * Nk)) and its Top-p blocks (the shortest
 *      largest-first prefix whose probability mass reaches p).  Sources: the
 *      SpargeAttention2 write-up "清華發明AI「注意力瘦身術」：視頻生成速度提升16倍
 *      的神奇技術" (arXiv:2602.13515), §一 (hybrid Top-k / Top-p) and §四
 *      (pool, select, block-level mask);
 *   2. the sparse branch: exact softmax attention of each query over the keys
 *      of its selected blocks only (SLA2 write-up, arXiv:2602.12675, §一);
 *   3. the linear branch: linear attention with phi(x) = elu(x) + 1 over the
 *      keys of the blocks NOT selected (SLA2 write-up §一), and the mix
 *      O = alpha_h * O_sparse + (1 - alpha_h) * O_linear with one alpha per
 *      head (SLA2 write-up §二);
 *   4. with the mask held fixed, the gradients of both branches, of the mix
 *      and of alpha (SLA2 write-up §四: training with the selection fixed
 *      per step), bf16; optionally from per-query terms the forward kept
 *      (sla_fused_fwd_save, sla_attn_bwd_saved).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  Q, K, V and
 *     outputs are contiguous [B, H, N, d] (d fastest) in the problem dtype
 *     (fp32 or bf16).  Blocks are consecutive tokens; the last block of a
 *     sequence may be partial.
 *   - The mask is CSR over rows r = (b * H + h) * Nq + i: row_ptr int32
 *     [R + 1], col_idx int32 (key-block indices ascending within a row),
 *     with Nq = ceil(N / bq), Nk = ceil(N / bk), R = B * H * Nq.
 *   - The library never allocates device memory and never synchronises.
 *     Scratch space comes from the caller's workspace (size from
 *     sla_workspace_bytes).  All work is enqueued on the caller's HIP stream
 *     (a hipStream_t passed as void*; NULL = the default stream).
 *   - Every function returns a status: SLA_OK (0) or a negative code.
 *     Argument errors are detected on the host before anything is launched
 *     and nothing is then written.  SLA_ERR_HIP reports a launch failure.
 *   - No global state, except the static scratch of sla_mask_noalloc (see
 *     there): other calls on different streams may run concurrently as long
 *     as their workspaces and outputs do not overlap.
 *   - Supported: dtype fp32 or bf16; d in {64, 128}; bq, bk in {64, 128};
 *     Nk <= 4096; B * H * N * d < 2^31.
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sla_dtype { SLA_F32 = 0, SLA_BF16 = 1 };

enum sla_status {
  SLA_OK = 0,
  SLA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, k_frac/p outside [0,1] or NaN */
  SLA_ERR_UNSUPPORTED = -2, /* d, bq, bk, dtype or size outside the supported set */
  SLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than sla_workspace_bytes */
  SLA_ERR_CAPACITY = -4,    /* col_idx capacity below B*H*Nq*Nk */
  SLA_ERR_HIP = -5,         /* a kernel launch failed */
  SLA_ERR_TOO_LARGE = -6    /* problem exceeds the static scratch of sla_mask_noalloc */
};

/* Problem shape.  dtype is an sla_dtype value. */
typedef struct sla_problem {
  int32_t B, H, N, d;
  int32_t bq, bk;
  int32_t dtype;
} sla_problem;

/* Selection parameters.
 *   k_frac  Top-k fraction in [0, 1]; k = ceil(k_frac * Nk - 1e-9) computed
 *           in double from this float.
 *   p       Top-p mass threshold in [0, 1]; the block whose cumulative mass
 *           first reaches p is kept; p = 0 keeps none by Top-p.
 *   Wq, Wk  optional router matrices (both or neither), DEVICE fp32 [d, d]
 *           row-major, shared by all heads: q_hat = q_bar . Wq (row vector
 *           times matrix), k_hat = k_bar . Wk.  SLA2 write-up §二: a learnable
 *           router of two projection matrices. */
typedef struct sla_select {
  float k_frac;
  float p;
  const float* Wq;
  const float* Wk;
} sla_select;

/* Bytes of device workspace every entry point below needs for this problem
 * (host-only arithmetic; 0 on invalid arguments).  sel may be NULL (no router). */
size_t sla_workspace_bytes(const sla_problem* prob, const sla_select* sel);

/* Worst-case number of mask entries, B * H * Nq * Nk (the col_idx capacity the
 * mask calls require), or -1 on invalid arguments. */
int64_t sla_mask_capacity(const sla_problem* prob);

/* SoftTop-k weights of every mask row (SLA2 write-up §四: in the router's
 * first training stage the hard Top-k is replaced by a sigmoid with a
 * temperature).  For row i of the pooled (and, with sel->Wq / Wk, routed)
 * logits S: M_ij = sigmoid((S_ij - tau_i) / T), with tau_i the threshold at
 * which the row's weights sum to k = ceil(k_frac * Nk); k = 0 gives zeros and
 * k = Nk ones.  sel->p is not used.
 *   T       temperature, finite and > 0
 *   Q, K    inputs [B, H, N, d]
 *   M       out, DEVICE float32 [B*H*Nq, Nk] (rows in (b, h, i) order)
 *   ws      workspace (>= sla_workspace_bytes(prob, sel))
 * Returns SLA_ERR_INVALID_ARG for T <= 0, non-finite T or a NULL pointer. */
int sla_soft_topk(const sla_problem* prob, const sla_select* sel, float T, const void* Q, const void* K,
                  float* M, void* ws, size_t ws_bytes, void* stream);

/* Build the block mask (SpargeAttention2 write-up §一, §四).
 *   Q, K          inputs [B, H, N, d]
 *   row_ptr       out, int32 [B*H*Nq + 1]; row_ptr[R] is the number of entries
 *   col_idx       out, int32 [capacity]; entries past row_ptr[R] are untouched
 *   capacity      must be >= sla_mask_capacity(prob)
 *   block_logits  optional out, double [B, H, Nq, Nk]: the pooled logits S that
 *                 the selection used (for inspection); NULL to skip
 *   ws, ws_bytes  workspace (>= sla_workspace_bytes) */
int sla_mask(const sla_problem* prob, const sla_select* sel, const void* Q, const void* K,
             int32_t* row_ptr, int32_t* col_idx, int64_t capacity, double* block_logits,
             void* ws, size_t ws_bytes, void* stream);

/* sla_mask without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, result and errors as sla_mask (no
 * block_logits).  Its scratch is a file-scope device array of
 * SLA_NOALLOC_SCRATCH_BYTES (64 MiB) that every GPU the library runs on holds
 * from the library's load until the process ends; the call allocates and
 * frees nothing.  Problems whose mask scratch (the pooled means, the pooled
 * logits, the per-row counts and bitmasks; sla_mask_noalloc_bytes) exceeds
 * it return SLA_ERR_TOO_LARGE before anything is launched - the 480p
 * workloads without the router need about 22 MB.  The array of the CURRENT
 * device is used: a non-NULL stream must belong to it (else
 * SLA_ERR_INVALID_ARG).  All calls on one GPU share its array, so calls that
 * overlap in time on one GPU (different streams, or host threads) race and
 * must be serialised by the caller; calls on one stream are ordered and safe.
 * Every word the kernels read from the array is written earlier in the same
 * call, so nothing depends on what a previous call left there. */
#define SLA_NOALLOC_SCRATCH_BYTES (64u << 20)
size_t sla_mask_noalloc_bytes(const sla_problem* prob, const sla_select* sel);
int sla_mask_noalloc(const sla_problem* prob, const sla_select* sel, const void* Q, const void* K,
                     int32_t* row_ptr, int32_t* col_idx, int64_t capacity, void* stream);

/* Sparse branch alone (SLA2 write-up §一): O_s[t] = softmax over the keys of the
 * blocks listed in row (b, h, t / bq) of the mask, of q_t . k / sqrt(d), times V.
 * Rows with no selected block are written as 0.  Output O_s [B, H, N, d].
 * Needs no workspace: K and V are read as they are. */
int sla_sparse_fwd(const sla_problem* prob, const void* Q, const void* K, const void* V,
                   const int32_t* row_ptr, const int32_t* col_idx, void* O_s, void* stream);

/* Linear branch alone (SLA2 write-up §一): O_l[t] = sum_u (phi(q_t).phi(k_u)) v_u /
 * sum_u phi(q_t).phi(k_u) over the keys u of the blocks NOT listed in the row;
 * phi(x) = elu(x) + 1.  Rows whose blocks are all listed are written as 0.
 * Output O_l [B, H, N, d].  Needs the workspace. */
int sla_linear_fwd(const sla_problem* prob, const void* Q, const void* K, const void* V,
                   const int32_t* row_ptr, const int32_t* col_idx, void* O_l,
                   void* ws, size_t ws_bytes, void* stream);

/* The whole forward: mask, then O = alpha_h * O_s + (1 - alpha_h) * O_l
 * (SLA2 write-up §二), written once in the input dtype (for bf16 the K/V
 * preparation pass runs first and pools K for the mask; see below).
 *   alpha    DEVICE fp32 [H], each in [0, 1]; a branch whose weight is exactly
 *            0 for a head is not evaluated for that head
 *   row_ptr, col_idx, capacity   the mask, returned as by sla_mask */
int sla_attn_fwd(const sla_problem* prob, const sla_select* sel, const void* Q, const void* K,
                 const void* V, const float* alpha, void* O, int32_t* row_ptr,
                 int32_t* col_idx, int64_t capacity, void* ws, size_t ws_bytes, void* stream);

/* The stages of sla_attn_fwd, for callers that time or schedule them
 * separately: sla_attn_fwd == sla_kv_prepare, sla_mask_prepared, then
 * sla_fused_fwd, on one workspace (sla_mask, sla_kv_prepare, sla_fused_fwd
 * gives the same mask and output and reads K once more).
 *
 * sla_kv_prepare: one pass over K and V that leaves in the workspace what the
 * fused stage reads: the per-head linear-attention totals H = sum_u phi(k_u)^T
 * v_u ([d, d]) and z = sum_u phi(k_u) ([d]) over every key (float32) and, for
 * bf16, phi(K) in 32-wide d slices (bf16 [B, H, d/32, Nk*bk, 32], keys past N
 * zero).  V is not copied: the attention kernels read V and K as the caller
 * passed them.  alpha (DEVICE fp32 [H]) may be NULL; heads whose alpha is
 * exactly 1 skip the pass when it is given.  For bf16 the pass also writes the
 * mean of every key block of the heads it processes (the mask's pooled K,
 * float64 sums of the bf16 values) into the workspace.
 *
 * sla_mask_prepared: sla_mask (same arguments and outputs, no block_logits)
 * for a workspace on which sla_kv_prepare has just run with the same K and
 * alpha: it pools Q and only the K of the heads that pass skipped (alpha
 * exactly 1; every head for fp32, whose pass writes no key-block means).  The
 * result is identical to sla_mask's.  Calling it without that pass is
 * undefined.
 *
 * sla_fused_fwd: O = alpha_h * O_s + (1 - alpha_h) * O_l over the given mask,
 * with O_l = phi(q) (H - G) / phi(q) (z - g), where G, g are the same sums
 * over the listed blocks only (SLA2 write-up §一, §二).  It reads what
 * sla_kv_prepare left in the SAME workspace for the same K, V and alpha;
 * calling it without that is undefined. */
int sla_kv_prepare(const sla_problem* prob, const void* K, const void* V, const float* alpha,
                   void* ws, size_t ws_bytes, void* stream);
int sla_mask_prepared(const sla_problem* prob, const sla_select* sel, const void* Q, const void* K,
                      const float* alpha, int32_t* row_ptr, int32_t* col_idx, int64_t capacity,
                      void* ws, size_t ws_bytes, void* stream);
int sla_fused_fwd(const sla_problem* prob, const void* Q, const void* K, const void* V,
                  const float* alpha, const int32_t* row_ptr, const int32_t* col_idx, void* O,
                  const void* ws, size_t ws_bytes, void* stream);

/* sla_fused_fwd for a training step: the same output O (bit for bit), and
 * also what the backward of the step reads back from the forward instead of
 * recomputing it (sla_attn_bwd_saved), all written by the same launch:
 *   lse2    float32 [sla_saved_terms_count] (DEVICE): for query t of mask row
 *           r = (b, h, i) at lse2[r * bq + t - i * bq], log2 of the sparse
 *           branch's softmax normaliser, sum over its listed keys u of
 *           exp2(c q.k_u), c = log2(e) / sqrt(d) (SLA2 write-up §一 with the
 *           textbook softmax); +inf where the row lists no block and past N;
 *   invden  float32, same layout: 1 / sum over the unlisted keys of
 *           phi(q).phi(k_u), the linear branch's denominator (SLA2 write-up
 *           §一); 0 where the row has no linear branch (every block listed)
 *           and past N;
 *   O_s, O_l  float32 [B, H, N, d]: the two branches' outputs (0 for a
 *           branch a row does not have).  float32, not bf16: the backward
 *           forms each query's D = dO . O_s from them, and the sparse
 *           branch's dQ carries D's error times the listed keys' common
 *           component (a bf16 O_s puts dQ about 1.5% off on the tests'
 *           inputs, float32 below 0.3%).
 * The sparse branch is computed for every head, also where alpha_h is 0; the
 * linear branch reads the totals of sla_kv_prepare, which skips heads whose
 * alpha is exactly 1: there O_l and invden hold 0 (the branch has no weight
 * in O, nor in the gradients of Q, K, V; the alpha gradient of such a head
 * would need O_l from sla_linear_fwd).
 * bf16 only (SLA_ERR_UNSUPPORTED otherwise); every pointer required.  The
 * extra writes cost about 2 * B*H*N*d*4 bytes of HBM traffic. */
int64_t sla_saved_terms_count(const sla_problem* prob);
int sla_fused_fwd_save(const sla_problem* prob, const void* Q, const void* K, const void* V,
                       const float* alpha, const int32_t* row_ptr, const int32_t* col_idx, void* O,
                       const void* ws, size_t ws_bytes, float* lse2, float* invden, float* O_s, float* O_l,
                       void* stream);

/* Dense attention softmax(Q K^T / sqrt(d)) V over every key: the textbook
 * formula that the explainer page "清华SpargeAttention2技术解析：如何让AI视频
 * 生成提速16倍" prints in its section 3 (implementation principle) as the
 * conventional computation the sparse path replaces; here it is the
 * comparator the sparse path is measured against.  Output O [B, H, N, d] in
 * the problem dtype (bq, bk only set the tiling).  Needs no workspace. */
int sla_dense_fwd(const sla_problem* prob, const void* Q, const void* K, const void* V, void* O,
                  void* stream);

/* ---- 8-bit sparse branch (SLA2 write-up §三: the sparse branch holds Q, K,
 * the attention probabilities P and V as 8-bit integers, scaled into the
 * 8-bit range and scaled back).  The granularity and rounding, which that
 * section leaves open, are:
 *   - symmetric codes in [-127, 127]: code = round-half-even(x * fl32(127 /
 *     amax)), scale = fl32(amax / 127) (amax = 0: scale 0, codes 0); Q has one
 *     scale per query block, K one per key block, V one per channel (d index)
 *     over the whole sequence of a head;
 *   - integer scores I = q8 . k8, S = fl32(I * c) with c = fl32(fl32(sq * sk)
 *     * fl32(1 / sqrt(d))), m = the row's largest S over its listed keys;
 *   - P codes = round-half-even(exp2(fma(I, a, -b))) in [0, 127], a = fl32(c *
 *     log2 e), b = fl32(fl32(m * log2 e) - log2 127): 127 exp(S - m) taken in
 *     float32 (exp2 by the hardware instruction, within an ulp);
 *   - O_s = sv * (sum_j code_j v8_j) / (sum_j code_j) from exact int32 sums;
 *     a row with no listed block gives 0.
 *
 * The quantised buffer (caller-owned device memory, qbuf_bytes >= total):
 *   q8     int8  [B*H][Nq*bq][d]   row-major, rows >= N zero
 *   k8     int8  [B*H][Nk*bk][d]   row-major, rows >= N zero
 *   vt8    int8  [B*H][Nk*bk/64][d][64]   V^T in tiles of 64 keys: key k of a
 *                tile sits at byte 32(k/32) + 16((k/4)%2) + 4((k%32)/8) + k%4
 *                of its channel's 64-byte row (keys >= N zero)
 *   sq     float [B*H][Nq],  sk float [B*H][Nk],  sv float [B*H][d]
 *   rv     float [B*H][d]    127 / amax per V channel (0 for amax 0)
 *   vpart  float [B*H][ceil(N/1024)][d]   channel maxima of 1024-row chunks
 * at the byte offsets sla_i8_layout_of returns (each 256-byte aligned).
 * Supported as for the other calls, and N <= 131072 (the int32 sums then
 * cannot overflow).  Inputs must be finite. */
typedef struct {
  size_t q8, k8, vt8, sq, sk, sv, rv, vpart, total;
} sla_i8_layout;

/* Offsets and total size of the quantised buffer for this problem. */
int sla_i8_layout_of(const sla_problem* prob, sla_i8_layout* layout);

/* Quantise Q, K, V (problem dtype) into qbuf. */
int sla_quantize_i8(const sla_problem* prob, const void* Q, const void* K, const void* V,
                    void* qbuf, size_t qbuf_bytes, void* stream);

/* The sparse branch on the codes in qbuf (as left by sla_quantize_i8), over
 * the CSR mask; writes O_s [B, H, N, d] in the problem dtype. */
int sla_sparse_fwd_i8(const sla_problem* prob, const void* qbuf, size_t qbuf_bytes,
                      const int32_t* row_ptr, const int32_t* col_idx, void* O_s, void* stream);

/* ---- The 8-bit sparse branch in one pass (SLA2 write-up §三): Q and K as the
 * integer codes above, P and V as 8-bit floating-point values in the E4M3
 * format of the OCP 8-bit floating-point specification (4 exponent bits with
 * bias 7, 3 mantissa bits, largest finite value 448), whose headroom lets the
 * row maximum rise while the row is being summed.  Where that section is
 * silent:
 *   - q8, k8, sq, sk exactly as sla_quantize_i8 makes them; V per channel:
 *     code = E4M3(fl32(x * fl32(448 / amax))) (nearest, ties to even), scale
 *     sv = fl32(amax / 448);
 *   - I = q8 . k8 exact, S = fl32(I * c), c = fl32(fl32(sq * sk) * fl32(1 /
 *     sqrt(d)));
 *   - the row's keys in 64-key units in CSR order; m = the largest S so far,
 *     the current unit's included; P codes = E4M3(256 exp(S - m)), taken as
 *     E4M3(exp2(fma(I, fl32(c log2 e), -(fl32(m log2 e) - 8)))) in float32;
 *     when m rises, the sums of the earlier units are multiplied by
 *     exp(m_old - m_new);
 *   - O_s = sv * (sum code v8) / (sum code), the sums on the E4M3 matrix
 *     instruction in float32; 0 for an empty row.
 * The buffer has the layout of sla_i8_layout_of (q8, k8, sq, sk as above; vt8
 * E4M3 bytes, sv the E4M3 scales, rv 448 / amax), except that in vt8 key k of
 * a 64-key tile sits at byte 32((k/4)%2) + 16(k/32) + 4((k%32)/8) + k%4 of its
 * channel row.  Supported as the int8 calls.
 *
 * sla_quantize_i8f8: the codes and scales of Q, K, V into qbuf.
 * sla_sparse_fwd_i8f8: the single-pass sparse branch on them over the CSR
 * mask; writes O_s [B, H, N, d] in the problem dtype. */
int sla_quantize_i8f8(const sla_problem* prob, const void* Q, const void* K, const void* V,
                      void* qbuf, size_t qbuf_bytes, void* stream);
int sla_sparse_fwd_i8f8(const sla_problem* prob, const void* qbuf, size_t qbuf_bytes,
                        const int32_t* row_ptr, const int32_t* col_idx, void* O_s, void* stream);

/* ---- Backward of the sparse branch, mask fixed (SLA2 write-up §一 for the
 * branch, §四 for training the attention end to end with the selection fixed
 * per step).  For L = sum(O_s * dO_s), with P the softmax over each row's
 * listed keys and D_t = dO_s[t] . O_s[t] = sum_u P_tu dP_tu:
 *   dV = P^T dO_s,  dP = dO_s V^T,  dS = P o (dP - D),  dQ = dS K / sqrt(d),
 *   dK = dS^T Q / sqrt(d)   over the listed (query block, key block) pairs.
 * D is formed from its second expression in float32 (the forward output is
 * not needed).  bf16 only (SLA_ERR_UNSUPPORTED for fp32).  dO_s is the
 * gradient reaching O_s (alpha_h dO for the mixed output).  Outputs dQ, dK,
 * dV [B, H, N, d] bf16
 * (every element written; rows of keys no row lists get 0).  Needs a
 * workspace of sla_bwd_workspace_bytes (the mask's transpose, per-query
 * terms, the column kernels' launch order).  Deterministic: every sum runs
 * in a fixed order (integer atomics in LDS pick which workgroup runs which
 * key block first, which no result depends on). */
size_t sla_bwd_workspace_bytes(const sla_problem* prob);
int sla_sparse_bwd(const sla_problem* prob, const void* Q, const void* K, const void* V, const void* dO_s, const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK,
                   void* dV, void* ws, size_t ws_bytes, void* stream);

/* ---- Backward of the linear branch, mask fixed (SLA2 write-up §一 for the
 * branch: phi = elu + 1 linear attention over the keys of the blocks a row
 * does not select, normalised over those keys; §四 for training with the
 * selection fixed per step).  For L = sum(O_l * dO_l), a = phi(q_t),
 * w_tu = a . phi(k_u), den_t = sum over the row's unselected keys of w_tu,
 * D~_t = dO_l[t] . O_l[t] and dw_tu = (dO_l[t] . v_u - D~_t) / den_t:
 *   dq_t = phi'(q_t) o sum_u dw_tu phi(k_u),
 *   dv_u = sum_t (w_tu / den_t) dO_l[t],  dk_u = phi'(k_u) o sum_t dw_tu a_t,
 * every sum over the (query, key) pairs outside the listed blocks.  Each is
 * formed as the sum over all pairs (float32 per-head totals) minus the sum
 * over the listed pairs (bf16 matrix-core tiles, as in the sparse branch's
 * gradient).  Rows whose blocks are all listed contribute nothing.  bf16 only
 * (SLA_ERR_UNSUPPORTED for fp32).  dO_l is the gradient reaching O_l
 * ((1 - alpha_h) dO for the mixed output).  Outputs dQ, dK, dV [B, H, N, d]
 * bf16, every element written; with accumulate != 0 the results are added to
 * what the buffers hold (for example the sparse branch's gradient) and
 * rounded to bf16 once more.  Needs the sla_bwd_workspace_bytes workspace
 * (its contents on entry are ignored).  Deterministic, as sla_sparse_bwd. */
int sla_linear_bwd(const sla_problem* prob, const void* Q, const void* K, const void* V, const void* dO_l,
                   const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK, void* dV,
                   int accumulate, void* ws, size_t ws_bytes, void* stream);

/* ---- Backward of the mixed output, mask fixed (SLA2 write-up §二 for
 * O = alpha_h O_s + (1 - alpha_h) O_l, §四 for training with the selection
 * fixed per step).  dQ, dK, dV of L = sum(O * dO) with respect to Q, K, V:
 * the sparse branch's gradient (as sla_sparse_bwd) taken with dO and scaled
 * by alpha_h, plus the linear branch's (as sla_linear_bwd) taken with dO and
 * scaled by 1 - alpha_h; both branches' gradients are linear in the
 * incoming gradient, so the scales are applied to the float32 results.  The
 * mask's transpose is built once for both.  alpha: float32 [H] (DEVICE),
 * the forward's mixing ratios.  bf16 only.  Outputs dQ, dK, dV [B, H, N, d]
 * bf16, every element written (the sparse part rounded to bf16, the linear
 * part added and rounded again).  Needs the sla_bwd_workspace_bytes
 * workspace.  dalpha (DEVICE float32 [H], nullable): also the gradient with
 * respect to alpha, sum over the head's queries of dO . (O_s - O_l), formed
 * as the float64 sum of the per-query D = dO . O_s and D~ = dO . O_l that the
 * branches' row kernels compute anyway (float32, from the exact branch
 * outputs; sla_alpha_grad does the same from O_s and O_l given).
 * Deterministic, as sla_sparse_bwd. */
int sla_attn_bwd(const sla_problem* prob, const void* Q, const void* K, const void* V, const void* dO,
                 const float* alpha, const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK, void* dV,
                 float* dalpha, void* ws, size_t ws_bytes, void* stream);

/* sla_attn_bwd with the terms sla_fused_fwd_save kept for the same Q, K, V,
 * alpha and mask: the branches' row kernels take each query's normalisers
 * from lse2 and invden and its D = dO . O_s (sparse) and dO . O_l (linear)
 * from one dot product, instead of a first pass over the row's keys that
 * recomputes the scores.  Same outputs and rounding as sla_attn_bwd up to
 * those terms (the forward's normaliser sums its bf16-rounded
 * probabilities), so within the same tolerance of the exact gradient, not
 * bit for bit.  dalpha (DEVICE float32 [H], nullable): also the alpha
 * gradient, sum over the head's queries of dO . (O_s - O_l), formed as the
 * float64 sum of the per-query D - D~ the row kernels computed from the
 * float32 O_s and O_l (no further pass over dO).
 * Terms from another forward are undefined. */
int sla_attn_bwd_saved(const sla_problem* prob, const void* Q, const void* K, const void* V, const void* dO,
                       const float* alpha, const int32_t* row_ptr, const int32_t* col_idx, const float* lse2,
                       const float* invden, const float* O_s, const float* O_l, void* dQ, void* dK, void* dV,
                       float* dalpha, void* ws, size_t ws_bytes, void* stream);

/* Gradient of sum(O * dO) with respect to alpha for O = alpha_h O_s +
 * (1 - alpha_h) O_l (SLA2 write-up §二): dalpha[h] = sum over the head's
 * tokens of dO . (O_s - O_l), float64 partial sums in a fixed order, written
 * as float32 [H] (DEVICE).  dO, O_s, O_l in the problem dtype.  Needs the
 * sla_bwd_workspace_bytes workspace. */
int sla_alpha_grad(const sla_problem* prob, const void* dO, const void* O_s, const void* O_l, float* dalpha,
                   void* ws, size_t ws_bytes, void* stream);

/* Static text for a status code. */
const char* sla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */
