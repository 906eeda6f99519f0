// Internal declarations shared by the host side of the C interface and the
// kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sla {

// Problem shape with derived block counts.
struct Shape {
  int B, H, N, d, bq, bk, dtype;
  int Nq, Nk;  // ceil(N / bq), ceil(N / bk)
  long long R() const { return (long long)B * H * Nq; }
  int words() const { return (Nk + 31) / 32; }  // bitmask words per mask row
};

// Byte offsets of the workspace regions (all 256-byte aligned).
struct WsLayout {
  size_t qbar, kbar;   // pooled means, double [B*H*Nq*d], [B*H*Nk*d]
  size_t qhat;         // router only: q_bar W_q W_k^T, double [B*H*Nq*d]
  size_t wqk;          // router only: W_q W_k^T, double [d*d]
  size_t S;            // pooled logits, double [B*H*Nq*Nk]
  size_t counts;       // int32 [R]
  size_t bits;         // uint32 [R * words]
  size_t hpart;        // linear summary partials, float [B*H*nchunk*(d*d + d)]
  size_t htot;         // linear summaries, float [B*H*(d*d + d)]: H then z; the
                       // bf16 path keeps H in MFMA fragment order (32 x 32 tile
                       // (mt, nt), lane, element), the fp32 path row-major
  size_t pk;           // bf16 path: phi(K), bf16 [B*H][d/32][Nk*bk][32] (keys >= N zero)
  size_t total;
  int nchunk;          // key-block chunks per head in the summary pass
  int chunk_blocks;    // key blocks per chunk
};

WsLayout ws_layout(const Shape& s, bool router);
// the mask's regions only (qbar, kbar, qhat, wqk, S, counts, bits), from offset 0
WsLayout mask_layout(const Shape& s, bool router);

// Byte offsets of the 8-bit sparse branch buffer (all 256-byte aligned).
struct I8Layout {
  size_t q8;     // int8 [B*H][Nq*bq][d], rows >= N zero
  size_t k8;     // int8 [B*H][Nk*bk][d], rows >= N zero
  size_t vt8;    // int8 [B*H][Nk*bk/64][d][64]: V^T in 64-key tiles (P operand key order)
  size_t sq;     // float [B*H][Nq]
  size_t sk;     // float [B*H][Nk]
  size_t sv;     // float [B*H][d]
  size_t rv;     // float [B*H][d]: 127 / amax of each V channel (0 for amax 0)
  size_t vpart;  // float [B*H][vchunks][d]: channel maxima of 1024-row chunks
  size_t total;
  int vchunks;
};

I8Layout i8_layout(const Shape& s);

// Byte offsets of the sparse-branch backward workspace (256-byte aligned).
struct BwdLayout {
  size_t bits;     // uint32 [R * words]: the mask's rows as bitmasks
  size_t counts;   // int32 [B*H*Nk*ceil(Nq/64)]: rows listing each key block, per 64-row chunk
  size_t col_ptr;  // int32 [B*H*Nk + 1]: the mask's transpose (CSC)
  size_t row_idx;  // int32 [B*H*Nq*Nk]: query block indices, ascending per column
  size_t order;    // int32 [B*H*Nk*(bk/64)]: the column kernels' 64-key units, most-listed key blocks first
  size_t lse2;     // float [R*bq]: log2-sum-exp of the scaled scores per query (+inf past N)
  size_t dd;       // float [R*bq]: D = dO . O per query (0 past N)
  size_t apart;    // double [B*H][achunks]: partial sums of the alpha gradient
  // linear-branch backward
  size_t phiq, phik;    // bf16 [B*H][N][d]: phi(Q), phi(K)
  size_t rsplit;        // uint4 2 x [B*H][(d/32)(d/16)*2][64]: two totals as hi + lo bf16 matrix-core fragments
  size_t invden, dt;    // float [R*bq]: 1 / linear denominator and h.O_l per query (0 where undefined)
  size_t tot_h, tot_m;  // float [B*H][d*d + d]: (H, z) and (M, m), row-major
  size_t lpart;         // float [B*H][lchunks][d*d + d]: chunk partials of those totals
  size_t total;
  int achunks;     // chunks of 65536 elements per (b, h) slice
  int lchunks;     // chunks of LROWS rows per head for the linear totals
};
constexpr int LROWS = 512;

BwdLayout bwd_layout(const Shape& s);

// Mode of the attention kernels.
enum Mode : int {
  MODE_SPARSE = 0,  // O = O_s over the CSR row
  MODE_LINEAR = 1,  // O = O_l over the complement of the CSR row
  MODE_FUSED = 2,   // O = alpha_h O_s + (1 - alpha_h) O_l
  MODE_DENSE = 3,   // O = softmax attention over every key block
};

// What the fused forward keeps for the backward of a training step (device
// pointers, all set; see sla_fused_fwd_save).  Per-query arrays are indexed
// by mask row and position in the query block: row * bq + t.
struct FwdSaved {
  float* lse2;     // float [R*bq]: log2-sum-exp of the scaled sparse-branch scores (+inf: no listed key, or past N)
  float* invden;   // float [R*bq]: 1 / the linear-branch denominator (0: no linear branch, or past N)
  float* os;       // float [B,H,N,d]: the sparse branch's output O_s
  float* ol;       // float [B,H,N,d]: the linear branch's output O_l
};
// The same, read by the backward.
struct BwdSaved {
  const float* lse2;
  const float* invden;
  const float* os;
  const float* ol;
};

// mask.hip: pooling, optional router, pooled logits, selection, CSR.
// kdone (device [H], nullable): the pooled K of every head whose value there
// is not exactly 1 is already in the workspace (written by the preparation
// pass), so only Q and the other heads' K are pooled.
hipError_t launch_mask(const Shape& s, int k, double p, const float* Wq, const float* Wk,
                       const void* Q, const void* K, int32_t* row_ptr, int32_t* col_idx,
                       double* logits_out, char* ws, const WsLayout& L, hipStream_t st,
                       const float* kdone = nullptr);

// mask.hip: the SoftTop-k weights [B*H*Nq, Nk] (float32) from the pooled
// (and optionally routed) logits.
hipError_t launch_soft_topk(const Shape& s, int k, double T, const float* Wq, const float* Wk,
                            const void* Q, const void* K, float* M, char* ws, const WsLayout& L,
                            hipStream_t st);

// attn_bf16.hip: the K/V preparation pass for the linear branch (phi(K) in
// 32-wide d slices and the per-head linear totals; nothing without lin;
// heads whose alpha is exactly 1 are skipped when alpha is given; kmeans:
// also the pooled K of the heads it processes, for the mask) and the
// attention kernels.
hipError_t launch_prep_bf16(const Shape& s, bool lin, const void* K, const void* V, const float* alpha,
                            bool kmeans,
                            char* ws, const WsLayout& L, hipStream_t st);
// saved (nullable, MODE_FUSED only): also write the per-query terms and the
// branch outputs the backward of a training step reads.
hipError_t launch_attn_bf16(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                            const int32_t* row_ptr, const int32_t* col_idx, const float* alpha,
                            const char* ws, const WsLayout& L, void* O, hipStream_t st,
                            const FwdSaved* saved = nullptr);
hipError_t launch_summary_reduce(const float* hpart, const float* alpha, int H, long long BH,
                                 int nchunk, int per, float* htot, hipStream_t st);

// attn_i8.hip: the 8-bit codes and scales of Q, K, V, and the 8-bit sparse
// branch over them.
hipError_t launch_quant_i8(const Shape& s, const void* Q, const void* K, const void* V, char* qbuf,
                           const I8Layout& L, hipStream_t st);
hipError_t launch_attn_i8(const Shape& s, const char* qbuf, const I8Layout& L, const int32_t* row_ptr,
                          const int32_t* col_idx, void* O, hipStream_t st);
// attn_i8.hip as well: int8 Q, K and E4M3 V codes (same buffer layout, V^T
// tiles in the key order of a 64-key P operand) and the single-pass sparse
// branch over them (int8 scores, E4M3 P V).
hipError_t launch_quant_i8f8(const Shape& s, const void* Q, const void* K, const void* V, char* qbuf,
                             const I8Layout& L, hipStream_t st);
hipError_t launch_attn_i8f8(const Shape& s, const char* qbuf, const I8Layout& L, const int32_t* row_ptr,
                            const int32_t* col_idx, void* O, hipStream_t st);

// attn_bwd.hip: gradient of the sparse branch (bf16) with the mask fixed.
// alpha (device [H], nullable): the outputs are scaled by alpha_h, the
// branch's weight in the mixed output; csc: build the mask's transpose into
// ws first (else it is already there, from a call on the same mask).
// saved (nullable): the forward's lse2 and O_s, so the row kernel skips the
// pass that recomputes them (D = dO . O_s per query).
hipError_t launch_sparse_bwd(const Shape& s, const void* Q, const void* K, const void* V, const void* dO,
                             const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK, void* dV,
                             const float* alpha, bool csc, char* ws, const BwdLayout& L, hipStream_t st,
                             const BwdSaved* saved = nullptr);
hipError_t launch_alpha_grad(const Shape& s, const void* dO, const void* Os, const void* Ol, float* dalpha,
                             char* ws, const BwdLayout& L, hipStream_t st);
// the same from the per-query terms D = dO . O_s and D~ = dO . O_l that the
// row kernels of a backward call with the forward's terms left in ws
hipError_t launch_alpha_grad_terms(const Shape& s, float* dalpha, char* ws, const BwdLayout& L, hipStream_t st);
// the mask's transpose (CSC) into the backward workspace
hipError_t launch_csc(const Shape& s, const int32_t* row_ptr, const int32_t* col_idx, char* ws, const BwdLayout& L,
                      hipStream_t st);
// attn_bwd_lin.hip: gradient of the linear branch (bf16) with the mask fixed;
// accumulate: add to dQ, dK, dV instead of writing them; alpha (nullable):
// the outputs are scaled by 1 - alpha_h; csc as for the sparse branch.
// saved (nullable): the forward's invden and O_l, so the row kernel skips
// the pass that recomputes them (D~ = dO . O_l per query).
hipError_t launch_linear_bwd(const Shape& s, const void* Q, const void* K, const void* V, const void* dO,
                             const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK, void* dV,
                             bool accumulate, const float* alpha, bool csc, char* ws, const BwdLayout& L,
                             hipStream_t st, const BwdSaved* saved = nullptr);

// attn_f32.hip: linear totals and attention for float32 inputs.
hipError_t launch_summary_f32(const Shape& s, const void* K, const void* V, const float* alpha,
                              char* ws, const WsLayout& L, hipStream_t st);
hipError_t launch_attn_f32(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                           const int32_t* row_ptr, const int32_t* col_idx, const float* alpha,
                           const float* htot, void* O, hipStream_t st);

}  // namespace sla
