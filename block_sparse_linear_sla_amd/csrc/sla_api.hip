// Host side of the C interface: argument validation, workspace carving and
// the launch sequence of each entry point.  Nothing here synchronises, copies
// device memory to the host or allocates.
#include <math.h>

#include <mutex>

#include "sla.h"
#include "sla_internal.h"

namespace {

// Scratch of sla_mask_noalloc: one copy per GPU, resident from the load of
// the library's code object on that GPU until the process ends.  In host code
// the name is only a handle for hipGetSymbolAddress; the device address of
// each GPU's copy is looked up once per device and kept below.
__device__ __align__(256) char scratch[SLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first
// call on that device, with the device current).
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

}  // namespace


namespace sla {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const Shape& s, bool router) {
  WsLayout L{};
  const size_t BH = (size_t)s.B * s.H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  // What the preparation pass writes (linear summaries, phi(K), the pooled K)
  // comes first, so its offsets do not depend on the router: the pass can run
  // with either layout, before or after the mask, on the same workspace.
  // The preparation pass runs one workgroup per chunk of key blocks of a head;
  // chunks are sized so the grid is a single round at two workgroups per CU
  // (about 512), which keeps the per-chunk partials few.
  int nch = (int)(512 / BH);
  if (nch < 1) nch = 1;
  if (nch > s.Nk) nch = s.Nk;
  const int cb = (s.Nk + nch - 1) / nch;
  L.chunk_blocks = cb;
  L.nchunk = (s.Nk + cb - 1) / cb;
  const size_t per = (size_t)s.d * s.d + s.d;
  L.htot = take(BH * per * sizeof(float));
  L.hpart = take(BH * L.nchunk * per * sizeof(float));
  const bool bf = s.dtype == SLA_BF16;
  L.pk = bf ? take(BH * (size_t)s.Nk * s.bk * s.d * 2) : 0;
  L.qbar = take(BH * s.Nq * s.d * sizeof(double));
  L.kbar = take(BH * s.Nk * s.d * sizeof(double));
  L.qhat = router ? take(BH * s.Nq * s.d * sizeof(double)) : 0;
  L.wqk = router ? take((size_t)s.d * s.d * sizeof(double)) : 0;
  L.S = take(BH * s.Nq * s.Nk * sizeof(double));
  L.counts = take((size_t)s.R() * sizeof(int32_t));
  L.bits = take((size_t)s.R() * s.words() * sizeof(uint32_t));
  L.total = off;
  return L;
}

// The mask's regions alone (pooled means, router products, logits, counts,
// bitmasks), packed from offset 0: the scratch of the allocation-free mask.
WsLayout mask_layout(const Shape& s, bool router) {
  WsLayout L{};
  const size_t BH = (size_t)s.B * s.H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.qbar = take(BH * s.Nq * s.d * sizeof(double));
  L.kbar = take(BH * s.Nk * s.d * sizeof(double));
  L.qhat = router ? take(BH * s.Nq * s.d * sizeof(double)) : 0;
  L.wqk = router ? take((size_t)s.d * s.d * sizeof(double)) : 0;
  L.S = take(BH * s.Nq * s.Nk * sizeof(double));
  L.counts = take((size_t)s.R() * sizeof(int32_t));
  L.bits = take((size_t)s.R() * s.words() * sizeof(uint32_t));
  L.total = off;
  return L;
}

}  // namespace sla

using sla::Mode;
using sla::Shape;
using sla::WsLayout;

namespace {

// Validates the shape; fills s on success.
int check_problem(const sla_problem* p, Shape* s) {
  if (p == nullptr) return SLA_ERR_INVALID_ARG;
  if (p->B < 1 || p->H < 1 || p->N < 1 || p->d < 1 || p->bq < 1 || p->bk < 1) return SLA_ERR_INVALID_ARG;
  if (p->dtype != SLA_F32 && p->dtype != SLA_BF16) return SLA_ERR_UNSUPPORTED;
  if (p->d != 64 && p->d != 128) return SLA_ERR_UNSUPPORTED;
  if ((p->bq != 64 && p->bq != 128) || (p->bk != 64 && p->bk != 128)) return SLA_ERR_UNSUPPORTED;
  const long long elems = (long long)p->B * p->H * p->N * p->d;
  if (elems >= (1LL << 31)) return SLA_ERR_UNSUPPORTED;
  s->B = p->B; s->H = p->H; s->N = p->N; s->d = p->d; s->bq = p->bq; s->bk = p->bk;
  s->dtype = p->dtype;
  s->Nq = (p->N + p->bq - 1) / p->bq;
  s->Nk = (p->N + p->bk - 1) / p->bk;
  if (s->Nk > 4096) return SLA_ERR_UNSUPPORTED;
  if ((long long)s->B * s->H * s->Nq * s->Nk >= (1LL << 31)) return SLA_ERR_UNSUPPORTED;
  return SLA_OK;
}

int check_select(const sla_select* sel, int* k, const Shape& s) {
  if (sel == nullptr) return SLA_ERR_INVALID_ARG;
  const float kf = sel->k_frac, p = sel->p;
  if (!(kf >= 0.f && kf <= 1.f) || !(p >= 0.f && p <= 1.f)) return SLA_ERR_INVALID_ARG;
  if ((sel->Wq == nullptr) != (sel->Wk == nullptr)) return SLA_ERR_INVALID_ARG;
  long long kk = (long long)ceil((double)kf * (double)s.Nk - 1e-9);
  if (kk < 0) kk = 0;
  if (kk > s.Nk) kk = s.Nk;
  *k = (int)kk;
  return SLA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SLA_OK : SLA_ERR_HIP; }

hipError_t run_prep(const Shape& s, bool lin, const void* K, const void* V, const float* alpha,
                    char* ws, const WsLayout& L, hipStream_t st, bool kmeans = false) {
  if (s.dtype == SLA_BF16) return sla::launch_prep_bf16(s, lin, K, V, alpha, kmeans, ws, L, st);
  return lin ? sla::launch_summary_f32(s, K, V, alpha, ws, L, st) : hipSuccess;
}

hipError_t run_attn(const Shape& s, Mode m, const void* Q, const void* K, const void* V,
                    const int32_t* rp, const int32_t* ci, const float* alpha, const char* ws,
                    const WsLayout& L, void* O, hipStream_t st) {
  if (s.dtype == SLA_BF16) return sla::launch_attn_bf16(s, m, Q, K, V, rp, ci, alpha, ws, L, O, st);
  // the linear totals are read only by the modes with a linear branch
  const bool lin = m == sla::MODE_FUSED || m == sla::MODE_LINEAR;
  return sla::launch_attn_f32(s, m, Q, K, V, rp, ci, alpha,
                              lin ? reinterpret_cast<const float*>(ws + L.htot) : nullptr, O, st);
}

}  // namespace

extern "C" {

size_t sla_workspace_bytes(const sla_problem* prob, const sla_select* sel) {
  Shape s;
  if (check_problem(prob, &s) != SLA_OK) return 0;
  const bool router = sel != nullptr && sel->Wq != nullptr;
  return sla::ws_layout(s, router).total;
}

int64_t sla_mask_capacity(const sla_problem* prob) {
  Shape s;
  if (check_problem(prob, &s) != SLA_OK) return -1;
  return (int64_t)s.B * s.H * s.Nq * s.Nk;
}

int sla_mask(const sla_problem* prob, const sla_select* sel, const void* Q, const void* K,
             int32_t* row_ptr, int32_t* col_idx, int64_t capacity, double* block_logits, void* ws,
             size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  int k;
  if ((rc = check_select(sel, &k, s)) != SLA_OK) return rc;
  if (Q == nullptr || K == nullptr || row_ptr == nullptr || col_idx == nullptr) return SLA_ERR_INVALID_ARG;
  if (capacity < (int64_t)s.B * s.H * s.Nq * s.Nk) return SLA_ERR_CAPACITY;
  const WsLayout L = sla::ws_layout(s, sel->Wq != nullptr);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_mask(s, k, (double)sel->p, sel->Wq, sel->Wk, Q, K, row_ptr, col_idx,
                                     block_logits, static_cast<char*>(ws), L,
                                     static_cast<hipStream_t>(stream)));
}

size_t sla_mask_noalloc_bytes(const sla_problem* prob, const sla_select* sel) {
  Shape s;
  if (check_problem(prob, &s) != SLA_OK) return 0;
  const bool router = sel != nullptr && sel->Wq != nullptr;
  return sla::mask_layout(s, router).total;
}

int sla_mask_noalloc(const sla_problem* prob, const sla_select* sel, const void* Q, const void* K,
                     int32_t* row_ptr, int32_t* col_idx, int64_t capacity, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  int k;
  if ((rc = check_select(sel, &k, s)) != SLA_OK) return rc;
  if (Q == nullptr || K == nullptr || row_ptr == nullptr || col_idx == nullptr) return SLA_ERR_INVALID_ARG;
  if (capacity < (int64_t)s.B * s.H * s.Nq * s.Nk) return SLA_ERR_CAPACITY;
  const WsLayout L = sla::mask_layout(s, sel->Wq != nullptr);
  if (L.total > (size_t)SLA_NOALLOC_SCRATCH_BYTES) return SLA_ERR_TOO_LARGE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (st != nullptr) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(st, &sdev) != hipSuccess) return SLA_ERR_HIP;
    if (sdev != cur) return SLA_ERR_INVALID_ARG;
  }
  void* ptr = nullptr;
  if (scratch_of_current_device(&ptr) != hipSuccess) return SLA_ERR_HIP;
  return hip_status(sla::launch_mask(s, k, (double)sel->p, sel->Wq, sel->Wk, Q, K, row_ptr, col_idx, nullptr,
                                     static_cast<char*>(ptr), L, st));
}

int sla_mask_prepared(const sla_problem* prob, const sla_select* sel, const void* Q, const void* K,
                      const float* alpha, int32_t* row_ptr, int32_t* col_idx, int64_t capacity, void* ws,
                      size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  int k;
  if ((rc = check_select(sel, &k, s)) != SLA_OK) return rc;
  if (Q == nullptr || K == nullptr || alpha == nullptr || row_ptr == nullptr || col_idx == nullptr)
    return SLA_ERR_INVALID_ARG;
  if (capacity < (int64_t)s.B * s.H * s.Nq * s.Nk) return SLA_ERR_CAPACITY;
  const WsLayout L = sla::ws_layout(s, sel->Wq != nullptr);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  // the bf16 preparation pass pooled K for the heads it processed
  return hip_status(sla::launch_mask(s, k, (double)sel->p, sel->Wq, sel->Wk, Q, K, row_ptr, col_idx, nullptr,
                                     static_cast<char*>(ws), L, static_cast<hipStream_t>(stream),
                                     s.dtype == SLA_BF16 ? alpha : nullptr));
}

int sla_soft_topk(const sla_problem* prob, const sla_select* sel, float T, const void* Q, const void* K,
                  float* M, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  int k;
  if ((rc = check_select(sel, &k, s)) != SLA_OK) return rc;
  if (!(T > 0.f) || !isfinite(T)) return SLA_ERR_INVALID_ARG;
  if (Q == nullptr || K == nullptr || M == nullptr) return SLA_ERR_INVALID_ARG;
  const WsLayout L = sla::ws_layout(s, sel->Wq != nullptr);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_soft_topk(s, k, (double)T, sel->Wq, sel->Wk, Q, K, M,
                                          static_cast<char*>(ws), L, static_cast<hipStream_t>(stream)));
}

int sla_sparse_fwd(const sla_problem* prob, const void* Q, const void* K, const void* V,
                   const int32_t* row_ptr, const int32_t* col_idx, void* O_s, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (!Q || !K || !V || !row_ptr || !col_idx || !O_s) return SLA_ERR_INVALID_ARG;
  // the softmax kernels read K and V as they are: no workspace region is used
  return hip_status(run_attn(s, sla::MODE_SPARSE, Q, K, V, row_ptr, col_idx, nullptr, nullptr, WsLayout{}, O_s,
                             static_cast<hipStream_t>(stream)));
}

int sla_linear_fwd(const sla_problem* prob, const void* Q, const void* K, const void* V,
                   const int32_t* row_ptr, const int32_t* col_idx, void* O_l, void* ws,
                   size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (!Q || !K || !V || !row_ptr || !col_idx || !O_l) return SLA_ERR_INVALID_ARG;
  const WsLayout L = sla::ws_layout(s, false);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (run_prep(s, true, K, V, nullptr, w, L, st) != hipSuccess) return SLA_ERR_HIP;
  return hip_status(run_attn(s, sla::MODE_LINEAR, Q, K, V, row_ptr, col_idx, nullptr, w, L, O_l, st));
}

int sla_attn_fwd(const sla_problem* prob, const sla_select* sel, const void* Q, const void* K,
                 const void* V, const float* alpha, void* O, int32_t* row_ptr, int32_t* col_idx,
                 int64_t capacity, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  int k;
  if ((rc = check_select(sel, &k, s)) != SLA_OK) return rc;
  if (!Q || !K || !V || !alpha || !O || !row_ptr || !col_idx) return SLA_ERR_INVALID_ARG;
  if (capacity < (int64_t)s.B * s.H * s.Nq * s.Nk) return SLA_ERR_CAPACITY;
  const WsLayout L = sla::ws_layout(s, sel->Wq != nullptr);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  // bf16: the preparation pass runs first and also pools K for the heads it
  // processes (alpha != 1), so the mask reads K only for the others
  const bool bf = s.dtype == SLA_BF16;
  if (bf && run_prep(s, true, K, V, alpha, w, L, st, true) != hipSuccess) return SLA_ERR_HIP;
  if (sla::launch_mask(s, k, (double)sel->p, sel->Wq, sel->Wk, Q, K, row_ptr, col_idx, nullptr, w, L, st,
                       bf ? alpha : nullptr) != hipSuccess)
    return SLA_ERR_HIP;
  if (!bf && run_prep(s, true, K, V, alpha, w, L, st) != hipSuccess) return SLA_ERR_HIP;
  return hip_status(run_attn(s, sla::MODE_FUSED, Q, K, V, row_ptr, col_idx, alpha, w, L, O, st));
}

int sla_kv_prepare(const sla_problem* prob, const void* K, const void* V, const float* alpha,
                   void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (!K || !V) return SLA_ERR_INVALID_ARG;
  const WsLayout L = sla::ws_layout(s, false);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(run_prep(s, true, K, V, alpha, static_cast<char*>(ws), L,
                             static_cast<hipStream_t>(stream), true));
}

int sla_fused_fwd(const sla_problem* prob, const void* Q, const void* K, const void* V,
                  const float* alpha, const int32_t* row_ptr, const int32_t* col_idx, void* O,
                  const void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (!Q || !K || !V || !alpha || !row_ptr || !col_idx || !O) return SLA_ERR_INVALID_ARG;
  const WsLayout L = sla::ws_layout(s, false);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(run_attn(s, sla::MODE_FUSED, Q, K, V, row_ptr, col_idx, alpha,
                             static_cast<const char*>(ws), L, O, static_cast<hipStream_t>(stream)));
}

int64_t sla_saved_terms_count(const sla_problem* prob) {
  Shape s;
  if (check_problem(prob, &s) != SLA_OK) return -1;
  return s.R() * s.bq;
}

int sla_fused_fwd_save(const sla_problem* prob, const void* Q, const void* K, const void* V,
                       const float* alpha, const int32_t* row_ptr, const int32_t* col_idx, void* O,
                       const void* ws, size_t ws_bytes, float* lse2, float* invden, float* O_s, float* O_l,
                       void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.dtype != SLA_BF16) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !alpha || !row_ptr || !col_idx || !O || !lse2 || !invden || !O_s || !O_l)
    return SLA_ERR_INVALID_ARG;
  const WsLayout L = sla::ws_layout(s, false);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  const sla::FwdSaved sv{lse2, invden, O_s, O_l};
  return hip_status(sla::launch_attn_bf16(s, sla::MODE_FUSED, Q, K, V, row_ptr, col_idx, alpha,
                                          static_cast<const char*>(ws), L, O, static_cast<hipStream_t>(stream),
                                          &sv));
}

int sla_dense_fwd(const sla_problem* prob, const void* Q, const void* K, const void* V, void* O,
                  void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (!Q || !K || !V || !O) return SLA_ERR_INVALID_ARG;
  return hip_status(run_attn(s, sla::MODE_DENSE, Q, K, V, nullptr, nullptr, nullptr, nullptr, WsLayout{}, O,
                             static_cast<hipStream_t>(stream)));
}

int sla_i8_layout_of(const sla_problem* prob, sla_i8_layout* layout) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (layout == nullptr) return SLA_ERR_INVALID_ARG;
  if (s.N > 131072) return SLA_ERR_UNSUPPORTED;
  const sla::I8Layout L = sla::i8_layout(s);
  layout->q8 = L.q8; layout->k8 = L.k8; layout->vt8 = L.vt8;
  layout->sq = L.sq; layout->sk = L.sk; layout->sv = L.sv; layout->rv = L.rv;
  layout->vpart = L.vpart; layout->total = L.total;
  return SLA_OK;
}

int sla_quantize_i8(const sla_problem* prob, const void* Q, const void* K, const void* V, void* qbuf,
                    size_t qbuf_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.N > 131072) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V) return SLA_ERR_INVALID_ARG;
  const sla::I8Layout L = sla::i8_layout(s);
  if (qbuf == nullptr || qbuf_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_quant_i8(s, Q, K, V, static_cast<char*>(qbuf), L,
                                         static_cast<hipStream_t>(stream)));
}

int sla_sparse_fwd_i8(const sla_problem* prob, const void* qbuf, size_t qbuf_bytes, const int32_t* row_ptr,
                      const int32_t* col_idx, void* O_s, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.N > 131072) return SLA_ERR_UNSUPPORTED;
  if (!row_ptr || !col_idx || !O_s) return SLA_ERR_INVALID_ARG;
  const sla::I8Layout L = sla::i8_layout(s);
  if (qbuf == nullptr || qbuf_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_attn_i8(s, static_cast<const char*>(qbuf), L, row_ptr, col_idx, O_s,
                                        static_cast<hipStream_t>(stream)));
}

int sla_quantize_i8f8(const sla_problem* prob, const void* Q, const void* K, const void* V, void* qbuf,
                     size_t qbuf_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.N > 131072) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V) return SLA_ERR_INVALID_ARG;
  const sla::I8Layout L = sla::i8_layout(s);
  if (qbuf == nullptr || qbuf_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_quant_i8f8(s, Q, K, V, static_cast<char*>(qbuf), L,
                                         static_cast<hipStream_t>(stream)));
}

int sla_sparse_fwd_i8f8(const sla_problem* prob, const void* qbuf, size_t qbuf_bytes, const int32_t* row_ptr,
                       const int32_t* col_idx, void* O_s, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.N > 131072) return SLA_ERR_UNSUPPORTED;
  if (!row_ptr || !col_idx || !O_s) return SLA_ERR_INVALID_ARG;
  const sla::I8Layout L = sla::i8_layout(s);
  if (qbuf == nullptr || qbuf_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_attn_i8f8(s, static_cast<const char*>(qbuf), L, row_ptr, col_idx, O_s,
                                        static_cast<hipStream_t>(stream)));
}

size_t sla_bwd_workspace_bytes(const sla_problem* prob) {
  Shape s;
  if (check_problem(prob, &s) != SLA_OK) return 0;
  return sla::bwd_layout(s).total;
}

int sla_sparse_bwd(const sla_problem* prob, const void* Q, const void* K, const void* V, const void* dO_s,
                   const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK, void* dV,
                   void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.dtype != SLA_BF16) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !dO_s || !row_ptr || !col_idx || !dQ || !dK || !dV) return SLA_ERR_INVALID_ARG;
  const sla::BwdLayout L = sla::bwd_layout(s);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_sparse_bwd(s, Q, K, V, dO_s, row_ptr, col_idx, dQ, dK, dV, nullptr, true,
                                           static_cast<char*>(ws), L, static_cast<hipStream_t>(stream)));
}

int sla_linear_bwd(const sla_problem* prob, const void* Q, const void* K, const void* V, const void* dO_l,
                   const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK, void* dV, int accumulate,
                   void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.dtype != SLA_BF16) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !dO_l || !row_ptr || !col_idx || !dQ || !dK || !dV) return SLA_ERR_INVALID_ARG;
  const sla::BwdLayout L = sla::bwd_layout(s);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_linear_bwd(s, Q, K, V, dO_l, row_ptr, col_idx, dQ, dK, dV, accumulate != 0,
                                           nullptr, true, static_cast<char*>(ws), L,
                                           static_cast<hipStream_t>(stream)));
}

int sla_attn_bwd(const sla_problem* prob, const void* Q, const void* K, const void* V, const void* dO,
                 const float* alpha, const int32_t* row_ptr, const int32_t* col_idx, void* dQ, void* dK, void* dV,
                 float* dalpha, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.dtype != SLA_BF16) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !dO || !alpha || !row_ptr || !col_idx || !dQ || !dK || !dV) return SLA_ERR_INVALID_ARG;
  const sla::BwdLayout L = sla::bwd_layout(s);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  if (sla::launch_sparse_bwd(s, Q, K, V, dO, row_ptr, col_idx, dQ, dK, dV, alpha, true, w, L, st) != hipSuccess)
    return SLA_ERR_HIP;
  if (sla::launch_linear_bwd(s, Q, K, V, dO, row_ptr, col_idx, dQ, dK, dV, true, alpha, false, w, L, st) !=
      hipSuccess)
    return SLA_ERR_HIP;
  if (dalpha == nullptr) return SLA_OK;
  return hip_status(sla::launch_alpha_grad_terms(s, dalpha, w, L, st));
}

int sla_attn_bwd_saved(const sla_problem* prob, const void* Q, const void* K, const void* V, const void* dO,
                       const float* alpha, const int32_t* row_ptr, const int32_t* col_idx, const float* lse2,
                       const float* invden, const float* O_s, const float* O_l, void* dQ, void* dK, void* dV,
                       float* dalpha, void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (s.dtype != SLA_BF16) return SLA_ERR_UNSUPPORTED;
  if (!Q || !K || !V || !dO || !alpha || !row_ptr || !col_idx || !lse2 || !invden || !O_s || !O_l || !dQ || !dK ||
      !dV)
    return SLA_ERR_INVALID_ARG;
  const sla::BwdLayout L = sla::bwd_layout(s);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const sla::BwdSaved sv{lse2, invden, O_s, O_l};
  if (sla::launch_sparse_bwd(s, Q, K, V, dO, row_ptr, col_idx, dQ, dK, dV, alpha, true, w, L, st, &sv) !=
      hipSuccess)
    return SLA_ERR_HIP;
  if (sla::launch_linear_bwd(s, Q, K, V, dO, row_ptr, col_idx, dQ, dK, dV, true, alpha, false, w, L, st, &sv) !=
      hipSuccess)
    return SLA_ERR_HIP;
  if (dalpha == nullptr) return SLA_OK;
  return hip_status(sla::launch_alpha_grad_terms(s, dalpha, w, L, st));
}

int sla_alpha_grad(const sla_problem* prob, const void* dO, const void* O_s, const void* O_l, float* dalpha,
                   void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  int rc = check_problem(prob, &s);
  if (rc != SLA_OK) return rc;
  if (!dO || !O_s || !O_l || !dalpha) return SLA_ERR_INVALID_ARG;
  const sla::BwdLayout L = sla::bwd_layout(s);
  if (ws == nullptr || ws_bytes < L.total) return SLA_ERR_WORKSPACE;
  return hip_status(sla::launch_alpha_grad(s, dO, O_s, O_l, dalpha, static_cast<char*>(ws), L,
                                           static_cast<hipStream_t>(stream)));
}

const char* sla_status_string(int status) {
  switch (status) {
    case SLA_OK: return "ok";
    case SLA_ERR_INVALID_ARG: return "invalid argument";
    case SLA_ERR_UNSUPPORTED: return "unsupported shape, block size or dtype";
    case SLA_ERR_WORKSPACE: return "workspace missing or too small";
    case SLA_ERR_CAPACITY: return "col_idx capacity below B*H*Nq*Nk";
    case SLA_ERR_HIP: return "HIP launch failure";
    case SLA_ERR_TOO_LARGE: return "problem exceeds the static scratch of the allocation-free mask";
    default: return "unknown status";
  }
}

}  // extern "C"
