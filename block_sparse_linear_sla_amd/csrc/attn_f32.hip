// fp32 attention over the block mask (plain FMA; one wavefront per query row).
//
// Sources as for the bf16 path: SLA2 write-up (arXiv:2602.12675) §一, §二 and
// the SpargeAttention2 write-up "清華發明AI「注意力瘦身術」：視頻生成速度提升
// 16倍的神奇技術" §四; phi(x) = elu(x) + 1 (Katharopoulos et al. 2020).
//
// The fp32 path serves small problems where float32 accuracy is the point,
// so it favours a direct formulation over speed:
//   sparse  online softmax over the keys of the listed blocks, 64 keys at a
//           time across the lanes; q.k is accumulated in float64 (the
//           products of two floats are exact there), because logits of
//           magnitude ~100 carry ~1e-5 absolute error in float32, which the
//           softmax passes straight into the output;
//   linear  with per-head totals H = sum_u phi(k_u)^T v_u and z = sum_u phi(k_u),
//           num = phi(q) H - sum_{listed keys} (phi(q).phi(k)) v and
//           den = phi(q) z - sum_{listed keys} phi(q).phi(k), i.e. the total
//           minus the listed blocks, applied after phi(q).
#include "sla_internal.h"

namespace sla {

hipError_t launch_summary_reduce(const float* hpart, const float* alpha, int H, long long BH,
                                 int nchunk, int per, float* htot, hipStream_t st);

namespace {

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : expf(x); }

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wmax(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

template <int D, int MODE>
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, const float* __restrict__ alpha,
    const float* __restrict__ htot, float* __restrict__ O, long long total_rows, int H, int N, int bq,
    int bk, int Nq, int Nk, double scale) {
  constexpr int C = D / 64;  // output columns per lane
  const int lane = threadIdx.x & 63;
  const long long t_glob = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);  // (bh, token)
  if (t_glob >= total_rows) return;  // whole wavefront; the kernel has no barrier
  const long long bh = t_glob / N;
  const int t = (int)(t_glob % N);
  const int h = (int)(bh % H);
  const int qi = t / bq;
  const long long row = bh * Nq + qi;

  int nsel, base = 0;
  if (MODE == MODE_DENSE) {
    nsel = Nk;
  } else {
    base = row_ptr[row];
    nsel = row_ptr[row + 1] - base;
  }
  float ws_ = 0.f, wl_ = 0.f;
  if (MODE == MODE_FUSED) {
    ws_ = alpha[h];
    wl_ = 1.f - ws_;
  } else if (MODE == MODE_LINEAR) {
    wl_ = 1.f;
  } else {
    ws_ = 1.f;
  }
  const bool do_s = ws_ != 0.f;
  const bool lin = (wl_ != 0.f) && (nsel < Nk);

  const float* Kb = K + (size_t)bh * N * D;
  const float* Vb = V + (size_t)bh * N * D;
  const float* qrow = Q + ((size_t)bh * N + t) * D;

  // query (and phi(query)) in every lane: cheap, D floats from L1/L2
  float acc[C], accl[C];
#pragma unroll
  for (int c = 0; c < C; ++c) { acc[c] = 0.f; accl[c] = 0.f; }
  double m_run = -INFINITY;
  float l_run = 0.f, lsel = 0.f;

  for (int b = 0; b < ((do_s || lin) ? nsel : 0); ++b) {
    const int j = (MODE == MODE_DENSE) ? b : col_idx[base + b];
    const int k0 = j * bk, k1 = min(N, k0 + bk);
    for (int kb = k0; kb < k1; kb += 64) {
      const int key = kb + lane;
      const bool ok = key < k1;
      double s = -INFINITY;
      float a = 0.f;
      if (ok) {
        const float* kr = Kb + (size_t)key * D;
        double dot = 0.0;
        float dl = 0.f;
        for (int e = 0; e < D; ++e) {
          const float kv = kr[e], qv = qrow[e];
          dot = fma((double)qv, (double)kv, dot);
          if (lin) dl = fmaf(phi(qv), phi(kv), dl);
        }
        s = dot * scale;
        a = dl;
      }
      float p = 0.f;
      if (do_s) {
        const double mx = wmax(s);
        const double m_new = fmax(m_run, mx);
        const float corr = expf((float)(m_run - m_new));
        p = ok ? expf((float)(s - m_new)) : 0.f;
        l_run = l_run * corr + wsum(p);
#pragma unroll
        for (int c = 0; c < C; ++c) acc[c] *= corr;
        m_run = m_new;
      }
      if (lin) lsel += wsum(a);
      const int nk = min(64, k1 - kb);
      for (int u = 0; u < nk; ++u) {
        const float pu = __shfl(p, u);
        const float au = __shfl(a, u);
        const float* vr = Vb + (size_t)(kb + u) * D;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float vv = vr[lane + 64 * c];
          if (do_s) acc[c] = fmaf(pu, vv, acc[c]);
          if (lin) accl[c] = fmaf(au, vv, accl[c]);
        }
      }
    }
  }

  float os[C], ol[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    os[c] = (do_s && l_run > 0.f) ? acc[c] / l_run : 0.f;
    ol[c] = 0.f;
  }
  if (lin) {
    const float* Hh = htot + (size_t)bh * (D * D + D);
    float num[C], den = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) num[c] = 0.f;
    for (int e = 0; e < D; ++e) {
      const float f = phi(qrow[e]);
      den = fmaf(f, Hh[D * D + e], den);
#pragma unroll
      for (int c = 0; c < C; ++c) num[c] = fmaf(f, Hh[e * D + lane + 64 * c], num[c]);
    }
    den -= lsel;
#pragma unroll
    for (int c = 0; c < C; ++c) ol[c] = (num[c] - accl[c]) / den;
  }
  float* orow = O + ((size_t)bh * N + t) * D;
#pragma unroll
  for (int c = 0; c < C; ++c) orow[lane + 64 * c] = ws_ * os[c] + wl_ * ol[c];
}

// Partial linear summaries over one chunk of key blocks of one head:
// thread (a, b-range) accumulates sum_u phi(k_u[a]) v_u[b] in fp32.
template <int D>
__global__ __launch_bounds__(256) void summary_f32_kernel(const float* __restrict__ K,
                                                          const float* __restrict__ V,
                                                          const float* __restrict__ alpha, int H,
                                                          int N, int bk, int chunk_blocks, int nchunk,
                                                          float* __restrict__ hpart) {
  constexpr int PER = D * D / 256;  // entries per thread
  constexpr int KC = 32;            // keys per LDS stage
  __shared__ float pk[KC][D];
  __shared__ float vs[KC][D];
  const long long bh = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  if (alpha != nullptr && alpha[bh % H] == 1.f) return;
  const int tid = threadIdx.x;
  const int a = tid % D;            // phi(k) column
  const int b0 = (tid / D) * PER;   // v columns b0 .. b0+PER-1
  const float* Kb = K + (size_t)bh * N * D;
  const float* Vb = V + (size_t)bh * N * D;
  const int u0 = chunk * chunk_blocks * bk, u1 = min(N, u0 + chunk_blocks * bk);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float z = 0.f;
  for (int u = u0; u < u1; u += KC) {
    __syncthreads();
    for (int e = tid; e < KC * D; e += 256) {
      const int r = e / D, c = e % D;
      const bool ok = u + r < u1;
      pk[r][c] = ok ? phi(Kb[(size_t)(u + r) * D + c]) : 0.f;
      vs[r][c] = ok ? Vb[(size_t)(u + r) * D + c] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < KC; ++r) {
      const float f = pk[r][a];
      if (b0 == 0) z += f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(f, vs[r][b0 + e], acc[e]);
    }
  }
  float* out = hpart + ((size_t)bh * nchunk + chunk) * (D * D + D);
#pragma unroll
  for (int e = 0; e < PER; ++e) out[a * D + b0 + e] = acc[e];
  if (b0 == 0) out[D * D + a] = z;
}

template <int D>
hipError_t attn_f32_dispatch(const Shape& s, Mode mode, const float* q, const float* k, const float* v,
                             const int32_t* rp, const int32_t* ci, const float* alpha,
                             const float* htot, float* o, hipStream_t st) {
  const long long rows = (long long)s.B * s.H * s.N;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const double scale = 1.0 / sqrt((double)D);
#define SLA_F32(M)                                                                                   \
  hipLaunchKernelGGL((attn_f32_kernel<D, M>), grid, block, 0, st, q, k, v, rp, ci, alpha, htot, o, \
                     rows, s.H, s.N, s.bq, s.bk, s.Nq, s.Nk, scale)
  switch (mode) {
    case MODE_SPARSE: SLA_F32(MODE_SPARSE); break;
    case MODE_LINEAR: SLA_F32(MODE_LINEAR); break;
    case MODE_FUSED: SLA_F32(MODE_FUSED); break;
    default: SLA_F32(MODE_DENSE); break;
  }
#undef SLA_F32
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                           const int32_t* rp, const int32_t* ci, const float* alpha, const float* htot,
                           void* O, hipStream_t st) {
  const float* q = static_cast<const float*>(Q);
  const float* k = static_cast<const float*>(K);
  const float* v = static_cast<const float*>(V);
  float* o = static_cast<float*>(O);
  if (s.d == 128) return attn_f32_dispatch<128>(s, mode, q, k, v, rp, ci, alpha, htot, o, st);
  if (s.d == 64) return attn_f32_dispatch<64>(s, mode, q, k, v, rp, ci, alpha, htot, o, st);
  return hipErrorInvalidValue;
}

hipError_t launch_summary_f32(const Shape& s, const void* K, const void* V, const float* alpha,
                              char* ws, const WsLayout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H;
  float* hpart = reinterpret_cast<float*>(ws + L.hpart);
  float* htot = reinterpret_cast<float*>(ws + L.htot);
  const dim3 grid((unsigned)(BH * L.nchunk)), block(256);
  if (s.d == 128)
    hipLaunchKernelGGL((summary_f32_kernel<128>), grid, block, 0, st, static_cast<const float*>(K),
                       static_cast<const float*>(V), alpha, s.H, s.N, s.bk, L.chunk_blocks, L.nchunk,
                       hpart);
  else
    hipLaunchKernelGGL((summary_f32_kernel<64>), grid, block, 0, st, static_cast<const float*>(K),
                       static_cast<const float*>(V), alpha, s.H, s.N, s.bk, L.chunk_blocks, L.nchunk,
                       hpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_summary_reduce(hpart, alpha, s.H, BH, L.nchunk, s.d * s.d + s.d, htot, st);
}

}  // namespace sla
