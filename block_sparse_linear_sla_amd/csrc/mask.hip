// Block mask: mean pooling, optional router, pooled logits, hybrid Top-k /
// Top-p selection, CSR emission.
//
// Sources: SpargeAttention2 write-up "清華發明AI「注意力瘦身術」：視頻生成速度
// 提升16倍的神奇技術" (arXiv:2602.13515) §四 (a quick pooled overview, then the
// hybrid selection, then an all-or-nothing mask over blocks) and §一 (Top-k
// keeps a fixed count, Top-p keeps items until their mass reaches p, the
// hybrid merges both); SLA2 write-up (arXiv:2602.12675) §二 (router of two
// learnable projections).
//
// Precision: pooled means, router, logits, softmax and the cumulative mass are
// float64.  Sums of bf16 values in float64 are exact, so the pooled means are
// the correctly rounded means; the logits then differ from an exact evaluation
// by a few float64 ulps, far inside any cut-off tolerance a float32 pipeline
// could meet (float32 logits of magnitude ~100 carry ~1e-5 absolute error).
//
// Pipeline (six launches, no host synchronisation):
//   pool      one workgroup per (b, h, block) of Q and of K   - HBM bound
//   router    pooled rows times W                               (optional)
//   score     per (b, h) 64x64-tiled float64 product q_hat k_hat^T / sqrt(d)
//   select    one workgroup per mask row: softmax, bitonic sort, prefix mass,
//             n = max(k, kp), bitmask of the kept blocks
//   scan      one workgroup: exclusive scan of the per-row counts -> row_ptr
//   emit      one wavefront per row: bitmask -> ascending col_idx
#include "sla_internal.h"

namespace sla {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Accumulate the 16-byte chunk v (VEC elements of T) into acc (float64).
template <typename T>
struct Chunk;

template <>
struct Chunk<float> {
  static constexpr int VEC = 4;
  __device__ __forceinline__ static void add(const uint4& v, double* acc) {
    acc[0] += (double)__uint_as_float(v.x);
    acc[1] += (double)__uint_as_float(v.y);
    acc[2] += (double)__uint_as_float(v.z);
    acc[3] += (double)__uint_as_float(v.w);
  }
};

template <>
struct Chunk<uint16_t> {  // bf16 bit patterns
  static constexpr int VEC = 8;
  __device__ __forceinline__ static void add(const uint4& v, double* acc) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += (double)bf16_bits_to_f32(w[i] & 0xffffu);
      acc[2 * i + 1] += (double)bf16_bits_to_f32(w[i] >> 16);
    }
  }
};

// Mean of the valid rows of one block of Q or K.  Workgroups [0, BH*Nq) pool Q
// blocks, the rest pool K blocks.  Each thread owns one 16-byte column chunk
// and walks rows with stride RPP; partial sums meet in LDS.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                        int N, int bq, int bk, int Nq, int Nk,
                                                        long long BH, double* __restrict__ qbar,
                                                        double* __restrict__ kbar) {
  constexpr int VEC = Chunk<T>::VEC;
  constexpr int TPR = D / VEC;         // threads per row
  constexpr int RPP = kThreads / TPR;  // rows per pass
  __shared__ double red[RPP][D];

  long long wg = blockIdx.x;
  const long long nqb = BH * Nq;
  const T* X;
  double* out;
  int bs, blk, nb;
  long long bh;
  if (wg < nqb) {
    bh = wg / Nq; blk = (int)(wg % Nq); X = Q; out = qbar; bs = bq; nb = Nq;
  } else {
    wg -= nqb;
    bh = wg / Nk; blk = (int)(wg % Nk); X = K; out = kbar; bs = bk; nb = Nk;
  }
  const int r0 = blk * bs;
  const int rows = min(bs, N - r0);
  const T* base = X + ((size_t)bh * N + r0) * D;
  const int tid = threadIdx.x;
  const int c = tid % TPR, rr = tid / TPR;

  double acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.0;
#pragma unroll 8
  for (int r = rr; r < rows; r += RPP) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + (size_t)r * D + c * VEC);
    Chunk<T>::add(v, acc);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) red[rr][c * VEC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < RPP; ++k) s += red[k][tid];
    out[((size_t)bh * nb + blk) * D + tid] = s / (double)rows;
  }
}

// y[m, :] = x[m, :] . W   (row vector times the [D, D] router matrix).
template <int D>
__global__ __launch_bounds__(kThreads) void router_kernel(const double* __restrict__ x,
                                                          const float* __restrict__ W,
                                                          double* __restrict__ y, long long M) {
  constexpr int ROWS = 32;
  constexpr int G = kThreads / D;  // row groups
  constexpr int RPT = ROWS / G;    // rows per thread
  __shared__ double xs[ROWS][D];
  const long long row0 = (long long)blockIdx.x * ROWS;
  const int tid = threadIdx.x;
  for (int e = tid; e < ROWS * D; e += kThreads) {
    const int r = e / D, cc = e % D;
    xs[r][cc] = (row0 + r < M) ? x[(size_t)(row0 + r) * D + cc] : 0.0;
  }
  __syncthreads();
  const int n = tid % D, g = tid / D;
  double acc[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) acc[j] = 0.0;
  for (int k = 0; k < D; ++k) {
    const double w = (double)W[k * D + n];
#pragma unroll
    for (int j = 0; j < RPT; ++j) acc[j] = fma(xs[g + G * j][k], w, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const long long r = row0 + g + G * j;
    if (r < M) y[(size_t)r * D + n] = acc[j];
  }
}

// S[bh, i, j] = qh[bh, i, :] . kh[bh, j, :] / sqrt(D); 64x64 tile per
// workgroup, 4x4 outputs per thread, float64 FMA.
template <int D>
__global__ __launch_bounds__(kThreads) void score_kernel(const double* __restrict__ qh,
                                                         const double* __restrict__ kh,
                                                         double* __restrict__ S, int Nq, int Nk) {
  constexpr int T = 64, KC = 16;
  __shared__ double As[KC][T + 1];
  __shared__ double Bs[KC][T + 1];
  const long long bh = blockIdx.z;
  const int i0 = blockIdx.y * T, j0 = blockIdx.x * T;
  const double* qb = qh + (size_t)bh * Nq * D;
  const double* kb = kh + (size_t)bh * Nk * D;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int kc = 0; kc < D; kc += KC) {
#pragma unroll
    for (int u = 0; u < (T * KC) / kThreads; ++u) {
      const int e = tid + kThreads * u;
      const int r = e / KC, kk = e % KC;
      As[kk][r] = (i0 + r < Nq) ? qb[(size_t)(i0 + r) * D + kc + kk] : 0.0;
      Bs[kk][r] = (j0 + r < Nk) ? kb[(size_t)(j0 + r) * D + kc + kk] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[kk][ty + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Bs[kk][tx + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
  const double sd = sqrt((double)D);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = i0 + ty + 16 * a;
    if (i >= Nq) continue;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j = j0 + tx + 16 * b;
      if (j < Nk) S[((size_t)bh * Nq + i) * Nk + j] = acc[a][b] / sd;
    }
  }
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// One workgroup per mask row.  NP = padded power of two >= Nk.
template <int NP>
__global__ __launch_bounds__(kThreads) void select_kernel(const double* __restrict__ S, int Nk, int k,
                                                          double p, int* __restrict__ counts,
                                                          uint32_t* __restrict__ bits, int W) {
  constexpr int NW = kThreads / 64;
  __shared__ double pv[NP];
  __shared__ int iv[NP];
  __shared__ double red_d[NW];
  __shared__ int red_i[NW];
  __shared__ double tot[kThreads];
  __shared__ uint32_t words[NP / 32];
  const long long row = blockIdx.x;
  const double* srow = S + (size_t)row * Nk;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // 1. logits, row max
  double lmax = -INFINITY;
  for (int j = tid; j < NP; j += kThreads) {
    const double s = (j < Nk) ? srow[j] : -INFINITY;
    pv[j] = s;
    iv[j] = j;
    lmax = fmax(lmax, s);
  }
  for (int w = tid; w < NP / 32; w += kThreads) words[w] = 0u;
  lmax = wave_max(lmax);
  if (lane == 0) red_d[wv] = lmax;
  __syncthreads();
  double m = red_d[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) m = fmax(m, red_d[w]);
  __syncthreads();
  // 2. softmax normaliser
  double lsum = 0.0;
  for (int j = tid; j < Nk; j += kThreads) lsum += exp(pv[j] - m);
  lsum = wave_sum(lsum);
  if (lane == 0) red_d[wv] = lsum;
  __syncthreads();
  double Z = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) Z += red_d[w];
  for (int j = tid; j < NP; j += kThreads) pv[j] = (j < Nk) ? exp(pv[j] - m) / Z : -1.0;
  __syncthreads();

  // 3. bitonic sort: probability descending, ties to the lower block index
  for (int size = 2; size <= NP; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < NP / 2; t += kThreads) {
        const int i = 2 * stride * (t / stride) + (t % stride);
        const int j = i + stride;
        const double pi = pv[i], pj = pv[j];
        const int ii = iv[i], ij = iv[j];
        const bool j_first = (pj > pi) || (pj == pi && ij < ii);
        const bool i_first = (pi > pj) || (pi == pj && ii < ij);
        const bool swap = ((i & size) == 0) ? j_first : i_first;
        if (swap) {
          pv[i] = pj; pv[j] = pi;
          iv[i] = ij; iv[j] = ii;
        }
      }
      __syncthreads();
    }
  }

  // 4. cumulative mass in sorted order; kp = first n with mass(n) >= p
  constexpr int E = (NP + kThreads - 1) / kThreads;
  const int e0 = tid * E;
  double local = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int n = e0 + e;
    if (n < Nk) local += pv[n];
  }
  tot[tid] = local;
  __syncthreads();
  // exclusive prefix over thread totals (Hillis-Steele in LDS)
  for (int off = 1; off < kThreads; off <<= 1) {
    const double add = (tid >= off) ? tot[tid - off] : 0.0;
    __syncthreads();
    tot[tid] += add;
    __syncthreads();
  }
  double run = (tid > 0) ? tot[tid - 1] : 0.0;
  int first = 0x7fffffff;
  if (p > 0.0) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int n = e0 + e;
      if (n < Nk) {
        run += pv[n];
        if (run >= p && first == 0x7fffffff) first = n + 1;
      }
    }
  }
  first = wave_min_int(first);
  if (lane == 0) red_i[wv] = first;
  __syncthreads();
  int kp = red_i[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) kp = min(kp, red_i[w]);
  if (p <= 0.0) kp = 0;
  else if (kp == 0x7fffffff) kp = Nk;
  const int nsel = max(min(k, Nk), kp);

  // 5. bitmask of the kept blocks
  for (int n = tid; n < nsel; n += kThreads) {
    const int j = iv[n];
    atomicOr(&words[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  for (int w = tid; w < W; w += kThreads) bits[(size_t)row * W + w] = words[w];
  if (tid == 0) counts[row] = nsel;
}

// Exclusive scan of counts[R] into row_ptr[R + 1] with one workgroup.
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ counts, long long R,
                                                    int* __restrict__ row_ptr) {
  __shared__ long long part[1024];
  const int tid = threadIdx.x;
  const long long per = (R + 1023) / 1024;
  const long long b = tid * per, e = min(R, b + per);
  long long s = 0;
  for (long long r = b; r < e; ++r) s += counts[r];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const long long add = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  long long run = (tid > 0) ? part[tid - 1] : 0;
  for (long long r = b; r < e; ++r) {
    row_ptr[r] = (int)run;
    run += counts[r];
  }
  if (tid == 1023) row_ptr[R] = (int)part[1023];
}

// One wavefront per row: bitmask words -> ascending block indices.
__global__ __launch_bounds__(kThreads) void emit_kernel(const uint32_t* __restrict__ bits,
                                                        const int* __restrict__ row_ptr,
                                                        int* __restrict__ col_idx, long long R, int W) {
  const long long row = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= R) return;
  const int lane = threadIdx.x & 63;
  const int WPL = (W + 63) / 64;  // words per lane (<= 2 for Nk <= 4096)
  uint32_t w[2] = {0u, 0u};
  int cnt = 0;
  for (int u = 0; u < WPL; ++u) {
    const int wi = lane * WPL + u;
    w[u] = (wi < W) ? bits[(size_t)row * W + wi] : 0u;
    cnt += __popc(w[u]);
  }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  int pos = row_ptr[row] + incl - cnt;
  for (int u = 0; u < WPL; ++u) {
    uint32_t x = w[u];
    const int base = (lane * WPL + u) * 32;
    while (x) {
      const int bpos = __ffs(x) - 1;
      col_idx[pos++] = base + bpos;
      x &= x - 1u;
    }
  }
}

template <int NP>
hipError_t launch_select(const double* S, long long R, int Nk, int k, double p, int* counts,
                         uint32_t* bits, int W, hipStream_t st) {
  hipLaunchKernelGGL((select_kernel<NP>), dim3((unsigned)R), dim3(kThreads), 0, st, S, Nk, k, p,
                     counts, bits, W);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mask(const Shape& s, int k, double p, const float* Wq, const float* Wk,
                       const void* Q, const void* K, int32_t* row_ptr, int32_t* col_idx,
                       double* logits_out, char* ws, const WsLayout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H;
  const long long R = s.R();
  double* qbar = reinterpret_cast<double*>(ws + L.qbar);
  double* kbar = reinterpret_cast<double*>(ws + L.kbar);
  double* S = logits_out ? logits_out : reinterpret_cast<double*>(ws + L.S);
  int* counts = reinterpret_cast<int*>(ws + L.counts);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + L.bits);
  const int W = s.words();

  const dim3 gpool((unsigned)(BH * (s.Nq + s.Nk)));
#define SLA_POOL(T, DD)                                                                          \
  hipLaunchKernelGGL((pool_kernel<T, DD>), gpool, dim3(kThreads), 0, st,                          \
                     reinterpret_cast<const T*>(Q), reinterpret_cast<const T*>(K), s.N, s.bq,   \
                     s.bk, s.Nq, s.Nk, BH, qbar, kbar)
  if (s.dtype == 1) {
    if (s.d == 128) SLA_POOL(uint16_t, 128); else SLA_POOL(uint16_t, 64);
  } else {
    if (s.d == 128) SLA_POOL(float, 128); else SLA_POOL(float, 64);
  }
#undef SLA_POOL
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const double* qh = qbar;
  const double* kh = kbar;
  if (Wq != nullptr) {
    double* qhat = reinterpret_cast<double*>(ws + L.qhat);
    double* khat = reinterpret_cast<double*>(ws + L.khat);
    const long long Mq = BH * s.Nq, Mk = BH * s.Nk;
    if (s.d == 128) {
      hipLaunchKernelGGL((router_kernel<128>), dim3((unsigned)((Mq + 31) / 32)), dim3(kThreads), 0,
                         st, qbar, Wq, qhat, Mq);
      hipLaunchKernelGGL((router_kernel<128>), dim3((unsigned)((Mk + 31) / 32)), dim3(kThreads), 0,
                         st, kbar, Wk, khat, Mk);
    } else {
      hipLaunchKernelGGL((router_kernel<64>), dim3((unsigned)((Mq + 31) / 32)), dim3(kThreads), 0,
                         st, qbar, Wq, qhat, Mq);
      hipLaunchKernelGGL((router_kernel<64>), dim3((unsigned)((Mk + 31) / 32)), dim3(kThreads), 0,
                         st, kbar, Wk, khat, Mk);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    qh = qhat;
    kh = khat;
  }

  const dim3 gscore((unsigned)((s.Nk + 63) / 64), (unsigned)((s.Nq + 63) / 64), (unsigned)BH);
  if (s.d == 128)
    hipLaunchKernelGGL((score_kernel<128>), gscore, dim3(kThreads), 0, st, qh, kh, S, s.Nq, s.Nk);
  else
    hipLaunchKernelGGL((score_kernel<64>), gscore, dim3(kThreads), 0, st, qh, kh, S, s.Nq, s.Nk);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  int np = 64;
  while (np < s.Nk) np <<= 1;
  switch (np) {
    case 64: e = launch_select<64>(S, R, s.Nk, k, p, counts, bits, W, st); break;
    case 128: e = launch_select<128>(S, R, s.Nk, k, p, counts, bits, W, st); break;
    case 256: e = launch_select<256>(S, R, s.Nk, k, p, counts, bits, W, st); break;
    case 512: e = launch_select<512>(S, R, s.Nk, k, p, counts, bits, W, st); break;
    case 1024: e = launch_select<1024>(S, R, s.Nk, k, p, counts, bits, W, st); break;
    case 2048: e = launch_select<2048>(S, R, s.Nk, k, p, counts, bits, W, st); break;
    default: e = launch_select<4096>(S, R, s.Nk, k, p, counts, bits, W, st); break;
  }
  if (e != hipSuccess) return e;

  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, R, row_ptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(emit_kernel, dim3((unsigned)((R + 3) / 4)), dim3(kThreads), 0, st, bits,
                     row_ptr, col_idx, R, W);
  return hipGetLastError();
}

}  // namespace sla
