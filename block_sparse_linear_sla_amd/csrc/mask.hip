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
// Pipeline (four launches, six with the router; no host synchronisation):
//   pool      one workgroup per (b, h, block) of Q and of K   - HBM bound
//   router    W_q W_k^T, then the pooled Q rows times it           (optional;
//             (q W_q).(k W_k) taken as (q W_q W_k^T).k)
//   score     per (b, h) 32x32-tiled float64 MFMA product q_hat k_bar^T / sqrt(d)
//             (q_hat = q_bar, or q_bar W_q W_k^T with the router)
//   select    one wavefront per mask row: softmax, the Top-k and Top-p cut
//             points by bisection over the order-preserving keys,
//             n = max(k, kp), bitmask of the kept blocks
//   scan+emit one thread per row, 256 rows per workgroup: the counts of all
//             earlier rows summed, row_ptr, bitmask -> ascending col_idx
#include <cfloat>

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
// blocks, the rest pool K blocks (except those of the heads whose kdone value
// is not exactly 1: the preparation pass has written their means).  Each thread owns one 16-byte column chunk
// and walks rows with stride RPP; partial sums meet in LDS.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                        int N, int bq, int bk, int Nq, int Nk,
                                                        long long BH, int H, const float* __restrict__ kdone,
                                                        double* __restrict__ qbar,
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
    if (kdone != nullptr && kdone[bh % H] != 1.f) return;  // pooled by the preparation pass
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

// W_qk = W_q W_k^T in float64 (row a: one workgroup; column b: one thread).
// The products of two float32 values are exact in float64.
template <int D>
__global__ __launch_bounds__(D) void router_pair_kernel(const float* __restrict__ Wq, const float* __restrict__ Wk,
                                                        double* __restrict__ Wqk) {
  const int a = blockIdx.x, b = threadIdx.x;
  double acc = 0.0;
  for (int c = 0; c < D; ++c) acc = fma((double)Wq[a * D + c], (double)Wk[b * D + c], acc);
  Wqk[a * D + b] = acc;
}

// y[m, :] = x[m, :] . W   (row vector times a [D, D] matrix).
template <int D, typename TW>
__global__ __launch_bounds__(kThreads) void router_kernel(const double* __restrict__ x,
                                                          const TW* __restrict__ W,
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

// S[bh, i, j] = qh[bh, i, :] . kh[bh, j, :] / sqrt(D) on the float64 matrix
// cores (v_mfma_f64_16x16x4f64: lane l supplies A row l%16 / B column l%16 and
// one k per step; accumulator element i of lane l is row 4*i + l/16, column
// l%16).  One workgroup per 32 x 32 tile of S (2 x 2 MFMA blocks); its four
// wavefronts split the contraction into quarters of D/4, each loading its
// operands for the whole quarter at once straight into registers (lane (r,
// g) = (l%16, l/16) reads D/16 consecutive k of row r and supplies them at
// successive steps; the order of the contraction is permuted the same way for
// both operands).  The four partial tiles are summed in a fixed order through
// LDS.  Workgroups are mapped so that each XCD walks a contiguous range of
// heads, whose pooled vectors then stay in its L2.
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(kThreads) void score_kernel(const double* __restrict__ qh,
                                                         const double* __restrict__ kh,
                                                         double* __restrict__ S, int Nq, int Nk,
                                                         int tiles_j, int tiles) {
  static_assert(kThreads == 256, "four wavefronts per tile");
  constexpr int KL = D / 16;  // k per lane (and MFMA steps per wavefront)
  __shared__ f64x4 part[4][4][64];  // [wavefront][MFMA block][lane]
  const int lane = threadIdx.x & 63, kq = threadIdx.x >> 6;
  // XCD-contiguous order of the workgroups (dispatch is round-robin over 8 XCDs)
  const long long nb = gridDim.x, b = blockIdx.x;
  const long long q8 = nb / 8, r8 = nb % 8, x = b % 8, loc = b / 8;
  const long long wg = x < r8 ? x * (q8 + 1) + loc : r8 * (q8 + 1) + (x - r8) * q8 + loc;
  const long long bh = wg / tiles;
  const int t = (int)(wg % tiles);
  const int i0 = (t / tiles_j) * 32, j0 = (t % tiles_j) * 32;
  const int r = lane & 15, g = lane >> 4;
  const int k0 = kq * (D / 4) + g * KL;
  double a[2][KL], bv[2][KL];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const bool ia = i0 + 16 * h + r < Nq, jb = j0 + 16 * h + r < Nk;
    const double2* qa = reinterpret_cast<const double2*>(qh + ((size_t)bh * Nq + (ia ? i0 + 16 * h + r : 0)) * D + k0);
    const double2* kb = reinterpret_cast<const double2*>(kh + ((size_t)bh * Nk + (jb ? j0 + 16 * h + r : 0)) * D + k0);
#pragma unroll
    for (int s = 0; s < KL / 2; ++s) {
      const double2 x2 = qa[s], y2 = kb[s];
      a[h][2 * s] = ia ? x2.x : 0.0;
      a[h][2 * s + 1] = ia ? x2.y : 0.0;
      bv[h][2 * s] = jb ? y2.x : 0.0;
      bv[h][2 * s + 1] = jb ? y2.y : 0.0;
    }
  }
  f64x4 acc[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[h][c] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < KL; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[h][c] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[h][s], bv[c][s], acc[h][c], 0, 0, 0);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) part[kq][2 * h + c][lane] = acc[h][c];
  __syncthreads();
  // wavefront kq finishes MFMA block kq: the quarters summed in order 0..3
  const f64x4 sum = ((part[0][kq][lane] + part[1][kq][lane]) + part[2][kq][lane]) + part[3][kq][lane];
  const double sd = sqrt((double)D);
  const int h = kq >> 1, c = kq & 1;
  const int j = j0 + 16 * c + r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = i0 + 16 * h + 4 * e + g;
    if (row < Nq && j < Nk) S[((size_t)bh * Nq + row) * Nk + j] = sum[e] / sd;
  }
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
// ---------------------------------------------------------------- selection
// One wavefront per mask row (four rows per workgroup, no barriers).  Lane l
// holds the row's blocks j = l + 64 e, e < E.  The order is taken on the
// float64 logits S (P = exp(S - max) / sum is non-decreasing in S; equal
// logits are ties), with an order-preserving 64-bit key per logit.
//
// The order is P descending with ties to the lower block index; Top-k keeps
// the first k, Top-p the first kp where kp is the smallest count whose
// cumulative mass reaches p, the union keeps the first max(k, kp) [SA2 §一].
// Both cut points are found without sorting, by bisection on the logit
// value: the Top-k cut is the largest t with count(S >= t) >= k, the Top-p
// cut the largest t with mass(S >= t) >= p.  A count is a sum of ballot
// popcounts (scalar), a mass a wavefront sum; each step halves the interval,
// which stops once a single element is left in it.  When the first k blocks
// already hold mass p, the union is the Top-k set and the Top-p cut is not
// searched (nor, when a float32 estimate settles that, the float64
// probabilities formed).  Mass is accumulated in 2^-62 fixed
// point, so the sums are exact and independent of the order the lanes add
// them in (the result is bit-for-bit repeatable); it differs from a
// sequential float64 cumulative sum by at most Nk * 2^-62.  Equal keys at
// the cut are taken in ascending block order, ranked with ballots.

constexpr double kMassScale = 4611686018427387904.0;  // 2^62

__device__ __forceinline__ unsigned long long mass_of(unsigned long long key) {
  const double pr = __longlong_as_double((long long)key);
  return (unsigned long long)(pr * kMassScale + 0.5);
}

// Wavefront sums and maxima of 64-bit values through the same DPP butterflies
// (quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror) and the
// 16- and 32-lane permlane swaps: every step combines a lane's value with its
// partner's, and the partner combines the same two numbers, so all 64 lanes
// end with bit-identical results (callers branch on them) at a few cycles per
// step.
__device__ __forceinline__ double f64_of(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ unsigned long long u64_of(uint32_t lo, uint32_t hi) {
  return ((unsigned long long)hi << 32) | lo;
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long u) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return u64_of(lo, hi);
}
// Op(a, b) over the wavefront for a commutative Op on 64-bit patterns.
template <class Op>
__device__ __forceinline__ unsigned long long wave_fold_u64(unsigned long long u, Op op) {
  u = op(u, dpp_u64<0xB1>(u));
  u = op(u, dpp_u64<0x4E>(u));
  u = op(u, dpp_u64<0x141>(u));
  u = op(u, dpp_u64<0x140>(u));
  {
    const auto a = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    u = op(u64_of(a[0], b[0]), u64_of(a[1], b[1]));
  }
  {
    const auto a = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    u = op(u64_of(a[0], b[0]), u64_of(a[1], b[1]));
  }
  return u;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  return __longlong_as_double((long long)wave_fold_u64(
      (unsigned long long)__double_as_longlong(v), [](unsigned long long a, unsigned long long b) {
        return (unsigned long long)__double_as_longlong(__longlong_as_double((long long)a) +
                                                       __longlong_as_double((long long)b));
      }));
}
__device__ __forceinline__ double wave_max_f64(double v) {
  return __longlong_as_double((long long)wave_fold_u64(
      (unsigned long long)__double_as_longlong(v), [](unsigned long long a, unsigned long long b) {
        return (unsigned long long)__double_as_longlong(
            fmax(__longlong_as_double((long long)a), __longlong_as_double((long long)b)));
      }));
}
// exact (the callers' totals stay below 2^64)
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  return wave_fold_u64(v, [](unsigned long long a, unsigned long long b) { return a + b; });
}

// Mask bits of one row: every valid block when all, else those whose key is
// above the cut key, and of the blocks whose key equals it the first
// ties_needed in block order (ranked with ballots).
template <int E>
__device__ __forceinline__ void emit_row_bits(const unsigned long long (&key)[E], unsigned long long valid_bits,
                                              bool all, int nsel, unsigned long long ckey, int ties_needed,
                                              int lane, uint32_t* __restrict__ brow, int W) {
  int ties_before = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool valid = (valid_bits >> e) & 1ull;
    const bool gt = valid && nsel > 0 && key[e] > ckey;
    const bool eq = valid && nsel > 0 && key[e] == ckey;
    const unsigned long long eqm = __ballot(eq);
    const int rank = ties_before + __popcll(eqm & ((1ull << lane) - 1ull));
    const bool sel = all ? valid : (gt || (eq && rank < ties_needed));
    ties_before += __popcll(eqm);
    const unsigned long long sm = __ballot(sel);
    if (lane == 0) {
      if (2 * e < W) brow[2 * e] = (uint32_t)(sm & 0xffffffffull);
      if (2 * e + 1 < W) brow[2 * e + 1] = (uint32_t)(sm >> 32);
    }
  }
}

// Float32 wavefront sums through the butterflies of wave_fold_u64 (bit-identical
// in every lane: the iteration below branches on them); float64 sums use
// wave_sum_f64.
template <int CTRL>
__device__ __forceinline__ float add_f32_dpp(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = add_f32_dpp<0xB1>(v);
  v = add_f32_dpp<0x4E>(v);
  v = add_f32_dpp<0x141>(v);
  v = add_f32_dpp<0x140>(v);
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Number of valid keys >= t (wave-uniform: popcounts of ballots).
template <int E>
__device__ __forceinline__ int count_ge(const unsigned long long (&key)[E], unsigned long long valid_bits,
                                        unsigned long long t) {
  int c = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) c += __popcll(__ballot(((valid_bits >> e) & 1ull) && key[e] >= t));
  return c;
}

// Fixed-point mass of the keys >= t (wave-uniform; padding has mass 0).
template <int E>
__device__ __forceinline__ unsigned long long mass_ge(const unsigned long long (&key)[E],
                                                      const unsigned long long (&mass)[E], unsigned long long t) {
  unsigned long long m = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) m += key[e] >= t ? mass[e] : 0ull;
  return wave_sum_u64(m);
}

// Number of valid logits >= t (wave-uniform); padding holds -inf.
template <int E>
__device__ __forceinline__ int count_s_ge(const double (&sv)[E], double t) {
  int c = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) c += __popcll(__ballot(sv[e] >= t));
  return c;
}

// Fixed-point mass of the blocks whose logit is >= t (wave-uniform).
template <int E>
__device__ __forceinline__ unsigned long long mass_s_ge(const double (&sv)[E], const unsigned long long (&mass)[E],
                                                        double t) {
  unsigned long long m = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) m += sv[e] >= t ? mass[e] : 0ull;
  return wave_sum_u64(m);
}

// Smallest valid key >= t (wave-uniform; the caller knows one exists).
template <int E>
__device__ __forceinline__ unsigned long long min_key_ge(const unsigned long long (&key)[E],
                                                         unsigned long long valid_bits, unsigned long long t) {
  unsigned long long m = ~0ull;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (((valid_bits >> e) & 1ull) && key[e] >= t && key[e] < m) m = key[e];
  return wave_fold_u64(m, [](unsigned long long a, unsigned long long b) { return a < b ? a : b; });
}

// Order-preserving 64-bit key of a logit (larger logit, larger key).
__device__ __forceinline__ unsigned long long skey(double x) {
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}
__device__ __forceinline__ double skey_value(unsigned long long k) {
  return __longlong_as_double((long long)((k >> 63) ? (k & 0x7fffffffffffffffull) : ~k));
}

// The selection of one mask row by one wavefront: srow points at the row's
// Nk logits (global memory or LDS); writes the row's W bitmask words and
// its count.
template <int E>
__device__ __forceinline__ void select_row(const double* srow, int Nk, int k, double p, int lane,
                                           uint32_t* __restrict__ brow, int W, int* __restrict__ count) {
  double sl[E];  // logits (padding -inf)
  unsigned long long key[E];
  unsigned long long valid_bits = 0;
  double mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    const bool ok = j < Nk;
    const double s = srow[ok ? j : 0];
    sl[e] = ok ? s : -INFINITY;
    key[e] = ok ? skey(s) : 0ull;
    valid_bits |= (ok ? 1ull : 0ull) << e;
    mx = fmax(mx, sl[e]);
    mn = ok ? fmin(mn, s) : mn;
  }
  mx = wave_max_f64(mx);
  mn = -wave_max_f64(-mn);
  const double above_max = mx + (fabs(mx) + 1.0);  // a finite logit above every block's

  // Bisection on the logit value keeps [lo, hi) around a cut (F(lo) meets
  // the condition, F(hi) does not) until one element is left in it, or until
  // the interval cannot shrink (equal logits); returns the key of the
  // smallest logit >= lo, the element at the cut.
  auto search = [&](auto meets, double lo, double hi, int clo, int chi) __attribute__((always_inline)) {
    while (clo - chi > 1) {
      const double mid = 0.5 * (lo + hi);
      if (!(mid > lo && mid < hi)) break;
      const int c = count_s_ge<E>(sl, mid);
      if (meets(mid, c)) {
        lo = mid;
        clo = c;
      } else {
        hi = mid;
        chi = c;
      }
    }
    return min_key_ge<E>(key, valid_bits, skey(lo));
  };

  // Top-k cut: the kk-th key in the order, and how many valid keys are above it
  const int kk = min(k, Nk);
  unsigned long long kkey = 0;
  int kabove = 0;
  if (kk > 0 && kk < Nk) {
    kkey = search([&](double, int c) { return c >= kk; }, mn, above_max, Nk, 0);  // count(S >= mn) = Nk
    kabove = count_ge<E>(key, valid_bits, kkey + 1);
  }

  // Top-p: needed only when the first kk blocks do not already hold mass p.
  // A float32 estimate of their share of the softmax decides that when it is
  // clear of p by a margin (1e-4 relative, against an estimate error below
  // 1e-5); otherwise, and whenever Top-p runs, the masses are float64.
  int kp = 0;
  unsigned long long pkey = 0;
  int pabove = 0;
  if (p > 0.0 && kk < Nk) {
    bool decided = false, k_enough = false;
    if (kk > 0) {
      const double tie_s = skey_value(kkey);
      float zf = 0.f, mf = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float ef = __builtin_amdgcn_exp2f((float)(sl[e] - mx) * 1.44269504f);  // padding: exp2(-inf) = 0
        zf += ef;
        mf += key[e] > kkey ? ef : 0.f;
      }
      zf = wave_sum_f32(zf);
      mf = wave_sum_f32(mf) + (float)(kk - kabove) * __builtin_amdgcn_exp2f((float)(tie_s - mx) * 1.44269504f);
      const double share = (double)mf / (double)zf;
      if (share >= p * (1.0 + 1e-4)) decided = k_enough = true;
      else if (share <= p * (1.0 - 1e-4)) decided = true;
    }
    if (!k_enough) {
      // float64 P = exp(S - max) / sum and its mass in 2^-62 fixed point
      double z = 0.0, ev[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ev[e] = exp(sl[e] - mx);
        z += ev[e];
      }
      z = wave_sum_f64(z);
      unsigned long long mass[E];
      unsigned long long tot = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        mass[e] = mass_of((unsigned long long)__double_as_longlong(ev[e] / z));
        tot += mass[e];
      }
      tot = wave_sum_u64(tot);
      const unsigned long long target = (unsigned long long)ceil(p * kMassScale);
      if (tot < target) {
        kp = Nk;  // p is never reached: every block
      } else {
        if (!decided) {
          const unsigned long long above_k = mass_ge<E>(key, mass, kkey + 1);
          unsigned long long tie_m = 0;  // mass of one block at the Top-k cut
#pragma unroll
          for (int e = 0; e < E; ++e) tie_m = (((valid_bits >> e) & 1ull) && key[e] == kkey) ? mass[e] : tie_m;
          tie_m = wave_fold_u64(tie_m, [](unsigned long long a, unsigned long long b) { return a > b ? a : b; });
          k_enough = kk > 0 && above_k + (unsigned long long)(kk - kabove) * tie_m >= target;
        }
        if (!k_enough) {
          // the largest logit t with mass(S >= t) >= target; the mass of the
          // blocks above the Top-k cut (or above the maximum) falls short
          double hi = above_max;
          int chi = 0;
          if (kk > 0 && kabove > 0) {
            double sk = INFINITY;  // smallest logit above the cut: S >= it exactly for those blocks
#pragma unroll
            for (int e = 0; e < E; ++e)
              if (((valid_bits >> e) & 1ull) && key[e] > kkey && sl[e] < sk) sk = sl[e];
            hi = -wave_max_f64(-sk);
            chi = kabove;
          }
          pkey = search([&](double t, int) { return mass_s_ge<E>(sl, mass, t) >= target; }, mn, hi, Nk, chi);
          pabove = count_ge<E>(key, valid_bits, pkey + 1);
          const int ptie = count_ge<E>(key, valid_bits, pkey) - pabove;
          const unsigned long long pw = mass_ge<E>(key, mass, pkey + 1);
          unsigned long long f = 0;  // mass of one block at the cut (> 0: it makes the total reach p)
#pragma unroll
          for (int e = 0; e < E; ++e) f = (((valid_bits >> e) & 1ull) && key[e] == pkey) ? mass[e] : f;
          f = wave_fold_u64(f, [](unsigned long long a, unsigned long long b) { return a > b ? a : b; });
          const unsigned long long nt = (target - pw + f - 1) / f;
          kp = pabove + (int)min(nt, (unsigned long long)ptie);
        }
      }
    }
  }
  const int nsel = max(kk, kp);
  const bool all = nsel >= Nk;
  const unsigned long long ckey = (nsel == kk) ? kkey : pkey;
  const int ties_needed = nsel - ((nsel == kk) ? kabove : pabove);

  emit_row_bits<E>(key, valid_bits, all, nsel, ckey, ties_needed, lane, brow, W);
  if (lane == 0) *count = nsel;
}

template <int E>
__global__ __launch_bounds__(256) void select_kernel(const double* __restrict__ S, long long R, int Nk,
                                                     int k, double p, int* __restrict__ counts,
                                                     uint32_t* __restrict__ bits, int W) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + wv;
  if (row >= R) return;  // whole wavefront; the kernel has no barrier
  select_row<E>(S + (size_t)row * Nk, Nk, k, p, lane, bits + (size_t)row * W, W, counts + row);
}

// ---------------------------------------------------------------- SoftTop-k
// One wavefront per mask row: M_j = sigmoid((S_j - tau) / T) with tau such
// that the weights of the row sum to k [SLA2 write-up §四: a sigmoid with a
// temperature replaces the hard Top-k in the router's first training stage].
// tau by a safeguarded Newton iteration on f(tau) = sum_j sigmoid((S_j -
// tau)/T) - k, decreasing in tau with f'(tau) = -sum_j M_j (1 - M_j) / T,
// inside a bisection bracket that starts where every weight is ~1 (f > 0)
// and ~0 (f < 0).  The iteration first runs in float32 (hardware
// exponential) to a starting point; plain float64 Newton steps from there
// converge quadratically (the safeguarded float64 iteration takes over if
// they do not settle), and the weights are written as float32.
__device__ __forceinline__ double sigmoid_f64(double x) {
  const double e = exp(-fabs(x));
  return x >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

template <int E>
__global__ __launch_bounds__(256) void soft_topk_kernel(const double* __restrict__ S, long long R, int Nk,
                                                        int k, double T, float* __restrict__ M) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;  // whole wavefront; the kernel has no barrier
  const double* srow = S + (size_t)row * Nk;
  float* mrow = M + (size_t)row * Nk;
  double sv[E];
  double lo_s = INFINITY, hi_s = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    sv[e] = j < Nk ? srow[j] : 0.0;
    if (j < Nk) {
      lo_s = fmin(lo_s, sv[e]);
      hi_s = fmax(hi_s, sv[e]);
    }
  }
  lo_s = -wave_max(-lo_s);
  hi_s = wave_max(hi_s);
  if (k <= 0 || k >= Nk) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = lane + 64 * e;
      if (j < Nk) mrow[j] = k <= 0 ? 0.f : 1.f;
    }
    return;
  }
  double lo = lo_s - 80.0 * T, hi = hi_s + 80.0 * T;  // f(lo) > 0 > f(hi)
  double tau = 0.5 * (lo + hi);
  const double inv_t = 1.0 / T;
  {
    // float32 phase: sigmoid(x) = 1 / (1 + 2^(-x log2 e)); stops once the
    // bracket or the step is at float32 resolution
    float l32 = (float)lo, h32 = (float)hi, t32 = (float)tau;
    const float it32 = (float)inv_t;
    for (int it = 0; it < 96; ++it) {
      float f = 0.f, g = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (lane + 64 * e < Nk) {
          const float x = ((float)sv[e] - t32) * it32;
          const float m = 1.f / (1.f + __builtin_amdgcn_exp2f(-1.44269504f * x));
          f += m;
          g += m * (1.f - m);
        }
      }
      f = wave_sum_f32(f) - (float)k;
      g = wave_sum_f32(g) * it32;
      if (f == 0.f) break;
      if (f > 0.f) l32 = t32; else h32 = t32;
      const float nt = g > 0.f ? t32 + f / g : 0.5f * (l32 + h32);
      const float next = (nt > l32 && nt < h32) ? nt : 0.5f * (l32 + h32);
      const bool done = next == t32 || h32 - l32 <= 1e-6f * fmaxf(fabsf(l32), fabsf(h32));
      t32 = next;
      if (done) break;
    }
    if ((double)t32 > lo && (double)t32 < hi) tau = (double)t32;
  }
  // float64 Newton from the float32 root (quadratic convergence: a few
  // steps); if it has not settled after 10, the safeguarded iteration below
  // starts again from the whole bracket
  bool done = false;
  {
    double t = tau;
    for (int it = 0; it < 10; ++it) {
      double f = 0.0, g = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (lane + 64 * e < Nk) {
          const double m = sigmoid_f64((sv[e] - t) * inv_t);
          f += m;
          g += m * (1.0 - m);
        }
      }
      f = wave_sum_f64(f) - (double)k;
      g = wave_sum_f64(g) * inv_t;
      if (f == 0.0) {
        done = true;
        break;
      }
      if (!(g > 0.0)) break;
      const double next = t + f / g;
      if (!(next > lo && next < hi)) break;
      const bool tiny = fabs(next - t) <= 4.0 * DBL_EPSILON * fmax(fabs(t), T);
      t = next;
      if (tiny) {
        done = true;
        break;
      }
    }
    if (done) tau = t;
    else tau = 0.5 * (lo + hi);
  }
  for (int it = 0; it < 200 && !done; ++it) {  // uniform: every lane sees the same sums
    double f = 0.0, g = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (lane + 64 * e < Nk) {
        const double m = sigmoid_f64((sv[e] - tau) * inv_t);
        f += m;
        g += m * (1.0 - m);
      }
    }
    f = wave_sum_f64(f) - (double)k;
    g = wave_sum_f64(g) * inv_t;
    if (f == 0.0) break;
    if (f > 0.0) lo = tau; else hi = tau;
    const double nt = g > 0.0 ? tau + f / g : 0.5 * (lo + hi);
    const double next = (nt > lo && nt < hi) ? nt : 0.5 * (lo + hi);
    if (next == tau || hi - lo <= 4.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi))) break;
    tau = next;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    if (j < Nk) mrow[j] = (float)sigmoid_f64((sv[e] - tau) * inv_t);
  }
}

// CSR from the per-row counts and bitmasks, in one launch.  Workgroup g
// (256 threads) owns rows [256 g, 256 g + 256), one thread per row: the
// counts of every earlier row are summed by the whole workgroup (int4 loads,
// wavefront reductions, the four wavefronts in a fixed order), its own 256
// counts scanned (wavefront scans, then the wavefront totals), the rows'
// row_ptr entries written (the last row's thread also row_ptr[R]), and each
// thread turns its row's bitmask words into ascending block indices.
constexpr int kEmitRows = kThreads;

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(kThreads) void scan_emit_kernel(const int* __restrict__ counts,
                                                             const uint32_t* __restrict__ bits,
                                                             int* __restrict__ row_ptr, int* __restrict__ col_idx,
                                                             long long R, int W) {
  __shared__ int wsum[kThreads / 64];
  __shared__ int wtot[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const long long r0 = (long long)blockIdx.x * kEmitRows;
  const long long row = r0 + tid;
  const int c = row < R ? counts[row] : 0;
  // counts of rows [0, r0) (r0 a multiple of 4)
  int acc = 0;
  for (long long i = 4 * (long long)tid; i < r0; i += 4 * kThreads) {
    const int4 q = *reinterpret_cast<const int4*>(counts + i);
    acc += (q.x + q.y) + (q.z + q.w);
  }
  acc = wave_sum_i32(acc);
  int incl = c;  // inclusive scan of this wavefront's counts
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 0) wsum[wv] = acc;
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  int start = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  for (int u = 0; u < wv; ++u) start += wtot[u];
  start += incl - c;
  if (row < R) {
    row_ptr[row] = start;
    if (row == R - 1) row_ptr[R] = start + c;
    const uint32_t* brow = bits + (size_t)row * W;
    int pos = start;
    // eight words loaded together, then expanded (the loads do not wait for
    // one another behind the stores)
    for (int w0 = 0; w0 < W; w0 += 8) {
      uint32_t x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = w0 + u < W ? brow[w0 + u] : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        while (x[u]) {
          col_idx[pos++] = 32 * (w0 + u) + (__ffs(x[u]) - 1);
          x[u] &= x[u] - 1u;
        }
      }
    }
  }
}




}  // namespace

namespace {

// Pooling, optional router and the pooled logits S [B, H, Nq, Nk] (float64).
hipError_t launch_scores(const Shape& s, const float* Wq, const float* Wk, const void* Q, const void* K,
                         double* S, char* ws, const WsLayout& L, hipStream_t st, const float* kdone = nullptr) {
  const long long BH = (long long)s.B * s.H;
  double* qbar = reinterpret_cast<double*>(ws + L.qbar);
  double* kbar = reinterpret_cast<double*>(ws + L.kbar);

  const dim3 gpool((unsigned)(BH * (s.Nq + s.Nk)));
#define SLA_POOL(T, DD)                                                                          \
  hipLaunchKernelGGL((pool_kernel<T, DD>), gpool, dim3(kThreads), 0, st,                          \
                     reinterpret_cast<const T*>(Q), reinterpret_cast<const T*>(K), s.N, s.bq,   \
                     s.bk, s.Nq, s.Nk, BH, s.H, kdone, qbar, kbar)
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
    // (q_bar W_q) . (k_bar W_k) = (q_bar W_q W_k^T) . k_bar: one projection,
    // of the query side (half as many rows as the key side), through the
    // product of the two matrices
    double* qhat = reinterpret_cast<double*>(ws + L.qhat);
    double* wqk = reinterpret_cast<double*>(ws + L.wqk);
    const long long Mq = BH * s.Nq;
    if (s.d == 128) {
      hipLaunchKernelGGL((router_pair_kernel<128>), dim3(128), dim3(128), 0, st, Wq, Wk, wqk);
      hipLaunchKernelGGL((router_kernel<128, double>), dim3((unsigned)((Mq + 31) / 32)), dim3(kThreads), 0,
                         st, qbar, wqk, qhat, Mq);
    } else {
      hipLaunchKernelGGL((router_pair_kernel<64>), dim3(64), dim3(64), 0, st, Wq, Wk, wqk);
      hipLaunchKernelGGL((router_kernel<64, double>), dim3((unsigned)((Mq + 31) / 32)), dim3(kThreads), 0,
                         st, qbar, wqk, qhat, Mq);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    qh = qhat;
  }

  const int tiles_j = (s.Nk + 31) / 32, tiles = ((s.Nq + 31) / 32) * tiles_j;
  const dim3 gscore((unsigned)(BH * tiles));
  if (s.d == 128)
    hipLaunchKernelGGL((score_kernel<128>), gscore, dim3(kThreads), 0, st, qh, kh, S, s.Nq, s.Nk, tiles_j, tiles);
  else
    hipLaunchKernelGGL((score_kernel<64>), gscore, dim3(kThreads), 0, st, qh, kh, S, s.Nq, s.Nk, tiles_j, tiles);
  return hipGetLastError();
}

template <int E>
hipError_t launch_soft(const double* S, long long R, int Nk, int k, double T, float* M, hipStream_t st) {
  hipLaunchKernelGGL((soft_topk_kernel<E>), dim3((unsigned)((R + 3) / 4)), dim3(kThreads), 0, st, S, R, Nk,
                     k, T, M);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_soft_topk(const Shape& s, int k, double T, const float* Wq, const float* Wk,
                            const void* Q, const void* K, float* M, char* ws, const WsLayout& L,
                            hipStream_t st) {
  double* S = reinterpret_cast<double*>(ws + L.S);
  hipError_t e = launch_scores(s, Wq, Wk, Q, K, S, ws, L, st);
  if (e != hipSuccess) return e;
  const long long R = s.R();
  int E = 1;
  while (64 * E < s.Nk) E <<= 1;
  switch (E) {
    case 1: return launch_soft<1>(S, R, s.Nk, k, T, M, st);
    case 2: return launch_soft<2>(S, R, s.Nk, k, T, M, st);
    case 4: return launch_soft<4>(S, R, s.Nk, k, T, M, st);
    case 8: return launch_soft<8>(S, R, s.Nk, k, T, M, st);
    case 16: return launch_soft<16>(S, R, s.Nk, k, T, M, st);
    case 32: return launch_soft<32>(S, R, s.Nk, k, T, M, st);
    default: return launch_soft<64>(S, R, s.Nk, k, T, M, st);
  }
}

hipError_t launch_mask(const Shape& s, int k, double p, const float* Wq, const float* Wk,
                       const void* Q, const void* K, int32_t* row_ptr, int32_t* col_idx,
                       double* logits_out, char* ws, const WsLayout& L, hipStream_t st,
                       const float* kdone) {
  const long long R = s.R();
  double* S = logits_out ? logits_out : reinterpret_cast<double*>(ws + L.S);
  int* counts = reinterpret_cast<int*>(ws + L.counts);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + L.bits);
  const int W = s.words();
  hipError_t e = launch_scores(s, Wq, Wk, Q, K, S, ws, L, st, kdone);
  if (e != hipSuccess) return e;

  // blocks per lane: the smallest listed E with 64 E >= Nk (element j of a row
  // is lane j % 64, slot j / 64; slots past Nk are invalid and cost work)
  static constexpr int kE[] = {1, 2, 4, 8, 12, 16, 20, 24, 32, 40, 48, 64};
  int E = 64;
  for (int c : kE)
    if (64 * c >= s.Nk) {
      E = c;
      break;
    }
  const dim3 gsel((unsigned)((R + 3) / 4));
#define SLA_SELECT(EE) \
  case EE: hipLaunchKernelGGL((select_kernel<EE>), gsel, dim3(kThreads), 0, st, S, R, s.Nk, k, p, counts, bits, W); break
  switch (E) {
    SLA_SELECT(1); SLA_SELECT(2); SLA_SELECT(4); SLA_SELECT(8); SLA_SELECT(12); SLA_SELECT(16);
    SLA_SELECT(20); SLA_SELECT(24); SLA_SELECT(32); SLA_SELECT(40); SLA_SELECT(48);
    default: hipLaunchKernelGGL((select_kernel<64>), gsel, dim3(kThreads), 0, st, S, R, s.Nk, k, p, counts, bits, W);
  }
#undef SLA_SELECT
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_emit_kernel, dim3((unsigned)((R + kEmitRows - 1) / kEmitRows)), dim3(kThreads), 0, st,
                     counts, bits, row_ptr, col_idx, R, W);
  return hipGetLastError();
}

}  // namespace sla
