// bf16 attention over the block mask on gfx950 matrix cores.
//
// Sources: SLA2 write-up (arXiv:2602.12675) §一 (exact sparse attention for the
// selected blocks, linear attention for the rest) and §二 (O = alpha O_s +
// (1 - alpha) O_l with a learnable ratio); SpargeAttention2 write-up
// "清華發明AI「注意力瘦身術」：視頻生成速度提升16倍的神奇技術" §四 (each block
// is computed whole or skipped whole).  phi(x) = elu(x) + 1 as in Katharopoulos
// et al. 2020.
//
// One workgroup per mask row (b, h, query block of BQ rows), BQ/32 wavefronts,
// each owning 32 query rows.  For every listed key block the K tile, V^T and
// (linear branch) phi(K)^T are staged in LDS; the next block's tiles are
// fetched into registers while the current one is computed.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16; lane l holds operand
// row/column l%32 and k-slice 8*(l/32) .. +7):
//   S^T  (keys x queries)  = K  . Q^T          A = K tile, B = Q (registers)
//   O^T  (d x queries)    += V^T . P^T         A = V^T tile, B = P (registers)
//   G    (d x d)          += phi(K)^T . V      A = phi(K)^T tile, B = V^T tile
// With queries on the lane axis of both S^T and O^T, every softmax statistic
// of a lane belongs to its own query: row max / sum need one exchange with
// lane l^32 and the output rescale is lane-local.  The accumulator layout of
// S^T lists keys in the order (0-3, 8-11 | 4-7, 12-15) per 16; V^T and
// phi(K)^T are stored in LDS with bits 2 and 3 of the key offset swapped so
// that the P fragment taken straight from the accumulator lines up with them.
//
// Linear branch: H_u = H - G and z_u = z - g where H, z are per-head totals
// from the summary pass and G, g the sums over the selected blocks, so
// O_l = phi(Q) H_u / phi(Q) z_u.  phi(Q) H_u is evaluated with a split
// (hi + lo bf16) of both factors, which keeps ~16 mantissa bits.
#include "sla_internal.h"

namespace sla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack2(float a, float b) { return f2bf(a) | (f2bf(b) << 16); }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// Position of key offset o inside its 16-key group in the LDS transposed tiles.
__device__ __forceinline__ int kperm(int o) { return (o & ~12) | ((o & 4) << 1) | ((o & 8) >> 1); }

// element e (0..7) of a 16-byte chunk of bf16
__device__ __forceinline__ uint32_t elem(const uint4& v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int D, int BQ, int BK>
struct Cfg {
  static constexpr int NW = BQ / 32;          // wavefronts
  static constexpr int NT = NW * 64;          // threads
  static constexpr int KST = D + 8;           // K tile row stride (elements)
  static constexpr int VST = BK + 8;          // V^T / phi(K)^T row stride
  static constexpr int HST = D + 8;           // H_u^T row stride
  static constexpr int PAIRS = (BK / 4) * (D / 8);         // (4-key group, 8-d chunk) pairs
  static constexpr int ST = (PAIRS + NT - 1) / NT;         // pairs per thread
  static constexpr int KS_BYTES = BK * KST * 2;
  static constexpr int VT_BYTES = D * VST * 2;
  static constexpr int LOOP_BYTES = KS_BYTES + 2 * VT_BYTES;
  static constexpr int HU_BYTES = 2 * D * HST * 2;
  static constexpr int MAIN_BYTES = LOOP_BYTES > HU_BYTES ? LOOP_BYTES : HU_BYTES;
  static constexpr int ZU_OFF = MAIN_BYTES;                // float z_u[D]
  static constexpr int GRED_OFF = ZU_OFF + D * 4;          // float [NT][8]
  static constexpr int SMEM = GRED_OFF + NT * 8 * 4;
  static constexpr int TT = (D / 32) * (D / 32);           // 32x32 tiles of G
  static constexpr int TPW = (TT + NW - 1) / NW;           // G tiles per wavefront
};

// Global -> register staging of one key block (K and V chunks of 4 keys x 8 d).
template <int D, int BQ, int BK>
struct Stage {
  using C = Cfg<D, BQ, BK>;
  uint4 k[C::ST][4];
  uint4 v[C::ST][4];

  __device__ __forceinline__ void load(const uint16_t* Kb, const uint16_t* Vb, int key0, int N,
                                       bool needK, int tid) {
#pragma unroll
    for (int s = 0; s < C::ST; ++s) {
      const int pi = tid + C::NT * s;
      const int c = pi % (D / 8), g = pi / (D / 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int key = key0 + 4 * g + u;
        const bool ok = (pi < C::PAIRS) && key < N;
        const size_t off = (size_t)key * D + c * 8;
        k[s][u] = (ok && needK) ? *reinterpret_cast<const uint4*>(Kb + off) : make_uint4(0, 0, 0, 0);
        v[s][u] = ok ? *reinterpret_cast<const uint4*>(Vb + off) : make_uint4(0, 0, 0, 0);
      }
    }
  }

  // Writes K (row-major), V^T and, if lin, phi(K)^T (permuted key order) to
  // LDS; accumulates the column sums of phi(K) over valid keys into gpart.
  // With split, phi(K)^T is written twice: hi part to pk, lo part to pk_lo.
  template <bool SPLIT>
  __device__ __forceinline__ void store(uint16_t* Ks, uint16_t* Vt, uint16_t* Pk, uint16_t* Pk_lo,
                                        bool doK, bool lin, int key0, int N, int tid,
                                        float* gpart) {
#pragma unroll
    for (int s = 0; s < C::ST; ++s) {
      const int pi = tid + C::NT * s;
      if (pi >= C::PAIRS) continue;
      const int c = pi % (D / 8), g = pi / (D / 8);
      const int col = (4 * g) & ~15;
      const int pos = col + kperm((4 * g) & 15);
      if (doK) {
#pragma unroll
        for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(Ks + (4 * g + u) * C::KST + c * 8) = k[s][u];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 w;
        w.x = elem(v[s][0], e) | (elem(v[s][1], e) << 16);
        w.y = elem(v[s][2], e) | (elem(v[s][3], e) << 16);
        *reinterpret_cast<uint2*>(Vt + (c * 8 + e) * C::VST + pos) = w;
      }
      if (lin) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float f[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const bool ok = key0 + 4 * g + u < N;
            f[u] = ok ? phi(bf2f(elem(k[s][u], e))) : 0.f;
            gpart[e] += f[u];
          }
          uint2 w;
          if (!SPLIT) {
            w.x = pack2(f[0], f[1]);
            w.y = pack2(f[2], f[3]);
            *reinterpret_cast<uint2*>(Pk + (c * 8 + e) * C::VST + pos) = w;
          } else {
            uint32_t h[4];
            float lo[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              h[u] = f2bf(f[u]);
              lo[u] = f[u] - bf2f(h[u]);
            }
            w.x = h[0] | (h[1] << 16);
            w.y = h[2] | (h[3] << 16);
            *reinterpret_cast<uint2*>(Pk + (c * 8 + e) * C::VST + pos) = w;
            w.x = pack2(lo[0], lo[1]);
            w.y = pack2(lo[2], lo[3]);
            *reinterpret_cast<uint2*>(Pk_lo + (c * 8 + e) * C::VST + pos) = w;
          }
        }
      }
    }
  }
};

template <int D, int BQ, int BK, int MODE>
__global__ __launch_bounds__(BQ / 32 * 64) void attn_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, const float* __restrict__ alpha,
    const float* __restrict__ htot, uint16_t* __restrict__ O, int H, int N, int Nq, int Nk,
    float scale_log2) {
  using C = Cfg<D, BQ, BK>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vt = reinterpret_cast<uint16_t*>(smem + C::KS_BYTES);
  uint16_t* Pk = reinterpret_cast<uint16_t*>(smem + C::KS_BYTES + C::VT_BYTES);
  uint16_t* HuHi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* HuLo = reinterpret_cast<uint16_t*>(smem + D * C::HST * 2);
  float* zu = reinterpret_cast<float*>(smem + C::ZU_OFF);
  float* gred = reinterpret_cast<float*>(smem + C::GRED_OFF);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const long long row = blockIdx.x;
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  const int h = (int)(bh % H);

  int nsel, base = 0;
  if (MODE == MODE_DENSE) {
    nsel = Nk;
  } else {
    base = row_ptr[row];
    nsel = row_ptr[row + 1] - base;
  }
  float ws_ = 0.f, wl_ = 0.f;
  if (MODE == MODE_FUSED) {
    const float a = alpha[h];
    ws_ = a;
    wl_ = 1.f - a;
  } else if (MODE == MODE_LINEAR) {
    wl_ = 1.f;
  } else {
    ws_ = 1.f;
  }
  const bool do_s = ws_ != 0.f;
  const bool lin = (wl_ != 0.f) && (nsel < Nk);
  const int nblk = (do_s || lin) ? nsel : 0;

  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;

  // Q fragments of this wavefront's 32 query rows
  const int q = qi * BQ + 32 * w + l32;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (q < N) v = *reinterpret_cast<const uint4*>(Q + ((size_t)bh * N + q) * D + 16 * t + 8 * hi);
    qf[t] = as_bf16x8(v);
  }

  f32x16 acc_o[D / 32];
  f32x16 acc_g[C::TPW];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = f32x16{};
#pragma unroll
  for (int t = 0; t < C::TPW; ++t) acc_g[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  float gpart[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gpart[e] = 0.f;

  Stage<D, BQ, BK> stg;
  if (nblk > 0) {
    const int j0 = (MODE == MODE_DENSE) ? 0 : col_idx[base];
    stg.load(Kb, Vb, j0 * BK, N, true, tid);
  }
  for (int b = 0; b < nblk; ++b) {
    const int j = (MODE == MODE_DENSE) ? b : col_idx[base + b];
    const int key0 = j * BK;
    __syncthreads();
    stg.template store<false>(Ks, Vt, Pk, nullptr, do_s, lin, key0, N, tid, gpart);
    __syncthreads();
    if (b + 1 < nblk) {
      const int jn = (MODE == MODE_DENSE) ? b + 1 : col_idx[base + b + 1];
      stg.load(Kb, Vb, jn * BK, N, true, tid);
    }
    if (do_s) {
      // S^T = K Q^T for BK/32 key tiles
      f32x16 sacc[BK / 32];
#pragma unroll
      for (int kt = 0; kt < BK / 32; ++kt) {
        f32x16 a = f32x16{};
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const uint4 kv = *reinterpret_cast<const uint4*>(Ks + (32 * kt + l32) * C::KST + 16 * t + 8 * hi);
          a = mfma(as_bf16x8(kv), qf[t], a);
        }
        sacc[kt] = a;
      }
      // mask keys past N (only the last block can be partial)
      if (key0 + BK > N) {
#pragma unroll
        for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kt + 8 * (i >> 2) + 4 * hi + (i & 3);
            if (key >= N) sacc[kt][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float corr = exp2f((m_run - m_new) * scale_log2);
      const float mneg = -m_new * scale_log2;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = exp2f(fmaf(sacc[kt][i], scale_log2, mneg));
          sacc[kt][i] = pv;
          psum += pv;
        }
      l_run = l_run * corr + psum;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) acc_o[t] *= corr;
      // O^T += V^T P^T
#pragma unroll
      for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint4 pb;
          pb.x = pack2(sacc[kt][8 * s + 0], sacc[kt][8 * s + 1]);
          pb.y = pack2(sacc[kt][8 * s + 2], sacc[kt][8 * s + 3]);
          pb.z = pack2(sacc[kt][8 * s + 4], sacc[kt][8 * s + 5]);
          pb.w = pack2(sacc[kt][8 * s + 6], sacc[kt][8 * s + 7]);
          const bf16x8 bp = as_bf16x8(pb);
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const uint4 vv = *reinterpret_cast<const uint4*>(Vt + (32 * dt + l32) * C::VST + 32 * kt + 16 * s + 8 * hi);
            acc_o[dt] = mfma(as_bf16x8(vv), bp, acc_o[dt]);
          }
        }
    }
    if (lin) {
      // G += phi(K)^T V over this block
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
#pragma unroll
        for (int u = 0; u < C::TPW; ++u) {
          const int tix = w * C::TPW + u;
          if (tix >= C::TT) continue;
          const int mt = tix / (D / 32), nt = tix % (D / 32);
          const uint4 av = *reinterpret_cast<const uint4*>(Pk + (32 * mt + l32) * C::VST + 16 * s + 8 * hi);
          const uint4 bv = *reinterpret_cast<const uint4*>(Vt + (32 * nt + l32) * C::VST + 16 * s + 8 * hi);
          acc_g[u] = mfma(as_bf16x8(av), as_bf16x8(bv), acc_g[u]);
        }
      }
    }
  }

  // ---------------- epilogue
  float inv_l = 0.f;
  if (do_s) {
    const float lt = l_run + __shfl_xor(l_run, 32);
    inv_l = lt > 0.f ? 1.f / lt : 0.f;
  }
  float den = 1.f;
  if (lin) {
    const float* Hh = htot + (size_t)bh * (D * D + D);
    __syncthreads();  // all wavefronts are done with the loop tiles
#pragma unroll
    for (int e = 0; e < 8; ++e) gred[tid * 8 + e] = gpart[e];
    // H_u^T = (H - G)^T as hi + lo bf16
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      const int tix = w * C::TPW + u;
      if (tix >= C::TT) continue;
      const int mt = tix / (D / 32), nt = tix % (D / 32);
      const int dv = 32 * nt + l32;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dk = 32 * mt + 8 * i4 + 4 * hi;
        float hv[4];
        uint32_t hb[4];
        float lv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hv[r] = Hh[(dk + r) * D + dv] - acc_g[u][4 * i4 + r];
          hb[r] = f2bf(hv[r]);
          lv[r] = hv[r] - bf2f(hb[r]);
        }
        uint2 wv;
        wv.x = hb[0] | (hb[1] << 16);
        wv.y = hb[2] | (hb[3] << 16);
        *reinterpret_cast<uint2*>(HuHi + dv * C::HST + dk) = wv;
        wv.x = pack2(lv[0], lv[1]);
        wv.y = pack2(lv[2], lv[3]);
        *reinterpret_cast<uint2*>(HuLo + dv * C::HST + dk) = wv;
      }
    }
    __syncthreads();
    if (tid < D) {
      const int c = tid >> 3, e = tid & 7;
      float g = 0.f;
      for (int t = c; t < C::NT; t += D / 8) g += gred[t * 8 + e];
      zu[tid] = Hh[D * D + tid] - g;
    }
    __syncthreads();
  }

  const size_t orow = ((size_t)bh * N + q) * D;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
    f32x16 ol = f32x16{};
    if (lin) {
      // phi(Q) fragments (hi, lo) and the denominator, recomputed per tile to
      // keep register pressure low
      f32x16 acc_n = f32x16{};
      float dpart = 0.f;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const uint4 qv = __builtin_bit_cast(uint4, qf[t]);
        float f[8];
        uint32_t fh[8];
        float fl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f[e] = phi(bf2f(elem(qv, e)));
          fh[e] = f2bf(f[e]);
          fl[e] = f[e] - bf2f(fh[e]);
          if (mt == 0) dpart = fmaf(f[e], zu[16 * t + 8 * hi + e], dpart);
        }
        const uint4 bh4 = make_uint4(fh[0] | (fh[1] << 16), fh[2] | (fh[3] << 16),
                                     fh[4] | (fh[5] << 16), fh[6] | (fh[7] << 16));
        const uint4 bl4 = make_uint4(pack2(fl[0], fl[1]), pack2(fl[2], fl[3]), pack2(fl[4], fl[5]),
                                     pack2(fl[6], fl[7]));
        const uint4 ah = *reinterpret_cast<const uint4*>(HuHi + (32 * mt + l32) * C::HST + 16 * t + 8 * hi);
        const uint4 al = *reinterpret_cast<const uint4*>(HuLo + (32 * mt + l32) * C::HST + 16 * t + 8 * hi);
        acc_n = mfma(as_bf16x8(ah), as_bf16x8(bh4), acc_n);
        acc_n = mfma(as_bf16x8(ah), as_bf16x8(bl4), acc_n);
        acc_n = mfma(as_bf16x8(al), as_bf16x8(bh4), acc_n);
      }
      if (mt == 0) den = dpart + __shfl_xor(dpart, 32);
      const float inv_den = 1.f / den;
#pragma unroll
      for (int i = 0; i < 16; ++i) ol[i] = acc_n[i] * inv_den;
    }
    if (q < N) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * i4 + r;
          o[r] = ws_ * (acc_o[mt][i] * inv_l) + wl_ * ol[i];
        }
        uint2 wv;
        wv.x = pack2(o[0], o[1]);
        wv.y = pack2(o[2], o[3]);
        *reinterpret_cast<uint2*>(O + orow + 32 * mt + 8 * i4 + 4 * hi) = wv;
      }
    }
  }
}

// Linear summaries of one chunk of key blocks of one head:
//   Gp = sum_u phi(k_u)^T v_u (d x d), zp = sum_u phi(k_u)
// with phi(K) split into hi + lo bf16 parts (V is exact in bf16).
template <int D, int BK>
__global__ __launch_bounds__(256) void summary_kernel(const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      const float* __restrict__ alpha, int H, int N,
                                                      int Nk, int chunk_blocks, int nchunk,
                                                      float* __restrict__ hpart) {
  constexpr int BQ = 128;  // 4 wavefronts
  using C = Cfg<D, BQ, BK>;
  __shared__ __attribute__((aligned(16))) char smem[3 * C::VT_BYTES + C::NT * 8 * 4];
  uint16_t* Vt = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Pk = reinterpret_cast<uint16_t*>(smem + C::VT_BYTES);
  uint16_t* PkLo = reinterpret_cast<uint16_t*>(smem + 2 * C::VT_BYTES);
  float* gred = reinterpret_cast<float*>(smem + 3 * C::VT_BYTES);

  const long long bh = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  const int h = (int)(bh % H);
  if (alpha != nullptr && alpha[h] == 1.f) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  const int jb = chunk * chunk_blocks, je = min(Nk, jb + chunk_blocks);

  f32x16 acc_g[C::TPW];
#pragma unroll
  for (int t = 0; t < C::TPW; ++t) acc_g[t] = f32x16{};
  float gpart[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gpart[e] = 0.f;

  Stage<D, BQ, BK> stg;
  if (jb < je) stg.load(Kb, Vb, jb * BK, N, true, tid);
  for (int j = jb; j < je; ++j) {
    __syncthreads();
    stg.template store<true>(nullptr, Vt, Pk, PkLo, false, true, j * BK, N, tid, gpart);
    __syncthreads();
    if (j + 1 < je) stg.load(Kb, Vb, (j + 1) * BK, N, true, tid);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
#pragma unroll
      for (int u = 0; u < C::TPW; ++u) {
        const int tix = w * C::TPW + u;
        if (tix >= C::TT) continue;
        const int mt = tix / (D / 32), nt = tix % (D / 32);
        const uint4 ah = *reinterpret_cast<const uint4*>(Pk + (32 * mt + l32) * C::VST + 16 * s + 8 * hi);
        const uint4 al = *reinterpret_cast<const uint4*>(PkLo + (32 * mt + l32) * C::VST + 16 * s + 8 * hi);
        const uint4 bv = *reinterpret_cast<const uint4*>(Vt + (32 * nt + l32) * C::VST + 16 * s + 8 * hi);
        acc_g[u] = mfma(as_bf16x8(ah), as_bf16x8(bv), acc_g[u]);
        acc_g[u] = mfma(as_bf16x8(al), as_bf16x8(bv), acc_g[u]);
      }
    }
  }
  float* out = hpart + ((size_t)bh * nchunk + chunk) * (D * D + D);
#pragma unroll
  for (int u = 0; u < C::TPW; ++u) {
    const int tix = w * C::TPW + u;
    if (tix >= C::TT) continue;
    const int mt = tix / (D / 32), nt = tix % (D / 32);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int dk = 32 * mt + 8 * (i >> 2) + 4 * hi + (i & 3);
      out[dk * D + 32 * nt + l32] = acc_g[u][i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) gred[tid * 8 + e] = gpart[e];
  __syncthreads();
  if (tid < D) {
    const int c = tid >> 3, e = tid & 7;
    float g = 0.f;
    for (int t = c; t < C::NT; t += D / 8) g += gred[t * 8 + e];
    out[D * D + tid] = g;
  }
}

}  // namespace

// Sum the per-chunk partials of every head in chunk order (deterministic).
__global__ __launch_bounds__(256) void summary_reduce_kernel(const float* __restrict__ hpart,
                                                             const float* __restrict__ alpha, int H,
                                                             int nchunk, int per, float* __restrict__ htot) {
  const long long bh = blockIdx.y;
  if (alpha != nullptr && alpha[bh % H] == 1.f) return;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= per) return;
  const float* src = hpart + (size_t)bh * nchunk * per + e;
  float s = 0.f;
  for (int c = 0; c < nchunk; ++c) s += src[(size_t)c * per];
  htot[(size_t)bh * per + e] = s;
}

namespace {

template <int D, int BQ, int BK>
hipError_t attn_dispatch(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                         const int32_t* rp, const int32_t* ci, const float* alpha, const float* htot,
                         void* O, hipStream_t st) {
  using C = Cfg<D, BQ, BK>;
  const dim3 grid((unsigned)s.R()), block(C::NT);
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(K);
  const uint16_t* v = static_cast<const uint16_t*>(V);
  uint16_t* o = static_cast<uint16_t*>(O);
  switch (mode) {
    case MODE_SPARSE:
      hipLaunchKernelGGL((attn_kernel<D, BQ, BK, MODE_SPARSE>), grid, block, 0, st, q, k, v, rp, ci,
                         alpha, htot, o, s.H, s.N, s.Nq, s.Nk, sl2);
      break;
    case MODE_LINEAR:
      hipLaunchKernelGGL((attn_kernel<D, BQ, BK, MODE_LINEAR>), grid, block, 0, st, q, k, v, rp, ci,
                         alpha, htot, o, s.H, s.N, s.Nq, s.Nk, sl2);
      break;
    case MODE_FUSED:
      hipLaunchKernelGGL((attn_kernel<D, BQ, BK, MODE_FUSED>), grid, block, 0, st, q, k, v, rp, ci,
                         alpha, htot, o, s.H, s.N, s.Nq, s.Nk, sl2);
      break;
    default:
      hipLaunchKernelGGL((attn_kernel<D, BQ, BK, MODE_DENSE>), grid, block, 0, st, q, k, v, rp, ci,
                         alpha, htot, o, s.H, s.N, s.Nq, s.Nk, sl2);
      break;
  }
  return hipGetLastError();
}

template <int D, int BK>
hipError_t summary_dispatch(const Shape& s, const void* K, const void* V, const float* alpha,
                            char* ws, const WsLayout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H;
  float* hpart = reinterpret_cast<float*>(ws + L.hpart);
  float* htot = reinterpret_cast<float*>(ws + L.htot);
  hipLaunchKernelGGL((summary_kernel<D, BK>), dim3((unsigned)(BH * L.nchunk)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), alpha, s.H,
                     s.N, s.Nk, L.chunk_blocks, L.nchunk, hpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per = D * D + D;
  hipLaunchKernelGGL(summary_reduce_kernel, dim3((unsigned)((per + 255) / 256), (unsigned)BH), dim3(256),
                     0, st, hpart, alpha, s.H, L.nchunk, per, htot);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                            const int32_t* rp, const int32_t* ci, const float* alpha,
                            const float* htot, void* O, hipStream_t st) {
#define SLA_ATTN(DD, QQ, KK)                                                           \
  if (s.d == DD && s.bq == QQ && s.bk == KK)                                           \
    return attn_dispatch<DD, QQ, KK>(s, mode, Q, K, V, rp, ci, alpha, htot, O, st);
  SLA_ATTN(128, 128, 64)
  SLA_ATTN(128, 128, 128)
  SLA_ATTN(128, 64, 64)
  SLA_ATTN(128, 64, 128)
  SLA_ATTN(64, 128, 64)
  SLA_ATTN(64, 128, 128)
  SLA_ATTN(64, 64, 64)
  SLA_ATTN(64, 64, 128)
#undef SLA_ATTN
  return hipErrorInvalidValue;
}

hipError_t launch_summary_reduce(const float* hpart, const float* alpha, int H, long long BH,
                                 int nchunk, int per, float* htot, hipStream_t st) {
  hipLaunchKernelGGL(summary_reduce_kernel, dim3((unsigned)((per + 255) / 256), (unsigned)BH), dim3(256),
                     0, st, hpart, alpha, H, nchunk, per, htot);
  return hipGetLastError();
}

hipError_t launch_summary_bf16(const Shape& s, const void* K, const void* V, const float* alpha,
                               char* ws, const WsLayout& L, hipStream_t st) {
  if (s.d == 128 && s.bk == 64) return summary_dispatch<128, 64>(s, K, V, alpha, ws, L, st);
  if (s.d == 128 && s.bk == 128) return summary_dispatch<128, 128>(s, K, V, alpha, ws, L, st);
  if (s.d == 64 && s.bk == 64) return summary_dispatch<64, 64>(s, K, V, alpha, ws, L, st);
  if (s.d == 64 && s.bk == 128) return summary_dispatch<64, 128>(s, K, V, alpha, ws, L, st);
  return hipErrorInvalidValue;
}

}  // namespace sla
