// bf16 attention over the block mask on gfx950 matrix cores.
//
// Sources: SLA2 write-up (arXiv:2602.12675) §一 (exact sparse attention for the
// selected blocks, linear attention for the rest) and §二 (O = alpha O_s +
// (1 - alpha) O_l with a learnable ratio); SpargeAttention2 write-up
// "清華發明AI「注意力瘦身術」：視頻生成速度提升16倍的神奇技術" §四 (each block
// is computed whole or skipped whole).  phi(x) = elu(x) + 1 as in Katharopoulos
// et al. 2020.
//
// Two kernels:
//
// prep_kernel (one workgroup per chunk of key blocks of one head) streams K and
//   V once and writes, per head, V^T and phi(K)^T as [d, Nk*bk] bf16 (keys past
//   N zero), the per-key-block column sums of phi(K) (float32), and partial
//   linear totals H = sum_u phi(k_u)^T v_u, z = sum_u phi(k_u) (phi(K) split
//   into hi + lo bf16 so the totals keep ~16 mantissa bits).  Within every 16
//   keys the transposed tiles store key offset o at position o with bits 2 and
//   3 swapped (see below).
//
// attn_kernel (one workgroup per mask row = (b, h, query block of BQ rows),
//   BQ/32 wavefronts of 32 query rows each) walks the row's key blocks.  The
//   K tile, the V^T tile and (linear branch) the phi(K)^T tile of a block go
//   straight from global memory to LDS (global_load_lds, 16 bytes per lane);
//   16-byte chunks are XOR-swizzled by row so the matrix-core operand reads are
//   free of bank conflicts.  Sparse and dense modes double-buffer the tiles.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16; lane l supplies operand
// row / column l%32 and a k-slice 8*(l/32) .. +7; accumulator element i of
// lane l is row 8*(i/4) + 4*(l/32) + i%4, column l%32):
//   S^T  (keys x queries)  = K . Q^T           A = K tile, B = Q (registers)
//   O^T  (d x queries)    += V^T . P^T          A = V^T tile, B = P (registers)
//   G    (d x d)          += phi(K)^T . V       A = phi(K)^T tile, B = V^T tile
// With queries on the lane axis of S^T and O^T, each lane's softmax state is
// its own query's: the row max / sum need one exchange with lane l^32 and the
// rescale of O is lane-local.  The S^T accumulator of a lane lists keys in the
// order (0-3, 8-11 | 4-7, 12-15) of every 16, which is exactly the k-slice
// order of the P operand once bits 2 and 3 of the key offset are swapped in
// the transposed tiles - so P goes from accumulator to operand in registers.
//
// Linear branch: H_u = H - G and z_u = z - g, where G and g are the sums over
// the row's listed blocks, so O_l = phi(Q) H_u / phi(Q) z_u; phi(Q) H_u is a
// hi + lo split product (three bf16 MFMAs), again ~16 mantissa bits.
#include "sla_internal.h"

namespace sla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void gbl_void;

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8), each
// XCD with its own L2.  Map them so that every XCD walks a contiguous range of
// mask rows: adjacent query blocks of a head select largely the same key
// blocks, so their K / V^T tiles are then shared in one L2.
__device__ __forceinline__ long long xcd_row(long long b, long long R) {
  constexpr long long NX = 8;
  const long long q = R / NX, r = R % NX;
  const long long x = b % NX, local = b / NX;
  return x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

// Position of key offset o inside its 16-key group in the transposed tiles.
__device__ __forceinline__ int kperm(int o) { return (o & ~12) | ((o & 4) << 1) | ((o & 8) >> 1); }

__device__ __forceinline__ uint32_t elem(const uint4& v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// 16-byte direct load global -> LDS; lane l of the wavefront writes
// lds_wave_base + 16 * l.
__device__ __forceinline__ void g2lds16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void*)gsrc, (lds_void*)lds_wave_base, 16, 0, 0);
}

// ------------------------------------------------------------------ prep
template <int D, int BK>
struct PrepCfg {
  static constexpr int NT = 256;
  static constexpr int VST = BK + 8;                    // padded LDS row stride (elements)
  static constexpr int PAIRS = (BK / 4) * (D / 8);      // (4-key group, 8-d chunk) pairs
  static constexpr int ST = (PAIRS + NT - 1) / NT;
  static constexpr int TILE = D * VST * 2;              // bytes of one transposed tile
  static constexpr int TT = (D / 32) * (D / 32);
  static constexpr int TPW = (TT + 3) / 4;              // G tiles per wavefront
};

// LIN = false: only V^T is written (sparse / dense callers).
template <int D, int BK, bool LIN>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ K,
                                                   const uint16_t* __restrict__ V,
                                                   const float* __restrict__ alpha, int H, int N,
                                                   int Nk, int chunk_blocks, int nchunk,
                                                   uint16_t* __restrict__ vt_g, uint16_t* __restrict__ pk_g,
                                                   float* __restrict__ zblk, float* __restrict__ hpart) {
  using C = PrepCfg<D, BK>;
  __shared__ __attribute__((aligned(16))) char smem[3 * C::TILE + (BK / 4) * D * 4];
  uint16_t* Vt = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Pk = reinterpret_cast<uint16_t*>(smem + C::TILE);
  uint16_t* PkLo = reinterpret_cast<uint16_t*>(smem + 2 * C::TILE);
  float* zred = reinterpret_cast<float*>(smem + 3 * C::TILE);  // [BK/4][D]

  const long long bh = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  const bool lin = LIN && !(alpha != nullptr && alpha[bh % H] == 1.f);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t npad = (size_t)Nk * BK;
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  const int jb = chunk * chunk_blocks, je = min(Nk, jb + chunk_blocks);

  f32x16 acc_g[C::TPW];
#pragma unroll
  for (int t = 0; t < C::TPW; ++t) acc_g[t] = f32x16{};
  float zpart = 0.f;

  // Block j's K/V chunks are fetched into registers while block j-1 is being
  // transposed, copied out and multiplied (two register buffers).
  auto fetch = [&](int j, uint4 (&kr_)[C::ST][4], uint4 (&vr_)[C::ST][4]) __attribute__((always_inline)) {
    const int key0 = j * BK;
#pragma unroll
    for (int s = 0; s < C::ST; ++s) {
      const int pi = tid + C::NT * s;
      const int c = pi % (D / 8), g = pi / (D / 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int key = key0 + 4 * g + u;
        const bool ok = pi < C::PAIRS && key < N;
        const size_t off = (size_t)key * D + c * 8;
        vr_[s][u] = ok ? *reinterpret_cast<const uint4*>(Vb + off) : make_uint4(0, 0, 0, 0);
        kr_[s][u] = (ok && lin) ? *reinterpret_cast<const uint4*>(Kb + off) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto process = [&](int j, const uint4 (&kr)[C::ST][4], const uint4 (&vr)[C::ST][4]) __attribute__((always_inline)) {
    const int key0 = j * BK;
    __syncthreads();  // previous block's tiles fully consumed
#pragma unroll
    for (int s = 0; s < C::ST; ++s) {
      const int pi = tid + C::NT * s;
      if (pi >= C::PAIRS) continue;
      const int c = pi % (D / 8), g = pi / (D / 8);
      const int pos = ((4 * g) & ~15) + kperm((4 * g) & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 wv;
        wv.x = elem(vr[s][0], e) | (elem(vr[s][1], e) << 16);
        wv.y = elem(vr[s][2], e) | (elem(vr[s][3], e) << 16);
        *reinterpret_cast<uint2*>(Vt + (c * 8 + e) * C::VST + pos) = wv;
      }
      if (lin) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float f[4], lo[4];
          uint32_t hb[4];
          float zs = 0.f;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const bool ok = key0 + 4 * g + u < N;
            f[u] = ok ? phi(bf2f(elem(kr[s][u], e))) : 0.f;
            zs += f[u];
            hb[u] = pk_bf16(f[u], 0.f) & 0xffffu;
            lo[u] = f[u] - bf2f(hb[u]);
          }
          zred[g * D + c * 8 + e] = zs;
          uint2 wv;
          wv.x = hb[0] | (hb[1] << 16);
          wv.y = hb[2] | (hb[3] << 16);
          *reinterpret_cast<uint2*>(Pk + (c * 8 + e) * C::VST + pos) = wv;
          wv.x = pk_bf16(lo[0], lo[1]);
          wv.y = pk_bf16(lo[2], lo[3]);
          *reinterpret_cast<uint2*>(PkLo + (c * 8 + e) * C::VST + pos) = wv;
        }
      }
    }
    __syncthreads();
    // copy the transposed tiles out: row d has BK keys = BK/8 chunks of 16 B
    for (int e = tid; e < D * (BK / 8); e += C::NT) {
      const int d = e / (BK / 8), ch = e % (BK / 8);
      const size_t go = ((size_t)bh * D + d) * npad + key0 + ch * 8;
      *reinterpret_cast<uint4*>(vt_g + go) = *reinterpret_cast<const uint4*>(Vt + d * C::VST + ch * 8);
      if (lin) *reinterpret_cast<uint4*>(pk_g + go) = *reinterpret_cast<const uint4*>(Pk + d * C::VST + ch * 8);
    }
    if (lin) {
      if (tid < D) {
        float z = 0.f;
#pragma unroll
        for (int g = 0; g < BK / 4; ++g) z += zred[g * D + tid];
        zblk[((size_t)bh * Nk + j) * D + tid] = z;
        zpart += z;
      }
      // G += phi(K)^T V (hi and lo parts of phi)
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
  };
  uint4 ka[C::ST][4], va[C::ST][4], kb2[C::ST][4], vb2[C::ST][4];
  if (jb < je) fetch(jb, ka, va);
  for (int j = jb; j < je; j += 2) {
    if (j + 1 < je) fetch(j + 1, kb2, vb2);
    process(j, ka, va);
    if (j + 1 < je) {
      if (j + 2 < je) fetch(j + 2, ka, va);
      process(j + 1, kb2, vb2);
    }
  }
  if (!lin) return;
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
  if (tid < D) out[D * D + tid] = zpart;
}

// ------------------------------------------------------------------ attention
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// LDS tiles are stored as "planes": every 16-element k-slice that an MFMA
// operand read takes is a plane of 32 bytes per row (two 16-byte halves), and
// row r keeps its halves swapped when bit 3 of r is set.  The 16 rows that a
// 16-lane group reads then sit in 16 distinct 16-byte bank groups, and every
// operand read is one per-lane base address plus a compile-time offset.
template <int D, int BK>
struct Tiles {
  static constexpr int KPB = BK * 32;        // bytes of one K plane (16 d of BK keys)
  static constexpr int VPB = D * 32;         // bytes of one V^T / phi(K)^T plane (16 keys)
  static constexpr int KT_BYTES = BK * D * 2;
  static constexpr int VT_BYTES = D * BK * 2;
  static constexpr int HPB = D * 32;         // bytes of one H_u^T plane (16 d_k)
};

__device__ __forceinline__ int lane_base(int lane) {
  const int l32 = lane & 31, hi = lane >> 5;
  return l32 * 32 + 16 * (hi ^ ((l32 >> 3) & 1));
}

__device__ __forceinline__ uint4 rd16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// Direct loads of key block j into the LDS stage at sb by wavefront w of NWL.
// Load slot u fills the 1 KB at sb + 1024 u: 32 rows x 32 bytes of one plane;
// lane l brings row l/2, stored half l%2.  K rows past N are clamped (their
// scores are masked); V^T / phi(K)^T are zero past N.
template <int D, int BK, int NWL>
__device__ __forceinline__ void load_tiles(const uint16_t* Kb, const uint16_t* Vtb, const uint16_t* Pkb,
                                           int j, int N, size_t npad, bool doK, bool doP, char* sb,
                                           int w, int lane) {
  using T = Tiles<D, BK>;
  const int lrow = lane >> 1, lpos = lane & 1;
  if (doK) {
#pragma unroll
    for (int ii = 0; ii < T::KT_BYTES / 1024 / NWL; ++ii) {
      const int u = w + NWL * ii;
      const int t = u / (T::KPB / 1024), r = (u % (T::KPB / 1024)) * 32 + lrow;
      const int hh = lpos ^ ((r >> 3) & 1);
      const int key = min(j * BK + r, N - 1);
      g2lds16(Kb + (size_t)key * D + 16 * t + 8 * hh, sb + 1024 * u);
    }
  }
#pragma unroll
  for (int ii = 0; ii < T::VT_BYTES / 1024 / NWL; ++ii) {
    const int u = w + NWL * ii;
    const int pl = u / (T::VPB / 1024), r = (u % (T::VPB / 1024)) * 32 + lrow;
    const int hh = lpos ^ ((r >> 3) & 1);
    const size_t go = (size_t)r * npad + (size_t)j * BK + 16 * pl + 8 * hh;
    g2lds16(Vtb + go, sb + T::KT_BYTES + 1024 * u);
    if (doP) g2lds16(Pkb + go, sb + T::KT_BYTES + T::VT_BYTES + 1024 * u);
  }
}

// max of v over lanes l and l^32 (v_permlane32_swap exchanges the two halves;
// taking the max with the own value makes the result independent of which
// output holds which half)
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(v, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Online-softmax attention of one wavefront's 32 queries over one key block,
// 32 keys at a time: S^T = K Q^T, running max / sum, O^T += V^T P^T.
template <int D, int BK, bool MASK>
__device__ __forceinline__ void attend_block(const char* Ks, const char* Vt, const bf16x8 (&qf)[D / 16],
                                             f32x16 (&acc_o)[D / 32], float& m_run, float& l_run,
                                             int lb, int hi, int key0, int N, float scale_log2) {
  using T = Tiles<D, BK>;
#pragma unroll
  for (int kt = 0; kt < BK / 32; ++kt) {
    f32x16 sa = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 16; ++t) sa = mfma(as_bf16x8(rd16(Ks + t * T::KPB + kt * 1024 + lb)), qf[t], sa);
    if (MASK) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 32 * kt + 8 * (i >> 2) + 4 * hi + (i & 3);
        if (key >= N) sa[i] = -INFINITY;
      }
    }
    float mx = sa[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sa[i]);
    mx = pair_max(mx);
    // Conditional rescale: the running max moves only when some lane's max
    // exceeds it by more than 2^8 in exp2 units, so P <= 2^8 and the O / l
    // rescale is skipped for most tiles.
    if (__ballot((mx - m_run) * scale_log2 > 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      l_run *= corr;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) acc_o[t] *= corr;
      m_run = m_new;
    }
    const float mneg = -m_run * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sa[i] = __builtin_amdgcn_exp2f(fmaf(sa[i], scale_log2, mneg));
      psum += sa[i];
    }
    l_run += psum;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 pb;
      pb.x = pk_bf16(sa[8 * s + 0], sa[8 * s + 1]);
      pb.y = pk_bf16(sa[8 * s + 2], sa[8 * s + 3]);
      pb.z = pk_bf16(sa[8 * s + 4], sa[8 * s + 5]);
      pb.w = pk_bf16(sa[8 * s + 6], sa[8 * s + 7]);
      const bf16x8 bp = as_bf16x8(pb);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        acc_o[dt] = mfma(as_bf16x8(rd16(Vt + (2 * kt + s) * T::VPB + dt * 1024 + lb)), bp, acc_o[dt]);
    }
  }
}

// Q fragments of 32 query rows (B operand of S^T = K Q^T), zero past N.
template <int D>
__device__ __forceinline__ void load_q(const uint16_t* Q, long long bh, int q, int N, int hi,
                                       bf16x8 (&qf)[D / 16]) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (q < N) v = *reinterpret_cast<const uint4*>(Q + ((size_t)bh * N + q) * D + 16 * t + 8 * hi);
    qf[t] = as_bf16x8(v);
  }
}

// Sparse (CSR row) or dense (every key block) softmax attention; BQ/32
// wavefronts of 32 queries, tiles double-buffered.
template <int D, int BQ, int BK, int MODE>
__global__ __launch_bounds__(BQ / 32 * 64, 2) void attn_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ vt_g,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, uint16_t* __restrict__ O, int N,
    int Nq, int Nk, float scale_log2) {
  using T = Tiles<D, BK>;
  constexpr int NW = BQ / 32;
  constexpr int STAGE = T::KT_BYTES + T::VT_BYTES;
  static_assert(T::KT_BYTES % (1024 * NW) == 0 && T::VT_BYTES % (1024 * NW) == 0, "tile split");
  // Two distinct LDS arrays: the compiler can then tell the prefetch into one
  // stage from the operand reads of the other.
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int lb = lane_base(lane);
  const long long row = xcd_row(blockIdx.x, (long long)gridDim.x);
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  const size_t npad = (size_t)Nk * BK;
  int nsel, base = 0;
  if (MODE == MODE_DENSE) {
    nsel = Nk;
  } else {
    base = row_ptr[row];
    nsel = row_ptr[row + 1] - base;
  }
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vtb = vt_g + (size_t)bh * D * npad;
  const int q = qi * BQ + 32 * w + l32;
  bf16x8 qf[D / 16];
  load_q<D>(Q, bh, q, N, hi, qf);
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto blk = [&](int b) { return (MODE == MODE_DENSE) ? b : col_idx[base + b]; };
  auto step = [&](int b, char* cur, char* nxt) __attribute__((always_inline)) {
    const int j = blk(b);
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's loads of block b have landed
    __syncthreads();                // ... and every wavefront's; block b-1 consumed
    if (b + 1 < nsel) load_tiles<D, BK, NW>(Kb, Vtb, nullptr, blk(b + 1), N, npad, true, false, nxt, w, lane);
    if ((j + 1) * BK > N)
      attend_block<D, BK, true>(cur, cur + T::KT_BYTES, qf, acc_o, m_run, l_run, lb, hi, j * BK, N, scale_log2);
    else
      attend_block<D, BK, false>(cur, cur + T::KT_BYTES, qf, acc_o, m_run, l_run, lb, hi, j * BK, N, scale_log2);
  };
  if (nsel > 0) load_tiles<D, BK, NW>(Kb, Vtb, nullptr, blk(0), N, npad, true, false, st0, w, lane);
  for (int b = 0; b < nsel; b += 2) {
    step(b, st0, st1);
    if (b + 1 < nsel) step(b + 1, st1, st0);
  }

  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv_l = lt > 0.f ? 1.f / lt : 0.f;
  if (q < N) {
    const size_t orow = ((size_t)bh * N + q) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        uint2 wv;
        wv.x = pk_bf16(acc_o[mt][4 * i4 + 0] * inv_l, acc_o[mt][4 * i4 + 1] * inv_l);
        wv.y = pk_bf16(acc_o[mt][4 * i4 + 2] * inv_l, acc_o[mt][4 * i4 + 3] * inv_l);
        *reinterpret_cast<uint2*>(O + orow + 32 * mt + 8 * i4 + 4 * hi) = wv;
      }
  }
}

// Fused sparse + linear (+ alpha mix) over the CSR row.  2*BQ/32 wavefronts:
// wavefronts [0, NA) run the softmax attention of 32 queries each, wavefronts
// [NA, 2 NA) accumulate G = sum phi(K_j)^T V_j over the row's blocks - one of
// each per SIMD, so G's matrix ops overlap the softmax's vector work.  After
// the loop the G wavefronts store H_u = H - G (hi + lo bf16) in LDS and the
// attention wavefronts apply it to phi(Q) and mix the branches.
template <int D, int BQ, int BK, int MODE>
__global__ __launch_bounds__(BQ / 32 * 128, 1) void fused_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ vt_g,
    const uint16_t* __restrict__ pk_g, const float* __restrict__ zblk, const int* __restrict__ row_ptr,
    const int* __restrict__ col_idx, const float* __restrict__ alpha, const float* __restrict__ htot,
    uint16_t* __restrict__ O, int H, int N, int Nq, int Nk, float scale_log2) {
  using T = Tiles<D, BK>;
  constexpr int NA = BQ / 32;                    // attention wavefronts
  constexpr int NWT = 2 * NA;                    // all wavefronts
  constexpr int STAGE = T::KT_BYTES + 2 * T::VT_BYTES;
  constexpr int HU = 2 * D * D * 2;
  constexpr int S0 = STAGE > HU ? STAGE : HU;
  constexpr bool TWO = S0 + STAGE + D * 4 <= 160 * 1024;   // double-buffer when LDS allows
  constexpr int TT = (D / 32) * (D / 32);
  constexpr int TPW = (TT + NA - 1) / NA;       // G tiles per G wavefront
  static_assert(T::KT_BYTES % (1024 * NWT) == 0 && T::VT_BYTES % (1024 * NWT) == 0, "tile split");
  __shared__ __attribute__((aligned(16))) char st0[S0];
  __shared__ __attribute__((aligned(16))) char st1[TWO ? STAGE : 16];
  __shared__ float zu[D];
  char* HuHi = st0;
  char* HuLo = st0 + D * D * 2;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool attn_wave = w < NA;
  const int wr = attn_wave ? w : w - NA;        // index within the role
  const int lb = lane_base(lane);
  const long long row = xcd_row(blockIdx.x, (long long)gridDim.x);
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  const int h = (int)(bh % H);
  const size_t npad = (size_t)Nk * BK;
  const int base = row_ptr[row];
  const int nsel = row_ptr[row + 1] - base;
  float ws_, wl_;
  if (MODE == MODE_FUSED) {
    ws_ = alpha[h];
    wl_ = 1.f - ws_;
  } else {
    ws_ = 0.f;
    wl_ = 1.f;
  }
  const bool do_s = ws_ != 0.f;
  const bool lin = (wl_ != 0.f) && (nsel < Nk);
  const int nblk = (do_s || lin) ? nsel : 0;

  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vtb = vt_g + (size_t)bh * D * npad;
  const uint16_t* Pkb = pk_g + (size_t)bh * D * npad;
  const float* Hh = htot + (size_t)bh * (D * D + D);

  // The block loop; both roles run it with the same loads and barriers, each
  // with its own per-block work, so neither role keeps the other's state live.
  auto run_loop = [&](auto&& work) __attribute__((always_inline)) {
    auto step = [&](int b, char* cur, char* nxt) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (TWO && b + 1 < nblk)
        load_tiles<D, BK, NWT>(Kb, Vtb, Pkb, col_idx[base + b + 1], N, npad, do_s, lin, nxt, w, lane);
      work(col_idx[base + b], cur);
      if (!TWO) {
        __syncthreads();  // the single stage is consumed before it is refilled
        if (b + 1 < nblk)
          load_tiles<D, BK, NWT>(Kb, Vtb, Pkb, col_idx[base + b + 1], N, npad, do_s, lin, cur, w, lane);
      }
    };
    if (nblk > 0) load_tiles<D, BK, NWT>(Kb, Vtb, Pkb, col_idx[base], N, npad, do_s, lin, st0, w, lane);
    if (TWO) {
      for (int b = 0; b < nblk; b += 2) {
        step(b, st0, st1);
        if (b + 1 < nblk) step(b + 1, st1, st0);
      }
    } else {
      for (int b = 0; b < nblk; ++b) step(b, st0, st0);
    }
    __syncthreads();  // every wavefront is done with the loop tiles
  };

  if (!attn_wave) {
    // ---- G wavefronts: G = sum over listed blocks of phi(K_j)^T V_j
    f32x16 acc_g[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc_g[t] = f32x16{};
    run_loop([&](int, const char* cur) __attribute__((always_inline)) {
      if (!lin) return;
      const char* Vt = cur + T::KT_BYTES;
      const char* Pk = cur + T::KT_BYTES + T::VT_BYTES;
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
          const int tix = wr * TPW + u;
          if (tix >= TT) continue;
          const int mt = tix / (D / 32), nt = tix % (D / 32);
          acc_g[u] = mfma(as_bf16x8(rd16(Pk + s * T::VPB + mt * 1024 + lb)),
                          as_bf16x8(rd16(Vt + s * T::VPB + nt * 1024 + lb)), acc_g[u]);
        }
      }
    });
    if (lin) {
      // H_u^T = (H - G)^T as hi + lo bf16 planes (rows d_v, 16-wide d_k slices)
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tix = wr * TPW + u;
        if (tix >= TT) continue;
        const int mt = tix / (D / 32), nt = tix % (D / 32);
        const int dv = 32 * nt + l32;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int dk = 32 * mt + 8 * i4 + 4 * hi;
          float hv[4], lv[4];
          uint32_t hb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            hv[r] = Hh[(dk + r) * D + dv] - acc_g[u][4 * i4 + r];
            hb[r] = pk_bf16(hv[r], 0.f) & 0xffffu;
            lv[r] = hv[r] - bf2f(hb[r]);
          }
          const int off = (dk >> 4) * T::HPB + dv * 32 + 16 * (((dk >> 3) & 1) ^ ((dv >> 3) & 1)) + 8 * hi;
          uint2 wv;
          wv.x = hb[0] | (hb[1] << 16);
          wv.y = hb[2] | (hb[3] << 16);
          *reinterpret_cast<uint2*>(HuHi + off) = wv;
          wv.x = pk_bf16(lv[0], lv[1]);
          wv.y = pk_bf16(lv[2], lv[3]);
          *reinterpret_cast<uint2*>(HuLo + off) = wv;
        }
      }
      __syncthreads();  // H_u^T and z_u complete
    }
    return;
  }

  // ---- attention wavefronts
  const int q = qi * BQ + 32 * wr + l32;
  bf16x8 qf[D / 16];
  load_q<D>(Q, bh, q, N, hi, qf);
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  run_loop([&](int j, const char* cur) __attribute__((always_inline)) {
    if (!do_s) return;
    if ((j + 1) * BK > N)
      attend_block<D, BK, true>(cur, cur + T::KT_BYTES, qf, acc_o, m_run, l_run, lb, hi, j * BK, N,
                                scale_log2);
    else
      attend_block<D, BK, false>(cur, cur + T::KT_BYTES, qf, acc_o, m_run, l_run, lb, hi, j * BK, N,
                                 scale_log2);
  });
  if (lin) {
    if (tid < D) {
      float g = 0.f;
      for (int b = 0; b < nsel; ++b) g += zblk[((size_t)bh * Nk + col_idx[base + b]) * D + tid];
      zu[tid] = Hh[D * D + tid] - g;
    }
    __syncthreads();  // H_u^T and z_u complete
  }

  float inv_l = 0.f;
  if (do_s) {
    const float lt = l_run + __shfl_xor(l_run, 32);
    inv_l = lt > 0.f ? 1.f / lt : 0.f;
  }
  f32x16 acc_n[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) acc_n[mt] = f32x16{};
  float den = 1.f;
  if (lin) {
    // num^T = H_u^T phi(Q)^T with phi(Q) split into hi + lo once per k-step
    float dpart = 0.f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const uint4 qv = __builtin_bit_cast(uint4, qf[t]);
      float f[8], fl[8];
      uint32_t fh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f[e] = phi(bf2f(elem(qv, e)));
        fh[e] = pk_bf16(f[e], 0.f) & 0xffffu;
        fl[e] = f[e] - bf2f(fh[e]);
        dpart = fmaf(f[e], zu[16 * t + 8 * hi + e], dpart);
      }
      const bf16x8 bh4 = as_bf16x8(make_uint4(fh[0] | (fh[1] << 16), fh[2] | (fh[3] << 16),
                                              fh[4] | (fh[5] << 16), fh[6] | (fh[7] << 16)));
      const bf16x8 bl4 = as_bf16x8(make_uint4(pk_bf16(fl[0], fl[1]), pk_bf16(fl[2], fl[3]),
                                              pk_bf16(fl[4], fl[5]), pk_bf16(fl[6], fl[7])));
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
        const uint4 ah = rd16(HuHi + t * T::HPB + mt * 1024 + lb);
        const uint4 al = rd16(HuLo + t * T::HPB + mt * 1024 + lb);
        acc_n[mt] = mfma(as_bf16x8(ah), bh4, acc_n[mt]);
        acc_n[mt] = mfma(as_bf16x8(ah), bl4, acc_n[mt]);
        acc_n[mt] = mfma(as_bf16x8(al), bh4, acc_n[mt]);
      }
    }
    den = dpart + __shfl_xor(dpart, 32);
  }
  const float wl_den = lin ? wl_ / den : 0.f;
  const float ws_l = ws_ * inv_l;
  if (q < N) {
    const size_t orow = ((size_t)bh * N + q) * D;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = ws_l * acc_o[mt][4 * i4 + r] + wl_den * acc_n[mt][4 * i4 + r];
        uint2 wv;
        wv.x = pk_bf16(o[0], o[1]);
        wv.y = pk_bf16(o[2], o[3]);
        *reinterpret_cast<uint2*>(O + orow + 32 * mt + 8 * i4 + 4 * hi) = wv;
      }
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

hipError_t launch_summary_reduce(const float* hpart, const float* alpha, int H, long long BH,
                                 int nchunk, int per, float* htot, hipStream_t st) {
  hipLaunchKernelGGL(summary_reduce_kernel, dim3((unsigned)((per + 255) / 256), (unsigned)BH), dim3(256),
                     0, st, hpart, alpha, H, nchunk, per, htot);
  return hipGetLastError();
}

namespace {

template <int D, int BK>
hipError_t prep_dispatch(const Shape& s, bool lin, const void* K, const void* V, const float* alpha,
                         char* ws, const WsLayout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H;
  const dim3 grid((unsigned)(BH * L.nchunk)), block(256);
  uint16_t* vt = reinterpret_cast<uint16_t*>(ws + L.vt);
  uint16_t* pk = reinterpret_cast<uint16_t*>(ws + L.pk);
  float* zb = reinterpret_cast<float*>(ws + L.zblk);
  float* hpart = reinterpret_cast<float*>(ws + L.hpart);
  const uint16_t* k = static_cast<const uint16_t*>(K);
  const uint16_t* v = static_cast<const uint16_t*>(V);
  if (lin)
    hipLaunchKernelGGL((prep_kernel<D, BK, true>), grid, block, 0, st, k, v, alpha, s.H, s.N, s.Nk,
                       L.chunk_blocks, L.nchunk, vt, pk, zb, hpart);
  else
    hipLaunchKernelGGL((prep_kernel<D, BK, false>), grid, block, 0, st, k, v, alpha, s.H, s.N, s.Nk,
                       L.chunk_blocks, L.nchunk, vt, pk, zb, hpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !lin) return e;
  return launch_summary_reduce(hpart, alpha, s.H, BH, L.nchunk, D * D + D,
                               reinterpret_cast<float*>(ws + L.htot), st);
}

template <int D, int BQ, int BK>
hipError_t attn_dispatch(const Shape& s, Mode mode, const void* Q, const void* K, const int32_t* rp,
                         const int32_t* ci, const float* alpha, const char* ws, const WsLayout& L,
                         void* O, hipStream_t st) {
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(K);
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(ws + L.vt);
  const uint16_t* pk = reinterpret_cast<const uint16_t*>(ws + L.pk);
  const float* zb = reinterpret_cast<const float*>(ws + L.zblk);
  const float* ht = reinterpret_cast<const float*>(ws + L.htot);
  uint16_t* o = static_cast<uint16_t*>(O);
  const dim3 grid((unsigned)s.R());
  switch (mode) {
    case MODE_SPARSE:
      hipLaunchKernelGGL((attn_kernel<D, BQ, BK, MODE_SPARSE>), grid, dim3(BQ / 32 * 64), 0, st, q, k, vt,
                         rp, ci, o, s.N, s.Nq, s.Nk, sl2);
      break;
    case MODE_DENSE:
      hipLaunchKernelGGL((attn_kernel<D, BQ, BK, MODE_DENSE>), grid, dim3(BQ / 32 * 64), 0, st, q, k, vt,
                         rp, ci, o, s.N, s.Nq, s.Nk, sl2);
      break;
    case MODE_LINEAR:
      hipLaunchKernelGGL((fused_kernel<D, BQ, BK, MODE_LINEAR>), grid, dim3(BQ / 32 * 128), 0, st, q, k,
                         vt, pk, zb, rp, ci, alpha, ht, o, s.H, s.N, s.Nq, s.Nk, sl2);
      break;
    default:
      hipLaunchKernelGGL((fused_kernel<D, BQ, BK, MODE_FUSED>), grid, dim3(BQ / 32 * 128), 0, st, q, k,
                         vt, pk, zb, rp, ci, alpha, ht, o, s.H, s.N, s.Nq, s.Nk, sl2);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_bf16(const Shape& s, bool lin, const void* K, const void* V, const float* alpha,
                            char* ws, const WsLayout& L, hipStream_t st) {
  if (s.d == 128 && s.bk == 64) return prep_dispatch<128, 64>(s, lin, K, V, alpha, ws, L, st);
  if (s.d == 128 && s.bk == 128) return prep_dispatch<128, 128>(s, lin, K, V, alpha, ws, L, st);
  if (s.d == 64 && s.bk == 64) return prep_dispatch<64, 64>(s, lin, K, V, alpha, ws, L, st);
  if (s.d == 64 && s.bk == 128) return prep_dispatch<64, 128>(s, lin, K, V, alpha, ws, L, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bf16(const Shape& s, Mode mode, const void* Q, const void* K,
                            const int32_t* rp, const int32_t* ci, const float* alpha, const char* ws,
                            const WsLayout& L, void* O, hipStream_t st) {
#define SLA_ATTN(DD, QQ, KK)                                                  \
  if (s.d == DD && s.bq == QQ && s.bk == KK)                                  \
    return attn_dispatch<DD, QQ, KK>(s, mode, Q, K, rp, ci, alpha, ws, L, O, st);
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

}  // namespace sla
