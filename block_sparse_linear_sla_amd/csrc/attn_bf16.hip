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
template <int D, int BQ, int BK, int MODE>
struct Cfg {
  static constexpr int NW = BQ / 32;                 // wavefronts
  static constexpr int NT = NW * 64;                 // threads
  static constexpr bool LINM = MODE == MODE_FUSED || MODE == MODE_LINEAR;
  static constexpr int NSTAGE = LINM ? 1 : 2;        // LDS buffers of the loop tiles
  static constexpr int CHK = D / 8;                  // 16-byte chunks per K-tile row
  static constexpr int CHV = BK / 8;                 // 16-byte chunks per transposed-tile row
  static constexpr int KT_BYTES = BK * D * 2;
  static constexpr int VT_BYTES = D * BK * 2;
  static constexpr int STAGE_BYTES = KT_BYTES + VT_BYTES + (LINM ? VT_BYTES : 0);
  static constexpr int LOOP_BYTES = STAGE_BYTES;       // stage 0; stage 1 has its own array
  static constexpr int HU_BYTES = LINM ? 2 * D * D * 2 : 0;
  static constexpr int MAIN_BYTES = LOOP_BYTES > HU_BYTES ? LOOP_BYTES : HU_BYTES;
  static constexpr int ZU_OFF = MAIN_BYTES;
  static constexpr int SMEM = ZU_OFF + (LINM ? D * 4 : 0);
  static constexpr int TT = (D / 32) * (D / 32);     // 32x32 tiles of G
  static constexpr int TPW = (TT + NW - 1) / NW;     // G tiles per wavefront
  // direct-load instructions per wavefront per tile (64 chunks of 16 B each)
  static constexpr int KLOADS = (BK * CHK) / (64 * NW);
  static constexpr int VLOADS = (D * CHV) / (64 * NW);
};

template <int D, int BQ, int BK, int MODE>
__global__ __launch_bounds__(BQ / 32 * 64, 2) void attn_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ vt_g,
    const uint16_t* __restrict__ pk_g, const float* __restrict__ zblk, const int* __restrict__ row_ptr,
    const int* __restrict__ col_idx, const float* __restrict__ alpha, const float* __restrict__ htot,
    uint16_t* __restrict__ O, int H, int N, int Nq, int Nk, float scale_log2) {
  using C = Cfg<D, BQ, BK, MODE>;
  static_assert(C::KLOADS >= 1 && C::VLOADS >= 1, "tile too small for the workgroup");
  static_assert(C::KLOADS * 64 * C::NW == BK * C::CHK && C::VLOADS * 64 * C::NW == D * C::CHV,
                "tiles must split evenly over the wavefronts");
  // Stage 0 (and the epilogue buffers) and stage 1 are distinct LDS arrays so
  // that the compiler can tell the prefetch into one from reads of the other.
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  __shared__ __attribute__((aligned(16))) char smem1[C::NSTAGE == 2 ? C::STAGE_BYTES : 16];
  uint16_t* HuHi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* HuLo = reinterpret_cast<uint16_t*>(smem + D * D * 2);
  float* zu = reinterpret_cast<float*>(smem + C::ZU_OFF);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const long long row = blockIdx.x;
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  const int h = (int)(bh % H);
  const size_t npad = (size_t)Nk * BK;

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
  const bool lin = C::LINM && (wl_ != 0.f) && (nsel < Nk);
  const int nblk = (do_s || lin) ? nsel : 0;

  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vtb = vt_g + (size_t)bh * D * npad;
  const uint16_t* Pkb = C::LINM ? pk_g + (size_t)bh * D * npad : nullptr;

  // Issue the direct loads of key block j into the LDS stage at sb.
  auto load_block = [&](int j, char* sb) {
    if (do_s) {
#pragma unroll
      for (int ii = 0; ii < C::KLOADS; ++ii) {
        const int u = w + C::NW * ii;               // 1 KB slot of the tile
        const int g = 64 * u + lane;                // 16-byte chunk slot
        const int r = g / C::CHK, pc = g % C::CHK;
        const int lc = pc ^ (r % C::CHK);
        const int key = min(j * BK + r, N - 1);     // rows past N are masked later
        g2lds16(Kb + (size_t)key * D + 8 * lc, sb + 1024 * u);
      }
    }
#pragma unroll
    for (int ii = 0; ii < C::VLOADS; ++ii) {
      const int u = w + C::NW * ii;
      const int g = 64 * u + lane;
      const int r = g / C::CHV, pc = g % C::CHV;
      const int lc = pc ^ (r % C::CHV);
      const size_t go = (size_t)r * npad + (size_t)j * BK + 8 * lc;
      g2lds16(Vtb + go, sb + C::KT_BYTES + 1024 * u);
      if (C::LINM && lin) g2lds16(Pkb + go, sb + C::KT_BYTES + C::VT_BYTES + 1024 * u);
    }
  };

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
  f32x16 acc_g[C::LINM ? C::TPW : 1];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = f32x16{};
#pragma unroll
  for (int t = 0; t < (C::LINM ? C::TPW : 1); ++t) acc_g[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // One key block: wait for its tiles in `cur`, prefetch the next block into
  // `nxt` (double-buffered modes), compute.
  auto block_step = [&](int b, char* cur, char* nxt) __attribute__((always_inline)) {
    const int j = (MODE == MODE_DENSE) ? b : col_idx[base + b];
    __builtin_amdgcn_s_waitcnt(0);  // this wavefront's loads of block b have landed
    __syncthreads();                // ... and every other wavefront's; block b-1 consumed
    if (C::NSTAGE == 2 && b + 1 < nblk) load_block((MODE == MODE_DENSE) ? b + 1 : col_idx[base + b + 1], nxt);
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(cur);
    const uint16_t* Vt = reinterpret_cast<const uint16_t*>(cur + C::KT_BYTES);
    const uint16_t* Pk = reinterpret_cast<const uint16_t*>(cur + C::KT_BYTES + C::VT_BYTES);
    const int key0 = j * BK;
    if (do_s) {
      // S^T = K Q^T for BK/32 key tiles
      f32x16 sacc[BK / 32];
#pragma unroll
      for (int kt = 0; kt < BK / 32; ++kt) {
        f32x16 a = f32x16{};
        const int r = 32 * kt + l32;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const int pc = (2 * t + hi) ^ (r % C::CHK);
          const uint4 kv = *reinterpret_cast<const uint4*>(Ks + r * D + 8 * pc);
          a = mfma(as_bf16x8(kv), qf[t], a);
        }
        sacc[kt] = a;
      }
      if (key0 + BK > N) {
#pragma unroll
        for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kt + 8 * (i >> 2) + 4 * hi + (i & 3);
            if (key >= N) sacc[kt][i] = -INFINITY;
          }
      }
      // G += phi(K)^T V over this block; independent of the softmax below, so
      // the scheduler can overlap these matrix ops with its vector work
      if (C::LINM && lin) {
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
          const int lc = 2 * s + hi;
#pragma unroll
          for (int u = 0; u < C::TPW; ++u) {
            const int tix = w * C::TPW + u;
            if (tix >= C::TT) continue;
            const int mt = tix / (D / 32), nt = tix % (D / 32);
            const int ra = 32 * mt + l32, rb = 32 * nt + l32;
            const uint4 av = *reinterpret_cast<const uint4*>(Pk + ra * BK + 8 * (lc ^ (ra % C::CHV)));
            const uint4 bv = *reinterpret_cast<const uint4*>(Vt + rb * BK + 8 * (lc ^ (rb % C::CHV)));
            acc_g[u] = mfma(as_bf16x8(av), as_bf16x8(bv), acc_g[u]);
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float corr = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      const float mneg = -m_new * scale_log2;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < BK / 32; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kt][i], scale_log2, mneg));
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
          pb.x = pk_bf16(sacc[kt][8 * s + 0], sacc[kt][8 * s + 1]);
          pb.y = pk_bf16(sacc[kt][8 * s + 2], sacc[kt][8 * s + 3]);
          pb.z = pk_bf16(sacc[kt][8 * s + 4], sacc[kt][8 * s + 5]);
          pb.w = pk_bf16(sacc[kt][8 * s + 6], sacc[kt][8 * s + 7]);
          const bf16x8 bp = as_bf16x8(pb);
          const int lc = 4 * kt + 2 * s + hi;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const int r = 32 * dt + l32;
            const uint4 vv = *reinterpret_cast<const uint4*>(Vt + r * BK + 8 * (lc ^ (r % C::CHV)));
            acc_o[dt] = mfma(as_bf16x8(vv), bp, acc_o[dt]);
          }
        }
    }
    if (C::LINM && lin && !do_s) {
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const int lc = 2 * s + hi;
#pragma unroll
        for (int u = 0; u < C::TPW; ++u) {
          const int tix = w * C::TPW + u;
          if (tix >= C::TT) continue;
          const int mt = tix / (D / 32), nt = tix % (D / 32);
          const int ra = 32 * mt + l32, rb = 32 * nt + l32;
          const uint4 av = *reinterpret_cast<const uint4*>(Pk + ra * BK + 8 * (lc ^ (ra % C::CHV)));
          const uint4 bv = *reinterpret_cast<const uint4*>(Vt + rb * BK + 8 * (lc ^ (rb % C::CHV)));
          acc_g[u] = mfma(as_bf16x8(av), as_bf16x8(bv), acc_g[u]);
        }
      }
    }
    if (C::NSTAGE == 1) {
      __syncthreads();  // the single stage is consumed before it is refilled
      if (b + 1 < nblk) load_block(col_idx[base + b + 1], cur);
    }
  };

  if (nblk > 0) load_block((MODE == MODE_DENSE) ? 0 : col_idx[base], smem);
  if (C::NSTAGE == 2) {
    for (int b = 0; b < nblk; b += 2) {
      block_step(b, smem, smem1);
      if (b + 1 < nblk) block_step(b + 1, smem1, smem);
    }
  } else {
    for (int b = 0; b < nblk; ++b) block_step(b, smem, smem);
  }

  // ---------------- epilogue
  float inv_l = 0.f;
  if (do_s) {
    const float lt = l_run + __shfl_xor(l_run, 32);
    inv_l = lt > 0.f ? 1.f / lt : 0.f;
  }
  float den = 1.f;
  if (C::LINM && lin) {
    const float* Hh = htot + (size_t)bh * (D * D + D);
    if (C::NSTAGE == 2) __syncthreads();
    // H_u^T = (H - G)^T as hi + lo bf16, rows d_v, 16-byte chunks of d_k swizzled
#pragma unroll
    for (int u = 0; u < C::TPW; ++u) {
      const int tix = w * C::TPW + u;
      if (tix >= C::TT) continue;
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
        const int pc = (4 * mt + i4) ^ (dv % (D / 8));
        uint2 wv;
        wv.x = hb[0] | (hb[1] << 16);
        wv.y = hb[2] | (hb[3] << 16);
        *reinterpret_cast<uint2*>(HuHi + dv * D + 8 * pc + 4 * hi) = wv;
        wv.x = pk_bf16(lv[0], lv[1]);
        wv.y = pk_bf16(lv[2], lv[3]);
        *reinterpret_cast<uint2*>(HuLo + dv * D + 8 * pc + 4 * hi) = wv;
      }
    }
    if (tid < D) {
      float g = 0.f;
      for (int b = 0; b < nsel; ++b) g += zblk[((size_t)bh * Nk + col_idx[base + b]) * D + tid];
      zu[tid] = Hh[D * D + tid] - g;
    }
    __syncthreads();
  }

  const size_t orow = ((size_t)bh * N + q) * D;
  f32x16 acc_n[D / 32];
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) acc_n[mt] = f32x16{};
  if (C::LINM && lin) {
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
        const int r = 32 * mt + l32;
        const int pc = (2 * t + hi) ^ (r % (D / 8));
        const uint4 ah = *reinterpret_cast<const uint4*>(HuHi + r * D + 8 * pc);
        const uint4 al = *reinterpret_cast<const uint4*>(HuLo + r * D + 8 * pc);
        acc_n[mt] = mfma(as_bf16x8(ah), bh4, acc_n[mt]);
        acc_n[mt] = mfma(as_bf16x8(ah), bl4, acc_n[mt]);
        acc_n[mt] = mfma(as_bf16x8(al), bh4, acc_n[mt]);
      }
    }
    den = dpart + __shfl_xor(dpart, 32);
  }
  const float wl_den = (C::LINM && lin) ? wl_ / den : 0.f;
  const float ws_l = ws_ * inv_l;
  if (q < N) {
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * i4 + r;
          o[r] = ws_l * acc_o[mt][i] + wl_den * acc_n[mt][i];
        }
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
  const dim3 grid((unsigned)s.R()), block(BQ / 32 * 64);
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(K);
  const uint16_t* vt = reinterpret_cast<const uint16_t*>(ws + L.vt);
  const uint16_t* pk = reinterpret_cast<const uint16_t*>(ws + L.pk);
  const float* zb = reinterpret_cast<const float*>(ws + L.zblk);
  const float* ht = reinterpret_cast<const float*>(ws + L.htot);
  uint16_t* o = static_cast<uint16_t*>(O);
#define SLA_GO(M)                                                                                  \
  hipLaunchKernelGGL((attn_kernel<D, BQ, BK, M>), grid, block, 0, st, q, k, vt, pk, zb, rp, ci,    \
                     alpha, ht, o, s.H, s.N, s.Nq, s.Nk, sl2)
  switch (mode) {
    case MODE_SPARSE: SLA_GO(MODE_SPARSE); break;
    case MODE_LINEAR: SLA_GO(MODE_LINEAR); break;
    case MODE_FUSED: SLA_GO(MODE_FUSED); break;
    default: SLA_GO(MODE_DENSE); break;
  }
#undef SLA_GO
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
