// 8-bit sparse branch on gfx950 matrix cores.
//
// Source: SLA2 write-up (arXiv:2602.12675) §三: the sparse branch holds Q, K,
// the attention probabilities P and V as 8-bit integers - values are scaled
// into the 8-bit range, the products are formed there, and the results are
// scaled back.  Granularity and rounding are not given there; this file
// implements (bit for bit where integers are decided):
//   * codes = round-half-even(x * fl32(127 / amax)) in [-127, 127], scale =
//     fl32(amax / 127); Q per query block, K per key block, V per channel over
//     the whole sequence of a head;
//   * scores I = q8 . k8 (exact int32), S = fl32(I * c), c = fl32(fl32(sq sk)
//     / sqrt(d)), m = the row's maximum S over its selected keys;
//   * P codes = round-half-even(exp2(fma(I, a, -b))) with a = fl32(c log2 e),
//     b = fl32(fl32(m log2 e) - log2 127), i.e. 127 exp(S - m) in float32;
//   * O = sv * (sum code v8) / (sum code), both sums exact int32.
//
// Kernels:
//   quant_block_kernel  Q or K: one workgroup per block of rows, absolute
//                       maximum, then codes (row-major [rows padded][d]);
//   vamax_kernel        V: per-channel maxima of 1024-row chunks;
//   vscale_kernel       V: per-channel scale and reciprocal from the chunks;
//   quant_v_kernel      V: codes as V^T in 64-key tiles [d][64], keys of
//                       every 32-key group in the order the P operand holds
//                       them (key 8a + 4h + b at byte 16h + 4a + b);
//   attn_i8_kernel      one workgroup of BQ/32 wavefronts per mask row; two
//                       passes over the row's 64-key units: pass 1 computes
//                       the integer scores and the exact row maximum (two
//                       units per step), pass 2 recomputes them, forms the P
//                       codes in registers and accumulates P V in int32 on
//                       the matrix cores (tiles loaded two steps ahead into a
//                       ring of three LDS stages).  With
//                       the maximum known before any code is formed, no
//                       rescale is ever needed: the output is one int32 sum
//                       per element, scaled once at the end.
//
// Matrix-core formulation (v_mfma_i32_32x32x32_i8; lane l supplies operand
// row / column l%32 and 16 bytes of the k range, half l/32; accumulator
// element i of lane l is row 8(i/4) + 4(l/32) + i%4, column l%32):
//   S^T (keys x queries) = K . Q^T     A = K tile rows, B = Q rows (registers)
//   O^T (d x queries)   += V^T . P^T   A = V^T tile rows, B = P codes
// The 16 S^T elements of a lane (one query, keys 8a + 4h + b) become the 16
// bytes of its P operand in element order, and the V^T tile stores those keys
// in that order, so P goes from accumulator to operand without a lane move.
#include <climits>
#include <math.h>

#include "sla.h"
#include "sla_internal.h"

namespace sla {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int QROWS = 1024;  // rows per chunk of the V channel maxima

template <int I>
struct IntTag {
  static constexpr int value = I;
};

// ------------------------------------------------------------------ helpers
// 16 bytes of input as floats: bf16 (8 values) or fp32 (4 values).
template <int ES>
struct Chunk;
template <>
struct Chunk<2> {
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
};
template <>
struct Chunk<4> {
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  }
};

// symmetric 8-bit code of x with reciprocal scale r, as a byte
__device__ __forceinline__ uint32_t code8(float x, float r) {
  const float c = fminf(fmaxf(rintf(x * r), -127.f), 127.f);
  return (uint32_t)(int)c & 0xffu;
}

// Code formats: symmetric int8 in [-127, 127], or E4M3 (the OCP 8-bit
// floating-point format, largest finite value 448).
enum Fmt : int { FMT_I8 = 0, FMT_F8 = 1 };
template <int F>
struct CodeFmt;
template <>
struct CodeFmt<FMT_I8> {
  static constexpr float RANGE = 127.f;
  // four codes of x * r, byte e = value e
  __device__ static uint32_t pack4(float x0, float x1, float x2, float x3, float r) {
    return code8(x0, r) | (code8(x1, r) << 8) | (code8(x2, r) << 16) | (code8(x3, r) << 24);
  }
};
template <>
struct CodeFmt<FMT_F8> {
  static constexpr float RANGE = 448.f;
  // the products x * r are rounded to E4M3 by the conversion instruction
  // (nearest, ties to even); |x * r| <= 448 up to one float32 rounding
  __device__ static uint32_t pack4(float x0, float x1, float x2, float x3, float r) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0 * r, x1 * r, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2 * r, x3 * r, lo, true);
  }
};

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
  return m;
}

// Workgroups go round-robin over the 8 XCDs (blockIdx % 8), each with its own
// L2: give every XCD a contiguous range of mask rows, so that adjacent query
// blocks of a head (which select largely the same key blocks) share an L2.
__device__ __forceinline__ long long xcd_row(long long b, long long R) {
  constexpr long long NX = 8;
  const long long q = R / NX, r = R % NX;
  const long long x = b % NX, local = b / NX;
  return x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Direct buffer load of 16 bytes per lane into LDS: lane l writes
// lds_wave_base + 16 l; the byte address is voff + soff in the buffer.
__device__ __forceinline__ void b2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                        void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt at their no-wait maxima).  Direct loads
// to LDS count on vmcnt in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint4 rd16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// v itself, opaque to the optimiser: per-lane offsets derived from it are
// recomputed where they are used instead of being kept live (or spilled)
// across the loop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ i32x16 mfma8(const i32x4& a, const i32x4& b, const i32x16& c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- quantisers
// Codes of one block of BR rows of X [BH][N][D] (rows past N read as zero),
// written to codes [BH][Nb * BR][D]; its scale to scales [BH][Nb].
template <int ES, int D, int BR, int F>
__global__ __launch_bounds__(256) void quant_block_kernel(const char* __restrict__ X, int N, int Nb,
                                                          int8_t* __restrict__ codes,
                                                          float* __restrict__ scales) {
  using CF = CodeFmt<F>;
  using C = Chunk<ES>;
  constexpr int CH = C::N, CPR = D / CH, NC = BR * CPR / 256;
  static_assert(NC * 256 == BR * CPR, "chunks per thread");
  __shared__ float red[4];
  const long long bh = blockIdx.x / Nb;
  const int blk = blockIdx.x % Nb;
  const char* xb = X + (size_t)bh * N * D * ES;
  float x[NC][CH];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int g = threadIdx.x + 256 * k, r = g / CPR, cc = g % CPR;
    const int row = blk * BR + r;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < N) v = *reinterpret_cast<const uint4*>(xb + ((size_t)row * D + cc * CH) * ES);
    C::unpack(v, x[k]);
#pragma unroll
    for (int e = 0; e < CH; ++e) amax = fmaxf(amax, fabsf(x[k][e]));
  }
  amax = block_max(amax, red);
  const float r = amax > 0.f ? __fdiv_rn(CF::RANGE, amax) : 0.f;
  int8_t* cb = codes + ((size_t)bh * Nb + blk) * BR * D;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int g = threadIdx.x + 256 * k, rr = g / CPR, cc = g % CPR;
    uint32_t wv[CH / 4];
#pragma unroll
    for (int j = 0; j < CH / 4; ++j)
      wv[j] = CF::pack4(x[k][4 * j], x[k][4 * j + 1], x[k][4 * j + 2], x[k][4 * j + 3], r);
    int8_t* dst = cb + (size_t)rr * D + cc * CH;
    if (CH == 8) *reinterpret_cast<uint2*>(dst) = make_uint2(wv[0], wv[CH / 4 - 1]);
    else *reinterpret_cast<uint32_t*>(dst) = wv[0];
  }
  if (threadIdx.x == 0) scales[bh * Nb + blk] = __fdiv_rn(amax, CF::RANGE);
}

// Per-channel absolute maxima of rows [chunk * QROWS, +QROWS) of V.
template <int ES, int D>
__global__ __launch_bounds__(256) void vamax_kernel(const char* __restrict__ V, int N, int nchunk,
                                                    float* __restrict__ vpart) {
  using C = Chunk<ES>;
  constexpr int CH = C::N, CPR = D / CH, TR = 256 / CPR;
  static_assert(TR * CPR == 256, "thread layout");
  __shared__ float red[TR][D];
  const long long bh = blockIdx.y;
  const int ch = blockIdx.x;
  const int rl = threadIdx.x / CPR, cc = threadIdx.x % CPR;
  const char* vb = V + (size_t)bh * N * D * ES;
  float m[CH];
#pragma unroll
  for (int e = 0; e < CH; ++e) m[e] = 0.f;
  const int r1 = min(N, (ch + 1) * QROWS);
  for (int r = ch * QROWS + rl; r < r1; r += TR) {
    float x[CH];
    C::unpack(*reinterpret_cast<const uint4*>(vb + ((size_t)r * D + cc * CH) * ES), x);
#pragma unroll
    for (int e = 0; e < CH; ++e) m[e] = fmaxf(m[e], fabsf(x[e]));
  }
#pragma unroll
  for (int e = 0; e < CH; ++e) red[rl][cc * CH + e] = m[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float a = 0.f;
    for (int t = 0; t < TR; ++t) a = fmaxf(a, red[t][threadIdx.x]);
    vpart[((size_t)bh * nchunk + ch) * D + threadIdx.x] = a;
  }
}

// sv = amax / R and rv = R / amax (0 when amax is 0) per channel, R the
// format's range (127 or 448).
template <int F>
__global__ __launch_bounds__(128) void vscale_kernel(const float* __restrict__ vpart, int nchunk, int D,
                                                     float* __restrict__ sv, float* __restrict__ rv) {
  constexpr float R = CodeFmt<F>::RANGE;
  const long long bh = blockIdx.x;
  const int c = threadIdx.x;
  if (c >= D) return;
  float a = 0.f;
  for (int k = 0; k < nchunk; ++k) a = fmaxf(a, vpart[((size_t)bh * nchunk + k) * D + c]);
  sv[bh * D + c] = __fdiv_rn(a, R);
  rv[bh * D + c] = a > 0.f ? __fdiv_rn(R, a) : 0.f;
}

// Codes of one 64-key tile of V, written transposed: vt8 [BH][ntile][D][64],
// key k of the tile at byte 32 (k / 32) + 16 ((k / 4) % 2) + 4 ((k % 32) / 8)
// + k % 4 of its channel row for int8 (the order of a 32-key P operand), at
// byte 32 ((k / 4) % 2) + 16 (k / 32) + 4 ((k % 32) / 8) + k % 4 for E4M3 (the
// order of a 64-key P operand); keys past N are zero.
template <int ES, int D, int F>
__global__ __launch_bounds__(256) void quant_v_kernel(const char* __restrict__ V, int N, int ntile,
                                                      const float* __restrict__ rv,
                                                      int8_t* __restrict__ vt8) {
  using CF = CodeFmt<F>;
  using C = Chunk<ES>;
  constexpr int CH = C::N, CPR = D / CH;
  constexpr int RS = 17;  // LDS row stride in words (64 bytes + 4 of padding against bank conflicts)
  __shared__ uint32_t T[D * RS];
  const long long bh = blockIdx.y;
  const int tile = blockIdx.x;
  const char* vb = V + (size_t)bh * N * D * ES;
  const float* rvh = rv + bh * D;
  for (int wi = threadIdx.x; wi < 16 * CPR; wi += 256) {
    const int kq = wi / CPR, cc = wi % CPR;  // keys 4 kq .. 4 kq + 3, channels cc CH ..
    float x[4][CH];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = tile * 64 + 4 * kq + j;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < N) v = *reinterpret_cast<const uint4*>(vb + ((size_t)key * D + cc * CH) * ES);
      C::unpack(v, x[j]);
    }
    const int k = 4 * kq;
    const int word = F == FMT_I8 ? 8 * (k >> 5) + 4 * ((k >> 2) & 1) + ((k & 31) >> 3)
                                 : 8 * ((k >> 2) & 1) + 4 * (k >> 5) + ((k & 31) >> 3);
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const int c = cc * CH + e;
      T[c * RS + word] = CF::pack4(x[0][e], x[1][e], x[2][e], x[3][e], rvh[c]);
    }
  }
  __syncthreads();
  uint32_t* dst = reinterpret_cast<uint32_t*>(vt8 + ((size_t)bh * ntile + tile) * D * 64);
  for (int g = threadIdx.x; g < D * 16; g += 256) dst[g] = T[(g >> 4) * RS + (g & 15)];
}

// ---------------------------------------------------------------- attention
// LDS layout of a unit (64 keys): the K tile, rows of D bytes with 16-byte
// chunk c of key r at c ^ swk(r), then the V^T tile, rows of 64 bytes with
// chunk e of channel c at e ^ swv(c).  The 16 lanes that read one operand
// chunk from 16 consecutive rows then hit 16 distinct groups of 4 banks.
template <int D>
struct I8Tiles {
  static constexpr int KT = 64 * D;   // bytes of the K tile
  static constexpr int VT = D * 64;   // bytes of the V^T tile
  static constexpr int CPR = D / 16;  // 16-byte chunks per K row
  static constexpr int KSH = CPR == 8 ? 1 : 2;
  __device__ static int swk(int r) { return (r >> KSH) & (CPR - 1); }
  __device__ static int swv(int c) { return (c >> 2) & 3; }
};

// Direct loads of a unit's tiles, split over NW wavefronts: load slot u fills
// the 1 KB at tile + 1024 u, lane l the 16 bytes at 16 l, from the chunk that
// belongs there in the swizzled layout.  K and V^T tiles of the unit starting
// at key key0 both begin at byte key0 * D of their per-head arrays.
template <int D, int NW>
struct I8Load {
  using TT = I8Tiles<D>;
  static constexpr int NK = TT::KT / 1024 / NW;
  static_assert(NK * NW * 1024 == TT::KT, "tile split");
  uint32_t kv[NK], vv[NK];
  int w;
  __device__ __forceinline__ I8Load(int w_, int lane) : w(w_) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int o = 1024 * (w + NW * i) + 16 * lane;
      const int r = o / D, pk = (o % D) / 16;
      kv[i] = (uint32_t)(r * D + 16 * (pk ^ TT::swk(r)));
      const int c = o / 64, pv = (o % 64) / 16;
      vv[i] = (uint32_t)(c * 64 + 16 * (pv ^ TT::swv(c)));
    }
  }
  // the K tile of the unit at key0 into dst (NK loads per wavefront)
  __device__ __forceinline__ void load_k(__amdgpu_buffer_rsrc_t rk, int key0, char* dst) const {
#pragma unroll
    for (int i = 0; i < NK; ++i) b2lds16(rk, kv[i], (uint32_t)key0 * D, dst + 1024 * (w + NW * i));
  }
  // its V^T tile into dst (NK loads per wavefront)
  __device__ __forceinline__ void load_v(__amdgpu_buffer_rsrc_t rv, int key0, char* dst) const {
#pragma unroll
    for (int i = 0; i < NK; ++i) b2lds16(rv, vv[i], (uint32_t)key0 * D, dst + 1024 * (w + NW * i));
  }
};

// S^T of one 32-key tile of a unit (D/32 k-steps), the K fragments read PF
// matrix ops ahead of their use (a rolling window of PF registers), in an
// order pinned with sched_group_barrier so that the LDS latency stays hidden
// behind the matrix ops already issued.
template <int D, int PF>
__device__ __forceinline__ i32x16 score_tile(const char* Kt, const i32x4 (&qf)[D / 32],
                                             const int (&koff)[D / 32]) {
  constexpr int NT = D / 32;
  static_assert(PF <= NT, "prefetch window");
  uint4 fr[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) fr[i] = rd16(Kt + koff[i]);
  i32x16 sc = i32x16{};
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const uint4 a = fr[i % PF];
    if (i + PF < NT) fr[i % PF] = rd16(Kt + koff[i + PF]);
    sc = mfma8(__builtin_bit_cast(i32x4, a), qf[i], sc);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // PF LDS reads
#pragma unroll
  for (int i = 0; i + PF < NT; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix op
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
  return sc;
}

template <int D, int BQ, int SUB, int OES>
__global__ __launch_bounds__(BQ / 32 * 64, 2) void attn_i8_kernel(
    const int8_t* __restrict__ q8, const int8_t* __restrict__ k8, const int8_t* __restrict__ vt8,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, char* __restrict__ O, int N, int Nq,
    int Nk, float lam, float l2e, float l2_127) {
  using TT = I8Tiles<D>;
  constexpr int NW = BQ / 32;
  constexpr int STAGE = TT::KT + TT::VT;
  // three distinct stage arrays, so the compiler can tell the loads into one
  // from the operand reads of another
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  __shared__ __attribute__((aligned(16))) char st2[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const long long row = xcd_row(blockIdx.x, (long long)gridDim.x);
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  const int base = row_ptr[row];
  const int nunits = (row_ptr[row + 1] - base) * SUB;
  const int Npad = Nk * SUB * 64;
  const int q = qi * BQ + 32 * w + l32;  // query rows are padded to Nq * BQ

  i32x4 qf[D / 32];
  const int8_t* qrow = q8 + ((size_t)bh * Nq * BQ + q) * D;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) qf[kk] = *reinterpret_cast<const i32x4*>(qrow + 32 * kk + 16 * hi);
  int koff[D / 32], voff[2];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) koff[kk] = l32 * D + 16 * ((2 * kk + hi) ^ TT::swk(l32));
#pragma unroll
  for (int g = 0; g < 2; ++g) voff[g] = l32 * 64 + 16 * ((2 * g + hi) ^ TT::swv(l32));

  i32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = i32x16{};
  uint32_t lsum = 0;  // this lane's sum of P codes
  if (nunits > 0) {
    const float sqv = sq[bh * Nq + qi];
    const float* skh = sk + bh * Nk;
    const auto rk = buf_rsrc(k8 + (size_t)bh * Npad * D, (uint32_t)Npad * D);
    const auto rv = buf_rsrc(vt8 + (size_t)bh * Npad * D, (uint32_t)Npad * D);
    using LP = I8Load<D, NW>;
    // Steps: pass 1 scores the K tiles of two units per step (n1 steps),
    // pass 2 takes one unit's K and V^T tiles per step.  Every step loads two
    // tiles (the second K tile of an odd last pass-1 step repeats the first),
    // so each step issues 2 NK loads per wavefront, two steps ahead of use
    // into a ring of three stages.
    const int n1 = (nunits + 1) >> 1;
    const int nsteps = n1 + nunits;
    float m = -INFINITY, nb = 0.f;
    auto blk_of = [&](int u) { return col_idx[base + u / SUB]; };
    auto key0_of = [&](int u, int blk) { return (blk * SUB + u % SUB) * 64; };
    auto issue = [&](int s, char* dst) __attribute__((always_inline)) {
      const LP lp(w, opaque(lane));
      if (s < n1) {
        const int u0 = 2 * s, u1 = min(2 * s + 1, nunits - 1);
        lp.load_k(rk, key0_of(u0, blk_of(u0)), dst);
        lp.load_k(rk, key0_of(u1, blk_of(u1)), dst + TT::KT);
      } else {
        const int u = s - n1;
        const int k0 = key0_of(u, blk_of(u));
        lp.load_k(rk, k0, dst);
        lp.load_v(rv, k0, dst + TT::KT);
      }
    };
    constexpr int PF = D == 128 ? 2 : 1;
    // pass 1 on the K tile of unit u: this lane's largest score.  MASK: the
    // unit runs past N (only the last unit of a sequence), keys at offset
    // >= lim do not exist; the common case carries no per-element test.
    auto pass1_unit = [&](const char* Ks, int u) __attribute__((always_inline)) {
      const int blk = blk_of(u);
      const int lim = min(64, N - key0_of(u, blk));  // valid keys of the unit
      const float cu = (sqv * skh[blk]) * lam;        // fl32(fl32(sq sk) / sqrt(d))
      auto body = [&](auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value != 0;
        const int limh = lim - 4 * hi;  // element i of tile kt is key 32 kt + 8 (i/4) + 4 hi + i%4
        int im = INT_MIN;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const i32x16 sc = score_tile<D, PF>(Ks + kt * 32 * D, qf, koff);
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const int a = (!MASK || 32 * kt + 8 * (i >> 2) + (i & 3) < limh) ? sc[i] : INT_MIN;
            const int b = (!MASK || 32 * kt + 8 * (i >> 2) + (i & 3) + 1 < limh) ? sc[i + 1] : INT_MIN;
            im = max(im, max(a, b));  // v_max3_i32
          }
        }
        if (im != INT_MIN) m = fmaxf(m, (float)im * cu);
      };
      if (lim < 64) body(IntTag<1>{});
      else body(IntTag<0>{});
    };
    // pass 2 on unit u (K tile at cur, V^T tile after it), one 32-key tile at
    // a time: scores, P codes (the B operand), then its share of P V
    auto pass2_unit = [&](const char* cur, int u) __attribute__((always_inline)) {
      if (u == 0) {
        // the row maximum of this query: lanes l and l^32 hold its two key halves
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        m = fmaxf(m, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
        nb = (m * l2e) - l2_127;  // fl32(fl32(m log2 e) - log2 127); no contraction in this file
      }
      const int blk = blk_of(u);
      const int lim = min(64, N - key0_of(u, blk));
      const float au = ((sqv * skh[blk]) * lam) * l2e;
      const char* Vs = cur + TT::KT;
      auto body = [&](auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value != 0;
        const int limh = lim - 4 * hi;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const i32x16 sc = score_tile<D, PF>(cur + kt * 32 * D, qf, koff);
          i32x4 pc;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t wd = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float t = __builtin_fmaf((float)sc[4 * e + j], au, -nb);
              if (MASK && 32 * kt + 8 * e + j >= limh) t = -INFINITY;
              wd = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_exp2f(t), j, wd);
            }
            pc[e] = (int)wd;
            lsum = __builtin_amdgcn_udot4(wd, 0x01010101u, lsum, false);
          }
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
            acc[dt] = mfma8(__builtin_bit_cast(i32x4, rd16(Vs + dt * 32 * 64 + voff[kt])), pc, acc[dt]);
        }
      };
      if (lim < 64) body(IntTag<1>{});
      else body(IntTag<0>{});
    };
    auto step = [&](int s, const char* cur, char* ahead) __attribute__((always_inline)) {
      if (s + 1 < nsteps) wait_vm<2 * LP::NK>();  // step s landed; step s+1 may be in flight
      else wait_vm<0>();
      __syncthreads();  // every wavefront's loads of step s landed; step s-1 consumed
      if (s + 2 < nsteps) issue(s + 2, ahead);
      if (s < n1) {
        pass1_unit(cur, 2 * s);
        if (2 * s + 1 < nunits) pass1_unit(cur + TT::KT, 2 * s + 1);
      } else {
        pass2_unit(cur, s - n1);
      }
    };
    issue(0, st0);
    if (nsteps > 1) issue(1, st1);
    int s = 0;
    for (; s + 3 <= nsteps; s += 3) {
      step(s, st0, st2);
      step(s + 1, st1, st0);
      step(s + 2, st2, st1);
    }
    if (s < nsteps) step(s, st0, st2);
    if (s + 1 < nsteps) step(s + 1, st1, st0);
  }

  const uint32_t L = lsum + (uint32_t)__shfl_xor((int)lsum, 32);
  const float inv = L ? 1.f / (float)L : 0.f;
  if (q >= N) return;
  const float* svh = sv + bh * D;
  char* orow = O + ((size_t)bh * N + q) * D * OES;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int c0 = 32 * dt + 8 * a + 4 * hi;
      const float4 s4 = *reinterpret_cast<const float4*>(svh + c0);
      const float sc4[4] = {s4.x, s4.y, s4.z, s4.w};
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = ((float)acc[dt][4 * a + j] * sc4[j]) * inv;
      if (OES == 4) {
        *reinterpret_cast<float4*>(orow + c0 * 4) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        // round to nearest even (v_cvt_pk_bf16_f32)
        const f32x2 lo = {o[0], o[1]}, hi2 = {o[2], o[3]};
        *reinterpret_cast<uint2*>(orow + c0 * 2) =
            make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                       __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, bf16x2)));
      }
    }
}

// ------------------------------------- single pass: int8 scores, E4M3 P V
// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and unit scales
// (E8M0 127 = 2^0): lane l supplies 32 bytes of operand row / column l%32
// from half l/32 of the k range; A and B take the same k order, whatever it
// is, so the operands below are built to agree with each other and not with
// any particular order.  Accumulator element i of lane l is row 8(i/4) +
// 4(l/32) + i%4, column l%32 (as every 32 x 32 float32 MFMA).  The products
// are exact; their sum is not always rounded once (measured: within 2^-12 of
// the sum of |products| for operands of wide exponent range).
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat8(const uint4& x, const uint4& y) {
  return i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
}

// One workgroup of BQ/32 wavefronts per mask row, ONE pass over the row's
// 64-key units (K and V^T tiles of unit u+2 loaded while unit u is computed,
// three LDS stages as in attn_i8_kernel):
//   S^T = K Q^T         int8 codes, exact int32 (score_tile); lane (query
//                       l%32, half h) holds keys 32 t + 8 a + 4 h + b of the
//                       unit (tile t, element 4 a + b)
//   m  = running maximum of S = fl32(I c) over the units so far (lanes l,
//        l^32 agree); when it rises, O and l are multiplied by
//        exp(m_old - m_new)
//   P codes = E4M3(exp2(fma(I, a, -nb))), a = fl32(c log2 e), nb =
//        fl32(m log2 e) - 8: 256 exp(S - m), keys past N give 0
//   O^T += V^T P^T      E4M3, 64 keys per MFMA; byte j of a lane's P operand
//                       is tile j/16, element j%16, and the V^T tile row
//                       holds key 32 t + 8 a + 4 h + b at byte 32 h + 16 t +
//                       4 a + b
//   l  += ones P^T      (one MFMA: every row of the result is the code sum)
//   O = sv O / l at the end.
template <int D, int BQ, int SUB, int OES>
__global__ __launch_bounds__(BQ / 32 * 64, 2) void attn_i8f8_kernel(
    const int8_t* __restrict__ q8, const int8_t* __restrict__ k8, const int8_t* __restrict__ vt8,
    const float* __restrict__ sq, const float* __restrict__ sk, const float* __restrict__ sv,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, char* __restrict__ O, int N, int Nq,
    int Nk, float lam, float l2e) {
  using TT = I8Tiles<D>;
  constexpr int NW = BQ / 32;
  constexpr int STAGE = TT::KT + TT::VT;
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  __shared__ __attribute__((aligned(16))) char st2[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const long long row = xcd_row(blockIdx.x, (long long)gridDim.x);
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  const int base = row_ptr[row];
  const int nunits = (row_ptr[row + 1] - base) * SUB;
  const int Npad = Nk * SUB * 64;
  const int q = qi * BQ + 32 * w + l32;  // query rows are padded to Nq * BQ

  i32x4 qf[D / 32];
  const int8_t* qrow = q8 + ((size_t)bh * Nq * BQ + q) * D;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) qf[kk] = *reinterpret_cast<const i32x4*>(qrow + 32 * kk + 16 * hi);
  int koff[D / 32], voff[2];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) koff[kk] = l32 * D + 16 * ((2 * kk + hi) ^ TT::swk(l32));
  // V^T operand (A of O^T): channel row l32 of a 32-row tile, bytes 32 hi ..
  // 32 hi + 31 of its 64-byte row (swizzled 16-byte chunks)
#pragma unroll
  for (int c = 0; c < 2; ++c) voff[c] = l32 * 64 + 16 * ((2 * hi + c) ^ TT::swv(l32));
  const i32x8 ones = i32x8{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                           0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0

  f32x16 acc[D / 32], lacc = f32x16{};
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};
  if (nunits > 0) {
    const float sqv = sq[bh * Nq + qi];
    const float* skh = sk + bh * Nk;
    const auto rk = buf_rsrc(k8 + (size_t)bh * Npad * D, (uint32_t)Npad * D);
    const auto rv = buf_rsrc(vt8 + (size_t)bh * Npad * D, (uint32_t)Npad * D);
    using LP = I8Load<D, NW>;
    constexpr int PF = D == 128 ? 2 : 1;
    float m = -INFINITY, nb = 0.f;
    auto blk_of = [&](int u) { return col_idx[base + u / SUB]; };
    auto key0_of = [&](int u, int blk) { return (blk * SUB + u % SUB) * 64; };
    auto issue = [&](int u, char* dst) __attribute__((always_inline)) {
      const LP lp(w, opaque(lane));
      const int k0 = key0_of(u, blk_of(u));
      lp.load_k(rk, k0, dst);
      lp.load_v(rv, k0, dst + TT::KT);
    };
    auto unit = [&](const char* cur, int u) __attribute__((always_inline)) {
      const int blk = blk_of(u);
      const int lim = min(64, N - key0_of(u, blk));  // keys of the unit below N (<= 0: none)
      if (lim <= 0) return;
      const float cu = (sqv * skh[blk]) * lam;       // fl32(fl32(sq sk) / sqrt(d))
      const float au = cu * l2e;
      i32x16 sc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) sc[t] = score_tile<D, PF>(cur + t * 32 * D, qf, koff);
      // A unit that runs past N (only the last unit of a sequence, lim < 64):
      // keys at offset >= lim do not exist; they are left out of the maximum
      // and their code bytes are cleared after the conversion
      const int limh = lim - 4 * hi;  // element i of tile t is key 32 t + 8 (i/4) + 4 hi + i%4
      int im = INT_MIN;
      if (lim < 64) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) im = max(im, 32 * t + 8 * (i >> 2) + (i & 3) < limh ? sc[t][i] : INT_MIN);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) im = max(im, max(sc[0][i], sc[1][i]));
      }
      im = max(im, __shfl_xor(im, 32));  // lanes l, l^32 hold the two key halves of one query
      const float mxs = (float)im * cu;  // the unit's largest S = fl32(I c) (c >= 0)
      if (__ballot(mxs > m)) {
        const float m_new = fmaxf(m, mxs);
        const float corr = __builtin_amdgcn_exp2f((m - m_new) * l2e);  // 0 on the first unit
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= corr;
        lacc *= corr;
        m = m_new;
        nb = (m * l2e) - 8.f;
      }
      // P codes: byte j of the operand = tile j/16, element j%16
      i32x8 pc;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sc[t][4 * e], au, -nb));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sc[t][4 * e + 1], au, -nb));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sc[t][4 * e + 2], au, -nb));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sc[t][4 * e + 3], au, -nb));
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          pc[4 * t + e] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, lo, true);
        }
      if (lim < 64) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int nv = min(4, max(0, limh - (32 * t + 8 * e)));  // valid keys of this word
            pc[4 * t + e] &= nv == 4 ? -1 : (int)((1u << (8 * nv)) - 1u);
          }
      }
      const char* Vs = cur + TT::KT;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        acc[dt] = mfma_f8(cat8(rd16(Vs + dt * 32 * 64 + voff[0]), rd16(Vs + dt * 32 * 64 + voff[1])), pc, acc[dt]);
      lacc = mfma_f8(ones, pc, lacc);
    };
    auto step = [&](int u, const char* cur, char* ahead) __attribute__((always_inline)) {
      if (u + 1 < nunits) wait_vm<2 * LP::NK>();  // unit u landed; unit u+1 may be in flight
      else wait_vm<0>();
      __syncthreads();  // every wavefront's loads of unit u landed; unit u-1 consumed
      if (u + 2 < nunits) issue(u + 2, ahead);
      unit(cur, u);
    };
    issue(0, st0);
    if (nunits > 1) issue(1, st1);
    int u = 0;
    for (; u + 3 <= nunits; u += 3) {
      step(u, st0, st2);
      step(u + 1, st1, st0);
      step(u + 2, st2, st1);
    }
    if (u < nunits) step(u, st0, st2);
    if (u + 1 < nunits) step(u + 1, st1, st0);
  }

  const float L = lacc[0];
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (q >= N) return;
  const float* svh = sv + bh * D;
  char* orow = O + ((size_t)bh * N + q) * D * OES;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int c0 = 32 * dt + 8 * a + 4 * hi;
      const float4 s4 = *reinterpret_cast<const float4*>(svh + c0);
      const float sc4[4] = {s4.x, s4.y, s4.z, s4.w};
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (acc[dt][4 * a + j] * sc4[j]) * inv;
      if (OES == 4) {
        *reinterpret_cast<float4*>(orow + c0 * 4) = make_float4(o[0], o[1], o[2], o[3]);
      } else {
        const f32x2 lo = {o[0], o[1]}, hi2 = {o[2], o[3]};
        *reinterpret_cast<uint2*>(orow + c0 * 2) =
            make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                       __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, bf16x2)));
      }
    }
}

// ------------------------------------------------------------------ launchers
// Q and K codes in format FQK, V codes in format FV.
template <int ES, int D, int FQK, int FV>
hipError_t quant_dispatch(const Shape& s, const void* Q, const void* K, const void* V, char* qb,
                          const I8Layout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H;
  const char* q = static_cast<const char*>(Q);
  const char* k = static_cast<const char*>(K);
  const char* v = static_cast<const char*>(V);
  int8_t* q8 = reinterpret_cast<int8_t*>(qb + L.q8);
  int8_t* k8 = reinterpret_cast<int8_t*>(qb + L.k8);
  float* sq = reinterpret_cast<float*>(qb + L.sq);
  float* sk = reinterpret_cast<float*>(qb + L.sk);
  if (s.bq == 128)
    hipLaunchKernelGGL((quant_block_kernel<ES, D, 128, FQK>), dim3((unsigned)(BH * s.Nq)), dim3(256), 0, st, q, s.N,
                       s.Nq, q8, sq);
  else
    hipLaunchKernelGGL((quant_block_kernel<ES, D, 64, FQK>), dim3((unsigned)(BH * s.Nq)), dim3(256), 0, st, q, s.N,
                       s.Nq, q8, sq);
  // K: one scale per key block of bk rows
  if (s.bk == 128)
    hipLaunchKernelGGL((quant_block_kernel<ES, D, 128, FQK>), dim3((unsigned)(BH * s.Nk)), dim3(256), 0, st, k, s.N,
                       s.Nk, k8, sk);
  else
    hipLaunchKernelGGL((quant_block_kernel<ES, D, 64, FQK>), dim3((unsigned)(BH * s.Nk)), dim3(256), 0, st, k, s.N,
                       s.Nk, k8, sk);
  float* vpart = reinterpret_cast<float*>(qb + L.vpart);
  float* sv = reinterpret_cast<float*>(qb + L.sv);
  float* rv = reinterpret_cast<float*>(qb + L.rv);
  hipLaunchKernelGGL((vamax_kernel<ES, D>), dim3((unsigned)L.vchunks, (unsigned)BH), dim3(256), 0, st, v, s.N,
                     L.vchunks, vpart);
  hipLaunchKernelGGL((vscale_kernel<FV>), dim3((unsigned)BH), dim3(128), 0, st, vpart, L.vchunks, D, sv, rv);
  const int ntile = s.Nk * s.bk / 64;
  hipLaunchKernelGGL((quant_v_kernel<ES, D, FV>), dim3((unsigned)ntile, (unsigned)BH), dim3(256), 0, st, v, s.N,
                     ntile, rv, reinterpret_cast<int8_t*>(qb + L.vt8));
  return hipGetLastError();
}

template <int D, int BQ, int SUB>
hipError_t attn_i8_dispatch(const Shape& s, const char* qb, const I8Layout& L, const int32_t* rp,
                            const int32_t* ci, void* O, hipStream_t st) {
  const float lam = (float)(1.0 / sqrt((double)D));
  const float l2e = (float)log2(M_E);
  const float l2_127 = (float)log2(127.0);
  const int8_t* q8 = reinterpret_cast<const int8_t*>(qb + L.q8);
  const int8_t* k8 = reinterpret_cast<const int8_t*>(qb + L.k8);
  const int8_t* vt8 = reinterpret_cast<const int8_t*>(qb + L.vt8);
  const float* sq = reinterpret_cast<const float*>(qb + L.sq);
  const float* sk = reinterpret_cast<const float*>(qb + L.sk);
  const float* sv = reinterpret_cast<const float*>(qb + L.sv);
  const dim3 grid((unsigned)s.R()), block(BQ / 32 * 64);
  char* o = static_cast<char*>(O);
  if (s.dtype == SLA_BF16)
    hipLaunchKernelGGL((attn_i8_kernel<D, BQ, SUB, 2>), grid, block, 0, st, q8, k8, vt8, sq, sk, sv, rp, ci, o,
                       s.N, s.Nq, s.Nk, lam, l2e, l2_127);
  else
    hipLaunchKernelGGL((attn_i8_kernel<D, BQ, SUB, 4>), grid, block, 0, st, q8, k8, vt8, sq, sk, sv, rp, ci, o,
                       s.N, s.Nq, s.Nk, lam, l2e, l2_127);
  return hipGetLastError();
}

template <int D, int BQ, int SUB>
hipError_t attn_i8f8_dispatch(const Shape& s, const char* qb, const I8Layout& L, const int32_t* rp,
                            const int32_t* ci, void* O, hipStream_t st) {
  const float lam = (float)(1.0 / sqrt((double)D));
  const float l2e = (float)log2(M_E);
  const int8_t* q8 = reinterpret_cast<const int8_t*>(qb + L.q8);
  const int8_t* k8 = reinterpret_cast<const int8_t*>(qb + L.k8);
  const int8_t* vt8 = reinterpret_cast<const int8_t*>(qb + L.vt8);
  const float* sq = reinterpret_cast<const float*>(qb + L.sq);
  const float* sk = reinterpret_cast<const float*>(qb + L.sk);
  const float* sv = reinterpret_cast<const float*>(qb + L.sv);
  const dim3 grid((unsigned)s.R()), block(BQ / 32 * 64);
  char* o = static_cast<char*>(O);
  if (s.dtype == SLA_BF16)
    hipLaunchKernelGGL((attn_i8f8_kernel<D, BQ, SUB, 2>), grid, block, 0, st, q8, k8, vt8, sq, sk, sv, rp, ci, o,
                       s.N, s.Nq, s.Nk, lam, l2e);
  else
    hipLaunchKernelGGL((attn_i8f8_kernel<D, BQ, SUB, 4>), grid, block, 0, st, q8, k8, vt8, sq, sk, sv, rp, ci, o,
                       s.N, s.Nq, s.Nk, lam, l2e);
  return hipGetLastError();
}

}  // namespace

I8Layout i8_layout(const Shape& s) {
  I8Layout L{};
  const size_t BH = (size_t)s.B * s.H;
  const size_t Npad = (size_t)s.Nk * s.bk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return o;
  };
  L.vchunks = (s.N + QROWS - 1) / QROWS;
  L.q8 = take(BH * s.Nq * s.bq * s.d);
  L.k8 = take(BH * Npad * s.d);
  L.vt8 = take(BH * Npad * s.d);
  L.sq = take(BH * s.Nq * sizeof(float));
  L.sk = take(BH * s.Nk * sizeof(float));
  L.sv = take(BH * s.d * sizeof(float));
  L.rv = take(BH * s.d * sizeof(float));
  L.vpart = take(BH * L.vchunks * s.d * sizeof(float));
  L.total = off;
  return L;
}

template <int FQK, int FV>
hipError_t quant_fmt(const Shape& s, const void* Q, const void* K, const void* V, char* qbuf, const I8Layout& L,
                     hipStream_t st) {
  const bool bf = s.dtype == SLA_BF16;
  if (s.d == 128)
    return bf ? quant_dispatch<2, 128, FQK, FV>(s, Q, K, V, qbuf, L, st)
              : quant_dispatch<4, 128, FQK, FV>(s, Q, K, V, qbuf, L, st);
  if (s.d == 64)
    return bf ? quant_dispatch<2, 64, FQK, FV>(s, Q, K, V, qbuf, L, st)
              : quant_dispatch<4, 64, FQK, FV>(s, Q, K, V, qbuf, L, st);
  return hipErrorInvalidValue;
}

hipError_t launch_quant_i8(const Shape& s, const void* Q, const void* K, const void* V, char* qbuf,
                           const I8Layout& L, hipStream_t st) {
  return quant_fmt<FMT_I8, FMT_I8>(s, Q, K, V, qbuf, L, st);
}

hipError_t launch_quant_i8f8(const Shape& s, const void* Q, const void* K, const void* V, char* qbuf,
                             const I8Layout& L, hipStream_t st) {
  return quant_fmt<FMT_I8, FMT_F8>(s, Q, K, V, qbuf, L, st);
}

hipError_t launch_attn_i8(const Shape& s, const char* qbuf, const I8Layout& L, const int32_t* rp,
                          const int32_t* ci, void* O, hipStream_t st) {
#define SLA_I8(DD, QQ, KK) \
  if (s.d == DD && s.bq == QQ && s.bk == KK) return attn_i8_dispatch<DD, QQ, KK / 64>(s, qbuf, L, rp, ci, O, st);
  SLA_I8(128, 128, 64)
  SLA_I8(128, 128, 128)
  SLA_I8(128, 64, 64)
  SLA_I8(128, 64, 128)
  SLA_I8(64, 128, 64)
  SLA_I8(64, 128, 128)
  SLA_I8(64, 64, 64)
  SLA_I8(64, 64, 128)
#undef SLA_I8
  return hipErrorInvalidValue;
}

hipError_t launch_attn_i8f8(const Shape& s, const char* qbuf, const I8Layout& L, const int32_t* rp,
                          const int32_t* ci, void* O, hipStream_t st) {
#define SLA_F8(DD, QQ, KK) \
  if (s.d == DD && s.bq == QQ && s.bk == KK) return attn_i8f8_dispatch<DD, QQ, KK / 64>(s, qbuf, L, rp, ci, O, st);
  SLA_F8(128, 128, 64)
  SLA_F8(128, 128, 128)
  SLA_F8(128, 64, 64)
  SLA_F8(128, 64, 128)
  SLA_F8(64, 128, 64)
  SLA_F8(64, 128, 128)
  SLA_F8(64, 64, 64)
  SLA_F8(64, 64, 128)
#undef SLA_F8
  return hipErrorInvalidValue;
}

}  // namespace sla
