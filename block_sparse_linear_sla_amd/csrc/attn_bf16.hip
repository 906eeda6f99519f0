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
// prep_kernel (linear branch only; one workgroup per chunk of key blocks of one
//   head) streams K and V once and writes phi(K) = elu(K) + 1 as bf16 in the
//   layout of K, the per-key-block column sums of phi(K) (float32), and the
//   chunk's partial linear totals H = sum_u phi(k_u)^T v_u, z = sum_u phi(k_u)
//   (phi split into hi + lo bf16 so the totals keep ~16 mantissa bits).
//
// attn_kernel / fused_kernel (one workgroup per mask row = (b, h, query block
//   of BQ rows)) walk the row's key blocks in units of 64 keys.  The K, V and
//   (linear branch) phi(K) tiles of a unit go straight from global memory to
//   LDS (buffer loads with an LDS destination, 16 bytes per lane), row-major
//   with 16-byte chunks XOR-swizzled by key so the operand reads are free of
//   bank conflicts.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16; lane l supplies operand
// row / column l%32 and a k-slice 8*(l/32) .. +7; accumulator element i of
// lane l is row 8*(i/4) + 4*(l/32) + i%4, column l%32):
//   S^T  (keys x queries)  = K . Q^T           A = K tile, B = Q (registers)
//   O^T  (d x queries)    += V^T . P^T          A = V^T (transposed read), B = P (registers)
//   G    (d x d)          += phi(K)^T . V       A = phi(K)^T, B = V^T (transposed reads)
// With queries on the lane axis of S^T and O^T, each lane's softmax state is
// its own query's: the row max / sum need one exchange with lane l^32 and the
// rescale of O is lane-local.  The S^T accumulator of a lane lists keys in the
// order (0-3, 8-11 | 4-7, 12-15) of every 16, and the V^T / phi(K)^T operands
// are read in that same key order with ds_read_b64_tr_b16 (two 4-key reads per
// operand), so P goes from accumulator to operand in registers.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <int I>
struct IntTag {
  static constexpr int value = I;
};

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

__device__ __forceinline__ uint32_t elem(const uint4& v, int e) {
  const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// ------------------------------------------------------------------ attention
constexpr int LDS_BYTES = 160 * 1024;  // LDS of one gfx950 compute unit
constexpr int KU = 64;                 // keys per attention unit; a listed block of BK keys is BK/64 units

// LDS tile layouts of one 64-key unit.  Every direct load instruction brings
// 64 x 16 bytes that land in LDS in lane order, so a tile is stored as rows of
// whole 128-byte global lines - [D/64 halves][64 keys][128 B], row-major like
// K, V and phi(K) in memory - and each load covers 8 complete lines.  Inside a
// row the 16-byte chunks are XOR-swizzled by the key:
//   K tiles       chunk c of key r at c ^ swk(r) = c ^ ((r >> 1) & 7): the 16
//                 keys that a 16-lane group reads for one S operand hit 16
//                 distinct bank groups;
//   V, phi(K)     chunk c of key r at c ^ swv(r) = c ^ (4 ((r >> 1) & 1)): the
//                 4 keys x 32 bytes that a 16-lane group reads with one
//                 transposed read hit distinct banks.
// H_u^T (written with ordinary LDS stores after the loop) keeps a "plane"
// layout: every 16-element k-slice is a plane of 32 bytes per row, the two
// 16-byte halves swapped when bit 3 of the row is set.
template <int D>
struct Tiles {
  static constexpr int KHALF = KU * 128;       // bytes of one 64-d half of a tile
  static constexpr int KT_BYTES = KU * D * 2;  // one [64 keys x D] tile
  static constexpr int HPB = D * 32;           // bytes of one H_u^T plane (16 d_k)
};

__device__ __forceinline__ int swk(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swv(int r) { return 4 * ((r >> 1) & 1); }

__device__ __forceinline__ int lane_base(int lane) {
  const int l32 = lane & 31, hi = lane >> 5;
  return l32 * 32 + 16 * (hi ^ ((l32 >> 3) & 1));
}

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 4-element pieces addressed by lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.
__device__ __forceinline__ s16x4 tr16(const char* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// Per-lane byte offsets of the MFMA operand reads (lane l: row l%32 of a
// 32-row tile, k-slice half l/32).
//   K (S operand): the 16-wide d step t of key subtile kt at (t/4) KHALF +
//     4096 kt + off[t%4] (one 16-byte read).
//   V^T / phi(K)^T (transposed reads of a row-major tile): rows d = 32 dt +
//     l%32, the 8 keys of key plane pl in the order 4h + {0..3}, 4h + 8 +
//     {0..3} (h = l/32).  Lanes 4m .. 4m+3 of a 16-lane group address key
//     4h + m (+ 8 for the second read) and 4 consecutive d each, so lane i
//     receives d = base + i across the 4 keys.
template <int D>
struct ReadPlan {
  int off[4], tro[2];
  __device__ __forceinline__ explicit ReadPlan(int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int t = 0; t < 4; ++t) off[t] = l32 * 128 + 16 * ((2 * t + hi) ^ swk(l32));
    const int i = lane & 15, g2 = (lane >> 4) & 1, kl = 4 * hi + (i >> 2);
#pragma unroll
    for (int p = 0; p < 2; ++p) {  // d offset 32 p inside a 64-d half
      const int d = 32 * p + 16 * g2 + 4 * (i & 3);
      tro[p] = kl * 128 + 16 * ((d >> 3) ^ swv(kl)) + 8 * ((d >> 2) & 1);
    }
  }
  __device__ __forceinline__ const char* kp(const char* Ks, int kt, int t) const {
    return Ks + (t / 4) * Tiles<D>::KHALF + kt * 4096 + off[t % 4];
  }
  __device__ __forceinline__ bf16x8 vt(const char* Vs, int dt, int pl) const {
    // dt may be a wave-uniform runtime value: select rather than index
    const char* b = Vs + (dt / 2) * Tiles<D>::KHALF + pl * 16 * 128 + ((dt & 1) ? tro[1] : tro[0]);
    const s16x4 a = tr16(b), c = tr16(b + 8 * 128);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, c, 0, 1, 2, 3, 4, 5, 6, 7));
  }
};

__device__ __forceinline__ uint4 rd16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their no-wait maxima).  Direct
// loads to LDS count on vmcnt, in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Buffer resource over [base, base + bytes) for raw (unstructured) buffer
// loads; reads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Direct buffer load of 16 (or 4) bytes per lane into LDS: lane l writes
// lds_wave_base + 16 l (4 l); the byte address is voff + soff in the buffer.
__device__ __forceinline__ void b2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                        void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void b2lds4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                       void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 4, (int)voff, (int)soff, 0, 0);
}

// Direct loads of one unit's tiles into LDS, split over NWL wavefronts.  Load
// slot u of a tile fills the 1 KB at tile + 1024 u (8 rows of 128 bytes, in
// the swizzled layouts above): lane l brings the 16-byte chunk that belongs at
// position l.  Each load is a per-head buffer resource over a row-major
// [N, D] array, the unit's byte offset (scalar) and a per-lane byte offset
// fixed for the kernel; rows past N read as zeros.
template <int D, int NWL>
struct LoadPlan {
  using T = Tiles<D>;
  static constexpr int NK = T::KT_BYTES / 1024 / NWL;   // slots per wavefront and tile
  static_assert(NK * NWL * 1024 == T::KT_BYTES, "tile split");
  uint32_t koff[NK], roff[NK];
  int w;

  __device__ __forceinline__ LoadPlan(int w_, int lane) : w(w_) {
#pragma unroll
    for (int ii = 0; ii < NK; ++ii) {
      const int u = w + NWL * ii;
      const int hd = u / 8, key = 8 * (u % 8) + (lane >> 3);
      koff[ii] = (uint32_t)(key * D * 2 + hd * 128 + 16 * ((lane & 7) ^ swk(key)));
      roff[ii] = (uint32_t)(key * D * 2 + hd * 128 + 16 * ((lane & 7) ^ swv(key)));
    }
  }
  // K tile (S operand layout) of the unit starting at key key0
  __device__ __forceinline__ void load_k(__amdgpu_buffer_rsrc_t rk, int key0, char* dst) const {
    const uint32_t soff = (uint32_t)key0 * (D * 2);
#pragma unroll
    for (int ii = 0; ii < NK; ++ii) b2lds16(rk, koff[ii], soff, dst + 1024 * (w + NWL * ii));
  }
  // V or phi(K) tile (transposed-read layout) of the unit starting at key key0
  __device__ __forceinline__ void load_r(__amdgpu_buffer_rsrc_t rr, int key0, char* dst) const {
    const uint32_t soff = (uint32_t)key0 * (D * 2);
#pragma unroll
    for (int ii = 0; ii < NK; ++ii) b2lds16(rr, roff[ii], soff, dst + 1024 * (w + NWL * ii));
  }
};

// max of v over lanes l and l^32 (v_permlane32_swap exchanges the two halves;
// taking the max with the own value makes the result independent of which
// output holds which half)
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(
      v, __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Running online-softmax state of one query; lanes l and l^32 hold the two
// key halves of the same query and keep identical m.
struct Softmax {
  float m;     // running max of the raw scores
  float thr;   // m + 8 / scale_log2: a unit max above it moves m
  float mneg;  // -m * scale_log2
  float l;     // this lane's running sum of the (bf16-rounded) P values
  __device__ __forceinline__ Softmax() : m(-INFINITY), thr(-INFINITY), mneg(0.f), l(0.f) {}
};

// S^T of a whole unit (two 32-key subtiles) with the K fragments read four
// MFMAs ahead of their use, so the LDS latency stays hidden behind the
// matrix ops already issued.
template <int D>
__device__ __forceinline__ void score_unit(const char* Ks, const bf16x8 (&qf)[D / 16], const ReadPlan<D>& rp,
                                           f32x16 (&s)[2]) {
  constexpr int NT = D / 16;        // k-steps per subtile
  constexpr int NI = 2 * NT;        // MFMAs of the unit
  constexpr int PF = 4;             // fragments in flight
  uint4 fr[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) fr[i] = rd16(rp.kp(Ks, i / NT, i % NT));
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint4 a = fr[i % PF];
    if (i + PF < NI) fr[i % PF] = rd16(rp.kp(Ks, (i + PF) / NT, (i + PF) % NT));
    s[i / NT] = mfma(as_bf16x8(a), qf[i % NT], s[i / NT]);
  }
  // keep that order: the scheduler would otherwise pull each read down to
  // just before its MFMA
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // PF LDS reads
#pragma unroll
  for (int i = 0; i + PF < NI; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
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

// Second half of a unit for one attention wavefront: the online softmax of
// its scores sc (two 32-key subtiles) and O^T += V^T P^T.  One max exchange
// and rescale test per 64 keys; P = exp2(S c - m c) with c = log2(e)/sqrt(d),
// rounded to bf16; l += sum of the rounded P (v_dot2 with ones).  The running
// max moves only when a unit max exceeds it by more than 2^8 in exp2 units,
// so P <= 2^8 and the O / l rescale is skipped for most units.  lim < 64
// marks a unit running past N: keys at offset >= lim get score -inf.
template <int D>
__device__ __forceinline__ void softmax_pv(const char* Vc, f32x16 (&sc)[2], f32x16 (&acc_o)[D / 32],
                                           Softmax& sm, const ReadPlan<D>& rp, int hi, int lim,
                                           float scale_log2, float thr8) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  // V^T fragments of the first key plane, read now so they land during the max
  bf16x8 vf[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) vf[dt] = rp.vt(Vc, dt, 0);
  if (lim < KU) {
    const int limh = lim - 4 * hi;  // key offset of element i of subtile h2: 32 h2 + 8 (i/4) + 4 hi + i%4
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * h2 + 8 * (i >> 2) + (i & 3) >= limh) sc[h2][i] = -INFINITY;
  }
  float mx = __builtin_elementwise_maximum(sc[0][0], sc[1][0]);
#pragma unroll
  for (int i = 1; i < 16; ++i)
    mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sc[0][i]), sc[1][i]);
  mx = pair_max(mx);
  if (__ballot(mx > sm.thr)) {
    const float m_new = fmaxf(sm.m, mx);
    const float corr = __builtin_amdgcn_exp2f((sm.m - m_new) * scale_log2);
    sm.l *= corr;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc_o[t] *= corr;
    sm.m = m_new;
    sm.mneg = -m_new * scale_log2;
    sm.thr = m_new + thr8;
  }
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    const int h2 = s4 >> 1, s = s4 & 1;
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[h2][8 * s + 2 * e], scale_log2, sm.mneg));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[h2][8 * s + 2 * e + 1], scale_log2, sm.mneg));
      pw[e] = pk_bf16(p0, p1);
      sm.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e]), ones, sm.l, false);
    }
    const bf16x8 bp = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const bf16x8 a = vf[dt];
      if (s4 + 1 < 4) vf[dt] = rp.vt(Vc, dt, s4 + 1);  // next key plane, one k-step ahead
      acc_o[dt] = mfma(a, bp, acc_o[dt]);
    }
  }
}

// Sparse (CSR row) or dense (every key block) softmax attention.  BQ/32
// wavefronts of 32 queries; two workgroups share a compute unit, so each SIMD
// holds one wavefront of each and the two interleave on their own.  The
// row's 64-key units stream through two LDS stages (K | V^T, distinct arrays,
// loop unrolled by two): unit b+1 loads while unit b is computed.  The load
// after the row's last unit repeats that unit, which keeps every step's count
// of loads fixed.
template <int D, int BQ, int SUB, int MODE>
__global__ __launch_bounds__(BQ / 32 * 64, 2) void attn_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int* __restrict__ row_ptr, const int* __restrict__ col_idx, uint16_t* __restrict__ O, int N,
    int Nq, int Nk, float scale_log2) {
  using T = Tiles<D>;
  constexpr int NW = BQ / 32;
  using LP = LoadPlan<D, NW>;
  constexpr int STAGE = 2 * T::KT_BYTES;
  static_assert(2 * STAGE <= LDS_BYTES / 2, "two workgroups per compute unit");
  // Two distinct LDS arrays: the compiler can then tell the loads into one
  // stage from the operand reads of the other.
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const ReadPlan<D> rdp(lane);
  const long long row = xcd_row(blockIdx.x, (long long)gridDim.x);
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  int nsel, base = 0;
  if (MODE == MODE_DENSE) {
    nsel = Nk;
  } else {
    base = row_ptr[row];
    nsel = row_ptr[row + 1] - base;
  }
  const int nunits = nsel * SUB;
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  const int q = qi * BQ + 32 * w + l32;
  bf16x8 qf[D / 16];
  load_q<D>(Q, bh, q, N, hi, qf);
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = f32x16{};
  Softmax sm;
  const float thr8 = 8.f / scale_log2;
  const LP lp(w, lane);
  const auto rk = buf_rsrc(Kb, (uint32_t)((size_t)N * D * 2));
  const auto rv = buf_rsrc(Vb, (uint32_t)((size_t)N * D * 2));

  // first key of unit x (clamped to the row's last unit)
  auto key0 = [&](int x) {
    const int xc = min(x, nunits - 1);
    const int blk = (MODE == MODE_DENSE) ? xc / SUB : col_idx[base + xc / SUB];
    return (blk * SUB + xc % SUB) * KU;
  };
  auto issue = [&](int k0x, char* sb) __attribute__((always_inline)) {
    lp.load_k(rk, k0x, sb);
    lp.load_r(rv, k0x, sb + T::KT_BYTES);
  };
  // kcur: first key of the unit being computed.  The next unit's column index
  // is read before the barrier, whose wait absorbs the scalar load, so the
  // LDS-read waits inside the step count LDS reads only.
  int kcur = nunits > 0 ? key0(0) : 0;
  auto step = [&](int b, char* cur, char* nxt) __attribute__((always_inline)) {
    const int knext = key0(b + 1);
    wait_vm<0>();     // this wavefront's loads of unit b have landed
    __syncthreads();  // ... and every wavefront's; unit b-1 consumed
    issue(knext, nxt);
    f32x16 sc[2];
    score_unit<D>(cur, qf, rdp, sc);
    softmax_pv<D>(cur + T::KT_BYTES, sc, acc_o, sm, rdp, hi, min(KU, N - kcur), scale_log2, thr8);
    kcur = knext;
  };
  if (nunits > 0) issue(kcur, st0);
  int b = 0;
  for (; b + 2 <= nunits; b += 2) {
    step(b, st0, st1);
    step(b + 1, st1, st0);
  }
  if (b < nunits) step(b, st0, st1);
  wait_vm<0>();  // no direct load outlives the workgroup

  const float lt = sm.l + __shfl_xor(sm.l, 32);
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

// S^T of the 32-key half KT of a unit (K tile Ks), K fragments read four
// MFMAs ahead (order pinned as in score_unit).
template <int D, int KT>
__device__ __forceinline__ f32x16 score_half(const char* Ks, const bf16x8 (&qf)[D / 16], const ReadPlan<D>& rp) {
  constexpr int NT = D / 16;
  constexpr int PF = 4;
  uint4 fr[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) fr[i] = rd16(rp.kp(Ks, KT, i));
  f32x16 s = f32x16{};
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const uint4 a = fr[i % PF];
    if (i + PF < NT) fr[i % PF] = rd16(rp.kp(Ks, KT, i + PF));
    s = mfma(as_bf16x8(a), qf[i], s);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
  for (int i = 0; i + PF < NT; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
  return s;
}

// G tiles of one wavefront in the fused kernel: TPW 32 x 32 tiles of the D x D
// product phi(K)^T V; tile u is (row tile mt, column tile nt).  When a
// wavefront has at least a full row of tiles the column tile is a constant.
template <int D, int TPW>
struct GTiles {
  static constexpr int NCT = D / 32;                    // column tiles per row
  __device__ static int mt(int wq, int u) { return (wq * TPW + u) / NCT; }
  __device__ static int nt(int wq, int u) { return TPW >= NCT ? u % NCT : (wq * TPW + u) % NCT; }
};

// B operand of a G tile: the V^T fragment of column tile nt (a register array
// index, so a constant nt folds and a wave-uniform one selects).
template <int D>
__device__ __forceinline__ bf16x8 pick_frag(const bf16x8 (&vf)[D / 32], int nt) {
  bf16x8 b = vf[0];
#pragma unroll
  for (int c = 1; c < D / 32; ++c)
    if (nt == c) b = vf[c];
  return b;
}

// Linear-branch preparation of one head's chunk of key blocks (one
// workgroup, four wavefronts): phi(K) = elu(K) + 1 rounded to bf16 in the
// layout of K (keys below N), the column sums of phi(K) over every key block
// (float32), and the chunk's partial totals H = sum_u phi(k_u)^T v_u and
// z = sum_u phi(k_u).  64-key units of K and V stream through two LDS stages
// (row-major tiles in the transposed-read layout).  Wavefront w owns the G
// tiles of the attention kernels' split (the d_k row tile mt = GTiles::mt(w, .)):
// its phi(K)^T operand is read transposed from the K tile with phi applied in
// fp32 and split into bf16 hi + lo (H keeps ~16 mantissa bits), and the V^T
// operand is read transposed from the V tile.  Heads whose alpha is exactly 1
// are skipped when alpha is given.
template <int D, int BK>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ K,
                                                   const uint16_t* __restrict__ V,
                                                   const float* __restrict__ alpha, int H, int N, int Nk,
                                                   int chunk_blocks, int nchunk, uint16_t* __restrict__ pk_g,
                                                   float* __restrict__ zblk, float* __restrict__ hpart) {
  using T = Tiles<D>;
  using LP = LoadPlan<D, 4>;
  constexpr int SUB = BK / KU;                  // units per key block
  constexpr int TT = (D / 32) * (D / 32);
  constexpr int TPW = TT / 4;                   // H tiles per wavefront
  using GT = GTiles<D, TPW>;
  constexpr int PCH = KU * (D / 8) / 256;       // 16-byte phi(K) chunks per thread and unit
  __shared__ __attribute__((aligned(16))) char k0[T::KT_BYTES];
  __shared__ __attribute__((aligned(16))) char k1[T::KT_BYTES];
  __shared__ __attribute__((aligned(16))) char v0[T::KT_BYTES];
  __shared__ __attribute__((aligned(16))) char v1[T::KT_BYTES];

  const long long bh = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  if (alpha != nullptr && alpha[bh % H] == 1.f) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const ReadPlan<D> rdp(lane);
  const LP lp(w, lane);
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  uint16_t* Pb = pk_g + (size_t)bh * N * D;
  const auto rk = buf_rsrc(Kb, (uint32_t)((size_t)N * D * 2));
  const auto rv = buf_rsrc(Vb, (uint32_t)((size_t)N * D * 2));
  const int jb = chunk * chunk_blocks, je = min(Nk, jb + chunk_blocks);
  const int nun = max(0, je - jb) * SUB;        // units of the chunk
  const int mt = GT::mt(w, 0);                  // the d_k row tile of this wavefront
  const bool zown = TPW >= D / 32 || GT::nt(w, 0) == 0;  // one wavefront per row tile keeps z

  f32x16 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
  float zblock = 0.f, zpart = 0.f;

  auto step = [&](int x, const char* ks, const char* vs, char* nks, char* nvs) __attribute__((always_inline)) {
    wait_vm<0>();     // this wavefront's loads of unit x have landed
    __syncthreads();  // ... and every wavefront's; unit x-1 consumed
    if (x + 1 < nun) {
      const int kn = (jb * SUB + x + 1) * KU;
      lp.load_r(rk, kn, nks);
      lp.load_r(rv, kn, nvs);
    }
    const int key0 = (jb * SUB + x) * KU;
    const int lim = min(KU, N - key0);          // keys of the unit below N
    // phi(K) rows to global memory
#pragma unroll
    for (int c = 0; c < PCH; ++c) {
      const int ch = tid + 256 * c;
      const int r = ch / (D / 8), cc = ch % (D / 8);
      const uint4 kv = rd16(ks + (cc >> 3) * T::KHALF + r * 128 + 16 * ((cc & 7) ^ swv(r)));
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pk_bf16(phi(bf2f(elem(kv, 2 * e))), phi(bf2f(elem(kv, 2 * e + 1))));
      if (r < lim) *reinterpret_cast<uint4*>(Pb + (size_t)(key0 + r) * D + 8 * cc) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    // H += phi(K)^T V (hi + lo) and z over the 4 key planes of the unit
#pragma unroll
    for (int pl = 0; pl < KU / 16; ++pl) {
      const uint4 kt = __builtin_bit_cast(uint4, rdp.vt(ks, mt, pl));
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of the fragment is key 16 pl + 4 hi + (e & 3) + 8 (e >> 2) of the unit
        const int key = 16 * pl + 4 * hi + (e & 3) + 8 * (e >> 2);
        f[e] = key < lim ? phi(bf2f(elem(kt, e))) : 0.f;
        zblock += f[e];
      }
      uint32_t fh[4], fl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        fh[e] = pk_bf16(f[2 * e], f[2 * e + 1]);
        fl[e] = pk_bf16(f[2 * e] - bf2f(fh[e] & 0xffffu), f[2 * e + 1] - bf2f(fh[e] >> 16));
      }
      const bf16x8 ah = as_bf16x8(make_uint4(fh[0], fh[1], fh[2], fh[3]));
      const bf16x8 al = as_bf16x8(make_uint4(fl[0], fl[1], fl[2], fl[3]));
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const bf16x8 b = rdp.vt(vs, GT::nt(w, u), pl);
        acc[u] = mfma(ah, b, acc[u]);
        acc[u] = mfma(al, b, acc[u]);
      }
    }
    if ((x + 1) % SUB == 0) {  // the key block ends: its phi(K) column sums
      const float zb = zblock + __shfl_xor(zblock, 32);
      if (zown && hi == 0) zblk[((size_t)bh * Nk + jb + x / SUB) * D + 32 * mt + l32] = zb;
      zpart += zb;
      zblock = 0.f;
    }
  };
  if (nun > 0) {
    lp.load_r(rk, jb * SUB * KU, k0);
    lp.load_r(rv, jb * SUB * KU, v0);
  }
  int x = 0;
  for (; x + 2 <= nun; x += 2) {
    step(x, k0, v0, k1, v1);
    step(x + 1, k1, v1, k0, v0);
  }
  if (x < nun) step(x, k0, v0, k1, v1);
  wait_vm<0>();

  float* out = hpart + ((size_t)bh * nchunk + chunk) * (D * D + D);
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int nt = GT::nt(w, u);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int dk = 32 * mt + 8 * (i >> 2) + 4 * hi + (i & 3);
      out[dk * D + 32 * nt + l32] = acc[u][i];
    }
  }
  if (zown && hi == 0) out[D * D + 32 * mt + l32] = zpart;
}

// One fused-kernel wavefront's share of a unit: keys [32 KT, 32 KT + 32),
// i.e. key planes 2 KT and 2 KT + 1 of the V^T / phi(K)^T tiles.
//   DO_S: online softmax of its scores sc (lim = keys of the unit below N)
//         and O^T += V^T P^T, as in softmax_pv but over 32 keys;
//   DO_G: G += phi(K)^T V for its G tiles; the V^T fragments read for the
//         P V product serve as the B operand, and these matrix ops do not
//         wait for the softmax.
template <int D, int TPW, int KT, bool DO_S, bool DO_G>
__device__ __forceinline__ void fused_half(const char* Vt, const char* Pk, f32x16& sc, f32x16 (&acc_o)[D / 32],
                                           Softmax& sm, f32x16 (&acc_g)[TPW], const ReadPlan<D>& rp, int wq,
                                           int hi, int lim, float scale_log2, float thr8) {
  using GT = GTiles<D, TPW>;
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  bf16x8 vf[2][D / 32];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) vf[j][dt] = rp.vt(Vt, dt, 2 * KT + j);
  if (DO_G) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const bf16x8 a = rp.vt(Pk, GT::mt(wq, u), 2 * KT + j);
        acc_g[u] = mfma(a, pick_frag<D>(vf[j], GT::nt(wq, u)), acc_g[u]);
      }
  }
  if (!DO_S) return;
  if (lim < 32 * KT + 32) {
    const int limh = lim - 32 * KT - 4 * hi;  // key offset of element i: 32 KT + 8 (i/4) + 4 hi + i%4
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + (i & 3) >= limh) sc[i] = -INFINITY;
  }
  float mx = __builtin_elementwise_maximum(sc[0], sc[1]);
#pragma unroll
  for (int i = 2; i < 16; i += 2)
    mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, sc[i]), sc[i + 1]);
  mx = pair_max(mx);
  if (__ballot(mx > sm.thr)) {
    const float m_new = fmaxf(sm.m, mx);
    const float corr = __builtin_amdgcn_exp2f((sm.m - m_new) * scale_log2);
    sm.l *= corr;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc_o[t] *= corr;
    sm.m = m_new;
    sm.mneg = -m_new * scale_log2;
    sm.thr = m_new + thr8;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[8 * j + 2 * e], scale_log2, sm.mneg));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[8 * j + 2 * e + 1], scale_log2, sm.mneg));
      pw[e] = pk_bf16(p0, p1);
      sm.l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[e]), ones, sm.l, false);
    }
    const bf16x8 bp = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc_o[dt] = mfma(vf[j][dt], bp, acc_o[dt]);
  }
}

// Fused sparse + linear (+ alpha mix) over the CSR row.  2*BQ/32 wavefronts in
// two groups; wavefront i of either group owns queries [32 i, 32 i + 32) of
// the query block, and group g takes keys [32 g, 32 g + 32) of every 64-key
// unit of the row: its half of S = K Q^T, the online softmax over those keys
// with O^T += V^T P^T, and its share of G = sum phi(K)^T V over them (the
// V^T fragments of P V reused as the B operand, one phi(K)^T read per key
// plane).  Units stream through a ring of NS LDS stages (K | V^T | phi(K)^T |
// the block's phi sums; distinct arrays, loop unrolled by NS), NS-1 units
// ahead.  Afterwards the two wavefronts of a query slice swap halves of their
// partials through LDS: each merges the two softmax partials over half of the
// d range and sums the two G partials over half of its G tiles; the G halves
// become H_u = H - G (hi + lo bf16) in LDS, and each wavefront applies H_u to
// phi(Q) for its half of d and mixes the branches into the output.
template <int D, int BQ, int SUB, int MODE>
__global__ __launch_bounds__(BQ / 32 * 128, 1) void fused_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ pk_g, const float* __restrict__ zblk, const int* __restrict__ row_ptr,
    const int* __restrict__ col_idx, const float* __restrict__ alpha, const float* __restrict__ htot,
    uint16_t* __restrict__ O, int H, int N, int Nq, int Nk, float scale_log2) {
  using T = Tiles<D>;
  constexpr int NA = BQ / 32;                    // wavefronts per group
  constexpr int NWT = 2 * NA;                    // all wavefronts
  constexpr int TT = (D / 32) * (D / 32);        // G tiles
  constexpr int TPW = TT / NA;                   // G tiles per wavefront (each group covers all)
  static_assert(TPW * NA == TT, "G tiles split");
  using GT = GTiles<D, TPW>;
  using LP = LoadPlan<D, NWT>;
  constexpr bool LOADK = MODE != MODE_LINEAR;    // the softmax branch needs K
  constexpr int OFF_V = LOADK ? T::KT_BYTES : 0; // V^T tile
  constexpr int OFF_P = OFF_V + T::KT_BYTES;     // phi(K) tile
  constexpr int OFF_Z = OFF_P + T::KT_BYTES;     // sum of phi(k) over the block's keys
  constexpr int STAGE = OFF_Z + D * 4;
  constexpr int HU_HALF = D * D * 2;             // H_u^T hi (or lo) part, bf16
  constexpr int NS = 3;
  // epilogue exchange areas: softmax halves in stages 0 / 1, G halves in stage 2
  constexpr int SXB = ((D / 64) * 16 + 2) * 64 * 4;           // one softmax half (O tiles + m, l)
  constexpr int PPS = STAGE / (2 * SXB);                      // query slices per stage
  constexpr int GXT = TPW >= 2 ? TPW / 2 : 1;                  // G tiles sent per wavefront
  constexpr int GXB = GXT * 16 * 64 * 2;                      // their bf16 bytes
  static_assert(NS * STAGE + D * 4 <= LDS_BYTES, "LDS");
  static_assert(HU_HALF <= STAGE && NA * 2 * GXB <= STAGE && (!LOADK || (PPS >= 1 && 2 * PPS >= NA)),
                "epilogue areas");
  // direct loads per unit of each wavefront; the last wavefront also brings
  // the block's phi sums (D floats, D/64 four-byte loads)
  constexpr int NL = (LOADK ? LP::NK : 0) + 2 * LP::NK;
  constexpr int NLZ = NL + D / 64;
  static_assert((NS - 1) * NLZ < 64, "vmcnt");
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  __shared__ __attribute__((aligned(16))) char st2[STAGE];
  __shared__ float zu[D];
  char* HuHi = st0;
  char* HuLo = st1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w / NA, wq = w % NA;
  const int l32 = lane & 31, hi = lane >> 5;
  const bool zwave = w == NWT - 1;
  const int lb = lane_base(lane);
  const ReadPlan<D> rdp(lane);
  const long long row = xcd_row(blockIdx.x, (long long)gridDim.x);
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  const int h = (int)(bh % H);
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
  const int nunits = (do_s || lin) ? nsel * SUB : 0;

  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  const uint16_t* Pkb = pk_g + (size_t)bh * N * D;
  const float* Zb = zblk + (size_t)bh * Nk * D;
  const float* Hh = htot + (size_t)bh * (D * D + D);
  const LP lp(w, lane);
  const auto rk = buf_rsrc(Kb, (uint32_t)((size_t)N * D * 2));
  const auto rv = buf_rsrc(Vb, (uint32_t)((size_t)N * D * 2));
  const auto rp = buf_rsrc(Pkb, (uint32_t)((size_t)N * D * 2));
  const auto rz = buf_rsrc(Zb, (uint32_t)((size_t)Nk * D * 4));

  auto stage = [&](int i) -> char* {
    i %= NS;
    return i == 0 ? st0 : i == 1 ? st1 : st2;
  };
  // listed block of unit x and its first key (x clamped to the row's last unit)
  auto blk_of = [&](int x) { return col_idx[base + min(x, nunits - 1) / SUB]; };
  auto key0 = [&](int x) {
    const int xc = min(x, nunits - 1);
    return (col_idx[base + xc / SUB] * SUB + xc % SUB) * KU;
  };
  auto issue = [&](int x, char* sb) __attribute__((always_inline)) {
    const int k0x = key0(x);
    if (LOADK) lp.load_k(rk, k0x, sb);
    lp.load_r(rv, k0x, sb + OFF_V);
    lp.load_r(rp, k0x, sb + OFF_P);
    if (zwave) {
      const uint32_t zoff = (uint32_t)blk_of(x) * (D * 4);
#pragma unroll
      for (int c = 0; c < D / 64; ++c) b2lds4(rz, (uint32_t)(64 * c + lane) * 4, zoff, sb + OFF_Z + 256 * c);
    }
  };

  // per-wavefront state
  const int q = qi * BQ + 32 * wq + l32;
  bf16x8 qf[D / 16];
  load_q<D>(Q, bh, q, N, hi, qf);
  f32x16 acc_o[D / 32], acc_g[TPW];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = f32x16{};
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc_g[t] = f32x16{};
  Softmax sm;
  const float thr8 = 8.f / scale_log2;
  const int zd = wq * 64 + lane;  // group 0: the d of g this lane keeps
  float gsum = 0.f;

  // The unit loop: every wavefront issues its share of the loads and passes
  // the same barriers; work(I, b, cur) is the per-unit computation.
  auto run_loop = [&](auto&& work) __attribute__((always_inline)) {
    if (nunits > 0) {
#pragma unroll
      for (int i = 0; i < NS - 1; ++i) issue(i, stage(i));
    }
    auto step = [&](auto rt, int b) __attribute__((always_inline)) {
      constexpr int r = decltype(rt)::value;
      if (b + 1 < nunits) {
        if (zwave) wait_vm<(NS - 2) * NLZ>(); else wait_vm<(NS - 2) * NL>();
      } else {
        wait_vm<0>();
      }
      __syncthreads();
      if (b + NS - 1 < nunits) issue(b + NS - 1, stage(r + NS - 1));
      work(rt, b, stage(r));
    };
    for (int b = 0; b < nunits; b += NS) {
      step(IntTag<0>{}, b);
      if (b + 1 < nunits) step(IntTag<1>{}, b + 1);
      if (b + 2 < nunits) step(IntTag<2>{}, b + 2);
    }
    __syncthreads();  // every wavefront is done with the loop tiles
  };
  // per-unit work of group KT with the branch flags known
  auto make_work = [&](auto kt_tag, auto s_tag, auto g_tag) {
    constexpr int KT_ = decltype(kt_tag)::value;
    constexpr bool S_ = decltype(s_tag)::value != 0, G_ = decltype(g_tag)::value != 0;
    return [&](auto rt, int b, const char* cur) __attribute__((always_inline)) {
      constexpr int r = decltype(rt)::value;
      f32x16 sc;
      if (S_) sc = score_half<D, KT_>(cur, qf, rdp);
      const int lim = S_ ? min(KU, N - key0(b)) : KU;
      fused_half<D, TPW, KT_, S_, G_>(cur + OFF_V, cur + OFF_P, sc, acc_o, sm, acc_g, rdp, wq, hi, lim,
                                       scale_log2, thr8);
      // the block's phi sums count once: group 0, first unit of the block (3 is a multiple of SUB
      // or SUB is 1... the unit index b decides)
      if (G_ && KT_ == 0 && zd < D && (b % SUB) == 0) gsum += reinterpret_cast<const float*>(cur + OFF_Z)[zd];
      (void)r;
    };
  };
  // the whole per-wavefront program, with the group index G as a constant
  auto body = [&](auto g_tag) __attribute__((always_inline)) {
  constexpr int G = decltype(g_tag)::value;
  if (do_s && lin) run_loop(make_work(g_tag, IntTag<1>{}, IntTag<1>{}));
  else if (do_s) run_loop(make_work(g_tag, IntTag<1>{}, IntTag<0>{}));
  else if (lin) run_loop(make_work(g_tag, IntTag<0>{}, IntTag<1>{}));
  else run_loop(make_work(g_tag, IntTag<0>{}, IntTag<0>{}));

  // ---- epilogue: swap halves of the partials within each query slice
  constexpr int HT = D / 64;     // O tiles per half of d
  constexpr int own0 = G * HT;   // first O tile this wavefront finishes
  constexpr int NTQ = D / 16;    // k-steps of phi(Q)
  constexpr int TQ0 = G * (NTQ / 2);                        // the phi(Q) k-steps this wavefront computes
  constexpr int PQB = (NTQ / 2) * 2 * 1024 + 256;           // its shared phi(Q) hi / lo fragments + dpart
  constexpr int PQ_S2 = STAGE / PQB, PQ_T = (STAGE - HU_HALF) / PQB;
  constexpr bool PQ_SHARE = PQ_S2 + 2 * PQ_T >= NWT;         // else each wavefront computes all of phi(Q)
  auto pq_slot = [&](int k) -> char* {  // phi(Q) share slot of wavefront (k / 2, group k % 2)
    if (k < PQ_S2) return st2 + k * PQB;
    k -= PQ_S2;
    if (k < PQ_T) return st0 + HU_HALF + k * PQB;
    k -= PQ_T;
    return st1 + HU_HALF + k * PQB;
  };
  // (A) hand the partner the halves it finishes: O tiles and (m, l) of the
  // softmax partial, G tiles (bf16); group 0 also sets z_u = z - g
  {
    char* sx = (wq / (PPS > 0 ? PPS : 1) == 0 ? st0 : st1) + (wq % (PPS > 0 ? PPS : 1)) * 2 * SXB;
    if (LOADK) {
      uint4* mine = reinterpret_cast<uint4*>(sx + G * SXB);
#pragma unroll
      for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const f32x16& a = acc_o[(1 - G) * HT + t];
          mine[(4 * t + e4) * 64 + lane] = make_uint4(__float_as_uint(a[4 * e4]), __float_as_uint(a[4 * e4 + 1]),
                                                      __float_as_uint(a[4 * e4 + 2]), __float_as_uint(a[4 * e4 + 3]));
        }
      reinterpret_cast<float2*>(sx + G * SXB + 16 * HT * 64 * 4)[lane] = make_float2(sm.m, sm.l);
    }
    if (lin && (TPW >= 2 || G == 1)) {
      uint4* gx = reinterpret_cast<uint4*>(st2 + wq * 2 * GXB + G * GXB);
      const int u0 = TPW >= 2 ? (1 - G) * GXT : 0;  // first G tile the partner finishes
#pragma unroll
      for (int t = 0; t < GXT; ++t)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const f32x16& a = acc_g[u0 + t];
          gx[(2 * t + h8) * 64 + lane] =
              make_uint4(pk_bf16(a[8 * h8], a[8 * h8 + 1]), pk_bf16(a[8 * h8 + 2], a[8 * h8 + 3]),
                         pk_bf16(a[8 * h8 + 4], a[8 * h8 + 5]), pk_bf16(a[8 * h8 + 6], a[8 * h8 + 7]));
        }
    }
    if (lin && G == 0 && zd < D) zu[zd] = Hh[D * D + zd] - gsum;
  }
  __syncthreads();
  // (B) merge the partner's halves into this wavefront's halves
  float l_all = 0.f;
  {
    const char* sx = (wq / (PPS > 0 ? PPS : 1) == 0 ? st0 : st1) + (wq % (PPS > 0 ? PPS : 1)) * 2 * SXB;
    if (LOADK) {
      const uint4* theirs = reinterpret_cast<const uint4*>(sx + (1 - G) * SXB);
      const float2 ml = reinterpret_cast<const float2*>(sx + (1 - G) * SXB + 16 * HT * 64 * 4)[lane];
      const float m = fmaxf(sm.m, ml.x);
      float c0 = 0.f, c1 = 0.f;
      if (m != -INFINITY) {
        c0 = __builtin_amdgcn_exp2f((sm.m - m) * scale_log2);
        c1 = __builtin_amdgcn_exp2f((ml.x - m) * scale_log2);
      }
      l_all = sm.l * c0 + ml.y * c1;
#pragma unroll
      for (int t = 0; t < HT; ++t)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const uint4 v = theirs[(4 * t + e4) * 64 + lane];
          f32x16& a = acc_o[own0 + t];
          a[4 * e4] = a[4 * e4] * c0 + __uint_as_float(v.x) * c1;
          a[4 * e4 + 1] = a[4 * e4 + 1] * c0 + __uint_as_float(v.y) * c1;
          a[4 * e4 + 2] = a[4 * e4 + 2] * c0 + __uint_as_float(v.z) * c1;
          a[4 * e4 + 3] = a[4 * e4 + 3] * c0 + __uint_as_float(v.w) * c1;
        }
    }
    if (lin && (TPW >= 2 || G == 0)) {
      const uint4* gx = reinterpret_cast<const uint4*>(st2 + wq * 2 * GXB + (1 - G) * GXB);
      const int u0 = TPW >= 2 ? G * GXT : 0;
#pragma unroll
      for (int t = 0; t < GXT; ++t)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
          const uint4 v = gx[(2 * t + h8) * 64 + lane];
          f32x16& a = acc_g[u0 + t];
          const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            a[8 * h8 + 2 * c] += bf2f(w4[c] & 0xffffu);
            a[8 * h8 + 2 * c + 1] += bf2f(w4[c] >> 16);
          }
        }
    }
  }
  __syncthreads();  // exchange areas read; stages 0 / 1 take H_u
  // (C) H_u^T = (H - G)^T for this wavefront's G tiles as hi + lo bf16 planes
  // (rows d_v, 16-wide d_k slices), and phi(Q) (hi + lo) of its k-steps
  uint4 qh[NTQ], ql[NTQ];
  float dpart = 0.f;
  if (lin) {
#pragma unroll
    for (int t = 0; t < GXT; ++t) {
      if (TPW < 2 && G != 0) break;
      const int u = TPW >= 2 ? G * GXT + t : 0;
      const int mt = GT::mt(wq, u), nt = GT::nt(wq, u);
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
    // phi(Q) of k-step t: 8 values per lane, split into bf16 hi + lo; dpart = phi(Q) . z_u
    auto phiq = [&](int t) __attribute__((always_inline)) {
      const uint4 qv = __builtin_bit_cast(uint4, qf[t]);
      const float4 z0 = *reinterpret_cast<const float4*>(zu + 16 * t + 8 * hi);
      const float4 z1 = *reinterpret_cast<const float4*>(zu + 16 * t + 8 * hi + 4);
      const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
      float f[8], fl[8];
      uint32_t fh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f[e] = phi(bf2f(elem(qv, e)));
        fh[e] = pk_bf16(f[e], 0.f) & 0xffffu;
        fl[e] = f[e] - bf2f(fh[e]);
        dpart = fmaf(f[e], zz[e], dpart);
      }
      qh[t] = make_uint4(fh[0] | (fh[1] << 16), fh[2] | (fh[3] << 16), fh[4] | (fh[5] << 16), fh[6] | (fh[7] << 16));
      ql[t] = make_uint4(pk_bf16(fl[0], fl[1]), pk_bf16(fl[2], fl[3]), pk_bf16(fl[4], fl[5]), pk_bf16(fl[6], fl[7]));
    };
    if (PQ_SHARE) {
      uint4* sh = reinterpret_cast<uint4*>(pq_slot(2 * wq + G));
#pragma unroll
      for (int i = 0; i < NTQ / 2; ++i) {
        phiq(TQ0 + i);
        sh[(2 * i) * 64 + lane] = qh[TQ0 + i];
        sh[(2 * i + 1) * 64 + lane] = ql[TQ0 + i];
      }
      reinterpret_cast<float*>(pq_slot(2 * wq + G) + (NTQ / 2) * 2 * 1024)[lane] = dpart;
    } else {
#pragma unroll
      for (int t = 0; t < NTQ; ++t) phiq(t);
    }
    __syncthreads();  // H_u^T and the shared phi(Q) complete
  }

  float inv_l = 0.f;
  if (do_s) {
    const float lt = l_all + __shfl_xor(l_all, 32);
    inv_l = lt > 0.f ? 1.f / lt : 0.f;
  }
  // (D) num^T = H_u^T phi(Q)^T over this wavefront's half of d
  f32x16 acc_n[HT];
#pragma unroll
  for (int t = 0; t < HT; ++t) acc_n[t] = f32x16{};
  float den = 1.f;
  if (lin) {
    if (PQ_SHARE) {
      const uint4* sh = reinterpret_cast<const uint4*>(pq_slot(2 * wq + (1 - G)));
      constexpr int TP0 = (1 - G) * (NTQ / 2);
#pragma unroll
      for (int i = 0; i < NTQ / 2; ++i) {
        qh[TP0 + i] = sh[(2 * i) * 64 + lane];
        ql[TP0 + i] = sh[(2 * i + 1) * 64 + lane];
      }
      dpart += reinterpret_cast<const float*>(pq_slot(2 * wq + (1 - G)) + (NTQ / 2) * 2 * 1024)[lane];
    }
#pragma unroll
    for (int t = 0; t < NTQ; ++t) {
#pragma unroll
      for (int mt = 0; mt < HT; ++mt) {
        const uint4 ah = rd16(HuHi + t * T::HPB + (own0 + mt) * 1024 + lb);
        const uint4 al = rd16(HuLo + t * T::HPB + (own0 + mt) * 1024 + lb);
        acc_n[mt] = mfma(as_bf16x8(ah), as_bf16x8(qh[t]), acc_n[mt]);
        acc_n[mt] = mfma(as_bf16x8(ah), as_bf16x8(ql[t]), acc_n[mt]);
        acc_n[mt] = mfma(as_bf16x8(al), as_bf16x8(qh[t]), acc_n[mt]);
      }
    }
    den = dpart + __shfl_xor(dpart, 32);
  }
  const float wl_den = lin ? wl_ / den : 0.f;
  const float ws_l = ws_ * inv_l;
  // each 16-byte store holds 8 consecutive d of one query: lanes l and l^32
  // hold the two 4-d halves of every 8-d chunk and swap one of them
  if (q < N) {
    const size_t orow = ((size_t)bh * N + q) * D;
#pragma unroll
    for (int mt = 0; mt < HT; ++mt)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint2 pv[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int i4 = 2 * j + c;
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = ws_l * acc_o[own0 + mt][4 * i4 + r] + wl_den * acc_n[mt][4 * i4 + r];
          pv[c] = make_uint2(pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3]));
        }
        // lane hi = 0 keeps chunk i4 = 2j (needs the partner's pv[0]); hi = 1 keeps 2j + 1 (needs pv[1])
        const uint2 send = hi ? pv[0] : pv[1];
        const uint2 recv = make_uint2(__shfl_xor(send.x, 32), __shfl_xor(send.y, 32));
        const uint4 outv = hi ? make_uint4(recv.x, recv.y, pv[1].x, pv[1].y)
                              : make_uint4(pv[0].x, pv[0].y, recv.x, recv.y);
        *reinterpret_cast<uint4*>(O + orow + 32 * (own0 + mt) + 16 * j + 8 * hi) = outv;
      }
  }
  };
  if (grp == 0) body(IntTag<0>{});
  else body(IntTag<1>{});
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
hipError_t prep_dispatch(const Shape& s, const void* K, const void* V, const float* alpha, char* ws,
                         const WsLayout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H;
  const dim3 grid((unsigned)(BH * L.nchunk)), block(256);
  uint16_t* pk = reinterpret_cast<uint16_t*>(ws + L.pk);
  float* zb = reinterpret_cast<float*>(ws + L.zblk);
  float* hpart = reinterpret_cast<float*>(ws + L.hpart);
  hipLaunchKernelGGL((prep_kernel<D, BK>), grid, block, 0, st, static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), alpha, s.H, s.N, s.Nk, L.chunk_blocks, L.nchunk, pk,
                     zb, hpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_summary_reduce(hpart, alpha, s.H, BH, L.nchunk, D * D + D,
                               reinterpret_cast<float*>(ws + L.htot), st);
}

template <int D, int BQ, int SUB>
hipError_t attn_dispatch(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                         const int32_t* rp, const int32_t* ci, const float* alpha, const char* ws,
                         const WsLayout& L, void* O, hipStream_t st) {
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(K);
  const uint16_t* vt = static_cast<const uint16_t*>(V);
  const uint16_t* pk = reinterpret_cast<const uint16_t*>(ws + L.pk);
  const float* zb = reinterpret_cast<const float*>(ws + L.zblk);
  const float* ht = reinterpret_cast<const float*>(ws + L.htot);
  uint16_t* o = static_cast<uint16_t*>(O);
  const dim3 grid((unsigned)s.R());
  switch (mode) {
    case MODE_SPARSE:
      hipLaunchKernelGGL((attn_kernel<D, BQ, SUB, MODE_SPARSE>), grid, dim3(BQ / 32 * 64), 0, st, q, k, vt,
                         rp, ci, o, s.N, s.Nq, s.Nk, sl2);
      break;
    case MODE_DENSE:
      hipLaunchKernelGGL((attn_kernel<D, BQ, SUB, MODE_DENSE>), grid, dim3(BQ / 32 * 64), 0, st, q, k, vt,
                         rp, ci, o, s.N, s.Nq, s.Nk, sl2);
      break;
    case MODE_LINEAR:
      hipLaunchKernelGGL((fused_kernel<D, BQ, SUB, MODE_LINEAR>), grid, dim3(BQ / 32 * 128), 0, st, q, k,
                         vt, pk, zb, rp, ci, alpha, ht, o, s.H, s.N, s.Nq, s.Nk, sl2);
      break;
    default:
      hipLaunchKernelGGL((fused_kernel<D, BQ, SUB, MODE_FUSED>), grid, dim3(BQ / 32 * 128), 0, st, q, k,
                         vt, pk, zb, rp, ci, alpha, ht, o, s.H, s.N, s.Nq, s.Nk, sl2);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_bf16(const Shape& s, bool lin, const void* K, const void* V, const float* alpha,
                            char* ws, const WsLayout& L, hipStream_t st) {
  if (!lin) return hipSuccess;  // the softmax kernels read K and V as they are
  if (s.d == 128 && s.bk == 64) return prep_dispatch<128, 64>(s, K, V, alpha, ws, L, st);
  if (s.d == 128 && s.bk == 128) return prep_dispatch<128, 128>(s, K, V, alpha, ws, L, st);
  if (s.d == 64 && s.bk == 64) return prep_dispatch<64, 64>(s, K, V, alpha, ws, L, st);
  if (s.d == 64 && s.bk == 128) return prep_dispatch<64, 128>(s, K, V, alpha, ws, L, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bf16(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                            const int32_t* rp, const int32_t* ci, const float* alpha, const char* ws,
                            const WsLayout& L, void* O, hipStream_t st) {
#define SLA_ATTN(DD, QQ, KK)                                                  \
  if (s.d == DD && s.bq == QQ && s.bk == KK)                                  \
    return attn_dispatch<DD, QQ, KK / 64>(s, mode, Q, K, V, rp, ci, alpha, ws, L, O, st);
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
