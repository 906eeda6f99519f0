// Device helpers shared by the bf16 attention kernels (forward and
// backward): matrix-core operand layouts, the swizzled LDS tile of a 64-key
// unit (K or V, row-major, 16-byte chunks XOR-swizzled by key), direct
// global-to-LDS loads, row and transposed operand reads, and the score loops.
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16): lane l supplies operand
// row / column l%32 and a k-slice 8*(l/32) .. +7; accumulator element i of
// lane l is row 8*(i/4) + 4*(l/32) + i%4, column l%32.
#pragma once

#include <utility>

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

// f(IntTag<0>{}), ..., f(IntTag<N - 1>{}) in order (compile-time indices)
template <class F, int... I>
__device__ __forceinline__ void for_each_tag(F&& f, std::integer_sequence<int, I...>) {
  (f(IntTag<I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  for_each_tag(f, std::make_integer_sequence<int, N>{});
}

// Lane N of v's 16-lane row, in every lane of that row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(N >= 0 && N < 16, "row lane");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xf, 0xf,
                                                               false));
}

// Per-query values of a 32-query accumulator tile, one value per lane: the
// lane that holds query term_query(l) of the tile.  Accumulator element i of
// lane l belongs to query 8 (i/4) + 4 (l/32) + i%4, and lanes 16 r .. 16 r + 15
// share l/32, so element i takes lane i of its row (row_bcast<i>).
__device__ __forceinline__ int term_query(int lane) {
  return 8 * ((lane & 15) >> 2) + (lane & 3) + 4 * (lane >> 5);
}

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
// blocks, so their K / V tiles are then shared in one L2.
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

// LDS tile layout of one 64-key unit of K or V.  Every direct load instruction
// brings 64 x 16 bytes that land in LDS in lane order, so a tile is stored as
// rows of whole 128-byte global lines - [D/64 halves][64 keys][128 B],
// row-major as in memory - and each load covers 8 complete lines.  Inside a
// row, 16-byte chunk c of key r sits at c ^ sw(r), sw(r) = f((r >> 1) & 7)
// with f(b) = 4 (b & 1) + (b >> 1):
//   * the 16 keys that a 16-lane group reads for one S operand (one chunk
//     each) hit 16 distinct bank groups (f is a permutation of 0..7);
//   * the 4 keys x 64 bytes of one transposed read by 32 lanes hit 64
//     distinct banks (keys r and r + 2 differ in bit 2 of sw).
// H_u^T (written with ordinary LDS stores after the loop) keeps a "plane"
// layout: every 16-element k-slice is a plane of 32 bytes per row, the two
// 16-byte halves swapped when bit 3 of the row is set.
template <int D>
struct Tiles {
  static constexpr int KHALF = KU * 128;       // bytes of one 64-d half of a tile
  static constexpr int KT_BYTES = KU * D * 2;  // one [64 keys x D] tile
  static constexpr int HPB = D * 32;           // bytes of one H_u^T plane (16 d_k)
};

__device__ __forceinline__ int sw(int r) {
  const int b = (r >> 1) & 7;
  return ((b & 1) << 2) | (b >> 1);
}

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

__device__ __forceinline__ bf16x8 cat_tr(const char* a, const char* b) {
  const s16x4 x = tr16(a), y = tr16(b);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Per-lane byte offsets of the MFMA operand reads (lane l: row l%32 of a
// 32-row tile, k-slice half l/32).
//   K (S operand): the 16-wide d step t of key subtile kt at (t/4) KHALF +
//     4096 kt + off[t%4] (one 16-byte read).
//   V^T / phi(K)^T (transposed reads of a row-major tile): rows d = 32 dt +
//     l%32, the 8 keys of key plane pl in the order 4h + {0..3}, 4h + 8 +
//     {0..3} (h = l/32).  Lanes 4m .. 4m+3 of a 16-lane group address key
//     4h + m (+ 8 for the second read, tro[1]) and 4 consecutive d each, so
//     lane i receives d = base + i across the 4 keys.
template <int D>
struct ReadPlan {
  int off[4], tro[2][2];  // tro[second read][32-d half of a 64-d half]
  __device__ __forceinline__ explicit ReadPlan(int lane) {
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int t = 0; t < 4; ++t) off[t] = l32 * 128 + 16 * ((2 * t + hi) ^ sw(l32));
    const int i = lane & 15, g2 = (lane >> 4) & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kl = 4 * hi + (i >> 2) + 8 * j;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int d = 32 * p + 16 * g2 + 4 * (i & 3);
        tro[j][p] = kl * 128 + 16 * ((d >> 3) ^ sw(kl)) + 8 * ((d >> 2) & 1);
      }
    }
  }
  __device__ __forceinline__ const char* kp(const char* Ks, int kt, int t) const {
    return Ks + (t / 4) * Tiles<D>::KHALF + kt * 4096 + off[t % 4];
  }
  __device__ __forceinline__ bf16x8 vt(const char* Vs, int dt, int pl) const {
    // dt may be a wave-uniform runtime value: select rather than index
    const char* b = Vs + (dt / 2) * Tiles<D>::KHALF + pl * 16 * 128;
    return cat_tr(b + ((dt & 1) ? tro[0][1] : tro[0][0]), b + ((dt & 1) ? tro[1][1] : tro[1][0]));
  }
};

__device__ __forceinline__ uint4 rd16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// v itself, opaque to the optimiser: per-lane offsets derived from it are
// then recomputed where they are used instead of being kept live (or
// spilled) across a loop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their no-wait maxima).  Direct
// loads to LDS count on vmcnt, in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0) only: every LDS read of this wavefront has returned.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier that orders LDS accesses only: each wavefront's LDS
// reads and writes have completed when it arrives (lgkmcnt 0), while its
// vector-memory loads in flight - direct loads of a later unit's tiles into
// another LDS buffer - stay in flight.  (__syncthreads, and a workgroup fence
// even when limited to LDS, also waits for those loads, since they write
// LDS.)  The memory clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Buffer resource over [base, base + bytes) for raw (unstructured) buffer
// loads; reads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Direct buffer load of 16 bytes per lane into LDS: lane l writes
// lds_wave_base + 16 l; the byte address is voff + soff in the buffer.
__device__ __forceinline__ void b2lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                        void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, (int)voff, (int)soff, 0, 0);
}

// Direct buffer load of 4 bytes per lane into LDS: lane l writes
// lds_wave_base + 4 l.
__device__ __forceinline__ void b2lds4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 4, (int)voff, (int)soff, 0, 0);
}

// Direct loads of one unit's K or V tile into LDS, split over NWL wavefronts.
// Load slot u of a tile fills the 1 KB at tile + 1024 u (8 rows of 128 bytes,
// in the swizzled layout above): lane l brings the 16-byte chunk that belongs
// at position l.  Each load is a per-head buffer resource over a row-major
// [N, D] array, the unit's byte offset (scalar) and a per-lane byte offset
// fixed for the kernel; rows past N read as zeros.
template <int D, int NWL>
struct LoadPlan {
  using T = Tiles<D>;
  static constexpr int NK = T::KT_BYTES / 1024 / NWL;   // slots per wavefront and tile
  static_assert(NK * NWL * 1024 == T::KT_BYTES, "tile split");
  uint32_t voff[NK];
  int w;

  __device__ __forceinline__ LoadPlan(int w_, int lane) : w(w_) {
#pragma unroll
    for (int ii = 0; ii < NK; ++ii) {
      const int u = w + NWL * ii;
      const int hd = u / 8, key = 8 * (u % 8) + (lane >> 3);
      voff[ii] = (uint32_t)(key * D * 2 + hd * 128 + 16 * ((lane & 7) ^ sw(key)));
    }
  }
  // the tile of the unit starting at key key0
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int key0, char* dst) const {
    const uint32_t soff = (uint32_t)key0 * (D * 2);
#pragma unroll
    for (int ii = 0; ii < NK; ++ii) b2lds16(r, voff[ii], soff, dst + 1024 * (w + NWL * ii));
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

// S^T of a whole unit (two 32-key subtiles) with the K fragments read PF
// MFMAs ahead of their use, so the LDS latency stays hidden behind the
// matrix ops already issued.
template <int D, int PF>
__device__ __forceinline__ void score_unit(const char* Ks, const bf16x8 (&qf)[D / 16], const ReadPlan<D>& rp,
                                           f32x16 (&s)[2]) {
  constexpr int NT = D / 16;        // k-steps per subtile
  constexpr int NI = 2 * NT;        // MFMAs of the unit
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

// S^T of the 32-key half KT of a unit (K fragments read PF MFMAs ahead,
// order pinned as in score_unit).
template <int D, int KT, int PF>
__device__ __forceinline__ f32x16 score_half(const char* Ks, const bf16x8 (&qf)[D / 16], const ReadPlan<D>& rp) {
  constexpr int NT = D / 16;
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

// Transposed operand reads in flight ahead of the backward's products (4 and 2
// measured alike; 6 spills the column kernels).
constexpr int BWD_PF = 4;

// Column-side products of a 64-query unit for one wavefront: acc0[t] +=
// T0^T op[0][pl] and acc1[t] += T1^T op[1][pl] over the four query planes pl,
// with T0, T1 row-major 64-row tiles (dO and Q, or h and phi(Q)) read
// transposed at d tile NDT DT + t.  Planes OWN, OWN + 1 come first (their
// operands are this wavefront's own), then the other two (from another
// wavefront through LDS).  Each transposed read is issued PF products ahead
// of its MFMA, so LDS latency stays behind the matrix ops already issued.
// XR: LDS reads just before (the other wavefront's operands), which the
// scheduling groups below have to count.
template <int D, int NDT, int DT, int OWN, int PF, int XR>
__device__ __forceinline__ void col_products(const char* T0, const char* T1, const ReadPlan<D>& rp,
                                             const bf16x8 (&op)[2][4], f32x16 (&acc0)[NDT],
                                             f32x16 (&acc1)[NDT]) {
  constexpr int NI = 4 * NDT * 2;  // products
  static_assert(PF >= 1 && PF < NI, "prefetch depth");
  auto plane = [](int i) { const int j = i / (2 * NDT); return j < 2 ? OWN + j : (OWN + j) & 3; };
  auto rd = [&](auto it) __attribute__((always_inline)) {
    constexpr int i = decltype(it)::value;
    constexpr int pl = plane(i), t = (i / 2) % NDT;
    return rp.vt(i % 2 == 0 ? T0 : T1, NDT * DT + t, pl);
  };
  bf16x8 fr[PF];
  static_for<PF>([&](auto it) __attribute__((always_inline)) { fr[decltype(it)::value] = rd(it); });
  static_for<NI>([&](auto it) __attribute__((always_inline)) {
    constexpr int i = decltype(it)::value;
    constexpr int pl = plane(i), t = (i / 2) % NDT;
    const bf16x8 a = fr[i % PF];
    if constexpr (i + PF < NI) fr[i % PF] = rd(IntTag<i + PF>{});
    if constexpr (i % 2 == 0) acc0[t] = mfma(a, op[0][pl], acc0[t]);
    else acc1[t] = mfma(a, op[1][pl], acc1[t]);
  });
  // keep that order (two transposed reads per operand)
  __builtin_amdgcn_sched_group_barrier(0x100, XR + 2 * PF, 0);
#pragma unroll
  for (int i = 0; i + PF < NI; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
}

// Row-side products of one 32-key half KT of a unit: acc[dt] += T^T b[pl]
// over the half's two key planes 2 KT + pl, T a row-major 64-row tile read
// transposed at d tile dt; each transposed read issued PF products ahead
// of its MFMA.
template <int D, int KT, int PF>
__device__ __forceinline__ void row_products(const char* Ts, const ReadPlan<D>& rp, const bf16x8 (&b)[2],
                                             f32x16 (&acc)[D / 32]) {
  constexpr int NI = 2 * (D / 32);   // products: plane-major
  constexpr int P = PF < NI ? PF : NI - 1;  // reads in flight
  static_assert(P >= 1, "prefetch depth");
  auto rd = [&](auto it) __attribute__((always_inline)) {
    constexpr int i = decltype(it)::value;
    return rp.vt(Ts, i % (D / 32), 2 * KT + i / (D / 32));
  };
  bf16x8 fr[P];
  static_for<P>([&](auto it) __attribute__((always_inline)) { fr[decltype(it)::value] = rd(it); });
  static_for<NI>([&](auto it) __attribute__((always_inline)) {
    constexpr int i = decltype(it)::value;
    const bf16x8 a = fr[i % P];
    if constexpr (i + P < NI) fr[i % P] = rd(IntTag<i + P>{});
    acc[i % (D / 32)] = mfma(a, b[i / (D / 32)], acc[i % (D / 32)]);
  });
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * P, 0);
#pragma unroll
  for (int i = 0; i + P < NI; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, P, 0);
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

// 16 fp32 values of a 32-key S^T half (element order) into the 2 bf16 P
// operands of its key planes (plane j: elements 8 j .. 8 j + 7)
__device__ __forceinline__ void pack_planes(const float (&v)[16], bf16x8 (&bp)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[e] = pk_bf16(v[8 * j + 2 * e], v[8 * j + 2 * e + 1]);
    bp[j] = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));
  }
}

}  // namespace
}  // namespace sla
