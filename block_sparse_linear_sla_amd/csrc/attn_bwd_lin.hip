// Backward of the linear branch (bf16) on gfx950.
//
// Source: SLA2 write-up (arXiv:2602.12675) §一 (the linear branch: linear
// attention, phi = elu + 1, over the keys of the blocks a row does not
// select), §二 (its output is normalised over those keys) and §四 (training
// with the selection fixed per step).  For a query t of row block i with
// unselected key set U, a = phi(q_t), w_u = a . phi(k_u), den = sum_U w_u,
// O_l = sum_U w_u v_u / den and h the gradient reaching O_l:
//   P~_u = w_u / den,  D~ = h . O_l,  dw_u = (h . v_u - D~) / den,
//   da = sum_U dw_u phi(k_u),  dq = phi'(q) o da,
//   dv_u = sum_{t: u in U_t} P~_tu h_t,  dphi(k_u) = sum_{t: u in U_t} dw_tu a_t.
// Every sum over U is the sum over all keys minus the sum over the row's
// listed blocks, as in the forward: with H = sum_u phi(k_u) v_u^T, z =
// sum_u phi(k_u), M = sum_t a_t (h_t / den_t)^T and m = sum_t (D~_t / den_t) a_t,
//   den = a . z - sum_sel w,   den D~ = a^T H h - sum_sel w (h . v),
//   da  = (H h - D~ z - sum_sel (h . v_u - D~) phi(k_u)) / den,
//   dv_u = M^T phi(k_u) - sum_sel P~ h,   dphi(k_u) = M v_u - m - sum_sel dw a.
// The listed-pair sums run on the matrix cores in the same row (CSR) and
// column (CSC) walks as the sparse branch's gradient, with phi(K) in place
// of K and no exponential; the totals are float32 products per head.
// A row whose blocks are all listed has no linear branch: its den, D~ and
// gradient contributions are 0.
//
// Kernels:
//   lin_phi_kernel     phi(Q), phi(K) as bf16 rows (the matrix-core tiles);
//   lin_outer_kernel   chunk partials of R = sum_t x_t y_t^T and s = sum_t
//                      e_t x_t per head on the matrix cores - (H, z) and (M, m);
//                      summed by the chunk reduction;
//   lin_split_kernel   a total as hi + lo bf16 matrix-core fragments;
//   lin_dq_kernel      per mask row: U = H h on the matrix cores from the
//                      fragments of H; pass A sums w and w (h . v) over the
//                      listed units, then den = a . z - sum w and den D~ =
//                      a . U - sum w (h . v); pass B subtracts phi(K)^T
//                      (h . v - D~) from U; then dq;
//   lin_dkdv_kernel    per 64-key unit over the rows that list it: P~ and dw in
//                      registers, dV^T += h^T P~ and dphi^T += phi(Q)^T dw, then
//                      dv = M^T phi(k) - dV and dphi = M v - m - dphi with the
//                      products on the matrix cores from the fragments of M^T, M.
#include "sla.h"
#include "sla_internal.h"
#include "bf16_tiles.h"

namespace sla {
namespace {

__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __expf(x); }

// 8 bf16 of a uint4 as floats
__device__ __forceinline__ void unpack8(const uint4& v, float (&x)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = bf2f(elem(v, e));
}

// v += the 4 bf16 values packed in old
__device__ __forceinline__ void add4(const uint2& old, float (&v)[4]) {
  v[0] += bf2f(old.x & 0xffffu);
  v[1] += bf2f(old.x >> 16);
  v[2] += bf2f(old.y & 0xffffu);
  v[3] += bf2f(old.y >> 16);
}

// the 4 values as 4 consecutive bf16 at p
__device__ __forceinline__ void store4(uint16_t* p, const float (&v)[4]) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]));
}


// ------------------------------------------------------------------ phi rows
__global__ __launch_bounds__(256) void lin_phi_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                      long long n8, uint16_t* __restrict__ A,
                                                      uint16_t* __restrict__ F) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= 2 * n8) return;
  const bool isk = t >= n8;
  const long long o = isk ? t - n8 : t;
  const uint4 v = reinterpret_cast<const uint4*>(isk ? K : Q)[o];
  float x[8];
  unpack8(v, x);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pk_bf16(phi(x[2 * e]), phi(x[2 * e + 1]));
  reinterpret_cast<uint4*>(isk ? F : A)[o] = make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------------ totals
// Partials over rows [chunk * LROWS, ...) of one head, on the matrix cores:
// R = sum_t (c_t phi(x_t)) y_t^T (D x D, row-major) and s = sum_t e_t c_t
// phi(x_t), x and y bf16 rows (x = K, y = V: H and z, c = e = 1; x = Q,
// y = dO_l: M and m, c = 1 / den, e = D~ from the per-query arrays
// [bh * QP + t], which hold 0 past N).  The 64-row units stream through two
// LDS stages; both operands are transposed reads of the row-major tiles
// (row t in the contraction): A = the x^T fragments of the wavefront's row
// tile of R, turned into c phi(x) in float32 and split into hi + lo bf16
// (two products, so that the totals keep about 2^-17 relative accuracy), and
// B = the y^T fragments of its column tiles.  Lanes keep the vector sums of
// their A elements in float32.
template <int D>
__global__ __launch_bounds__(256, 2) void lin_outer_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Y,
                                                           const float* __restrict__ inv,
                                                           const float* __restrict__ dtq, int N, long long QP,
                                                           int nchunk, float* __restrict__ part) {
  using T = Tiles<D>;
  using LP = LoadPlan<D, 4>;
  constexpr int NT = D / 32, TPW = NT * NT / 4;
  // X and Y tiles of a 64-row unit, then (M pass) the unit's 64 values of
  // 1/den and of D~, loaded with the tiles so that no load of a later unit
  // is waited for in the middle of a step
  constexpr int STAGE = 2 * T::KT_BYTES + 2 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  const int tid = threadIdx.x, lane = tid & 63, hi = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ReadPlan<D> rdp(lane);
  const long long bh = blockIdx.y;
  const int chunk = blockIdx.x;
  const int r0 = chunk * LROWS;
  const int nun = (min(LROWS, N - r0) + KU - 1) / KU;
  const int gt0 = w * TPW;  // this wavefront's tiles gt0 .. gt0 + TPW - 1 (one row tile)
  const int at = gt0 / NT;
  const bool sown = gt0 % NT == 0;  // keeps the vector sums of row tile at
  const auto rx = buf_rsrc(X + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
  const auto ry = buf_rsrc(Y + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
  f32x16 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
  float sp = 0.f;
  const auto ri = buf_rsrc(inv + (inv != nullptr ? (size_t)bh * QP : 0), (uint32_t)(QP * 4));
  const auto re = buf_rsrc(dtq + (dtq != nullptr ? (size_t)bh * QP : 0), (uint32_t)(QP * 4));
  auto issue = [&](int x, char* sb) __attribute__((always_inline)) {
    const LP lp(w, opaque(lane));
    lp.load(rx, r0 + x * KU, sb);
    lp.load(ry, r0 + x * KU, sb + T::KT_BYTES);
    if (inv != nullptr && w == 0) {
      b2lds4(ri, 4u * (uint32_t)lane, 4u * (uint32_t)(r0 + x * KU), sb + 2 * T::KT_BYTES);
      b2lds4(re, 4u * (uint32_t)lane, 4u * (uint32_t)(r0 + x * KU), sb + 2 * T::KT_BYTES + 256);
    }
  };
  auto step = [&](int x, char* cur, char* nxt) __attribute__((always_inline)) {
    wait_vm<0>();
    __syncthreads();
    if (x + 1 < nun) issue(x + 1, nxt);
    const int t0 = r0 + x * KU;
#pragma unroll
    for (int pl = 0; pl < 4; ++pl) {
      // element e of a plane fragment: row 16 pl + 4 hi + e % 4 + 8 (e / 4);
      // rows past N are zero in the tile, and phi(0) = 1 is cancelled by c = 0
      // (M) or by the row mask below (H)
      const uint4 av = __builtin_bit_cast(uint4, rdp.vt(cur, at, pl));
      float xs[8];
      if (inv != nullptr) {
        const float* iu = reinterpret_cast<const float*>(cur + 2 * T::KT_BYTES) + 16 * pl + 4 * hi;
        const float4 i0 = *reinterpret_cast<const float4*>(iu);
        const float4 i1 = *reinterpret_cast<const float4*>(iu + 8);
        const float4 e0 = *reinterpret_cast<const float4*>(iu + 64);
        const float4 e1 = *reinterpret_cast<const float4*>(iu + 72);
        const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
        const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xs[e] = phi(bf2f(elem(av, e))) * iv[e];
          if (sown) sp = fmaf(xs[e], ev[e], sp);
        }
      } else {
        const int lim = N - (t0 + 16 * pl + 4 * hi);  // element e is a row when e%4 + 8 (e/4) < lim
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xs[e] = (e % 4) + 8 * (e / 4) < lim ? phi(bf2f(elem(av, e))) : 0.f;
          if (sown) sp += xs[e];
        }
      }
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = pk_bf16(xs[2 * e], xs[2 * e + 1]);
        l[e] = pk_bf16(xs[2 * e] - bf2f(h[e] & 0xffffu), xs[2 * e + 1] - bf2f(h[e] >> 16));
      }
      const bf16x8 ah = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
      const bf16x8 al = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const bf16x8 b = rdp.vt(cur + T::KT_BYTES, (gt0 + u) % NT, pl);
        acc[u] = mfma(ah, b, acc[u]);
        acc[u] = mfma(al, b, acc[u]);
      }
    }
  };
  if (nun > 0) {
    issue(0, st0);
    int x = 0;
    for (; x + 2 <= nun; x += 2) {
      step(x, st0, st1);
      step(x + 1, st1, st0);
    }
    if (x < nun) step(x, st0, st1);
    wait_vm<0>();
  }
  // element i of tile u: R row 32 at + 8 (i/4) + 4 hi + i%4, column 32 bt + lane % 32
  const size_t per = (size_t)D * D + D;
  float* out = part + ((size_t)bh * nchunk + chunk) * per;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int bt = (gt0 + u) % NT;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      out[(size_t)(32 * at + 8 * (i >> 2) + 4 * hi + (i & 3)) * D + 32 * bt + (lane & 31)] = acc[u][i];
  }
  const float st = sp + __shfl_xor(sp, 32);
  if (sown && hi == 0) out[(size_t)D * D + 32 * at + (lane & 31)] = st;
}

// One head's D x D total R (row-major in tot) as matrix-core operand
// fragments of y_t = R' x_t (the A operand of y^T = R' x^T: rows o, k-slices
// i), R' = R (TRANS = 0: y[o] = sum_i R[o][i] x[i]) or R^T (TRANS = 1:
// y[o] = sum_i R[i][o] x[i]).  Fragment (dt, kk) of lane l holds
// R'[o][i] for o = 32 dt + l % 32 and i = 16 kk + 8 (l / 32) + 0..7, each
// value split as hi = bf16(x) and lo = bf16(x - hi), so that the two
// bf16 products keep R to about 2^-17 relative.  Layout: uint4
// [bh][(dt * D/16 + kk) * 2 + part][lane].
template <int D>
__global__ __launch_bounds__(256) void lin_split_kernel(const float* __restrict__ tot, int trans,
                                                        uint4* __restrict__ frag) {
  constexpr int NKK = D / 16, PER_HEAD = (D / 32) * NKK * 64;
  const long long bh = blockIdx.y;
  const int g = blockIdx.x * 256 + threadIdx.x;  // (dt, kk, lane)
  if (g >= PER_HEAD) return;
  const int lane = g & 63, f = g >> 6;
  const int dt = f / NKK, kk = f % NKK;
  const int o = 32 * dt + (lane & 31), i0 = 16 * kk + 8 * (lane >> 5);
  const float* R = tot + (size_t)bh * ((size_t)D * D + D);
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x[2], hf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = i0 + 2 * e + c;
      x[c] = trans ? R[(size_t)i * D + o] : R[(size_t)o * D + i];
    }
    h[e] = pk_bf16(x[0], x[1]);
    hf[0] = bf2f(h[e] & 0xffffu);
    hf[1] = bf2f(h[e] >> 16);
    l[e] = pk_bf16(x[0] - hf[0], x[1] - hf[1]);
  }
  uint4* dst = frag + (size_t)bh * 2 * PER_HEAD + (size_t)(2 * f) * 64 + lane;
  dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
  dst[64] = make_uint4(l[0], l[1], l[2], l[3]);
}

// ------------------------------------------------------------------ dq
template <int D, int BQ, int SUB>
__global__ __launch_bounds__(BQ / 32 * 64, 2) void lin_dq_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ F, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ G, const uint16_t* __restrict__ Qraw, const int* __restrict__ row_ptr,
    const int* __restrict__ col_idx, const uint4* __restrict__ fragH, const float* __restrict__ tot_h,
    float* __restrict__ invden_out, float* __restrict__ dt_out, uint16_t* __restrict__ dQ, int add,
    const float* __restrict__ alpha, int H, int N, int Nq, int Nk, const float* __restrict__ invden_in,
    const float* __restrict__ ol_in) {
  using T = Tiles<D>;
  constexpr int NW = BQ / 32;
  using LP = LoadPlan<D, NW>;
  constexpr int STAGE = 2 * T::KT_BYTES;
  constexpr int NDT = D / 32, NKK = D / 16;
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const ReadPlan<D> rdp(lane);
  const long long row = xcd_row(blockIdx.x, (long long)gridDim.x);
  const long long bh = row / Nq;
  const int qi = (int)(row % Nq);
  const int base = row_ptr[row];
  const int nsel = row_ptr[row + 1] - base;
  const int nunits = nsel * SUB;
  const int q = qi * BQ + 32 * w + (lane & 31);
  const bool qv = q < N;
  const size_t qidx = (size_t)row * BQ + 32 * w + (lane & 31);  // per-query arrays

  bf16x8 af[NKK], hf[NKK];
  load_q<D>(A, bh, q, N, hi, af);
  load_q<D>(G, bh, q, N, hi, hf);
  // acc^T starts as U^T = (H h)^T for this wavefront's queries (H as hi + lo
  // fragments; element i of tile dt: d = 32 dt + 8 (i/4) + 4 hi + i%4) and
  // ends as U - sum_sel (h . v - D~) phi(k)
  // The fragments (a contiguous per-head block, fragment f at 1024 f) come
  // into the stages once per workgroup by direct loads, a share per
  // wavefront, and every wavefront reads all of them there, each PF MFMAs
  // ahead.
  f32x16 acc[NDT];
  {
    constexpr int NF = 2 * NDT * NKK, FPS = STAGE / 1024, PF = 4;
    static_assert(NF <= 2 * FPS && NF % NW == 0, "the fragments fit the stages");
    auto frag_at = [&](int f) -> const char* { return f < FPS ? st0 + 1024 * f : st1 + 1024 * (f - FPS); };
    const auto r = buf_rsrc(fragH + (size_t)bh * NF * 64, (uint32_t)(NF * 1024));
#pragma unroll
    for (int i = 0; i < NF / NW; ++i) {
      const int f = (NF / NW) * w + i;
      b2lds16(r, (uint32_t)(16 * lane + 1024 * f), 0u, (char*)frag_at(f));
    }
    wait_vm<0>();
    __syncthreads();
    uint4 fr[PF];
    static_for<PF>([&](auto it) __attribute__((always_inline)) {
      fr[decltype(it)::value] = rd16(frag_at(decltype(it)::value) + 16 * lane);
    });
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
    // fragment i: tile i / (2 NKK), k-step (i / 2) % NKK, hi then lo
    static_for<NF>([&](auto it) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;
      const uint4 a = fr[i % PF];
      if constexpr (i + PF < NF) fr[i % PF] = rd16(frag_at(i + PF) + 16 * lane);
      acc[i / (2 * NKK)] = mfma(as_bf16x8(a), hf[(i / 2) % NKK], acc[i / (2 * NKK)]);
    });
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int i = 0; i + PF < NF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
    __syncthreads();  // every wavefront has read the fragments; the stages are free
  }
  float sw = 0.f, swh = 0.f;  // this lane's sums of w and w (h . v) over its listed keys
  float inv = 0.f, dtv = 0.f;  // 1 / den and D~ (0 for a row without a linear branch)
  const size_t qrow = ((size_t)bh * N + (qv ? q : 0)) * D;
  const float* z = tot_h + (size_t)bh * ((size_t)D * D + D) + (size_t)D * D;
  // phi(q) . z and phi(q) . (H h) over this lane's d of the accumulator
  // tiles; the two halves (lanes l, l^32) are added in settle
  float p1 = 0.f, p2 = 0.f;
  // with the forward's terms: 1 / den as it kept it (0 where the row has no
  // linear branch) and D~ = h . O_l (this lane's half of d, then the pair
  // sum); pass A is skipped
  const bool saved = invden_in != nullptr;
  if (saved) {
    float part = 0.f;
    if (qv) {
      const float* orow = ol_in + ((size_t)bh * N + q) * D;
#pragma unroll
      for (int t = 0; t < NKK; ++t) {
        const uint4 a = __builtin_bit_cast(uint4, hf[t]);
        const float4 o0 = *reinterpret_cast<const float4*>(orow + 16 * t + 8 * hi);
        const float4 o1 = *reinterpret_cast<const float4*>(orow + 16 * t + 8 * hi + 4);
        const float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(bf2f(elem(a, e)), o[e], part);
      }
    }
    const float X = part + __shfl_xor(part, 32);
    inv = qv ? invden_in[qidx] : 0.f;
    dtv = inv != 0.f ? X : 0.f;
  }
  if (qv && !saved) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * dt + 8 * a + 4 * hi;
        const uint2 q2 = *reinterpret_cast<const uint2*>(Qraw + qrow + d0);
        const float4 z4 = *reinterpret_cast<const float4*>(z + d0);
        const float qq[4] = {bf2f(q2.x & 0xffffu), bf2f(q2.x >> 16), bf2f(q2.y & 0xffffu), bf2f(q2.y >> 16)};
        const float zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float fq = phi(qq[c]);
          p1 = fmaf(fq, zz[c], p1);
          p2 = fmaf(fq, acc[dt][4 * a + c], p2);
        }
      }
  }
  auto settle = [&]() {
    const float SW = sw + __shfl_xor(sw, 32), SWH = swh + __shfl_xor(swh, 32);
    const float den = p1 + __shfl_xor(p1, 32) - SW;
    const float X = p2 + __shfl_xor(p2, 32) - SWH;
    if (qv && nsel < Nk && den > 0.f) {
      inv = 1.f / den;
      dtv = X * inv;
    }
  };
  if (nunits > 0) {
    const auto rf = buf_rsrc(F + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
    const auto rv = buf_rsrc(V + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
    auto issue = [&](int x, char* sb) __attribute__((always_inline)) {
      const LP lp(w, opaque(lane));
      const int k0 = (col_idx[base + x / SUB] * SUB + x % SUB) * KU;
      lp.load(rf, k0, sb);
      lp.load(rv, k0, sb + T::KT_BYTES);
    };
    // keys past N read as zero rows of phi(K) and V (buffer loads past the
    // head's range return 0), so they add nothing to either pass
    auto step = [&](auto pass, int x, char* cur, char* nxt) __attribute__((always_inline)) {
      constexpr int PASS = decltype(pass)::value;
      wait_vm<0>();
      __syncthreads();
      if (x + 1 < nunits) issue(x + 1, nxt);
      static_for<2>([&](auto kt_tag) __attribute__((always_inline)) {
        constexpr int KT = decltype(kt_tag)::value;
        const f32x16 dp = score_half<D, KT, 2>(cur + T::KT_BYTES, hf, rdp);
        if (PASS == 0) {
          // pass A: w and w (h . v) summed over this lane's keys
          const f32x16 s = score_half<D, KT, 2>(cur, af, rdp);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            sw += s[i];
            swh = fmaf(s[i], dp[i], swh);
          }
        } else {
          // pass B: acc -= phi(K)^T (h . v - D~) over this half's two key planes
          float c[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) c[i] = dtv - dp[i];
          bf16x8 bp[2];
          pack_planes(c, bp);
          row_products<D, KT, BWD_PF>(cur, rdp, bp, acc);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto run = [&](auto pass) __attribute__((always_inline)) {
      issue(0, st0);
      int x = 0;
      for (; x + 2 <= nunits; x += 2) {
        step(pass, x, st0, st1);
        step(pass, x + 1, st1, st0);
      }
      if (x < nunits) step(pass, x, st0, st1);
      wait_vm<0>();
      __syncthreads();  // every wavefront is done with both stages
    };
    if (!saved) {
      run(IntTag<0>{});
      settle();
    }
    run(IntTag<1>{});
  } else if (!saved) {
    settle();
  }
  if (hi == 0) {
    invden_out[qidx] = inv;
    dt_out[qidx] = dtv;
  }
  if (!qv) return;
  // da = (acc - D~ z) / den; dq = phi'(q) o da, times the branch's weight in
  // the mixed output
  const float os = alpha != nullptr ? 1.f - alpha[bh % H] : 1.f;
  const float sinv = os * inv;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    // the tile's loads together, so their latencies overlap
    float4 z4[4];
    uint2 q2[4], old[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hi;
      z4[a] = *reinterpret_cast<const float4*>(z + d0);
      q2[a] = *reinterpret_cast<const uint2*>(Qraw + qrow + d0);
      if (add) old[a] = *reinterpret_cast<const uint2*>(dQ + qrow + d0);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hi;
      const float zz[4] = {z4[a].x, z4[a].y, z4[a].z, z4[a].w};
      const float qq[4] = {bf2f(q2[a].x & 0xffffu), bf2f(q2[a].x >> 16), bf2f(q2[a].y & 0xffffu),
                           bf2f(q2[a].y >> 16)};
      float o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = dphi(qq[c]) * ((acc[dt][4 * a + c] - dtv * zz[c]) * sinv);
      if (add) add4(old[a], o);
      store4(dQ + qrow + d0, o);
    }
  }
}

// ------------------------------------------------------------------ dk, dv
template <int D, int BQ, int SUB>
__global__ __launch_bounds__(256, 2) void lin_dkdv_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ F, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ G, const uint16_t* __restrict__ Kraw, const int* __restrict__ col_ptr,
    const int* __restrict__ row_idx, const int* __restrict__ order, const float* __restrict__ invden,
    const float* __restrict__ dtq,
    const uint4* __restrict__ fragMT, const uint4* __restrict__ fragM, const float* __restrict__ tot_m,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int add, const float* __restrict__ alpha, int H, int N,
    int Nq, int Nk) {
  using T = Tiles<D>;
  using LP = LoadPlan<D, 4>;
  constexpr int STAGE = 2 * T::KT_BYTES;  // phi(Q) and h tiles of 64 queries
  constexpr int NDT = D / 64;
  constexpr int QU = BQ / KU;
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint4 xch[4][4][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int kh = w & 1, dh = w >> 1;
  const int partner = w ^ 2;
  const ReadPlan<D> rdp(lane);
  // (bh, key block, 64-key part), most-listed key blocks first
  const long long unit = order[blockIdx.x];
  if (unit < 0 || unit >= (long long)gridDim.x) return;
  const long long bh = unit / ((long long)Nk * SUB);
  const int ku = (int)(unit % ((long long)Nk * SUB));
  const int j = ku / SUB;
  const int key = ku * KU + 32 * kh + (lane & 31);
  const bool kv = key < N;
  const long long col = bh * Nk + j;
  const int cb = col_ptr[col];
  const int nunits = (col_ptr[col + 1] - cb) * QU;

  bf16x8 ff[D / 16], vf[D / 16];
  load_q<D>(F, bh, key, N, hi, ff);
  load_q<D>(V, bh, key, N, hi, vf);
  f32x16 adv[NDT], adk[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    adv[t] = f32x16{};
    adk[t] = f32x16{};
  }
  if (nunits > 0) {
    const auto ra = buf_rsrc(A + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
    const auto rg = buf_rsrc(G + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
    auto qrow_of = [&](int x) { return row_idx[cb + x / QU]; };
    auto issue = [&](int x, char* sb) __attribute__((always_inline)) {
      const LP lp(w, opaque(lane));
      const int q0 = qrow_of(x) * BQ + (x % QU) * KU;
      lp.load(ra, q0, sb);
      lp.load(rg, q0, sb + T::KT_BYTES);
    };
    // the unit's per-query terms (1 / den and D~), one value per lane
    // (term_query) of this wavefront's 32 queries, loaded with the unit's
    // tiles so that the only wait for them is the one for the tiles
    const int tq = 32 * dh + term_query(lane);
    auto terms_at = [&](int x) { return ((size_t)(bh * Nq + qrow_of(x))) * BQ + (x % QU) * KU + tq; };
    float In = invden[terms_at(0)], Dn = dtq[terms_at(0)];
    auto step = [&](int x, char* cur, char* nxt) __attribute__((always_inline)) {
      wait_vm<0>();
      __syncthreads();
      const float Ic = In, Dc = Dn;
      if (x + 1 < nunits) {
        const size_t tn = terms_at(x + 1);
        In = invden[tn];
        Dn = dtq[tn];
        issue(x + 1, nxt);
      }
      auto body = [&](auto qh_tag) __attribute__((always_inline)) {
        constexpr int QH = decltype(qh_tag)::value;
        constexpr int OWN = 2 * QH, OTH = 2 - OWN;
        // w and h . v of this wavefront's 32 queries x its 32 keys (element
        // i: query 32 QH + 8 (i/4) + 4 hi + i%4); P~ = w / den, dw = (h . v - D~) / den
        const f32x16 s = score_half<D, QH, 4>(cur, ff, rdp);
        const f32x16 dp = score_half<D, QH, 4>(cur + T::KT_BYTES, vf, rdp);
        float pv[16], ds[16];
        static_for<16>([&](auto it) __attribute__((always_inline)) {
          constexpr int i = decltype(it)::value;
          const float iq = row_bcast<i>(Ic);
          pv[i] = s[i] * iq;
          ds[i] = (dp[i] - row_bcast<i>(Dc)) * iq;
        });
        bf16x8 op[2][4];
        bf16x8 bp[2], bs[2];
        pack_planes(pv, bp);
        pack_planes(ds, bs);
        op[0][OWN] = bp[0];
        op[0][OWN + 1] = bp[1];
        op[1][OWN] = bs[0];
        op[1][OWN + 1] = bs[1];
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
          for (int pl = 0; pl < 2; ++pl) xch[w][2 * o + pl][lane] = __builtin_bit_cast(uint4, op[o][OWN + pl]);
        lds_barrier();  // the next unit's tiles stay in flight
#pragma unroll
        for (int o = 0; o < 2; ++o)
#pragma unroll
          for (int pl = 0; pl < 2; ++pl)
            op[o][OTH + pl] = __builtin_bit_cast(bf16x8, xch[partner][2 * o + pl][lane]);
        // dV^T += h^T P~ and dphi^T += phi(Q)^T dw, d rows of this wavefront's half
        col_products<D, NDT, QH, OWN, BWD_PF, 4>(cur + T::KT_BYTES, cur, rdp, op, adv, adk);
      };
      if (dh == 0) body(IntTag<0>{});
      else body(IntTag<1>{});
    };
    issue(0, st0);
    int x = 0;
    for (; x + 2 <= nunits; x += 2) {
      step(x, st0, st1);
      step(x + 1, st1, st0);
    }
    if (x < nunits) step(x, st0, st1);
    wait_vm<0>();
  }
  // dv = M^T phi(k) - acc_v and dphi = M v - m - acc_k, the products with M
  // on the matrix cores (M^T and M as hi + lo fragments, phi(k) and v from
  // this lane's key fragments); dk = phi'(k) o dphi.  Element i of tile t:
  // d = 32 (NDT dh + t) + 8 (i/4) + 4 hi + i%4.  Each fragment set (a
  // contiguous per-head block, fragment f at 1024 f) comes into the free
  // stages once per workgroup by direct loads, a quarter per wavefront, and
  // is read from there by the two wavefronts that use each fragment.
  constexpr int NKK = D / 16;
  constexpr int NF = 2 * (D / 32) * NKK;  // fragments per set
  constexpr int FPS = STAGE / 1024;       // fragments per stage array
  static_assert(NF <= 2 * FPS && NF % 4 == 0, "a fragment set fits the stages");
  const float* mv = tot_m + (size_t)bh * ((size_t)D * D + D) + (size_t)D * D;
  const size_t krow = ((size_t)bh * N + (kv ? key : 0)) * D;
  const float os = alpha != nullptr ? 1.f - alpha[bh % H] : 1.f;
  auto frag_at = [&](int f) -> const char* { return (f < FPS ? st0 + 1024 * f : st1 + 1024 * (f - FPS)) + 16 * lane; };
  auto stage_set = [&](const uint4* set) __attribute__((always_inline)) {
    const auto r = buf_rsrc(set + (size_t)bh * NF * 64, (uint32_t)(NF * 1024));
#pragma unroll
    for (int i = 0; i < NF / 4; ++i) {
      const int f = (NF / 4) * w + i;
      b2lds16(r, (uint32_t)(16 * lane + 1024 * f), 0u, (char*)frag_at(f) - 16 * lane);
    }
  };
  // y[t] = sum over k-steps of (hi + lo fragment of tile NDT dh + t) x x[kk],
  // each fragment read PF products ahead of its MFMA
  auto products = [&](const bf16x8 (&x)[NKK], f32x16 (&y)[NDT]) __attribute__((always_inline)) {
    constexpr int NI = NDT * 2 * NKK, PF = 4;
    const int f0 = 2 * NDT * dh * NKK;  // first fragment of this wavefront's tiles
    uint4 fr[PF];
    static_for<PF>([&](auto it) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;
      fr[i] = rd16(frag_at(f0 + i));
    });
#pragma unroll
    for (int t = 0; t < NDT; ++t) y[t] = f32x16{};
    static_for<NI>([&](auto it) __attribute__((always_inline)) {
      constexpr int i = decltype(it)::value;  // fragment f0 + i: tile i / (2 NKK), k-step (i / 2) % NKK
      const uint4 a = fr[i % PF];
      if constexpr (i + PF < NI) fr[i % PF] = rd16(frag_at(f0 + i + PF));
      y[i / (2 * NKK)] = mfma(as_bf16x8(a), x[(i / 2) % NKK], y[i / (2 * NKK)]);
    });
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int i = 0; i + PF < NI; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
  };
  // the tile's elementwise terms: m, the raw k and, when adding, what dV and dK hold
  float4 m4[NDT][4];
  uint2 k2[NDT][4], pv2[NDT][4], pk2[NDT][4];
  auto load_terms = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * (NDT * dh + t) + 8 * a + 4 * hi;
      m4[t][a] = *reinterpret_cast<const float4*>(mv + d0);
      k2[t][a] = *reinterpret_cast<const uint2*>(Kraw + krow + d0);
      if (add) {
        pv2[t][a] = *reinterpret_cast<const uint2*>(dV + krow + d0);
        pk2[t][a] = *reinterpret_cast<const uint2*>(dK + krow + d0);
      }
    }
  };
  f32x16 yv[NDT], yk[NDT];
  __syncthreads();  // every wavefront is done with the stages
  stage_set(fragMT);
  wait_vm<0>();
  __syncthreads();
  products(ff, yv);
  __syncthreads();  // M^T read by every wavefront
  load_terms(0);
  stage_set(fragM);
  wait_vm<0>();
  __syncthreads();
  products(vf, yk);
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    if (t + 1 < NDT) load_terms(t + 1);
    if (!kv) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * (NDT * dh + t) + 8 * a + 4 * hi;
      const float MM[4] = {m4[t][a].x, m4[t][a].y, m4[t][a].z, m4[t][a].w};
      const float kk4[4] = {bf2f(k2[t][a].x & 0xffffu), bf2f(k2[t][a].x >> 16), bf2f(k2[t][a].y & 0xffffu),
                            bf2f(k2[t][a].y >> 16)};
      float ov[4], ok[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ov[c] = os * (yv[t][4 * a + c] - adv[t][4 * a + c]);
        ok[c] = os * dphi(kk4[c]) * (yk[t][4 * a + c] - MM[c] - adk[t][4 * a + c]);
      }
      if (add) {
        add4(pv2[t][a], ov);
        add4(pk2[t][a], ok);
      }
      store4(dV + krow + d0, ov);
      store4(dK + krow + d0, ok);
    }
  }
}

template <int D, int BQ, int SUB>
hipError_t lin_dispatch(const Shape& s, const void* Qv, const void* Kv, const void* Vv, const void* dOv,
                        const int32_t* rp, const int32_t* ci, void* dQ, void* dK, void* dV, bool add,
                        const float* alpha, bool csc, char* ws, const BwdLayout& L, hipStream_t st,
                        const BwdSaved* saved) {
  const long long BH = (long long)s.B * s.H;
  const long long QP = (long long)s.Nq * s.bq;  // per-query arrays: [bh * QP + t]
  const uint16_t* Q = static_cast<const uint16_t*>(Qv);
  const uint16_t* K = static_cast<const uint16_t*>(Kv);
  const uint16_t* V = static_cast<const uint16_t*>(Vv);
  const uint16_t* G = static_cast<const uint16_t*>(dOv);
  uint16_t* A = reinterpret_cast<uint16_t*>(ws + L.phiq);
  uint16_t* F = reinterpret_cast<uint16_t*>(ws + L.phik);
  uint4* frag0 = reinterpret_cast<uint4*>(ws + L.rsplit);
  uint4* frag1 = frag0 + (size_t)BH * (2 * (D / 32) * (D / 16) * 64);
  float* invden = reinterpret_cast<float*>(ws + L.invden);
  float* dtq = reinterpret_cast<float*>(ws + L.dt);
  float* tot_h = reinterpret_cast<float*>(ws + L.tot_h);
  float* tot_m = reinterpret_cast<float*>(ws + L.tot_m);
  float* part = reinterpret_cast<float*>(ws + L.lpart);
  const int per = D * D + D;
  hipError_t e = hipSuccess;
  if (csc && (e = launch_csc(s, rp, ci, ws, L, st)) != hipSuccess) return e;
  const long long n8 = BH * s.N * D / 8;
  hipLaunchKernelGGL(lin_phi_kernel, dim3((unsigned)((2 * n8 + 255) / 256)), dim3(256), 0, st, Q, K, n8, A, F);
  // H, z
  hipLaunchKernelGGL((lin_outer_kernel<D>), dim3((unsigned)L.lchunks, (unsigned)BH), dim3(256), 0, st, K, V,
                     (const float*)nullptr, (const float*)nullptr, s.N, QP, L.lchunks, part);
  if ((e = launch_summary_reduce(part, nullptr, s.H, BH, L.lchunks, per, tot_h, st)) != hipSuccess) return e;
  // H as matrix-core fragments for the rows' H h
  const dim3 gsplit((unsigned)((D / 32 * D / 16 * 64 + 255) / 256), (unsigned)BH);
  hipLaunchKernelGGL((lin_split_kernel<D>), gsplit, dim3(256), 0, st, tot_h, 0, frag0);
  // rows: den, D~ and dq
  hipLaunchKernelGGL((lin_dq_kernel<D, BQ, SUB>), dim3((unsigned)s.R()), dim3(BQ / 32 * 64), 0, st, A, F, V, G, Q,
                     rp, ci, frag0, tot_h, invden, dtq, static_cast<uint16_t*>(dQ), add ? 1 : 0, alpha, s.H, s.N,
                     s.Nq, s.Nk, saved ? saved->invden : nullptr, saved ? saved->ol : nullptr);
  // M = sum (phi(q) / den) h^T, m = sum (D~ / den) phi(q)
  hipLaunchKernelGGL((lin_outer_kernel<D>), dim3((unsigned)L.lchunks, (unsigned)BH), dim3(256), 0, st, Q, G, invden,
                     dtq, s.N, QP, L.lchunks, part);
  if ((e = launch_summary_reduce(part, nullptr, s.H, BH, L.lchunks, per, tot_m, st)) != hipSuccess) return e;
  // M^T and M as fragments for the keys' M^T phi(k) and M v
  hipLaunchKernelGGL((lin_split_kernel<D>), gsplit, dim3(256), 0, st, tot_m, 1, frag0);
  hipLaunchKernelGGL((lin_split_kernel<D>), gsplit, dim3(256), 0, st, tot_m, 0, frag1);
  // keys: dk, dv
  const int* col_ptr = reinterpret_cast<const int*>(ws + L.col_ptr);
  const int* row_idx = reinterpret_cast<const int*>(ws + L.row_idx);
  const int* order = reinterpret_cast<const int*>(ws + L.order);
  hipLaunchKernelGGL((lin_dkdv_kernel<D, BQ, SUB>), dim3((unsigned)(BH * s.Nk * SUB)), dim3(256), 0, st, A, F, V, G,
                     K, col_ptr, row_idx, order, invden, dtq, frag0, frag1, tot_m, static_cast<uint16_t*>(dK),
                     static_cast<uint16_t*>(dV), add ? 1 : 0, alpha, s.H, s.N, s.Nq, s.Nk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_bwd(const Shape& s, const void* Q, const void* K, const void* V, const void* dO,
                             const int32_t* rp, const int32_t* ci, void* dQ, void* dK, void* dV, bool accumulate,
                             const float* alpha, bool csc, char* ws, const BwdLayout& L, hipStream_t st,
                             const BwdSaved* saved) {
#define SLA_LBWD(DD, QQ, KK) \
  if (s.d == DD && s.bq == QQ && s.bk == KK) \
    return lin_dispatch<DD, QQ, KK / 64>(s, Q, K, V, dO, rp, ci, dQ, dK, dV, accumulate, alpha, csc, ws, L, st, \
                                         saved);
  SLA_LBWD(128, 128, 64)
  SLA_LBWD(128, 128, 128)
  SLA_LBWD(128, 64, 64)
  SLA_LBWD(128, 64, 128)
  SLA_LBWD(64, 128, 64)
  SLA_LBWD(64, 128, 128)
  SLA_LBWD(64, 64, 64)
  SLA_LBWD(64, 64, 128)
#undef SLA_LBWD
  return hipErrorInvalidValue;
}

}  // namespace sla
