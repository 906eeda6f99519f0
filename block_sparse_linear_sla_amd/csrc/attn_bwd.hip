// Backward of the sparse branch (bf16) on gfx950 matrix cores.
//
// Source: SLA2 write-up (arXiv:2602.12675) §一 (the sparse branch: exact
// softmax attention of each query over the keys of its selected blocks) and
// §四 (the attention is trained end to end with the block selection fixed per
// step).  With the mask held fixed, for each (query block i, key block j) pair
// of the mask and P = softmax over the row's selected keys:
//   dV_j += P^T dO_i,   dP = dO_i V_j^T,   dS = P o (dP - D_i),
//   dQ_i += dS K_j / sqrt(d),   dK_j += dS^T Q_i / sqrt(d),
// with D_t = dO_t . O_t = sum_u P_tu dP_tu per query - the textbook
// softmax-attention gradient restricted to the listed pairs.  D is formed
// here from the second form, in float32 with the same P as the gradient
// (rather than from a rounded forward output, whose error would shift every
// dS of the row by the same amount).
//
// Kernels:
//   csc_bits_kernel / csc_count_kernel / csc_scan_kernel / csc_fill_kernel
//       the mask's transpose: the rows as bitmasks (one thread per row),
//       then for each key block the query blocks that list it, in ascending
//       order (one thread per key block and 64-row chunk reads its bit of
//       each row; column totals are scanned, and a chunk's rows go after
//       those of the column's earlier chunks: deterministic, no atomics).
//       The scan also orders the column kernels' units by their column's
//       total, largest first: a key block listed by many query blocks is
//       the longest workgroup, and started late it would finish alone;
//   bwd_dq_kernel    one workgroup per mask row (BQ/32 wavefronts, 32
//       queries each, queries on the lane axis as in the forward).  Pass A
//       walks the row's 64-key units with S^T = K Q^T and dP^T = V dO^T for
//       each query's log-sum-exp and D (online, like the forward's softmax);
//       pass B recomputes both, forms dS in registers, and accumulates
//       dQ^T += K^T dS^T with K read transposed (as the forward reads V).
//       Writes dQ, and the log-sum-exp (base 2) and D of every query for the
//       next kernel (+inf / 0 past N);
//   bwd_dkdv_kernel  one workgroup per 64-key unit, walking the query blocks
//       that list its key block in 64-query units.  Wavefront w keeps the
//       K and V rows of 32 keys (half w%2) in registers and the dK^T, dV^T
//       tiles of half w/2 of d.  Per unit it forms S = Q K^T and dP = dO V^T
//       (queries x keys, keys on the lane axis) for half w/2 of the queries,
//       P and dS in registers, swaps those operands with the wavefront that
//       shares its keys (through LDS), then accumulates dV^T += dO^T P and
//       dK^T += Q^T dS over all of the unit's queries with Q and dO read
//       transposed (the reads a few products ahead of their MFMAs).  The
//       per-query log-sum-exp and D come one value per lane with the unit's
//       tiles and reach the accumulator elements by row broadcasts, and the
//       operand swap's barrier leaves the next unit's loads in flight.
#include "sla.h"
#include <algorithm>

#include "sla_internal.h"
#include "bf16_tiles.h"

namespace sla {
namespace {

// ------------------------------------------------------------ mask transpose
// bits[r][w]: bit j%32 of word j/32 set when row r lists key block j (one
// thread per row writes all of its row's words)
__global__ __launch_bounds__(256) void csc_bits_kernel(const int* __restrict__ row_ptr,
                                                       const int* __restrict__ col_idx, long long R, int words,
                                                       uint32_t* __restrict__ bits) {
  const long long r = (long long)blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  uint32_t* row = bits + r * words;
  for (int x = 0; x < words; ++x) row[x] = 0u;
  for (int p = row_ptr[r]; p < row_ptr[r + 1]; ++p) {
    const int j = col_idx[p];
    row[j >> 5] |= 1u << (j & 31);
  }
}

// The transpose works on (column, chunk) cells: column c = bh * Nk + j, chunk
// k = rows [64 k, 64 k + 64) of the head.  counts[c * nch + k] = rows of the
// chunk that list j (one thread per cell; the 32 threads of a bitmask word
// read it together).
constexpr int CROWS = 64;
__global__ __launch_bounds__(256) void csc_count_kernel(const uint32_t* __restrict__ bits, int Nq, int Nk,
                                                        int words, int nch, long long BH,
                                                        int* __restrict__ counts) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= BH * Nk * nch) return;
  const int k = (int)(t % nch);
  const long long c = t / nch;
  const long long bh = c / Nk;
  const int j = (int)(c % Nk);
  const uint32_t* b = bits + bh * Nq * words + (j >> 5);
  int n = 0;
  const int i1 = min(Nq, (k + 1) * CROWS);
  for (int i = k * CROWS; i < i1; ++i) n += (b[(size_t)i * words] >> (j & 31)) & 1u;
  counts[t] = n;
}

// col_ptr = exclusive prefix sum of the column totals (each the sum of the
// column's nch cell counts; n columns, one workgroup): 1024 consecutive
// columns per pass, a shuffle scan within each wavefront, then one across the
// 16 wavefronts, plus the carry of the earlier passes.
// Then the launch order of the column kernels' units (sub 64-key units per
// column): by the column's total in OB classes of rows, largest first, so
// the longest workgroups start first and the short ones fill in behind them
// (a column listed by many query blocks would otherwise often start late
// and finish alone).  Within a class the order is whatever the LDS atomics
// give: it decides only which workgroup runs which unit, not any result.
constexpr int OB = 64;
__global__ __launch_bounds__(1024) void csc_scan_kernel(const int* __restrict__ counts, long long n, int nch,
                                                        int Nq, int sub, int* __restrict__ col_ptr,
                                                        int* __restrict__ order) {
  __shared__ int wsum[16];
  __shared__ int carry;
  __shared__ int cls[OB];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  if (t == 0) carry = 0;
  __syncthreads();
  for (long long base = 0; base < n; base += 1024) {
    const long long x = base + t;
    int v = 0;
    if (x < n)
      for (int k = 0; k < nch; ++k) v += counts[x * nch + k];
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int wpre = 0;
    for (int u = 0; u < wv; ++u) wpre += wsum[u];
    const int c0 = carry;
    if (x < n) col_ptr[x] = c0 + wpre + incl - v;
    __syncthreads();  // every thread has read wsum and carry
    if (t == 1023) carry = c0 + wpre + incl;
    __syncthreads();
  }
  if (t == 0) col_ptr[n] = carry;
  if (t < OB) cls[t] = 0;
  __syncthreads();  // col_ptr complete and visible to the workgroup
  auto class_of = [&](long long c) { return (OB - 1) - (int)((long long)(col_ptr[c + 1] - col_ptr[c]) * OB / (Nq + 1)); };
  for (long long c = t; c < n; c += 1024) atomicAdd(&cls[class_of(c)], sub);
  __syncthreads();
  if (t < 64) {  // exclusive scan of the OB class sizes (one wavefront)
    const int v = t < OB ? cls[t] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (t >= off) incl += y;
    }
    if (t < OB) cls[t] = incl - v;
  }
  __syncthreads();
  const long long units = n * sub;
  for (long long u = t; u < units; u += 1024) {
    const int pos = atomicAdd(&cls[class_of(u / sub)], 1);
    if (pos < units) order[pos] = (int)u;
  }
}

// row_idx[...] = the rows of cell (c, k) that list j, ascending, starting
// after the column's earlier cells
__global__ __launch_bounds__(256) void csc_fill_kernel(const uint32_t* __restrict__ bits, int Nq, int Nk,
                                                       int words, int nch, long long BH,
                                                       const int* __restrict__ counts,
                                                       const int* __restrict__ col_ptr, int* __restrict__ row_idx) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= BH * Nk * nch) return;
  const int k = (int)(t % nch);
  const long long c = t / nch;
  const long long bh = c / Nk;
  const int j = (int)(c % Nk);
  int o = col_ptr[c];
  for (int k2 = 0; k2 < k; ++k2) o += counts[c * nch + k2];
  const uint32_t* b = bits + bh * Nq * words + (j >> 5);
  const int i1 = min(Nq, (k + 1) * CROWS);
  for (int i = k * CROWS; i < i1; ++i)
    if ((b[(size_t)i * words] >> (j & 31)) & 1u) row_idx[o++] = i;
}

// ------------------------------------------------------------------ helpers
// Store the D/32-row-tile accumulators acc (rows d = 32 (T0 + t) + ..., one
// column per lane: this lane's row `row`) times scale as bf16, NT tiles.
// Each 16-byte store holds 8 consecutive d of one row: lanes l and l^32 hold
// the two 4-d halves of every 8-d chunk and swap one of them.
template <int NT>
__device__ __forceinline__ void store_T(const f32x16 (&acc)[NT], float scale, uint16_t* dst, int d0, bool valid,
                                        int hi) {
#pragma unroll
  for (int mt = 0; mt < NT; ++mt) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint2 pv[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int i4 = 2 * j + c;
        pv[c] = make_uint2(pk_bf16(scale * acc[mt][4 * i4], scale * acc[mt][4 * i4 + 1]),
                           pk_bf16(scale * acc[mt][4 * i4 + 2], scale * acc[mt][4 * i4 + 3]));
      }
      const uint2 send = hi ? pv[0] : pv[1];
      const uint2 recv = make_uint2(__shfl_xor(send.x, 32), __shfl_xor(send.y, 32));
      const uint4 outv = hi ? make_uint4(recv.x, recv.y, pv[1].x, pv[1].y)
                            : make_uint4(pv[0].x, pv[0].y, recv.x, recv.y);
      if (valid) *reinterpret_cast<uint4*>(dst + d0 + 32 * mt + 16 * j + 8 * hi) = outv;
    }
  }
}

// ------------------------------------------------------------------ dQ
template <int D, int BQ, int SUB>
__global__ __launch_bounds__(BQ / 32 * 64, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const int* __restrict__ row_ptr,
    const int* __restrict__ col_idx, uint16_t* __restrict__ dQ, float* __restrict__ lse2_out,
    float* __restrict__ dd_out, const float* __restrict__ alpha, int H, int N, int Nq, int Nk, float scale_log2,
    float inv_sqrt_d, const float* __restrict__ lse2_in, const float* __restrict__ os_in) {
  using T = Tiles<D>;
  constexpr int NW = BQ / 32;
  using LP = LoadPlan<D, NW>;
  constexpr int STAGE = 2 * T::KT_BYTES;
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
  const int nunits = (row_ptr[row + 1] - base) * SUB;
  const int q = qi * BQ + 32 * w + (lane & 31);
  const bool qv = q < N;

  bf16x8 qf[D / 16], df[D / 16];
  load_q<D>(Q, bh, q, N, hi, qf);
  load_q<D>(dO, bh, q, N, hi, df);
  float dd = 0.f;  // D of this query (after pass A)

  f32x16 acc[D / 32];
  float lse2 = INFINITY;  // log2-sum-exp of the scaled scores; +inf: no key (P = 0)
  // with the forward's terms: lse2 as it kept it and D = dO . O_s (this
  // lane's half of d, then the pair sum); pass A is skipped
  const bool saved = lse2_in != nullptr;
  if (saved) {
    float part = 0.f;
    if (qv) {
      const float* orow = os_in + ((size_t)bh * N + q) * D;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const uint4 a = __builtin_bit_cast(uint4, df[t]);
        const float4 o0 = *reinterpret_cast<const float4*>(orow + 16 * t + 8 * hi);
        const float4 o1 = *reinterpret_cast<const float4*>(orow + 16 * t + 8 * hi + 4);
        const float o[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf(bf2f(elem(a, e)), o[e], part);
      }
    }
    dd = part + __shfl_xor(part, 32);
    lse2 = qv ? lse2_in[(size_t)row * BQ + 32 * w + (lane & 31)] : INFINITY;
  }
  if (nunits > 0) {
    const auto rk = buf_rsrc(K + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
    const auto rv = buf_rsrc(V + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
    auto key0 = [&](int x) {
      const int u = x % nunits;  // pass A units, then pass B units
      return (col_idx[base + u / SUB] * SUB + u % SUB) * KU;
    };
    auto issue = [&](int x, char* sb) __attribute__((always_inline)) {
      const LP lp(w, opaque(lane));
      const int k0 = key0(x);
      lp.load(rk, k0, sb);
      lp.load(rv, k0, sb + T::KT_BYTES);
    };
    // S (keys past N at -inf) and dP of key half KT of the unit at kcur
    auto scores = [&](const char* cur, int kcur, auto kt_tag, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
      constexpr int KT = decltype(kt_tag)::value;
      const int limh = min(KU, N - kcur) - 32 * KT - 4 * hi;  // element i: key 32 KT + 8 (i/4) + 4 hi + i%4
      s = score_half<D, KT, 2>(cur, qf, rdp);
      if (limh < 32 - 4 * hi) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) >= limh) s[i] = -INFINITY;
      }
      dp = score_half<D, KT, 2>(cur + T::KT_BYTES, df, rdp);
    };
    // pass A: running max (raw scores), sum of exp2 and sum of exp2 * dP
    float m = -INFINITY, l = 0.f, dn = 0.f;
    auto stepA = [&](int x, char* cur, char* nxt) __attribute__((always_inline)) {
      const int kcur = key0(x);
      wait_vm<0>();
      __syncthreads();
      issue(x + 1, nxt);  // after the last unit: pass B's first
      static_for<2>([&](auto kt) __attribute__((always_inline)) {
        f32x16 s, dp;
        scores(cur, kcur, kt, s, dp);
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
        const float mn = fmaxf(m, mx);
        if (mn != -INFINITY) {
          float sl = 0.f, sd = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f((s[i] - mn) * scale_log2);
            sl += e;
            sd = fmaf(e, dp[i], sd);
          }
          const float c = __builtin_amdgcn_exp2f((m - mn) * scale_log2);
          l = l * c + sl;
          dn = dn * c + sd;
          m = mn;
        }
        // one 32-key half at a time: keeps the two halves' scores from being live together
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // pass B: dS in registers, dQ^T += K^T dS^T with K read transposed
    auto stepB = [&](int x, char* cur, char* nxt) __attribute__((always_inline)) {
      const int kcur = key0(x);
      wait_vm<0>();
      __syncthreads();
      if (x + 1 < nunits) issue(x + 1, nxt);
      static_for<2>([&](auto kt) __attribute__((always_inline)) {
        f32x16 s, dp;
        scores(cur, kcur, kt, s, dp);
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -lse2));
          ds[i] = p * (dp[i] - dd);
        }
        bf16x8 bp[2];
        pack_planes(ds, bp);
        row_products<D, decltype(kt)::value, BWD_PF>(cur, rdp, bp, acc);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // two loops, so that pass A holds no dQ accumulators; the unit after
    // pass A's last (pass B's first) sits in stage nunits % 2
    issue(0, st0);
    if (!saved) {
      int x = 0;
      for (; x + 2 <= nunits; x += 2) {
        stepA(x, st0, st1);
        stepA(x + 1, st1, st0);
      }
      if (x < nunits) stepA(x, st0, st1);
      // the query's log2-sum-exp and D over both key halves (lanes l, l^32)
      const float M = pair_max(m);
      const float c = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - M) * scale_log2);
      const float L = l * c + __shfl_xor(l * c, 32);
      const float Dn = dn * c + __shfl_xor(dn * c, 32);
      lse2 = M * scale_log2 + __log2f(L);
      dd = Dn / L;
    }
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    auto passB = [&](char* b0, char* b1) __attribute__((always_inline)) {
      int y = 0;
      for (; y + 2 <= nunits; y += 2) {
        stepB(y, b0, b1);
        stepB(y + 1, b1, b0);
      }
      if (y < nunits) stepB(y, b0, b1);
    };
    // pass B's first unit sits in stage nunits % 2 after pass A, in stage 0
    // without it
    if (saved || nunits % 2 == 0) passB(st0, st1);
    else passB(st1, st0);
    wait_vm<0>();
  } else {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
  }
  const size_t qrow = (size_t)bh * N + min(q, N - 1);
  const float os = alpha != nullptr ? alpha[bh % H] : 1.f;  // the branch's weight in the mixed output
  store_T<D / 32>(acc, os * inv_sqrt_d, dQ + qrow * D, 0, qv, hi);
  if (hi == 0) {
    const size_t r = (size_t)row * BQ + 32 * w + (lane & 31);
    lse2_out[r] = qv ? lse2 : INFINITY;
    dd_out[r] = qv ? dd : 0.f;
  }
}

// ------------------------------------------------------------------ dK, dV
template <int D, int BQ, int SUB>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const int* __restrict__ col_ptr, const int* __restrict__ row_idx,
    const int* __restrict__ order, const float* __restrict__ lse2, const float* __restrict__ ddv, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, const float* __restrict__ alpha, int H, int N, int Nq, int Nk, float scale_log2,
    float inv_sqrt_d) {
  using T = Tiles<D>;
  using LP = LoadPlan<D, 4>;
  constexpr int STAGE = 2 * T::KT_BYTES;  // Q and dO tiles of 64 queries
  constexpr int NDT = D / 64;             // 32-row d tiles per wavefront (half of d)
  constexpr int QU = BQ / KU;             // 64-query units per query block
  constexpr int XCH = 4 * 64 * 16;        // one wavefront's P and dS operands (2 planes each)
  static_assert(2 * (2 * STAGE + 4 * XCH) <= LDS_BYTES, "two workgroups per compute unit");
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint4 xch[4][4][64];  // [wavefront][operand][lane]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  // key half kh (32 keys); wavefront pair (kh, 0), (kh, 1) share those keys:
  // each scores half dh of every unit's queries and accumulates half dh of d
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

  bf16x8 kf[D / 16], vf[D / 16];
  load_q<D>(K, bh, key, N, hi, kf);
  load_q<D>(V, bh, key, N, hi, vf);
  f32x16 adv[NDT], adk[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    adv[t] = f32x16{};
    adk[t] = f32x16{};
  }
  if (nunits > 0) {
    const auto rq = buf_rsrc(Q + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
    const auto rg = buf_rsrc(dO + (size_t)bh * N * D, (uint32_t)((size_t)N * D * 2));
    // first query of unit x, and its mask row (for the per-query terms)
    auto qrow_of = [&](int x) { return row_idx[cb + x / QU]; };
    auto issue = [&](int x, char* sb) __attribute__((always_inline)) {
      const LP lp(w, opaque(lane));
      const int q0 = qrow_of(x) * BQ + (x % QU) * KU;
      lp.load(rq, q0, sb);
      lp.load(rg, q0, sb + T::KT_BYTES);
    };
    // S and dP of this wavefront's 32 queries (half QH of the unit) x its 32
    // keys (element i: query 32 QH + 8 (i/4) + 4 hi + i%4, key = this
    // lane's); P and dS packed as the B operands of query planes 2 QH, 2 QH + 1
    auto score = [&](const char* cur, float Lc, float Dc, bf16x8 (&bp)[2], bf16x8 (&bs)[2], auto qh_tag)
        __attribute__((always_inline)) {
      constexpr int QH = decltype(qh_tag)::value;
      const f32x16 s = score_half<D, QH, 4>(cur, kf, rdp);
      const f32x16 dp = score_half<D, QH, 4>(cur + T::KT_BYTES, vf, rdp);
      float pv[16], ds[16];
      static_for<16>([&](auto it) __attribute__((always_inline)) {
        constexpr int i = decltype(it)::value;
        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -row_bcast<i>(Lc)));
        pv[i] = p;
        ds[i] = p * (dp[i] - row_bcast<i>(Dc));
      });
      pack_planes(pv, bp);
      pack_planes(ds, bs);
    };
    // the unit's per-query terms (log2-sum-exp and D), one value per lane
    // (term_query) of this wavefront's 32 queries, loaded with the unit's
    // tiles so that the only wait for them is the one for the tiles
    const int tq = 32 * dh + term_query(lane);
    auto terms_at = [&](int x) { return ((size_t)(bh * Nq + qrow_of(x))) * BQ + (x % QU) * KU + tq; };
    float Ln = lse2[terms_at(0)], Dn = ddv[terms_at(0)];
    auto step = [&](int x, char* cur, char* nxt) __attribute__((always_inline)) {
      wait_vm<0>();
      __syncthreads();  // the unit's tiles landed; the previous unit's exchange consumed
      const float Lc = Ln, Dc = Dn;
      if (x + 1 < nunits) {
        const size_t tn = terms_at(x + 1);
        Ln = lse2[tn];
        Dn = ddv[tn];
        issue(x + 1, nxt);
      }
      // all operand indices below are compile-time (a runtime index would put
      // the operand array in scratch memory)
      auto body = [&](auto qh_tag) __attribute__((always_inline)) {
        constexpr int QH = decltype(qh_tag)::value;
        constexpr int OWN = 2 * QH, OTH = 2 - OWN;
        bf16x8 op[2][4];  // [P, dS][query plane 0..3]
        bf16x8 bp[2], bs[2];
        score(cur, Lc, Dc, bp, bs, qh_tag);
        op[0][OWN] = bp[0];
        op[0][OWN + 1] = bp[1];
        op[1][OWN] = bs[0];
        op[1][OWN + 1] = bs[1];
        // hand this half's operands to the partner, take the partner's half
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
        // dV^T += dO^T P and dK^T += Q^T dS over the unit's four query
        // planes, d rows of this wavefront's half
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
  const size_t krow = ((size_t)bh * N + min(key, N - 1)) * D;
  const float os = alpha != nullptr ? alpha[bh % H] : 1.f;
  store_T<NDT>(adv, os, dV + krow, 32 * NDT * dh, kv, hi);
  store_T<NDT>(adk, os * inv_sqrt_d, dK + krow, 32 * NDT * dh, kv, hi);
}

// ------------------------------------------------------------------ d alpha
// Partial sums of dO . (O_s - O_l) over chunks of one (b, h) slice: each
// workgroup sums ACH elements in float64 (fixed order: thread-strided, then a
// tree), one partial per (bh, chunk).
constexpr int ACH = 65536;
template <int ES>
__global__ __launch_bounds__(256) void alpha_part_kernel(const char* __restrict__ dO, const char* __restrict__ Os,
                                                         const char* __restrict__ Ol, long long per, int nch,
                                                         double* __restrict__ part) {
  constexpr int VE = 16 / ES;  // elements per 16-byte load (per is a multiple: d is 64 or 128)
  __shared__ double red[256];
  const long long bh = blockIdx.y;
  const long long a = (long long)blockIdx.x * ACH, b = min(per, a + ACH);
  double acc = 0.0;
  for (long long e = a + (long long)threadIdx.x * VE; e < b; e += 256 * VE) {
    const size_t o = (size_t)(bh * per + e) * ES;
    const uint4 g4 = *reinterpret_cast<const uint4*>(dO + o);
    const uint4 x4 = *reinterpret_cast<const uint4*>(Os + o);
    const uint4 y4 = *reinterpret_cast<const uint4*>(Ol + o);
    if (ES == 2) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        acc += (double)bf2f(elem(g4, k)) * ((double)bf2f(elem(x4, k)) - (double)bf2f(elem(y4, k)));
    } else {
      const float g[4] = {__uint_as_float(g4.x), __uint_as_float(g4.y), __uint_as_float(g4.z), __uint_as_float(g4.w)};
      const float x[4] = {__uint_as_float(x4.x), __uint_as_float(x4.y), __uint_as_float(x4.z), __uint_as_float(x4.w)};
      const float y[4] = {__uint_as_float(y4.x), __uint_as_float(y4.y), __uint_as_float(y4.z), __uint_as_float(y4.w)};
#pragma unroll
      for (int k = 0; k < 4; ++k) acc += (double)g[k] * ((double)x[k] - (double)y[k]);
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[bh * nch + blockIdx.x] = red[0];
}

// dalpha[h] = sum over b and chunks, in order
__global__ __launch_bounds__(64) void alpha_sum_kernel(const double* __restrict__ part, int B, int H, int nch,
                                                       float* __restrict__ dalpha) {
  const int h = blockIdx.x * 64 + threadIdx.x;
  if (h >= H) return;
  double s = 0.0;
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < nch; ++c) s += part[((long long)b * H + h) * nch + c];
  dalpha[h] = (float)s;
}

template <int D, int BQ, int SUB>
hipError_t bwd_dispatch(const Shape& s, const void* Q, const void* K, const void* V, const void* dO, const int32_t* rp,
                        const int32_t* ci, void* dQ, void* dK, void* dV, const float* alpha, bool csc, char* ws,
                        const BwdLayout& L, hipStream_t st, const BwdSaved* saved) {
  const long long BH = (long long)s.B * s.H;
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const float isd = 1.f / sqrtf((float)D);
  const int* col_ptr = reinterpret_cast<const int*>(ws + L.col_ptr);
  const int* row_idx = reinterpret_cast<const int*>(ws + L.row_idx);
  const int* order = reinterpret_cast<const int*>(ws + L.order);
  float* lse2 = reinterpret_cast<float*>(ws + L.lse2);
  float* ddv = reinterpret_cast<float*>(ws + L.dd);
  if (csc) {
    const hipError_t e = launch_csc(s, rp, ci, ws, L, st);
    if (e != hipSuccess) return e;
  }
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(K);
  const uint16_t* v = static_cast<const uint16_t*>(V);
  const uint16_t* g = static_cast<const uint16_t*>(dO);
  hipLaunchKernelGGL((bwd_dq_kernel<D, BQ, SUB>), dim3((unsigned)s.R()), dim3(BQ / 32 * 64), 0, st, q, k, v,
                     g, rp, ci, static_cast<uint16_t*>(dQ), lse2, ddv, alpha, s.H, s.N, s.Nq, s.Nk, sl2, isd,
                     saved ? saved->lse2 : nullptr, saved ? saved->os : nullptr);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, BQ, SUB>), dim3((unsigned)(BH * s.Nk * SUB)), dim3(256), 0, st, q, k, v,
                     g, col_ptr, row_idx, order, lse2, ddv, static_cast<uint16_t*>(dK), static_cast<uint16_t*>(dV),
                     alpha, s.H, s.N, s.Nq, s.Nk, sl2, isd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_csc(const Shape& s, const int32_t* rp, const int32_t* ci, char* ws, const BwdLayout& L,
                      hipStream_t st) {
  const long long BH = (long long)s.B * s.H;
  int* counts = reinterpret_cast<int*>(ws + L.counts);
  int* col_ptr = reinterpret_cast<int*>(ws + L.col_ptr);
  int* row_idx = reinterpret_cast<int*>(ws + L.row_idx);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + L.bits);
  const int words = s.words();
  const int nch = (s.Nq + CROWS - 1) / CROWS;
  const long long ncell = BH * s.Nk * nch;
  const unsigned gcell = (unsigned)((ncell + 255) / 256);
  hipLaunchKernelGGL(csc_bits_kernel, dim3((unsigned)((s.R() + 255) / 256)), dim3(256), 0, st, rp, ci, s.R(), words,
                     bits);
  hipLaunchKernelGGL(csc_count_kernel, dim3(gcell), dim3(256), 0, st, bits, s.Nq, s.Nk, words, nch, BH, counts);
  int* order = reinterpret_cast<int*>(ws + L.order);
  hipLaunchKernelGGL(csc_scan_kernel, dim3(1), dim3(1024), 0, st, counts, BH * s.Nk, nch, s.Nq, s.bk / KU, col_ptr,
                     order);
  hipLaunchKernelGGL(csc_fill_kernel, dim3(gcell), dim3(256), 0, st, bits, s.Nq, s.Nk, words, nch, BH, counts,
                     col_ptr, row_idx);
  return hipGetLastError();
}

BwdLayout bwd_layout(const Shape& s) {
  BwdLayout L{};
  const size_t BH = (size_t)s.B * s.H;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return o;
  };
  L.bits = take((size_t)s.R() * s.words() * sizeof(uint32_t));
  const size_t ncell = BH * s.Nk * (size_t)((s.Nq + CROWS - 1) / CROWS);
  L.counts = take(ncell * sizeof(int));
  L.col_ptr = take((BH * s.Nk + 1) * sizeof(int));
  L.row_idx = take(BH * (size_t)s.Nq * s.Nk * sizeof(int));
  L.order = take(BH * s.Nk * (size_t)(s.bk / 64) * sizeof(int));
  L.lse2 = take((size_t)s.R() * s.bq * sizeof(float));
  L.dd = take((size_t)s.R() * s.bq * sizeof(float));
  L.achunks = (int)(((long long)s.N * s.d + ACH - 1) / ACH);
  L.apart = take(BH * L.achunks * sizeof(double));
  // linear branch
  const size_t rows = BH * (size_t)s.N * s.d;
  const size_t per = (size_t)s.d * s.d + s.d;
  L.lchunks = (s.N + LROWS - 1) / LROWS;
  L.phiq = take(rows * 2);
  L.phik = take(rows * 2);
  L.rsplit = take(2 * BH * (size_t)(s.d / 32) * (s.d / 16) * 2 * 64 * 16);
  L.invden = take((size_t)s.R() * s.bq * sizeof(float));
  L.dt = take((size_t)s.R() * s.bq * sizeof(float));
  L.tot_h = take(BH * per * sizeof(float));
  L.tot_m = take(BH * per * sizeof(float));
  L.lpart = take(BH * L.lchunks * per * sizeof(float));
  L.total = off;
  return L;
}

// The alpha gradient from the row kernels' per-query terms: dO . (O_s - O_l)
// = D - D~ for every query, so each head's sum is a float64 sum of those
// differences (chunks of `chunk` queries in a fixed order, then
// alpha_sum_kernel).
__global__ __launch_bounds__(256) void alpha_terms_part_kernel(const float* __restrict__ dd,
                                                               const float* __restrict__ dt, long long per,
                                                               long long chunk, int nch, double* __restrict__ part) {
  __shared__ double red[256];
  const long long bh = blockIdx.y;
  const long long a = (long long)blockIdx.x * chunk, b = min(per, a + chunk);
  double acc = 0.0;
  for (long long e = a + threadIdx.x; e < b; e += 256) acc += (double)dd[bh * per + e] - (double)dt[bh * per + e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[bh * nch + blockIdx.x] = red[0];
}

hipError_t launch_alpha_grad_terms(const Shape& s, float* dalpha, char* ws, const BwdLayout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H, per = (long long)s.Nq * s.bq;
  // chunks of 2048 queries (eight per thread) where the partials fit the
  // region sized for L.achunks per head, longer ones otherwise
  const long long chunk = std::max<long long>(2048, (per + L.achunks - 1) / L.achunks);
  const int nch = (int)((per + chunk - 1) / chunk);
  double* part = reinterpret_cast<double*>(ws + L.apart);
  hipLaunchKernelGGL(alpha_terms_part_kernel, dim3((unsigned)nch, (unsigned)BH), dim3(256), 0, st,
                     reinterpret_cast<const float*>(ws + L.dd), reinterpret_cast<const float*>(ws + L.dt), per, chunk,
                     nch, part);
  hipLaunchKernelGGL(alpha_sum_kernel, dim3((unsigned)((s.H + 63) / 64)), dim3(64), 0, st, part, s.B, s.H, nch,
                     dalpha);
  return hipGetLastError();
}

hipError_t launch_alpha_grad(const Shape& s, const void* dO, const void* Os, const void* Ol, float* dalpha,
                             char* ws, const BwdLayout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H, per = (long long)s.N * s.d;
  double* part = reinterpret_cast<double*>(ws + L.apart);
  const dim3 grid((unsigned)L.achunks, (unsigned)BH);
  const char* g = static_cast<const char*>(dO);
  const char* x = static_cast<const char*>(Os);
  const char* y = static_cast<const char*>(Ol);
  if (s.dtype == SLA_BF16)
    hipLaunchKernelGGL(alpha_part_kernel<2>, grid, dim3(256), 0, st, g, x, y, per, L.achunks, part);
  else
    hipLaunchKernelGGL(alpha_part_kernel<4>, grid, dim3(256), 0, st, g, x, y, per, L.achunks, part);
  hipLaunchKernelGGL(alpha_sum_kernel, dim3((unsigned)((s.H + 63) / 64)), dim3(64), 0, st, part, s.B, s.H,
                     L.achunks, dalpha);
  return hipGetLastError();
}

hipError_t launch_sparse_bwd(const Shape& s, const void* Q, const void* K, const void* V, const void* dO,
                             const int32_t* rp, const int32_t* ci, void* dQ, void* dK, void* dV, const float* alpha,
                             bool csc, char* ws, const BwdLayout& L, hipStream_t st, const BwdSaved* saved) {
#define SLA_BWD(DD, QQ, KK) \
  if (s.d == DD && s.bq == QQ && s.bk == KK) \
    return bwd_dispatch<DD, QQ, KK / 64>(s, Q, K, V, dO, rp, ci, dQ, dK, dV, alpha, csc, ws, L, st, saved);
  SLA_BWD(128, 128, 64)
  SLA_BWD(128, 128, 128)
  SLA_BWD(128, 64, 64)
  SLA_BWD(128, 64, 128)
  SLA_BWD(64, 128, 64)
  SLA_BWD(64, 128, 128)
  SLA_BWD(64, 64, 64)
  SLA_BWD(64, 64, 128)
#undef SLA_BWD
  return hipErrorInvalidValue;
}

}  // namespace sla
