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
//   head) streams K and V once and writes phi(K) = elu(K) + 1 as bf16 in 32-wide
//   d slices ([d/32][keys][32], keys up to the last full block, zero past N) and
//   the chunk's partial linear totals H = sum_u phi(k_u)^T v_u, z = sum_u
//   phi(k_u) (phi split into hi + lo bf16 so the totals keep ~16 mantissa bits).
//
// attn_kernel (one workgroup of BQ/32 wavefronts per mask row = (b, h, query
//   block of BQ rows), two workgroups per compute unit) walks the row's key
//   blocks in units of 64 keys.  The K and V tiles of a unit go straight from
//   global memory to LDS (buffer loads with an LDS destination, 16 bytes per
//   lane), row-major with 16-byte chunks XOR-swizzled by key so that both the
//   row reads and the transposed reads of the operands are free of bank
//   conflicts.  With the linear branch, each wavefront also keeps its own
//   slice of phi(K) (the rows of G it accumulates) in a private LDS region.
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
// operand), so P goes from accumulator to operand in registers, and the V^T
// fragment of P V serves again as the B operand of G.
//
// Linear branch: H_u = H - G and z_u = z - g, where G and g are the sums over
// the row's listed blocks, so O_l = phi(Q) H_u / phi(Q) z_u; phi(Q) H_u is a
// hi + lo split product (three bf16 MFMAs), again ~16 mantissa bits.
#include "sla_internal.h"
#include "bf16_tiles.h"

namespace sla {
namespace {

// How the D x D tiles of G = phi(K)^T V are split over NW wavefronts: each
// takes TPW 32 x 32 tiles, MTN whole row tiles (d_k) when it has at least a
// full row, else a part of one row.  Tile u of wavefront w is row tile
// mt0(w) + m(u), column tile nt(w, u).  zown: the wavefront that keeps the
// column sums g of its row tile (one per row tile).
template <int D, int NW>
struct GSplit {
  static constexpr int NCT = D / 32;
  static constexpr int TPW = NCT * NCT / NW;
  static_assert(TPW * NW == NCT * NCT && TPW >= 1, "G split");
  static constexpr int MTN = TPW >= NCT ? TPW / NCT : 1;
  __device__ static int mt0(int w) { return (w * TPW) / NCT; }
  __device__ static int m(int u) { return TPW >= NCT ? u / NCT : 0; }
  __device__ static int nt(int w, int u) { return TPW >= NCT ? u % NCT : (w * TPW + u) % NCT; }
  __device__ static bool zown(int w) { return TPW >= NCT || nt(w, 0) == 0; }
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

// A wavefront's private phi(K) region: MTN row tiles x [64 keys][64 B] (the 32
// d of one row tile, plain row-major: the transposed reads of 4 keys x 64
// bytes by 32 lanes are conflict free).  Filled by 4 direct loads per row
// tile from the [d/32][keys][32] phi(K) array (1 KB contiguous each).
struct PhiPlan {
  int tro;  // lane's transposed-read offset inside a 16-key plane
  __device__ __forceinline__ explicit PhiPlan(int lane) {
    const int i = lane & 15, g2 = (lane >> 4) & 1, hi = lane >> 5;
    tro = (4 * hi + (i >> 2)) * 64 + 2 * (16 * g2 + 4 * (i & 3));
  }
  // key plane pl of row tile m from the region half that holds it
  __device__ __forceinline__ bf16x8 read(const char* half, int m, int pl) const {
    const char* b = half + m * 2048 + (pl & 1) * 1024 + tro;
    return cat_tr(b, b + 512);
  }
};
// Half HF (key planes 2 HF, 2 HF + 1) of a wavefront's phi(K) region for the
// unit starting at key key0: MTN x 2 loads.  The two halves live in distinct
// LDS arrays, so the compiler can tell a load into one half from the reads
// of the other (it would otherwise wait for every load in flight).
template <int MTN, int HF>
__device__ __forceinline__ void load_phi(__amdgpu_buffer_rsrc_t r, int mt0, int Npad, int key0, int lane,
                                         char* half) {
#pragma unroll
  for (int m = 0; m < MTN; ++m) {
    const uint32_t soff = (uint32_t)((mt0 + m) * Npad + key0) * 64u;
#pragma unroll
    for (int j = 2 * HF; j < 2 * HF + 2; ++j)
      b2lds16(r, (uint32_t)(16 * lane + 1024 * j), soff, half + m * 2048 + 1024 * (j & 1));
  }
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

// Online softmax of one wavefront's scores sc over a unit (two 32-key
// subtiles) into the P operands bp of its 4 key planes.  One max exchange and
// rescale test per 64 keys; P = exp2(S c - m c) with c = log2(e)/sqrt(d),
// rounded to bf16; l += sum of the rounded P (v_dot2 with ones).  The running
// max moves only when a unit max exceeds it by more than 2^8 in exp2 units,
// so P <= 2^8 and the O / l rescale is skipped for most units.  lim < 64 marks
// a unit running past N: keys at offset >= lim get score -inf.
template <int D>
__device__ __forceinline__ void softmax_p(f32x16 (&sc)[2], bf16x8 (&bp)[4], f32x16 (&acc_o)[D / 32],
                                          Softmax& sm, int hi, int lim, float scale_log2, float thr8) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
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
    bp[s4] = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));
  }
}

// softmax_p for the 32-key half KT of a unit alone (its P feeds P V before
// the other half's scores move the running max).
template <int D, int KT>
__device__ __forceinline__ void softmax_half(f32x16& sc, bf16x8 (&bp)[2], f32x16 (&acc_o)[D / 32], Softmax& sm,
                                             int hi, int lim, float scale_log2, float thr8) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
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
    bp[j] = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));
  }
}

// The products of key planes PL0 .. PL1-1 of a unit (V tile Vc):
//   DO_S: O^T += V^T P^T (bp: the P operands of those planes);
//   DO_G: G += phi(K)^T V for the wavefront's G tiles (the V^T fragments of
//         P V as the B operand) and, for the wavefront that keeps them, the
//         column sums g of its phi(K) row tiles.  The phi(K)^T fragments of
//         these planes come from Ph, the half of the wavefront's private
//         region that holds them (PL0, PL1 within one half), one plane
//         ahead: ready() runs before the first read (it waits for the
//         region's load), refill() after the last (it hands that part of the
//         region to the next unit's load).
template <int D, int NW, bool DO_S, bool DO_G, int PL0, int PL1, class Ready, class Refill>
__device__ __forceinline__ void pv_g(const char* Vc, const char* Ph, const PhiPlan& pp,
                                     const bf16x8 (&bp)[PL1 - PL0], f32x16 (&acc_o)[D / 32],
                                     f32x16 (&acc_g)[GSplit<D, NW>::TPW], float (&gs)[GSplit<D, NW>::MTN],
                                     const ReadPlan<D>& rp, int w, Ready&& ready, Refill&& refill) {
  using GS = GSplit<D, NW>;
  static_assert(!DO_G || (PL0 % 2 == 0 && PL1 == PL0 + 2), "planes of one region half");
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  bf16x8 vf[D / 32], pf[GS::MTN];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) vf[dt] = rp.vt(Vc, dt, PL0);
  if (DO_G) {
    ready();
#pragma unroll
    for (int m = 0; m < GS::MTN; ++m) pf[m] = pp.read(Ph, m, PL0);
  }
  const bool zw = GS::zown(w);
#pragma unroll
  for (int s4 = PL0; s4 < PL1; ++s4) {
    bf16x8 pc[GS::MTN];
    if (DO_G) {
#pragma unroll
      for (int m = 0; m < GS::MTN; ++m) {
        pc[m] = pf[m];
        if (s4 + 1 < PL1) pf[m] = pp.read(Ph, m, s4 + 1);
      }
      if (s4 + 1 == PL1) refill();
      if (zw) {
#pragma unroll
        for (int m = 0; m < GS::MTN; ++m) {
          const uint4 v = __builtin_bit_cast(uint4, pc[m]);
          gs[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), ones, gs[m], false);
          gs[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), ones, gs[m], false);
          gs[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), ones, gs[m], false);
          gs[m] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), ones, gs[m], false);
        }
      }
    }
    if (GS::TPW >= GS::NCT) {
      // whole rows of G tiles: the fragment of column tile dt feeds P V and
      // the G tiles of that column, then its register takes the next plane's
      // fragment (one set of D/32 fragments live)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const bf16x8 a = vf[dt];
        if (DO_G) {
#pragma unroll
          for (int m = 0; m < GS::MTN; ++m) acc_g[m * GS::NCT + dt] = mfma(pc[m], a, acc_g[m * GS::NCT + dt]);
        }
        if (DO_S) acc_o[dt] = mfma(a, bp[s4 - PL0], acc_o[dt]);
        if (s4 + 1 < PL1) vf[dt] = rp.vt(Vc, dt, s4 + 1);
      }
    } else {
      bf16x8 cur[D / 32];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        cur[dt] = vf[dt];
        if (s4 + 1 < PL1) vf[dt] = rp.vt(Vc, dt, s4 + 1);  // next key plane, one k-step ahead
      }
      if (DO_G) {
#pragma unroll
        for (int u = 0; u < GS::TPW; ++u)
          acc_g[u] = mfma(pc[GS::m(u)], pick_frag<D>(cur, GS::nt(w, u)), acc_g[u]);
      }
      if (DO_S) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc_o[dt] = mfma(cur[dt], bp[s4 - PL0], acc_o[dt]);
      }
    }
  }
}

// Linear-branch preparation of one head's chunk of key blocks (one
// workgroup, four wavefronts): phi(K) = elu(K) + 1 rounded to bf16 into the
// [d/32][Npad][32] array (zero for keys >= N), and the chunk's partial totals
// H = sum_u phi(k_u)^T v_u (in MFMA fragment order: 32 x 32 tile (mt, nt),
// lane, accumulator element) and z = sum_u phi(k_u).  64-key units of K and V
// stream through two LDS stages and are only read there: each thread turns
// its 16-byte chunks of the unit's K tile into phi for the global array,
// and wavefront w accumulates the G tiles of the attention kernel's split
// (GSplit<D, 4>) from transposed reads of the raw K tile (phi applied in
// float32 and split into hi + lo bf16, so H keeps ~16 mantissa bits) and of
// the V tile.  The wavefronts that keep z also sum the raw K values of their
// d rows in float64 (sums of bf16 values, exact in float64) and, with kbar
// given, write each key block's mean there (the mask's pooled K).  Heads
// whose alpha is exactly 1 are skipped when alpha is given.
template <int D, int BK>
__global__ __launch_bounds__(256) void prep_kernel(const uint16_t* __restrict__ K,
                                                   const uint16_t* __restrict__ V,
                                                   const float* __restrict__ alpha, int H, int N, int Nk,
                                                   int chunk_blocks, int nchunk, uint16_t* __restrict__ pk_g,
                                                   float* __restrict__ hpart, double* __restrict__ kbar) {
  using T = Tiles<D>;
  using LP = LoadPlan<D, 4>;
  using GS = GSplit<D, 4>;
  static_assert(GS::MTN == 1, "one row tile per wavefront");
  constexpr int SUB = BK / KU;                  // units per key block
  constexpr int TPW = GS::TPW;
  constexpr int PCH = KU * (D / 8) / 256;       // 16-byte K chunks per thread and unit
  __shared__ __attribute__((aligned(16))) char k0[T::KT_BYTES];
  __shared__ __attribute__((aligned(16))) char k1[T::KT_BYTES];
  __shared__ __attribute__((aligned(16))) char v0[T::KT_BYTES];
  __shared__ __attribute__((aligned(16))) char v1[T::KT_BYTES];

  const long long bh = blockIdx.x / nchunk;
  const int chunk = blockIdx.x % nchunk;
  if (alpha != nullptr && alpha[bh % H] == 1.f) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, l32 = lane & 31;
  const ReadPlan<D> rdp(lane);
  const LP lp(w, lane);
  const int Npad = Nk * BK;
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  uint16_t* Pb = pk_g + (size_t)bh * Npad * D;
  const auto rk = buf_rsrc(Kb, (uint32_t)((size_t)N * D * 2));
  const auto rv = buf_rsrc(Vb, (uint32_t)((size_t)N * D * 2));
  const int jb = chunk * chunk_blocks, je = min(Nk, jb + chunk_blocks);
  const int nun = max(0, je - jb) * SUB;        // units of the chunk
  const int mt = GS::mt0(w);                    // the d_k row tile of this wavefront
  const bool zown = GS::zown(w);

  f32x16 acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};
  float zpart = 0.f;
  double ksum = 0.0;  // raw K over this lane's keys of the current block, d row 32 mt + l32

  auto step = [&](int x, const char* ks, const char* vs, char* nks, char* nvs) __attribute__((always_inline)) {
    wait_vm<0>();     // this wavefront's loads of unit x have landed
    __syncthreads();  // ... and every wavefront's; unit x-1 consumed
    if (x + 1 < nun) {
      const int kn = (jb * SUB + x + 1) * KU;
      lp.load(rk, kn, nks);
      lp.load(rv, kn, nvs);
    }
    const int key0 = (jb * SUB + x) * KU;
    const int lim = min(KU, N - key0);          // keys of the unit below N
    // thread chunk ch: d slice ch / 256, key (ch / 4) % 64, 8 d at 8 (ch % 4);
    // consecutive threads write consecutive 16 bytes of the phi(K) array
#pragma unroll
    for (int c = 0; c < PCH; ++c) {
      const int ch = tid + 256 * c;
      const int dt = ch / (4 * KU), r = (ch / 4) % KU, c4 = ch % 4;
      const int cc = 4 * dt + c4;               // 16-byte chunk of the key row
      const uint4 kv = rd16(ks + (cc >> 3) * T::KHALF + r * 128 + 16 * ((cc & 7) ^ sw(r)));
      uint32_t oh[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float f0 = phi(bf2f(elem(kv, 2 * e))), f1 = phi(bf2f(elem(kv, 2 * e + 1)));
        if (r >= lim) f0 = f1 = 0.f;
        oh[e] = pk_bf16(f0, f1);
      }
      *reinterpret_cast<uint4*>(Pb + ((size_t)dt * Npad + key0 + r) * 32 + 8 * c4) =
          make_uint4(oh[0], oh[1], oh[2], oh[3]);
    }
    // H += phi(K)^T V (hi + lo) over the 4 key planes of the unit; element e
    // of a plane fragment is key 16 pl + 4 hi + e % 4 + 8 (e / 4)
#pragma unroll
    for (int pl = 0; pl < KU / 16; ++pl) {
      const uint4 kr = __builtin_bit_cast(uint4, rdp.vt(ks, mt, pl));
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xv = bf2f(elem(kr, e));
        f[e] = 16 * pl + 4 * hi + (e & 3) + 8 * (e >> 2) < lim ? phi(xv) : 0.f;
        if (zown) {
          zpart += f[e];
          ksum += (double)xv;  // keys past N read as 0
        }
      }
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = pk_bf16(f[2 * e], f[2 * e + 1]);
        l[e] = pk_bf16(f[2 * e] - bf2f(h[e] & 0xffffu), f[2 * e + 1] - bf2f(h[e] >> 16));
      }
      const bf16x8 ah = as_bf16x8(make_uint4(h[0], h[1], h[2], h[3]));
      const bf16x8 al = as_bf16x8(make_uint4(l[0], l[1], l[2], l[3]));
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const bf16x8 b = rdp.vt(vs, GS::nt(w, u), pl);
        acc[u] = mfma(ah, b, acc[u]);
        acc[u] = mfma(al, b, acc[u]);
      }
    }
    if (x % SUB == SUB - 1) {
      // the key block is complete: its mean over the valid rows
      const double t = ksum + __shfl_xor(ksum, 32);
      const int j = jb + x / SUB;
      if (kbar != nullptr && zown && hi == 0)
        kbar[((size_t)bh * Nk + j) * D + 32 * mt + l32] = t / (double)min(BK, N - j * BK);
      ksum = 0.0;
    }
  };
  if (nun > 0) {
    lp.load(rk, jb * SUB * KU, k0);
    lp.load(rv, jb * SUB * KU, v0);
  }
  int x = 0;
  for (; x + 2 <= nun; x += 2) {
    step(x, k0, v0, k1, v1);
    step(x + 1, k1, v1, k0, v0);
  }
  if (x < nun) step(x, k0, v0, k1, v1);
  wait_vm<0>();

  // H in MFMA fragment order (tile (mt, nt), lane, accumulator element): the
  // order in which the attention kernel's epilogue holds G
  float* out = hpart + ((size_t)bh * nchunk + chunk) * (D * D + D);
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tile = (mt + GS::m(u)) * GS::NCT + GS::nt(w, u);
    float4* o4 = reinterpret_cast<float4*>(out + ((size_t)tile * 64 + lane) * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) o4[c] = make_float4(acc[u][4 * c], acc[u][4 * c + 1], acc[u][4 * c + 2], acc[u][4 * c + 3]);
  }
  // column sums of phi(K) over the chunk for this wavefront's row tile
  const float zt = zpart + __shfl_xor(zpart, 32);
  if (zown && hi == 0) out[D * D + 32 * mt + l32] = zt;
}

// Softmax attention over the CSR row (sparse), over every key block (dense),
// or the fused sparse + linear output with the per-head ratio alpha (fused;
// linear: the linear branch alone).  BQ/32 query wavefronts of 32 queries;
// two workgroups share a compute unit, so each SIMD holds one wavefront of
// each and the two interleave on their own.  The row's 64-key units stream
// through two LDS stages (K | V, distinct arrays, loop unrolled by two): unit
// b+1 loads while unit b is computed.  The load after the row's last unit
// repeats that unit, which keeps every step's count of loads fixed.
//
// With the linear branch every wavefront accumulates its GSplit share of G
// over the listed keys; its phi(K) slice of the next unit is loaded into its
// private LDS region as soon as the slice of the current unit is in
// registers.  At d = 128 the G tiles are always split four ways: a workgroup
// of two query wavefronts (BQ = 64) gets two more that only accumulate G.
// After the loop: H_u = H - G as hi + lo bf16 planes in LDS (the stages are
// free by then), z_u = z - g, then each query wavefront forms phi(Q) H_u for
// its queries (three MFMAs per step), divides by phi(Q) z_u and mixes the two
// branches into the output.
template <int D, int BQ, int MODE>
struct AttnShape {
  static constexpr bool LIN = MODE == MODE_FUSED || MODE == MODE_LINEAR;
  static constexpr int NQW = BQ / 32;                                  // query wavefronts
  static constexpr int NWT = (LIN && D == 128 && NQW < 4) ? 4 : NQW;   // all wavefronts
};
template <int D, int BQ, int SUB, int MODE, bool SAVE = false>
__global__ __launch_bounds__((AttnShape<D, BQ, MODE>::NWT * 64), 2) void attn_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ pk_g, const int* __restrict__ row_ptr, const int* __restrict__ col_idx,
    const float* __restrict__ alpha, const float* __restrict__ htot, uint16_t* __restrict__ O, int H, int N,
    int Nq, int Nk, float scale_log2, FwdSaved sv) {
  static_assert(!SAVE || MODE == MODE_FUSED, "the saved terms come from the fused mode");
  using T = Tiles<D>;
  using AS = AttnShape<D, BQ, MODE>;
  constexpr int NQW = AS::NQW, NW = AS::NWT;
  using LP = LoadPlan<D, NW>;
  using GS = GSplit<D, NW>;
  constexpr bool LIN = AS::LIN;
  constexpr int STAGE = 2 * T::KT_BYTES;
  constexpr int PHH = LIN ? NW * GS::MTN * 2048 : 16;  // halves of the private phi(K) regions
  static_assert(2 * (2 * STAGE + 2 * PHH) <= LDS_BYTES, "two workgroups per compute unit");
  static_assert(!LIN || (D * D * 2 <= STAGE && D * 4 <= PHH), "epilogue areas");
  // Two distinct LDS arrays: the compiler can then tell the loads into one
  // stage from the operand reads of the other.
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  __shared__ __attribute__((aligned(16))) char phr0[PHH];
  __shared__ __attribute__((aligned(16))) char phr1[PHH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool qw = NW == NQW || w < NQW;  // a query wavefront
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
  float ws_ = 1.f, wl_ = 0.f;  // weights of the two branches
  if (MODE == MODE_FUSED) {
    ws_ = alpha[bh % H];
    wl_ = 1.f - ws_;
  } else if (MODE == MODE_LINEAR) {
    ws_ = 0.f;
    wl_ = 1.f;
  }
  // the saving variant computes the sparse branch of every head (its output
  // is kept even where alpha is 0); the linear branch needs the totals,
  // which the preparation pass skips for heads whose alpha is exactly 1
  const bool do_s = SAVE || ws_ != 0.f;
  const bool lin = LIN && (wl_ != 0.f) && (nsel < Nk);
  const int nunits = (do_s || lin) ? nsel * SUB : 0;
  const int Npad = Nk * SUB * KU;
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  const int q = qw ? qi * BQ + 32 * w + l32 : N;
  bf16x8 qf[D / 16];
  load_q<D>(Q, bh, q, N, hi, qf);
  f32x16 acc_o[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc_o[t] = f32x16{};
  f32x16 acc_g[GS::TPW];  // used with the linear branch only
  float gs[GS::MTN];
#pragma unroll
  for (int u = 0; u < GS::TPW; ++u) acc_g[u] = f32x16{};
#pragma unroll
  for (int m = 0; m < GS::MTN; ++m) gs[m] = 0.f;
  Softmax sm;
  const float thr8 = 8.f / scale_log2;
  char* myphi0 = phr0 + (LIN ? w * GS::MTN * 2048 : 0);  // key planes 0, 1 of the wavefront's region
  char* myphi1 = phr1 + (LIN ? w * GS::MTN * 2048 : 0);  // key planes 2, 3
  const auto rk = buf_rsrc(Kb, (uint32_t)((size_t)N * D * 2));
  const auto rv = buf_rsrc(Vb, (uint32_t)((size_t)N * D * 2));
  const auto rph = buf_rsrc(LIN ? pk_g + (size_t)bh * Npad * D : pk_g, (uint32_t)((size_t)Npad * D * 2));
  const int mt0 = GS::mt0(w);

  // first key of unit x (clamped to the row's last unit)
  auto key0 = [&](int x) {
    const int xc = min(x, nunits - 1);
    const int blk = (MODE == MODE_DENSE) ? xc / SUB : col_idx[base + xc / SUB];
    return (blk * SUB + xc % SUB) * KU;
  };

  auto run = [&](auto s_tag, auto g_tag) __attribute__((always_inline)) {
    constexpr bool S_ = decltype(s_tag)::value != 0, G_ = decltype(g_tag)::value != 0;
    // every wavefront brings its share of both tiles, whatever it computes
    auto issue = [&](int k0x, char* sb) __attribute__((always_inline)) {
      const LP lp(w, G_ ? opaque(lane) : lane);
      if (do_s) lp.load(rk, k0x, sb);
      lp.load(rv, k0x, sb + T::KT_BYTES);
    };
    // kcur: first key of the unit being computed.  The next unit's column
    // index is read before the barrier, whose wait absorbs the scalar load, so
    // the LDS-read waits inside the step count LDS reads only.
    int kcur = key0(0);
    // Direct loads of a wavefront, in issue order per unit b: K | V of unit
    // b+1 at the top (NKV instructions), then (linear branch) the two halves
    // of its phi(K) region for unit b+1 (NPH each), each as soon as the
    // current unit's fragments of that half are in registers.  The vmcnt
    // waits below count exactly those.
    constexpr int NPH = 2 * GS::MTN;
    auto wait_kv = [&]() __attribute__((always_inline)) {  // K | V of the current unit
      if (G_) wait_vm<2 * NPH>();
      else wait_vm<0>();
    };
    auto wait_phi = [&]() __attribute__((always_inline)) {  // the next phi half of the current unit
      if (do_s) wait_vm<2 * LP::NK + NPH>();
      else wait_vm<LP::NK + NPH>();
    };
    auto step = [&](int b, char* cur, char* nxt) __attribute__((always_inline)) {
      const int knext = key0(b + 1);
      wait_kv();      // this wavefront's K | V loads of unit b have landed
      lds_barrier();  // ... and every wavefront's; unit b-1 consumed; phi(K) loads stay in flight
      issue(knext, nxt);
      const int lim = min(KU, N - kcur);
      const int ln = G_ ? opaque(lane) : lane;
      const PhiPlan pp(ln);
      auto refill0 = [&]() __attribute__((always_inline)) {
        wait_lds();  // planes 0, 1 of the region are in registers
        load_phi<GS::MTN, 0>(rph, mt0, Npad, knext, ln, myphi0);
      };
      auto refill1 = [&]() __attribute__((always_inline)) {
        wait_lds();  // planes 2, 3 as well
        load_phi<GS::MTN, 1>(rph, mt0, Npad, knext, ln, myphi1);
      };
      const char* Vc = cur + T::KT_BYTES;
      if (S_ && G_) {
        // both branches: the unit as two 32-key halves (S, softmax, products),
        // which keeps half of the score and P registers live
        f32x16 s0 = score_half<D, 0, 4>(cur, qf, rdp);
        bf16x8 bp0[2];
        softmax_half<D, 0>(s0, bp0, acc_o, sm, hi, lim, scale_log2, thr8);
        pv_g<D, NW, true, true, 0, 2>(Vc, myphi0, pp, bp0, acc_o, acc_g, gs, rdp, w, wait_phi, refill0);
        f32x16 s1 = score_half<D, 1, 4>(cur, qf, rdp);
        bf16x8 bp1[2];
        softmax_half<D, 1>(s1, bp1, acc_o, sm, hi, lim, scale_log2, thr8);
        pv_g<D, NW, true, true, 2, 4>(Vc, myphi1, pp, bp1, acc_o, acc_g, gs, rdp, w, wait_phi, refill1);
      } else if (S_) {
        f32x16 sc[2];
        score_unit<D, 4>(cur, qf, rdp, sc);
        bf16x8 bp[4];
        softmax_p<D>(sc, bp, acc_o, sm, hi, lim, scale_log2, thr8);
        pv_g<D, NW, true, false, 0, 4>(Vc, myphi0, pp, bp, acc_o, acc_g, gs, rdp, w, wait_phi, refill1);
      } else if (G_) {
        bf16x8 bp[2];
        pv_g<D, NW, false, true, 0, 2>(Vc, myphi0, pp, bp, acc_o, acc_g, gs, rdp, w, wait_phi, refill0);
        pv_g<D, NW, false, true, 2, 4>(Vc, myphi1, pp, bp, acc_o, acc_g, gs, rdp, w, wait_phi, refill1);
      }
      kcur = knext;
    };
    issue(kcur, st0);
    if (G_) {
      load_phi<GS::MTN, 0>(rph, mt0, Npad, kcur, lane, myphi0);
      load_phi<GS::MTN, 1>(rph, mt0, Npad, kcur, lane, myphi1);
    }
    int b = 0;
    for (; b + 2 <= nunits; b += 2) {
      step(b, st0, st1);
      step(b + 1, st1, st0);
    }
    if (b < nunits) step(b, st0, st1);
    wait_vm<0>();  // no direct load outlives the loop
  };
  if (nunits > 0) {
    if (!LIN) run(IntTag<1>{}, IntTag<0>{});
    else if (qw) {
      if (do_s && lin) run(IntTag<1>{}, IntTag<1>{});
      else if (do_s) run(IntTag<1>{}, IntTag<0>{});
      else run(IntTag<0>{}, IntTag<1>{});
    } else {  // G-only wavefront: loads and barriers alone when the row has no linear branch
      if (lin) run(IntTag<0>{}, IntTag<1>{});
      else run(IntTag<0>{}, IntTag<0>{});
    }
  }

  const float lt = sm.l + __shfl_xor(sm.l, 32);
  const float inv_l = lt > 0.f ? 1.f / lt : 0.f;
  const float ws_l = ws_ * inv_l;
  float wl_den = 0.f;
  float inv_den = 0.f;  // 1 / den with a linear branch (kept by SAVE)
  constexpr int NTQ = D / 16;  // k-steps of phi(Q)
  uint4 qh[LIN ? NTQ : 1], ql[LIN ? NTQ : 1];
  char* HuHi = st0;
  char* HuLo = st1;
  float* zu = reinterpret_cast<float*>(phr0);
  if (LIN) {
    const float* Hh = htot + (size_t)bh * (D * D + D);
    // this wavefront's tiles of H (fragment order, as G is held), loaded
    // before the barrier so that the wait covers their latency
    float4 hf[GS::TPW][4];
    if (lin) {
#pragma unroll
      for (int u = 0; u < GS::TPW; ++u) {
        const int tile = (mt0 + GS::m(u)) * GS::NCT + GS::nt(w, u);
        const float4* h4 = reinterpret_cast<const float4*>(Hh + ((size_t)tile * 64 + lane) * 16);
#pragma unroll
        for (int c = 0; c < 4; ++c) hf[u][c] = h4[c];
      }
    }
    __syncthreads();  // every wavefront is done with the stages and its phi(K) region
    if (lin) {
      // H_u^T = (H - G)^T for this wavefront's G tiles as hi + lo bf16 planes
      // (rows d_v, 16-wide d_k slices)
#pragma unroll
      for (int u = 0; u < GS::TPW; ++u) {
        const int mt = mt0 + GS::m(u), nt = GS::nt(w, u);
        const int dv = 32 * nt + l32;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int dk = 32 * mt + 8 * i4 + 4 * hi;
          const float hq[4] = {hf[u][i4].x, hf[u][i4].y, hf[u][i4].z, hf[u][i4].w};
          float hv[4], lv[4];
          uint32_t hb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            hv[r] = hq[r] - acc_g[u][4 * i4 + r];
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
      // z_u = z - g over the row tiles this wavefront keeps the sums of
      if (GS::zown(w)) {
#pragma unroll
        for (int m = 0; m < GS::MTN; ++m) {
          const float g = gs[m] + __shfl_xor(gs[m], 32);
          const int dz = 32 * (mt0 + m) + l32;
          if (hi == 0) zu[dz] = Hh[D * D + dz] - g;
        }
      }
    }
    // phi(Q) of every k-step: 8 values per lane, split into bf16 hi + lo
    float fq[LIN ? NTQ : 1][8];
    if (lin && qw) {
#pragma unroll
      for (int t = 0; t < NTQ; ++t) {
        const uint4 qv = __builtin_bit_cast(uint4, qf[t]);
        uint32_t fh[8];
        float fl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          fq[t][e] = phi(bf2f(elem(qv, e)));
          fh[e] = pk_bf16(fq[t][e], 0.f) & 0xffffu;
          fl[e] = fq[t][e] - bf2f(fh[e]);
        }
        qh[t] = make_uint4(fh[0] | (fh[1] << 16), fh[2] | (fh[3] << 16), fh[4] | (fh[5] << 16), fh[6] | (fh[7] << 16));
        ql[t] = make_uint4(pk_bf16(fl[0], fl[1]), pk_bf16(fl[2], fl[3]), pk_bf16(fl[4], fl[5]), pk_bf16(fl[6], fl[7]));
      }
    }
    __syncthreads();  // H_u^T and z_u complete
    if (lin && qw) {
      // den = phi(Q) . z_u (this lane's half of d, then the pair sum)
      float dpart = 0.f;
#pragma unroll
      for (int t = 0; t < NTQ; ++t) {
        const float4 z0 = *reinterpret_cast<const float4*>(zu + 16 * t + 8 * hi);
        const float4 z1 = *reinterpret_cast<const float4*>(zu + 16 * t + 8 * hi + 4);
        const float zz[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = fmaf(fq[t][e], zz[e], dpart);
      }
      const float den = dpart + __shfl_xor(dpart, 32);
      wl_den = wl_ / den;
      if (SAVE && den > 0.f) inv_den = 1.f / den;
    }
  }
  if (!qw) return;
  if (SAVE && hi == 0) {
    // per-query terms for the backward: log2 of the sparse branch's
    // normaliser, sum_u exp2(s_u c), as m c + log2 l (the sum of the rounded
    // P relative to the running maximum); 1 / den of the linear branch
    const size_t t = (size_t)row * BQ + 32 * w + l32;
    sv.lse2[t] = (q < N && lt > 0.f) ? fmaf(sm.m, scale_log2, __log2f(lt)) : INFINITY;
    sv.invden[t] = q < N ? inv_den : 0.f;
  }
  const int lb = lane_base(lane);
  const size_t orow = ((size_t)bh * N + min(q, N - 1)) * D;
  // O = ws_l O_s + wl_den num, num^T = H_u^T phi(Q)^T (the D/32 output tiles
  // accumulated together).  Each 16-byte store holds 8 consecutive d of one
  // query: lanes l and l^32 hold the two 4-d halves of every 8-d chunk and
  // swap one of them.
  f32x16 acc_n[LIN ? D / 32 : 1];
#pragma unroll
  for (int mt = 0; mt < (LIN ? D / 32 : 1); ++mt) acc_n[mt] = f32x16{};
  if (LIN && lin) {
#pragma unroll
    for (int t = 0; t < NTQ; ++t)
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt) {
        const uint4 ah = rd16(HuHi + t * T::HPB + mt * 1024 + lb);
        const uint4 al = rd16(HuLo + t * T::HPB + mt * 1024 + lb);
        acc_n[mt] = mfma(as_bf16x8(ah), as_bf16x8(qh[t]), acc_n[mt]);
        acc_n[mt] = mfma(as_bf16x8(ah), as_bf16x8(ql[t]), acc_n[mt]);
        acc_n[mt] = mfma(as_bf16x8(al), as_bf16x8(qh[t]), acc_n[mt]);
      }
  }
  // dst = fs O_s~ + fl num, O_s~ the unnormalised sparse accumulator
  auto put = [&](uint16_t* dst, float fs, float fl) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint2 pv[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int i4 = 2 * j + c;
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            o[r] = fs * acc_o[mt][4 * i4 + r];
            if (LIN) o[r] = fmaf(fl, acc_n[LIN ? mt : 0][4 * i4 + r], o[r]);
          }
          pv[c] = make_uint2(pk_bf16(o[0], o[1]), pk_bf16(o[2], o[3]));
        }
        // lane hi = 0 keeps chunk i4 = 2j (needs the partner's pv[0]); hi = 1 keeps 2j + 1 (needs pv[1])
        const uint2 send = hi ? pv[0] : pv[1];
        const uint2 recv = make_uint2(__shfl_xor(send.x, 32), __shfl_xor(send.y, 32));
        const uint4 outv = hi ? make_uint4(recv.x, recv.y, pv[1].x, pv[1].y)
                              : make_uint4(pv[0].x, pv[0].y, recv.x, recv.y);
        if (q < N) *reinterpret_cast<uint4*>(dst + orow + 32 * mt + 16 * j + 8 * hi) = outv;
      }
    }
  };
  put(O, ws_l, wl_den);
  if (SAVE && q < N) {
    // the branch outputs in float32: lane (query, hi) holds d = 32 mt + 8 i4
    // + 4 hi + r of tile mt, four runs of four consecutive d
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const size_t o = orow + 32 * mt + 8 * i4 + 4 * hi;
        const f32x16& a = acc_o[mt];
        *reinterpret_cast<float4*>(sv.os + o) =
            make_float4(inv_l * a[4 * i4], inv_l * a[4 * i4 + 1], inv_l * a[4 * i4 + 2], inv_l * a[4 * i4 + 3]);
        const f32x16& n = acc_n[LIN ? mt : 0];
        *reinterpret_cast<float4*>(sv.ol + o) = make_float4(inv_den * n[4 * i4], inv_den * n[4 * i4 + 1],
                                                            inv_den * n[4 * i4 + 2], inv_den * n[4 * i4 + 3]);
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
#pragma unroll 8
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
hipError_t prep_dispatch(const Shape& s, const void* K, const void* V, const float* alpha, bool kmeans,
                         char* ws, const WsLayout& L, hipStream_t st) {
  const long long BH = (long long)s.B * s.H;
  const dim3 grid((unsigned)(BH * L.nchunk)), block(256);
  uint16_t* pk = reinterpret_cast<uint16_t*>(ws + L.pk);
  float* hpart = reinterpret_cast<float*>(ws + L.hpart);
  double* kbar = kmeans ? reinterpret_cast<double*>(ws + L.kbar) : nullptr;
  hipLaunchKernelGGL((prep_kernel<D, BK>), grid, block, 0, st, static_cast<const uint16_t*>(K),
                     static_cast<const uint16_t*>(V), alpha, s.H, s.N, s.Nk, L.chunk_blocks, L.nchunk, pk,
                     hpart, kbar);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_summary_reduce(hpart, alpha, s.H, BH, L.nchunk, D * D + D,
                               reinterpret_cast<float*>(ws + L.htot), st);
}

template <int D, int BQ, int SUB>
hipError_t attn_dispatch(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                         const int32_t* rp, const int32_t* ci, const float* alpha, const char* ws,
                         const WsLayout& L, void* O, hipStream_t st, const FwdSaved* saved) {
  const float sl2 = 1.4426950408889634f / sqrtf((float)D);
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(K);
  const uint16_t* v = static_cast<const uint16_t*>(V);
  const uint16_t* pk = reinterpret_cast<const uint16_t*>(ws + L.pk);
  const float* ht = reinterpret_cast<const float*>(ws + L.htot);
  uint16_t* o = static_cast<uint16_t*>(O);
  const dim3 grid((unsigned)s.R());
#define SLA_LAUNCH(M)                                                                                     \
  hipLaunchKernelGGL((attn_kernel<D, BQ, SUB, M>), grid, dim3(AttnShape<D, BQ, M>::NWT * 64), 0, st, q, k, v, \
                     pk, rp, ci, alpha, ht, o, s.H, s.N, s.Nq, s.Nk, sl2, FwdSaved{})
  if (saved != nullptr) {
    if (mode != MODE_FUSED) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<D, BQ, SUB, MODE_FUSED, true>), grid,
                       dim3(AttnShape<D, BQ, MODE_FUSED>::NWT * 64), 0, st, q, k, v, pk, rp, ci, alpha, ht, o, s.H,
                       s.N, s.Nq, s.Nk, sl2, *saved);
    return hipGetLastError();
  }
  switch (mode) {
    case MODE_SPARSE: SLA_LAUNCH(MODE_SPARSE); break;
    case MODE_DENSE: SLA_LAUNCH(MODE_DENSE); break;
    case MODE_LINEAR: SLA_LAUNCH(MODE_LINEAR); break;
    default: SLA_LAUNCH(MODE_FUSED); break;
  }
#undef SLA_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prep_bf16(const Shape& s, bool lin, const void* K, const void* V, const float* alpha,
                            bool kmeans, char* ws, const WsLayout& L, hipStream_t st) {
  if (!lin) return hipSuccess;  // the softmax kernels read K and V as they are
  if (s.d == 128 && s.bk == 64) return prep_dispatch<128, 64>(s, K, V, alpha, kmeans, ws, L, st);
  if (s.d == 128 && s.bk == 128) return prep_dispatch<128, 128>(s, K, V, alpha, kmeans, ws, L, st);
  if (s.d == 64 && s.bk == 64) return prep_dispatch<64, 64>(s, K, V, alpha, kmeans, ws, L, st);
  if (s.d == 64 && s.bk == 128) return prep_dispatch<64, 128>(s, K, V, alpha, kmeans, ws, L, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bf16(const Shape& s, Mode mode, const void* Q, const void* K, const void* V,
                            const int32_t* rp, const int32_t* ci, const float* alpha, const char* ws,
                            const WsLayout& L, void* O, hipStream_t st, const FwdSaved* saved) {
#define SLA_ATTN(DD, QQ, KK)                                                  \
  if (s.d == DD && s.bq == QQ && s.bk == KK)                                  \
    return attn_dispatch<DD, QQ, KK / 64>(s, mode, Q, K, V, rp, ci, alpha, ws, L, O, st, saved);
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
