// qs_big.h -- the persistent decode kernel for batches above kSmallT tokens
// (batched decode / speculative verify): every layer of a decode call in one
// cooperative launch, five grid-wide steps per layer.
//
//   R   router logits and RMS scales; the rows were copied into LDS during
//       the previous barrier
//   --- barrier (meanwhile: this workgroup's first shared gate/up rows -> LDS)
//   K   top-k of each token (one wave per token) and x -> fixed-point limbs
//   --- barrier
//   GU  grouping (every workgroup rebuilds it in LDS), the shared expert's
//       gate/up rows, then this workgroup's routed gate/up items:
//         GEMV item: 16 rows of one expert for every token of its bucket;
//         MFMA item: 128 rows of one expert, tokens in tiles of 16, integer
//                    matrix cores (buckets of at least mfma_min tokens)
//   --- barrier (meanwhile: this workgroup's first shared down rows -> LDS)
//   D   shared down rows (all tokens), then routed down items over one
//       expert's bucket each (GEMV: 64 rows; MFMA: 128 rows), writing the
//       expert output o[bucket position][h]
//   --- barrier
//   C   y[t] = sum_j w_tj o[pos_tj] + shared + residual, summed in the
//       same fixed order as the small-batch kernel (no atomics)
//   --- barrier (meanwhile: the next layer's router rows -> LDS)
//
// Routed items are split over the workgroups by a cost model: workgroup b
// takes the items whose cost midpoint falls in the b-th 1/G of the total, a
// contiguous run of the (expert, rows) order, so consecutive items mostly
// belong to one expert.
//
// GEMV items use the same per-row arithmetic as the small-batch kernel
// (results are bitwise equal to it).  MFMA items compute the same integer
// dot products with v_mfma_i32_16x16x64_i8: the 2-bit codes, with their
// 4-bit sub-block scale folded in, are exact int8 (codebook s*c <= 105,
// Q2_K sc*q <= 45); the activations are the two int8 limbs of 16-bit fixed
// point.  A 256-weight block's int32 sums are exact, and the fp16 block
// scales are applied once per block in fp32.  The down MFMA needs one
// activation scale per 256 inputs, so MFMA buckets hand the SwiGLU output
// over in fp32 and the down items quantise it per 256-block.
#pragma once
#include "qs_persist.h"

namespace qs {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMfmaRows = 128;     // rows of a down MFMA item (8 waves x 16)
constexpr int kMguRows = 64;       // rows of a gate/up MFMA item (4 row groups x 16, two waves each)
constexpr int kMfmaTok = 16;       // tokens per MFMA column tile
constexpr int kDnRows = 64;        // rows of a GEMV down item (8 waves x kDownRows)
constexpr int kXgMax = 16;         // tokens staged per GEMV gate/up pass
constexpr int kLdsPad = 16;        // row padding of MFMA operand tiles in LDS (bank spread)
constexpr int kBatchMax = 32;      // routed GEMV items staged together

// ------------------------------------------------------------ LDS ---
struct BigLayout {
  uint32_t tab, cnt, off, act, aoff, nact, mask, ids, pairs, tok_order, pos_of, wl, gjlo, gjhi, djlo, djhi, red,
      sred, sh, ga, qtmp, bat, pfb, end;
};

__host__ __device__ inline BigLayout big_layout(int E, int T, int P, bool cb2, uint32_t pfb) {
  BigLayout l;
  uint32_t o = 0;
  auto take = [&](uint32_t n) {
    const uint32_t r = o;
    o += al16(n);
    return r;
  };
  l.tab = take(cb2 ? (uint32_t)kCbTabWords * 4 : 0);
  l.cnt = take((uint32_t)E * 4);
  l.off = take((uint32_t)(E + 1) * 4);
  l.act = take((uint32_t)E * 4);
  l.aoff = take((uint32_t)(E + 1) * 4);
  l.nact = take(4);
  l.mask = take((uint32_t)E * 32);
  l.ids = take((uint32_t)P * 4);
  l.pairs = take((uint32_t)P * 4);
  l.tok_order = take((uint32_t)P * 4);
  l.pos_of = take((uint32_t)P * 4);
  l.wl = take((uint32_t)P * 4);
  l.gjlo = take((uint32_t)E * 4);
  l.gjhi = take((uint32_t)E * 4);
  l.djlo = take((uint32_t)E * 4);
  l.djhi = take((uint32_t)E * 4);
  l.red = take(8 * 64 * 8);
  l.sred = take((uint32_t)8 * T * 2 * 4);
  l.sh = take((uint32_t)T * kDownRows * 4);
  l.ga = take((uint32_t)kXgMax * kGateTile * 4);
  l.qtmp = take((uint32_t)kXgMax * kGateTile * 4);
  l.bat = take((uint32_t)kBatchMax * 16);
  l.pfb = take(pfb);
  l.end = o;
  return l;
}

struct BigL {
  PersistLds P;          // the fields the shared helpers use
  QS_LDS int* gjlo;      // [E] this workgroup's gate/up items of active expert u: [gjlo, gjhi)
  QS_LDS int* gjhi;
  QS_LDS int* djlo;      // [E] its down items
  QS_LDS int* djhi;
  QS_LDS int* bat;       // [kBatchMax][4] staged batch: expert, first row, weight and activation offsets
};

template <class A>
__device__ __forceinline__ BigL carve_big(uint8_t* raw, const A& a, bool cb2) {
  const BigLayout l = big_layout(a.E, a.T, a.T * a.k, cb2, a.pfb);
  QS_LDS uint8_t* b = (QS_LDS uint8_t*)raw;
  BigL L;
  PersistLds& P = L.P;
  P = PersistLds{};
  P.tab = (QS_LDS uint32_t*)(b + l.tab);
  P.cnt = (QS_LDS int*)(b + l.cnt);
  P.off = (QS_LDS int*)(b + l.off);
  P.act = (QS_LDS int*)(b + l.act);
  P.aoff = (QS_LDS int*)(b + l.aoff);
  P.nact = (QS_LDS int*)(b + l.nact);
  P.mask = (QS_LDS uint32_t*)(b + l.mask);
  P.ids = (QS_LDS int*)(b + l.ids);
  P.pairs = (QS_LDS int*)(b + l.pairs);
  P.tok_order = (QS_LDS int*)(b + l.tok_order);
  P.pos_of = (QS_LDS int*)(b + l.pos_of);
  P.wl = (QS_LDS float*)(b + l.wl);
  P.red = (QS_LDS double*)(b + l.red);
  P.sred = (QS_LDS float*)(b + l.sred);
  P.sh = (QS_LDS float*)(b + l.sh);
  P.ga = (QS_LDS float*)(b + l.ga);
  P.qtmp = (QS_LDS int*)(b + l.qtmp);
  P.pfb = b + l.pfb;
  L.gjlo = (QS_LDS int*)(b + l.gjlo);
  L.gjhi = (QS_LDS int*)(b + l.gjhi);
  L.djlo = (QS_LDS int*)(b + l.djlo);
  L.djhi = (QS_LDS int*)(b + l.djhi);
  L.bat = (QS_LDS int*)(b + l.bat);
  return L;
}

// ------------------------------------------------------ staging plans ---
// Byte sizes of the pieces a phase stages into the LDS buffer; pure
// functions of the arguments (the host checks the same sizes).
__host__ __device__ inline uint32_t big_item_b(int H, bool sq8) { return (uint32_t)kSharedItemRows * 2 * srow_bytes(H, sq8); }
__host__ __device__ inline uint32_t big_sdrows_b(int Fs, bool sq8) { return (uint32_t)kDownRows * srow_bytes(Fs, sq8); }
__host__ __device__ inline uint32_t big_tile_b(int H, int gfmt) {
  return 2u * (uint32_t)kGateTile * (H / kBlockW) * blk_bytes(gfmt);
}
// one staged token of the GEMV gate/up pass: limbs hi, lo, scales (, sums
// for the formats with a min term)
__host__ __device__ inline uint32_t big_xtok_b(int H, int gfmt) {
  return 2u * H + (gfmt != kFmtCB2 ? 2u : 1u) * (H / 4);
}
__host__ __device__ inline uint32_t big_dnw_b(int F, int dfmt) {
  return (uint32_t)kDnRows * (F / kBlockW) * blk_bytes(dfmt);
}
// one staged pair of the GEMV down pass: limbs hi, lo, scales, sums, and its
// kDnRows outputs
__host__ __device__ inline uint32_t big_apair_b(int F) { return 2u * F + 2u * (F / 4) + kDnRows * 4u; }
// MFMA gate/up: K-slice of kb blocks for 16 tokens (hi, lo rows padded) + scales
__host__ __device__ inline uint32_t big_mgu_b(int kb) {
  return 2u * kMfmaTok * (kb * kBlockW + kLdsPad) + kMfmaTok * kb * 16u * 4u;
}
// MFMA down: fp32 slice, limbs hi/lo, one scale per block
__host__ __device__ inline uint32_t big_mdn_b(int kb) {
  return kMfmaTok * kb * kBlockW * 4u + 2u * kMfmaTok * (kb * kBlockW + kLdsPad) + kMfmaTok * kb * 4u;
}

// Offsets inside the buffer: the shared piece (prefetched during the
// barrier before its phase) first, the routed area after it.
__host__ __device__ inline uint32_t big_gu_area(int H, int Fs, bool sq8) { return Fs ? al16(big_item_b(H, sq8)) : 0u; }
__host__ __device__ inline uint32_t big_dn_area(int Fs, bool sq8) { return Fs ? al16(big_sdrows_b(Fs, sq8)) : 0u; }

struct BigPlan {
  int xg;     // tokens per GEMV gate/up pass
  int xp;     // pairs per GEMV down pass
  int kbg;    // blocks per MFMA gate/up K-slice
  int kbd;    // blocks per MFMA down K-slice
  int shtok;  // tokens of shared SwiGLU vectors staged per down pass
  bool ok;
};

__host__ __device__ inline BigPlan big_plan(int H, int F, int Fs, bool sq8, int gfmt, int dfmt, uint32_t pfb,
                                            int rtr_bytes) {
  BigPlan p;
  const int nbh = H / kBlockW, nb = F / kBlockW;
  const uint32_t ga = big_gu_area(H, Fs, sq8), da = big_dn_area(Fs, sq8);
  const uint32_t gfree = pfb > ga ? pfb - ga : 0u, dfree = pfb > da ? pfb - da : 0u;
  const uint32_t tb = al16(big_tile_b(H, gfmt));
  p.xg = gfree > tb ? (int)((gfree - tb) / big_xtok_b(H, gfmt)) : 0;
  if (p.xg > kXgMax) p.xg = kXgMax;
  const uint32_t wb = al16(big_dnw_b(F, dfmt));
  p.xp = dfree > wb ? (int)((dfree - wb) / big_apair_b(F)) : 0;
  if (p.xp > kXgMax) p.xp = kXgMax;
  p.kbg = 0;
  for (int kb = nbh; kb >= 1; --kb)
    if (big_mgu_b(kb) <= gfree) {
      p.kbg = kb;
      break;
    }
  p.kbd = 0;
  for (int kb = nb; kb >= 1; --kb)
    if (big_mdn_b(kb) <= dfree) {
      p.kbd = kb;
      break;
    }
  p.shtok = Fs ? (int)(dfree / ((uint32_t)Fs * 4u)) : 1;
  if (p.shtok > kMaxTokens) p.shtok = kMaxTokens;
  p.ok = p.xg >= 1 && p.xp >= 1 && p.kbg >= 1 && p.kbd >= 1 && p.shtok >= 1 && (uint32_t)rtr_bytes <= pfb &&
         (Fs == 0 || (big_item_b(H, sq8) <= pfb && big_sdrows_b(Fs, sq8) <= pfb));
  return p;
}

template <class A>
__device__ __forceinline__ BigPlan big_plan_of(const A& a) {
  return big_plan(a.H, a.F, a.Fs, a.sq8 != 0, a.gfmt, a.dfmt, a.pfb, (int)router_bytes(a));
}

// ------------------------------------------------------- cost model ---
// Rough cost of an item in units of 256 bytes streamed by one workgroup; a
// staging round trip (~1.5 us) is kStageCost.  Only the ratios matter.
constexpr int kStageCost = 240;

template <class A>
__device__ __forceinline__ int gu_gemv_cost(const A& a, int n) {
  const int w = (int)(big_tile_b(a.H, a.gfmt) >> 8);
  return kStageCost + w + (3 * w * n) / 5;
}
template <class A>
__device__ __forceinline__ int gu_mfma_cost(const A& a, int n) {
  const int w = (int)(big_tile_b(a.H, a.gfmt) >> 8) * (kMguRows / kGateTile);
  const int ng = (n + kMfmaTok - 1) / kMfmaTok;
  return w + ng * (kStageCost + 16 * (a.H / kBlockW));
}
template <class A>
__device__ __forceinline__ int dn_gemv_cost(const A& a, int n) {
  const int w = (int)(big_dnw_b(a.F, a.dfmt) >> 8);
  return kStageCost + w + (w * n) / 8;
}
template <class A>
__device__ __forceinline__ int dn_mfma_cost(const A& a, int n) {
  const int w = (int)(big_dnw_b(a.F, a.dfmt) >> 8) * (kMfmaRows / kDnRows);
  const int ng = (n + kMfmaTok - 1) / kMfmaTok;
  return w + ng * (kStageCost + 16 * (a.F / kBlockW));
}

// Items of active expert u in one phase: count m and unit cost c.
template <class A>
__device__ __forceinline__ void gu_items_of(const A& a, const PersistLds& L, int u, int& m, int& c) {
  const int n = L.aoff[u + 1] - L.aoff[u];
  if (n >= a.mfma_min) {
    m = a.F / kMguRows;
    c = gu_mfma_cost(a, n);
  } else {
    m = a.F / kGateTile;
    c = gu_gemv_cost(a, n);
  }
}
template <class A>
__device__ __forceinline__ void dn_items_of(const A& a, const PersistLds& L, int u, int& m, int& c) {
  const int n = L.aoff[u + 1] - L.aoff[u];
  if (n >= a.mfma_min) {
    m = a.H / kMfmaRows;
    c = dn_mfma_cost(a, n);
  } else {
    m = a.H / kDnRows;
    c = dn_gemv_cost(a, n);
  }
}

// Workgroup b takes item j of expert u iff floor(G*(2*(S_u + j*c_u) + c_u) /
// (2*C)) == b, S_u the cost of all earlier items and C the total.  Wave 0
// computes, for every active expert, the range [jlo, jhi) of its items this
// workgroup owns (an empty range for most).  Every workgroup evaluates the
// same integers, so the items are split exactly once.
template <class MC, class A>
__device__ __forceinline__ void assign_items(const A& a, const PersistLds& L, QS_LDS int* jlo,
                                             QS_LDS int* jhi, MC&& items_of) {
  const int lane = qs_tid() & 63, na = *L.nact;
  if ((qs_tid() >> 6) != 0) return;
  int carry = 0;
  for (int u0 = 0; u0 < na; u0 += 64) {
    const int u = u0 + lane;
    int m = 0, c = 0;
    if (u < na) items_of(u, m, c);
    const int v = m * c;
    const int incl = wave_incl_scan(v) + carry;
    if (u < na) jlo[u] = incl - v;           // S_u, replaced below
    carry = __builtin_amdgcn_readlane(incl, 63);
  }
  const long long C = carry, G = a.G, b = blockIdx.x;
  for (int u = lane; u < na; u += 64) {
    int m, c;
    items_of(u, m, c);
    const long long S = jlo[u];
    // number of items of u owned by workgroups below B
    auto below = [&](long long B) -> int {
      const long long num = 2 * B * C - G * (2 * S + c);
      if (num <= 0) return 0;
      const long long den = 2 * G * c;
      const long long q = (num + den - 1) / den;
      return q > m ? m : (int)q;
    };
    jlo[u] = below(b);
    jhi[u] = below(b + 1);
  }
}

// ------------------------------------------------------ copy issuers ---
// Rows [r0, r0+n) of one down matrix (Q2_K- or Q4_K-style) as
// [codes | scales | d,dmin].
template <class A>
__device__ __forceinline__ void copy_dn_rows(const A& a, const LayerPtrs& Lp, QS_LDS uint8_t* dst, int e,
                                             int r0, int n, int w, int nw) {
  const uint32_t nb = a.F / kBlockW;
  const MatPlanes pl = fmt_planes(a.dfmt, (size_t)a.H * nb);
  const BlkGeom g = blk_geom(a.dfmt);
  const uint8_t* base = ex_mat(a, Lp, 2, e);
  const size_t b0 = (size_t)r0 * nb;
  const uint32_t nq = (uint32_t)n * nb * g.q, ns = (uint32_t)n * nb * g.s;
  dma_to_lds<0>(base + pl.q + b0 * g.q, dst, nq, w, nw);
  dma_to_lds<0>(base + pl.s + b0 * g.s, dst + nq, ns, w, nw);
  dma_to_lds<0>(base + pl.d + b0 * g.d, dst + nq + ns, (uint32_t)n * nb * g.d, w, nw);
}

// Gather `rows` rows of `rb` bytes (a multiple of 16): row i from
// src(i) -> dst + i*stride.  Each instruction moves up to 1 KiB of one row
// (global_load_lds writes 64 consecutive 16-byte slots), so rows may be
// padded in LDS.  AUX = kCoherent for data written in this launch.
template <int AUX, class SRC>
__device__ __forceinline__ void dma_rows(SRC&& src, QS_LDS uint8_t* dst, uint32_t stride, uint32_t rb, int rows,
                                         int w, int nw) {
  const uint32_t lane = qs_tid() & 63;
  const uint32_t segs = (rb + 1023u) >> 10;
  const uint32_t total = (uint32_t)rows * segs;
  for (uint32_t q = (uint32_t)w; q < total; q += (uint32_t)nw) {
    const uint32_t r = q / segs, sg = q % segs;
    const uint32_t off = (sg << 10) + (lane << 4);
    const uint32_t d = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dst + r * stride + (sg << 10)));
    if (off < rb) dma16<AUX>((const uint8_t*)src((int)r) + off, d);
  }
}

// ------------------------------------------------------------ router ---
// One expert per workgroup (E <= G): the tokens in passes of kRtTok, each
// pass issuing the x loads of all its tokens before any use (one round
// trip).  The per-token order of the fp64 sums is phase_router's, so the
// logits equal the small-batch kernel's bit for bit.
constexpr int kRtTok = 8;

template <class A>
__device__ __forceinline__ void big_router(const A& a, const LayerPtrs& Lp, const float* x, PersistLds& L) {
  if (a.r_et != 1) {
    phase_router<false>(a, Lp, x, L);
    return;
  }
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, nw = kPersistThreads >> 6;
  const int hw = a.H / nw;
  const QS_LDS float* wr = (const QS_LDS float*)L.pfb;
  wait_all_and_sync();   // router rows prefetched during the last barrier
  int i = 0;
  for (int e = blockIdx.x; e < a.E; e += a.G, ++i) {
    if (i > 0) stage_now([&](int w, int n) { copy_router_rows(a, Lp, L, e, w, n); });
    const double b = (double)Lp.bias[e];
#pragma unroll 1
    for (int t0 = 0; t0 < a.T; t0 += kRtTok) {
      const int nt = a.T - t0 < kRtTok ? a.T - t0 : kRtTok;
      double acc[kRtTok], ss[kRtTok];
#pragma unroll
      for (int j = 0; j < kRtTok; ++j) acc[j] = ss[j] = 0.0;
#pragma unroll 1
      for (int h = wave * hw + 4 * lane; h < (wave + 1) * hw; h += 256) {
        float4 xv[kRtTok];
#pragma unroll
        for (int j = 0; j < kRtTok; ++j)
          xv[j] = j < nt ? cldf4(x + (size_t)(t0 + j) * a.H + h) : make_float4(0, 0, 0, 0);
        const float4 w = lds_f4(wr + h);
#pragma unroll
        for (int j = 0; j < kRtTok; ++j) {
          acc[j] = fma((double)w.x, (double)xv[j].x, acc[j]);
          acc[j] = fma((double)w.y, (double)xv[j].y, acc[j]);
          acc[j] = fma((double)w.z, (double)xv[j].z, acc[j]);
          acc[j] = fma((double)w.w, (double)xv[j].w, acc[j]);
          if (a.prenorm) ss[j] = sumsq_part(xv[j], ss[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < kRtTok; ++j) {
        if (j >= nt) break;
        const double sv = bfly_sum_f64<6>(acc[j]);
        const double qv = bfly_sum_f64<6>(ss[j]);
        if (lane == 0) {
          L.red[32 + wave * 32 + j] = sv;
          L.red[32 + wave * 32 + 16 + j] = qv;
        }
      }
      __syncthreads();
      if (qs_tid() < nt) {
        const int j = qs_tid(), t = t0 + j;
        double sv = 0.0, qv = 0.0;
        for (int w = 0; w < nw; ++w) {
          sv += L.red[32 + w * 32 + j];
          qv += L.red[32 + w * 32 + 16 + j];
        }
        const double r = a.prenorm ? rms_inv_of(qv, a.H) : 1.0;
        cstd(&a.logits[(size_t)t * a.E + e], a.prenorm ? fma(sv, r, b) : sv + b);
        if (e == 0) cstd(&a.rinv[t], r);
      }
      __syncthreads();
    }
  }
}

// Shared gate/up rows [2*item, 2*item+2) (in LDS) for every token; x of
// kShTok tokens per pass is loaded before use.  The per-token arithmetic is
// shared_gu_item's (bitwise equal results).
constexpr int kShTok = 8;

template <class A>
__device__ __forceinline__ void shared_gu_item_big(const A& a, lds_cptr wbase, const float* x, int item,
                                                   PersistLds& L) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63;
  const int rw = wave >> 2, qtr = wave & 3;
  const int hq = a.H / 4;
  const int T = a.T;
  const uint32_t row = srow_bytes(a.H, a.sq8 != 0);
  lds_cptr gsrc = wbase + (2 * rw) * row;
  lds_cptr usrc = wbase + (2 * rw + 1) * row;
#pragma unroll 1
  for (int t0 = 0; t0 < T; t0 += kShTok) {
    const int nt = T - t0 < kShTok ? T - t0 : kShTok;
    float g[kShTok], u[kShTok];
#pragma unroll
    for (int j = 0; j < kShTok; ++j) g[j] = u[j] = 0.f;
#pragma unroll 1
    for (int h = qtr * hq + 8 * lane; h < (qtr + 1) * hq; h += 512) {
      float4 x0[kShTok], x1[kShTok];
#pragma unroll
      for (int j = 0; j < kShTok; ++j) {
        x0[j] = j < nt ? cldf4(x + (size_t)(t0 + j) * a.H + h) : make_float4(0, 0, 0, 0);
        x1[j] = j < nt ? cldf4(x + (size_t)(t0 + j) * a.H + h + 4) : make_float4(0, 0, 0, 0);
      }
      float gw[8], uw[8];
      shared_w8(a, gsrc, a.H, h, gw);
      shared_w8(a, usrc, a.H, h, uw);
#pragma unroll
      for (int j = 0; j < kShTok; ++j) {
        const float xv[8] = {x0[j].x, x0[j].y, x0[j].z, x0[j].w, x1[j].x, x1[j].y, x1[j].z, x1[j].w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          g[j] = fmaf(gw[c], xv[c], g[j]);
          u[j] = fmaf(uw[c], xv[c], u[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kShTok; ++j) {
      if (j >= nt) break;
      const float gs = bfly_sum<6>(g[j]), us = bfly_sum<6>(u[j]);
      if (lane == 0) {
        L.sred[(wave * T + t0 + j) * 2] = gs;
        L.sred[(wave * T + t0 + j) * 2 + 1] = us;
      }
    }
  }
  __syncthreads();
  for (int q = qs_tid(); q < kSharedItemRows * T; q += kPersistThreads) {
    const int r = q / T, t = q % T;
    const int ff = item * kSharedItemRows + r;
    float gg = 0.f, uu = 0.f;
    for (int w4 = 0; w4 < 4; ++w4) {
      gg += L.sred[((r * 4 + w4) * T + t) * 2];
      uu += L.sred[((r * 4 + w4) * T + t) * 2 + 1];
    }
    const float rs = (float)cldd(&a.rinv[t]);
    cstf(&a.ash[(size_t)t * a.Fs + ff], silu_mul(gg * rs, uu * rs));
  }
  __syncthreads();
}

// ------------------------------------------------ shared gate/up (GU) ---
template <bool PRE, class A>
__device__ __forceinline__ void big_shared_gu(const A& a, const LayerPtrs& Lp, const float* x, BigL& L) {
  int j = 0;
  for (int it = blockIdx.x; it < n_shared_items<false>(a); it += a.G, ++j) {
    if (j > 0 || !PRE) stage_now([&](int w, int n) { copy_shared_item<false>(a, Lp, L.P.pfb, it, w, n); });
    else wait_all_and_sync();
    shared_gu_item_big(a, L.P.pfb, x, it, L.P);
  }
}

// ------------------------------------------ routed gate/up, GEMV item ---
// x limbs of the staged tokens: [xg][H/4] hi, [xg][H/4] lo, [xg][H/16]
// scales, [xg][H/16] sums (Q2_K consumers only).
struct XStage {
  QS_LDS uint32_t* xh;
  QS_LDS uint32_t* xl;
  QS_LDS float* xs;
  QS_LDS int* xa;
};
template <class A>
__device__ __forceinline__ XStage x_stage(const A& a, QS_LDS uint8_t* base, int xg) {
  XStage s;
  s.xh = (QS_LDS uint32_t*)base;
  s.xl = s.xh + (size_t)xg * (a.H / 4);
  s.xs = (QS_LDS float*)(s.xl + (size_t)xg * (a.H / 4));
  s.xa = (QS_LDS int*)(s.xs + (size_t)xg * (a.H / kSubW));
  return s;
}

// Tokens of bucket positions [q0, q0+n) -> staged slots 0..n-1.
template <class A>
__device__ __forceinline__ void copy_x_tokens(const A& a, const PersistLds& L, const XStage& s, int q0,
                                              int n, int w, int nw) {
  const int H = a.H, k = a.k;
  auto tok = [&](int i) { return L.pairs[q0 + i] / k; };
  dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.xh + (size_t)tok(i) * (H / 4)); },
                      (QS_LDS uint8_t*)s.xh, (uint32_t)H, (uint32_t)H, n, w, nw);
  dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.xl + (size_t)tok(i) * (H / 4)); },
                      (QS_LDS uint8_t*)s.xl, (uint32_t)H, (uint32_t)H, n, w, nw);
  dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.xs + (size_t)tok(i) * (H / kSubW)); },
                      (QS_LDS uint8_t*)s.xs, (uint32_t)H / 4, (uint32_t)H / 4, n, w, nw);
  if (a.gfmt != kFmtCB2)   // the min term needs the sums
    dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.xa + (size_t)tok(i) * (H / kSubW)); },
                        (QS_LDS uint8_t*)s.xa, (uint32_t)H / 4, (uint32_t)H / 4, n, w, nw);
}

template <class A>
__device__ __forceinline__ void x_chunk_st(const A& a, const XStage& s, int slot, int ch,
                                           uint32_t (&xh)[16], uint32_t (&xl)[16], float (&xs)[4], int (&xa)[4]) {
  const size_t xo = (size_t)slot * (a.H / 4) + ch * 16;
  const size_t si = (size_t)slot * (a.H / kSubW) + ch * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 h = lds_u4(s.xh + xo + 4 * i), l = lds_u4(s.xl + xo + 4 * i);
    xh[4 * i] = h.x; xh[4 * i + 1] = h.y; xh[4 * i + 2] = h.z; xh[4 * i + 3] = h.w;
    xl[4 * i] = l.x; xl[4 * i + 1] = l.y; xl[4 * i + 2] = l.z; xl[4 * i + 3] = l.w;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xs[i] = s.xs[si + i];
    xa[i] = a.gfmt != kFmtCB2 ? s.xa[si + i] : 0;
  }
}

// Rows [f0, f0+16) of the tile in LDS for the ng staged tokens whose bucket
// positions start at q0.  The per-(row, token) arithmetic -- lanes per row,
// chunk order, butterfly, SwiGLU, per-16 quantisation -- is routed_gu_tile's.
template <int FMT, class A>
__device__ __forceinline__ void gu_gemv_compute(const A& a, lds_cptr tile, const XStage& xst, int q0,
                                                int ng, int f0, PersistLds& L) {
  const int nbh = a.H / kBlockW;
  const int nch = a.H / kChunkW;
  const int lpr = lanes_per_row(nch);
  const int cpl = nch / lpr;
  const int slots = kPersistThreads / lpr;
  const int slot = qs_tid() / lpr, j = qs_tid() % lpr;
  constexpr bool q2k = FMT == 1;
  const TileLds tl = tile_lds(a);
  lds_cptr gq = tile, uq_ = tile + tl.qb, gs = tile + tl.s, us = tile + tl.s + tl.sb, gd = tile + tl.d,
           ud = tile + tl.d + tl.db;
#pragma unroll 1
  for (int r = slot; r < kGateTile; r += slots) {
#pragma unroll 1
    for (int tg = 0; tg < ng; tg += 4) {
      float gacc[4] = {0.f, 0.f, 0.f, 0.f}, uacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int cc = 0; cc < cpl; ++cc) {
        const int ch = j + cc * lpr;
        const uint32_t blk = (uint32_t)r * nbh + ch / 4;
        const int c = ch & 3;
        uint32_t gw[16], uw[16];
        uint32_t gsc, usc, gdd, udd;
        if constexpr (FMT == kFmtQ4K) {   // 32 code bytes per chunk; its two scales and mins
          const uint4 g0 = ld16(gq + blk * 128 + c * 32), g1 = ld16(gq + blk * 128 + c * 32 + 16);
          const uint4 u0 = ld16(uq_ + blk * 128 + c * 32), u1 = ld16(uq_ + blk * 128 + c * 32 + 16);
          gw[0] = g0.x; gw[1] = g0.y; gw[2] = g0.z; gw[3] = g0.w; gw[4] = g1.x; gw[5] = g1.y; gw[6] = g1.z; gw[7] = g1.w;
          uw[0] = u0.x; uw[1] = u0.y; uw[2] = u0.z; uw[3] = u0.w; uw[4] = u1.x; uw[5] = u1.y; uw[6] = u1.z; uw[7] = u1.w;
          gsc = ld2(gs + blk * 16 + 2 * c) | ld2(gs + blk * 16 + 8 + 2 * c) << 16;
          usc = ld2(us + blk * 16 + 2 * c) | ld2(us + blk * 16 + 8 + 2 * c) << 16;
          gdd = ld4(gd + blk * 4);
          udd = ld4(ud + blk * 4);
        }
        const uint4 gv = FMT == kFmtQ4K ? make_uint4(0, 0, 0, 0) : ld16(gq + blk * 64 + c * 16);
        const uint4 uv = FMT == kFmtQ4K ? make_uint4(0, 0, 0, 0) : ld16(uq_ + blk * 64 + c * 16);
        if (FMT == kFmtQ4K) {
        } else if (q2k) {
          gsc = ld4(gs + blk * 16 + c * 4);
          usc = ld4(us + blk * 16 + c * 4);
          gdd = ld4(gd + blk * 4);
          udd = ld4(ud + blk * 4);
          gw[0] = gv.x; gw[1] = gv.y; gw[2] = gv.z; gw[3] = gv.w;
          uw[0] = uv.x; uw[1] = uv.y; uw[2] = uv.z; uw[3] = uv.w;
        } else {
          gsc = ld1(gs + blk * 4 + c);
          usc = ld1(us + blk * 4 + c);
          gdd = ld2(gd + blk * 2);
          udd = ld2(ud + blk * 2);
          cb2_decode_dword(L.tab, gv.x, gw[0], gw[1], gw[2], gw[3]);
          cb2_decode_dword(L.tab, gv.y, gw[4], gw[5], gw[6], gw[7]);
          cb2_decode_dword(L.tab, gv.z, gw[8], gw[9], gw[10], gw[11]);
          cb2_decode_dword(L.tab, gv.w, gw[12], gw[13], gw[14], gw[15]);
          cb2_decode_dword(L.tab, uv.x, uw[0], uw[1], uw[2], uw[3]);
          cb2_decode_dword(L.tab, uv.y, uw[4], uw[5], uw[6], uw[7]);
          cb2_decode_dword(L.tab, uv.z, uw[8], uw[9], uw[10], uw[11]);
          cb2_decode_dword(L.tab, uv.w, uw[12], uw[13], uw[14], uw[15]);
        }
#pragma unroll 1
        for (int tt = 0; tt < 4; ++tt) {
          if (tg + tt >= ng) break;
          uint32_t xh[16], xl[16];
          float xs[4];
          int xa[4];
          x_chunk_st(a, xst, tg + tt, ch, xh, xl, xs, xa);
          float gp, up;
          if (FMT == kFmtQ4K) {
            const uint32_t g8[8] = {gw[0], gw[1], gw[2], gw[3], gw[4], gw[5], gw[6], gw[7]};
            const uint32_t u8[8] = {uw[0], uw[1], uw[2], uw[3], uw[4], uw[5], uw[6], uw[7]};
            gp = q4k_chunk_dot(g8, gsc, half_to_f32(gdd & 0xFFFFu), half_to_f32(gdd >> 16), xh, xl, xs, xa);
            up = q4k_chunk_dot(u8, usc, half_to_f32(udd & 0xFFFFu), half_to_f32(udd >> 16), xh, xl, xs, xa);
          } else if (q2k) {
            const uint32_t g4[4] = {gw[0], gw[1], gw[2], gw[3]}, u4[4] = {uw[0], uw[1], uw[2], uw[3]};
            gp = q2k_chunk_dot(g4, gsc, half_to_f32(gdd & 0xFFFFu), half_to_f32(gdd >> 16), xh, xl, xs, xa);
            up = q2k_chunk_dot(u4, usc, half_to_f32(udd & 0xFFFFu), half_to_f32(udd >> 16), xh, xl, xs, xa);
          } else {
            gp = half_to_f32(gdd) * xs[0] * (float)cb2_chunk_dot(gw, xh, xl, gsc);
            up = half_to_f32(udd) * xs[0] * (float)cb2_chunk_dot(uw, xh, xl, usc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            gacc[i] = i == tt ? gacc[i] + gp : gacc[i];
            uacc[i] = i == tt ? uacc[i] + up : uacc[i];
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (tg + tt >= ng) continue;
        const float g = bfly_sum_dyn(gacc[tt], lpr);
        const float uu = bfly_sum_dyn(uacc[tt], lpr);
        if (j == 0) L.ga[(tg + tt) * kGateTile + r] = silu_mul(g, uu);
      }
    }
  }
  __syncthreads();
  // quantise each staged token's 16 outputs: 16 lanes per token
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, nw = kPersistThreads >> 6;
  for (int tb = wave * 4; tb < ng; tb += nw * 4) {
    const int tt = tb + (lane >> 4), r = lane & 15;
    const bool live = tt < ng;
    const float v = live ? L.ga[tt * kGateTile + r] : 0.f;
    const float m = bfly_max<4>(fabsf(v));
    const int ex = fixed_exp(m);
    const int q = to_fixed(v, ex);
    const int s = bfly_sum_i32<4>(q);
    if (live) L.qtmp[tt * kGateTile + r] = q;
    __builtin_amdgcn_wave_barrier();
    if (live) {
      const int pair = L.pairs[q0 + tt];
      if (r < 4) {   // dword r: elements r, 4+r, 8+r, 12+r (Q2_K down) or 4r..4r+3 (Q4_K down)
        int h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          split_limbs(L.qtmp[tt * kGateTile + (FMT == kFmtQ4K ? 4 * r + i : 4 * i + r)], h[i], l[i]);
        cst(&a.ah[(size_t)pair * (a.F / 4) + f0 / 4 + r], pack4(h[0], h[1], h[2], h[3]));
        cst(&a.al[(size_t)pair * (a.F / 4) + f0 / 4 + r], pack4(l[0], l[1], l[2], l[3]));
      }
      if (r == 0) {
        cstf(&a.as[(size_t)pair * (a.F / kSubW) + f0 / kSubW], ldexpf(1.0f, ex - kFixedBits));
        csti(&a.aa[(size_t)pair * (a.F / kSubW) + f0 / kSubW], s);
      }
    }
  }
  __syncthreads();
}

// One GEMV gate/up item.  `pre`: its first staging (weights and the first
// token group) was issued earlier.  `xkeep`: the staged tokens of the
// previous item are this bucket's (same expert, whole bucket staged).
template <int FMT, class A>
__device__ __forceinline__ void gu_gemv_item(const A& a, const LayerPtrs& Lp, BigL& L, const BigPlan& pp,
                                             int u, int f0, bool pre, bool xkeep) {
  PersistLds& P = L.P;
  const int q0 = P.aoff[u], n = P.aoff[u + 1] - q0, e = P.act[u];
  QS_LDS uint8_t* wt = P.pfb + big_gu_area(a.H, a.Fs, a.sq8 != 0);
  const XStage xst = x_stage(a, wt + al16(big_tile_b(a.H, a.gfmt)), pp.xg);
  for (int g0 = 0; g0 < n; g0 += pp.xg) {
    const int ng = n - g0 < pp.xg ? n - g0 : pp.xg;
    if (g0 == 0 && pre) {
      wait_all_and_sync();
    } else {
      const bool cx = !(g0 == 0 && xkeep);
      stage_now([&](int w, int nw) {
        if (g0 == 0) copy_tile(a, Lp, wt, e, f0, w, nw);
        if (cx) copy_x_tokens(a, P, xst, q0 + g0, ng, w, nw);
      });
    }
    gu_gemv_compute<FMT>(a, wt, xst, q0 + g0, ng, f0, P);
  }
}

// ------------------------------------------ routed gate/up, MFMA item ---
// A-operand of v_mfma_i32_16x16x64_i8: lane l supplies row l%16 and K
// positions 16*(l/16)..+15 of a 64-wide K step.  Within a 256-weight block
// the lanes of group g = l/16 take, over the four K steps s, the 64-weight
// chunk g (16 bytes of codes), step s covering block positions 64g+16s..+15;
// the B operand (activation limbs) uses the same positions, so the
// permutation of K cancels in the dot product.

// low byte of each signed byte times s (0 <= s <= 15): even and odd bytes
// widened to 16-bit lanes, multiplied, repacked
__device__ __forceinline__ uint32_t scale_s8x4(uint32_t d, uint32_t s) {
  const uint32_t ev = __builtin_amdgcn_perm(0u, d, 0x0C020C00u) * s;
  const uint32_t od = __builtin_amdgcn_perm(0u, d, 0x0C030C01u) * s;
  return __builtin_amdgcn_perm(od, ev, 0x06020400u);
}

// codebook chunk dword (two 8-weight groups) -> 16 signed weights s*c*sign
__device__ __forceinline__ v4i cb2_afrag(const QS_LDS uint32_t* tab, uint32_t v, uint32_t s) {
  uint32_t q0, q1, q2, q3;
  cb2_decode_dword(tab, v, q0, q1, q2, q3);
  v4i r;
  r[0] = (int)scale_s8x4(q0, s);
  r[1] = (int)scale_s8x4(q1, s);
  r[2] = (int)scale_s8x4(q2, s);
  r[3] = (int)scale_s8x4(q3, s);
  return r;
}

// Q2_K sub-block dword -> 16 weights sc*q in the Q2_K consumer order
// (dword p = weights p, 4+p, 8+p, 12+p)
__device__ __forceinline__ v4i q2k_afrag(uint32_t qd, uint32_t sc) {
  v4i r;
  r[0] = (int)((qd & 0x03030303u) * sc);
  r[1] = (int)(((qd >> 2) & 0x03030303u) * sc);
  r[2] = (int)(((qd >> 4) & 0x03030303u) * sc);
  r[3] = (int)(((qd >> 6) & 0x03030303u) * sc);
  return r;
}

__device__ __forceinline__ v4i splat4(uint32_t m) {
  const int v = (int)(m * 0x01010101u);
  v4i r = {v, v, v, v};
  return r;
}

__device__ __forceinline__ v4i lds_v4i(const QS_LDS uint8_t* p) {
  const u32x4_t v = *(const QS_LDS u32x4_t*)p;
  v4i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  return r;
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Weights of one (row, block) for one lane of an MFMA item: the lane's
// 16-byte code chunk, its scale bytes, and the fp16 scales of the four rows
// it accumulates (D layout: rows 4*(l/16)+i).
struct GuFrag {
  uint4 q;
  uint32_t sc;
  uint32_t d[4];
};

template <int FMT>
__device__ __forceinline__ GuFrag load_gu_frag(const uint8_t* mat, const MatPlanes& pl, int nbh, int arow, int drow0,
                                               int blk, int g) {
  constexpr bool q2k = FMT == 1;
  GuFrag f;
  const size_t ab = (size_t)arow * nbh + blk;
  f.q = *(const uint4*)(mat + pl.q + ab * 64 + 16 * g);
  if (q2k) f.sc = *(const uint32_t*)(mat + pl.s + ab * 16 + 4 * g);       // sub-blocks 4g..4g+3
  else f.sc = mat[pl.s + ab * 4 + g];                                      // 32-weight sub-blocks 2g, 2g+1
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const size_t db = (size_t)(drow0 + i) * nbh + blk;
    f.d[i] = q2k ? *(const uint32_t*)(mat + pl.d + db * 4) : (uint32_t)*(const uint16_t*)(mat + pl.d + db * 2);
  }
  return f;
}

// MFMA gate/up tile views: per slot (token) [K-slice + pad] hi bytes, the
// same for lo, then [slot][kb*16] scales (one float per 16 elements).
struct MguStage {
  QS_LDS uint8_t* xh;
  QS_LDS uint8_t* xl;
  QS_LDS float* xs;
  uint32_t stride;
};
__device__ __forceinline__ MguStage mgu_stage(QS_LDS uint8_t* base, int kb) {
  MguStage s;
  s.stride = (uint32_t)kb * kBlockW + kLdsPad;
  s.xh = base;
  s.xl = base + kMfmaTok * s.stride;
  s.xs = (QS_LDS float*)(base + 2 * kMfmaTok * s.stride);
  return s;
}

template <int FMT, class A>
__device__ __forceinline__ void gu_mfma_item(const A& a, const LayerPtrs& Lp, BigL& L, const BigPlan& pp,
                                             int u, int f0) {
  constexpr bool q2k = FMT == 1;
  PersistLds& P = L.P;
  const int q0 = P.aoff[u], n = P.aoff[u + 1] - q0, e = P.act[u];
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, r = lane & 15, g = lane >> 4;
  // waves w and w+4 take row group w&3; wave w>>2 == 0 the even blocks of
  // each staged slice, == 1 the odd ones (their sums are added at the end)
  const int rg = wave & 3, kh = wave >> 2;
  const int H = a.H, nbh = H / kBlockW;
  const MatPlanes pl = q2k ? q2k_planes((size_t)a.F * nbh) : cb2_planes((size_t)a.F * nbh);
  const uint8_t* gm = ex_mat(a, Lp, 0, e);
  const uint8_t* um = ex_mat(a, Lp, 1, e);
  const int arow = f0 + 16 * rg + r, drow0 = f0 + 16 * rg + 4 * g;
  const MguStage st = mgu_stage(P.pfb + big_gu_area(H, a.Fs, a.sq8 != 0), pp.kbg);
#pragma unroll 1
  for (int g0 = 0; g0 < n; g0 += kMfmaTok) {
    const int ng = n - g0 < kMfmaTok ? n - g0 : kMfmaTok;
    float ag[4] = {0.f, 0.f, 0.f, 0.f}, au[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int k0 = 0; k0 < nbh; k0 += pp.kbg) {
      const int kb = nbh - k0 < pp.kbg ? nbh - k0 : pp.kbg;
      // slots beyond the bucket repeat its last token (their columns are dropped)
      auto tok = [&](int i) { return P.pairs[q0 + g0 + (i < ng ? i : ng - 1)] / a.k; };
      // this wave's first block of the slice is requested before the wait
      // for the tokens
      const int kf = kh < kb ? k0 + kh : k0;
      GuFrag fg = load_gu_frag<FMT>(gm, pl, nbh, arow, drow0, kf, g);
      GuFrag fu = load_gu_frag<FMT>(um, pl, nbh, arow, drow0, kf, g);
      stage_now([&](int w, int nw) {
        dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.xh + (size_t)tok(i) * (H / 4)) + k0 * kBlockW; },
                            st.xh, st.stride, (uint32_t)kb * kBlockW, kMfmaTok, w, nw);
        dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.xl + (size_t)tok(i) * (H / 4)) + k0 * kBlockW; },
                            st.xl, st.stride, (uint32_t)kb * kBlockW, kMfmaTok, w, nw);
        dma_rows<kCoherent>(
            [&](int i) { return (const uint8_t*)(a.xs + (size_t)tok(i) * (H / kSubW) + k0 * 16); },
            (QS_LDS uint8_t*)st.xs, (uint32_t)pp.kbg * 64, (uint32_t)kb * 64, kMfmaTok, w, nw);
      });
#pragma unroll 1
      for (int b = kh; b < kb; b += 2) {
        GuFrag ng_ = fg, nu_ = fu;
        if (b + 2 < kb) {
          ng_ = load_gu_frag<FMT>(gm, pl, nbh, arow, drow0, k0 + b + 2, g);
          nu_ = load_gu_frag<FMT>(um, pl, nbh, arow, drow0, k0 + b + 2, g);
        }
        v4i ihg = {0, 0, 0, 0}, ilg = ihg, ihu = ihg, ilu = ihg;
        v4i mhg = ihg, mlg = ihg, mhu = ihg, mlu = ihg;   // Q2_K min terms
        const uint32_t qg[4] = {fg.q.x, fg.q.y, fg.q.z, fg.q.w}, qu[4] = {fu.q.x, fu.q.y, fu.q.z, fu.q.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const QS_LDS uint8_t* bp = st.xh + r * st.stride + b * kBlockW + 64 * g + 16 * s;
          const v4i bh = lds_v4i(bp);
          const v4i bl = lds_v4i(bp + (st.xl - st.xh));
          v4i A_g, A_u;
          if (q2k) {
            const uint32_t scg = (fg.sc >> (8 * s)) & 0xFFu, scu = (fu.sc >> (8 * s)) & 0xFFu;
            A_g = q2k_afrag(qg[s], scg & 15u);
            A_u = q2k_afrag(qu[s], scu & 15u);
            const v4i M_g = splat4(scg >> 4), M_u = splat4(scu >> 4);
            mhg = mfma_i8(M_g, bh, mhg);
            mlg = mfma_i8(M_g, bl, mlg);
            mhu = mfma_i8(M_u, bh, mhu);
            mlu = mfma_i8(M_u, bl, mlu);
          } else {
            const uint32_t sh = 4u * (uint32_t)(s >> 1);
            A_g = cb2_afrag(P.tab, qg[s], (fg.sc >> sh) & 15u);
            A_u = cb2_afrag(P.tab, qu[s], (fu.sc >> sh) & 15u);
          }
          ihg = mfma_i8(A_g, bh, ihg);
          ilg = mfma_i8(A_g, bl, ilg);
          ihu = mfma_i8(A_u, bh, ihu);
          ilu = mfma_i8(A_u, bl, ilu);
        }
        const float xsc = st.xs[r * (pp.kbg * 16) + b * 16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sg = (float)(ihg[i] * 256 + ilg[i]), su = (float)(ihu[i] * 256 + ilu[i]);
          if (q2k) {
            const float mg = (float)(mhg[i] * 256 + mlg[i]), mu = (float)(mhu[i] * 256 + mlu[i]);
            ag[i] = fmaf(xsc, fmaf(half_to_f32(fg.d[i] & 0xFFFFu), sg, -(half_to_f32(fg.d[i] >> 16) * mg)), ag[i]);
            au[i] = fmaf(xsc, fmaf(half_to_f32(fu.d[i] & 0xFFFFu), su, -(half_to_f32(fu.d[i] >> 16) * mu)), au[i]);
          } else {
            ag[i] = fmaf(half_to_f32(fg.d[i]) * xsc, sg, ag[i]);
            au[i] = fmaf(half_to_f32(fu.d[i]) * xsc, su, au[i]);
          }
        }
        fg = ng_;
        fu = nu_;
      }
    }
    // the odd blocks' sums join the even ones' through the staging area
    // (8 KiB <= its two token tiles; every wave is done with them first)
    __syncthreads();
    QS_LDS float* part = (QS_LDS float*)st.xh + (rg * 64 + lane) * 8;
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part[i] = ag[i];
        part[4 + i] = au[i];
      }
    }
    __syncthreads();
    if (kh == 0 && r < ng) {
      const int pair = P.pairs[q0 + g0 + r];
      float* o = a.af + (size_t)pair * a.F + drow0;
#pragma unroll
      for (int i = 0; i < 4; ++i) cstf(o + i, silu_mul(ag[i] + part[i], au[i] + part[4 + i]));
    }
  }
  __syncthreads();   // every wave is done with the staged tiles
}

// --------------------------------------------------- GU phase (batched) ---
// Routed GEMV items are staged in batches: the copies of as many items as
// fit in the buffer (each item's weights; each expert's tokens once) are
// issued together, waited for once, and computed one after another.  A
// bucket too large for one staging takes the multi-pass item; MFMA items
// stage their own tiles.
struct Batcher {
  QS_LDS uint8_t* area;
  uint32_t cap, fill;
  int n, last_u;
  uint32_t last_x;
};

template <int FMT, class A>
__device__ __forceinline__ void big_gu_phase(const A& a, const LayerPtrs& Lp, const float* x, BigL& L,
                                             const BigPlan& pp) {
  PersistLds& P = L.P;
  build_groups<false>(a, P);
  assign_items(a, P, L.gjlo, L.gjhi, [&](int u, int& m, int& c) { gu_items_of(a, P, u, m, c); });
  assign_items(a, P, L.djlo, L.djhi, [&](int u, int& m, int& c) { dn_items_of(a, P, u, m, c); });
  __syncthreads();
  const int na = *P.nact;
  const int wave = qs_tid() >> 6, nw = kPersistThreads >> 6;
  const uint32_t tb = al16(big_tile_b(a.H, a.gfmt)), xtok = big_xtok_b(a.H, a.gfmt);
  Batcher B;
  B.area = P.pfb + big_gu_area(a.H, a.Fs, a.sq8 != 0);
  B.cap = a.pfb - big_gu_area(a.H, a.Fs, a.sq8 != 0);
  B.fill = 0;
  B.n = 0;
  B.last_u = -1;
  B.last_x = 0;
  bool shared_done = false;
  auto shared = [&]() {
    if (!shared_done) big_shared_gu<true>(a, Lp, x, L);   // overlaps the first batch's copies
    shared_done = true;
  };
  auto flush = [&]() {
    shared();
    if (B.n == 0) return;
    wait_all_and_sync();
    for (int i = 0; i < B.n; ++i) {
      const int u = L.bat[4 * i], r0 = L.bat[4 * i + 1];
      const uint32_t wo = (uint32_t)L.bat[4 * i + 2], xo = (uint32_t)L.bat[4 * i + 3];
      const int q0 = P.aoff[u], n = P.aoff[u + 1] - q0;
      gu_gemv_compute<FMT>(a, B.area + wo, x_stage(a, B.area + xo, n), q0, n, r0, P);
    }
    B.n = 0;
    B.fill = 0;
    B.last_u = -1;
  };
  // one pass over this workgroup's items; each routine has one call site
  int u = 0, j = 0;
  if (na > 0) j = L.gjlo[0];
#pragma unroll 1
  while (true) {
    while (u < na && j >= L.gjhi[u]) {
      ++u;
      if (u < na) j = L.gjlo[u];
    }
    const bool end = u >= na;
    const int q0 = end ? 0 : P.aoff[u], n = end ? 0 : P.aoff[u + 1] - q0;
    const bool mf = !end && n >= a.mfma_min;
    const uint32_t xb = al16((uint32_t)n * xtok);
    // bucket larger than one staging (or than the SwiGLU tile buffers)
    const bool big = !end && !mf && (tb + xb > B.cap || n > kXgMax);
    const bool room = B.fill + tb + (u != B.last_u ? xb : 0u) <= B.cap && B.n < kBatchMax;
    if (end || mf || big || !room) {
      if (B.n > 0 || !shared_done) {
        flush();
        continue;
      }
      if (end) break;
      if constexpr (FMT != kFmtQ4K) {   // (the Q4_K layers run GEMV items only)
        if (mf) gu_mfma_item<FMT>(a, Lp, L, pp, u, j * kMguRows);
        else gu_gemv_item<FMT>(a, Lp, L, pp, u, j * kGateTile, false, false);
      } else {
        gu_gemv_item<FMT>(a, Lp, L, pp, u, j * kGateTile, false, false);
      }
      ++j;
      continue;
    }
    const uint32_t wo = B.fill;
    B.fill += tb;
    if (u != B.last_u) {
      B.last_x = B.fill;
      B.fill += xb;
      copy_x_tokens(a, P, x_stage(a, B.area + B.last_x, n), q0, n, wave, nw);
      B.last_u = u;
    }
    copy_tile(a, Lp, B.area + wo, P.act[u], j * kGateTile, wave, nw);
    if (qs_tid() == 0) {
      L.bat[4 * B.n] = u;
      L.bat[4 * B.n + 1] = j * kGateTile;
      L.bat[4 * B.n + 2] = (int)wo;
      L.bat[4 * B.n + 3] = (int)B.last_x;
    }
    ++B.n;
    ++j;
  }
}

// ------------------------------------------------- D phase (batched) ---
// SwiGLU limbs of the staged pairs: [xp][F/4] hi, lo, [xp][F/16] scales, sums.
struct AStage {
  QS_LDS uint32_t* ah;
  QS_LDS uint32_t* al;
  QS_LDS float* as;
  QS_LDS int* aa;
  QS_LDS float* o;     // [xp][kDnRows] outputs (accumulated over chunks)
};
template <class A>
__device__ __forceinline__ AStage a_stage(const A& a, QS_LDS uint8_t* base, int xp) {
  AStage s;
  s.ah = (QS_LDS uint32_t*)base;
  s.al = s.ah + (size_t)xp * (a.F / 4);
  s.as = (QS_LDS float*)(s.al + (size_t)xp * (a.F / 4));
  s.aa = (QS_LDS int*)(s.as + (size_t)xp * (a.F / kSubW));
  s.o = (QS_LDS float*)(s.aa + (size_t)xp * (a.F / kSubW));
  return s;
}

template <class A>
__device__ __forceinline__ void copy_a_pairs(const A& a, const PersistLds& L, const AStage& s, int q0, int n,
                                             int w, int nw) {
  const int F = a.F;
  auto pr = [&](int i) { return L.pairs[q0 + i]; };
  dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.ah + (size_t)pr(i) * (F / 4)); },
                      (QS_LDS uint8_t*)s.ah, (uint32_t)F, (uint32_t)F, n, w, nw);
  dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.al + (size_t)pr(i) * (F / 4)); },
                      (QS_LDS uint8_t*)s.al, (uint32_t)F, (uint32_t)F, n, w, nw);
  dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.as + (size_t)pr(i) * (F / kSubW)); },
                      (QS_LDS uint8_t*)s.as, (uint32_t)F / 4, (uint32_t)F / 4, n, w, nw);
  dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.aa + (size_t)pr(i) * (F / kSubW)); },
                      (QS_LDS uint8_t*)s.aa, (uint32_t)F / 4, (uint32_t)F / 4, n, w, nw);
}

// One wave: its 8 rows (of the item's 64, in LDS) against the ng staged
// pairs; the per-(row, pair) arithmetic is down_expert's (Q4_K: the same
// with 32-byte chunks and q4k_chunk_dot).
template <int FMT, class A>
__device__ __forceinline__ void dn_gemv_rows(const A& a, lds_cptr w, int wrow0, const AStage& st, int ng) {
  const int lane = qs_tid() & 63;
  const int nb = a.F / kBlockW;
  const int nch = a.F / kChunkW;
  const int lpr = lanes_per_row(nch);
  const int cpl = nch / lpr;
  const int rpi = 64 / lpr;
  const int rsub = lane / lpr, j = lane % lpr;
  constexpr bool q4k = FMT == kFmtQ4K;
  const BlkGeom g = blk_geom(q4k ? kFmtQ4K : kFmtQ2K);
  lds_cptr wq = w, ws = w + kDnRows * nb * g.q, wd = ws + kDnRows * nb * g.s;
#pragma unroll 1
  for (int rr = rsub; rr < kDownRows; rr += rpi) {
    const int row = wrow0 + rr;       // row within the item
#pragma unroll 1
    for (int cc = 0; cc < cpl; ++cc) {
      const int ch = j + cc * lpr;
      const int c = ch & 3;
      const uint32_t blk = (uint32_t)row * nb + ch / 4;
      uint32_t qw[8];
      uint32_t scm;
      if (q4k) {
        const uint4 q0 = ld16(wq + blk * 128 + c * 32), q1 = ld16(wq + blk * 128 + c * 32 + 16);
        qw[0] = q0.x; qw[1] = q0.y; qw[2] = q0.z; qw[3] = q0.w; qw[4] = q1.x; qw[5] = q1.y; qw[6] = q1.z; qw[7] = q1.w;
        scm = ld2(ws + blk * 16 + 2 * c) | ld2(ws + blk * 16 + 8 + 2 * c) << 16;
      } else {
        const uint4 qv = ld16(wq + blk * 64 + c * 16);
        qw[0] = qv.x; qw[1] = qv.y; qw[2] = qv.z; qw[3] = qv.w;
        scm = ld4(ws + blk * 16 + c * 4);
      }
      const uint32_t dd = ld4(wd + blk * 4);
      const float d = half_to_f32(dd & 0xFFFFu), dm = half_to_f32(dd >> 16);
#pragma unroll 1
      for (int sl = 0; sl < ng; ++sl) {
        uint32_t xh[16], xl[16];
        float xs[4];
        int xa[4];
        const size_t ao = (size_t)sl * (a.F / 4) + ch * 16;
        const size_t si = (size_t)sl * (a.F / kSubW) + ch * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint4 hv = lds_u4(st.ah + ao + 4 * i);
          const uint4 lv = lds_u4(st.al + ao + 4 * i);
          xh[4 * i] = hv.x; xh[4 * i + 1] = hv.y; xh[4 * i + 2] = hv.z; xh[4 * i + 3] = hv.w;
          xl[4 * i] = lv.x; xl[4 * i + 1] = lv.y; xl[4 * i + 2] = lv.z; xl[4 * i + 3] = lv.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xs[i] = st.as[si + i];
          xa[i] = st.aa[si + i];
        }
        float part;
        if (q4k) {
          part = q4k_chunk_dot(qw, scm, d, dm, xh, xl, xs, xa);
        } else {
          const uint32_t q4[4] = {qw[0], qw[1], qw[2], qw[3]};
          part = q2k_chunk_dot(q4, scm, d, dm, xh, xl, xs, xa);
        }
        part = bfly_sum_dyn(part, lpr);
        if (j == 0) st.o[sl * kDnRows + row] = cc == 0 ? part : st.o[sl * kDnRows + row] + part;
      }
    }
  }
}

template <int FMT, class A>
__device__ __forceinline__ void dn_gemv_item(const A& a, const LayerPtrs& Lp, BigL& L, const BigPlan& pp,
                                             int u, int h0, bool pre) {
  PersistLds& P = L.P;
  const int q0 = P.aoff[u], n = P.aoff[u + 1] - q0, e = P.act[u];
  const int wave = qs_tid() >> 6;
  QS_LDS uint8_t* wt = P.pfb + big_dn_area(a.Fs, a.sq8 != 0);
  const AStage st = a_stage(a, wt + al16(big_dnw_b(a.F, a.dfmt)), pp.xp);
  for (int g0 = 0; g0 < n; g0 += pp.xp) {
    const int ng = n - g0 < pp.xp ? n - g0 : pp.xp;
    if (g0 == 0 && pre) {
      wait_all_and_sync();
    } else {
      stage_now([&](int w, int nw) {
        if (g0 == 0) copy_dn_rows(a, Lp, wt, e, h0, kDnRows, w, nw);
        copy_a_pairs(a, P, st, q0 + g0, ng, w, nw);
      });
    }
    dn_gemv_rows<FMT>(a, wt, wave * kDownRows, st, ng);
    __syncthreads();
    for (int i = qs_tid(); i < ng * kDnRows; i += kPersistThreads) {
      const int sl = i / kDnRows, row = i % kDnRows;
      cstf(&a.ob[(size_t)(q0 + g0 + sl) * a.H + h0 + row], st.o[sl * kDnRows + row]);
    }
  }
  __syncthreads();   // the outputs are read out before the buffer is reused
}

// MFMA down: per 16-pair tile and K-slice, the fp32 SwiGLU outputs are
// staged, quantised per 256-block (one wave per pair and block) into limbs
// in the Q2_K consumer order, then multiplied.
struct MdnStage {
  QS_LDS float* af;     // [16][kb*256]
  QS_LDS uint8_t* lh;   // [16][kb*256 + pad]
  QS_LDS uint8_t* ll;
  QS_LDS float* sc;     // [16][kb]
  uint32_t stride;
};
__device__ __forceinline__ MdnStage mdn_stage(QS_LDS uint8_t* base, int kb) {
  MdnStage s;
  s.stride = (uint32_t)kb * kBlockW + kLdsPad;
  s.af = (QS_LDS float*)base;
  s.lh = base + kMfmaTok * kb * kBlockW * 4;
  s.ll = s.lh + kMfmaTok * s.stride;
  s.sc = (QS_LDS float*)(s.ll + kMfmaTok * s.stride);
  return s;
}

struct DnFrag {
  uint4 q;
  uint32_t scm;
  uint32_t dd[4];
};
__device__ __forceinline__ DnFrag load_dn_frag(const uint8_t* mat, const MatPlanes& pl, int nb, int arow, int drow0,
                                               int blk, int g) {
  DnFrag f;
  const size_t ab = (size_t)arow * nb + blk;
  f.q = *(const uint4*)(mat + pl.q + ab * 64 + 16 * g);
  f.scm = *(const uint32_t*)(mat + pl.s + ab * 16 + 4 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.dd[i] = *(const uint32_t*)(mat + pl.d + ((size_t)(drow0 + i) * nb + blk) * 4);
  return f;
}

template <class A>
__device__ __forceinline__ void dn_mfma_item(const A& a, const LayerPtrs& Lp, BigL& L, const BigPlan& pp,
                                             int u, int h0) {
  PersistLds& P = L.P;
  const int q0 = P.aoff[u], n = P.aoff[u + 1] - q0, e = P.act[u];
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, r = lane & 15, g = lane >> 4, nw = kPersistThreads >> 6;
  const int F = a.F, nb = F / kBlockW;
  const MatPlanes pl = q2k_planes((size_t)a.H * nb);
  const uint8_t* dm = ex_mat(a, Lp, 2, e);
  const int arow = h0 + 16 * wave + r, drow0 = h0 + 16 * wave + 4 * g;
  const MdnStage st = mdn_stage(P.pfb + big_dn_area(a.Fs, a.sq8 != 0), pp.kbd);
#pragma unroll 1
  for (int g0 = 0; g0 < n; g0 += kMfmaTok) {
    const int ng = n - g0 < kMfmaTok ? n - g0 : kMfmaTok;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int k0 = 0; k0 < nb; k0 += pp.kbd) {
      const int kb = nb - k0 < pp.kbd ? nb - k0 : pp.kbd;
      auto pr = [&](int i) { return P.pairs[q0 + g0 + (i < ng ? i : ng - 1)]; };
      DnFrag f = load_dn_frag(dm, pl, nb, arow, drow0, k0, g);
      stage_now([&](int w, int nw2) {
        dma_rows<kCoherent>([&](int i) { return (const uint8_t*)(a.af + (size_t)pr(i) * F + k0 * kBlockW); },
                            (QS_LDS uint8_t*)st.af, (uint32_t)kb * kBlockW * 4, (uint32_t)kb * kBlockW * 4,
                            kMfmaTok, w, nw2);
      });
      // quantise: one wave per (slot, block); lane holds elements 4l..4l+3
      for (int unit = wave; unit < kMfmaTok * kb; unit += nw) {
        const int sl = unit / kb, b = unit % kb;
        const float4 v = lds_f4(st.af + (size_t)sl * kb * kBlockW + b * kBlockW + 4 * lane);
        const float m = bfly_max<6>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        const int ex = fixed_exp(m);
        int h0_, l0_, h1_, l1_, h2_, l2_, h3_, l3_;
        split_limbs(to_fixed(v.x, ex), h0_, l0_);
        split_limbs(to_fixed(v.y, ex), h1_, l1_);
        split_limbs(to_fixed(v.z, ex), h2_, l2_);
        split_limbs(to_fixed(v.w, ex), h3_, l3_);
        const uint32_t ph = q2k_order(pack4(h0_, h1_, h2_, h3_)), plo = q2k_order(pack4(l0_, l1_, l2_, l3_));
        *(QS_LDS uint32_t*)(st.lh + sl * st.stride + b * kBlockW + 4 * lane) = ph;
        *(QS_LDS uint32_t*)(st.ll + sl * st.stride + b * kBlockW + 4 * lane) = plo;
        if (lane == 0) st.sc[sl * pp.kbd + b] = ldexpf(1.0f, ex - kFixedBits);
      }
      __syncthreads();
#pragma unroll 1
      for (int b = 0; b < kb; ++b) {
        DnFrag fn = f;
        if (b + 1 < kb) fn = load_dn_frag(dm, pl, nb, arow, drow0, k0 + b + 1, g);
        v4i mh = {0, 0, 0, 0}, ml = mh, nh = mh, nl = mh;
        const uint32_t qd[4] = {f.q.x, f.q.y, f.q.z, f.q.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t scm = (f.scm >> (8 * s)) & 0xFFu;
          const v4i Wm = q2k_afrag(qd[s], scm & 15u), M = splat4(scm >> 4);
          const QS_LDS uint8_t* bp = st.lh + r * st.stride + b * kBlockW + 64 * g + 16 * s;
          const v4i bh = lds_v4i(bp), bl = lds_v4i(bp + (st.ll - st.lh));
          mh = mfma_i8(Wm, bh, mh);
          ml = mfma_i8(Wm, bl, ml);
          nh = mfma_i8(M, bh, nh);
          nl = mfma_i8(M, bl, nl);
        }
        const float asc = st.sc[r * pp.kbd + b];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sm = (float)(mh[i] * 256 + ml[i]), mn = (float)(nh[i] * 256 + nl[i]);
          acc[i] = fmaf(asc, fmaf(half_to_f32(f.dd[i] & 0xFFFFu), sm, -(half_to_f32(f.dd[i] >> 16) * mn)), acc[i]);
        }
        f = fn;
      }
    }
    if (r < ng) {
      float* o = a.ob + (size_t)(q0 + g0 + r) * a.H + drow0;
#pragma unroll
      for (int i = 0; i < 4; ++i) cstf(o + i, acc[i]);
    }
  }
  __syncthreads();   // every wave is done with the staged tiles
}

// Shared down rows [r0, r0+8) (in LDS at `srows`, one row per wave) for
// tokens [t0, t0+nt) whose SwiGLU vectors are staged at `as_` ([nt][Fs]);
// the per-token arithmetic is shared_down_row's.
template <class A>
__device__ __forceinline__ void big_shared_dn_tile(const A& a, lds_cptr srows, const QS_LDS float* as_,
                                                   int t0, int nt, int r0, BigL& L) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63;
  lds_cptr srow = srows + (uint32_t)wave * srow_bytes(a.Fs, a.sq8 != 0);
#pragma unroll 1
  for (int j = 0; j < nt; ++j) {
    float sum = 0.f;
#pragma unroll 1
    for (int f = 8 * lane; f < a.Fs; f += 512) {
      float ww[8];
      shared_w8(a, srow, a.Fs, f, ww);
      const float4 a0 = lds_f4(as_ + j * a.Fs + f), a1 = lds_f4(as_ + j * a.Fs + f + 4);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) sum = fmaf(ww[c], av[c], sum);
    }
    sum = bfly_sum<6>(sum);
    if (lane == 0) L.P.sh[j * kDownRows + wave] = sum;
  }
  __syncthreads();
  for (int i = qs_tid(); i < nt * kDownRows; i += kPersistThreads) {
    const int j = i / kDownRows, rr = i % kDownRows;
    cstf(&a.sb[(size_t)(t0 + j) * a.H + r0 + rr], L.P.sh[i]);
  }
  __syncthreads();
}

template <int FMT, class A>
__device__ __forceinline__ void big_dn_phase(const A& a, const LayerPtrs& Lp, BigL& L, const BigPlan& pp) {
  PersistLds& P = L.P;
  const int na = *P.nact;
  if (a.Fs && (int)blockIdx.x < a.H / kDownRows) {
    // the shared SwiGLU vectors of as many tokens as fit beside the rows
    QS_LDS float* as_ = (QS_LDS float*)(P.pfb + big_dn_area(a.Fs, a.sq8 != 0));
    const int tg = pp.shtok;
    for (int t0 = 0; t0 < a.T; t0 += tg) {
      const int nt = a.T - t0 < tg ? a.T - t0 : tg;
      int j = 0;
      for (int tile = blockIdx.x; tile < a.H / kDownRows; tile += a.G, ++j) {
        const bool rows = j > 0 || t0 > 0;
        stage_now([&](int w, int n) {
          if (rows) copy_sd_rows(a, Lp, P.pfb, tile * kDownRows, w, n);
          if (j == 0)
            dma_to_lds<kCoherent>(a.ash + (size_t)t0 * a.Fs, (QS_LDS void*)as_, (uint32_t)nt * a.Fs * 4, w, n);
        });
        big_shared_dn_tile(a, P.pfb, as_, t0, nt, tile * kDownRows, L);
      }
    }
  }
  // routed items, GEMV ones staged in batches as in the gate/up phase
  const int wave = qs_tid() >> 6, nw = kPersistThreads >> 6;
  const uint32_t wb = al16(big_dnw_b(a.F, a.dfmt)), pb = big_apair_b(a.F);
  Batcher B;
  B.area = P.pfb + big_dn_area(a.Fs, a.sq8 != 0);
  B.cap = a.pfb - big_dn_area(a.Fs, a.sq8 != 0);
  B.fill = 0;
  B.n = 0;
  B.last_u = -1;
  B.last_x = 0;
  auto flush = [&]() {
    if (B.n == 0) return;
    wait_all_and_sync();
    for (int i = 0; i < B.n; ++i) {
      const int u = L.bat[4 * i], h0 = L.bat[4 * i + 1];
      const uint32_t wo = (uint32_t)L.bat[4 * i + 2], xo = (uint32_t)L.bat[4 * i + 3];
      const int q0 = P.aoff[u], n = P.aoff[u + 1] - q0;
      const AStage st = a_stage(a, B.area + xo, n);
      dn_gemv_rows<FMT>(a, B.area + wo, wave * kDownRows, st, n);
      __syncthreads();
      for (int k = qs_tid(); k < n * kDnRows; k += kPersistThreads) {
        const int sl = k / kDnRows, row = k % kDnRows;
        cstf(&a.ob[(size_t)(q0 + sl) * a.H + h0 + row], st.o[sl * kDnRows + row]);
      }
      __syncthreads();
    }
    B.n = 0;
    B.fill = 0;
    B.last_u = -1;
  };
  int u = 0, j = 0;
  if (na > 0) j = L.djlo[0];
#pragma unroll 1
  while (true) {
    while (u < na && j >= L.djhi[u]) {
      ++u;
      if (u < na) j = L.djlo[u];
    }
    const bool end = u >= na;
    const int q0 = end ? 0 : P.aoff[u], n = end ? 0 : P.aoff[u + 1] - q0;
    const bool mf = !end && n >= a.mfma_min;
    const uint32_t xb = al16((uint32_t)n * pb);
    const bool big = !end && !mf && wb + xb > B.cap;
    const bool room = B.fill + wb + (u != B.last_u ? xb : 0u) <= B.cap && B.n < kBatchMax;
    if (end || mf || big || !room) {
      if (B.n > 0) {
        flush();
        continue;
      }
      if (end) break;
      if constexpr (FMT != kFmtQ4K) {   // (the Q4_K layers run GEMV items only)
        if (mf) dn_mfma_item(a, Lp, L, pp, u, j * kMfmaRows);
        else dn_gemv_item<FMT>(a, Lp, L, pp, u, j * kDnRows, false);
      } else {
        dn_gemv_item<FMT>(a, Lp, L, pp, u, j * kDnRows, false);
      }
      ++j;
      continue;
    }
    const uint32_t wo = B.fill;
    B.fill += wb;
    if (u != B.last_u) {
      B.last_x = B.fill;
      B.fill += xb;
      copy_a_pairs(a, P, a_stage(a, B.area + B.last_x, n), q0, n, wave, nw);
      B.last_u = u;
    }
    copy_dn_rows(a, Lp, B.area + wo, P.act[u], j * kDnRows, kDnRows, wave, nw);
    if (qs_tid() == 0) {
      L.bat[4 * B.n] = u;
      L.bat[4 * B.n + 1] = j * kDnRows;
      L.bat[4 * B.n + 2] = (int)wo;
      L.bat[4 * B.n + 3] = (int)B.last_x;
    }
    ++B.n;
    ++j;
  }
}

// -------------------------------------------------- C phase (combine) ---
template <class A>
__device__ __forceinline__ void big_combine(const A& a, const PersistLds& L, const float* x, float* y) {
  const int N = a.T * a.H;
  for (int i = (int)blockIdx.x * kPersistThreads + qs_tid(); i < N; i += a.G * kPersistThreads) {
    const int t = i / a.H, h = i % a.H;
    float acc = 0.f;
    for (int jj = 0; jj < a.k; ++jj) {
      const int pos = L.tok_order[t * a.k + jj];
      const int pair = L.pairs[pos];
      acc = fmaf(L.wl[pair], cldf(&a.ob[(size_t)pos * a.H + h]), acc);
    }
    if (a.Fs) acc += cldf(&a.sb[i]);
    if (a.residual) acc += cldf(&x[i]);
    cstf(&y[i], acc);
  }
}

// ------------------------------------------------------------- kernel ---
// Steered combine, in two halves around one more grid barrier.  Workgroup b
// owns rows [b*rpw, (b+1)*rpw) of every token; a group of gl lanes (the
// rows, gl a power of two) takes one token at a time.  First half: the MoE
// output m of those rows into mb and the workgroup's partial d . m per token
// into part[t][b] (lane order, then a fixed tree).  Second half: d . m summed
// over the G partials in a fixed order, then m - sscale * d * (d . m) (+ x).
template <class A>
__device__ __forceinline__ int steer_rows(const A& a) { return (a.H + a.G - 1) / a.G; }
__device__ __forceinline__ int steer_lanes(int rpw) {
  int gl = 1;
  while (gl < rpw && gl < 64) gl <<= 1;
  return gl;
}

template <class A>
__device__ __forceinline__ void big_steer_partials(const A& a, const PersistLds& L, const float* dir) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, nw = kPersistThreads >> 6;
  const int rpw = steer_rows(a), gl = steer_lanes(rpw), per = 64 / gl;
  const int r0 = blockIdx.x * rpw, r1 = r0 + rpw < a.H ? r0 + rpw : a.H;
  const int g = lane % gl;
  for (int t0 = wave * per; t0 < a.T; t0 += nw * per) {   // wave-uniform
    const int t = t0 + lane / gl;
    float p = 0.f;
    for (int h = r0 + g; h < r1; h += gl) {
      if (t >= a.T) break;
      float acc = 0.f;
      for (int jj = 0; jj < a.k; ++jj) {
        const int pos = L.tok_order[t * a.k + jj];
        acc = fmaf(L.wl[L.pairs[pos]], cldf(&a.ob[(size_t)pos * a.H + h]), acc);
      }
      if (a.Fs) acc += cldf(&a.sb[(size_t)t * a.H + h]);
      cstf(&a.mb[(size_t)t * a.H + h], acc);
      p = fmaf(dir[h], acc, p);
    }
    p = bfly_sum_dyn(p, gl);
    if (g == 0 && t < a.T) cstf(&a.part[(size_t)t * a.G + blockIdx.x], p);
  }
}

template <class A>
__device__ __forceinline__ void big_steer_apply(const A& a, const float* dir, const float* x, float* y) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, nw = kPersistThreads >> 6;
  const int rpw = steer_rows(a);
  const int r0 = blockIdx.x * rpw, r1 = r0 + rpw < a.H ? r0 + rpw : a.H;
  if (r0 >= r1) return;
  for (int t = wave; t < a.T; t += nw) {
    float dm = 0.f;
    for (int b = lane; b < a.G; b += 64) dm += cldf(&a.part[(size_t)t * a.G + b]);
    dm = bfly_sum<6>(dm);   // every lane holds the sum
    for (int h = r0 + lane; h < r1; h += 64) {
      const size_t i = (size_t)t * a.H + h;
      float acc = cldf(&a.mb[i]) - a.sscale * dir[h] * dm;
      if (a.residual) acc += cldf(&x[i]);
      cstf(&y[i], acc);
    }
  }
}

template <int FMT, bool STEER, class A>
__device__ __forceinline__ void persist_big_body(const A& a) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  BigL L = carve_big(lds_raw, a, FMT == 2);
  const BigPlan pp = big_plan_of(a);
  const int wave = qs_tid() >> 6, nw = kPersistThreads >> 6;
  if (FMT == 2) dma_to_lds<0>(a.cbtab, L.P.tab, (uint32_t)kCbTabWords * 4, wave, nw);
  if ((int)blockIdx.x < router_groups(a)) copy_router_rows(a, a.layers[0], L.P, blockIdx.x, wave, nw);
  wait_all_and_sync();
  uint32_t epoch = a.epoch0;
  for (int li = 0; li < a.n_layers; ++li) {
    const LayerPtrs Lp = a.layers[li];
    const float* x = li == 0 ? a.x_in : ((li - 1) & 1 ? a.xbuf1 : a.xbuf0);
    float* y = li == a.n_layers - 1 ? a.y_out : (li & 1 ? a.xbuf1 : a.xbuf0);
    const bool more = li + 1 < a.n_layers;
    // ---- R
    QS_STAMP(li, 0);
    big_router(a, Lp, x, L.P);
    QS_STAMP(li, 1);
    if (!grid_barrier(a, ++epoch, [&](int w, int n) {
          if ((int)blockIdx.x < n_shared_items<false>(a)) copy_shared_item<false>(a, Lp, L.P.pfb, blockIdx.x, w, n);
        }))
      return;
    QS_STAMP(li, 2);
    // ---- K
    {
      const int nb = a.H / kBlockW, units = a.T + a.T * nb;
      for (int u = blockIdx.x * nw + wave; u < units; u += a.G * nw) {
        if (u < a.T) topk_wave<false>(a, u, li, L.P, true);
        else quant_x_wave<false>(a, x, (u - a.T) / nb, (u - a.T) % nb, L.P);
      }
    }
    QS_STAMP(li, 3);
    if (!grid_barrier(a, ++epoch, [](int, int) {})) return;
    QS_STAMP(li, 4);
    // ---- GU
    big_gu_phase<FMT>(a, Lp, x, L, pp);
    QS_STAMP(li, 5);
    if (!grid_barrier(a, ++epoch, [&](int w, int n) {
          if (a.Fs && (int)blockIdx.x < a.H / kDownRows) copy_sd_rows(a, Lp, L.P.pfb, blockIdx.x * kDownRows, w, n);
        }))
      return;
    QS_STAMP(li, 6);
    // ---- D
    big_dn_phase<FMT>(a, Lp, L, pp);
    QS_STAMP(li, 7);
    if (!grid_barrier(a, ++epoch, [](int, int) {})) return;
    QS_STAMP(li, 8);
    // ---- C
    if constexpr (STEER) {
      const float* dir = a.sdir + (size_t)li * a.H;
      big_steer_partials(a, L.P, dir);
      if (!grid_barrier(a, ++epoch, [](int, int) {})) return;
      big_steer_apply(a, dir, x, y);
    } else {
      big_combine(a, L.P, x, y);
    }
    QS_STAMP(li, 9);
    if (more && !grid_barrier(a, ++epoch, [&](int w, int n) {
          if ((int)blockIdx.x < router_groups(a)) copy_router_rows(a, a.layers[li + 1], L.P, blockIdx.x, w, n);
        }))
      return;
  }
}

template <int FMT, bool STEER>
__global__ void __launch_bounds__(kPersistThreads) k_persist_big(PersistArgs a) {
  persist_big_body<FMT, STEER>(a);
}

template <int FMT, bool STEER>
__global__ void __launch_bounds__(kPersistThreads) k_persist_big_paged(PersistArgs a) {
  persist_big_body<FMT, STEER>(static_cast<const PagedArgs&>(a));
}

// The layer shape fixed at compile time, the batch size at run time (as
// FixedArgs for the small-batch kernel).
template <int FMT, int H_, int E_, int K_, int F_, int FS_, int SQ8_, int G_, bool PG = false>
struct FixedBigArgs : PersistArgs {
  static constexpr int H = H_, E = E_, k = K_, F = F_, Fs = FS_, sq8 = SQ8_, G = G_;
  static constexpr int gq2k = FMT == 1, r_et = 1;
  static constexpr int gfmt = FMT, dfmt = FMT == kFmtQ4K ? kFmtQ4K : kFmtQ2K;
  static constexpr bool kPaged = PG;
};

// PG: for launches over paged layers
template <int FMT, int H, int E, int K, int F, int FS, int SQ8, int G, bool STEER = false, bool PG = false>
__global__ void __launch_bounds__(kPersistThreads) k_persist_big_fixed(PersistArgs a) {
  persist_big_body<FMT, STEER>(static_cast<const FixedBigArgs<FMT, H, E, K, F, FS, SQ8, G, PG>&>(a));
}

}  // namespace qs
