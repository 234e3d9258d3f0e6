// qs_persist.h -- the whole decode call (every layer, every step of the MoE
// path) as one persistent cooperative kernel on gfx950.
//
// Why one kernel: each layer has three all-to-all dependencies (all logits
// before top-k, all SwiGLU outputs of an expert before its down GEMV, all of
// x_{l+1} before the next router).  A kernel boundary costs ~2.5 us on
// MI355X and a grid barrier about the same, but inside one kernel the
// weights that do not depend on the pending result (router rows, shared
// expert rows, the down rows of experts already chosen) are requested before
// the wait, straight into LDS, so their HBM latency hides behind it.
//
// Phases of one layer (G workgroups x 512 threads, one per CU):
//   R   router logits (fp64, exact products) and the per-token RMS scale;
//       then the shared gate/up rows of this workgroup's first item are issued
//   K   top-k per token (one wave each) and x -> fixed-point limbs; for
//       T <= kSmallT every workgroup does this itself into LDS, which saves
//       the barrier after K
//   GU  grouping rebuilt in LDS by every workgroup; shared-expert and routed
//       gate/up items; then the down rows of this workgroup's first tile
//   D   down row tiles + combine + shared down + residual -> x_{l+1}; then
//       the next layer's router rows
// The three prefetches share one LDS buffer: each is consumed before the
// next is issued.  Phases are joined by a fence-free grid barrier: per-XCD
// arrival counters, a global counter bumped by each XCD's last arriver, and
// per-XCD release lines written by the global last arriver.  Data crossing a
// barrier is written and read with agent-scope (sc1) atomic accesses, which
// are coherent across the XCDs' separate L2s without the whole-L2
// writeback/invalidate of a release or acquire fence; an s_waitcnt before
// arriving orders them (and completes the LDS prefetches).  Every wait is
// bounded: a workgroup that gives up raises an error flag and every
// workgroup leaves at its next barrier, so the grid always drains.
#pragma once
#include "qs_kernels.h"
#include "qs_wave.h"

namespace qs {

constexpr int kPersistThreads = 512;
constexpr int kSmallT = 4;
constexpr int kSpinMax = 1 << 22;
// sync words (uint32 index): [16*x] per-XCD counters, [128] global counter,
// [144 + 16*x] release lines, [272] error flag
constexpr int kSyncWords = 512;
constexpr int kSyncGlobal = 128, kSyncRelease = 144, kSyncError = 272;
constexpr int kSharedItemRows = 2;    // shared gate/up rows per item (4 waves per row)
constexpr size_t kPfbMax = 64 * 1024; // LDS prefetch buffer upper bound

struct LayerPtrs {
  const float* router;
  const float* bias;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const uint16_t* sg;
  const uint16_t* su;
  const uint16_t* sd;
};

struct PersistArgs {
  const LayerPtrs* layers;   // device array, first entry = layer0
  int n_layers, T, H, E, k, F, Fs;
  int gq2k, prenorm, residual, small;
  int r_et, r_tt;            // router tile: experts x tokens per unit
  int pfb;                   // bytes of the LDS prefetch buffer
  size_t gu_stride, dn_stride;
  const uint32_t* cbtab;
  const float* x_in;
  float* y_out;
  int32_t* ids_out;
  float* w_out;
  double* logits;            // [T][E]
  double* rinv;              // [T]
  int32_t* ids;              // [T][k]      (T > kSmallT)
  float* wts;                // [T][k]      (T > kSmallT)
  uint32_t* xh;              // [T][H/4]    (T > kSmallT)
  uint32_t* xl;
  float* xs;                 // [T][H/16]
  int32_t* xa;
  uint32_t* ah;              // [T*k][F/4]
  uint32_t* al;
  float* as;                 // [T*k][F/16]
  int32_t* aa;
  float* ash;                // [T][Fs]
  float* xbuf0;              // [T][H] residual stream between layers
  float* xbuf1;
  uint32_t* sync;
  uint32_t epoch0;
};

// ------------------------------------------------- coherent accesses ---
__device__ __forceinline__ uint32_t cld(const uint32_t* p) {
  return __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t cld64(const void* p) {
  return __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int cldi(const int32_t* p) { return (int)cld((const uint32_t*)p); }
__device__ __forceinline__ float cldf(const float* p) { return __uint_as_float(cld((const uint32_t*)p)); }
__device__ __forceinline__ double cldd(const double* p) {
  return __longlong_as_double((long long)cld64(p));
}
__device__ __forceinline__ float4 cldf4(const float* p) {
  const uint64_t a = cld64(p), b = cld64(p + 2);
  return make_float4(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)),
                     __uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32)));
}
__device__ __forceinline__ void cst(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void csti(int32_t* p, int v) { cst((uint32_t*)p, (uint32_t)v); }
__device__ __forceinline__ void cstf(float* p, float v) { cst((uint32_t*)p, __float_as_uint(v)); }
__device__ __forceinline__ void cstd(double* p, double v) {
  __hip_atomic_store((uint64_t*)p, (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t catomic_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copy `bytes` (a multiple of 16) from global memory straight into LDS with
// global_load_lds_dwordx4: each wave instruction moves 64 x 16 bytes to
// consecutive LDS slots.  Completion is awaited by the next s_waitcnt(0).
__device__ __forceinline__ void copy_to_lds(const void* g, void* lds, size_t bytes) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const size_t n16 = bytes / 16;
  for (size_t base = (size_t)wave * 64; base < n16; base += (size_t)nw * 64) {
    if (base + lane < n16)
      __builtin_amdgcn_global_load_lds((const uint4*)g + base + lane,
                                       (__attribute__((address_space(3))) void*)((uint4*)lds + base),
                                       16, 0, 0);
  }
}

// ------------------------------------------------------- grid barrier ---
__device__ bool grid_barrier(const PersistArgs& a, uint32_t epoch) {
  const uint32_t G = gridDim.x, x = blockIdx.x & 7u, per = G >> 3;
  __builtin_amdgcn_s_waitcnt(0);     // coherent stores and LDS prefetches have completed
  __syncthreads();
  int ok = 1;
  if (threadIdx.x == 0) {
    uint32_t* s = a.sync;
    const uint32_t old = catomic_add(&s[16 * x], 1u);
    if (old == epoch * per - 1u) {
      const uint32_t g = catomic_add(&s[kSyncGlobal], 1u);
      if (g == epoch * 8u - 1u)
        for (int i = 0; i < 8; ++i) cst(&s[kSyncRelease + 16 * i], epoch);
    }
    int spins = 0;
    while (cld(&s[kSyncRelease + 16 * x]) < epoch) {
      if (++spins > kSpinMax) {
        cst(&s[kSyncError], 1u);
        ok = 0;
        break;
      }
      if ((spins & 63) == 0 && cld(&s[kSyncError])) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return __syncthreads_and(ok);
}

// --------------------------------------------------------- LDS layout ---
struct PersistLds {
  uint32_t* tab;        // [8192] codebook quads (codebook gate/up only)
  int* cnt;             // [E]
  int* off;             // [E+1]
  int* act;             // [E]
  int* nact;            // [1]
  uint32_t* mask;       // [E*8]
  int* ids;             // [P]   expert of pair id
  int* pairs;           // [P]   pair id at bucket position
  int* tok_order;       // [P]   per token, positions by ascending expert
  int* pos_of;          // [P]   bucket position of pair id
  float* wl;            // [P]   router weight of pair id
  float* o;             // [P*kDownRows] down outputs
  double* red;          // [8*64] router cross-wave partials
  float* sh;            // [T*kDownRows] shared-expert down outputs
  float* ga;            // [T*kGateTile] SwiGLU tile, per bucket token
  float* sred;          // [8*T*2] shared gate/up cross-wave partials
  int* qtmp;            // [T*kGateTile] fixed-point tile values
  uint32_t* xh;         // [T*H/4] small path: x limbs
  uint32_t* xl;
  float* xs;            // [T*H/16]
  int* xa;
  uint8_t* pfb;         // prefetch buffer
};

template <typename LdsT>
__host__ __device__ inline size_t carve_lds_impl(uint8_t* base, int E, int T, int P, int H,
                                                 bool cb2, bool small, size_t pfb, LdsT* L) {
  size_t off = 0;
  auto take = [&](size_t n) {
    uint8_t* r = base ? base + off : nullptr;
    off += align_up(n, 16);
    return r;
  };
  uint8_t* tab = take(cb2 ? (size_t)kCbTabWords * 4 : 0);
  uint8_t* cnt = take((size_t)E * 4);
  uint8_t* offp = take((size_t)(E + 1) * 4);
  uint8_t* act = take((size_t)E * 4);
  uint8_t* nact = take(4);
  uint8_t* mask = take((size_t)E * 32);
  uint8_t* ids = take((size_t)P * 4);
  uint8_t* pairs = take((size_t)P * 4);
  uint8_t* tok_order = take((size_t)P * 4);
  uint8_t* pos_of = take((size_t)P * 4);
  uint8_t* wl = take((size_t)P * 4);
  uint8_t* o = take((size_t)P * kDownRows * 4);
  uint8_t* red = take(8 * 64 * 8);
  uint8_t* sh = take((size_t)T * kDownRows * 4);
  uint8_t* ga = take((size_t)T * kGateTile * 4);
  uint8_t* sred = take((size_t)8 * T * 2 * 4);
  uint8_t* qtmp = take((size_t)T * kGateTile * 4);
  const size_t xq = small ? (size_t)T * H : 0;
  uint8_t* xh = take(xq);          // T*H/4 dwords
  uint8_t* xl = take(xq);
  uint8_t* xs = take(xq / 4);      // T*H/16 floats
  uint8_t* xa = take(xq / 4);
  uint8_t* pf = take(pfb);
  if (L) {
    L->tab = (uint32_t*)tab;
    L->cnt = (int*)cnt;
    L->off = (int*)offp;
    L->act = (int*)act;
    L->nact = (int*)nact;
    L->mask = (uint32_t*)mask;
    L->ids = (int*)ids;
    L->pairs = (int*)pairs;
    L->tok_order = (int*)tok_order;
    L->pos_of = (int*)pos_of;
    L->wl = (float*)wl;
    L->o = (float*)o;
    L->red = (double*)red;
    L->sh = (float*)sh;
    L->ga = (float*)ga;
    L->sred = (float*)sred;
    L->qtmp = (int*)qtmp;
    L->xh = (uint32_t*)xh;
    L->xl = (uint32_t*)xl;
    L->xs = (float*)xs;
    L->xa = (int*)xa;
    L->pfb = pf;
  }
  return off;
}

inline size_t persist_lds_bytes(int E, int T, int P, int H, bool cb2, bool small, size_t pfb) {
  return carve_lds_impl<PersistLds>(nullptr, E, T, P, H, cb2, small, pfb, nullptr);
}

__device__ inline PersistLds carve_lds(uint8_t* base, const PersistArgs& a, bool cb2) {
  PersistLds L;
  carve_lds_impl(base, a.E, a.T, a.T * a.k, a.H, cb2, (bool)a.small, (size_t)a.pfb, &L);
  return L;
}

// ------------------------------------------------------------ phase R ---
// Unit = (ET experts, TT tokens); the 8 waves split H into slices of H/8.
// The router rows of this workgroup's first unit are prefetched into the
// LDS buffer as [ET][H] floats when they fit.
__device__ __forceinline__ bool router_pf_fits(const PersistArgs& a) {
  return (size_t)a.r_et * a.H * 4 <= (size_t)a.pfb;
}

__device__ void router_prefetch(const PersistArgs& a, const LayerPtrs& Lp, PersistLds& L) {
  const int ET = a.r_et, TT = a.r_tt;
  const int ntt = (a.T + TT - 1) / TT, net = (a.E + ET - 1) / ET;
  if ((int)blockIdx.x >= net * ntt || !router_pf_fits(a)) return;
  const int e0 = ((int)blockIdx.x / ntt) * ET;
  const int ne = a.E - e0 < ET ? a.E - e0 : ET;
  copy_to_lds(Lp.router + (size_t)e0 * a.H, L.pfb, (size_t)ne * a.H * 4);
}

__device__ void phase_router(const PersistArgs& a, const LayerPtrs& Lp, const float* x, PersistLds& L) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int ET = a.r_et, TT = a.r_tt;
  const int net = (a.E + ET - 1) / ET, ntt = (a.T + TT - 1) / TT;
  const int hw = a.H / nw;                     // elements per wave (multiple of 32)
  const int V = ET * TT + TT;
  const float* pfr = (const float*)L.pfb;
  for (int u = blockIdx.x; u < net * ntt; u += gridDim.x) {
    const int e0 = (u / ntt) * ET, t0 = (u % ntt) * TT;
    const bool from_lds = u == (int)blockIdx.x && router_pf_fits(a);
    double acc[4][4], ss[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ss[i] = 0.0;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    }
    for (int h = wave * hw + 4 * lane; h < (wave + 1) * hw; h += 256) {
      float4 xv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xv[j] = (j < TT && t0 + j < a.T) ? cldf4(x + (size_t)(t0 + j) * a.H + h) : make_float4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= ET || e0 + i >= a.E) continue;
        const float4 w = from_lds ? *(const float4*)(pfr + (size_t)i * a.H + h)
                                  : *(const float4*)(Lp.router + (size_t)(e0 + i) * a.H + h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j >= TT) continue;
          acc[i][j] = fma((double)w.x, (double)xv[j].x, acc[i][j]);
          acc[i][j] = fma((double)w.y, (double)xv[j].y, acc[i][j]);
          acc[i][j] = fma((double)w.z, (double)xv[j].z, acc[i][j]);
          acc[i][j] = fma((double)w.w, (double)xv[j].w, acc[i][j]);
        }
      }
      if (a.prenorm) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j >= TT) continue;
          ss[j] = fma((double)xv[j].x, (double)xv[j].x, ss[j]);
          ss[j] = fma((double)xv[j].y, (double)xv[j].y, ss[j]);
          ss[j] = fma((double)xv[j].z, (double)xv[j].z, ss[j]);
          ss[j] = fma((double)xv[j].w, (double)xv[j].w, ss[j]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i < ET && j < TT) {
          const double s = bfly_sum_f64<6>(acc[i][j]);
          if (lane == 0) L.red[wave * V + i * TT + j] = s;
        }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < TT) {
        const double s = bfly_sum_f64<6>(ss[j]);
        if (lane == 0) L.red[wave * V + ET * TT + j] = s;
      }
    __syncthreads();
    if ((int)threadIdx.x < ET * TT) {
      const int i = threadIdx.x / TT, j = threadIdx.x % TT;
      const int e = e0 + i, t = t0 + j;
      if (e < a.E && t < a.T) {
        double s = 0.0, q = 0.0;
        for (int w = 0; w < nw; ++w) {
          s += L.red[w * V + i * TT + j];
          q += L.red[w * V + ET * TT + j];
        }
        double r = 1.0;
        if (a.prenorm) r = 1.0 / sqrt(q / (double)a.H + kRmsEps);
        const double b = (double)Lp.bias[e];
        cstd(&a.logits[(size_t)t * a.E + e], a.prenorm ? fma(s, r, b) : s + b);
        if (e == 0) cstd(&a.rinv[t], r);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------ phase K ---
// Top-k of token t by one wave: (logit desc, index asc), weights are the
// softmax over the k picks.  Results go to LDS (small path, every
// workgroup) or to global scratch (one wave per token); workgroup 0 / the
// token's wave also writes the caller's ids_out / w_out.
__device__ void topk_wave(const PersistArgs& a, int t, int layer_i, PersistLds* L, bool write_out) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  double v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    const double l = e < E ? cldd(&a.logits[(size_t)t * E + e]) : 0.0;
    v[i] = l != l ? -INFINITY : l;     // NaN ranks last; every pick stays valid and distinct
  }
  uint32_t taken = 0;
  double top0 = 0.0, selv = 0.0;
  int seli = 0;
  for (int j = 0; j < k; ++j) {
    double bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (bi == 0x7FFFFFFF || v[i] > bv)) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) top0 = bv;
    if (lane == j) {
      selv = bv;
      seli = bi;
    }
  }
  const double z = lane < k ? exp(selv - top0) : 0.0;
  const double sum = bfly_sum_f64<6>(z);
  if (lane < k) {
    const float w = (float)(z / sum);
    if (L) {
      L->ids[t * k + lane] = seli;
      L->wl[t * k + lane] = w;
    } else {
      csti(&a.ids[t * k + lane], seli);
      cstf(&a.wts[t * k + lane], w);
    }
    if (write_out) {
      const size_t o = (size_t)layer_i * a.T * k + t * k + lane;
      if (a.ids_out) a.ids_out[o] = seli;
      if (a.w_out) a.w_out[o] = w;
    }
  }
}

// x block b (256 elements) of token t -> limbs, one wave; into LDS when
// `L` is given, else into global scratch.
__device__ void quant_x_wave(const PersistArgs& a, const float* x, int t, int b, PersistLds* L) {
  const int lane = threadIdx.x & 63;
  const float4 v = cldf4(x + (size_t)t * a.H + b * kBlockW + 4 * lane);
  const float r = (float)cldd(&a.rinv[t]);
  const float m = bfly_max<6>(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  const int e = fixed_exp(m);
  const int q0 = to_fixed(v.x, e), q1 = to_fixed(v.y, e), q2 = to_fixed(v.z, e), q3 = to_fixed(v.w, e);
  int h0, l0, h1, l1, h2, l2, h3, l3;
  split_limbs(q0, h0, l0);
  split_limbs(q1, h1, l1);
  split_limbs(q2, h2, l2);
  split_limbs(q3, h3, l3);
  uint32_t ph = pack4(h0, h1, h2, h3), pl = pack4(l0, l1, l2, l3);
  if (a.gq2k) {
    // dword 4i+p of sub-block i gathers element p of lanes 4i..4i+3
    const int p = lane & 3;
    uint32_t bh[4], bl[4];
    bh[0] = ph; bl[0] = pl;
    bh[1] = partner_u32<0>(ph); bl[1] = partner_u32<0>(pl);        // lane ^ 1
    bh[2] = partner_u32<1>(ph); bl[2] = partner_u32<1>(pl);        // lane ^ 2
    bh[3] = partner_u32<1>(bh[1]); bl[3] = partner_u32<1>(bl[1]);  // lane ^ 3
    uint32_t oh = 0, ol = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const int src = bb ^ p;                    // bh[src] holds group lane bb's dword
      const uint32_t hv = src == 0 ? bh[0] : src == 1 ? bh[1] : src == 2 ? bh[2] : bh[3];
      const uint32_t lv = src == 0 ? bl[0] : src == 1 ? bl[1] : src == 2 ? bl[2] : bl[3];
      oh |= ((hv >> (8 * p)) & 0xFFu) << (8 * bb);
      ol |= ((lv >> (8 * p)) & 0xFFu) << (8 * bb);
    }
    ph = oh;
    pl = ol;
  }
  const int s = bfly_sum_i32<2>(q0 + q1 + q2 + q3);
  const float scale = ldexpf(r, e - kFixedBits);
  const size_t base = (size_t)t * (a.H / 4) + b * 64;
  const size_t si = (size_t)t * (a.H / kSubW) + b * 16 + (lane >> 2);
  if (L) {
    L->xh[base + lane] = ph;
    L->xl[base + lane] = pl;
    if ((lane & 3) == 0) {
      L->xs[si] = scale;
      L->xa[si] = s;
    }
  } else {
    cst(&a.xh[base + lane], ph);
    cst(&a.xl[base + lane], pl);
    if ((lane & 3) == 0) {
      cstf(&a.xs[si], scale);
      csti(&a.xa[si], s);
    }
  }
}

// T > kSmallT: one wave per token (top-k) and per x block (limbs), global.
__device__ void phase_topk_quant(const PersistArgs& a, const float* x, int layer_i) {
  const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6;
  const int nb = a.H / kBlockW;
  const int units = a.T + a.T * nb;
  for (int u = blockIdx.x * nw + wave; u < units; u += gridDim.x * nw) {
    if (u < a.T) topk_wave(a, u, layer_i, nullptr, true);
    else quant_x_wave(a, x, (u - a.T) / nb, (u - a.T) % nb, nullptr);
  }
}

// T <= kSmallT: every workgroup routes all tokens and quantises all of x
// into its own LDS.
__device__ void local_topk_quant(const PersistArgs& a, const float* x, int layer_i, PersistLds& L) {
  const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6;
  const int nb = a.H / kBlockW;
  const int units = a.T + a.T * nb;
  for (int u = wave; u < units; u += nw) {
    if (u < a.T) topk_wave(a, u, layer_i, &L, blockIdx.x == 0);
    else quant_x_wave(a, x, (u - a.T) / nb, (u - a.T) % nb, &L);
  }
  __syncthreads();
}

// ------------------------------------------------------ grouping (LDS) ---
// Stable bucket sort of (token, slot) pairs by expert.
__device__ void build_groups(const PersistArgs& a, PersistLds& L) {
  const int tid = threadIdx.x, nt = blockDim.x, E = a.E, k = a.k, T = a.T, P = T * k;
  const int wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < E; i += nt) L.cnt[i] = 0;
  for (int i = tid; i < E * 8; i += nt) L.mask[i] = 0;
  if (!a.small) {
    for (int p = tid; p < P; p += nt) {
      L.ids[p] = cldi(&a.ids[p]);
      L.wl[p] = cldf(&a.wts[p]);
    }
  }
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int e = valid_id(L.ids[p], E), t = p / k;
    atomicAdd(&L.cnt[e], 1);
    atomicOr(&L.mask[e * 8 + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  // exclusive scans of counts and of the non-empty flags, 64 experts per wave
  // and pass, wave totals combined through LDS (E <= 1024)
  int* wsum = (int*)L.red;              // [2 * 16] chunk totals (router scratch is free here)
  const int nchunk = (E + 63) / 64;
  for (int c = wave; c < nchunk; c += nt / 64) {
    const int e = c * 64 + lane;
    const int cv = e < E ? L.cnt[e] : 0;
    const int sc = wave_incl_scan(cv);
    const int sf = wave_incl_scan(cv > 0 ? 1 : 0);
    if (lane == 63) {
      wsum[2 * c] = sc;
      wsum[2 * c + 1] = sf;
    }
  }
  __syncthreads();
  for (int c = wave; c < nchunk; c += nt / 64) {
    int bc = 0, bf = 0;
    for (int i = 0; i < c; ++i) {
      bc += wsum[2 * i];
      bf += wsum[2 * i + 1];
    }
    const int e = c * 64 + lane;
    const int cv = e < E ? L.cnt[e] : 0;
    const int sc = wave_incl_scan(cv) + bc;
    const int sf = wave_incl_scan(cv > 0 ? 1 : 0) + bf;
    if (e < E) {
      L.off[e] = sc - cv;
      if (cv > 0) L.act[sf - 1] = e;
      if (e == E - 1) {
        L.off[E] = sc;
        *L.nact = sf;
      }
    }
  }
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int e = valid_id(L.ids[p], E), t = p / k;
    int rank = 0;
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(L.mask[e * 8 + w]);
    rank += __popc(L.mask[e * 8 + (t >> 5)] & ((1u << (t & 31)) - 1u));
    const int pos = L.off[e] + rank;
    L.pairs[pos] = p;
    L.pos_of[p] = pos;
  }
  __syncthreads();
  // per token, its bucket positions in ascending order (= ascending expert):
  // the rank of a position among the token's k positions
  for (int p = tid; p < P; p += nt) {
    const int t = p / k, q = L.pos_of[p];
    int rank = 0;
    for (int j = 0; j < k; ++j) rank += L.pos_of[t * k + j] < q ? 1 : 0;
    L.tok_order[t * k + rank] = q;
  }
  __syncthreads();
}

// ----------------------------------------------------------- phase GU ---
__device__ __forceinline__ void x_chunk(const PersistArgs& a, const PersistLds& L, int t, int ch,
                                        uint32_t (&xh)[16], uint32_t (&xl)[16], float (&xs)[4],
                                        int (&xa)[4]) {
  const size_t xo = (size_t)t * (a.H / 4) + ch * 16;
  const size_t si = (size_t)t * (a.H / kSubW) + ch * 4;
  if (a.small) {
    const uint4* ph = (const uint4*)(L.xh + xo);
    const uint4* pl = (const uint4*)(L.xl + xo);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 h = ph[i], l = pl[i];
      xh[4 * i] = h.x; xh[4 * i + 1] = h.y; xh[4 * i + 2] = h.z; xh[4 * i + 3] = h.w;
      xl[4 * i] = l.x; xl[4 * i + 1] = l.y; xl[4 * i + 2] = l.z; xl[4 * i + 3] = l.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[i] = L.xs[si + i];
      xa[i] = L.xa[si + i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t h = cld64(a.xh + xo + 2 * i), l = cld64(a.xl + xo + 2 * i);
      xh[2 * i] = (uint32_t)h;
      xh[2 * i + 1] = (uint32_t)(h >> 32);
      xl[2 * i] = (uint32_t)l;
      xl[2 * i + 1] = (uint32_t)(l >> 32);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[i] = cldf(&a.xs[si + i]);
      xa[i] = cldi(&a.xa[si + i]);
    }
  }
}

// Shared-expert gate/up item: rows [2*item, 2*item+2), 4 waves per row, each
// over a quarter of H; fp32 FMA on bf16 weights.  The first item of a
// workgroup has its rows in the LDS buffer as [row][gate, up][H] bf16.
__device__ __forceinline__ bool shared_pf_fits(const PersistArgs& a) {
  return (size_t)kSharedItemRows * 2 * a.H * 2 <= (size_t)a.pfb;
}

__device__ void shared_gu_prefetch(const PersistArgs& a, const LayerPtrs& Lp, PersistLds& L) {
  const int n_shared = a.Fs / kSharedItemRows;
  if ((int)blockIdx.x >= n_shared || !shared_pf_fits(a)) return;
  for (int r = 0; r < kSharedItemRows; ++r) {
    const int f = blockIdx.x * kSharedItemRows + r;
    copy_to_lds(Lp.sg + (size_t)f * a.H, L.pfb + (size_t)(2 * r) * a.H * 2, (size_t)a.H * 2);
    copy_to_lds(Lp.su + (size_t)f * a.H, L.pfb + (size_t)(2 * r + 1) * a.H * 2, (size_t)a.H * 2);
  }
}

__device__ void shared_gu_item(const PersistArgs& a, const LayerPtrs& Lp, const float* x, int item,
                               PersistLds& L) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rw = wave >> 2, qtr = wave & 3;
  const int f = item * kSharedItemRows + rw;
  const int hq = a.H / 4;
  const int T = a.T;
  const bool from_lds = item == (int)blockIdx.x && shared_pf_fits(a);
  const uint16_t* gsrc = from_lds ? (const uint16_t*)(L.pfb + (size_t)(2 * rw) * a.H * 2) : Lp.sg + (size_t)f * a.H;
  const uint16_t* usrc = from_lds ? (const uint16_t*)(L.pfb + (size_t)(2 * rw + 1) * a.H * 2) : Lp.su + (size_t)f * a.H;
  for (int t = 0; t < T; ++t) {
    float g = 0.f, u = 0.f;
    for (int h = qtr * hq + 8 * lane; h < (qtr + 1) * hq; h += 512) {
      const uint4 wg = *(const uint4*)(gsrc + h), wu = *(const uint4*)(usrc + h);
      const float4 x0 = cldf4(x + (size_t)t * a.H + h), x1 = cldf4(x + (size_t)t * a.H + h + 4);
      const uint32_t gw[4] = {wg.x, wg.y, wg.z, wg.w}, uw[4] = {wu.x, wu.y, wu.z, wu.w};
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        g = fmaf(bf16_to_f32(gw[c] & 0xFFFFu), xv[2 * c], g);
        g = fmaf(bf16_to_f32(gw[c] >> 16), xv[2 * c + 1], g);
        u = fmaf(bf16_to_f32(uw[c] & 0xFFFFu), xv[2 * c], u);
        u = fmaf(bf16_to_f32(uw[c] >> 16), xv[2 * c + 1], u);
      }
    }
    g = bfly_sum<6>(g);
    u = bfly_sum<6>(u);
    if (lane == 0) {
      L.sred[(wave * T + t) * 2] = g;
      L.sred[(wave * T + t) * 2 + 1] = u;
    }
  }
  __syncthreads();
  // combine the 4 quarter-row partials in a fixed order
  for (int q = threadIdx.x; q < kSharedItemRows * T; q += blockDim.x) {
    const int r = q / T, t = q % T;
    const int ff = item * kSharedItemRows + r;
    float g = 0.f, u = 0.f;
    for (int w4 = 0; w4 < 4; ++w4) {
      g += L.sred[((r * 4 + w4) * T + t) * 2];
      u += L.sred[((r * 4 + w4) * T + t) * 2 + 1];
    }
    const float rs = (float)cldd(&a.rinv[t]);
    cstf(&a.ash[(size_t)t * a.Fs + ff], silu_mul(g * rs, u * rs));
  }
  __syncthreads();
}

// Routed gate/up tile: rows [16*tile, +16) of expert act[u] for every token
// of its bucket, four tokens per pass over the decoded weights.
template <int FMT>
__device__ void routed_gu_tile(const PersistArgs& a, const LayerPtrs& Lp, int u, int tile,
                               PersistLds& L) {
  const int e = L.act[u];
  const int p0 = L.off[e], n = L.off[e + 1] - p0;
  const int nch = a.H / kChunkW;
  const int lpr = lanes_per_row(nch);
  const int cpl = nch / lpr;
  const int slots = blockDim.x / lpr;
  const int slot = threadIdx.x / lpr, j = threadIdx.x % lpr;
  const size_t nblk = (size_t)a.F * (a.H / kBlockW);
  constexpr bool q2k = FMT == 1;
  const MatPlanes pl = q2k ? q2k_planes(nblk) : cb2_planes(nblk);
  const uint8_t* gbase = Lp.gate + (size_t)e * a.gu_stride;
  const uint8_t* ubase = Lp.up + (size_t)e * a.gu_stride;
  const int f0 = tile * kGateTile;
  for (int r = slot; r < kGateTile; r += slots) {
    const int f = f0 + r;
    for (int tg = 0; tg < n; tg += 4) {
      float gacc[4] = {0.f, 0.f, 0.f, 0.f}, uacc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int cc = 0; cc < cpl; ++cc) {
        const int ch = j + cc * lpr;
        const size_t blk = (size_t)f * (a.H / kBlockW) + ch / 4;
        const int c = ch & 3;
        uint32_t gq[16], uq[16];
        uint32_t gsc, usc, gdd, udd;
        const uint4 gv = *(const uint4*)(gbase + pl.q + blk * 64 + c * 16);
        const uint4 uv = *(const uint4*)(ubase + pl.q + blk * 64 + c * 16);
        if (q2k) {
          gsc = *(const uint32_t*)(gbase + pl.s + blk * 16 + c * 4);
          usc = *(const uint32_t*)(ubase + pl.s + blk * 16 + c * 4);
          gdd = *(const uint32_t*)(gbase + pl.d + blk * 4);
          udd = *(const uint32_t*)(ubase + pl.d + blk * 4);
          gq[0] = gv.x; gq[1] = gv.y; gq[2] = gv.z; gq[3] = gv.w;
          uq[0] = uv.x; uq[1] = uv.y; uq[2] = uv.z; uq[3] = uv.w;
        } else {
          gsc = gbase[pl.s + blk * 4 + c];
          usc = ubase[pl.s + blk * 4 + c];
          gdd = *(const uint16_t*)(gbase + pl.d + blk * 2);
          udd = *(const uint16_t*)(ubase + pl.d + blk * 2);
          cb2_decode_dword(L.tab, gv.x, gq[0], gq[1], gq[2], gq[3]);
          cb2_decode_dword(L.tab, gv.y, gq[4], gq[5], gq[6], gq[7]);
          cb2_decode_dword(L.tab, gv.z, gq[8], gq[9], gq[10], gq[11]);
          cb2_decode_dword(L.tab, gv.w, gq[12], gq[13], gq[14], gq[15]);
          cb2_decode_dword(L.tab, uv.x, uq[0], uq[1], uq[2], uq[3]);
          cb2_decode_dword(L.tab, uv.y, uq[4], uq[5], uq[6], uq[7]);
          cb2_decode_dword(L.tab, uv.z, uq[8], uq[9], uq[10], uq[11]);
          cb2_decode_dword(L.tab, uv.w, uq[12], uq[13], uq[14], uq[15]);
        }
        // one token at a time (its x chunk is 40 registers); the decoded
        // weights stay live across the four tokens
#pragma unroll 1
        for (int tt = 0; tt < 4; ++tt) {
          if (tg + tt >= n) break;
          const int t = L.pairs[p0 + tg + tt] / a.k;
          uint32_t xh[16], xl[16];
          float xs[4];
          int xa[4];
          x_chunk(a, L, t, ch, xh, xl, xs, xa);
          float gp, up;
          if (q2k) {
            const uint32_t gw[4] = {gq[0], gq[1], gq[2], gq[3]}, uw[4] = {uq[0], uq[1], uq[2], uq[3]};
            gp = q2k_chunk_dot(gw, gsc, half_to_f32(gdd & 0xFFFFu), half_to_f32(gdd >> 16), xh, xl, xs, xa);
            up = q2k_chunk_dot(uw, usc, half_to_f32(udd & 0xFFFFu), half_to_f32(udd >> 16), xh, xl, xs, xa);
          } else {
            gp = half_to_f32(gdd) * xs[0] * (float)cb2_chunk_dot(gq, xh, xl, gsc);
            up = half_to_f32(udd) * xs[0] * (float)cb2_chunk_dot(uq, xh, xl, usc);
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
        if (tg + tt >= n) continue;
        const float g = bfly_sum_dyn(gacc[tt], lpr);
        const float uu = bfly_sum_dyn(uacc[tt], lpr);
        if (j == 0) L.ga[(tg + tt) * kGateTile + r] = silu_mul(g, uu);
      }
    }
  }
  __syncthreads();
  // quantise each bucket token's 16 outputs: 16 lanes per token
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  for (int tb = wave * 4; tb < n; tb += nw * 4) {
    const int tt = tb + (lane >> 4), r = lane & 15;
    const bool live = tt < n;
    const float v = live ? L.ga[tt * kGateTile + r] : 0.f;
    const float m = bfly_max<4>(fabsf(v));
    const int ex = fixed_exp(m);
    const int q = to_fixed(v, ex);
    const int s = bfly_sum_i32<4>(q);
    if (live) L.qtmp[tt * kGateTile + r] = q;
    __builtin_amdgcn_wave_barrier();
    if (live) {
      const int pair = L.pairs[p0 + tt];
      if (r < 4) {
        int h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split_limbs(L.qtmp[tt * kGateTile + 4 * i + r], h[i], l[i]);
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

template <int FMT>
__device__ void phase_gateup(const PersistArgs& a, const LayerPtrs& Lp, const float* x, PersistLds& L) {
  const int n_shared = a.Fs / kSharedItemRows;
  const int tiles = a.F / kGateTile;
  const int na = *L.nact;
  const int n_items = n_shared + na * tiles;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    if (it < n_shared) {
      shared_gu_item(a, Lp, x, it, L);
    } else {
      const int r = it - n_shared;
      routed_gu_tile<FMT>(a, Lp, r / tiles, r % tiles, L);
    }
  }
}

// ------------------------------------------------------------ phase D ---
// The first tile of a workgroup (rows r0 = 8*blockIdx.x ..) has its shared
// down rows ([8][Fs] bf16) and the Q2_K planes of up to `npf` experts
// ([qs 8*nb*64][scales 8*nb*16][d,dmin 8*nb*4], nb = F/256) in the LDS
// buffer.
struct DownPfPlan {
  size_t sd_bytes, per_expert;
  int npf;
};

__device__ __forceinline__ DownPfPlan down_pf_plan(const PersistArgs& a, int na) {
  DownPfPlan p;
  const int nb = a.F / kBlockW;
  p.sd_bytes = a.Fs ? (size_t)kDownRows * a.Fs * 2 : 0;
  if (p.sd_bytes > (size_t)a.pfb) p.sd_bytes = 0;          // shared rows do not fit: not prefetched
  p.per_expert = (size_t)kDownRows * nb * kQ2KBytes;
  const size_t room = (size_t)a.pfb - p.sd_bytes;
  const int fit = (int)(room / p.per_expert);
  p.npf = na < fit ? na : fit;
  return p;
}

__device__ void down_prefetch(const PersistArgs& a, const LayerPtrs& Lp, PersistLds& L) {
  const int r0 = blockIdx.x * kDownRows;
  if (r0 >= a.H) return;
  const DownPfPlan p = down_pf_plan(a, *L.nact);
  const int nb = a.F / kBlockW;
  if (p.sd_bytes) copy_to_lds(Lp.sd + (size_t)r0 * a.Fs, L.pfb, p.sd_bytes);
  const size_t nblk = (size_t)a.H * nb;
  const MatPlanes pl = q2k_planes(nblk);
  for (int u = 0; u < p.npf; ++u) {
    const uint8_t* base = Lp.down + (size_t)L.act[u] * a.dn_stride;
    uint8_t* dst = L.pfb + p.sd_bytes + (size_t)u * p.per_expert;
    const size_t b0 = (size_t)r0 * nb;
    copy_to_lds(base + pl.q + b0 * 64, dst, (size_t)kDownRows * nb * 64);
    copy_to_lds(base + pl.s + b0 * 16, dst + (size_t)kDownRows * nb * 64, (size_t)kDownRows * nb * 16);
    copy_to_lds(base + pl.d + b0 * 4, dst + (size_t)kDownRows * nb * 80, (size_t)kDownRows * nb * 4);
  }
}

__device__ void phase_down(const PersistArgs& a, const LayerPtrs& Lp, const float* x, float* y,
                           PersistLds& L) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int nb = a.F / kBlockW;
  const int nch = a.F / kChunkW;
  const int lpr = lanes_per_row(nch);
  const int cpl = nch / lpr;
  const int rpi = 64 / lpr;
  const int rsub = lane / lpr, j = lane % lpr;
  const size_t nblk = (size_t)a.H * nb;
  const MatPlanes pl = q2k_planes(nblk);
  const int na = *L.nact;
  const int n_tiles = a.H / kDownRows;
  const int T = a.T;
  const DownPfPlan pp = down_pf_plan(a, na);
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const int r0 = tile * kDownRows;
    const bool first = tile == (int)blockIdx.x;
    for (int u = wave; u < na; u += nw) {
      const int e = L.act[u];
      const bool lds_w = first && u < pp.npf;
      const uint8_t* gbase = Lp.down + (size_t)e * a.dn_stride;
      const uint8_t* lbase = L.pfb + pp.sd_bytes + (size_t)u * pp.per_expert;
      const int q0 = L.off[e], q1 = L.off[e + 1];
      for (int rr = rsub; rr < kDownRows; rr += rpi) {
        const int h = r0 + rr;
        // one 64-weight chunk of this row at a time, read once for all pairs
#pragma unroll 1
        for (int cc = 0; cc < cpl; ++cc) {
          const int ch = j + cc * lpr;
          const int c = ch & 3;
          uint4 qv;
          uint32_t scm, dd;
          if (lds_w) {
            const size_t lb = (size_t)rr * nb + ch / 4;      // block within the tile
            qv = *(const uint4*)(lbase + lb * 64 + c * 16);
            scm = *(const uint32_t*)(lbase + (size_t)kDownRows * nb * 64 + lb * 16 + c * 4);
            dd = *(const uint32_t*)(lbase + (size_t)kDownRows * nb * 80 + lb * 4);
          } else {
            const size_t blk = (size_t)h * nb + ch / 4;
            qv = *(const uint4*)(gbase + pl.q + blk * 64 + c * 16);
            scm = *(const uint32_t*)(gbase + pl.s + blk * 16 + c * 4);
            dd = *(const uint32_t*)(gbase + pl.d + blk * 4);
          }
          const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
          const float d = half_to_f32(dd & 0xFFFFu), dm = half_to_f32(dd >> 16);
          for (int pos = q0; pos < q1; ++pos) {
            const int pair = L.pairs[pos];
            uint32_t xh[16], xl[16];
            float xs[4];
            int xa[4];
            const uint32_t* ph = a.ah + (size_t)pair * (a.F / 4) + ch * 16;
            const uint32_t* plw = a.al + (size_t)pair * (a.F / 4) + ch * 16;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const uint64_t hv = cld64(ph + 2 * i), lv = cld64(plw + 2 * i);
              xh[2 * i] = (uint32_t)hv;
              xh[2 * i + 1] = (uint32_t)(hv >> 32);
              xl[2 * i] = (uint32_t)lv;
              xl[2 * i + 1] = (uint32_t)(lv >> 32);
            }
            const size_t si = (size_t)pair * (a.F / kSubW) + ch * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              xs[i] = cldf(&a.as[si + i]);
              xa[i] = cldi(&a.aa[si + i]);
            }
            float part = q2k_chunk_dot(qw, scm, d, dm, xh, xl, xs, xa);
            part = bfly_sum_dyn(part, lpr);
            // lane j == 0 of this row group owns the entry for every chunk
            if (j == 0) L.o[pos * kDownRows + rr] = cc == 0 ? part : L.o[pos * kDownRows + rr] + part;
          }
        }
      }
    }
    // shared expert down: one row per wave, lanes over Fs, all tokens
    if (a.Fs && wave < kDownRows) {
      const int h = r0 + wave;
      const uint16_t* srow = (first && pp.sd_bytes) ? (const uint16_t*)L.pfb + (size_t)wave * a.Fs
                                                    : Lp.sd + (size_t)h * a.Fs;
      for (int t = 0; t < T; ++t) {
        const float* at = a.ash + (size_t)t * a.Fs;
        float s = 0.f;
        for (int f = 8 * lane; f < a.Fs; f += 512) {
          const uint4 w = *(const uint4*)(srow + f);
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint64_t av = cld64(at + f + 2 * c);
            s = fmaf(bf16_to_f32(ww[c] & 0xFFFFu), __uint_as_float((uint32_t)av), s);
            s = fmaf(bf16_to_f32(ww[c] >> 16), __uint_as_float((uint32_t)(av >> 32)), s);
          }
        }
        s = bfly_sum<6>(s);
        if (lane == 0) L.sh[t * kDownRows + wave] = s;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < T * kDownRows; idx += blockDim.x) {
      const int t = idx / kDownRows, rr = idx % kDownRows, h = r0 + rr;
      float acc = 0.f;
      for (int jj = 0; jj < a.k; ++jj) {
        const int pos = L.tok_order[t * a.k + jj];
        const int pair = L.pairs[pos];
        acc = fmaf(L.wl[pair], L.o[pos * kDownRows + rr], acc);
      }
      if (a.Fs) acc += L.sh[idx];
      if (a.residual) acc += cldf(&x[(size_t)t * a.H + h]);
      cstf(&y[(size_t)t * a.H + h], acc);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------- kernel ---
template <int FMT>
__global__ void __launch_bounds__(kPersistThreads) k_persist(PersistArgs a) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  PersistLds L = carve_lds(lds_raw, a, FMT == 2);
  if (FMT == 2) copy_to_lds(a.cbtab, L.tab, (size_t)kCbTabWords * 4);
  router_prefetch(a, a.layers[0], L);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t epoch = a.epoch0;
  for (int li = 0; li < a.n_layers; ++li) {
    const LayerPtrs Lp = a.layers[li];
    const float* x = li == 0 ? a.x_in : ((li - 1) & 1 ? a.xbuf1 : a.xbuf0);
    float* y = li == a.n_layers - 1 ? a.y_out : (li & 1 ? a.xbuf1 : a.xbuf0);
    phase_router(a, Lp, x, L);
    shared_gu_prefetch(a, Lp, L);              // buffer is free: the router rows are consumed
    if (!grid_barrier(a, ++epoch)) return;
    if (a.small) {
      local_topk_quant(a, x, li, L);
    } else {
      phase_topk_quant(a, x, li);
      if (!grid_barrier(a, ++epoch)) return;
    }
    build_groups(a, L);
    phase_gateup<FMT>(a, Lp, x, L);
    down_prefetch(a, Lp, L);                   // shared gate/up rows are consumed
    if (!grid_barrier(a, ++epoch)) return;
    phase_down(a, Lp, x, y, L);
    if (li + 1 < a.n_layers) {
      router_prefetch(a, a.layers[li + 1], L); // down rows are consumed
      if (!grid_barrier(a, ++epoch)) return;
    }
  }
}

}  // namespace qs
