// qs_persist.h -- the whole decode call (every layer, every step of the MoE
// path) as one persistent cooperative kernel on gfx950.
//
// Why one kernel: each layer has three all-to-all dependencies (all logits
// before top-k, all SwiGLU outputs of an expert before its down GEMV, all of
// x_{l+1} before the next router).  A kernel boundary costs ~2.5 us on
// MI355X and a grid barrier about the same; inside one kernel the weights
// that do not depend on the pending result (router rows, shared-expert rows,
// the down rows of experts already chosen) are copied into LDS while the
// workgroup waits, so their HBM latency hides behind the wait.
//
// Every weight the kernel multiplies is read from LDS: a workgroup's first
// piece of each kind is copied during the preceding wait, later pieces are
// copied on demand.  Each compute routine therefore exists once, which keeps
// the kernel's code small enough for the instruction cache: a layer walks
// through all of it, so code that does not fit is re-fetched every layer.
//
// This file holds the small-batch kernel (T <= kSmallT) and the helpers both
// persistent kernels share; qs_big.h holds the batched kernel.
// Small batches, per layer:
//   R   x -> LDS (one coherent copy); per-token RMS scale; router logits;
//       the shared expert's gate/up items (they need only x)
//   --- barrier
//   K   logits -> LDS; top-k of every token and the grouping, redundantly
//       in every workgroup (this saves a barrier); routed gate/up tiles ->
//       LDS while x becomes fixed-point limbs
//   GU  SwiGLU outputs of the routed tiles
//   --- barrier (meanwhile: down rows, next layer's router rows and shared
//       items -> LDS)
//   D   SwiGLU limbs -> LDS; down GEMVs + combine + shared down + residual
//   --- barrier
//
// Barrier: per-XCD arrival counters, a global counter bumped by each XCD's
// last arriver, per-XCD release lines written by the global last arriver.
// Data crossing a barrier is written and read with agent-scope (sc1)
// accesses, coherent across the XCDs' separate L2s without the whole-L2
// writeback/invalidate of a release or acquire fence.  Before arriving, a
// workgroup drains its own stores; the prefetch copies are issued after
// that drain by waves 1..7 while wave 0 arrives and polls.  Every wait is
// bounded: a workgroup that gives up raises an error flag and every
// workgroup leaves at its next barrier, so the grid always drains.
#pragma once
#include "qs_kernels.h"
#include "qs_wave.h"

#define QS_LDS __attribute__((address_space(3)))

namespace qs {

constexpr int kPersistThreads = 512;
constexpr int kSmallT = 4;
constexpr int kGuWinMax = 4;           // SMALL: routed gate/up tiles in flight per workgroup, at most
constexpr int kShPairsLds = 8;        // shared gate/up items per register round (their LDS partials)
constexpr int kShDnRegs = 8;          // shared down chunks per thread per register round
constexpr int kSpinMax = 1 << 22;
constexpr int kLLSpinMax = 1 << 16;    // polls of a flagged read (about 0.1 s) before it gives up
// sync words (uint32 index): [16*x] per-XCD counters, [128] global counter,
// [144 + 16*x] release lines, [272] error flag
constexpr int kSyncWords = 512;
constexpr int kSyncGlobal = 128, kSyncRelease = 144, kSyncError = 272;
constexpr int kSharedItemRows = 2;     // shared gate/up rows per item (4 waves per row)
constexpr uint32_t kPfbMax = 128 * 1024;
constexpr int kCoherent = 16;          // cache-policy bits of an agent-coherent (sc1) load

struct LayerPtrs {
  const float* router;
  const float* bias;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const uint8_t* sg;          // shared expert rows (bf16, or the 8-bit rows below)
  const uint8_t* su;
  const uint8_t* sd;
  const uint64_t* emap;       // paged layer: [E] address of each expert's record, else null
};

// Expert e's gate (which 0), up (1) or down (2) matrix.  A resident layer
// holds each kind as one array of E matrices.  A paged layer holds one
// record per expert, [gate | up | down] at offsets 0, gu_stride and
// 2 gu_stride, at the address its expert map gives: an HBM cache slot, or
// the expert's copy in pinned host memory, which the loads then read over
// PCIe.  The map does not change during a launch.
// Only the kernels built for paged layers (kPaged) read the map; the
// others keep the resident addressing alone.
template <class A>
__device__ __forceinline__ const uint8_t* ex_mat(const A& a, const LayerPtrs& Lp, int which, int e) {
  if constexpr (A::kPaged) {
    if (Lp.emap) {
      const uint8_t* rec = (const uint8_t*)(uintptr_t)Lp.emap[e];
      return rec + (size_t)which * a.gu_stride;
    }
  }
  return which == 0 ? Lp.gate + (size_t)e * a.gu_stride
                    : which == 1 ? Lp.up + (size_t)e * a.gu_stride : Lp.down + (size_t)e * a.dn_stride;
}

struct PersistArgs {
  static constexpr bool kFixedShape = false;
  static constexpr bool kPaged = false;
  const LayerPtrs* layers;   // device array, first entry = layer0
  int G;                     // workgroups of the launch (a multiple of 8)
  int n_layers, T, H, E, k, F, Fs;
  int gq2k, prenorm, residual;
  int gfmt, dfmt;            // routed gate/up and down formats (kFmt*): Q4_K layers have both at kFmtQ4K
  int sq8;                   // shared expert in 8-bit blocks (else bf16)
  int r_et, r_tt;            // router unit: experts x tokens
  uint32_t pfb;              // bytes of the LDS weight-staging buffer
  uint32_t pfa;              // SMALL: bytes of its first region (router, shared items, gate/up tiles);
                             // the rest holds the down rows
  size_t gu_stride, dn_stride;
  const uint32_t* cbtab;
  const float* x_in;
  float* y_out;
  int32_t* ids_out;
  float* w_out;
  double* logits;            // [T][E]
  double* rinv;              // [T]
  int32_t* ids;              // [T][k]      (not SMALL)
  float* wts;                // [T][k]      (not SMALL)
  uint32_t* xh;              // [T][H/4]    (not SMALL)
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
  int spin_ll;               // polls of a flagged read before it gives up
  int spin_bar;              // polls of a grid-barrier wait before it gives up
  // small-batch flow: flagged copies of the data that crosses workgroups
  uint64_t* ll_lg;           // [T][E][2]  logits (low, high words)
  uint64_t* ll_a;            // [ah | al | as | aa | ash] words of the SwiGLU outputs
  uint64_t* llx0;            // [T][H]     residual stream between layers
  uint64_t* llx1;
  uint32_t ll_epoch;         // flags of this call: ll_epoch + 3*layer + {0: x in, 1: logits, 2: SwiGLU}
  uint64_t* ll_dot;          // [T][G] steering: per-workgroup partial dot products (flag of the SwiGLU words)
  // steering (the STEER instantiations): m_l -> m_l - sscale * d_l * (d_l . m_l) before the residual add
  float sscale;
  const float* sdir;         // [n_layers][H] directions of this call's layers
  float* mb;                 // [T][H] MoE outputs before steering
  float* part;               // [T][G] batched flow: per-workgroup partial dot products
  // batched flow only
  int mfma_min;              // bucket size from which the MFMA path runs
  float* af;                 // [T*k][F] SwiGLU outputs of MFMA buckets (by pair id)
  float* ob;                 // [T*k][H] routed down outputs (by bucket position)
  float* sb;                 // [T][H]   shared-expert down outputs
};

// Phase stamps for profiling builds (-DQS_STAMPS): thread 0 of each
// workgroup records the 100 MHz wall clock at point k of layer li.  The
// default build compiles them out.
#ifdef QS_STAMPS
constexpr int kStampLayers = 64, kStampWgs = 256, kStampPts = 24;
__device__ uint64_t g_qs_stamps[kStampLayers * kStampWgs * kStampPts];
__device__ int g_qs_stamp_li[kStampWgs];   // layer of the workgroup's current stamps
#define QS_STAMP(li, k)                                                                   \
  do {                                                                                    \
    if (threadIdx.x == 0 && (li) < kStampLayers && blockIdx.x < kStampWgs) {             \
      g_qs_stamps[((li) * kStampWgs + blockIdx.x) * kStampPts + (k)] = __builtin_amdgcn_s_memrealtime(); \
      g_qs_stamp_li[blockIdx.x] = (li);                                                   \
    }                                                                                     \
  } while (0)
#define QS_STAMP2(k) QS_STAMP(g_qs_stamp_li[blockIdx.x], k)
// point k of whichever layer ran last, in the spare row kStampLayers - 1
// (no load of the current layer)
#define QS_STAMP3(k)                                                                      \
  do {                                                                                    \
    if (threadIdx.x == 0 && blockIdx.x < kStampWgs)                                       \
      g_qs_stamps[((kStampLayers - 1) * kStampWgs + blockIdx.x) * kStampPts + (k)] =      \
          __builtin_amdgcn_s_memrealtime();                                               \
  } while (0)
#else
#define QS_STAMP(li, k) \
  do {                  \
  } while (0)
#define QS_STAMP2(k) \
  do {               \
  } while (0)
#define QS_STAMP3(k) \
  do {               \
  } while (0)
#endif

// Thread index through an opaque move: values derived from it are then
// recomputed in each phase instead of being hoisted out of the layer loop
// and kept live (in registers) across every phase.
__device__ __forceinline__ int qs_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

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

// ---------------------------------------------------- flagged words ---
// Data that one workgroup writes and every other one reads, without a grid
// barrier between them: each 8-byte word carries 32 bits of data and a 32-bit
// flag, written by one 64-bit store (8-byte stores are single-copy atomic),
// so a reader that sees the flag it expects has the data of the same store.
// Flags grow with every layer of every call, so stale words never match.
__device__ __forceinline__ void ll_store(uint64_t* p, uint32_t v, uint32_t flag) {
  __hip_atomic_store(p, (uint64_t)v | ((uint64_t)flag << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waves [0, nwp) of the workgroup read words [0, n) of src into dst (their
// data halves), re-reading the words whose flag is not `flag` yet.  Thread
// tid owns words tid + 64*nwp*j (j < 32, so n <= 2048*nwp).  Each wave polls
// on its own until its words are in; the other waves only meet them at the
// closing barrier, so they may have copies into LDS in flight (a wave that
// has issued one waits for it at its next LDS access).  Bounded: false for
// every thread (after raising the error word) when the data does not arrive;
// `err` is an LDS word that is 0 at kernel start.
template <class A>
__device__ __forceinline__ bool ll_read(const A& a, const uint64_t* src, QS_LDS uint32_t* dst, int n,
                                        uint32_t flag, QS_LDS int* err, int nwp = kPersistThreads / 64) {
  const int tid = qs_tid(), nth = nwp * 64;
  if (tid < nth) {
    uint32_t missing = 0;
    for (int j = 0; j < 32; ++j)
      if (tid + j * nth < n) missing |= 1u << j;
    for (int spins = 0;; ++spins) {
      // a batch of loads in flight at once, then the checks
      for (int j0 = 0; j0 < 32; j0 += 8) {
        if (!((missing >> j0) & 0xFFu)) continue;
        uint64_t w[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if ((missing >> (j0 + jj)) & 1u) w[jj] = cld64(src + tid + (j0 + jj) * nth);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (((missing >> (j0 + jj)) & 1u) && (uint32_t)(w[jj] >> 32) == flag) {
            dst[tid + (j0 + jj) * nth] = (uint32_t)w[jj];
            missing &= ~(1u << (j0 + jj));
          }
      }
      if (!__builtin_amdgcn_ballot_w64(missing != 0)) break;
      if (spins + 1 >= a.spin_ll) {     // a.spin_ll polls have found the data missing
        if ((tid & 63) == 0) {
          cst(&a.sync[kSyncError], 1u);
          *err = 1;
        }
        break;
      }
      if ((spins & 63) == 63 && cld(&a.sync[kSyncError])) {
        if ((tid & 63) == 0) *err = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);   // (measured: 2 slightly ahead of 0, 1 and 4)
    }
  }
  __syncthreads();
  return *err == 0;
}

// --------------------------------------------------------- LDS loads ---
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef const QS_LDS uint8_t* lds_cptr;
__device__ __forceinline__ uint4 ld16(lds_cptr p) {
  const u32x4_t v = *(const QS_LDS u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld4(lds_cptr p) { return *(const QS_LDS uint32_t*)p; }
__device__ __forceinline__ uint32_t ld2(lds_cptr p) { return *(const QS_LDS uint16_t*)p; }
__device__ __forceinline__ uint32_t ld1(lds_cptr p) { return *p; }
__device__ __forceinline__ float4 lds_f4(const QS_LDS float* p) {
  const f32x4_t v = *(const QS_LDS f32x4_t*)p;
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 lds_u4(const QS_LDS uint32_t* p) { return ld16((lds_cptr)p); }

// ------------------------------------------------------ global -> LDS ---
// Copy `bytes` (rounded up to 16) from global memory straight into LDS with
// global_load_lds_dwordx4, spread over waves w = 0..nw-1 of the calling
// set; each wave instruction moves 64 x 16 bytes to consecutive LDS slots
// starting at M0.  AUX = kCoherent reads through to the agent-coherent level
// (sc1: data written by other workgroups in this launch).
//
// The instruction is issued from inline assembly on purpose: for the
// compiler's own form it must assume that any later LDS read may alias the
// copy and waits for it there, which would serialise every prefetch with the
// work it is meant to overlap.  The kernel orders these copies itself: an
// s_waitcnt (wait_all_and_sync or a grid barrier) precedes every read of a
// copied region, and a __syncthreads precedes every copy into a region that
// was read before.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int AUX>
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  if (AUX == kCoherent)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off sc1"
                 : : "s"(lds_addr), "v"(g) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 : : "s"(lds_addr), "v"(g) : "memory", "m0");
}
#pragma clang diagnostic pop

// Instruction i of a copy (1 KiB) goes to wave (lds/1024 + i) mod nw, so
// the many small copies at different destinations spread over the waves
// instead of all landing on the first one.
template <int AUX>
__device__ __forceinline__ void dma_to_lds(const void* g, QS_LDS void* lds, uint32_t bytes, int w, int nw) {
  const uint32_t lane = qs_tid() & 63;
  const uint32_t n16 = (bytes + 15u) >> 4;
  const uint32_t rot = ((uint32_t)(uintptr_t)lds >> 10) % (uint32_t)nw;
  const uint32_t first = ((uint32_t)w + (uint32_t)nw - rot) % (uint32_t)nw;
  for (uint32_t base = first * 64u; base < n16; base += (uint32_t)nw * 64u) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((QS_LDS uint4*)lds + base));
    if (base + lane < n16) dma16<AUX>((const uint4*)g + base + lane, dst);
  }
}

__device__ __forceinline__ void wait_all_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// A whole-workgroup copy that is consumed at once: the slot is free (every
// wave is past its previous use), copy, wait, and make it visible.
template <class CP>
__device__ __forceinline__ void stage_now(CP&& cp) {
  __syncthreads();
  cp((int)(qs_tid() >> 6), (int)(kPersistThreads >> 6));
  wait_all_and_sync();
}

// ------------------------------------------------------- grid barrier ---
// `pf(w, nw)` issues this workgroup's prefetch copies (waves 1..7 run it,
// after the drain and while wave 0 waits); they complete in the background
// and whoever reads them first waits (wait_all_and_sync).
template <class PF, class A>
__device__ __forceinline__ bool grid_barrier(const A& a, uint32_t epoch, PF&& pf) {
  const uint32_t x = blockIdx.x & 7u, per = (uint32_t)a.G >> 3;
  __builtin_amdgcn_s_waitcnt(0);     // this wave's coherent stores have completed
  __syncthreads();
  const int wave = qs_tid() >> 6, nw = kPersistThreads >> 6;
  if (wave > 0) pf(wave - 1, nw - 1);
  int ok = 1;
  if (qs_tid() == 0) {
    uint32_t* s = a.sync;
    const uint32_t old = catomic_add(&s[16 * x], 1u);
    if (old == epoch * per - 1u) {
      const uint32_t g = catomic_add(&s[kSyncGlobal], 1u);
      if (g == epoch * 8u - 1u)
        for (int i = 0; i < 8; ++i) cst(&s[kSyncRelease + 16 * i], epoch);
    }
    int spins = 0;
    while (cld(&s[kSyncRelease + 16 * x]) < epoch) {
      if (++spins >= a.spin_bar) {      // a.spin_bar polls have found the barrier closed
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
  // the prefetch copies may still be in flight: their consumer waits for them
  const int all = __syncthreads_and(ok);
  if (!all) __builtin_amdgcn_s_waitcnt(0);   // leaving: nothing may still write LDS
  return all;
}

// --------------------------------------------------------- LDS layout ---
__host__ __device__ inline uint32_t al16(uint32_t v) { return (v + 15u) & ~15u; }

// A shared-expert row of K weights: K bf16, or (8-bit blocks of 32 weights)
// the K int8 codes followed by the K/32 binary16 block scales, padded to 16
// bytes.  The same stride in HBM and LDS.
__host__ __device__ inline uint32_t srow_bytes(int K, bool q8) {
  return q8 ? al16((uint32_t)K + (uint32_t)K / 16) : (uint32_t)K * 2;
}

// SMALL activation buffer: [x fp32 T*H | logits fp64 T*E] during R and K;
// [a limbs hi | lo | scales | sums | shared SwiGLU T*Fs] during D.
__host__ __device__ inline uint32_t abuf_bytes(int T, int H, int E, int P, int F, int Fs) {
  const uint32_t rk = al16((uint32_t)T * H * 4) + al16((uint32_t)T * E * 8);
  const uint32_t dn = 2 * al16((uint32_t)P * F) + 2 * al16((uint32_t)P * F / 4) + al16((uint32_t)T * Fs * 4);
  return rk > dn ? rk : dn;
}

struct LdsLayout {
  uint32_t tab, cnt, off, act, aoff, nact, llerr, mask, ids, pairs, tok_order, cw, pos_of, wl, o, red, sh, ga, sred,
      qtmp, rinv, kf, cand, ncand, sv, xh, xl, xs, xa, abuf, emap, pfb, sdr, end;
};

__host__ __device__ inline int kf_stride(int E) { return (E + 7) & ~7; }

__host__ __device__ inline LdsLayout lds_layout(int E, int T, int P, int H, int F, int Fs, bool sq8, bool cb2,
                                                bool small, uint32_t pfb, bool shregs = false, bool paged = false) {
  LdsLayout l;
  uint32_t o = 0;
  auto take = [&](uint32_t n) {
    const uint32_t r = o;
    o += al16(n);
    return r;
  };
  l.tab = take(cb2 ? (uint32_t)kCbTabWords * 4 : 0);
  l.cnt = take(small ? 0 : (uint32_t)E * 4);           // general grouping only
  l.off = take(small ? 0 : (uint32_t)(E + 1) * 4);
  l.act = take((uint32_t)E * 4);
  l.aoff = take((uint32_t)(E + 1) * 4);
  l.nact = take(4);
  l.llerr = take(4);
  l.mask = take(small ? 0 : (uint32_t)E * 32);
  l.ids = take((uint32_t)P * 4);
  l.pairs = take((uint32_t)P * 4);
  l.tok_order = take((uint32_t)P * 4);
  l.cw = take(small ? (uint32_t)P * 4 : 0);
  l.pos_of = take((uint32_t)P * 4);
  l.wl = take((uint32_t)P * 4);
  l.o = take((uint32_t)P * kDownRows * 4);
  l.red = take(8 * 64 * 8);
  l.sh = take((uint32_t)T * kDownRows * 4);
  l.ga = take((uint32_t)(small && T > 1 ? kGuWinMax : 1) * T * kGateTile * 4);
  l.sred = take((uint32_t)(shregs ? kShPairsLds : 1) * 8 * T * 2 * 4);
  l.qtmp = take((uint32_t)(small && T > 1 ? kGuWinMax : 1) * T * kGateTile * 4);
  l.rinv = take((uint32_t)T * 8);
  // SMALL top-k: keys [T][S], group maxima [T][S/8], thresholds [T]
  l.kf = take(small && E > 256 ? (uint32_t)T * kf_stride(E) * 4 + (uint32_t)T * (((kf_stride(E) / 8) + 3) & ~3) * 4 +
                                     (uint32_t)T * 4 : 0);
  l.cand = take(small ? (uint32_t)T * E * 4 : 0);
  l.ncand = take(small ? (uint32_t)T * 4 : 0);
  l.sv = take(small ? (uint32_t)P * 8 : 0);
  l.abuf = take(small ? abuf_bytes(T, H, E, P, F, Fs) : 0);
  l.emap = take(small && paged ? (uint32_t)E * 8 : 0);   // a paged layer's expert map, a layer ahead
  l.pfb = take(pfb);
  // SMALL: the x limbs follow the staging buffer, so that once the gate/up
  // tiles are done the down rows can spill over them; the shared down rows
  // (copied a layer ahead) have their own slot.
  const uint32_t xq = small ? (uint32_t)T * H : 0;
  l.xh = take(xq);          // T*H/4 dwords
  l.xl = take(xq);
  l.xs = take(xq / 4);      // T*H/16 floats
  l.xa = take(xq / 4);
  l.sdr = take(small && !shregs ? (uint32_t)kDownRows * srow_bytes(Fs, sq8) : 0);
  l.end = o;
  return l;
}

struct PersistLds {
  QS_LDS uint32_t* tab;   // [8192] codebook quads (codebook gate/up only)
  QS_LDS int* cnt;        // [E]
  QS_LDS int* off;        // [E+1]
  QS_LDS int* act;        // [E]   active experts, ascending
  QS_LDS int* aoff;       // [E+1] bucket of active expert u: positions [aoff[u], aoff[u+1])
  QS_LDS int* nact;       // [1]
  QS_LDS int* llerr;      // [1] a flagged read gave up (0 at kernel start)
  QS_LDS uint32_t* mask;  // [E*8]
  QS_LDS int* ids;        // [P]   expert of pair id
  QS_LDS int* pairs;      // [P]   pair id at bucket position
  QS_LDS int* tok_order;  // [P]   per token, positions by ascending expert
  QS_LDS float* cw;       // [P]   SMALL: router weight of tok_order's entry
  QS_LDS int* pos_of;     // [P]   bucket position of pair id
  QS_LDS float* wl;       // [P]   router weight of pair id
  QS_LDS float* o;        // [P*kDownRows] down outputs
  QS_LDS double* red;     // [8*64] cross-wave partials
  QS_LDS float* sh;       // [T*kDownRows] shared-expert down outputs
  QS_LDS float* ga;       // SMALL: [kGuWinMax][T*kGateTile] SwiGLU tiles, per bucket token (one slot at T = 1)
  QS_LDS float* sred;     // [8*T*2] shared gate/up cross-wave partials
  QS_LDS int* qtmp;       // SMALL: [kGuWinMax][T*kGateTile] fixed-point tile values (one slot at T = 1)
  QS_LDS double* rinv;    // [T] per-token RMS scale
  QS_LDS float* kf;       // SMALL [T][kf_stride(E)] fp32 selection keys
  QS_LDS int* cand;       // SMALL [T][E] top-k candidates
  QS_LDS int* ncand;      // SMALL [T]
  QS_LDS double* sv;      // SMALL [T*k] selected logits in rank order
  QS_LDS uint32_t* xh;    // [T*H/4] SMALL: x limbs
  QS_LDS uint32_t* xl;
  QS_LDS float* xs;       // [T*H/16]
  QS_LDS uint64_t* emap;  // [E] paged layers (small-batch kernel): the layer's expert map
  QS_LDS int* xa;
  QS_LDS uint8_t* pfb;    // weight staging buffer
  QS_LDS uint8_t* sdr;    // SMALL: shared-expert down rows of this workgroup's output rows
  // SMALL views into the activation buffer
  QS_LDS float* ax;       // [T][H] x
  QS_LDS double* lg;      // [T][E] logits
  QS_LDS uint32_t* dah;   // [P][F/4]
  QS_LDS uint32_t* dal;
  QS_LDS float* das;      // [P][F/16]
  QS_LDS int* daa;
  QS_LDS float* dash;     // [T][Fs]
};

template <bool SMALL, class A>
__device__ __forceinline__ PersistLds carve_lds(uint8_t* raw, const A& a, bool cb2) {
  const uint32_t T = a.T, H = a.H, E = a.E, F = a.F, P = T * a.k;
  const LdsLayout l = lds_layout(E, T, P, H, F, a.Fs, a.sq8 != 0, cb2, SMALL, a.pfb, SMALL && sh_regs(a), A::kPaged);
  QS_LDS uint8_t* b = (QS_LDS uint8_t*)raw;
  PersistLds L;
  L.tab = (QS_LDS uint32_t*)(b + l.tab);
  L.cnt = (QS_LDS int*)(b + l.cnt);
  L.off = (QS_LDS int*)(b + l.off);
  L.act = (QS_LDS int*)(b + l.act);
  L.aoff = (QS_LDS int*)(b + l.aoff);
  L.nact = (QS_LDS int*)(b + l.nact);
  L.llerr = (QS_LDS int*)(b + l.llerr);
  L.mask = (QS_LDS uint32_t*)(b + l.mask);
  L.ids = (QS_LDS int*)(b + l.ids);
  L.pairs = (QS_LDS int*)(b + l.pairs);
  L.tok_order = (QS_LDS int*)(b + l.tok_order);
  L.cw = (QS_LDS float*)(b + l.cw);
  L.pos_of = (QS_LDS int*)(b + l.pos_of);
  L.wl = (QS_LDS float*)(b + l.wl);
  L.o = (QS_LDS float*)(b + l.o);
  L.red = (QS_LDS double*)(b + l.red);
  L.sh = (QS_LDS float*)(b + l.sh);
  L.ga = (QS_LDS float*)(b + l.ga);
  L.sred = (QS_LDS float*)(b + l.sred);
  L.qtmp = (QS_LDS int*)(b + l.qtmp);
  L.rinv = (QS_LDS double*)(b + l.rinv);
  L.kf = (QS_LDS float*)(b + l.kf);
  L.cand = (QS_LDS int*)(b + l.cand);
  L.ncand = (QS_LDS int*)(b + l.ncand);
  L.sv = (QS_LDS double*)(b + l.sv);
  L.xh = (QS_LDS uint32_t*)(b + l.xh);
  L.xl = (QS_LDS uint32_t*)(b + l.xl);
  L.xs = (QS_LDS float*)(b + l.xs);
  L.emap = (QS_LDS uint64_t*)(b + l.emap);
  L.xa = (QS_LDS int*)(b + l.xa);
  L.pfb = b + l.pfb;
  L.sdr = b + l.sdr;
  QS_LDS uint8_t* ab = b + l.abuf;
  L.ax = (QS_LDS float*)ab;
  L.lg = (QS_LDS double*)(ab + al16(T * H * 4));
  L.dah = (QS_LDS uint32_t*)ab;
  L.dal = (QS_LDS uint32_t*)(ab + al16(P * F));
  L.das = (QS_LDS float*)(ab + 2 * al16(P * F));
  L.daa = (QS_LDS int*)(ab + 2 * al16(P * F) + al16(P * F / 4));
  L.dash = (QS_LDS float*)(ab + 2 * al16(P * F) + 2 * al16(P * F / 4));
  return L;
}

// ------------------------------------------------------ staging plans ---
// Pure functions of the arguments, the workgroup index and (for routed
// work) the active-expert count: a workgroup computes the same offsets when
// it issues a copy and when it consumes it.  The host checks that the
// buffer holds at least one piece of each kind next to its neighbours.
template <class A>
__device__ __forceinline__ int my_count(const A& a, int n) {   // items b + j*G below n
  const int b = blockIdx.x, G = a.G;
  return b < n ? (n - 1 - b) / G + 1 : 0;
}

// router: expert group eg = b + i*G of r_et rows, staged at [0, router_bytes)
template <class A>
__device__ __forceinline__ int router_groups(const A& a) { return (a.E + a.r_et - 1) / a.r_et; }
template <class A>
__device__ __forceinline__ uint32_t router_bytes(const A& a) { return (uint32_t)a.r_et * a.H * 4; }

// Shared gate/up rows per item (both kernels).
template <bool SMALL, class A>
__device__ __forceinline__ int sh_rows(const A& a) { return kSharedItemRows; }
// The small-batch kernel's shared expert streams through registers instead
// of LDS staging in its fixed-shape instantiations of hidden sizes above
// 2048 (the only ones above 2048): there the rows are too many to prefetch a
// layer ahead, and staging them would crowd the routed down rows out of LDS.
// Below, LDS staging a layer ahead by the copy waves measured faster.
template <class A>
__device__ __forceinline__ bool sh_regs(const A& a) { return A::kFixedShape && a.H > 2048; }
// the same at compile time
template <class A>
constexpr bool wide_fixed() {
  if constexpr (A::kFixedShape) return A::H > 2048;
  else return false;
}
template <bool SMALL, class A>
__device__ __forceinline__ int n_shared_items(const A& a) { return a.Fs / sh_rows<SMALL>(a); }
template <bool SMALL, class A>
__device__ __forceinline__ uint32_t shared_item_bytes(const A& a) {
  return (uint32_t)sh_rows<SMALL>(a) * 2 * srow_bytes(a.H, a.sq8 != 0);
}
template <class A>
__device__ __forceinline__ uint32_t gu_tile_bytes(const A& a) {
  return 2u * (uint32_t)kGateTile * (a.H / kBlockW) * blk_bytes(a.gfmt);
}
template <class A>
__device__ __forceinline__ uint32_t sd_bytes(const A& a) { return (uint32_t)kDownRows * srow_bytes(a.Fs, a.sq8 != 0); }
template <class A>
__device__ __forceinline__ uint32_t dn_expert_bytes(const A& a) {
  return (uint32_t)kDownRows * (a.F / kBlockW) * blk_bytes(a.dfmt);
}

// SMALL: region A = [0, pfa) holds the router rows and shared items (phase
// R), then the routed gate/up tiles (K and GU); region B = [pfa, pfb) holds
// the down rows (copied during GU, used in D).  Otherwise the whole buffer
// is reused phase by phase.
// shared items: SMALL after the router rows; otherwise at 0 with room for one tile
template <bool SMALL, class A>
__device__ __forceinline__ uint32_t shared_off(const A& a) {
  return SMALL ? al16(router_bytes(a)) : 0;
}
template <bool SMALL, class A>
__device__ __forceinline__ int shared_pf_count(const A& a) {
  const uint32_t off = shared_off<SMALL>(a), end = SMALL ? a.pfa : a.pfb - gu_tile_bytes(a);
  const int fit = end > off ? (int)((end - off) / shared_item_bytes<SMALL>(a)) : 0;
  const int mine = my_count(a, n_shared_items<SMALL>(a));
  return mine < fit ? mine : fit;
}

// down: [shared rows | a chunk of experts' rows] from down_base; the first
// chunk of the first tile is copied ahead (SMALL: during GU, otherwise during
// the barrier before D)
template <bool SMALL, class A>
__device__ __forceinline__ uint32_t down_base(const A& a) { return SMALL ? a.pfa : 0; }
// SMALL: bytes of the x limbs, which follow the staging buffer
template <class A>
__device__ __forceinline__ uint32_t xlimb_bytes(const A& a) {
  return 2 * al16((uint32_t)a.T * a.H) + 2 * al16((uint32_t)a.T * a.H / 4);
}
template <bool SMALL, class A>
__device__ __forceinline__ int down_chunk(const A& a) {
  // SMALL: region B and the x limbs (free once the gate/up tiles are done);
  // the shared down rows have their own slot.  Otherwise after the shared rows.
  const uint32_t fixed = SMALL ? down_base<SMALL>(a) : al16(sd_bytes(a));
  const uint32_t end = SMALL ? a.pfb + xlimb_bytes(a) : a.pfb;
  return end > fixed ? (int)((end - fixed) / dn_expert_bytes(a)) : 0;
}
template <bool SMALL, class A>
__device__ __forceinline__ int down_pf_count(const A& a, int na) {
  if ((int)blockIdx.x * kDownRows >= a.H) return 0;
  const int fit = down_chunk<SMALL>(a);
  return na < fit ? na : fit;
}

// ------------------------------------------------------ copy issuers ---
template <class A>
__device__ __forceinline__ void copy_router_rows(const A& a, const LayerPtrs& Lp, PersistLds& L, int eg,
                                                 int w, int nw) {
  const int e0 = eg * a.r_et;
  const int ne = a.E - e0 < a.r_et ? a.E - e0 : a.r_et;
  dma_to_lds<0>(Lp.router + (size_t)e0 * a.H, L.pfb, (uint32_t)ne * a.H * 4, w, nw);
}

template <bool SMALL, class A>
__device__ __forceinline__ void copy_shared_item(const A& a, const LayerPtrs& Lp, QS_LDS uint8_t* dst,
                                                 int item, int w, int nw) {
  const uint32_t row = srow_bytes(a.H, a.sq8 != 0);
  const int rows = sh_rows<SMALL>(a);
  for (int r = 0; r < rows; ++r) {
    const int f = item * rows + r;
    dma_to_lds<0>(Lp.sg + (size_t)f * row, dst + (2 * r) * row, row, w, nw);
    dma_to_lds<0>(Lp.su + (size_t)f * row, dst + (2 * r + 1) * row, row, w, nw);
  }
}

// Routed gate/up tile (expert e, rows f0..f0+15) in LDS as
// [gate codes | up codes | gate scales | up scales | gate d | up d].
struct TileLds {
  uint32_t qb, sb, db, s, d;
};
template <class A>
__device__ __forceinline__ TileLds tile_lds(const A& a) {
  TileLds t;
  const uint32_t nbh = a.H / kBlockW;
  const BlkGeom g = blk_geom(a.gfmt);
  t.qb = (uint32_t)kGateTile * nbh * g.q;
  t.sb = (uint32_t)kGateTile * nbh * g.s;
  t.db = (uint32_t)kGateTile * nbh * g.d;
  t.s = 2 * t.qb;
  t.d = 2 * t.qb + 2 * t.sb;
  return t;
}

template <class A>
__device__ __forceinline__ void copy_tile(const A& a, const LayerPtrs& Lp, QS_LDS uint8_t* dst, int e,
                                          int f0, int w, int nw) {
  const uint32_t nbh = a.H / kBlockW;
  const size_t nblk = (size_t)a.F * nbh;
  const MatPlanes pl = fmt_planes(a.gfmt, nblk);
  const BlkGeom g = blk_geom(a.gfmt);
  const TileLds tl = tile_lds(a);
  const size_t b0 = (size_t)f0 * nbh;
  for (int m = 0; m < 2; ++m) {
    const uint8_t* src = ex_mat(a, Lp, m, e);
    dma_to_lds<0>(src + pl.q + b0 * g.q, dst + m * tl.qb, tl.qb, w, nw);
    dma_to_lds<0>(src + pl.s + b0 * g.s, dst + tl.s + m * tl.sb, tl.sb, w, nw);
    dma_to_lds<0>(src + pl.d + b0 * g.d, dst + tl.d + m * tl.db, tl.db, w, nw);
  }
}


// Routed down rows r0..r0+7 of expert e as [codes | scales | d,dmin] (per
// block 64 | 16 | 4 bytes for Q2_K, 128 | 16 | 4 for the Q4_K-style planes).
// rec: a paged expert's record (its down matrix at 2 gu_stride), or null.
template <class A>
__device__ __forceinline__ void copy_down_rows(const A& a, const LayerPtrs& Lp, QS_LDS uint8_t* dst,
                                               int e, int r0, int w, int nw, const uint8_t* rec = nullptr) {
  const uint32_t nb = a.F / kBlockW;
  const MatPlanes pl = fmt_planes(a.dfmt, (size_t)a.H * nb);
  const BlkGeom g = blk_geom(a.dfmt);
  const uint8_t* base = rec ? rec + 2 * a.gu_stride : ex_mat(a, Lp, 2, e);
  const size_t b0 = (size_t)r0 * nb;
  dma_to_lds<0>(base + pl.q + b0 * g.q, dst, kDownRows * nb * g.q, w, nw);
  dma_to_lds<0>(base + pl.s + b0 * g.s, dst + kDownRows * nb * g.q, kDownRows * nb * g.s, w, nw);
  dma_to_lds<0>(base + pl.d + b0 * g.d, dst + kDownRows * nb * (g.q + g.s), kDownRows * nb * g.d, w, nw);
}

template <class A>
__device__ __forceinline__ void copy_sd_rows(const A& a, const LayerPtrs& Lp, QS_LDS uint8_t* dst, int r0,
                                             int w, int nw) {
  if (a.Fs) dma_to_lds<0>(Lp.sd + (size_t)r0 * srow_bytes(a.Fs, a.sq8 != 0), dst, sd_bytes(a), w, nw);
}

// prefetches issued during barriers
template <bool SMALL, class A>
__device__ __forceinline__ void pf_router_and_shared(const A& a, const LayerPtrs& Lp, PersistLds& L,
                                                     int w, int nw) {
  if ((int)blockIdx.x < router_groups(a)) copy_router_rows(a, Lp, L, blockIdx.x, w, nw);
  if constexpr (SMALL && A::kPaged) {
    if (Lp.emap) dma_to_lds<0>(Lp.emap, L.emap, (uint32_t)a.E * 8, w, nw);
  }
  if (SMALL && !sh_regs(a)) {
    const int n = shared_pf_count<true>(a);
    for (int j = 0; j < n; ++j)
      copy_shared_item<true>(a, Lp, L.pfb + shared_off<true>(a) + (uint32_t)j * shared_item_bytes<true>(a),
                       (int)blockIdx.x + j * a.G, w, nw);
  }
}

template <class A>
__device__ __forceinline__ void pf_shared_items(const A& a, const LayerPtrs& Lp, PersistLds& L, int w,
                                                int nw) {
  const int n = shared_pf_count<false>(a);
  for (int j = 0; j < n; ++j)
    copy_shared_item<false>(a, Lp, L.pfb + (uint32_t)j * shared_item_bytes<false>(a), (int)blockIdx.x + j * a.G, w,
                     nw);
}

// A wave that has issued a copy into LDS waits at its next LDS access until
// the copied data has landed, so the expert ids a burst of copies needs are
// read first: L.act[u0 + lane] (0 past n) in every lane.
__device__ __forceinline__ int act_lanes(const PersistLds& L, int u0, int n) {
  const int i = u0 + (int)(qs_tid() & 63);
  return i < n ? L.act[i] : 0;
}

// SMALL: the experts' rows of the workgroup's second down tile are copied
// ahead as well, after the first tile's, when both tiles' rows fit the region
// at once and the shared down rows need no staging beside them (they stream
// through registers, or there are none).
template <class A>
__device__ __forceinline__ bool down_pf_second(const A& a, int na) {
  return a.H / kDownRows > a.G && (int)blockIdx.x + a.G < a.H / kDownRows && 2 * na <= down_chunk<true>(a) &&
         (sh_regs(a) || !a.Fs);
}

template <bool SMALL, class A>
__device__ __forceinline__ void pf_down(const A& a, const LayerPtrs& Lp, PersistLds& L, int w, int nw) {
  const int r0 = blockIdx.x * kDownRows;
  if (r0 >= a.H) return;
  QS_LDS uint8_t* base = L.pfb + down_base<SMALL>(a);
  const int na = *L.nact;
  const int n = down_pf_count<SMALL>(a, na);
  const bool two = SMALL && down_pf_second(a, na);
  if (!SMALL) copy_sd_rows(a, Lp, base, r0, w, nw);   // SMALL: in L.sdr, copied a layer ahead
  for (int u0 = 0; u0 < n; u0 += 64) {
    const int el = act_lanes(L, u0, n);
    const int m = n - u0 < 64 ? n - u0 : 64;
    // paged layer: the experts' records, gathered into lanes from the LDS
    // map before any copy is issued (a wave with copies in flight waits for
    // them at its next LDS access)
    uint64_t rl = 0;
    if constexpr (SMALL && A::kPaged) {
      if (Lp.emap && (int)(qs_tid() & 63) < m) rl = L.emap[el];
    }
    for (int i = 0; i < m; ++i) {
      const uint8_t* rec = nullptr;
      if constexpr (SMALL && A::kPaged) {
        if (Lp.emap)
          rec = (const uint8_t*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(rl >> 32), i) << 32) |
                                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)rl, i));
      }
      const int e = __builtin_amdgcn_readlane(el, i);
      QS_LDS uint8_t* dst = base + (SMALL ? 0u : al16(sd_bytes(a))) + (uint32_t)(u0 + i) * dn_expert_bytes(a);
      copy_down_rows(a, Lp, dst, e, r0, w, nw, rec);
      if (two) copy_down_rows(a, Lp, dst + (uint32_t)na * dn_expert_bytes(a), e, r0 + a.G * kDownRows, w, nw, rec);
    }
  }
}

// ------------------------------------------------------------ phase R ---
__device__ __forceinline__ double sumsq_part(float4 v, double s) {
  s = fma((double)v.x, (double)v.x, s);
  s = fma((double)v.y, (double)v.y, s);
  s = fma((double)v.z, (double)v.z, s);
  s = fma((double)v.w, (double)v.w, s);
  return s;
}

__device__ __forceinline__ double rms_inv_of(double q, int H) { return 1.0 / sqrt(q / (double)H + kRmsEps); }

template <bool SMALL, class A>
__device__ __forceinline__ float4 x_f4(const A& a, const PersistLds& L, const float* x, int t, int h) {
  if (SMALL) return lds_f4(L.ax + t * a.H + h);
  return cldf4(x + (size_t)t * a.H + h);
}

// Per-token RMS scales of tokens t0..t0+n-1 into LDS: wave w covers
// [w*H/8, (w+1)*H/8) with lane stride 4, fp64 FMAs in order, a butterfly,
// then the waves in order -- the same order phase_router uses, so the scale
// is the same for every batch size.
template <bool SMALL, class A>
__device__ __forceinline__ void token_rinv(const A& a, PersistLds& L, const float* x, int t0, int n) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, nw = kPersistThreads >> 6;
  const int hw = a.H / nw;
  for (int j = 0; j < n; ++j) {
    double s = 0.0;
#pragma unroll 1
    for (int h = wave * hw + 4 * lane; h < (wave + 1) * hw; h += 256) s = sumsq_part(x_f4<SMALL>(a, L, x, t0 + j, h), s);
    s = bfly_sum_f64<6>(s);
    if (lane == 0) L.red[wave * 4 + j] = s;
  }
  __syncthreads();
  if (qs_tid() < n) {
    double q = 0.0;
    for (int w = 0; w < nw; ++w) q += L.red[w * 4 + qs_tid()];
    L.rinv[t0 + qs_tid()] = a.prenorm ? rms_inv_of(q, a.H) : 1.0;
  }
  __syncthreads();
}

// The router bias of the logit this thread finishes for expert group eg
// (0 on the other threads).
template <class A>
__device__ __forceinline__ double router_bias(const A& a, const LayerPtrs& Lp, int eg) {
  const int e = eg * a.r_et + qs_tid() / a.r_tt;
  return qs_tid() < a.r_et * a.r_tt && eg < router_groups(a) && e < a.E ? (double)Lp.bias[e] : 0.0;
}

// Router: this workgroup's expert groups (rows in LDS) against every token
// group.  Each workgroup also sums x^2 of the tokens it routes (same order
// as token_rinv).  SMALL: the sums give L.rinv, read after the next block
// barrier (workgroups without a router group call token_rinv instead).
// Otherwise: the owner of expert group 0 publishes the RMS scales.
template <bool SMALL, class A>
__device__ __forceinline__ void phase_router(const A& a, const LayerPtrs& Lp, const float* x,
                                             PersistLds& L, uint32_t flag = 0) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, nw = kPersistThreads >> 6;
  const int ET = a.r_et, TT = a.r_tt;
  const int ntt = (a.T + TT - 1) / TT;
  const int hw = a.H / nw;
  const int V = ET * TT + TT;
  const bool want_ss = a.prenorm;
  const QS_LDS float* wr = (const QS_LDS float*)L.pfb;
  if (!SMALL) wait_all_and_sync();   // router rows prefetched during the last barrier
  int i = 0;
  for (int eg = blockIdx.x; eg < router_groups(a); eg += a.G, ++i) {
    if (i > 0) stage_now([&](int w, int n) { copy_router_rows(a, Lp, L, eg, w, n); });
    const int e0 = eg * ET;
    // the bias of the logit this thread finishes, requested before the sums
    const double bias = router_bias(a, Lp, eg);
#pragma unroll 1
    for (int tg = 0; tg < ntt; ++tg) {
      const int t0 = tg * TT, nt = a.T - t0 < TT ? a.T - t0 : TT;
      double acc[4][4], ss[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        ss[ii] = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[ii][j] = 0.0;
      }
#pragma unroll 1
      for (int h = wave * hw + 4 * lane; h < (wave + 1) * hw; h += 256) {
        float4 xv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xv[j] = j < nt ? x_f4<SMALL>(a, L, x, t0 + j, h) : make_float4(0, 0, 0, 0);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          if (ii >= ET || e0 + ii >= a.E) continue;
          const float4 w = lds_f4(wr + ii * a.H + h);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[ii][j] = fma((double)w.x, (double)xv[j].x, acc[ii][j]);
            acc[ii][j] = fma((double)w.y, (double)xv[j].y, acc[ii][j]);
            acc[ii][j] = fma((double)w.z, (double)xv[j].z, acc[ii][j]);
            acc[ii][j] = fma((double)w.w, (double)xv[j].w, acc[ii][j]);
          }
        }
        if (want_ss) {
#pragma unroll
          for (int j = 0; j < 4; ++j) ss[j] = sumsq_part(xv[j], ss[j]);
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (ii < ET && j < TT) {
            const double s = bfly_sum_f64<6>(acc[ii][j]);
            if (lane == 0) L.red[32 + wave * V + ii * TT + j] = s;
          }
      if (want_ss) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j < TT) {
            const double s = bfly_sum_f64<6>(ss[j]);
            if (lane == 0) L.red[32 + wave * V + ET * TT + j] = s;
          }
      }
      QS_STAMP3(20);
      __syncthreads();
      QS_STAMP3(21);
      if (qs_tid() < ET * TT) {
        const int ii = qs_tid() / TT, j = qs_tid() % TT;
        const int e = e0 + ii, t = t0 + j;
        if (e < a.E && j < nt) {
          // every wave's partials requested at once, then summed in wave
          // order (the q slots hold no sums without the pre-norm; unused)
          double sp[kPersistThreads / 64], qp[kPersistThreads / 64];
#pragma unroll
          for (int w = 0; w < kPersistThreads / 64; ++w) {
            sp[w] = L.red[32 + w * V + ii * TT + j];
            qp[w] = L.red[32 + w * V + ET * TT + j];
          }
          __builtin_amdgcn_sched_barrier(0);
          double s = 0.0, q = 0.0;
#pragma unroll
          for (int w = 0; w < kPersistThreads / 64; ++w) {
            s += sp[w];
            q += qp[w];
          }
          const double r = a.prenorm ? rms_inv_of(q, a.H) : 1.0;
          const double lv = a.prenorm ? fma(s, r, bias) : s + bias;
          if (SMALL && ii == 0) L.rinv[t] = r;
          if (SMALL) {
            const uint64_t bits = (uint64_t)__double_as_longlong(lv);
            uint64_t* wp = a.ll_lg + 2 * ((size_t)t * a.E + e);
            ll_store(wp, (uint32_t)bits, flag);
            ll_store(wp + 1, (uint32_t)(bits >> 32), flag);
          } else {
            cstd(&a.logits[(size_t)t * a.E + e], lv);
          }
          if (!SMALL && e == 0) cstd(&a.rinv[t], r);
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------- shared gate/up item ---
// Weights [h, h+8) of a staged shared-expert row of K weights (h a multiple
// of 8).  8-bit blocks: w = d*q, exact in fp32 (an 11-bit significand times
// a 7-bit magnitude); bf16 widens exactly.
template <class A>
__device__ __forceinline__ void shared_w8(const A& a, lds_cptr row, int K, int h, float w[8]) {
  if (a.sq8) {
    const uint32_t q0 = ld4(row + h), q1 = ld4(row + h + 4);
    const float d = half_to_f32(ld2(row + K + (h >> 5) * 2));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[c] = d * (float)(int8_t)(q0 >> (8 * c));
      w[4 + c] = d * (float)(int8_t)(q1 >> (8 * c));
    }
  } else {
    const uint4 v = ld16(row + h * 2);
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[2 * c] = bf16_to_f32(vw[c] & 0xFFFFu);
      w[2 * c + 1] = bf16_to_f32(vw[c] >> 16);
    }
  }
}

// Rows of the item from LDS ([row][gate, up] shared rows), 8/rows waves
// per row, each over a slice of H; fp32 FMA.
// Word offsets of the SwiGLU outputs in the flagged buffer, in the order
// the down phase copies them into LDS: [ah P*F/4 | al | as P*F/16 | aa | ash T*Fs].
template <class A>
__device__ __forceinline__ size_t ll_al(const A& a) { return (size_t)a.T * a.k * (a.F / 4); }
template <class A>
__device__ __forceinline__ size_t ll_as(const A& a) { return 2 * (size_t)a.T * a.k * (a.F / 4); }
template <class A>
__device__ __forceinline__ size_t ll_aa(const A& a) { return ll_as(a) + (size_t)a.T * a.k * (a.F / kSubW); }
template <class A>
__device__ __forceinline__ size_t ll_ash(const A& a) { return ll_as(a) + 2 * (size_t)a.T * a.k * (a.F / kSubW); }
template <class A>
__device__ __forceinline__ int ll_a_words(const A& a) { return (int)(ll_ash(a) + (size_t)a.T * a.Fs); }
// SMALL flow: waves [copy_w0, 8) issue the copies that overlap a flagged
// read, waves [0, copy_w0) poll (when the words fit 32 per thread of them).
// (Measured choices; T is a compile-time constant in the fixed-shape
// kernels.)
template <class A>
__device__ __forceinline__ int copy_w0(const A& a) { return a.T == 1 ? 7 : 6; }
template <class A>
__device__ __forceinline__ int ll_waves(const A& a, int words) {
  return words <= 32 * 64 * copy_w0(a) ? copy_w0(a) : kPersistThreads / 64;
}
template <class A>
__device__ __forceinline__ int ll_a_waves(const A& a) { return ll_waves(a, ll_a_words(a)); }

template <bool SMALL, class A>
__device__ __forceinline__ void shared_gu_item(const A& a, lds_cptr wbase, const float* x, int item,
                                               PersistLds& L, uint32_t flag = 0) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63;
  const int rows = sh_rows<SMALL>(a), wpr = (kPersistThreads / 64) / rows;   // waves per row
  const int rw = wave / wpr, qtr = wave % wpr;
  const int hq = a.H / wpr;
  const int T = a.T;
  const uint32_t row = srow_bytes(a.H, a.sq8 != 0);
  lds_cptr gsrc = wbase + (2 * rw) * row;
  lds_cptr usrc = wbase + (2 * rw + 1) * row;
#pragma unroll 1
  for (int t = 0; t < T; ++t) {
    float g = 0.f, u = 0.f;
#pragma unroll 1
    for (int h = qtr * hq + 8 * lane; h < (qtr + 1) * hq; h += 512) {
      float gw[8], uw[8];
      shared_w8(a, gsrc, a.H, h, gw);
      shared_w8(a, usrc, a.H, h, uw);
      const float4 x0 = x_f4<SMALL>(a, L, x, t, h), x1 = x_f4<SMALL>(a, L, x, t, h + 4);
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        g = fmaf(gw[c], xv[c], g);
        u = fmaf(uw[c], xv[c], u);
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
  // combine the per-wave partials of a row in a fixed order
  for (int q = qs_tid(); q < rows * T; q += kPersistThreads) {
    const int r = q / T, t = q % T;
    const int ff = item * rows + r;
    float g = 0.f, u = 0.f;
    for (int w4 = 0; w4 < wpr; ++w4) {
      g += L.sred[((r * wpr + w4) * T + t) * 2];
      u += L.sred[((r * wpr + w4) * T + t) * 2 + 1];
    }
    const float rs = SMALL ? (float)L.rinv[t] : (float)cldd(&a.rinv[t]);
    const float v = silu_mul(g * rs, u * rs);
    if (SMALL) ll_store(a.ll_a + ll_ash(a) + (size_t)t * a.Fs + ff, __float_as_uint(v), flag);
    else cstf(&a.ash[(size_t)t * a.Fs + ff], v);
  }
  __syncthreads();
}

template <bool SMALL, class A>
__device__ __forceinline__ void shared_items(const A& a, const LayerPtrs& Lp, const float* x,
                                             PersistLds& L, uint32_t flag = 0) {
  const int npf = shared_pf_count<SMALL>(a);
  const uint32_t off = shared_off<SMALL>(a), item_b = shared_item_bytes<SMALL>(a);
  int j = 0;
  for (int it = blockIdx.x; it < n_shared_items<SMALL>(a); it += a.G, ++j) {
    uint32_t slot = off + (uint32_t)j * item_b;
    if (j >= npf) {      // not prefetched: copy into the first slot (already consumed)
      slot = off;
      stage_now([&](int w, int n) { copy_shared_item<SMALL>(a, Lp, L.pfb + off, it, w, n); });
    }
    shared_gu_item<SMALL>(a, L.pfb + slot, x, it, L, flag);
  }
}

// ------------------------------ shared expert through registers (SMALL) ---
// With sh_regs the small-batch kernel streams the shared expert's rows from
// HBM straight into registers (no LDS staging).  A 16-byte chunk holds 8
// weights: bf16, or (8-bit rows) 8 code bytes with the block's scale bits
// in .z.
// Chunks per thread in flight: (gate, up) pairs and down chunks.
template <class A>
constexpr int sh_pairs() { return kShPairsLds; }
template <class A>
constexpr int sh_dn_regs() { return kShDnRegs; }

template <class A>
__device__ __forceinline__ uint4 sh_chunk_load(const A& a, const uint8_t* row, int K, int h) {
  if (a.sq8) {
    const uint2 q = *(const uint2*)(row + h);
    return make_uint4(q.x, q.y, *(const uint16_t*)(row + K + (h >> 5) * 2), 0u);
  }
  return *(const uint4*)(row + (size_t)h * 2);
}
// the 8 weights of a chunk (the values shared_w8 gives)
template <class A>
__device__ __forceinline__ void sh_chunk_decode(const A& a, uint4 v, float w[8]) {
  if (a.sq8) {
    const float d = half_to_f32(v.z);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[c] = d * (float)(int8_t)(v.x >> (8 * c));
      w[4 + c] = d * (float)(int8_t)(v.y >> (8 * c));
    }
  } else {
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w[2 * c] = bf16_to_f32(vw[c] & 0xFFFFu);
      w[2 * c + 1] = bf16_to_f32(vw[c] >> 16);
    }
  }
}

// Gate/up: item `it` is rows [2 it, 2 it + 2); waves 4r..4r+3 take row r,
// wave quarter q covers h in [q H/4, (q+1) H/4) with lane chunks
// h = q H/4 + 8 lane + 512 i -- the batched kernel's mapping, so both
// kernels produce bitwise the same SwiGLU values.  A round holds
// sh_pairs / ni items (ni chunks per lane); the workgroup's items are
// it = b + j G.  (A round never exceeds the items a workgroup has, so the
// fixed-shape kernels keep only the registers they use.)
template <class A>
__device__ __forceinline__ int sh_gu_chunks(const A& a) { return (a.H / 4 + 511) / 512; }
template <class A>
__device__ __forceinline__ int sh_gu_round(const A& a) {   // (at most the items any workgroup has)
  const int cap = sh_pairs<A>() / sh_gu_chunks(a), most = (n_shared_items<true>(a) + a.G - 1) / a.G;
  return cap < most ? cap : most;
}

template <class A, int NP>
__device__ __forceinline__ void sh_gu_issue(const A& a, const LayerPtrs& Lp, int j0, uint4 (&g)[NP],
                                            uint4 (&u)[NP]) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63;
  const int rw = wave >> 2, qtr = wave & 3, hq = a.H / 4, ni = sh_gu_chunks(a), nr = sh_gu_round(a);
  const uint32_t rb = srow_bytes(a.H, a.sq8 != 0);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int k = p / ni, i = p % ni;
    const int it = (int)blockIdx.x + (j0 + k) * a.G;
    const int h = qtr * hq + 8 * lane + 512 * i;
    if (k < nr && it < n_shared_items<true>(a) && h < (qtr + 1) * hq) {
      const size_t f = (size_t)it * kSharedItemRows + rw;
      g[p] = sh_chunk_load(a, Lp.sg + f * rb, a.H, h);
      u[p] = sh_chunk_load(a, Lp.su + f * rb, a.H, h);
    }
  }
}

// The SwiGLU outputs of the round's items (x, the RMS scales in LDS) as
// flagged words.
template <class A, int NP>
__device__ __forceinline__ void sh_gu_compute(const A& a, const uint4 (&g)[NP], const uint4 (&u)[NP], int j0,
                                              PersistLds& L, uint32_t flag) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, T = a.T;
  const int qtr = wave & 3, hq = a.H / 4, ni = sh_gu_chunks(a), nr = sh_gu_round(a);
  float ga[kSmallT], ua[kSmallT];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int k = p / ni, i = p % ni;
    const int it = (int)blockIdx.x + (j0 + k) * a.G;
    if (k >= nr || it >= n_shared_items<true>(a)) break;   // (wave-uniform)
    if (i == 0) {
#pragma unroll
      for (int t = 0; t < kSmallT; ++t) ga[t] = ua[t] = 0.f;
    }
    const int h = qtr * hq + 8 * lane + 512 * i;
    if (h < (qtr + 1) * hq) {
      float wg[8], wu[8];
      sh_chunk_decode(a, g[p], wg);
      sh_chunk_decode(a, u[p], wu);
#pragma unroll
      for (int t = 0; t < kSmallT; ++t) {
        if (t >= T) break;
        const float4 x0 = lds_f4(L.ax + t * a.H + h), x1 = lds_f4(L.ax + t * a.H + h + 4);
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          ga[t] = fmaf(wg[c], xv[c], ga[t]);
          ua[t] = fmaf(wu[c], xv[c], ua[t]);
        }
      }
    }
    if (i == ni - 1) {
#pragma unroll
      for (int t = 0; t < kSmallT; ++t) {
        if (t >= T) break;
        const float gs = bfly_sum<6>(ga[t]), us = bfly_sum<6>(ua[t]);
        if (lane == 0) {
          L.sred[((k * 8 + wave) * T + t) * 2] = gs;
          L.sred[((k * 8 + wave) * T + t) * 2 + 1] = us;
        }
      }
    }
  }
  __syncthreads();
  // the 4 wave partials of each row in a fixed order
  int nk = 0;
  for (int k = 0; k < nr; ++k)
    if ((int)blockIdx.x + (j0 + k) * a.G < n_shared_items<true>(a)) nk = k + 1;
  for (int q = qs_tid(); q < nk * kSharedItemRows * T; q += kPersistThreads) {
    const int k = q / (kSharedItemRows * T), r = (q / T) % kSharedItemRows, t = q % T;
    float gg = 0.f, uu = 0.f;
    for (int w4 = 0; w4 < 4; ++w4) {
      gg += L.sred[((k * 8 + r * 4 + w4) * T + t) * 2];
      uu += L.sred[((k * 8 + r * 4 + w4) * T + t) * 2 + 1];
    }
    const float rs = (float)L.rinv[t];
    const int ff = ((int)blockIdx.x + (j0 + k) * a.G) * kSharedItemRows + r;
    ll_store(a.ll_a + ll_ash(a) + (size_t)t * a.Fs + ff, __float_as_uint(silu_mul(gg * rs, uu * rs)), flag);
  }
  __syncthreads();
}

// Down: wave w takes row 8 tile + w of each of the workgroup's tiles
// (tile = b + j G), lane chunks f = 8 lane + 512 i -- the batched kernel's
// mapping.  A round holds sh_dn_regs / nd tiles (nd chunks per lane).
template <class A>
__device__ __forceinline__ int sh_dn_chunks(const A& a) { return (a.Fs + 511) / 512; }
template <class A>
__device__ __forceinline__ int sh_dn_round(const A& a) {   // (at most the tiles any workgroup has)
  const int cap = sh_dn_regs<A>() / sh_dn_chunks(a), most = (a.H / kDownRows + a.G - 1) / a.G;
  return cap < most ? cap : most;
}

template <class A, int ND>
__device__ __forceinline__ void sh_dn_issue(const A& a, const LayerPtrs& Lp, int j0, uint4 (&v)[ND]) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63;
  const int nd = sh_dn_chunks(a), nr = sh_dn_round(a), n_tiles = a.H / kDownRows;
  const uint32_t rb = srow_bytes(a.Fs, a.sq8 != 0);
#pragma unroll
  for (int p = 0; p < ND; ++p) {
    const int j = p / nd, i = p % nd;
    const int tile = (int)blockIdx.x + (j0 + j) * a.G, f = 8 * lane + 512 * i;
    if (j < nr && tile < n_tiles && f < a.Fs)
      v[p] = sh_chunk_load(a, Lp.sd + (size_t)(tile * kDownRows + wave) * rb, a.Fs, f);
  }
}

// The shared down outputs of round-local tile j (its rows' chunks in v) for
// every token, from the shared SwiGLU vector in LDS, into L.sh[t][row].
template <class A, int ND>
__device__ __forceinline__ void sh_dn_compute(const A& a, const uint4 (&v)[ND], int j, PersistLds& L) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, T = a.T, nd = sh_dn_chunks(a);
  float s[kSmallT];
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) s[t] = 0.f;
#pragma unroll
  for (int p = 0; p < ND; ++p) {
    const int i = p - j * nd, f = 8 * lane + 512 * i;
    if (i < 0 || i >= nd || f >= a.Fs) continue;
    float w[8];
    sh_chunk_decode(a, v[p], w);
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) {
      if (t >= T) break;
      const float4 a0 = lds_f4(L.dash + t * a.Fs + f), a1 = lds_f4(L.dash + t * a.Fs + f + 4);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int c = 0; c < 8; ++c) s[t] = fmaf(w[c], av[c], s[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < kSmallT; ++t) {
    if (t >= T) break;
    const float r = bfly_sum<6>(s[t]);
    if (lane == 0) L.sh[t * kDownRows + wave] = r;
  }
}

// ------------------------------------------------------------ phase K ---
// Top-k of token t by one wave: (logit desc, index asc), weights are the
// softmax over the k picks.  SMALL: logits from LDS, results into LDS (every
// workgroup); otherwise logits and results in global scratch (one wave per
// token).  Workgroup 0 / the token's wave also writes ids_out / w_out.
template <bool SMALL, class A>
__device__ __forceinline__ void topk_wave(const A& a, int t, int layer_i, PersistLds& L, bool write_out) {
  const int lane = qs_tid() & 63;
  const int E = a.E, k = a.k;
  double v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    double l = 0.0;
    if (e < E) l = SMALL ? L.lg[t * E + e] : cldd(&a.logits[(size_t)t * E + e]);
    v[i] = l != l ? -INFINITY : l;     // NaN ranks last; every pick stays valid and distinct
  }
  uint32_t taken = 0;
  double top0 = 0.0, selv = 0.0;
  int seli = 0;
#pragma unroll 1
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
  const float z = lane < k ? __expf((float)(selv - top0)) : 0.f;
  const float sum = bfly_sum<6>(z);
  if (lane < k) {
    const float w = __fdividef(z, sum);
    if (SMALL) {
      L.ids[t * k + lane] = seli;
      L.wl[t * k + lane] = w;
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

// SMALL top-k of every token by the whole workgroup, exact in (logit desc,
// index asc).  Rounding a logit to fp32 is monotone, so fp32 keys give a
// cheap superset of the top-k: take the largest key of each group of 8
// experts; the k-th largest of those group maxima, tau, is a lower bound of
// the key of every top-k expert (k groups hold an expert with a key >= tau,
// and a key that is larger means a larger logit).  The experts with key >=
// tau -- usually few more than k -- are then ranked exactly in fp64.  NaN
// logits rank as -inf.
__device__ __forceinline__ double nan_low(double v) { return v != v ? -INFINITY : v; }

// order-preserving int of a float (for an atomic minimum)
__device__ __forceinline__ int f32_ord(float f) {
  const int i = __float_as_int(f);
  return i >= 0 ? i : (int)(0x80000000u - (uint32_t)i) ;
}
__device__ __forceinline__ float f32_unord(int o) {
  return __int_as_float(o >= 0 ? o : (int)(0x80000000u - (uint32_t)o));
}

// Order-preserving integer image of an fp64 value, -0 taken as +0: a
// larger value has a larger image, equal values the same image.
__device__ __forceinline__ uint64_t f64_ord(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v + 0.0);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}
__device__ __forceinline__ double f64_unord(uint64_t o) {
  return __longlong_as_double((long long)((o >> 63) ? (o & ~(1ull << 63)) : ~o));
}

// The renormalised softmax over token t's picks (their logits in L.sv in
// rank order): the exponent of the fp64 difference to the top pick, in fp32.
// One wave.
template <class A>
__device__ __forceinline__ void topk_weights(const A& a, int layer_i, int t, PersistLds& L) {
  const int lane = qs_tid() & 63, k = a.k;
  const double top0 = L.sv[t * k];
  const float z = lane < k ? __expf((float)(L.sv[t * k + lane] - top0)) : 0.f;
  const float sum = bfly_sum<6>(z);
  if (lane < k) {
    const float w = __fdividef(z, sum);
    L.wl[t * k + lane] = w;
    if (blockIdx.x == 0) {
      const size_t o = (size_t)layer_i * a.T * k + t * k + lane;
      if (a.ids_out) a.ids_out[o] = L.ids[t * k + lane];
      if (a.w_out) a.w_out[o] = w;
    }
  }
}

// T = 1, in the wave that ranked the token: the grouping of its k distinct
// experts (what group_small gives for one token): position u of a pair is the
// rank of its expert among the k, each bucket holds one pair.
template <class A>
__device__ __forceinline__ void group_one_token(const A& a, PersistLds& L) {
  const int lane = qs_tid() & 63, k = a.k;
  const bool live = lane < k;
  const int e = live ? L.ids[lane] : 0x7FFFFFFF;
  int u = 0;
  for (int q = 0; q < k; ++q) u += __builtin_amdgcn_readlane(e, q) < e ? 1 : 0;
  if (live) {
    L.act[u] = e;
    L.aoff[u] = u;
    L.pairs[u] = lane;
    L.tok_order[u] = u;
    L.cw[u] = L.wl[lane];
  }
  if (lane == 0) {
    *L.nact = k;
    L.aoff[k] = k;
  }
}

// E <= 256: one wave per token, no block barrier before the last.  Lane l
// holds experts 4l..4l+3 and their fp32 selection keys (order-preserving
// integer images of the fp32 roundings of the fp64 logits).  A lane quad is
// a group of 16 experts: the k-th largest of the 16 group maxima, tau,
// bounds every top-k key from below (k groups hold a key >= tau, and a
// larger key means a larger logit).  The experts with key >= tau -- about
// k + 3 at these shapes -- are compacted in index order and each ranks
// itself against all of them: on their fp32 keys when no two candidates
// share one (a larger key means a larger logit), else on the
// order-preserving images of their fp64 logits, ties to the lower position,
// i.e. the lower expert id.  The picks
// are then moved to the lane of their rank (one crossbar permute) so that
// the weights are summed in rank order, as the batched kernel does.
template <class A>
__device__ __forceinline__ void topk_small_lds(const A& a, int layer_i, PersistLds& L);

__device__ __forceinline__ uint32_t f32_ordkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

template <class A>
__device__ __forceinline__ void topk_small(const A& a, int layer_i, PersistLds& L) {
  if (a.E > 256) {
    topk_small_lds(a, layer_i, L);
    return;
  }
  const int lane = qs_tid() & 63, wave = qs_tid() >> 6;
  const int E = a.E, k = a.k, T = a.T;
  if (wave < T) {
    const int t = wave, e0 = 4 * lane;
    QS_LDS double* lg = L.lg + t * E;
    double v[4];
    uint32_t ku[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = e0 + j < E ? nan_low(lg[e0 + j]) : -INFINITY;
      ku[j] = e0 + j < E ? f32_ordkey((float)v[j]) : 0u;   // padding below every real key
    }
    uint32_t g = max(max(ku[0], ku[1]), max(ku[2], ku[3]));
    g = max(g, partner_u32<0>(g));
    g = max(g, partner_u32<1>(g));
    // the 16 group maxima through LDS (the head of this token's candidate
    // row, rewritten only after these reads: a wave's LDS accesses are in order)
    QS_LDS int* cd = L.cand + t * E;
    QS_LDS uint32_t* gm = (QS_LDS uint32_t*)cd;
    if ((lane & 3) == 0 && e0 < E) gm[lane >> 2] = g;
    const int ng = (E + 15) >> 4;
    int c = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < ng) c += gm[j] > g ? 1 : 0;
    // fewer than k groups: tau = 0, every expert is a candidate
    uint32_t tau = c < k && e0 < E ? g : 0xFFFFFFFFu;
    tau = min(tau, partner_u32<2>(tau));
    tau = min(tau, partner_u32<3>(tau));
    tau = min(tau, partner_u32<4>(tau));
    tau = min(tau, partner_u32<5>(tau));
    if (ng < k) tau = 0;
    QS_STAMP3(22);
    bool p[4];
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = e0 + j < E && ku[j] >= tau;
      cnt += p[j];
    }
    const int incl = wave_incl_scan(cnt);
    const int m = __builtin_amdgcn_readlane(incl, 63);
    // candidates in index order: ids in cd, fp64 keys over this token's
    // logit row (read into registers above), fp32 keys in the router's
    // partials area (free until the next layer's router)
    QS_LDS uint64_t* ck = (QS_LDS uint64_t*)lg;
    static_assert(kSmallT * 80 * 4 <= 8 * 64 * 8, "fp32 candidate keys fit the router partials area");
    QS_LDS uint32_t* c32 = (QS_LDS uint32_t*)L.red + t * 80;
    int pos = incl - cnt;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (p[j]) {
        cd[pos] = e0 + j;
        ck[pos] = f64_ord(v[j]);
        c32[pos] = ku[j];
        ++pos;
      }
    if (m <= 64) {
      const bool live = lane < m;
      if (lane < 16) c32[m + lane] = 0u;   // padding: below every real key
      const uint64_t K = live ? ck[lane] : 0;
      const uint32_t K32 = live ? c32[lane] : 0u;
      const int e = live ? cd[lane] : 0;
      // rank on the fp32 keys: a larger key means a larger logit, so when no
      // two candidates share an fp32 key the rank is the count of larger keys
      int r = 0, eq = 0;
      for (int j0 = 0; j0 < m; j0 += 16) {
        uint32_t w[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v4 = lds_u4(c32 + j0 + 4 * q);
          w[4 * q] = v4.x;
          w[4 * q + 1] = v4.y;
          w[4 * q + 2] = v4.z;
          w[4 * q + 3] = v4.w;
        }
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          r += w[jj] > K32 ? 1 : 0;
          eq += w[jj] == K32 ? 1 : 0;
        }
      }
      if (__builtin_amdgcn_ballot_w64(live && eq > 1)) {
        // equal fp32 keys: rank on the order-preserving images of the fp64
        // logits, ties to the lower position (the lower expert id)
        r = 0;
        for (int j0 = 0; j0 < m; j0 += 16) {
          uint64_t w[16];
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) w[jj] = j0 + jj < m ? ck[j0 + jj] : 0;
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int j = j0 + jj;
            r += (j < m && (w[jj] > K || (w[jj] == K && j < lane))) ? 1 : 0;
          }
        }
      }
      const bool sel = live && r < k;
      QS_STAMP3(23);
      // move each pick to the lane of its rank: expert, logit image, and its
      // position among the picks in ascending expert order
      const int u = wave_incl_scan(sel ? 1 : 0) - 1;
      const int dst = (sel ? r : 63) * 4;
      const int er = __builtin_amdgcn_ds_permute(dst, e);
      const int ur = __builtin_amdgcn_ds_permute(dst, u);
      const int khi = __builtin_amdgcn_ds_permute(dst, (int)(K >> 32));
      const int klo = __builtin_amdgcn_ds_permute(dst, (int)(uint32_t)K);
      const double vr = f64_unord(((uint64_t)(uint32_t)khi << 32) | (uint32_t)klo);
      const uint64_t k0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(khi, 0) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane(klo, 0);
      const float z = lane < k ? __expf((float)(vr - f64_unord(k0))) : 0.f;
      const float sum = bfly_sum<6>(z);
      if (lane < k) {
        const float w = __fdividef(z, sum);
        L.ids[t * k + lane] = er;
        L.wl[t * k + lane] = w;
        if (blockIdx.x == 0) {
          const size_t o = (size_t)layer_i * a.T * k + t * k + lane;
          if (a.ids_out) a.ids_out[o] = er;
          if (a.w_out) a.w_out[o] = w;
        }
        if (T == 1) {       // the grouping of one token's k distinct experts
          L.act[ur] = er;
          L.aoff[ur] = ur;
          L.pairs[ur] = lane;
          L.tok_order[ur] = ur;
          L.cw[ur] = w;
        }
      }
      if (T == 1 && lane == 0) {
        *L.nact = k;
        L.aoff[k] = k;
      }
    } else {
      // many exact ties at the threshold: rank in chunks
      for (int i0 = 0; i0 < m; i0 += 64) {
        const int i = i0 + lane;
        const uint64_t K = i < m ? ck[i] : 0;
        int r = 0;
        for (int j = 0; j < m; ++j) {
          const uint64_t w = ck[j];
          r += (w > K || (w == K && j < i)) ? 1 : 0;
        }
        if (i < m && r < k) {
          L.ids[t * k + r] = cd[i];
          L.sv[t * k + r] = f64_unord(K);
        }
      }
      topk_weights(a, layer_i, t, L);
      if (T == 1) group_one_token(a, L);
    }
  }
  __syncthreads();
}

// Any E: keys and group maxima by (token, group) threads, the threshold with
// an LDS minimum, then one wave per token ranks its candidates.
template <class A>
__device__ __forceinline__ void topk_small_lds(const A& a, int layer_i, PersistLds& L) {
  const int tid = qs_tid(), nt = kPersistThreads, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k, T = a.T, S = kf_stride(E), NG = S / 8, G4 = (NG + 3) & ~3;
  QS_LDS float* gm = L.kf + T * S;                 // [T][G4] group maxima, -inf padded
  QS_LDS int* tau = (QS_LDS int*)(gm + T * G4);    // [T]
  // keys of one group of 8 experts and their maximum, one thread per (token, group)
  for (int i = tid; i < T * G4; i += nt) {
    const int t = i / G4, g = i % G4;
    float mx = -INFINITY;
    if (g < NG) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 8 * g + j;
        const float key = e < E ? (float)nan_low(L.lg[t * E + e]) : -INFINITY;
        L.kf[t * S + e] = key;
        mx = fmaxf(mx, key);
      }
    }
    gm[i] = mx;
  }
  // fewer than k groups: no bound, every expert is a candidate
  if (tid < T) tau[tid] = NG < k ? f32_ord(-INFINITY) : 0x7FFFFFFF;
  __syncthreads();
  // tau = the smallest group maximum with fewer than k larger ones
  if (NG >= k) {
    for (int i = tid; i < T * G4; i += nt) {
      const int t = i / G4;
      if (i % G4 >= NG) continue;
      const QS_LDS float* row = gm + t * G4;
      const float g = gm[i];
      int c = 0;
#pragma unroll 4
      for (int j = 0; j < G4; j += 4) {
        const float4 q = lds_f4(row + j);
        c += (q.x > g) + (q.y > g) + (q.z > g) + (q.w > g);
      }
      if (c < k) __hip_atomic_fetch_min(&tau[t], f32_ord(g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();
  if (wave < T) {
    // one wave per token from here on (its own LDS rows, no block barrier):
    // the experts with key >= tau, compacted in index order by ballots
    const int t = wave;
    const float thr = f32_unord(tau[t]);
    QS_LDS int* cd = L.cand + t * E;
    const uint64_t below = (1ull << lane) - 1ull;
    int m = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const bool p = e < E && L.kf[t * S + e] >= thr;
      const uint64_t bm = __ballot(p);
      if (p) cd[m + __popcll(bm & below)] = e;
      m += __popcll(bm);
    }
    // exact rank among the candidates in (logit desc, index asc)
    for (int i0 = 0; i0 < m; i0 += 64) {
      const int i = i0 + lane;
      const int e = i < m ? cd[i] : 0;
      const double v = i < m ? nan_low(L.lg[t * E + e]) : 0.0;
      int r = 0;
      for (int j0 = 0; j0 < m; j0 += 64) {
        // candidates j0..j0+63 broadcast from the lanes that hold them
        const int ej = j0 + lane < m ? cd[j0 + lane] : 0;
        const double vj = j0 + lane < m ? nan_low(L.lg[t * E + ej]) : 0.0;
        const int nj = m - j0 < 64 ? m - j0 : 64;
        for (int j = 0; j < nj; ++j) {
          const int e2 = __builtin_amdgcn_readlane(ej, j);
          const double v2 = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(vj), j),
                                             __builtin_amdgcn_readlane(__double2loint(vj), j));
          r += (v2 > v || (v2 == v && e2 < e)) ? 1 : 0;
        }
      }
      if (i < m && r < k) {
        L.ids[t * k + r] = e;
        L.sv[t * k + r] = v;
      }
    }
    topk_weights(a, layer_i, t, L);
    if (T == 1) group_one_token(a, L);
  }
  __syncthreads();
}

// SMALL grouping by wave 0 (P = T*k <= 64 pairs, one per lane): sort the
// pairs by (expert, pair id) -- stable by token -- with a rank count, move
// each to the lane of its rank, mark the first pair of each expert (a scan
// of the marks numbers the active experts), and place each position in its
// token's ascending list with one ballot per token.
template <class A>
__device__ __forceinline__ void group_small(const A& a, PersistLds& L) {
  const int lane = qs_tid() & 63, k = a.k, P = a.T * k;
  if ((qs_tid() >> 6) == 0) {
    const bool live = lane < P;
    const int e = live ? valid_id(L.ids[lane], a.E) : 0x7FFF;
    const int key = e * 64 + lane;                 // unique; dead lanes sort last
    int rank = 0;
    for (int q = 0; q < P; ++q) rank += (int)(__builtin_amdgcn_readlane(key, q) < key);
    // lane r receives the key of the pair ranked r
    const int ks = __builtin_amdgcn_ds_permute(rank * 4, key);
    const int es = ks >> 6, ps = ks & 63;
    const int prev = __builtin_amdgcn_ds_bpermute((lane > 0 ? lane - 1 : 0) * 4, es);
    const int head = (lane < P && (lane == 0 || prev != es)) ? 1 : 0;
    const int u = wave_incl_scan(head) - 1;
    if (head) {
      L.act[u] = es;
      L.aoff[u] = lane;
    }
    const int na = __builtin_amdgcn_readlane(u, 63) + 1;
    if (lane == 0) {
      *L.nact = na;
      L.aoff[na] = P;
    }
    const int tok = ps / k;
    if (live) L.pairs[lane] = ps;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int tt = 0; tt < a.T; ++tt) {
      const uint64_t m = __ballot(live && tok == tt);
      if (live && tok == tt) {
        L.tok_order[tt * k + __popcll(m & below)] = lane;
        L.cw[tt * k + __popcll(m & below)] = L.wl[ps];
      }
    }
  }
  __syncthreads();
}

// Lane l holds the limb bytes of elements 4l..4l+3 of a 256-element block
// (byte j = element 4l+j).  Returns this lane's dword in the Q2_K consumer
// order: dword 4i+p of the block holds elements p, 4+p, 8+p, 12+p of 16-wide
// sub-block i, gathered from byte p of lanes 4i..4i+3.
__device__ __forceinline__ uint32_t q2k_order(uint32_t v) {
  const int p = qs_tid() & 3;
  uint32_t bv[4];
  bv[0] = v;
  bv[1] = partner_u32<0>(v);         // lane ^ 1
  bv[2] = partner_u32<1>(v);         // lane ^ 2
  bv[3] = partner_u32<1>(bv[1]);     // lane ^ 3
  uint32_t o = 0;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const int src = bb ^ p;          // bv[src] holds the word of lane 4i+bb
    const uint32_t w = src == 0 ? bv[0] : src == 1 ? bv[1] : src == 2 ? bv[2] : bv[3];
    o |= ((w >> (8 * p)) & 0xFFu) << (8 * bb);
  }
  return o;
}

// x block b (256 elements) of token t -> limbs, one wave.  SMALL: from and
// into LDS; otherwise global scratch.
template <bool SMALL, class A>
__device__ __forceinline__ void quant_x_wave(const A& a, const float* x, int t, int b, PersistLds& L) {
  const int lane = qs_tid() & 63;
  const float4 v = x_f4<SMALL>(a, L, x, t, b * kBlockW + 4 * lane);
  const float r = SMALL ? (float)L.rinv[t] : (float)cldd(&a.rinv[t]);
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
    ph = q2k_order(ph);
    pl = q2k_order(pl);
  }
  const int s = bfly_sum_i32<2>(q0 + q1 + q2 + q3);
  const float scale = ldexpf(r, e - kFixedBits);
  const size_t base = (size_t)t * (a.H / 4) + b * 64;
  const size_t si = (size_t)t * (a.H / kSubW) + b * 16 + (lane >> 2);
  if (SMALL) {
    L.xh[base + lane] = ph;
    L.xl[base + lane] = pl;
    if ((lane & 3) == 0) {
      L.xs[si] = scale;
      L.xa[si] = s;
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

// ------------------------------------------------------ grouping (LDS) ---
// Stable bucket sort of (token, slot) pairs by expert.
template <bool SMALL, class A>
__device__ __forceinline__ void build_groups(const A& a, PersistLds& L) {
  const int tid = qs_tid(), nt = kPersistThreads, E = a.E, k = a.k, T = a.T, P = T * k;
  const int wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < E; i += nt) L.cnt[i] = 0;
  for (int i = tid; i < E * 8; i += nt) L.mask[i] = 0;
  if (!SMALL) {
    for (int p = tid; p < P; p += nt) {
      L.ids[p] = cldi(&a.ids[p]);
      L.wl[p] = cldf(&a.wts[p]);
    }
  }
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int e = valid_id(L.ids[p], E), t = p / k;
    __hip_atomic_fetch_add(&L.cnt[e], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_or(&L.mask[e * 8 + (t >> 5)], 1u << (t & 31), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  // exclusive scans of counts and of the non-empty flags, 64 experts per wave
  // and pass, chunk totals combined through LDS (E <= 1024)
  QS_LDS int* wsum = (QS_LDS int*)L.red;   // [2 * 16] chunk totals
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
      if (cv > 0) {
        L.act[sf - 1] = e;
        L.aoff[sf - 1] = sc - cv;
      }
      if (e == E - 1) {
        L.off[E] = sc;
        L.aoff[sf] = sc;
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
template <bool SMALL, class A>
__device__ __forceinline__ void x_chunk(const A& a, const PersistLds& L, int t, int ch,
                                        uint32_t (&xh)[16], uint32_t (&xl)[16], float (&xs)[4],
                                        int (&xa)[4]) {
  const size_t xo = (size_t)t * (a.H / 4) + ch * 16;
  const size_t si = (size_t)t * (a.H / kSubW) + ch * 4;
  if (SMALL) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 h = lds_u4(L.xh + xo + 4 * i), l = lds_u4(L.xl + xo + 4 * i);
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

// Routed gate/up tiles of the small-batch kernel, streamed from HBM into
// registers.  The workgroup's tiles are items b, b+G, ... of the (active
// expert, 16-row tile) list.  In a tile, thread (slot, j) takes rows slot,
// slot + slots, ... and chunks j + cc*lpr of each row (the lane-per-chunk
// layout of every gate/up GEMV here), so each 64-weight chunk is decoded
// once and applied to every token of the bucket; a row's lanes then sum by
// butterfly.  The chunks of the first tiles (GuWin) are requested as soon as
// the grouping is known, and each computed tile's registers are refilled
// with the tile GuWin ahead, so no tile waits for its own round trip.
constexpr int kGuUnits = 2;    // (row, chunk) units per thread and tile: H <= 4096

struct GuChunk {
  uint4 gq, uq;                // 16 code bytes of the gate and up chunk
  uint32_t gs, us;             // codebook: the block's 4 scale bytes; Q2_K: the chunk's 4 scale/min bytes
  uint32_t gd, ud;             // codebook: d; Q2_K: d | dmin << 16
};
struct GuTile {
  GuChunk c[kGuUnits];
};
// Q4_K-style chunks: 32 code bytes per matrix (gq, gq2 / uq, uq2); gs, us
// the chunk's two scales (bytes 0, 1) and mins (bytes 2, 3); gd, ud d | dmin << 16.
struct GuChunk4 : GuChunk {
  uint4 gq2, uq2;
};
struct GuTile4 {
  GuChunk4 c[kGuUnits];
};
template <int FMT> struct GuTileOf { typedef GuTile T; };
template <> struct GuTileOf<kFmtQ4K> { typedef GuTile4 T; };

// Tiles in flight: four for the fixed shapes of several tokens up to hidden
// 2048 (one (row, chunk) unit per thread and tile; a workgroup's run there
// is up to four items), three otherwise (register budget, code size).
template <class A, bool FIXED = A::kFixedShape>
struct GuWin {
  static constexpr int v = 3;
};
template <class A>
struct GuWin<A, true> {
  static constexpr int v = A::H <= 2048 && A::T > 1 ? kGuWinMax : 3;
};

// The routed gate/up items (active expert u, 16-row tile), u-major, of
// workgroup b: items i0 + m * stride, m < n.  One token: every bucket holds
// one pair, so an even split (runs of N / G items when G divides the N
// items, else items b, b + G, ...).  More tokens: split by cost -- an item of a
// bucket of n tokens costs n + 1 (its chunks are decoded once, then dotted
// with each token's), and workgroup b takes the items whose cost midpoint
// falls in the b-th 1/G of the total, a contiguous run.  Every wave computes
// the same run (the host bounds 2 (G + 1) times the total cost below 2^31).
struct GuRange {
  int i0, stride, n;
};
template <class A>
__device__ __forceinline__ GuRange gu_range(const A& a, const PersistLds& L) {
  const int lane = qs_tid() & 63, na = *L.nact, tiles = a.F / kGateTile;
  if (a.T == 1) {   // (a run of N / G items when G divides them: adjacent tiles of one expert)
    const int N = na * tiles;
    if (N % a.G == 0) return {(int)blockIdx.x * (N / a.G), 1, N / a.G};
    return {(int)blockIdx.x, a.G, my_count(a, N)};
  }
  const uint32_t G = (uint32_t)a.G, C = (uint32_t)tiles * (uint32_t)(L.aoff[na] + na), b = blockIdx.x;
  // items of this lane's experts whose owner is below x: owner(u, t) < x
  // <=> G (2 S_u + (2 t + 1) c_u) < 2 x C, S_u the cost of the items before u
  int c0 = 0, c1 = 0;
  for (int u = lane; u < na; u += 64) {
    const uint32_t cu = (uint32_t)(L.aoff[u + 1] - L.aoff[u] + 1), S = (uint32_t)tiles * (uint32_t)(L.aoff[u] + u);
    const uint32_t base = G * (2 * S + cu), den = 2 * G * cu;
    auto below = [&](uint32_t x) {
      const uint32_t lim = 2 * x * C;
      if (lim <= base) return 0;
      const uint32_t t = (lim - base + den - 1) / den;
      return (int)(t < (uint32_t)tiles ? t : (uint32_t)tiles);
    };
    c0 += below(b);
    c1 += below(b + 1);
  }
  c0 = bfly_sum_i32<6>(c0);
  c1 = bfly_sum_i32<6>(c1);
  return {__builtin_amdgcn_readfirstlane(c0), 1, __builtin_amdgcn_readfirstlane(c1 - c0)};
}

template <int FMT, class A>
__device__ __forceinline__ void gu_tile_load(const A& a, const LayerPtrs& Lp, const PersistLds& L, int item,
                                             typename GuTileOf<FMT>::T& t) {
  const int tiles = a.F / kGateTile, nch = a.H / kChunkW, lpr = lanes_per_row(nch), cpl = nch / lpr;
  const int slots = kPersistThreads / lpr, slot = qs_tid() / lpr, j = qs_tid() % lpr;
  const int u = item / tiles, f0 = (item % tiles) * kGateTile;
  const int e = L.act[u];
  const uint32_t nbh = a.H / kBlockW;
  const size_t nblk = (size_t)a.F * nbh;
  const MatPlanes pl = fmt_planes(FMT, nblk);
  const uint8_t* g;
  const uint8_t* up;
  if constexpr (A::kPaged) {   // the record's address from the layer's map in LDS
    const uint8_t* rec = Lp.emap ? (const uint8_t*)(uintptr_t)L.emap[e] : nullptr;
    g = rec ? rec : ex_mat(a, Lp, 0, e);
    up = rec ? rec + a.gu_stride : ex_mat(a, Lp, 1, e);
  } else {
    g = ex_mat(a, Lp, 0, e);
    up = ex_mat(a, Lp, 1, e);
  }
#pragma unroll
  for (int i = 0; i < kGuUnits; ++i) {
    const int r = slot + (i / cpl) * slots, ch = j + (i % cpl) * lpr;
    if (r >= kGateTile || i >= ((kGateTile - 1 - slot) / slots + 1) * cpl) continue;
    const size_t blk = (size_t)(f0 + r) * nbh + ch / 4;
    const int c = ch & 3;
    auto& w = t.c[i];
    if constexpr (FMT == kFmtQ4K) {
      w.gq = *(const uint4*)(g + pl.q + blk * 128 + c * 32);
      w.gq2 = *(const uint4*)(g + pl.q + blk * 128 + c * 32 + 16);
      w.uq = *(const uint4*)(up + pl.q + blk * 128 + c * 32);
      w.uq2 = *(const uint4*)(up + pl.q + blk * 128 + c * 32 + 16);
      w.gs = (uint32_t)*(const uint16_t*)(g + pl.s + blk * 16 + 2 * c) |
             (uint32_t)*(const uint16_t*)(g + pl.s + blk * 16 + 8 + 2 * c) << 16;
      w.us = (uint32_t)*(const uint16_t*)(up + pl.s + blk * 16 + 2 * c) |
             (uint32_t)*(const uint16_t*)(up + pl.s + blk * 16 + 8 + 2 * c) << 16;
      w.gd = *(const uint32_t*)(g + pl.d + blk * 4);
      w.ud = *(const uint32_t*)(up + pl.d + blk * 4);
      continue;
    }
    w.gq = *(const uint4*)(g + pl.q + blk * 64 + c * 16);
    w.uq = *(const uint4*)(up + pl.q + blk * 64 + c * 16);
    if (FMT == 1) {
      w.gs = *(const uint32_t*)(g + pl.s + blk * 16 + c * 4);
      w.us = *(const uint32_t*)(up + pl.s + blk * 16 + c * 4);
      w.gd = *(const uint32_t*)(g + pl.d + blk * 4);
      w.ud = *(const uint32_t*)(up + pl.d + blk * 4);
    } else {
      w.gs = *(const uint32_t*)(g + pl.s + blk * 4);
      w.us = *(const uint32_t*)(up + pl.s + blk * 4);
      w.gd = *(const uint16_t*)(g + pl.d + blk * 2);
      w.ud = *(const uint16_t*)(up + pl.d + blk * 2);
    }
  }
}

// One wave: quantise the 16 SwiGLU outputs of each bucket token (16 lanes
// per token; a bucket holds at most kSmallT = 4 tokens) from the tile's slot
// ga, and store them as flagged words (qt: this wave's scratch slot).
template <class A>
__device__ __forceinline__ void gu_tile_store_wave(const A& a, int p0, int n, int f0, const QS_LDS float* ga,
                                                   QS_LDS int* qt, const PersistLds& L, uint32_t flag) {
  const int lane = qs_tid() & 63;
  const int tt = lane >> 4, r = lane & 15;
  const bool live = tt < n;
  const float v = live ? ga[tt * kGateTile + r] : 0.f;
  const float m = bfly_max<4>(fabsf(v));
  const int ex = fixed_exp(m);
  const int q = to_fixed(v, ex);
  const int s = bfly_sum_i32<4>(q);
  if (live) qt[tt * kGateTile + r] = q;
  __builtin_amdgcn_wave_barrier();
  if (live) {
    const int pair = L.pairs[p0 + tt];
    if (r < 4) {
      int h[4], l[4];
#pragma unroll
      // (word r: values r, 4+r, 8+r, 12+r for the Q2_K down dot; 4r..4r+3
      // for the Q4_K-style one)
      for (int i = 0; i < 4; ++i)
        split_limbs(qt[tt * kGateTile + (a.dfmt == kFmtQ4K ? 4 * r + i : 4 * i + r)], h[i], l[i]);
      const size_t wi = (size_t)pair * (a.F / 4) + f0 / 4 + r;
      ll_store(a.ll_a + wi, pack4(h[0], h[1], h[2], h[3]), flag);
      ll_store(a.ll_a + ll_al(a) + wi, pack4(l[0], l[1], l[2], l[3]), flag);
    }
    if (r == 0) {
      const size_t si = (size_t)pair * (a.F / kSubW) + f0 / kSubW;
      ll_store(a.ll_a + ll_as(a) + si, __float_as_uint(ldexpf(1.0f, ex - kFixedBits)), flag);
      ll_store(a.ll_a + ll_aa(a) + si, (uint32_t)s, flag);
    }
  }
}

// An item's active-expert slot u and first row f0.
template <class A>
__device__ __forceinline__ void gu_tile_item(const A& a, int item, int& u, int& f0) {
  const int tiles = a.F / kGateTile;
  u = item / tiles;
  f0 = (item % tiles) * kGateTile;
}

// Item `item` from its registers: SwiGLU of its 16 rows for every token of
// the bucket (at most kSmallT), into the slot ga.
template <int FMT, class A>
__device__ __forceinline__ void gu_tile_dots(const A& a, const typename GuTileOf<FMT>::T& t, int item,
                                             const PersistLds& L, QS_LDS float* ga) {
  const int nch = a.H / kChunkW, lpr = lanes_per_row(nch), cpl = nch / lpr;
  const int slots = kPersistThreads / lpr, slot = qs_tid() / lpr, j = qs_tid() % lpr;
  int u, f0;
  gu_tile_item(a, item, u, f0);
  (void)f0;
  const int p0 = L.aoff[u], n = L.aoff[u + 1] - p0;
  constexpr bool q2k = FMT == 1;
  float gacc[4] = {0.f, 0.f, 0.f, 0.f}, uacc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kGuUnits; ++i) {
    const int r = slot + (i / cpl) * slots, ch = j + (i % cpl) * lpr, cc = i % cpl;
    if (r >= kGateTile || i >= ((kGateTile - 1 - slot) / slots + 1) * cpl) continue;
    if (cc == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) gacc[q] = uacc[q] = 0.f;
    }
    const auto& w = t.c[i];
    const int c = ch & 3;
    uint32_t gw[16], uw[16];
    uint32_t gsc, usc;
    if constexpr (FMT == kFmtQ4K) {
      gsc = w.gs;
      usc = w.us;
      gw[0] = w.gq.x; gw[1] = w.gq.y; gw[2] = w.gq.z; gw[3] = w.gq.w;
      gw[4] = w.gq2.x; gw[5] = w.gq2.y; gw[6] = w.gq2.z; gw[7] = w.gq2.w;
      uw[0] = w.uq.x; uw[1] = w.uq.y; uw[2] = w.uq.z; uw[3] = w.uq.w;
      uw[4] = w.uq2.x; uw[5] = w.uq2.y; uw[6] = w.uq2.z; uw[7] = w.uq2.w;
    } else if (q2k) {
      gsc = w.gs;
      usc = w.us;
      gw[0] = w.gq.x; gw[1] = w.gq.y; gw[2] = w.gq.z; gw[3] = w.gq.w;
      uw[0] = w.uq.x; uw[1] = w.uq.y; uw[2] = w.uq.z; uw[3] = w.uq.w;
    } else {
      gsc = (w.gs >> (8 * c)) & 0xFFu;
      usc = (w.us >> (8 * c)) & 0xFFu;
      cb2_decode_dword(L.tab, w.gq.x, gw[0], gw[1], gw[2], gw[3]);
      cb2_decode_dword(L.tab, w.gq.y, gw[4], gw[5], gw[6], gw[7]);
      cb2_decode_dword(L.tab, w.gq.z, gw[8], gw[9], gw[10], gw[11]);
      cb2_decode_dword(L.tab, w.gq.w, gw[12], gw[13], gw[14], gw[15]);
      cb2_decode_dword(L.tab, w.uq.x, uw[0], uw[1], uw[2], uw[3]);
      cb2_decode_dword(L.tab, w.uq.y, uw[4], uw[5], uw[6], uw[7]);
      cb2_decode_dword(L.tab, w.uq.z, uw[8], uw[9], uw[10], uw[11]);
      cb2_decode_dword(L.tab, w.uq.w, uw[12], uw[13], uw[14], uw[15]);
    }
    // one token at a time (its x chunk is 40 registers); the decoded
    // weights stay live across the tokens
#pragma unroll 1
    for (int tt = 0; tt < 4; ++tt) {
      if (tt >= n) break;
      const int tok = L.pairs[p0 + tt] / a.k;
      uint32_t xh[16], xl[16];
      float xs[4];
      int xa[4];
      x_chunk<true>(a, L, tok, ch, xh, xl, xs, xa);
      float gp, up;
      if constexpr (FMT == kFmtQ4K) {
        const uint32_t g8[8] = {gw[0], gw[1], gw[2], gw[3], gw[4], gw[5], gw[6], gw[7]};
        const uint32_t u8[8] = {uw[0], uw[1], uw[2], uw[3], uw[4], uw[5], uw[6], uw[7]};
        gp = q4k_chunk_dot(g8, gsc, half_to_f32(w.gd & 0xFFFFu), half_to_f32(w.gd >> 16), xh, xl, xs, xa);
        up = q4k_chunk_dot(u8, usc, half_to_f32(w.ud & 0xFFFFu), half_to_f32(w.ud >> 16), xh, xl, xs, xa);
      } else if (q2k) {
        const uint32_t g4[4] = {gw[0], gw[1], gw[2], gw[3]}, u4[4] = {uw[0], uw[1], uw[2], uw[3]};
        gp = q2k_chunk_dot(g4, gsc, half_to_f32(w.gd & 0xFFFFu), half_to_f32(w.gd >> 16), xh, xl, xs, xa);
        up = q2k_chunk_dot(u4, usc, half_to_f32(w.ud & 0xFFFFu), half_to_f32(w.ud >> 16), xh, xl, xs, xa);
      } else {
        gp = half_to_f32(w.gd) * xs[0] * (float)cb2_chunk_dot(gw, xh, xl, gsc);
        up = half_to_f32(w.ud) * xs[0] * (float)cb2_chunk_dot(uw, xh, xl, usc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gacc[q] = q == tt ? gacc[q] + gp : gacc[q];
        uacc[q] = q == tt ? uacc[q] + up : uacc[q];
      }
    }
    if (cc == cpl - 1) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (tt >= n) continue;
        const float g = bfly_sum_dyn(gacc[tt], lpr);
        const float uu = bfly_sum_dyn(uacc[tt], lpr);
        if (j == 0) ga[tt * kGateTile + r] = silu_mul(g, uu);
      }
    }
  }
}

// The first W items of this workgroup are requested by gu_tiles_issue.
template <int FMT, class A, int W>
__device__ __forceinline__ void gu_tiles_issue(const A& a, const LayerPtrs& Lp, const PersistLds& L,
                                               const GuRange& R, typename GuTileOf<FMT>::T (&b)[W]) {
#pragma unroll
  for (int i = 0; i < W; ++i)
    if (i < R.n) gu_tile_load<FMT>(a, Lp, L, R.i0 + i * R.stride, b[i]);
}

// Every tile in registers at once (n <= W): the dots of all of them, one
// block barrier, then tile m's stores by wave m, side by side.  More tiles:
// each tile's dots, a barrier, its stores by wave 0 and a barrier before its
// slot is reused, and its registers are refilled with the tile W ahead.
template <int FMT, class A, int W>
__device__ __forceinline__ void gu_tiles_run(const A& a, const LayerPtrs& Lp, PersistLds& L, const GuRange& R,
                                             typename GuTileOf<FMT>::T (&b)[W], uint32_t flag) {
  static_assert(W <= kGuWinMax && W <= kPersistThreads / 64, "an LDS slot and a storing wave per tile");
  const int n = R.n;
  const int wave = qs_tid() >> 6, slot = a.T * kGateTile;   // (LDS: kGuWinMax slots of T * kGateTile above one token)
  const bool side = n <= W && a.T > 1;   // (one token: one slot in LDS)
  auto store = [&](int m, int s) {
    int u, f0;
    gu_tile_item(a, R.i0 + m * R.stride, u, f0);
    const int p0 = L.aoff[u];
    gu_tile_store_wave(a, p0, L.aoff[u + 1] - p0, f0, L.ga + s * slot, L.qtmp + s * slot, L, flag);
  };
#pragma unroll 1
  for (int m0 = 0; m0 < n; m0 += W) {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if (m0 + i >= n) break;
      gu_tile_dots<FMT>(a, b[i], R.i0 + (m0 + i) * R.stride, L, L.ga + (side ? i : 0) * slot);
      if (side) continue;
      __syncthreads();
      if (wave == 0) store(m0 + i, 0);
      __syncthreads();   // (the slot is rewritten by the next tile)
      if (m0 + i + W < n) gu_tile_load<FMT>(a, Lp, L, R.i0 + (m0 + i + W) * R.stride, b[i]);
    }
  }
  if (side) {
    QS_STAMP3(1);
    __syncthreads();
    if (wave < n) store(wave, wave);
    // (also keeps the other waves' polls and copies of the next phase behind
    // these stores)
    __syncthreads();
  }
}

// ------------------------------------------------------------ phase D ---
// One wave: rows r0..r0+7 of active expert u (in LDS) against every pair of its bucket.
template <bool SMALL, class A>
__device__ __forceinline__ void down_expert(const A& a, lds_cptr w, int u, PersistLds& L) {
  const int lane = qs_tid() & 63;
  const int nb = a.F / kBlockW;
  const int nch = a.F / kChunkW;
  const int lpr = lanes_per_row(nch);
  const int cpl = nch / lpr;
  const int rpi = 64 / lpr;
  const int rsub = lane / lpr, j = lane % lpr;
  const int q0 = L.aoff[u], q1 = L.aoff[u + 1];
  const bool q4k = a.dfmt == kFmtQ4K;   // else Q2_K
  const BlkGeom g = blk_geom(a.dfmt);
  lds_cptr wq = w, ws = w + kDownRows * nb * g.q, wd = ws + kDownRows * nb * g.s;
#pragma unroll 1
  for (int rr = rsub; rr < kDownRows; rr += rpi) {
    // one 64-weight chunk of this row at a time, read once for all pairs
#pragma unroll 1
    for (int cc = 0; cc < cpl; ++cc) {
      const int ch = j + cc * lpr;
      const int c = ch & 3;
      const uint32_t blk = (uint32_t)rr * nb + ch / 4;
      uint32_t qw[8];
      uint32_t scm;
      if (q4k) {   // 32 code bytes per chunk; its two scales and mins
        const uint4 qa = ld16(wq + blk * 128 + c * 32), qb = ld16(wq + blk * 128 + c * 32 + 16);
        qw[0] = qa.x; qw[1] = qa.y; qw[2] = qa.z; qw[3] = qa.w; qw[4] = qb.x; qw[5] = qb.y; qw[6] = qb.z; qw[7] = qb.w;
        scm = ld2(ws + blk * 16 + 2 * c) | ld2(ws + blk * 16 + 8 + 2 * c) << 16;
      } else {
        const uint4 qv = ld16(wq + blk * 64 + c * 16);
        qw[0] = qv.x; qw[1] = qv.y; qw[2] = qv.z; qw[3] = qv.w;
        qw[4] = qw[5] = qw[6] = qw[7] = 0u;
        scm = ld4(ws + blk * 16 + c * 4);
      }
      const uint32_t dd = ld4(wd + blk * 4);
      const float d = half_to_f32(dd & 0xFFFFu), dm = half_to_f32(dd >> 16);
#pragma unroll 1
      for (int pos = q0; pos < q1; ++pos) {
        const int pair = L.pairs[pos];
        uint32_t xh[16], xl[16];
        float xs[4];
        int xa[4];
        const size_t ao = (size_t)pair * (a.F / 4) + ch * 16;
        const size_t si = (size_t)pair * (a.F / kSubW) + ch * 4;
        if (SMALL) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 hv = lds_u4(L.dah + ao + 4 * i);
            const uint4 lv = lds_u4(L.dal + ao + 4 * i);
            xh[4 * i] = hv.x; xh[4 * i + 1] = hv.y; xh[4 * i + 2] = hv.z; xh[4 * i + 3] = hv.w;
            xl[4 * i] = lv.x; xl[4 * i + 1] = lv.y; xl[4 * i + 2] = lv.z; xl[4 * i + 3] = lv.w;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            xs[i] = L.das[si + i];
            xa[i] = L.daa[si + i];
          }
          // (every read above in flight before the first use: one wait;
          // not where the registers are spent on the shared expert)
          if constexpr (!wide_fixed<A>()) __builtin_amdgcn_sched_barrier(0);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint64_t hv = cld64(a.ah + ao + 2 * i), lv = cld64(a.al + ao + 2 * i);
            xh[2 * i] = (uint32_t)hv;
            xh[2 * i + 1] = (uint32_t)(hv >> 32);
            xl[2 * i] = (uint32_t)lv;
            xl[2 * i + 1] = (uint32_t)(lv >> 32);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            xs[i] = cldf(&a.as[si + i]);
            xa[i] = cldi(&a.aa[si + i]);
          }
        }
        float part;
        if (q4k) {
          part = q4k_chunk_dot(qw, scm, d, dm, xh, xl, xs, xa);
        } else {
          const uint32_t q2[4] = {qw[0], qw[1], qw[2], qw[3]};
          part = q2k_chunk_dot(q2, scm, d, dm, xh, xl, xs, xa);
        }
        part = bfly_sum_dyn(part, lpr);
        // lane j == 0 of this row group owns the entry for every chunk
        if (j == 0) L.o[pos * kDownRows + rr] = cc == 0 ? part : L.o[pos * kDownRows + rr] + part;
      }
    }
  }
}

// Shared expert down row (in LDS), one wave, lanes over Fs, all tokens.
template <bool SMALL, class A>
__device__ __forceinline__ void shared_down_row(const A& a, lds_cptr srow, PersistLds& L) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63;
#pragma unroll 1
  for (int t = 0; t < a.T; ++t) {
    float s = 0.f;
#pragma unroll 1
    for (int f = 8 * lane; f < a.Fs; f += 512) {
      float ww[8];
      shared_w8(a, srow, a.Fs, f, ww);
      float av[8];
      if (SMALL) {
        const float4 a0 = lds_f4(L.dash + t * a.Fs + f);
        const float4 a1 = lds_f4(L.dash + t * a.Fs + f + 4);
        av[0] = a0.x; av[1] = a0.y; av[2] = a0.z; av[3] = a0.w;
        av[4] = a1.x; av[5] = a1.y; av[6] = a1.z; av[7] = a1.w;
      } else {
        const float* at = a.ash + (size_t)t * a.Fs + f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint64_t v = cld64(at + 2 * c);
          av[2 * c] = __uint_as_float((uint32_t)v);
          av[2 * c + 1] = __uint_as_float((uint32_t)(v >> 32));
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) s = fmaf(ww[c], av[c], s);
    }
    s = bfly_sum<6>(s);
    if (lane == 0) L.sh[t * kDownRows + wave] = s;
  }
}

// Steering of the small-batch kernel's layer output (the instantiations
// with steering compiled in; the others carry none of it).  The combine left each output m of
// the workgroup's first tile in the register macc of thread idx (dres: its
// direction entry), those of later tiles in mb.  Every workgroup publishes
// its partial d . m per token (lanes 8t..8t+7 of wave 0, tile by tile, then
// a fixed tree) as flagged words, reads all G of them (the same words in
// every workgroup), sums them per token in a fixed order and writes
// m - sscale * d * (d . m) (+ x) for its rows.  The partial words are reused
// from layer to layer, which is safe for the reason the other flagged words
// are: every workgroup owns output rows.
template <class A>
__device__ __forceinline__ bool steer_small(const A& a, const float* dir, float macc, float dres, float xres,
                                         const float* x, const uint64_t* xll, float* y, uint64_t* yll,
                                         uint32_t flag, uint32_t flag_y, QS_LDS uint32_t* pw, QS_LDS float* dm,
                                         QS_LDS int* err) {
  const int wave = qs_tid() >> 6, lane = qs_tid() & 63, T = a.T;
  const int n_tiles = a.H / kDownRows;
  if (wave == 0) {   // T * kDownRows <= 32 lanes of wave 0 hold a tile's outputs
    float part = 0.f;
    const int t = lane / kDownRows;
    for (int tile = blockIdx.x; tile < n_tiles; tile += a.G) {
      const int h = tile * kDownRows + lane % kDownRows;
      const bool first = tile == (int)blockIdx.x;
      const float m = lane >= T * kDownRows ? 0.f : first ? macc : a.mb[(size_t)t * a.H + h];
      part += bfly_sum<3>(lane < T * kDownRows ? (first ? dres : dir[h]) * m : 0.f);
    }
    if ((lane & 7) == 0 && t < T)
      ll_store(a.ll_dot + (size_t)t * a.G + blockIdx.x, __float_as_uint(part), flag);
  }
  if (!ll_read(a, a.ll_dot, pw, T * a.G, flag, err, ll_waves(a, T * a.G))) return false;
  if (wave < T) {   // token `wave`: lanes take the partials g = lane + 64 i in order, then a fixed tree
    float s = 0.f;
    for (int g = lane; g < a.G; g += 64) s += __uint_as_float(pw[wave * a.G + g]);
    s = bfly_sum<6>(s);
    if (lane == 0) dm[wave] = s;
  }
  __syncthreads();
  for (int tile = blockIdx.x; tile < n_tiles; tile += a.G)
    for (int idx = qs_tid(); idx < T * kDownRows; idx += kPersistThreads) {
      const int t = idx / kDownRows, h = tile * kDownRows + idx % kDownRows;
      const size_t xi = (size_t)t * a.H + h;
      const bool first = tile == (int)blockIdx.x;   // (its output and residual input are in registers)
      float acc = (first ? macc : a.mb[xi]) - a.sscale * (first ? dres : dir[h]) * dm[t];
      if (a.residual)
        acc += first ? xres : (xll ? __uint_as_float((uint32_t)cld64(xll + xi)) : cldf(&x[xi]));
      if (yll) ll_store(yll + xi, __float_as_uint(acc), flag_y);
      else cstf(&y[xi], acc);
    }
  __syncthreads();   // dm (L.sh) is rewritten by the next layer
  return true;
}

// Down phase of the small-batch kernel.  The SwiGLU outputs arrive as
// flagged words (flag_a); the layer input x is plain (layer 0) or flagged
// words xll, already checked complete by this workgroup in phase R; the
// output goes to y (plain, last layer) or as flagged words (flag_y) to yll.
// The down rows of the first chunk were copied ahead into region B.
// `spare(w, nw)` runs once, on the waves that have no combine work of the
// last tile.  STEER: the layer output is steered (steer_small).
template <bool STEER, class A, class HK>
__device__ __forceinline__ bool phase_down_small(const A& a, int li, const LayerPtrs& Lp, const float* x,
                                                 const uint64_t* xll, float* y, uint64_t* yll, uint32_t flag_a,
                                                 uint32_t flag_y, PersistLds& L, HK&& spare) {
  const int wave = qs_tid() >> 6;
  const int na = *L.nact;
  const int n_tiles = a.H / kDownRows;
  const int T = a.T;
  const int chunk = down_chunk<true>(a);
  const uint32_t pe = dn_expert_bytes(a);
  QS_LDS uint8_t* base = L.pfb + down_base<true>(a);   // experts' rows; the shared rows are in L.sdr
  // residual inputs of the first tile, requested before the waits
  float xres = 0.f;
  const bool own_res = a.residual && qs_tid() < T * kDownRows && (int)blockIdx.x < n_tiles;
  if (own_res) {
    const size_t xi = (size_t)(qs_tid() / kDownRows) * a.H + blockIdx.x * kDownRows + qs_tid() % kDownRows;
    xres = xll ? __uint_as_float((uint32_t)cld64(xll + xi)) : cldf(&x[xi]);
  }
  // steering: the direction entries of the first tile, also before the waits
  const float* dir = STEER ? a.sdir + (size_t)li * a.H : nullptr;
  const float dres = dir && qs_tid() < T * kDownRows && (int)blockIdx.x < n_tiles
                         ? dir[blockIdx.x * kDownRows + qs_tid() % kDownRows] : 0.f;
  // every pair's SwiGLU limbs and the shared SwiGLU vector -> LDS (on the
  // waves without down-row copies in flight, when the words fit them)
  if (!ll_read(a, a.ll_a, (QS_LDS uint32_t*)L.dah, ll_a_words(a), flag_a, L.llerr, ll_a_waves(a))) return false;
  QS_STAMP(li, 11);
  float macc = 0.f;   // steering: this thread's output of the first tile (idx = thread)
  wait_all_and_sync();   // the down rows copied ahead
  QS_STAMP(li, 12);
  // sh_regs: the shared down rows of this workgroup's first tiles, into
  // registers; requested after both waits (the flagged read's polls and the
  // copies' landing would each wait for them: a wave's memory operations
  // complete in order), they land during the routed down GEMVs
  static_assert(kDownRows == kPersistThreads / 64, "one shared down row per wave");
  uint4 sdv[sh_dn_regs<A>()];
  if (sh_regs(a) && a.Fs) sh_dn_issue(a, Lp, 0, sdv);
  const bool two = down_pf_second(a, na);   // the second tile's rows were copied ahead too
  for (int tile = blockIdx.x; tile < n_tiles; tile += a.G) {
    const int r0 = tile * kDownRows;
    const bool first = tile == (int)blockIdx.x;
    // experts in chunks that fit beside the shared rows
    for (int u0 = 0; u0 < na; u0 += chunk) {       // na >= 1, chunk >= 1
      const int u1 = na - u0 < chunk ? na : u0 + chunk;
      const int jq = (tile - (int)blockIdx.x) / a.G;
      if (u0 == 0 && jq < 2) QS_STAMP3(12 + 4 * jq);
      const bool ahead = first ? u0 == 0 : two && jq == 1;   // (then u0 == 0: one chunk holds every expert)
      QS_LDS uint8_t* rows = base + (first || !ahead ? 0u : (uint32_t)na * pe);
      if (!ahead) {
        stage_now([&](int w, int n) {
          if (u0 == 0 && !sh_regs(a)) copy_sd_rows(a, Lp, L.sdr, r0, w, n);
          for (int c0 = u0; c0 < u1; c0 += 64) {
            const int el = act_lanes(L, c0, u1);
            const int m = u1 - c0 < 64 ? u1 - c0 : 64;
            for (int i = 0; i < m; ++i)
              copy_down_rows(a, Lp, base + (uint32_t)(c0 + i - u0) * pe, __builtin_amdgcn_readlane(el, i), r0, w, n);
          }
        });
      }
      if (u0 == 0 && jq < 2) QS_STAMP3(13 + 4 * jq);
      for (int u = u0 + wave; u < u1; u += kPersistThreads / 64) down_expert<true>(a, rows + (uint32_t)(u - u0) * pe, u, L);
      if (u0 == 0 && jq < 2) QS_STAMP3(14 + 4 * jq);
      if (u0 == 0 && a.Fs) {
        if (!sh_regs(a)) {
          shared_down_row<true>(a, L.sdr + (uint32_t)wave * srow_bytes(a.Fs, a.sq8 != 0), L);
        } else {
          const int jr = (tile - (int)blockIdx.x) / a.G, nr = sh_dn_round(a);
          if (jr > 0 && jr % nr == 0) sh_dn_issue(a, Lp, jr, sdv);   // the next round of rows
          sh_dn_compute(a, sdv, jr % nr, L);
        }
        if (jq < 2) QS_STAMP3(15 + 4 * jq);
      }
    }
    __syncthreads();
    QS_STAMP(li, 13);
    // wave 0 has the combine work (T * kDownRows <= 64 words)
    if (tile + a.G >= n_tiles && wave >= copy_w0(a)) spare(wave - copy_w0(a), kPersistThreads / 64 - copy_w0(a));
    for (int idx = qs_tid(); idx < T * kDownRows; idx += kPersistThreads) {
      const int t = idx / kDownRows, rr = idx % kDownRows, h = r0 + rr;
      float acc = 0.f;
      for (int jj = 0; jj < a.k; ++jj) {
        const int pos = L.tok_order[t * a.k + jj];
        acc = fmaf(L.cw[t * a.k + jj], L.o[pos * kDownRows + rr], acc);
      }
      if (a.Fs) acc += L.sh[idx];
      if (dir) {        // kept until the layer's d . m is known
        if (first) macc = acc;
        else a.mb[(size_t)t * a.H + h] = acc;
        continue;
      }
      if (a.residual) {
        const size_t xi = (size_t)t * a.H + h;
        acc += first && own_res && idx == qs_tid() ? xres
                                                   : (xll ? __uint_as_float((uint32_t)cld64(xll + xi)) : cldf(&x[xi]));
      }
      if (yll) ll_store(yll + (size_t)t * a.H + h, __float_as_uint(acc), flag_y);
      else cstf(&y[(size_t)t * a.H + h], acc);
    }
    QS_STAMP(li, 14);
    __syncthreads();     // L.o and L.sh are rewritten by the next tile
  }
  if ((int)blockIdx.x >= n_tiles && wave >= copy_w0(a)) spare(wave - copy_w0(a), kPersistThreads / 64 - copy_w0(a));
  // (the SwiGLU limbs are consumed: their LDS takes the partial words)
  if (dir)
    return steer_small(a, dir, macc, dres, own_res ? xres : 0.f, x, xll, y, yll, flag_a, flag_y,
                       (QS_LDS uint32_t*)L.dah, L.sh, L.llerr);
  return true;
}

// ------------------------------------------------------------- kernel ---
// The small-batch kernel (T <= kSmallT); qs_big.h holds the batched one.
// Every step takes its arguments as `const A&`: PersistArgs, or FixedArgs,
// whose compile-time shape constants shadow the runtime fields.
template <int FMT, bool STEER, class A>
__device__ __forceinline__ void persist_small_body(const A& a) {
  extern __shared__ __align__(16) uint8_t lds_raw[];
  PersistLds L = carve_lds<true>(lds_raw, a, FMT == 2);
  const int wave = qs_tid() >> 6, nw = kPersistThreads >> 6;
  if (qs_tid() == 0) *L.llerr = 0;
  if (FMT == 2) dma_to_lds<0>(a.cbtab, L.tab, (uint32_t)kCbTabWords * 4, wave, nw);
  LayerPtrs Lp = a.layers[0];
  pf_router_and_shared<true>(a, Lp, L, wave, nw);
  if (!sh_regs(a) && (int)blockIdx.x * kDownRows < a.H)
    copy_sd_rows(a, Lp, L.sdr, blockIdx.x * kDownRows, wave, nw);
  wait_all_and_sync();
  for (int li = 0; li < a.n_layers; ++li) {
    const bool more = li + 1 < a.n_layers;
    const LayerPtrs Ln = a.layers[more ? li + 1 : li];   // requested now, used at the end of D
    // flags of this layer: fl = its input x, fl+1 logits, fl+2 SwiGLU, fl+3 its output
    const uint32_t fl = a.ll_epoch + 3u * (uint32_t)li;
    const uint64_t* xll = li == 0 ? nullptr : ((li - 1) & 1 ? a.llx1 : a.llx0);
    uint64_t* yll = more ? (li & 1 ? a.llx1 : a.llx0) : nullptr;
    // ---- R: x -> LDS, RMS scales, router, shared gate/up
    QS_STAMP(li, 0);
    if (li == 0) dma_to_lds<kCoherent>(a.x_in, L.ax, (uint32_t)a.T * a.H * 4, wave, nw);
    else if (!ll_read(a, xll, (QS_LDS uint32_t*)L.ax, a.T * a.H, fl, L.llerr, ll_waves(a, a.T * a.H))) return;
    QS_STAMP(li, 1);
    // sh_regs: the first round of this workgroup's shared gate/up rows is
    // requested into registers now (after the x wait, which its loads would
    // delay); the wait below takes it with the router rows.  Requested after
    // the router instead, it delays every wave's logits polls by as long
    // (a wave's memory operations complete in order): measured the same.
    uint4 shg[sh_pairs<A>()], shu[sh_pairs<A>()];
    if (sh_regs(a) && a.Fs) sh_gu_issue(a, Lp, 0, shg, shu);
    QS_STAMP3(8);
    wait_all_and_sync();   // (and this layer's router rows and staged shared items)
    QS_STAMP(li, 2);
    if ((int)blockIdx.x >= router_groups(a)) token_rinv<true>(a, L, a.x_in, 0, a.T);
    phase_router<true>(a, Lp, a.x_in, L, fl + 1);   // ends with a block barrier
    QS_STAMP(li, 3);
    if (!sh_regs(a)) {
      shared_items<true>(a, Lp, a.x_in, L, fl + 2);
    } else if (a.Fs) {
      const int nr = sh_gu_round(a), mine = my_count(a, n_shared_items<true>(a));
      for (int j0 = 0; j0 < mine; j0 += nr) {
        if (j0 > 0) sh_gu_issue(a, Lp, j0, shg, shu);
        sh_gu_compute(a, shg, shu, j0, L, fl + 2);
        if (j0 / nr < 3) QS_STAMP3(9 + j0 / nr);
      }
    }
    QS_STAMP(li, 4);
    // ---- K: logits -> LDS, top-k, grouping, routed tiles -> LDS, x limbs
    if (!ll_read(a, a.ll_lg, (QS_LDS uint32_t*)L.lg, 2 * a.T * a.E, fl + 1, L.llerr)) return;
    QS_STAMP(li, 5);
    topk_small(a, li, L);   // (groups one token itself)
    if (a.T > 1) group_small(a, L);
    QS_STAMP(li, 6);
    // the routed gate/up tiles' chunks are requested at once (registers);
    // meanwhile x becomes fixed-point limbs
    typename GuTileOf<FMT>::T gut[GuWin<A>::v];
    const GuRange gr = gu_range(a, L);
    gu_tiles_issue<FMT>(a, Lp, L, gr, gut);
    QS_STAMP3(0);
    {
      const int nb = a.H / kBlockW;
      for (int u = wave; u < a.T * nb; u += nw) quant_x_wave<true>(a, a.x_in, u / nb, u % nb, L);
    }
    QS_STAMP(li, 7);
    __syncthreads();
    QS_STAMP(li, 8);
    // ---- GU
    gu_tiles_run<FMT>(a, Lp, L, gr, gut, fl + 2);
    QS_STAMP(li, 9);
    // region B (unused during GU) receives the down rows of the active
    // experts, from the waves that do not poll the SwiGLU words
    {
      const int dw = ll_a_waves(a) == copy_w0(a) ? copy_w0(a) : 0;
      if (wave >= dw) pf_down<true>(a, Lp, L, wave - dw, nw - dw);
    }
    // ---- D; region A is free: the next layer's router rows and shared
    // items are issued beside the combine
    QS_STAMP(li, 10);
    if (!phase_down_small<STEER>(a, li, Lp, a.x_in, xll, a.y_out, yll, fl + 2, fl + 3, L, [&](int w, int n) {
          if (!more) return;
          pf_router_and_shared<true>(a, Ln, L, w, n);
          // the shared down rows are no longer read by this layer
          if (!sh_regs(a) && (int)blockIdx.x * kDownRows < a.H)
            copy_sd_rows(a, Ln, L.sdr, blockIdx.x * kDownRows, w, n);
        }))
      return;
    QS_STAMP(li, 15);
    Lp = Ln;
  }
}

// Any shape: the layer shapes come from the arguments.  STEER: with the
// steered combine (every layer's output steered).
template <int FMT, bool STEER>
__global__ void __launch_bounds__(kPersistThreads) k_persist_small(PersistArgs a) {
  persist_small_body<FMT, STEER>(a);
}

// Launches over paged layers (experts read through the layer's expert map).
struct PagedArgs : PersistArgs {
  static constexpr bool kPaged = true;
};

template <int FMT, bool STEER>
__global__ void __launch_bounds__(kPersistThreads) k_persist_small_paged(PersistArgs a) {
  persist_small_body<FMT, STEER>(static_cast<const PagedArgs&>(a));
}

// One layer shape fixed at compile time.  The launch passes the same values
// in the runtime fields (the host checks); the static members shadow them,
// so every loop bound, offset and division by a shape folds to a constant.
template <int FMT, int H_, int E_, int K_, int F_, int FS_, int SQ8_, int T_, int G_, bool PG = false>
struct FixedArgs : PersistArgs {
  static constexpr int H = H_, E = E_, k = K_, F = F_, Fs = FS_, sq8 = SQ8_, T = T_, G = G_;
  static constexpr int gq2k = FMT == 1, r_et = 1, r_tt = T_;
  static constexpr int gfmt = FMT, dfmt = FMT == kFmtQ4K ? kFmtQ4K : kFmtQ2K;
  static constexpr bool kFixedShape = true;
  static constexpr bool kPaged = PG;
};

// PG: for launches over paged layers
template <int FMT, int H, int E, int K, int F, int FS, int SQ8, int T, int G, bool STEER = false, bool PG = false>
__global__ void __launch_bounds__(kPersistThreads) k_persist_small_fixed(PersistArgs a) {
  persist_small_body<FMT, STEER>(static_cast<const FixedArgs<FMT, H, E, K, F, FS, SQ8, T, G, PG>&>(a));
}

}  // namespace qs
