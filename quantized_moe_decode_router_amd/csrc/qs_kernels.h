// qs_kernels.h -- HIP kernels of the routed-expert MoE decode step (gfx950).
//
// Data flow of one layer (all on the caller's stream):
//   k_router    logits[t][e] = sum_h Wr[e][h]*x[t][h] + b[e] in fp64
//   k_topk      per token: top-k by (logit desc, index asc); renormalised
//               softmax weights
//   k_group     stable bucket sort of (token, slot) pairs by expert; the
//               ascending list of experts in use
//   k_quant_x   x -> 16-bit fixed point limbs for the integer dot products
//   k_gateup    per (expert in use, 16-row tile): fused dequant + gate/up
//               GEMV + SwiGLU for every token in the expert's bucket, output
//               quantised per 16 rows; shared-expert gate/up in fp32
//   k_down      per 8 output rows: fused dequant + down GEMV for every pair,
//               then the weighted combine in a fixed order, shared-expert
//               down, residual
// The pages' engines fuse dequantisation into GEMV kernels for the same
// reason (Quasar README, "Design decisions"); the integer formulation and
// the layout are this library's own.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "qs_layout.h"

namespace qs {

// ------------------------------------------------------------ helpers ---

__device__ __forceinline__ float half_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Lanes cooperating on one matrix row: the largest power of two <= 64 that
// divides the row's chunk count (a multiple of 4), so row groups align with
// the xor butterflies of group_sum_dyn.
__device__ __forceinline__ int lanes_per_row(int nch) {
  int l = 64;
  while (nch % l) l >>= 1;
  return l;
}

__device__ __forceinline__ float group_sum_dyn(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float wave_max_abs(float v) {
  v = fabsf(v);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Fixed-point exponent for a group whose largest magnitude is `amax`:
// values are scaled by 2^(14-e) so that |v * 2^(14-e)| <= 2^14.
__device__ __forceinline__ int fixed_exp(float amax) {
  int e = 0;
  (void)frexpf(amax, &e);   // amax = f * 2^e, f in [0.5, 1); 0 -> e = 0
  return e < -100 ? -100 : e;
}

__device__ __forceinline__ int to_fixed(float v, int e) {
  return (int)rintf(ldexpf(v, kFixedBits - e));
}

// int16-range value -> (hi, lo) int8 limbs with v = 256*hi + lo.
__device__ __forceinline__ void split_limbs(int v, int& hi, int& lo) {
  hi = (v + 128) >> 8;
  lo = v - (hi << 8);
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)(d & 0xFF) << 24);
}

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Expert ids come from k_topk and are always in range; the clamp keeps every
// index derived from them inside its buffer whatever the input data.
__device__ __forceinline__ int valid_id(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// --------------------------------------------- codebook 2-bit decoding ---
// Two LDS tables of signed int8 quads built from the codebook:
//   tab[idx*16 + s]           weights 0..3 of a group with row idx, sign nibble s
//   tab[4096 + s*256 + idx]   weights 4..7, sign nibble s
// A code dword holds two groups (low half: group 2i, high half: 2i+1).
template <typename TabPtr>   // the tables in LDS (any address-space-qualified pointer)
__device__ __forceinline__ void cb2_decode_dword(TabPtr tab, uint32_t v,
                                                 uint32_t& q0, uint32_t& q1, uint32_t& q2,
                                                 uint32_t& q3) {
  q0 = tab[v & 0xFFFu];
  q1 = tab[4096u + ((v >> 4) & 0xFFFu)];
  q2 = tab[(v >> 16) & 0xFFFu];
  q3 = tab[4096u + (v >> 20)];
}

// 64-weight codebook chunk dot product against one token's limbs:
// returns sum over the chunk's two 32-weight sub-blocks of s_i * S_i (int).
__device__ __forceinline__ int cb2_chunk_dot(const uint32_t (&wq)[16], const uint32_t (&xh)[16],
                                             const uint32_t (&xl)[16], uint32_t scbyte) {
  int h0 = 0, l0 = 0, h1 = 0, l1 = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    h0 = sdot4(wq[q], xh[q], h0);
    l0 = sdot4(wq[q], xl[q], l0);
  }
#pragma unroll
  for (int q = 8; q < 16; ++q) {
    h1 = sdot4(wq[q], xh[q], h1);
    l1 = sdot4(wq[q], xl[q], l1);
  }
  const int s0 = (int)(scbyte & 15u), s1 = (int)((scbyte >> 4) & 15u);
  return s0 * (h0 * 256 + l0) + s1 * (h1 * 256 + l1);
}

// --------------------------------------------- Q2_K-style decoding ---
// qs dword i of a chunk holds weights 16i + 4*byte + p at bits 2p of each
// byte; (qw >> 2p) & 0x03030303 is the quad {p, 4+p, 8+p, 12+p}.
__device__ __forceinline__ float q2k_chunk_dot(const uint32_t (&qw)[4], uint32_t scm, float d,
                                               float dmin, const uint32_t (&xh)[16],
                                               const uint32_t (&xl)[16], const float (&xs)[4],
                                               const int (&xa)[4]) {
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int sh = 0, sl = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t b = (qw[i] >> (2 * p)) & 0x03030303u;
      sh = sdot4(b, xh[4 * i + p], sh);
      sl = sdot4(b, xl[4 * i + p], sl);
    }
    const int S = sh * 256 + sl;
    const float sc = (float)((scm >> (8 * i)) & 15u);
    const float m = (float)((scm >> (8 * i + 4)) & 15u);
    part = fmaf(xs[i], fmaf(d * sc, (float)S, -(dmin * m) * (float)xa[i]), part);
  }
  return part;
}

// ----------------------------------------------------------- repack ---

// Raw codebook 2-bit blocks -> QD/SC/D planes; one thread per block.
__global__ void k_repack_cb2(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                             size_t nblk_per_mat, size_t mat_stride, size_t n_mat) {
  const size_t gi = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= nblk_per_mat * n_mat) return;
  const size_t mat = gi / nblk_per_mat, blk = gi % nblk_per_mat;
  const uint8_t* s = src + gi * kCB2Bytes;
  const MatPlanes pl = cb2_planes(nblk_per_mat);
  uint8_t* base = dst + mat * mat_stride;
  uint16_t* qd = (uint16_t*)(base + pl.q + blk * 64);
  for (int g = 0; g < 32; ++g) {
    const uint32_t idx = s[6 + g], sg = s[38 + g];
    qd[g] = (uint16_t)(((sg >> 4) << 12) | (idx << 4) | (sg & 15u));
  }
  for (int i = 0; i < 4; ++i) base[pl.s + blk * 4 + i] = s[2 + i];
  base[pl.d + blk * 2] = s[0];
  base[pl.d + blk * 2 + 1] = s[1];
}

// Raw Q2_K-style blocks -> QS/SCM/DD planes; one thread per block.
__global__ void k_repack_q2k(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                             size_t nblk_per_mat, size_t mat_stride, size_t n_mat) {
  const size_t gi = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= nblk_per_mat * n_mat) return;
  const size_t mat = gi / nblk_per_mat, blk = gi % nblk_per_mat;
  const uint8_t* s = src + gi * kQ2KBytes;
  const MatPlanes pl = q2k_planes(nblk_per_mat);
  uint8_t* base = dst + mat * mat_stride;
  for (int i = 0; i < 64; ++i) base[pl.q + blk * 64 + i] = s[16 + i];
  for (int i = 0; i < 16; ++i) base[pl.s + blk * 16 + i] = s[i];
  for (int i = 0; i < 4; ++i) base[pl.d + blk * 4 + i] = s[80 + i];
}

// ---------------------------------------------------------- dequant ---
// One thread per block: the GEMV kernels' field decoding, written out as
// fp32 weights in natural order (used by tests through qs_moe_dequant).
__global__ void k_dequant_cb2(const uint8_t* __restrict__ mat, const uint32_t* __restrict__ cbtab,
                              size_t nblk, float* __restrict__ out) {
  __shared__ uint32_t tab[kCbTabWords];
  for (int i = threadIdx.x; i < kCbTabWords; i += blockDim.x) tab[i] = cbtab[i];
  __syncthreads();
  const size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblk) return;
  const MatPlanes pl = cb2_planes(nblk);
  const uint32_t* qd = (const uint32_t*)(mat + pl.q + blk * 64);
  const uint32_t sc = *(const uint32_t*)(mat + pl.s + blk * 4);
  const float d = half_to_f32(*(const uint16_t*)(mat + pl.d + blk * 2));
  float* o = out + blk * kBlockW;
  for (int w = 0; w < 16; ++w) {                 // 16 code dwords = 32 groups
    uint32_t q[4];
    cb2_decode_dword(tab, qd[w], q[0], q[1], q[2], q[3]);
    const int sub = w / 2;                        // 32-weight sub-block
    const float ds = d * (float)((sc >> (4 * sub)) & 15u);
    for (int k = 0; k < 4; ++k)
      for (int b = 0; b < 4; ++b) o[16 * w + 4 * k + b] = ds * (float)(int8_t)(q[k] >> (8 * b));
  }
}

__global__ void k_dequant_q2k(const uint8_t* __restrict__ mat, size_t nblk, float* __restrict__ out) {
  const size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblk) return;
  const MatPlanes pl = q2k_planes(nblk);
  const uint32_t* qs = (const uint32_t*)(mat + pl.q + blk * 64);
  const uint8_t* scm = mat + pl.s + blk * 16;
  const uint32_t dd = *(const uint32_t*)(mat + pl.d + blk * 4);
  const float d = half_to_f32(dd & 0xFFFFu), dmin = half_to_f32(dd >> 16);
  float* o = out + blk * kBlockW;
  for (int i = 0; i < 16; ++i) {                  // 16-weight sub-blocks
    const float dsc = d * (float)(scm[i] & 15u);
    const float dm = dmin * (float)(scm[i] >> 4);
    for (int p = 0; p < 4; ++p) {
      const uint32_t quad = (qs[i] >> (2 * p)) & 0x03030303u;
      for (int b = 0; b < 4; ++b) o[16 * i + 4 * b + p] = fmaf(dsc, (float)((quad >> (8 * b)) & 3u), -dm);
    }
  }
}

// ----------------------------------------------------------- router ---
constexpr double kRmsEps = 1e-6;

// One wave per expert row; fp64 accumulation of exact fp32 x fp32 products.
// With prenorm the logit is (Wr x) * r + b, r = 1/sqrt(mean(x^2) + eps) in
// fp64 (the router is linear, so this is Wr applied to RMSNorm(x)); every
// wave computes r in the same order and the wave of expert 0 stores it.
__global__ void k_router(const float* __restrict__ wr, const float* __restrict__ bias,
                         const float* __restrict__ x, int T, int H, int E, int prenorm,
                         double* __restrict__ logits, double* __restrict__ rinv) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * (blockDim.x >> 6) + wave;
  if (e >= E) return;
  const float4* row = (const float4*)(wr + (size_t)e * H);
  const double b = (double)bias[e];
  for (int t = 0; t < T; ++t) {
    const float4* xt = (const float4*)(x + (size_t)t * H);
    double acc = 0.0, ss = 0.0;
    for (int i = lane; i < H / 4; i += 64) {
      const float4 a = row[i], v = xt[i];
      acc = fma((double)a.x, (double)v.x, acc);
      acc = fma((double)a.y, (double)v.y, acc);
      acc = fma((double)a.z, (double)v.z, acc);
      acc = fma((double)a.w, (double)v.w, acc);
      if (prenorm) {
        ss = fma((double)v.x, (double)v.x, ss);
        ss = fma((double)v.y, (double)v.y, ss);
        ss = fma((double)v.z, (double)v.z, ss);
        ss = fma((double)v.w, (double)v.w, ss);
      }
    }
    acc = wave_sum_f64(acc);
    double r = 1.0;
    if (prenorm) r = 1.0 / sqrt(wave_sum_f64(ss) / (double)H + kRmsEps);
    if (lane == 0) {
      logits[(size_t)t * E + e] = prenorm ? fma(acc, r, b) : acc + b;
      if (e == 0) rinv[t] = r;
    }
  }
}

// ------------------------------------------------------------ top-k ---
// One wave per token.  E <= 1024 (16 logits per lane).
__global__ void k_topk(const double* __restrict__ logits, int E, int k, int32_t* __restrict__ ids,
                       float* __restrict__ wts, int32_t* __restrict__ ids_out,
                       float* __restrict__ w_out) {
  const int t = blockIdx.x, lane = threadIdx.x;
  __shared__ double sv[16];
  __shared__ int si[16];
  double v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane + 64 * i;
    const double l = e < E ? logits[(size_t)t * E + e] : 0.0;
    v[i] = l != l ? -INFINITY : l;   // NaN ranks last, so every pick is a valid, distinct expert
  }
  uint32_t taken = 0;
  for (int j = 0; j < k; ++j) {
    double bv = 0.0;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (bi == 0x7FFFFFFF || v[i] > bv)) {
        // first untaken candidate, then strictly larger ones (lower index wins ties)
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const double ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      const bool better = (oi != 0x7FFFFFFF) &&
                          (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi));
      if (better) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == 0) {
      sv[j] = bv;
      si[j] = bi;
    }
  }
  __syncthreads();
  if (lane == 0) {
    double z[16], sum = 0.0;
    for (int j = 0; j < k; ++j) {
      z[j] = exp(sv[j] - sv[0]);
      sum += z[j];
    }
    for (int j = 0; j < k; ++j) {
      const float w = (float)(z[j] / sum);
      ids[t * k + j] = si[j];
      wts[t * k + j] = w;
      if (ids_out) ids_out[t * k + j] = si[j];
      if (w_out) w_out[t * k + j] = w;
    }
  }
}

// ------------------------------------------------------------ group ---
// One workgroup of 1024 threads.  Stable bucket sort of the pairs
// p = t*k + j by expert; within a bucket pairs are ordered by token (a
// token selects an expert at most once).
struct GroupOut {
  int32_t* cnt;        // [E]
  int32_t* off;        // [E+1]
  int32_t* pairs;      // [T*k]   pair id at each bucket position
  int32_t* n_active;   // [1]
  int32_t* active;     // [E]     experts in use, ascending, then -1
  int32_t* tok_order;  // [T*k]   per token, bucket positions of its pairs by ascending expert
};

__global__ void k_group(const int32_t* __restrict__ ids, int T, int k, int E, GroupOut g) {
  __shared__ int cnt[1024];
  __shared__ int off[1025];
  __shared__ int act[1024];
  __shared__ uint32_t mask[1024 * 8];          // token bitmap per expert, T <= 256
  const int tid = threadIdx.x, nt = blockDim.x, P = T * k;
  for (int i = tid; i < E; i += nt) cnt[i] = 0;
  for (int i = tid; i < E * 8; i += nt) mask[i] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int e = valid_id(ids[p], E), t = p / k;
    atomicAdd(&cnt[e], 1);
    atomicOr(&mask[e * 8 + (t >> 5)], 1u << (t & 31));
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0, na = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = run;
      run += cnt[e];
      if (cnt[e] > 0) act[na++] = e;
    }
    off[E] = run;
    *g.n_active = na;
    for (int e = na; e < E; ++e) act[e] = -1;
  }
  __syncthreads();
  for (int i = tid; i < E; i += nt) {
    g.cnt[i] = cnt[i];
    g.off[i] = off[i];
    g.active[i] = act[i];
  }
  if (tid == 0) g.off[E] = off[E];
  for (int p = tid; p < P; p += nt) {
    const int e = valid_id(ids[p], E), t = p / k;
    int rank = 0;
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(mask[e * 8 + w]);
    rank += __popc(mask[e * 8 + (t >> 5)] & ((1u << (t & 31)) - 1u));
    g.pairs[off[e] + rank] = p;
  }
  for (int t = tid; t < T; t += nt) {
    // the token's k (expert, bucket position) sorted by expert id
    int ee[16], pp[16];
    for (int j = 0; j < k; ++j) {
      const int e = valid_id(ids[t * k + j], E);
      int rank = 0;
      for (int w = 0; w < (t >> 5); ++w) rank += __popc(mask[e * 8 + w]);
      rank += __popc(mask[e * 8 + (t >> 5)] & ((1u << (t & 31)) - 1u));
      int i = j;
      while (i > 0 && ee[i - 1] > e) {
        ee[i] = ee[i - 1];
        pp[i] = pp[i - 1];
        --i;
      }
      ee[i] = e;
      pp[i] = off[e] + rank;
    }
    for (int j = 0; j < k; ++j) g.tok_order[t * k + j] = pp[j];
  }
}

// -------------------------------------------------------- quantise x ---
// One workgroup (4 waves) per token; one wave per 256-element block with a
// shared exponent.  Writes limbs packed for the gate/up format, the per-16
// scale 2^(e-14) and (Q2_K consumers) the per-16 sums of the fixed values.
template <bool Q2K>
__global__ void k_quant_x(const float* __restrict__ x, int H, const double* __restrict__ rinv,
                          uint32_t* __restrict__ xh, uint32_t* __restrict__ xl,
                          float* __restrict__ xs, int32_t* __restrict__ xa) {
  const int t = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nblk = H / kBlockW;
  const float r = (float)rinv[t];          // 1, or the RMSNorm scale folded into x's scales
  for (int b = wave; b < nblk; b += blockDim.x >> 6) {
    const float4 v = *(const float4*)(x + (size_t)t * H + b * kBlockW + 4 * lane);
    const int e = fixed_exp(wave_max_abs(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)))));
    const int q0 = to_fixed(v.x, e), q1 = to_fixed(v.y, e), q2 = to_fixed(v.z, e), q3 = to_fixed(v.w, e);
    int h0, l0, h1, l1, h2, l2, h3, l3;
    split_limbs(q0, h0, l0);
    split_limbs(q1, h1, l1);
    split_limbs(q2, h2, l2);
    split_limbs(q3, h3, l3);
    uint32_t ph = pack4(h0, h1, h2, h3), pl = pack4(l0, l1, l2, l3);
    const size_t base = (size_t)t * (H / 4) + b * 64;
    if (Q2K) {
      // dword 4i+p of sub-block i gathers element p of lanes 4i..4i+3
      const int grp = lane & ~3, p = lane & 3;
      uint32_t oh = 0, ol = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const uint32_t sh = __shfl(ph, grp + bb, 64), sl = __shfl(pl, grp + bb, 64);
        oh |= ((sh >> (8 * p)) & 0xFFu) << (8 * bb);
        ol |= ((sl >> (8 * p)) & 0xFFu) << (8 * bb);
      }
      ph = oh;
      pl = ol;
    }
    xh[base + lane] = ph;
    xl[base + lane] = pl;
    int s = q0 + q1 + q2 + q3;
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if ((lane & 3) == 0) {
      const size_t si = (size_t)t * (H / kSubW) + b * 16 + (lane >> 2);
      xs[si] = ldexpf(r, e - kFixedBits);
      if (Q2K) xa[si] = s;
    }
  }
}

// ---------------------------------------------------------- gate/up ---
struct GateUpArgs {
  const uint8_t* gate;       // repacked expert matrices of this layer
  const uint8_t* up;
  size_t mat_stride;         // bytes per expert matrix
  const uint32_t* cbtab;     // codebook tables (global)
  int H, F, k, T;
  const uint32_t* xh;        // [T][H/4]
  const uint32_t* xl;
  const float* xs;           // [T][H/16]
  const int32_t* xa;         // [T][H/16] (Q2_K gate/up only)
  const int32_t* pairs;
  const int32_t* off;
  const int32_t* active;
  const int32_t* n_active;
  uint32_t* ah;              // [T*k][F/4]   SwiGLU output limbs (Q2_K packing)
  uint32_t* al;
  float* as;                 // [T*k][F/16]
  int32_t* aa;               // [T*k][F/16]
  // shared expert
  const uint16_t* sg;        // bf16 [Fs][H]
  const uint16_t* su;
  const float* x;            // fp32 [T][H]
  const double* rinv;        // [T] input scale (RMSNorm or 1)
  float* ash;                // fp32 [T][Fs]
  int Fs;
  int n_shared_items;
};

// silu(g) * u with the hardware reciprocal (about 1 ulp), not an IEEE divide
__device__ __forceinline__ float silu_mul(float g, float u) { return __fdividef(g, 1.0f + __expf(-g)) * u; }

// Shared-expert gate/up rows: one wave per row, fp32 FMA over bf16 weights.
__device__ void shared_gateup_item(const GateUpArgs& a, int item) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f = item * kSharedRows + wave;
  if (f >= a.Fs) return;
  const uint4* gr = (const uint4*)(a.sg + (size_t)f * a.H);
  const uint4* ur = (const uint4*)(a.su + (size_t)f * a.H);
  const int n16 = a.H / 8;
  for (int t = 0; t < a.T; ++t) {
    const float4* xt = (const float4*)(a.x + (size_t)t * a.H);
    float g = 0.f, u = 0.f;
    for (int i = lane; i < n16; i += 64) {
      const uint4 wg = gr[i], wu = ur[i];
      const float4 x0 = xt[2 * i], x1 = xt[2 * i + 1];
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
    const float r = (float)a.rinv[t];
    g = group_sum<64>(g) * r;
    u = group_sum<64>(u) * r;
    if (lane == 0) a.ash[(size_t)t * a.Fs + f] = silu_mul(g, u);
  }
}

// Load one lane's x limbs for chunk `ch` of a token.
__device__ __forceinline__ void load_x_chunk(const GateUpArgs& a, int t, int ch, uint32_t (&xh)[16],
                                             uint32_t (&xl)[16], float (&xs)[4], int (&xa)[4],
                                             bool q2k) {
  const uint4* ph = (const uint4*)(a.xh + (size_t)t * (a.H / 4) + ch * 16);
  const uint4* pl = (const uint4*)(a.xl + (size_t)t * (a.H / 4) + ch * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 h = ph[i], l = pl[i];
    xh[4 * i] = h.x; xh[4 * i + 1] = h.y; xh[4 * i + 2] = h.z; xh[4 * i + 3] = h.w;
    xl[4 * i] = l.x; xl[4 * i + 1] = l.y; xl[4 * i + 2] = l.z; xl[4 * i + 3] = l.w;
  }
  const size_t si = (size_t)t * (a.H / kSubW) + ch * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xs[i] = a.xs[si + i];
    xa[i] = q2k ? a.xa[si + i] : 0;
  }
}

// Routed gate/up task: rows [16*tile, 16*tile+16) of expert active[u], for
// every token of its bucket, two tokens at a time.
template <int FMT>
__device__ void routed_gateup_item(const GateUpArgs& a, int u, int tile, uint32_t* tab,
                                   float* lds_a) {
  const int e = a.active[u];
  const int p0 = a.off[e], n = a.off[e + 1] - p0;
  const int nch = a.H / kChunkW;                      // chunks per row
  const int lpr = lanes_per_row(nch);
  const int cpl = nch / lpr;                          // chunks per lane
  const int slots = blockDim.x / lpr;
  const int slot = threadIdx.x / lpr, j = threadIdx.x % lpr;
  const size_t nblk = (size_t)a.F * (a.H / kBlockW);
  const bool q2k = FMT == 1;
  const MatPlanes pl = q2k ? q2k_planes(nblk) : cb2_planes(nblk);
  const uint8_t* gbase = a.gate + (size_t)e * a.mat_stride;
  const uint8_t* ubase = a.up + (size_t)e * a.mat_stride;
  const int f0 = tile * kGateTile;
  for (int tg = 0; tg < n; tg += 2) {
    const int pa = a.pairs[p0 + tg];
    const int pb = tg + 1 < n ? a.pairs[p0 + tg + 1] : -1;
    const int nt = pb >= 0 ? 2 : 1;
    for (int r = slot; r < kGateTile; r += slots) {
      const int f = f0 + r;
      float gacc[2] = {0.f, 0.f}, uacc[2] = {0.f, 0.f};
      for (int cc = 0; cc < cpl; ++cc) {
        const int ch = j + cc * lpr;
        const size_t blk = (size_t)f * (a.H / kBlockW) + ch / 4;
        const int c = ch & 3;
        for (int tt = 0; tt < nt; ++tt) {
          const int t = (tt == 0 ? pa : pb) / a.k;
          uint32_t xh[16], xl[16];
          float xs[4];
          int xa[4];
          load_x_chunk(a, t, ch, xh, xl, xs, xa, q2k);
          for (int m = 0; m < 2; ++m) {
            const uint8_t* base = m == 0 ? gbase : ubase;
            float part;
            if (q2k) {
              const uint4 qv = *(const uint4*)(base + pl.q + blk * 64 + c * 16);
              const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
              const uint32_t scm = *(const uint32_t*)(base + pl.s + blk * 16 + c * 4);
              const uint32_t dd = *(const uint32_t*)(base + pl.d + blk * 4);
              part = q2k_chunk_dot(qw, scm, half_to_f32(dd & 0xFFFFu), half_to_f32(dd >> 16), xh,
                                   xl, xs, xa);
            } else {
              const uint4 cv = *(const uint4*)(base + pl.q + blk * 64 + c * 16);
              uint32_t wq[16];
              cb2_decode_dword(tab, cv.x, wq[0], wq[1], wq[2], wq[3]);
              cb2_decode_dword(tab, cv.y, wq[4], wq[5], wq[6], wq[7]);
              cb2_decode_dword(tab, cv.z, wq[8], wq[9], wq[10], wq[11]);
              cb2_decode_dword(tab, cv.w, wq[12], wq[13], wq[14], wq[15]);
              const uint32_t scb = base[pl.s + blk * 4 + c];
              const float d = half_to_f32(*(const uint16_t*)(base + pl.d + blk * 2));
              part = d * xs[0] * (float)cb2_chunk_dot(wq, xh, xl, scb);
            }
            if (m == 0) gacc[tt] += part;
            else uacc[tt] += part;
          }
        }
      }
      for (int tt = 0; tt < nt; ++tt) {
        const float g = group_sum_dyn(gacc[tt], lpr);
        const float uu = group_sum_dyn(uacc[tt], lpr);
        if (j == 0) lds_a[tt * kGateTile + r] = silu_mul(g, uu);
      }
    }
    __syncthreads();
    // quantise the 16 SwiGLU outputs of each token: lanes 16*tt + r
    if (threadIdx.x < 32) {
      const int tt = threadIdx.x >> 4, r = threadIdx.x & 15;
      const float v = tt < nt ? lds_a[tt * kGateTile + r] : 0.f;
      float m = fabsf(v);
#pragma unroll
      for (int s = 1; s < 16; s <<= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
      const int ex = fixed_exp(m);
      const int q = to_fixed(v, ex);
      int hi, lo;
      split_limbs(q, hi, lo);
      // dword p gathers q_p, q_{4+p}, q_{8+p}, q_{12+p}
      const int grp = threadIdx.x & ~15, p = r & 3;
      const int h0 = __shfl(hi, grp + p, 64), h1 = __shfl(hi, grp + 4 + p, 64);
      const int h2 = __shfl(hi, grp + 8 + p, 64), h3 = __shfl(hi, grp + 12 + p, 64);
      const int l0 = __shfl(lo, grp + p, 64), l1 = __shfl(lo, grp + 4 + p, 64);
      const int l2 = __shfl(lo, grp + 8 + p, 64), l3 = __shfl(lo, grp + 12 + p, 64);
      int s = q;
#pragma unroll
      for (int sft = 1; sft < 16; sft <<= 1) s += __shfl_xor(s, sft, 64);
      if (tt < nt) {
        const int pair = tt == 0 ? pa : pb;
        if (r < 4) {
          a.ah[(size_t)pair * (a.F / 4) + f0 / 4 + r] = pack4(h0, h1, h2, h3);
          a.al[(size_t)pair * (a.F / 4) + f0 / 4 + r] = pack4(l0, l1, l2, l3);
        }
        if (r == 0) {
          a.as[(size_t)pair * (a.F / kSubW) + f0 / kSubW] = ldexpf(1.0f, ex - kFixedBits);
          a.aa[(size_t)pair * (a.F / kSubW) + f0 / kSubW] = s;
        }
      }
    }
    __syncthreads();
  }
}

template <int FMT>
__global__ void __launch_bounds__(256) k_gateup(GateUpArgs a) {
  __shared__ uint32_t tab[FMT == 2 ? kCbTabWords : 1];
  __shared__ float lds_a[2 * kGateTile];
  const int item = blockIdx.x;
  if (item < a.n_shared_items) {
    shared_gateup_item(a, item);
    return;
  }
  const int r = item - a.n_shared_items;
  const int tiles = a.F / kGateTile;
  const int u = r / tiles, tile = r % tiles;
  if (u >= *a.n_active) return;
  if (FMT == 2) {
    const uint4* src = (const uint4*)a.cbtab;
    uint4* dst = (uint4*)tab;
    for (int i = threadIdx.x; i < kCbTabWords / 4; i += blockDim.x) dst[i] = src[i];
    __syncthreads();
  }
  routed_gateup_item<FMT>(a, u, tile, tab, lds_a);
}

// ------------------------------------------------------------- down ---
struct DownArgs {
  const uint8_t* down;       // repacked Q2_K expert matrices [E] of [H][F/256]
  size_t mat_stride;
  int H, F, k, T, E;
  const uint32_t* ah;        // [T*k][F/4]
  const uint32_t* al;
  const float* as;           // [T*k][F/16]
  const int32_t* aa;
  const int32_t* pairs;
  const int32_t* off;
  const int32_t* active;
  const int32_t* n_active;
  const int32_t* tok_order;  // [T][k]
  const float* wts;          // [T][k]
  const uint16_t* sd;        // bf16 [H][Fs] or null
  const float* ash;          // [T][Fs]
  int Fs;
  const float* xres;         // residual input [T][H] or null
  float* y;                  // [T][H]
};

__global__ void __launch_bounds__(256) k_down(DownArgs a) {
  extern __shared__ float o[];                       // [T*k][kDownRows]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int r0 = blockIdx.x * kDownRows;
  const int nch = a.F / kChunkW;
  const int lpr = lanes_per_row(nch);
  const int cpl = nch / lpr;
  const int rpi = 64 / lpr;                          // rows per wave instruction
  const int rsub = lane / lpr, j = lane % lpr;
  const size_t nblk = (size_t)a.H * (a.F / kBlockW);
  const MatPlanes pl = q2k_planes(nblk);
  const int na = *a.n_active;
  for (int u = wave; u < na; u += nw) {
    const int e = a.active[u];
    const uint8_t* base = a.down + (size_t)e * a.mat_stride;
    const int q0 = a.off[e], q1 = a.off[e + 1];
    for (int rr = rsub; rr < kDownRows; rr += rpi) {
      const int h = r0 + rr;
      for (int pos = q0; pos < q1; ++pos) {
        const int pair = a.pairs[pos];
        float part = 0.f;
        for (int cc = 0; cc < cpl; ++cc) {
          const int ch = j + cc * lpr;
          const size_t blk = (size_t)h * (a.F / kBlockW) + ch / 4;
          const int c = ch & 3;
          const uint4 qv = *(const uint4*)(base + pl.q + blk * 64 + c * 16);
          const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
          const uint32_t scm = *(const uint32_t*)(base + pl.s + blk * 16 + c * 4);
          const uint32_t dd = *(const uint32_t*)(base + pl.d + blk * 4);
          uint32_t xh[16], xl[16];
          float xs[4];
          int xa[4];
          const uint4* ph = (const uint4*)(a.ah + (size_t)pair * (a.F / 4) + ch * 16);
          const uint4* plw = (const uint4*)(a.al + (size_t)pair * (a.F / 4) + ch * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 hv = ph[i], lv = plw[i];
            xh[4 * i] = hv.x; xh[4 * i + 1] = hv.y; xh[4 * i + 2] = hv.z; xh[4 * i + 3] = hv.w;
            xl[4 * i] = lv.x; xl[4 * i + 1] = lv.y; xl[4 * i + 2] = lv.z; xl[4 * i + 3] = lv.w;
          }
          const size_t si = (size_t)pair * (a.F / kSubW) + ch * 4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            xs[i] = a.as[si + i];
            xa[i] = a.aa[si + i];
          }
          part += q2k_chunk_dot(qw, scm, half_to_f32(dd & 0xFFFFu), half_to_f32(dd >> 16), xh, xl,
                                xs, xa);
        }
        part = group_sum_dyn(part, lpr);
        if (j == 0) o[pos * kDownRows + rr] = part;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < a.T * kDownRows; idx += blockDim.x) {
    const int t = idx / kDownRows, rr = idx % kDownRows, h = r0 + rr;
    float acc = 0.f;
    for (int jj = 0; jj < a.k; ++jj) {
      const int pos = a.tok_order[t * a.k + jj];
      const int slot = a.pairs[pos] - t * a.k;
      acc = fmaf(a.wts[t * a.k + slot], o[pos * kDownRows + rr], acc);
    }
    if (a.Fs) {
      const uint16_t* srow = a.sd + (size_t)h * a.Fs;
      const float* at = a.ash + (size_t)t * a.Fs;
      float s = 0.f;
      for (int f = 0; f < a.Fs; ++f) s = fmaf(bf16_to_f32(srow[f]), at[f], s);
      acc += s;
    }
    if (a.xres) acc += a.xres[(size_t)t * a.H + h];
    a.y[(size_t)t * a.H + h] = acc;
  }
}

}  // namespace qs
