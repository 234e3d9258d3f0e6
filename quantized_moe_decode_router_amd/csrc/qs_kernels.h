// qs_kernels.h -- device helpers shared by the decode kernels (fixed-point
// activations, the two block decoders, SwiGLU) and the stand-alone kernels
// around the persistent decode kernel (gfx950):
//   k_repack_*   raw blocks -> the planes the GEMVs read (at upload)
//   k_dequant_*  one matrix decoded with the GEMVs' field decoding (tests)
//   k_router, k_topk, k_group
//                the routing steps of one layer with every intermediate
//                written out (qs_moe_route: diagnostics and tests)
// The pages' engines fuse dequantisation into GEMV kernels (Quasar README,
// "Design decisions"); the integer formulation and the layout are this
// library's own.
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

// One 64-weight chunk of a Q4_K-style block against activation limbs in
// natural order.  qw: its 32 code bytes; dword k holds in its low nibbles
// weights 4k..4k+3 of the chunk (k < 8), in its high nibbles weights
// 32+4k..32+4k+3.  scm: the chunk's two sub-block scales in bytes 0, 1 and
// its two mins in bytes 2, 3.  16-element group g belongs to sub-block g/2.
__device__ __forceinline__ float q4k_chunk_dot(const uint32_t (&qw)[8], uint32_t scm, float d,
                                               float dmin, const uint32_t (&xh)[16],
                                               const uint32_t (&xl)[16], const float (&xs)[4],
                                               const int (&xa)[4]) {
  float part = 0.f;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    int sh = 0, sl = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t src = qw[(g & 1) * 4 + k];
      const uint32_t b = g < 2 ? (src & 0x0F0F0F0Fu) : ((src >> 4) & 0x0F0F0F0Fu);
      sh = sdot4(b, xh[4 * g + k], sh);
      sl = sdot4(b, xl[4 * g + k], sl);
    }
    const int S = sh * 256 + sl;
    const float sc = (float)((scm >> (8 * (g >> 1))) & 0xFFu);
    const float m = (float)((scm >> (16 + 8 * (g >> 1))) & 0xFFu);
    part = fmaf(xs[g], fmaf(d * sc, (float)S, -(dmin * m) * (float)xa[g]), part);
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

// Q4_K-style blocks -> planes (one thread per block): codes unchanged, the
// 12 packed scale bytes unpacked into 8 scales and 8 mins, d and dmin.
__global__ void k_repack_q4k(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                             size_t nblk_per_mat, size_t mat_stride, size_t n_mat) {
  const size_t gi = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= nblk_per_mat * n_mat) return;
  const size_t mat = gi / nblk_per_mat, blk = gi % nblk_per_mat;
  const uint8_t* s = src + gi * kQ4KBytes;
  const MatPlanes pl = q4k_planes(nblk_per_mat);
  uint8_t* base = dst + mat * mat_stride;
  for (int i = 0; i < 128; ++i) base[pl.q + blk * 128 + i] = s[16 + i];
  const uint8_t* sc = s + 4;
  uint8_t* o = base + pl.s + blk * 16;
  for (int j = 0; j < 8; ++j) {
    if (j < 4) {
      o[j] = sc[j] & 63;
      o[8 + j] = sc[j + 4] & 63;
    } else {
      o[j] = (uint8_t)((sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4));
      o[8 + j] = (uint8_t)((sc[j + 4] >> 4) | ((sc[j] >> 6) << 4));
    }
  }
  for (int i = 0; i < 4; ++i) base[pl.d + blk * 4 + i] = s[i];
}

// 8-bit shared-expert blocks (d binary16, then 32 int8 codes; row-major
// [rows][K/32]) -> padded rows [K codes | K/32 scales] of row_bytes each.
// One thread per block.
__global__ void k_repack_q8(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, size_t rows, int K,
                            uint32_t row_bytes) {
  const size_t nb = (size_t)K / kQ8W;
  const size_t gi = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= rows * nb) return;
  const size_t r = gi / nb, j = gi % nb;
  const uint8_t* s = src + gi * kQ8Bytes;
  uint8_t* o = dst + r * row_bytes;
  for (int i = 0; i < kQ8W; ++i) o[j * kQ8W + i] = s[2 + i];
  o[K + 2 * j] = s[0];
  o[K + 2 * j + 1] = s[1];
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

__global__ void k_dequant_q4k(const uint8_t* __restrict__ mat, size_t nblk, float* __restrict__ out) {
  const size_t blk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblk) return;
  const MatPlanes pl = q4k_planes(nblk);
  const uint8_t* qs = mat + pl.q + blk * 128;
  const uint8_t* scm = mat + pl.s + blk * 16;
  const uint32_t dd = *(const uint32_t*)(mat + pl.d + blk * 4);
  const float d = half_to_f32(dd & 0xFFFFu), dmin = half_to_f32(dd >> 16);
  float* o = out + blk * kBlockW;
  for (int j = 0; j < kBlockW; ++j) {
    const int c = j / 64, r = j % 64, sub = j / 32;
    const uint32_t byte = qs[32 * c + (r & 31)];
    const float q = (float)(r < 32 ? byte & 15u : byte >> 4);
    // d*sc and dmin*m are exact in fp32; one rounding of the difference
    o[j] = fmaf(d * (float)scm[sub], q, -(dmin * (float)scm[8 + sub]));
  }
}

// A shared-expert matrix as the kernels hold it (bf16 rows, or padded
// 8-bit rows) -> fp32 [rows][K]; one thread per weight.
__global__ void k_dequant_shared(const uint8_t* __restrict__ mat, size_t rows, int K, int q8,
                                 uint32_t row_bytes, float* __restrict__ out) {
  const size_t gi = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= rows * (size_t)K) return;
  const size_t r = gi / K;
  const int h = (int)(gi % K);
  const uint8_t* row = mat + r * row_bytes;
  if (q8) {
    const int j = h / kQ8W;
    const uint32_t dbits = (uint32_t)row[K + 2 * j] | ((uint32_t)row[K + 2 * j + 1] << 8);
    out[gi] = half_to_f32(dbits) * (float)(int8_t)row[h];
  } else {
    out[gi] = bf16_to_f32((uint32_t)row[2 * h] | ((uint32_t)row[2 * h + 1] << 8));
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

// silu(g) * u with the hardware reciprocal (about 1 ulp), not an IEEE divide
__device__ __forceinline__ float silu_mul(float g, float u) { return __fdividef(g, 1.0f + __expf(-g)) * u; }

}  // namespace qs
