// qs_layout.h -- device-side layout of the routed-expert matrices and of the
// fixed-point activations, shared by the host code that sizes buffers and
// the kernels that read them.
//
// Routed matrices are re-laid out at upload into planes per expert matrix of
// N rows x nb blocks (block = 256 weights), keeping the byte count of the
// format.  Row n, block b is block number n*nb + b in every plane.
//
//   codebook 2-bit (70 B/block):
//     QD  [N*nb][64]  one 16-bit code per 8-weight group g:
//                     code = (sign_hi << 12) | (idx << 4) | sign_lo
//                     where sign_lo/sign_hi are the low/high nibble of sign[g]
//     SC  [N*nb][4]   the four scale bytes, unchanged
//     D   [N*nb][2]   d, unchanged
//   Q2_K-style (84 B/block):
//     QS  [N*nb][64]  qs, unchanged
//     SCM [N*nb][16]  scales, unchanged
//     DD  [N*nb][4]   d, dmin
//   Q4_K-style (144 B/block raw, 148 repacked):
//     QS  [N*nb][128] qs, unchanged (chunk c: bytes 32c..32c+31, low nibbles
//                     weights 64c..64c+31, high nibbles 64c+32..64c+63)
//     SCM [N*nb][16]  the eight 6-bit scales, then the eight 6-bit mins,
//                     one byte each (unpacked from the 12 packed bytes)
//     DD  [N*nb][4]   d, dmin
//
// A 64-weight "chunk" c (0..3) of a block is the unit one lane of a GEMV
// handles: 16 bytes of QD or QS (32 bytes of the Q4_K QS).
//
// Activations feeding an integer dot product are 16-bit fixed point with a
// power-of-two scale 2^(e-14) per 16 consecutive elements (one scale per 256
// for x, per 16 for the SwiGLU output), split into two int8 limbs
// v = 256*hi + lo, lo in [-128, 127], so that v_dot4_i32_i8 gives exact int32
// sums.  Limb bytes are packed four to a dword in the order the weight
// unpacking produces:
//   codebook consumer: dword q of a 16-element sub-block holds elements
//                      4q..4q+3 (natural order);
//   Q2_K consumer:     dword p holds elements p, 4+p, 8+p, 12+p;
//   Q4_K consumer:     natural order, as the codebook consumer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace qs {

constexpr int kBlockW = 256;          // weights per block
constexpr int kQ2KBytes = 84;
constexpr int kQ4KBytes = 144;        // raw Q4_K-style block
// routed formats (the values of qs_format)
constexpr int kFmtQ2K = 1, kFmtCB2 = 2, kFmtQ4K = 4;
constexpr int kCB2Bytes = 70;
constexpr int kQ8Bytes = 34;           // 8-bit shared-expert block: d binary16 + 32 int8
constexpr int kQ8W = 32;               // weights per 8-bit block
constexpr int kChunkW = 64;           // weights per lane chunk
constexpr int kSubW = 16;             // activation scale granularity
constexpr int kCbTabWords = 8192;     // two 4096-entry signed-quad tables
constexpr int kFixedBits = 14;        // |v| <= 2^14 after scaling
constexpr int kDownRows = 8;          // output rows per down-GEMV workgroup
constexpr int kGateTile = 16;         // gate/up rows per workgroup task
constexpr int kMaxTokens = 256;
constexpr int kMaxGrid = 1024;        // workgroups of a persistent launch (steering partials)
constexpr int kMaxPairs = 1024;

__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Plane offsets within one repacked expert matrix of `nblk` blocks.
struct MatPlanes {
  size_t q, s, d, bytes;
};

__host__ __device__ inline MatPlanes cb2_planes(size_t nblk) {
  MatPlanes p;
  p.q = 0;
  p.s = nblk * 64;
  p.d = p.s + nblk * 4;
  p.bytes = p.d + nblk * 2;
  return p;
}

__host__ __device__ inline MatPlanes q2k_planes(size_t nblk) {
  MatPlanes p;
  p.q = 0;
  p.s = nblk * 64;
  p.d = p.s + nblk * 16;
  p.bytes = p.d + nblk * 4;
  return p;
}

__host__ __device__ inline MatPlanes q4k_planes(size_t nblk) {
  MatPlanes p;
  p.q = 0;
  p.s = nblk * 128;
  p.d = p.s + nblk * 16;
  p.bytes = p.d + nblk * 4;
  return p;
}

// Bytes per block in the code, scale and d planes of a repacked matrix.
struct BlkGeom {
  uint32_t q, s, d;
};
__host__ __device__ inline BlkGeom blk_geom(int fmt) {
  if (fmt == kFmtCB2) return BlkGeom{64u, 4u, 2u};
  if (fmt == kFmtQ4K) return BlkGeom{128u, 16u, 4u};
  return BlkGeom{64u, 16u, 4u};
}
__host__ __device__ inline MatPlanes fmt_planes(int fmt, size_t nblk) {
  return fmt == kFmtCB2 ? cb2_planes(nblk) : fmt == kFmtQ4K ? q4k_planes(nblk) : q2k_planes(nblk);
}
// repacked bytes per block
__host__ __device__ inline uint32_t blk_bytes(int fmt) {
  const BlkGeom g = blk_geom(fmt);
  return g.q + g.s + g.d;
}

}  // namespace qs
