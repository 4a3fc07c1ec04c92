// Shared device helpers for the gfx950 kernels: element types, bf16
// conversion, 16-byte chunk access, MFMA wrappers and the LDS swizzle used by
// every MFMA operand tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Storage types: bf16 is held as its uint16 bit pattern.
struct bf16_t { uint16_t bits; };

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;   // elements per 16-byte chunk
  static constexpr int kBytes = 2;
};
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  static constexpr int kBytes = 4;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Two values rounded to nearest even and packed (a in the low half): one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
}
// The two halves of a packed pair as floats.
__device__ __forceinline__ float bf16_lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float load_elem(const bf16_t *p, long i) { return bf16_to_f32(p[i].bits); }
__device__ __forceinline__ float load_elem(const float *p, long i) { return p[i]; }
__device__ __forceinline__ void store_elem(bf16_t *p, long i, float v) { p[i].bits = f32_to_bf16(v); }
__device__ __forceinline__ void store_elem(float *p, long i, float v) { p[i] = v; }
// 4 consecutive values in one store (p 8-byte aligned for bf16, 16 for f32).
__device__ __forceinline__ void store4(bf16_t *p, const float (&v)[4]) {
  *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void store4(float *p, const float (&v)[4]) {
  *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Unpack / pack one 16-byte chunk to / from floats.
__device__ __forceinline__ void chunk_to_f32(const uint4 &c, float *o, bf16_t) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void chunk_to_f32(const uint4 &c, float *o, float) {
  o[0] = __uint_as_float(c.x); o[1] = __uint_as_float(c.y);
  o[2] = __uint_as_float(c.z); o[3] = __uint_as_float(c.w);
}
__device__ __forceinline__ uint4 f32_to_chunk(const float *v, bf16_t) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}
__device__ __forceinline__ uint4 f32_to_chunk(const float *v, float) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}

// ---------------------------------------------------------------------------
// MFMA on one 16-byte chunk per lane and operand.
//
// 32x32 blocks: lane l supplies row (l & 31) of A and column (l & 31) of B;
// the lane's chunk covers K-slots (l >> 5) * E .. +E of a 2E-wide K slice
// (E = elements per chunk).  bf16: one v_mfma_f32_32x32x16_bf16.  f32: four
// v_mfma_f32_32x32x2f32, the t-th taking element t of both chunks, so slot
// (l>>5)*4 + t of A always meets the same slot of B.
// Result layout (all 32x32 MFMAs): lane l, register r holds
//   row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mma32(const uint4 &a, const uint4 &b, f32x16 &acc, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(const uint4 &a, const uint4 &b, f32x16 &acc, float) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// 16x16 blocks: lane l supplies row (l & 15) of A / column (l & 15) of B; its
// chunk covers K-slots (l >> 4) * E .. +E of a 4E-wide slice.  Result: lane
// l, register r holds row 4*(l/16) + r, column l%16.
__device__ __forceinline__ void mma16(const uint4 &a, const uint4 &b, f32x4 &acc, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(const uint4 &a, const uint4 &b, f32x4 &acc, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// LDS operand tiles: rows of 128 bytes (8 chunks of 16 B).  gfx950's LDS
// serves 256 bytes (64 banks) per cycle, i.e. a row pair; a 16-lane group
// reading one logical chunk of 16 consecutive rows must therefore spread over
// both halves and all eight chunk slots: chunk c of row r lives at physical
// chunk c ^ ((r >> 1) & 7) of its row, and r's parity picks the half.
__device__ __forceinline__ int lds_off128(int row, int chunk) {
  return (row << 7) + (((chunk ^ (row >> 1)) & 7) << 4);
}

// Transpose an E x E block held as E chunks (chunk i = row i, E elements)
// into E chunks (chunk j = column j).
__device__ __forceinline__ void transpose_chunks(uint4 *c, bf16_t) {
  // 8x8 block of 16-bit values.  Word w of chunk i holds elements (i, 2w),
  // (i, 2w+1).  Output chunk j, word w = (2w, j) | (2w+1, j) << 16.
  uint32_t in[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) { in[i][0] = c[i].x; in[i][1] = c[i].y; in[i][2] = c[i].z; in[i][3] = c[i].w; }
  uint32_t out[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = in[2 * w][j >> 1];
      const uint32_t hi = in[2 * w + 1][j >> 1];
      out[j][w] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = make_uint4(out[j][0], out[j][1], out[j][2], out[j][3]);
}
__device__ __forceinline__ void transpose_chunks(uint4 *c, float) {
  uint32_t in[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { in[i][0] = c[i].x; in[i][1] = c[i].y; in[i][2] = c[i].z; in[i][3] = c[i].w; }
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = make_uint4(in[0][j], in[1][j], in[2][j], in[3][j]);
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double warp_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Blocks are dispatched round-robin over the 8 XCDs (block i -> XCD i % 8).
// Map block ids so each XCD gets a contiguous range of logical ids and
// neighbouring logical work shares that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int ntiles) {
  const int q = ntiles >> 3, r = ntiles & 7;
  const int x = bid & 7, j = bid >> 3;
  return x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
}
// Reverse of SwiGLU at one element: from the gate pre-activation g, the up
// pre-activation u and the incoming gradient dgs of silu(g) u, the product
// sw = silu(g) u, dg = dgs u silu'(g) with silu'(g) = sig(g) (1 + g (1 -
// sig(g))), and du = dgs silu(g).
__device__ __forceinline__ void swiglu_bwd_elem(float g, float u, float dgs, float &sw, float &dg, float &du) {
  const float sig = __fdividef(1.f, 1.f + __expf(-g));
  const float sl = g * sig;
  sw = sl * u;
  dg = dgs * u * sig * (1.f + g * (1.f - sig));
  du = dgs * sl;
}
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace mtp
