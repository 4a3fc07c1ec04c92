// MFMA GEMM core for gfx950: C[m, n] = sum_k A[m, k] * B[k, n] with fp32
// accumulation, 256 threads (4 waves as 2 x 2), BM x BN output tile, K staged
// through LDS in slices of 128 bytes per row, double-buffered.
//
// Operands are described by loaders:
//   * K-major  (K contiguous; A[m][k] = base[rowA(m) * ld + k]): direct 16-byte
//     chunk copies, optional per-row source (gather / interleaved matrices);
//   * MN-major (M or N contiguous; A[m][k] = base[k * ld + m]): 8x8 (bf16) or
//     4x4 (f32) blocks transposed in registers on their way to LDS, so the LDS
//     tile is always K-contiguous.
// Epilogues receive the accumulators in the MFMA result layout (see
// common.hpp) and do the stores / reductions.
#pragma once

#include "common.hpp"

namespace mtp {

constexpr int kGemmThreads = 256;

template <int BM_, int BN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = BM / 2, WN = BN / 2;     // per-wave tile
  static constexpr int MB = WM / 32, NB = WN / 32;   // 32x32 blocks per wave
  static constexpr int LDS_STAGE = (BM + BN) * 128;  // bytes per stage
  static constexpr int LDS_BYTES = 2 * LDS_STAGE;
};

// ---------------------------------------------------------------------------
// Row sources for K-major operands: pointer of source row r of the operand
// (r in [0, rows)), or nullptr for a row past the end (zero fill).
// ---------------------------------------------------------------------------
template <typename T>
struct RowsDense {
  const T *base; long ld; int rows;
  __device__ __forceinline__ const T *row(int r) const { return r < rows ? base + (long)r * ld : nullptr; }
};
template <typename T>
struct RowsGather {   // row r reads base[idx[r]] (idx clamped into [0, nsrc))
  const T *base; long ld; int rows; const int *idx; int nsrc;
  __device__ __forceinline__ const T *row(int r) const {
    if (r >= rows) return nullptr;
    int s = idx[r];
    s = s < 0 ? 0 : (s >= nsrc ? nsrc - 1 : s);
    return base + (long)s * ld;
  }
};
// SwiGLU pairing: a tile of BN columns holds BN/2 output features.  Within
// each wave's WN columns, blocks [0, NB/2) read gate rows and [NB/2, NB) read
// up rows of the same features, so one lane holds gate(j) and up(j).
template <typename T, int BN>
struct RowsSwiGLU {
  const T *gate; const T *up; long ld; int f;
  __device__ __forceinline__ const T *row(int r) const {  // r = tile_n * BN + c
    const int tile = r / BN, c = r % BN;
    constexpr int WN = BN / 2, NBh = WN / 64;
    const int wn = c / WN, cc = c % WN, blk = cc / 32, lane = cc % 32;
    const bool is_up = blk >= NBh;
    const int feat = tile * (BN / 2) + wn * (WN / 2) + (is_up ? blk - NBh : blk) * 32 + lane;
    if (feat >= f) return nullptr;
    return (is_up ? up : gate) + (long)feat * ld;
  }
};

// ---------------------------------------------------------------------------
// Loaders: global -> registers (load) and registers -> LDS (store).
// ROWS = operand rows in the tile (BM for A, BN for B).
// ---------------------------------------------------------------------------
template <typename T, int ROWS, class Rows>
struct LoadKMajor {
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int NREG = ROWS * 8 / kGemmThreads;   // chunks per thread
  Rows src; int K;
  __device__ __forceinline__ void load(int row0, int k0, uint4 *reg) const {
    const int t = threadIdx.x;
    const int q = t & 7;
    const int k = k0 + q * E;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      const int r = (t >> 3) + 32 * i;
      const T *p = src.row(row0 + r);
      reg[i] = (p != nullptr && k < K) ? *reinterpret_cast<const uint4 *>(p + k) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(const uint4 *reg, char *lds) const {
    const int t = threadIdx.x;
    const int q = t & 7;
#pragma unroll
    for (int i = 0; i < NREG; ++i) {
      const int r = (t >> 3) + 32 * i;
      *reinterpret_cast<uint4 *>(lds + lds_off128(r, q)) = reg[i];
    }
  }
};

template <typename T, int ROWS>
struct LoadMNMajor {   // operand[r][k] = base[k * ld + r], r < rows, k < K
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int NBLK = 8 * (ROWS / E);                 // E x E blocks per tile
  static constexpr int BPT = (NBLK + kGemmThreads - 1) / kGemmThreads;
  static constexpr int NREG = BPT * E;
  const T *base; long ld; int rows; int K;
  __device__ __forceinline__ void load(int row0, int k0, uint4 *reg) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int blk = t + b * kGemmThreads;
      const int kc = blk & 7, mb = blk >> 3;
      const int m = row0 + mb * E;
      const bool okm = blk < NBLK && m < rows;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int k = k0 + kc * E + e;
        reg[b * E + e] = (okm && k < K) ? *reinterpret_cast<const uint4 *>(base + (long)k * ld + m)
                                        : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint4 *reg, char *lds) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int blk = t + b * kGemmThreads;
      if (blk >= NBLK) continue;
      const int kc = blk & 7, mb = blk >> 3;
      transpose_chunks(reg + b * E, T{});
#pragma unroll
      for (int j = 0; j < E; ++j)
        *reinterpret_cast<uint4 *>(lds + lds_off128(mb * E + j, kc)) = reg[b * E + j];
    }
  }
};

// ---------------------------------------------------------------------------
// Tile scheduling: blocks are dispatched round-robin over the 8 XCDs; give
// each XCD a contiguous range of logical tiles (shared L2), then walk the
// logical range in column-groups of `group_m` row tiles.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tile_coords(int logical, int mt, int nt, int group_m, int &tm, int &tn) {
  const int per_group = group_m * nt;
  const int g = logical / per_group;
  const int first = g * group_m;
  const int gsz = min(mt - first, group_m);
  const int in = logical - g * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

struct TileSched { int mt, nt, group_m, k_splits; };

// ---------------------------------------------------------------------------
// The kernel body.  Each block computes one BM x BN tile (optionally one K
// split of it) and hands the accumulators to the epilogue.
// ---------------------------------------------------------------------------
template <typename T, class Cfg, class LA, class LB, class Epi>
__device__ __forceinline__ void gemm_body(const LA &la, const LB &lb, const Epi &epi, int K,
                                          const TileSched &ts, char *lds) {
  constexpr int E = Elem<T>::kPerChunk;
  constexpr int BK = 8 * E;                    // K elements per LDS slice
  constexpr int MB = Cfg::MB, NB = Cfg::NB;
  const int ntiles = ts.mt * ts.nt * ts.k_splits;
  const int logical = xcd_remap(blockIdx.x, ntiles);
  const int split = logical % ts.k_splits;
  int tm, tn;
  tile_coords(logical / ts.k_splits, ts.mt, ts.nt, ts.group_m, tm, tn);
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;

  const int nk_total = (K + BK - 1) / BK;
  const int per = (nk_total + ts.k_splits - 1) / ts.k_splits;
  const int kt0 = split * per;
  const int kt1 = min(nk_total, kt0 + per);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[LA::NREG], rb[LB::NREG];
  if (kt0 < kt1) {
    la.load(m0, kt0 * BK, ra);
    lb.load(n0, kt0 * BK, rb);
    la.store(ra, lds);
    lb.store(rb, lds + Cfg::BM * 128);
  }
  __syncthreads();

  const int arow = wm * Cfg::WM + (lane & 31);
  const int brow = wn * Cfg::WN + (lane & 31);
  const int hsel = lane >> 5;
  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    char *sa = lds + cur * Cfg::LDS_STAGE;
    char *sb = sa + Cfg::BM * 128;
    const bool more = kt + 1 < kt1;
    if (more) {
      la.load(m0, (kt + 1) * BK, ra);
      lb.load(n0, (kt + 1) * BK, rb);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = 2 * s + hsel;
      uint4 fa[MB], fb[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        fa[i] = *reinterpret_cast<const uint4 *>(sa + lds_off128(arow + 32 * i, ch));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        fb[j] = *reinterpret_cast<const uint4 *>(sb + lds_off128(brow + 32 * j, ch));
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) mma32(fa[i], fb[j], acc[i][j], T{});
    }
    if (more) {
      char *na = lds + (cur ^ 1) * Cfg::LDS_STAGE;
      la.store(ra, na);
      lb.store(rb, na + Cfg::BM * 128);
    }
    __syncthreads();
  }
  epi.template apply<Cfg>(acc, m0, n0, wm, wn, lane, split, lds);
}

// Result-layout helpers: row / column of accumulator register r of block
// (i, j) for this lane, relative to the tile origin.
template <class Cfg>
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * Cfg::WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
template <class Cfg>
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * Cfg::WN + j * 32 + (lane & 31);
}

}  // namespace mtp
