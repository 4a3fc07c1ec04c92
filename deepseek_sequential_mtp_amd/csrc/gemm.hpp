// MFMA GEMM core for gfx950: C[m, n] = sum_k A[m, k] * B[k, n] with fp32
// accumulation, WGM x WGN waves per workgroup, BM x BN output tile.
//
// K is staged through LDS in slices of 64 bytes per operand row (32 bf16 or
// 16 f32 elements) in NS stages.  Operands go global -> LDS directly
// (buffer_load ... lds): no staging registers and no ds_write.  The loads of
// slice kt + NS - 1 go into the stage that slice kt - 1 used, so the one
// barrier of each slice only needs the reads of the slice before it retired
// and the MFMA pipe never drains behind a wait for reads just issued.  The
// stages are distinct LDS objects and the K loop is unrolled by NS, so the
// compiler can tell that a fragment read of one stage does not depend on the
// loads in flight into the others.
//
// Operands are described by loaders: K-major (K contiguous), optionally with
// interleaved row sources, or MN-major (M or N contiguous), read back with
// the transposing LDS read.  Epilogues receive the accumulators in the MFMA
// result layout (see common.hpp) and do the stores / reductions.
#pragma once

#include <utility>

#include "common.hpp"

namespace mtp {

template <int BM_, int BN_, int WGM_ = 2, int WGN_ = 2, int NS_ = 4, int BNL_ = BN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int BNL = BNL_;                    // B rows held in LDS (>= BN)
  static constexpr int WGM = WGM_, WGN = WGN_;       // waves along M and N
  static constexpr int NT = 64 * WGM * WGN;           // threads per workgroup
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // per-wave tile
  static constexpr int MB = WM / 32, NB = WN / 32;    // 32x32 blocks per wave
  static constexpr int ROWB = 64;                     // bytes per operand row and stage
  static constexpr int NS = NS_;                      // LDS stages
  static_assert(NS >= 4 && NS <= 8, "stage count");
  static_assert(BNL >= BN, "LDS holds every B row of the tile");
  static constexpr int LDS_STAGE = (BM + BNL) * ROWB; // bytes per stage
};

// ---------------------------------------------------------------------------
// Global loads go through raw buffer resources: one resource per tile (or
// per K slice) in SGPRs, a 32-bit byte offset per lane, and the hardware
// returns zeros for offsets at or past the resource's size.  Masked lanes get
// kOOB.  No branches and no 64-bit address arithmetic per load.
// ---------------------------------------------------------------------------
constexpr unsigned kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, long bytes) {
  const long cap = 0x7ffffff0L;
  // The resource lives in SGPRs: make its inputs provably wave-uniform.
  const int n = __builtin_amdgcn_readfirstlane((int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)));
  const unsigned long a = reinterpret_cast<unsigned long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  void *pu = reinterpret_cast<void *>(((unsigned long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// Scalar element access through a buffer resource: loads past the resource
// return 0, stores past it are dropped (used for masked epilogue lanes).
__device__ __forceinline__ float buf_load_elem(__amdgpu_buffer_rsrc_t r, unsigned off, float) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_elem(__amdgpu_buffer_rsrc_t r, unsigned off, bf16_t) {
  return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store_elem(__amdgpu_buffer_rsrc_t r, unsigned off, float v, float) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store_elem(__amdgpu_buffer_rsrc_t r, unsigned off, float v, bf16_t) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS operand tiles (K-major): rows of 64 bytes (4 chunks of 16 B).  The LDS
// serves 256 bytes (64 banks) per cycle, i.e. 4 rows; a 16-lane group reading
// one logical chunk of 16 consecutive rows must hit 16 distinct 16-byte bank
// groups: chunk c of row r lives at physical chunk c ^ ((r >> 2) & 3).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lds_off64(int row, int chunk) {
  return (row << 6) + (((chunk ^ (row >> 2)) & 3) << 4);
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads: one instruction moves 64 lanes x 16 B into 1 KB
// of LDS at M0 + lane * 16.  The lane's source is split into a per-lane byte
// offset and a wave-uniform one carried in the instruction's SGPR offset.
// Lanes past K get kOOB; with the SGPR offset below the resource size,
// kOOB + offset still lies past it and does not wrap.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ lds_char *to_lds(char *p) { return (lds_char *)p; }

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, char *lds_dst, unsigned voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)to_lds(lds_dst), 16,
                                           voff, __builtin_amdgcn_readfirstlane(soff), 0, 0);
}

// K-major dense operand, op[r][k] = base[r * ld + k].  A 1 KB load block holds
// 16 tile rows; lane L fills physical chunk L & 3 of row L >> 2 and fetches
// the logical chunk the swizzle places there, (L & 3) ^ (L >> 4) (the block's
// first row is a multiple of 16, so the swizzle term depends on L only).
// With CAP < ROWS the tile has CAP rows in a ROWS-row LDS layout: the load
// blocks past CAP get out-of-range lane offsets (no memory traffic, zeros in
// LDS), so every wave still issues the same number of loads.
template <typename T, int ROWS, int NT, int CAP = ROWS>
struct DmaKMajor {
  static_assert(CAP <= ROWS && CAP % 16 == 0, "row cap");
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int NBLK = ROWS / 16, WAVES = NT / 64, PER_WAVE = NBLK / WAVES;
  static_assert(NBLK % WAVES == 0, "blocks per wave");
  static constexpr int kLoads = PER_WAVE;   // load instructions per wave and slice
  static constexpr int kReads = 1;          // LDS read instructions per fragment
  const T *base; long ld; int rows; int K;
  // Fragment of the 32-row block starting at tile row r0, K sub-step s
  // (32 bytes of K): lane l holds row r0 + l % 32, chunk 2 s + l / 32.
  __device__ static __forceinline__ uint4 frag(const char *region, int r0, int s, int lane) {
    return *reinterpret_cast<const uint4 *>(region + lds_off64(r0 + (lane & 31), 2 * s + (lane >> 5)));
  }
  __device__ __forceinline__ void issue(int row0, int k0, char *region) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long nrow = rows - row0 < CAP ? rows - row0 : CAP;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (long)row0 * ld, nrow * ld * (long)sizeof(T));
    const int ldb = (int)(ld * sizeof(T));
    const int c = (lane & 3) ^ (lane >> 4);
    const unsigned voff = k0 + c * E < K ? (unsigned)((lane >> 2) * ldb + c * 16) : kOOB;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave * PER_WAVE + i;
      dma16(rs, region + q * 1024, (CAP == ROWS || 16 * q < CAP) ? voff : kOOB,
            16 * q * ldb + k0 * (int)sizeof(T));
    }
  }
};

// K-major A operand in 128-byte rows: one row holds two consecutive 64-byte
// slices (a "pair"), so a 1 KB load block covers 8 rows x 128 bytes, i.e. 8
// whole 128-byte lines, where DmaKMajor's block touches 16 half lines.  The
// pair region is ROWS x 128 bytes; chunk c (0..7) of row r sits at physical
// chunk c ^ ((r >> 1) & 7), so the 16 rows a 16-lane group reads at one
// logical chunk fall on 16 distinct 16-byte bank groups.  Lane L of block q
// fills row 8 q + L / 8, physical chunk L % 8, and fetches the logical chunk
// the swizzle places there, (L % 8) ^ ((4 (q & 1) + L / 16) & 7).
template <typename T, int ROWS, int NT>
struct DmaKMajor128 {
  static constexpr bool kPairRows = true;
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int NBLK = ROWS / 8, WAVES = NT / 64, PER_WAVE = NBLK / WAVES;
  static_assert(NBLK % WAVES == 0, "blocks per wave");
  static constexpr int kLoads = PER_WAVE;   // load instructions per wave and pair
  static constexpr int kReads = 1;
  static constexpr int kRegionBytes = ROWS * 128;
  const T *base; long ld; int rows; int K;
  // Fragment of the 32-row block at tile row r0, K sub-step s (0..3) of the
  // pair: lane l holds row r0 + l % 32, logical chunk 2 s + l / 32.
  __device__ static __forceinline__ uint4 frag(const char *region, int r0, int s, int lane) {
    const int row = r0 + (lane & 31);
    const int c = 2 * s + (lane >> 5);
    return *reinterpret_cast<const uint4 *>(region + row * 128 + (((c ^ (row >> 1)) & 7) << 4));
  }
  __device__ __forceinline__ void issue(int row0, int k0, char *region) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long nrow = rows - row0 < ROWS ? rows - row0 : ROWS;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (long)row0 * ld, nrow * ld * (long)sizeof(T));
    const int ldb = (int)(ld * sizeof(T));
    unsigned voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int c = (lane & 7) ^ ((4 * par + (lane >> 4)) & 7);
      voff[par] = k0 + c * E < K ? (unsigned)((lane >> 3) * ldb + c * 16) : kOOB;
    }
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave * PER_WAVE + i;
      dma16(rs, region + q * 1024, voff[q & 1], 8 * q * ldb + k0 * (int)sizeof(T));
    }
  }
};

// SwiGLU-interleaved B operand: tile column c of wave column wn holds, for
// block b = (c mod WN) / 32, gate features (b < NB/2) or up features
// (b >= NB/2) of the same feature range, so the epilogue pairs them in-lane.
// Every 16-row load block lies in one 32-row block and hence reads one matrix.
template <typename T, class Cfg>
struct DmaKMajorSwiGLU {
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int BN = Cfg::BN, NT = Cfg::NT, WN = Cfg::WN, NBh = WN / 64;
  static constexpr int NBLK = BN / 16, WAVES = NT / 64, PER_WAVE = NBLK / WAVES;
  static_assert(NBLK % WAVES == 0, "blocks per wave");
  static constexpr int kLoads = PER_WAVE;
  static constexpr int kReads = 1;
  const T *gate; const T *up; long ld; int f; int K;
  __device__ static __forceinline__ uint4 frag(const char *region, int r0, int s, int lane) {
    return *reinterpret_cast<const uint4 *>(region + lds_off64(r0 + (lane & 31), 2 * s + (lane >> 5)));
  }
  __device__ __forceinline__ void issue(int row0, int k0, char *region) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int feat0 = (row0 / BN) * (BN / 2);
    const long nfeat = f - feat0 < BN / 2 ? f - feat0 : BN / 2;
    const long bytes = nfeat * ld * (long)sizeof(T);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gate + (long)feat0 * ld, bytes);
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(up + (long)feat0 * ld, bytes);
    const int ldb = (int)(ld * sizeof(T));
    const int c = (lane & 3) ^ (lane >> 4);
    const unsigned voff = k0 + c * E < K ? (unsigned)((lane >> 2) * ldb + c * 16) : kOOB;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave * PER_WAVE + i;
      const int row = 16 * q;                               // first tile column of the block
      const int wn = row / WN, blk = (row % WN) / 32;
      const bool is_up = blk >= NBh;
      const int fl = wn * (WN / 2) + (is_up ? blk - NBh : blk) * 32 + (row % 32);
      dma16(is_up ? ru : rg, region + q * 1024, voff, fl * ldb + k0 * (int)sizeof(T));
    }
  }
};

// MN-major operand, op[r][k] = base[k * ld + r] (r < rows, k < K): the stage
// region holds BK k-rows of ROWS elements each (CPR 16-byte chunks per k-row);
// chunk c of k-row k sits at physical chunk c ^ (4 (k & 3)).  A 1 KB load
// block covers RPB = 64 / CPR whole k-rows, so a lane's swizzle depends only
// on its position and the block parity.
//
// Fragments (K-major from the MFMA's point of view) are read with gfx950's
// transposing LDS read ds_read_b64_tr_b16: in each 16-lane group, lane j
// addresses 4 consecutive elements (4 m values) of k-row K0 + j / 4 at
// m = M0 + 4 (j % 4), and lane i receives the 4 values of column m = M0 + i
// for k = K0 .. K0 + 3.  Two such reads (K0 and K0 + 4) give the 8 K-values a
// 32x32x16 bf16 operand lane needs; with k-rows k .. k+3 in distinct 64-byte
// bank groups (the swizzle above) each half-wave is conflict-free.  f32
// operands (no transposing read) are read element by element.
template <typename T, int ROWS, int NT>
struct DmaMNMajor {
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int BK = 4 * E;                     // K elements per 64-byte slice
  static constexpr int ROWB = ROWS * (int)sizeof(T);
  static constexpr int CPR = ROWB / 16;
  static constexpr int RPB = 64 / CPR;
  static_assert(CPR == 16 || CPR == 32, "k-row of 256 or 512 bytes");
  static constexpr int NBLK = BK / RPB, WAVES = NT / 64, PER_WAVE = NBLK / WAVES;
  static_assert(NBLK % WAVES == 0, "blocks per wave");
  static constexpr int kLoads = PER_WAVE;
  static constexpr int kReads = sizeof(T) == 2 ? 2 : 4;
  const T *base; long ld; int rows; int K;

  __device__ static __forceinline__ int off(int k, int m) {
    return k * ROWB + ((((m / E) ^ (4 * (k & 3)))) << 4) + (m % E) * (int)sizeof(T);
  }
  __device__ static __forceinline__ uint4 frag(const char *region, int r0, int s, int lane) {
    if constexpr (sizeof(T) == 2) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s lds_v4s;
      const int g = lane >> 4, j = lane & 15;
      const int k = 16 * s + 8 * (g >> 1) + (j >> 2);
      const int m = r0 + 16 * (g & 1) + 4 * (j & 3);
      const char *p = region + off(k, m);
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)to_lds(const_cast<char *>(p)));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)to_lds(const_cast<char *>(p + 4 * ROWB)));
      const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
      return make_uint4(a.x, a.y, b.x, b.y);
    } else {
      const int m = r0 + (lane & 31);
      const int k = 8 * s + 4 * (lane >> 5);
      uint4 v;
      v.x = *reinterpret_cast<const unsigned *>(region + off(k, m));
      v.y = *reinterpret_cast<const unsigned *>(region + off(k + 1, m));
      v.z = *reinterpret_cast<const unsigned *>(region + off(k + 2, m));
      v.w = *reinterpret_cast<const unsigned *>(region + off(k + 3, m));
      return v;
    }
  }
  __device__ __forceinline__ void issue(int row0, int k0, char *region) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long nk = K - k0 < BK ? K - k0 : BK;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + (long)k0 * ld, nk * ld * (long)sizeof(T));
    const int kl = lane / CPR, pc = lane % CPR;
    const int ldb = (int)(ld * sizeof(T));
    unsigned voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int c = pc ^ (4 * ((RPB * par + kl) & 3));
      voff[par] = row0 + c * E < rows ? (unsigned)(kl * ldb + c * 16) : kOOB;
    }
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave * PER_WAVE + i;
      dma16(rs, region + q * 1024, voff[q & 1], RPB * q * ldb + row0 * (int)sizeof(T));
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

struct TileSched {
  int mt, nt, group_m, k_splits;
  int tile0, ntiles;   // the launch covers tiles [tile0, tile0 + ntiles)
  float *ws;           // partial-tile slots (the split tail of the balanced schedule)
};

// Waits until at most VM of this wave's vector-memory operations and at most
// LGKM of its LDS operations are outstanding, then barriers.  s_waitcnt
// layout on gfx9: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt
// [11:8].  LDS operations complete in order, so "at most LGKM outstanding"
// means every LDS operation issued before the last LGKM has completed; a
// count above the field's maximum is clamped (a stricter wait).
template <int VM, int LGKM = 0>
__device__ __forceinline__ void wait_vm_lds_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  constexpr int L = LGKM > 15 ? 15 : LGKM;
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (L << 8));
  __builtin_amdgcn_s_barrier();
}

// Scheduling pattern of one sub-step: NM slots of one MFMA followed by the
// slot's share of the NR LDS reads of the next sub-step and of NV global
// loads (spread out so that a wave never stalls on a burst of loads queued
// in front of its MFMAs).
template <int NM, int NR, int NV = 0, int Q = 0>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (Q < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
    constexpr int nr = (Q + 1) * NR / NM - Q * NR / NM;
    if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);  // DS read
    constexpr int nv = (Q + 1) * NV / NM - Q * NV / NM;
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);  // VMEM read
    sched_interleave<NM, NR, NV, Q + 1>();
  }
}

// ---------------------------------------------------------------------------
// Main loop over slices [kt0, kt0 + nk) of one BM x BN tile at (m0, n0):
// leaves the tile's partial sums in acc.  On return no load is in flight and
// every wave has finished reading the stages (an epilogue may reuse them).
//
// Slice kt lives in stage kt % NS and is consumed in two sub-steps of 32
// bytes of K each.  In the middle of slice kt (after the first
// sub-step's MFMAs, whose shadow hides the second sub-step's fragment reads)
// every wave waits until its loads of slice kt + 1 have landed -- the loads
// of slices kt + 2 .. kt + NS - 2 may stay in flight -- and until every LDS
// read it issued before this slice's second sub-step has completed; the
// block barrier then makes both true for all waves.  Stage (kt - 1) % NS is
// thereby retired and receives the loads of slice kt + NS - 1.  Slices past
// the range are issued as all-out-of-range loads (no memory traffic), so the
// number of loads in flight, and with it the wait count, is the same for
// every slice.
// ---------------------------------------------------------------------------
template <typename T, class Cfg, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop(const LA &la, const LB &lb, int m0, int n0, int kt0, int nk, int K,
                                              char *const *st, f32x16 (&acc)[Cfg::MB][Cfg::NB]) {
  constexpr int E = Elem<T>::kPerChunk;
  constexpr int BK = 4 * E;                    // K elements per 64-byte slice
  constexpr int MB = Cfg::MB, NB = Cfg::NB, NS = Cfg::NS;
  constexpr int LOADS = LA::kLoads + LB::kLoads;   // load instructions per wave and slice
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 fa[2][MB], fb[2][NB];
  const int ar0 = wm * Cfg::WM, br0 = wn * Cfg::WN;
  auto read_frags = [&](const char *stage, int s, uint4 *a, uint4 *b) {
#pragma unroll
    for (int i = 0; i < MB; ++i) a[i] = LA::frag(stage, ar0 + 32 * i, s, lane);
#pragma unroll
    for (int j = 0; j < NB; ++j) b[j] = LB::frag(stage + Cfg::BM * Cfg::ROWB, br0 + 32 * j, s, lane);
  };
  // slice it (relative to kt0) into a stage; past the range: out-of-range loads
  auto issue = [&](int it, char *stage) {
    const int k0 = it < nk ? (kt0 + it) * BK : K;
    la.issue(m0, k0, stage);
    lb.issue(n0, k0, stage + Cfg::BM * Cfg::ROWB);
  };
  constexpr int NM = MB * NB;                                  // MFMAs per sub-step
  constexpr int NR = MB * LA::kReads + NB * LB::kReads;        // LDS reads per sub-step
  auto mfmas = [&](int s) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) mma32(fa[s][i], fb[s][j], acc[i][j], T{});
  };
  // one slice on stage sc; sn is the next slice's stage, sp the previous one's
  auto slice = [&](int it, char *sc, const char *sn, char *sp) {
    read_frags(sc, 1, fa[1], fb[1]);
    mfmas(0);
    if constexpr (sizeof(T) == 2) sched_interleave<NM, NR>();
    wait_vm_lds_barrier<(NS - 3) * LOADS, NR>();   // slice it+1 landed, stage sp retired
    issue(it + NS - 1, sp);
    read_frags(sn, 0, fa[0], fb[0]);
    mfmas(1);
    if constexpr (sizeof(T) == 2) sched_interleave<NM, NR, LOADS>();
  };

#pragma unroll
  for (int j = 0; j < NS - 1; ++j) issue(j, st[j]);
  wait_vm_lds_barrier<(NS - 2) * LOADS>();     // slice 0 landed
  read_frags(st[0], 0, fa[0], fb[0]);
  int it = 0;
  for (; it + NS - 1 < nk; it += NS) {
#pragma unroll
    for (int j = 0; j < NS; ++j) slice(it + j, st[j], st[(j + 1) % NS], st[(j + NS - 1) % NS]);
  }
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (it + j < nk) slice(it + j, st[j], st[j + 1], st[(j + NS - 1) % NS]);
  wait_vm_lds_barrier<0>();                    // no load in flight into the stages
}

// ---------------------------------------------------------------------------
// Main loop (as gemm_mainloop) for an A operand in 128-byte rows
// (DmaKMajor128) and a B operand in 64-byte slices; kt0 must be even.  A pair p (slices 2p, 2p+1 of the block's K
// range) lives in A region p % 3, slice kt of B in B stage kt % 4 (3 x BM x
// 128 + 4 x BN x 64 bytes: 160 KB for 256 x 256).  The barrier in the middle
// of slice kt (same conditions as in gemm_mainloop) retires B stage (kt - 1) % 4,
// which receives B slice kt + 3, and, for even kt, A region (kt / 2 - 1) % 3,
// which receives pair kt / 2 + 2.  Loads are issued in the same order at
// every barrier, so the wait for slice kt + 1 always leaves one B slice and
// one A pair in flight.  The loop is unrolled by 12 slices (both rings come
// back to their first stage).
// ---------------------------------------------------------------------------
template <typename T, class Cfg, class LA, class LB>
__device__ __forceinline__ void gemm_mainloop_pairs(const LA &la, const LB &lb, int m0, int n0, int kt0, int nk,
                                                    int K, char *const *sa, char *const *sb,
                                                    f32x16 (&acc)[Cfg::MB][Cfg::NB]) {
  static_assert(sizeof(T) == 2, "pair rows are for bf16 operands");
  constexpr int E = Elem<T>::kPerChunk;
  constexpr int BK = 4 * E;                    // K elements per 64-byte slice
  constexpr int MB = Cfg::MB, NB = Cfg::NB;
  constexpr int LA2 = LA::kLoads, LB1 = LB::kLoads;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::WGN, wn = wave % Cfg::WGN;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 fa[2][MB], fb[2][NB];
  const int ar0 = wm * Cfg::WM, br0 = wn * Cfg::WN;
  // sub-step sa (0..3) of an A pair region, sub-step sb (0..1) of a B stage
  auto read_frags = [&](const char *ra, int sa_, const char *rb, int sb_, uint4 *a, uint4 *b) {
#pragma unroll
    for (int i = 0; i < MB; ++i) a[i] = LA::frag(ra, ar0 + 32 * i, sa_, lane);
#pragma unroll
    for (int j = 0; j < NB; ++j) b[j] = LB::frag(rb, br0 + 32 * j, sb_, lane);
  };
  auto issue_b = [&](int it, char *stage) {
    lb.issue(n0, it < nk ? (kt0 + it) * BK : K, stage);
  };
  auto issue_a = [&](int p, char *region) {
    la.issue(m0, 2 * p < nk ? (kt0 + 2 * p) * BK : K, region);
  };
  constexpr int NM = MB * NB;
  constexpr int NR = MB * LA::kReads + NB * LB::kReads;
  auto mfmas = [&](int s) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) mma32(fa[s][i], fb[s][j], acc[i][j], T{});
  };
  // slice it = 12 q + J (J fixes the stages at compile time)
  auto slice = [&](int it, auto Jc) {
    constexpr int J = decltype(Jc)::value;
    constexpr int P = J / 2, H = J & 1;        // pair index mod 6, half of the pair
    char *ra = sa[P % 3];
    char *rb = sb[J % 4];
    read_frags(ra, 2 * H + 1, rb, 1, fa[1], fb[1]);
    mfmas(0);
    sched_interleave<NM, NR>();
    wait_vm_lds_barrier<LB1 + LA2, NR>();      // slice it+1 landed; B stage J-1, A region P-1 retired
    issue_b(it + 3, sb[(J + 3) % 4]);
    if constexpr (H == 0) issue_a(it / 2 + 2, sa[(P + 2) % 3]);
    read_frags(sa[((J + 1) / 2) % 3], 2 * ((J + 1) & 1), sb[(J + 1) % 4], 0, fa[0], fb[0]);
    mfmas(1);
    sched_interleave<NM, NR, LB1 + (H == 0 ? LA2 : 0)>();
  };

  // the same issue order as the barriers of slices -4 .. -1 would produce
  issue_a(0, sa[0]);
  issue_b(0, sb[0]);
  issue_b(1, sb[1]);
  issue_a(1, sa[1]);
  issue_b(2, sb[2]);
  wait_vm_lds_barrier<2 * LB1 + LA2>();        // slice 0 (A pair 0, B slice 0) landed
  read_frags(sa[0], 0, sb[0], 0, fa[0], fb[0]);
  int it = 0;
  for (; it + 11 < nk; it += 12) {
    slice(it + 0, std::integral_constant<int, 0>{});
    slice(it + 1, std::integral_constant<int, 1>{});
    slice(it + 2, std::integral_constant<int, 2>{});
    slice(it + 3, std::integral_constant<int, 3>{});
    slice(it + 4, std::integral_constant<int, 4>{});
    slice(it + 5, std::integral_constant<int, 5>{});
    slice(it + 6, std::integral_constant<int, 6>{});
    slice(it + 7, std::integral_constant<int, 7>{});
    slice(it + 8, std::integral_constant<int, 8>{});
    slice(it + 9, std::integral_constant<int, 9>{});
    slice(it + 10, std::integral_constant<int, 10>{});
    slice(it + 11, std::integral_constant<int, 11>{});
  }
  if (it + 0 < nk) slice(it + 0, std::integral_constant<int, 0>{});
  if (it + 1 < nk) slice(it + 1, std::integral_constant<int, 1>{});
  if (it + 2 < nk) slice(it + 2, std::integral_constant<int, 2>{});
  if (it + 3 < nk) slice(it + 3, std::integral_constant<int, 3>{});
  if (it + 4 < nk) slice(it + 4, std::integral_constant<int, 4>{});
  if (it + 5 < nk) slice(it + 5, std::integral_constant<int, 5>{});
  if (it + 6 < nk) slice(it + 6, std::integral_constant<int, 6>{});
  if (it + 7 < nk) slice(it + 7, std::integral_constant<int, 7>{});
  if (it + 8 < nk) slice(it + 8, std::integral_constant<int, 8>{});
  if (it + 9 < nk) slice(it + 9, std::integral_constant<int, 9>{});
  if (it + 10 < nk) slice(it + 10, std::integral_constant<int, 10>{});
  wait_vm_lds_barrier<0>();                    // no load in flight into the stages
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
