// GEMM epilogues.  Each receives the wave's accumulators acc[MB][NB] in the
// 32x32 MFMA result layout (lane l, register r -> row 8*(r/4)+4*(l/32)+r%4,
// column l%32 of block (i, j)) plus the tile origin.
#pragma once

#include <type_traits>

#include "gemm.hpp"

namespace mtp {

// ---------------------------------------------------------------------------
// Cross-lane helpers for the result layout.
//
// Lane-pair stores for 2-byte outputs: lanes l and l ^ 1 hold columns c and
// c ^ 1 of the same rows, and registers r, r + 1 (r even) hold rows R, R + 1
// of one column.  Trading one value over the lane pair (a DPP move) leaves
// the even lane with row R and the odd lane with row R + 1, each with the two
// adjacent columns (c & ~1, c | 1): one 4-byte store instead of two 2-byte
// stores, and a half-wave writes whole 128-byte lines.  (4-byte outputs keep
// one store per value: a half-wave already covers a whole line per row.)
// Every output stored this way has an even row length.
//
// Half-wave reductions: max or sum over the 32 lanes of a half-wave (one
// accumulator row) with DPP moves folded into the arithmetic: the two quad
// permutations, the half-row and row mirrors reduce each 16-lane row, and a
// broadcast of lane 15 of rows 0 and 2 into rows 1 and 3 completes the
// half-wave, whose result is valid in lanes 16..31 and 48..63.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL, ROW_MASK, 0xF,
                                                    false));
}
__device__ __forceinline__ void pair_rows(float a, float b, bool odd, float &lo, float &hi) {
  const float got = dpp_f<0xB1>(0.f, odd ? a : b);   // quad_perm [1,0,3,2]: lane l ^ 1
  lo = odd ? got : a;
  hi = odd ? b : got;
}
template <typename OutT>
__device__ __forceinline__ void store_pair(__amdgpu_buffer_rsrc_t r, unsigned off, float lo, float hi) {
  if constexpr (sizeof(OutT) == 4) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = {__float_as_uint(lo), __float_as_uint(hi)};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
  } else if constexpr (std::is_same_v<OutT, bf16_t>) {
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(lo, hi), r, off, 0, 0);
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 v = {(_Float16)lo, (_Float16)hi};
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, off, 0, 0);
  }
}
template <bool MAX>
__device__ __forceinline__ float halfwave_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  const float id = MAX ? -INFINITY : 0.f;
  x = op(x, dpp_f<0xB1>(id, x));          // quad_perm [1,0,3,2]
  x = op(x, dpp_f<0x4E>(id, x));          // quad_perm [2,3,0,1]
  x = op(x, dpp_f<0x141>(id, x));         // row_half_mirror
  x = op(x, dpp_f<0x140>(id, x));         // row_mirror
  x = op(x, dpp_f<0x142, 0xA>(id, x));    // row_bcast:15 into rows 1 and 3
  return x;
}

// ---------------------------------------------------------------------------
// C = alpha * acc (+ residual) (+ C if accumulate).  One K-split writes its
// own slab C + split * split_stride.  Branch-free: C and R are addressed
// through buffer resources that start at the tile's first row and end at
// row M, columns past N get an out-of-range offset, so a block's loads are
// issued back to back and masked lanes neither read nor write.
// ---------------------------------------------------------------------------
template <typename OutT, typename ResT>
struct EpiStore {
  OutT *C; long ldc; int M, N; float alpha;
  const float *alpha_dev;       // if set, alpha is read from device memory
  const ResT *R; long ldr;      // residual added after scaling (nullable)
  int accumulate;               // add into existing C
  long split_stride;
  template <class Cfg>
  __device__ __forceinline__ void apply(f32x16 (&acc)[Cfg::MB][Cfg::NB], int m0, int n0, int wm,
                                        int wn, int lane, int split, char *, char *) const {
    OutT *Cs = C + split * split_stride;
    const float al = alpha_dev != nullptr ? *alpha_dev : alpha;
    const long rows = M - m0 < Cfg::BM ? M - m0 : Cfg::BM;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(Cs + (long)m0 * ldc, rows * ldc * (long)sizeof(OutT));
    const __amdgpu_buffer_rsrc_t rr =
        make_rsrc(R != nullptr ? R + (long)m0 * ldr : nullptr, R != nullptr ? rows * ldr * (long)sizeof(ResT) : 0);
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
      for (int j = 0; j < Cfg::NB; ++j) {
        const int col = n0 + acc_col<Cfg>(wn, j, lane);
        const bool cok = col < N;
        unsigned oc[16], orr[16];
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row<Cfg>(wm, i, r, lane);
          oc[r] = cok ? (unsigned)(((long)row * ldc + col) * sizeof(OutT)) : kOOB;
          orr[r] = cok ? (unsigned)(((long)row * ldr + col) * sizeof(ResT)) : kOOB;
          v[r] = al * acc[i][j][r];
        }
        if (R != nullptr) {
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] += buf_load_elem(rr, orr[r], ResT{});
        }
        if (accumulate) {
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] += buf_load_elem(rc, oc[r], OutT{});
        }
        if constexpr (sizeof(OutT) == 2) {
          // lane-pair stores (whole 128-byte lines per half-wave): row R (even
          // lane) or R + 1 (odd lane), columns c & ~1, c | 1
          const bool odd = lane & 1;
          const unsigned pc = (unsigned)((col & ~1) * sizeof(OutT));
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            float lo, hi;
            pair_rows(v[r], v[r + 1], odd, lo, hi);
            const int row = acc_row<Cfg>(wm, i, r, lane) + (odd ? 1 : 0);
            store_pair<OutT>(rc, cok ? pc + (unsigned)((long)row * ldc * sizeof(OutT)) : kOOB, lo, hi);
          }
        } else {
          // 4-byte values: a half-wave already writes one whole 128-byte line per row
#pragma unroll
          for (int r = 0; r < 16; ++r) buf_store_elem(rc, oc[r], v[r], OutT{});
        }
      }
  }
};

// ---------------------------------------------------------------------------
// Fused QKV + rotate-half RoPE.  Output [M, 3*A] with q = cols [0, A),
// k = [A, 2A), v = [2A, 3A).  q and k are rotated at position pos[row]:
// with jj = j mod HALF (j = column inside the head), (c, s) = rope[pos][jj],
//   out_j = x_j c - x_(j+HALF) s      (j <  HALF)
//   out_j = x_j c + x_(j-HALF) s      (j >= HALF)
// The partner column sits in the same lane, HALF/32 blocks away (HALF >= 32:
// the wave's column range covers whole heads), or HALF lanes away (HALF < 32).
// Stores go through a buffer resource ending at row M (branch-free, as in
// EpiStore); whether a 32-column block is rotated is decided per wave.
// ---------------------------------------------------------------------------
template <typename OutT, int HALF>
struct EpiRope {
  OutT *C; long ldc; int M, N, A;
  const int *pos;               // [M] position of each row inside its run
  const float2 *rope;           // [max_pos][HALF] (cos, sin); nullptr = no RoPE
  template <class Cfg>
  __device__ __forceinline__ void apply(f32x16 (&acc)[Cfg::MB][Cfg::NB], int m0, int n0, int wm,
                                        int wn, int lane, int, char *, char *) const {
    constexpr int HD = 2 * HALF;
    static_assert(HALF < 32 || (Cfg::WN % HD) == 0, "wave columns must cover whole heads");
    const long rows = M - m0 < Cfg::BM ? M - m0 : Cfg::BM;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C + (long)m0 * ldc, rows * ldc * (long)sizeof(OutT));
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(pos + m0, rows * (long)sizeof(int));
    const bool odd = lane & 1;
    // rotated values of block j into out[j]; then lane-pair stores
    float out[Cfg::NB][16];
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i) {
      int p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p[r] = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, (unsigned)(acc_row<Cfg>(wm, i, r, lane) * 4), 0, 0);
      if constexpr (HALF >= 32) {
        // block j (j & PB == 0) holds the first half of a head, block j | PB
        // the second half of the same columns: one (cos, sin) serves both
        constexpr int PB = HALF / 32;
#pragma unroll
        for (int j = 0; j < Cfg::NB; ++j) {
          if ((j & PB) != 0) continue;
          const int col = n0 + acc_col<Cfg>(wn, j, lane);
          const int jj = col % HD;                         // < HALF
          const int col0 = n0 + acc_col<Cfg>(wn, j, 0);
          const bool rot = rope != nullptr && __builtin_amdgcn_readfirstlane(col0) < 2 * A;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float xl = acc[i][j][r], xh = acc[i][j | PB][r];
            out[j][r] = xl;
            out[j | PB][r] = xh;
            if (rot) {
              const float2 cs = rope[(long)p[r] * HALF + jj];
              out[j][r] = xl * cs.x - xh * cs.y;
              out[j | PB][r] = xh * cs.x + xl * cs.y;
            }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < Cfg::NB; ++j) {
          const int col = n0 + acc_col<Cfg>(wn, j, lane);
          const int jh = col % HD;
          const bool lo = jh < HALF;
          const int jj = lo ? jh : jh - HALF;
          const int col0 = n0 + acc_col<Cfg>(wn, j, 0);
          const bool rot = rope != nullptr && __builtin_amdgcn_readfirstlane(col0) < 2 * A;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = acc[i][j][r];
            const float partner = __shfl_xor(x, HALF);
            out[j][r] = x;
            if (rot) {
              const float2 cs = rope[(long)p[r] * HALF + jj];
              out[j][r] = lo ? (x * cs.x - partner * cs.y) : (x * cs.x + partner * cs.y);
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < Cfg::NB; ++j) {
        const int col = n0 + acc_col<Cfg>(wn, j, lane);
        const unsigned pc = (unsigned)((col & ~1) * sizeof(OutT));
        const bool cok = col < N;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float lo, hi;
          pair_rows(out[j][r], out[j][r + 1], odd, lo, hi);
          const int row = acc_row<Cfg>(wm, i, r, lane) + (odd ? 1 : 0);
          store_pair<OutT>(rc, cok ? pc + (unsigned)((long)row * ldc * sizeof(OutT)) : kOOB, lo, hi);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Fused gate/up + SwiGLU (pairs with RowsSwiGLU): block j < NB/2 holds gate
// features, block j + NB/2 the up features of the same columns.
// out[row, feat] = silu(gate) * up, feat = tn*(BN/2) + wn*(WN/2) + j*32 + lane.
// Branch-free stores through a buffer resource ending at row M.
// ---------------------------------------------------------------------------
template <typename OutT>
struct EpiSwiGLU {
  OutT *C; long ldc; int M, f;
  float *pre;   // optional: the pre-activations, gate at [row, feat] and up at [row, f + feat] (f32)
  template <class Cfg>
  __device__ __forceinline__ void apply(f32x16 (&acc)[Cfg::MB][Cfg::NB], int m0, int n0, int wm,
                                        int wn, int lane, int, char *, char *) const {
    constexpr int NBh = Cfg::NB / 2;
    const int tile_n = n0 / Cfg::BN;
    const long rows = M - m0 < Cfg::BM ? M - m0 : Cfg::BM;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C + (long)m0 * ldc, rows * ldc * (long)sizeof(OutT));
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc(pre != nullptr ? pre + (long)m0 * 2 * f : nullptr, pre != nullptr ? rows * 2L * f * 4 : 0);
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
      for (int j = 0; j < NBh; ++j) {
        const int feat = tile_n * (Cfg::BN / 2) + wn * (Cfg::WN / 2) + j * 32 + (lane & 31);
        const bool fok = feat < f;
        const bool odd = lane & 1;
        const unsigned pc = (unsigned)((feat & ~1) * sizeof(OutT));
        if (pre != nullptr) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const long row = acc_row<Cfg>(wm, i, r, lane);
            buf_store_elem(rp, fok ? (unsigned)((row * 2 * f + feat) * 4) : kOOB, acc[i][j][r], float{});
            buf_store_elem(rp, fok ? (unsigned)((row * 2 * f + f + feat) * 4) : kOOB, acc[i][j + NBh][r], float{});
          }
        }
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float g = acc[i][j][r], u = acc[i][j + NBh][r];
          v[r] = __fdividef(g, 1.f + __expf(-g)) * u;
        }
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float lo, hi;
          pair_rows(v[r], v[r + 1], odd, lo, hi);
          const int row = acc_row<Cfg>(wm, i, r, lane) + (odd ? 1 : 0);
          store_pair<OutT>(rc, fok ? pc + (unsigned)((long)row * ldc * sizeof(OutT)) : kOOB, lo, hi);
        }
      }
  }
};

// ---------------------------------------------------------------------------
// Reverse of SwiGLU on the recomputed gate/up products (pairs with
// DmaKMajorSwiGLU, as EpiSwiGLU): with gate g, up u and the incoming
// gradient dgsw[row, feat] of silu(g) u,
//   gsw[row, feat]       = silu(g) u                         (for dW_down)
//   dgu[row, feat]       = dgsw u silu'(g),  silu'(g) = sig(g) (1 + g (1 - sig(g)))
//   dgu[row, f + feat]   = dgsw silu(g)
// All three in bf16 (dgu feeds the dy and dW_gate / dW_up products).
// swiglu_bwd_elem (common.hpp) is the per-element arithmetic, shared with
// the kernel that reads saved pre-activations instead (the same values, bit
// for bit).
// ---------------------------------------------------------------------------
template <typename OutT>
struct EpiSwiGLUBwd {
  const OutT *dgsw; OutT *gsw; OutT *dgu; int M, f;
  template <class Cfg>
  __device__ __forceinline__ void apply(f32x16 (&acc)[Cfg::MB][Cfg::NB], int m0, int n0, int wm,
                                        int wn, int lane, int, char *, char *) const {
    constexpr int NBh = Cfg::NB / 2;
    const int tile_n = n0 / Cfg::BN;
    const long rows = M - m0 < Cfg::BM ? M - m0 : Cfg::BM;
    const long ldg = f, ldd = 2L * f;
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(dgsw + (long)m0 * ldg, rows * ldg * (long)sizeof(OutT));
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gsw + (long)m0 * ldg, rows * ldg * (long)sizeof(OutT));
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dgu + (long)m0 * ldd, rows * ldd * (long)sizeof(OutT));
    const bool odd = lane & 1;
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
      for (int j = 0; j < NBh; ++j) {
        const int feat = tile_n * (Cfg::BN / 2) + wn * (Cfg::WN / 2) + j * 32 + (lane & 31);
        const bool fok = feat < f;
        float vs[16], vg[16], vu[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row<Cfg>(wm, i, r, lane);
          const float dg_in =
              buf_load_elem(rin, fok ? (unsigned)(((long)row * ldg + feat) * sizeof(OutT)) : kOOB, OutT{});
          swiglu_bwd_elem(acc[i][j][r], acc[i][j + NBh][r], dg_in, vs[r], vg[r], vu[r]);
        }
        const unsigned pc = (unsigned)((feat & ~1) * sizeof(OutT));
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int row = acc_row<Cfg>(wm, i, r, lane) + (odd ? 1 : 0);
          float lo, hi;
          pair_rows(vs[r], vs[r + 1], odd, lo, hi);
          store_pair<OutT>(rg, fok ? pc + (unsigned)((long)row * ldg * sizeof(OutT)) : kOOB, lo, hi);
          pair_rows(vg[r], vg[r + 1], odd, lo, hi);
          store_pair<OutT>(rd, fok ? pc + (unsigned)((long)row * ldd * sizeof(OutT)) : kOOB, lo, hi);
          pair_rows(vu[r], vu[r + 1], odd, lo, hi);
          store_pair<OutT>(rd, fok ? pc + (unsigned)(((long)row * ldd + f) * sizeof(OutT)) : kOOB, lo, hi);
        }
      }
  }
};

// ---------------------------------------------------------------------------
// Linear-CE forward, one BM x BN tile of logits z = x_hat W^T: per row, the
// tile's max m_t and s_t = sum exp(z - m_t) over its valid columns go to
// part[row * nt + tile_n] (float2), and the target logit z[row, label[row]]
// to target[row] when the label falls in this tile.  The fp32 logits are also
// stored to zout [M, V] for the backward (softmax - onehot needs the row's
// final log-sum-exp, known only after every vocabulary tile).  Reductions go
// through LDS (the staging buffers are free after the main loop).  Logit and
// label accesses go through buffer resources ending at row M (branch-free);
// the target store is skipped by the whole wave when no lane holds a label
// column.  Requires BM * V * 4 < 2^31 (checked by the caller).
//
// ZT = float keeps the logits as they are.  ZT = _Float16 keeps z - m_t, the
// logit relative to its tile's row max (<= 0; part[] holds m_t), in half
// precision: half the bytes, with a rounding error of at most 2^-11 |z - m_t|
// (exact near the max, where the softmax weight is).
// ---------------------------------------------------------------------------
template <typename ZT>
struct EpiCEFwd {
  const int *labels; float2 *part; float *target; ZT *zout; int M, V, nt;
  template <class Cfg>
  __device__ __forceinline__ void apply(f32x16 (&acc)[Cfg::MB][Cfg::NB], int m0, int n0, int wm,
                                        int wn, int lane, int, char *lds, char *) const {
    // The 32 lanes of a half-wave hold one row (per accumulator register) in
    // 32 different columns: reduce across them with lane shuffles, then over
    // the WGN = 2 column waves through LDS ([WGN][BM] floats per quantity).
    static_assert(Cfg::WGN == 2, "two column waves per row");
    float *redm = reinterpret_cast<float *>(lds);          // [2][BM] row max per column wave
    float *reds = redm + 2 * Cfg::BM;                        // [2][BM] row sum-exp per column wave
    const bool writer = (lane & 31) == 31;                   // holds the half-wave reductions
    const bool odd = lane & 1;
    const long rows = M - m0 < Cfg::BM ? M - m0 : Cfg::BM;
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(zout + (long)m0 * V, rows * V * (long)sizeof(ZT));
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(labels + m0, rows * 4L);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(target + m0, rows * 4L);
    int col[Cfg::NB];
    bool cok[Cfg::NB];
#pragma unroll
    for (int j = 0; j < Cfg::NB; ++j) {
      col[j] = n0 + acc_col<Cfg>(wn, j, lane);
      cok[j] = col[j] < V;
    }
    // 1) row max over this wave's columns
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < Cfg::NB; ++j) mx = cok[j] ? fmaxf(mx, acc[i][j][r]) : mx;
        mx = halfwave_reduce<true>(mx);
        if (writer) redm[wn * Cfg::BM + acc_row<Cfg>(wm, i, r, lane)] = mx;
      }
    __syncthreads();
    // 2) sum of exp(z - m_row) over this wave's columns; target logit; logits
    //    (two rows at a time for the lane-pair stores)
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float zs[2][Cfg::NB];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rr = acc_row<Cfg>(wm, i, r + h, lane);
          const float mt = fmaxf(redm[rr], redm[Cfg::BM + rr]);
          const float nm = -mt * kLog2e;
          const int lab0 = (int)__builtin_amdgcn_raw_buffer_load_b32(rl, (unsigned)(rr * 4), 0, 0);
          const int lab = rr < rows ? lab0 : -1;
          float sum = 0.f, tv = 0.f;
          bool has = false;
#pragma unroll
          for (int j = 0; j < Cfg::NB; ++j) {
            const float z = acc[i][j][r + h];
            sum += cok[j] ? __builtin_amdgcn_exp2f(fmaf(z, kLog2e, nm)) : 0.f;
            zs[h][j] = sizeof(ZT) == 4 ? z : z - mt;
            const bool hit = col[j] == lab;
            tv = hit ? z : tv;
            has = has || hit;
          }
          if (__builtin_amdgcn_ballot_w64(has) != 0)
            buf_store_elem(rt, has ? (unsigned)(rr * 4) : kOOB, tv, float{});
          sum = halfwave_reduce<false>(sum);
          if (writer) reds[wn * Cfg::BM + rr] = sum;
        }
        if constexpr (sizeof(ZT) == 2) {
          const int row = acc_row<Cfg>(wm, i, r, lane) + (odd ? 1 : 0);
#pragma unroll
          for (int j = 0; j < Cfg::NB; ++j) {
            float lo, hi;
            pair_rows(zs[0][j], zs[1][j], odd, lo, hi);
            const unsigned zoff = cok[j] ? (unsigned)(((long)row * V + (col[j] & ~1)) * sizeof(ZT)) : kOOB;
            store_pair<ZT>(rz, zoff, lo, hi);
          }
        } else {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int row = acc_row<Cfg>(wm, i, r + h, lane);
#pragma unroll
            for (int j = 0; j < Cfg::NB; ++j)
              buf_store_elem(rz, cok[j] ? (unsigned)(((long)row * V + col[j]) * 4) : kOOB, zs[h][j], float{});
          }
        }
      }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < Cfg::BM && m0 + t < M)
      part[(long)(m0 + t) * nt + n0 / Cfg::BN] =
          make_float2(fmaxf(redm[t], redm[Cfg::BM + t]), reds[t] + reds[Cfg::BM + t]);
  }
};

// ---------------------------------------------------------------------------
// Linear-CE forward on the transposed tile: one BM x BN tile of z^T = W x_hat^T
// (vocabulary ids on rows, the slab's rows -- "tokens" -- on columns), so that
// the shared head W is the pair-row A operand and x_hat^T the MN-major B
// operand (both move in whole 128-byte lines).  Per token column: the tile's
// max m_t and s_t = sum exp(z - m_t) over its valid vocabulary rows go to
// part[token * nt + tile_m] (float2), the target logit to target[token] when
// the label falls in this tile, and the fp16 offsets z - m_t to zout[token, v]
// (staged through LDS per column block, then 16-byte stores along each token's
// row; direct 8-byte stores from the accumulators took twice as long).  A
// tile whose vocabulary rows all lie below M skips the row checks.  A lane
// holds one token column and 16 vocabulary rows per block; the 32 rows of a
// block pair live in lanes l and l ^ 32, and the WGM row waves meet through
// LDS (2 x WGM x BN floats).
// Requires BN * V * 2 < 2^31 and V % 4 == 0 (checked by the caller).
// ---------------------------------------------------------------------------
struct EpiCEFwdT {
  const int *labels; float2 *part; float *target; _Float16 *zout; int M, V, ntok, nt;
  // stage: 64 token rows x 256 ids of fp16 (32 KB) for the coalesced logit stores
  template <class Cfg>
  __device__ __forceinline__ void apply(f32x16 (&acc)[Cfg::MB][Cfg::NB], int m0, int n0, int wm,
                                        int wn, int lane, int, char *lds, char *stage) const {
    static_assert(Cfg::BM == 256 && Cfg::WGN == 2, "staged stores assume 256 ids and two column waves");
    float *redm = reinterpret_cast<float *>(lds);          // [WGM][BN] column max per row wave
    float *reds = redm + Cfg::WGM * Cfg::BN;               // [WGM][BN] column sum-exp per row wave
    const int hl = lane >> 5, c32 = lane & 31;
    const long cols = ntok - n0 < Cfg::BN ? ntok - n0 : Cfg::BN;
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(labels + n0, cols * 4L);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(target + n0, cols * 4L);
    // a tile whose vocabulary rows all lie below M needs no row checks
    const bool full = m0 + Cfg::BM <= M;
    // 1) column max over this wave's rows
#pragma unroll
    for (int j = 0; j < Cfg::NB; ++j) {
      float mx = -INFINITY;
      if (full) {
#pragma unroll
        for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
      } else {
#pragma unroll
        for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            mx = m0 + acc_row<Cfg>(wm, i, r, lane) < M ? fmaxf(mx, acc[i][j][r]) : mx;
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (hl == 0) redm[wm * Cfg::BN + acc_col<Cfg>(wn, j, lane)] = mx;
    }
    __syncthreads();
    // 2) per column: the tile max, sum of exp(z - m_t), the target logit
    float mtj[Cfg::NB];
#pragma unroll
    for (int j = 0; j < Cfg::NB; ++j) {
      const int col = acc_col<Cfg>(wn, j, lane);
      float mt = redm[col];
#pragma unroll
      for (int w = 1; w < Cfg::WGM; ++w) mt = fmaxf(mt, redm[w * Cfg::BN + col]);
      mtj[j] = mt;
      const float nm = -mt * kLog2e;
      const int lab0 = (int)__builtin_amdgcn_raw_buffer_load_b32(rl, (unsigned)(col * 4), 0, 0);
      // the label's row relative to this wave's first row, if it is one of this lane's
      const int rel = (col < cols ? lab0 : -1) - (m0 + wm * Cfg::WM);
      float sum = 0.f, tv = 0.f;
      if (full) {
#pragma unroll
        for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int vr = i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const float z = acc[i][j][r];
            sum += __builtin_amdgcn_exp2f(fmaf(z, kLog2e, nm));
            tv = vr == rel ? z : tv;
          }
      } else {
#pragma unroll
        for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int vr = i * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const float z = acc[i][j][r];
            sum += m0 + wm * Cfg::WM + vr < M ? __builtin_amdgcn_exp2f(fmaf(z, kLog2e, nm)) : 0.f;
            tv = vr == rel ? z : tv;
          }
      }
      const bool has = rel >= 0 && rel < Cfg::WM && ((rel >> 2) & 1) == hl;
      if (__builtin_amdgcn_ballot_w64(has) != 0) buf_store_elem(rt, has ? (unsigned)(col * 4) : kOOB, tv, float{});
      sum += __shfl_xor(sum, 32);
      if (hl == 0) reds[wm * Cfg::BN + col] = sum;
    }
    // 3) logits as fp16 offsets z - m_t: per column block j, the 64 token rows
    //    of both column waves staged in LDS (8-byte unit u of token row t at
    //    u ^ (t & 63): a half-wave's 32 rows hit distinct banks), then copied
    //    out in 16-byte chunks along each token's row
    const int nthr = Cfg::NT;
#pragma unroll
    for (int j = 0; j < Cfg::NB; ++j) {
      __syncthreads();
      const int tl = wn * 32 + c32;                          // token row in the stage
#pragma unroll
      for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          const h4 hv = {(_Float16)(acc[i][j][4 * q] - mtj[j]), (_Float16)(acc[i][j][4 * q + 1] - mtj[j]),
                         (_Float16)(acc[i][j][4 * q + 2] - mtj[j]), (_Float16)(acc[i][j][4 * q + 3] - mtj[j])};
          const int u = (wm * Cfg::WM + i * 32 + 8 * q + 4 * hl) >> 2;   // 8-byte unit of the id row
          *reinterpret_cast<h4 *>(stage + tl * 512 + ((u ^ (tl & 63)) << 3)) = hv;
        }
      __syncthreads();
      for (int c = threadIdx.x; c < 64 * 32; c += nthr) {
        const int row = c >> 5, cu = (c & 31) * 2;             // token row, first 8-byte unit
        const int tok = n0 + (row >> 5) * Cfg::WN + j * 32 + (row & 31);
        const int v = m0 + cu * 4;
        if (tok >= ntok || v >= M) continue;
        const uint2 lo = *reinterpret_cast<const uint2 *>(stage + row * 512 + ((cu ^ (row & 63)) << 3));
        const uint2 hi = *reinterpret_cast<const uint2 *>(stage + row * 512 + (((cu + 1) ^ (row & 63)) << 3));
        *reinterpret_cast<uint4 *>(zout + (long)tok * V + v) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < Cfg::BN && n0 + t < ntok) {
      float mt = redm[t], st = reds[t];
#pragma unroll
      for (int w = 1; w < Cfg::WGM; ++w) {
        mt = fmaxf(mt, redm[w * Cfg::BN + t]);
        st += reds[w * Cfg::BN + t];
      }
      part[(long)(n0 + t) * nt + m0 / Cfg::BM] = make_float2(mt, st);
    }
  }
};

// Whether a loader stages its operand in 128-byte pair rows.
template <class L, class = void>
struct PairRows : std::false_type {};
template <class L>
struct PairRows<L, std::void_t<decltype(L::kPairRows)>> : std::bool_constant<L::kPairRows> {};

// One BM x BN tile, K slices [kt0, kt0 + nk), into acc.
template <typename T, class Cfg, class LA, class LB>
__device__ __forceinline__ void gemm_segment(const LA &la, const LB &lb, int m0, int n0, int kt0, int nk, int K,
                                             char *const *r0, char *const *r1, f32x16 (&acc)[Cfg::MB][Cfg::NB]) {
  if constexpr (PairRows<LA>::value) gemm_mainloop_pairs<T, Cfg>(la, lb, m0, n0, kt0, nk, K, r0, r1, acc);
  else gemm_mainloop<T, Cfg>(la, lb, m0, n0, kt0, nk, K, r0, acc);
}

// LDS of one GEMM block: the pair-row layout (3 A regions of BM x 128 bytes,
// 4 B stages of BNL x 64 bytes) or NS stages of (BM + BN) x 64 bytes.  An
// epilogue may use the first two regions as scratch once the main loop has
// returned.
#define MTP_GEMM_LDS(Cfg, LA)                                                                   \
  char *r0[PairRows<LA>::value ? 3 : Cfg::NS];                                                  \
  char *r1[4];                                                                                  \
  if constexpr (PairRows<LA>::value) {                                                          \
    __shared__ __attribute__((aligned(1024))) char a0[Cfg::BM * 128], a1[Cfg::BM * 128],        \
        a2[Cfg::BM * 128];                                                                      \
    __shared__ __attribute__((aligned(1024))) char b0[Cfg::BNL * 64], b1[Cfg::BNL * 64],        \
        b2[Cfg::BNL * 64], b3[Cfg::BNL * 64];                                                   \
    r0[0] = a0; r0[1] = a1; r0[2] = a2;                                                         \
    r1[0] = b0; r1[1] = b1; r1[2] = b2; r1[3] = b3;                                             \
  } else {                                                                                      \
    __shared__ __attribute__((aligned(1024))) char st0[Cfg::LDS_STAGE], st1[Cfg::LDS_STAGE],    \
        st2[Cfg::LDS_STAGE], st3[Cfg::LDS_STAGE];                                               \
    r0[0] = st0; r0[1] = st1; r0[2] = st2; r0[3] = st3;                                         \
    if constexpr (Cfg::NS >= 5) {                                                               \
      __shared__ __attribute__((aligned(1024))) char st4[Cfg::LDS_STAGE];                       \
      r0[4] = st4;                                                                              \
    }                                                                                           \
    if constexpr (Cfg::NS >= 6) {                                                               \
      __shared__ __attribute__((aligned(1024))) char st5[Cfg::LDS_STAGE];                       \
      r0[5] = st5;                                                                              \
    }                                                                                           \
    if constexpr (Cfg::NS >= 7) {                                                               \
      __shared__ __attribute__((aligned(1024))) char st6[Cfg::LDS_STAGE];                       \
      r0[6] = st6;                                                                              \
    }                                                                                           \
    if constexpr (Cfg::NS >= 8) {                                                               \
      __shared__ __attribute__((aligned(1024))) char st7[Cfg::LDS_STAGE];                       \
      r0[7] = st7;                                                                              \
    }                                                                                           \
  }

// Floats of one partial tile (the block's accumulators).
template <class Cfg>
constexpr long partial_floats() { return (long)Cfg::MB * Cfg::NB * 16 * Cfg::NT; }

// Partial tiles are kept in the accumulator layout: float4 q of thread t at
// slot[(q * NT + t) * 4], so each wave moves 1 KB per instruction.
template <class Cfg>
__device__ __forceinline__ void store_partial(float *slot, const f32x16 (&acc)[Cfg::MB][Cfg::NB]) {
  float4 *p = reinterpret_cast<float4 *>(slot) + threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::NB; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int q = (i * Cfg::NB + j) * 4 + c;
        p[q * Cfg::NT] = make_float4(acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2],
                                     acc[i][j][4 * c + 3]);
      }
}
template <class Cfg>
__device__ __forceinline__ void add_partial(const float *slot, f32x16 (&acc)[Cfg::MB][Cfg::NB]) {
  const float4 *p = reinterpret_cast<const float4 *>(slot) + threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::NB; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 v = p[((i * Cfg::NB + j) * 4 + c) * Cfg::NT];
        acc[i][j][4 * c] += v.x;
        acc[i][j][4 * c + 1] += v.y;
        acc[i][j][4 * c + 2] += v.z;
        acc[i][j][4 * c + 3] += v.w;
      }
}

// One block per tile and K split.  The launch covers tiles [tile0, tile0 +
// ntiles) of the grouped raster order, split-major (blocks that run together
// share a K range and neighbouring tiles).  Without ws each block hands its
// accumulators to the epilogue (K splits then write separate output slabs);
// with ws it stores them as an fp32 partial tile, slot split * ntiles + tile,
// for gemm_fixup_kernel.
template <typename T, class Cfg, class LA, class LB, class Epi>
__global__ __launch_bounds__(Cfg::NT) void gemm_kernel(LA la, LB lb, Epi epi, int K, TileSched ts) {
  constexpr int BK = 4 * Elem<T>::kPerChunk;
  MTP_GEMM_LDS(Cfg, LA)
  const int logical = xcd_remap(blockIdx.x, ts.ntiles * ts.k_splits);
  const int split = logical / ts.ntiles;
  const int tl = logical - split * ts.ntiles;
  int tm, tn;
  tile_coords(ts.tile0 + tl, ts.mt, ts.nt, ts.group_m, tm, tn);
  const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;
  const int nk_total = (K + BK - 1) / BK;
  int per = (nk_total + ts.k_splits - 1) / ts.k_splits;
  if constexpr (PairRows<LA>::value) per += per & 1;   // K splits start on a pair
  const int kt0 = split * per;
  const int kt1 = min(nk_total, kt0 + per);
  const int nk = kt1 > kt0 ? kt1 - kt0 : 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x16 acc[Cfg::MB][Cfg::NB];
  gemm_segment<T, Cfg>(la, lb, m0, n0, kt0, nk, K, r0, r1, acc);
  if (ts.ws != nullptr) {
    store_partial<Cfg>(ts.ws + ((long)split * ts.ntiles + tl) * partial_floats<Cfg>(), acc);
    return;
  }
  epi.template apply<Cfg>(acc, m0, n0, wave / Cfg::WGN, wave % Cfg::WGN, lane, split, r0[0], r0[1]);
}

// Block b sums the k_splits partial tiles of tile tile0 + b and runs the
// epilogue on the sum.
template <class Cfg, class Epi>
__global__ __launch_bounds__(Cfg::NT) void gemm_fixup_kernel(Epi epi, TileSched ts) {
  __shared__ __attribute__((aligned(16))) char lds[2 * Cfg::WGM * (Cfg::BM > Cfg::BN ? Cfg::BM : Cfg::BN) * sizeof(float)];
  // a second region for epilogues that stage their stores (32 KB)
  __shared__ __attribute__((aligned(16))) char lds2[std::is_same_v<Epi, EpiCEFwdT> ? 32768 : 16];
  const int tl = blockIdx.x;
  int tm, tn;
  tile_coords(ts.tile0 + tl, ts.mt, ts.nt, ts.group_m, tm, tn);
  f32x16 acc[Cfg::MB][Cfg::NB];
#pragma unroll
  for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int sp = 0; sp < ts.k_splits; ++sp)
    add_partial<Cfg>(ts.ws + ((long)sp * ts.ntiles + tl) * partial_floats<Cfg>(), acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  epi.template apply<Cfg>(acc, tm * Cfg::BM, tn * Cfg::BN, wave / Cfg::WGN, wave % Cfg::WGN, lane, 0, lds,
                          lds2);
}

// Host-side launch helpers.  launch_gemm: every tile, K split k_splits ways,
// each split through the epilogue.
template <typename T, class Cfg, class LA, class LB, class Epi>
inline hipError_t launch_gemm(const LA &la, const LB &lb, const Epi &epi, int M, int N, int K,
                              int group_m, int k_splits, hipStream_t stream) {
  TileSched ts;
  ts.mt = (M + Cfg::BM - 1) / Cfg::BM;
  ts.nt = (N + Cfg::BN - 1) / Cfg::BN;
  ts.group_m = group_m < 1 ? 1 : (group_m > ts.mt ? ts.mt : group_m);
  ts.k_splits = k_splits < 1 ? 1 : k_splits;
  ts.tile0 = 0;
  ts.ntiles = ts.mt * ts.nt;
  ts.ws = nullptr;
  const long blocks = (long)ts.ntiles * ts.k_splits;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<T, Cfg, LA, LB, Epi>), dim3((unsigned)blocks), dim3(Cfg::NT), 0, stream, la,
                     lb, epi, K, ts);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Balanced launch for tiles that take a whole compute unit each (kGemmSlots
// blocks resident at a time).  The tiles fill floor(T / G) whole rounds; the
// R = T mod G left over would leave the last round partly idle, so they are
// split s ways over K (s chosen so that R * s fills whole rounds best),
// stored as partial tiles and summed by gemm_fixup_kernel, which runs the
// epilogue once per tile.
// ---------------------------------------------------------------------------
constexpr int kGemmSlots = 256;
constexpr int kTailSlots = 3 * kGemmSlots;      // partial tiles of the tail at most

template <class Cfg>
constexpr size_t tail_ws_bytes() { return (size_t)kTailSlots * partial_floats<Cfg>() * sizeof(float); }

// K splits for R tail tiles of nk slices: the fewest rounds per unit of
// work, if that beats one unsplit round.
inline int tail_splits(long R, int nk) {
  if (R <= 0) return 1;
  int best = 1;
  double best_t = 1.0;
  for (int s = 2; s <= 8; ++s) {
    if (R * s > kTailSlots || 2 * s > nk) break;
    const double t = (double)((R * s + kGemmSlots - 1) / kGemmSlots) / s;
    if (t < best_t - 1e-9) { best_t = t; best = s; }
  }
  return best;
}

template <typename T, class Cfg, class LA, class LB, class Epi>
inline hipError_t launch_gemm_balanced(const LA &la, const LB &lb, const Epi &epi, int M, int N, int K,
                                       int group_m, float *ws, hipStream_t stream) {
  constexpr int BK = 4 * Elem<T>::kPerChunk;
  TileSched ts;
  ts.mt = (M + Cfg::BM - 1) / Cfg::BM;
  ts.nt = (N + Cfg::BN - 1) / Cfg::BN;
  ts.group_m = group_m < 1 ? 1 : (group_m > ts.mt ? ts.mt : group_m);
  const long ntiles = (long)ts.mt * ts.nt;
  if (ntiles <= 0) return hipSuccess;
  const long R = ntiles % kGemmSlots;
  const int s = ws == nullptr ? 1 : tail_splits(R, (K + BK - 1) / BK);
  // whole rounds (every tile if the tail is not split)
  ts.k_splits = 1;
  ts.tile0 = 0;
  ts.ntiles = (int)(s > 1 ? ntiles - R : ntiles);
  ts.ws = nullptr;
  if (ts.ntiles > 0) {
    hipLaunchKernelGGL((gemm_kernel<T, Cfg, LA, LB, Epi>), dim3((unsigned)ts.ntiles), dim3(Cfg::NT), 0, stream,
                       la, lb, epi, K, ts);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (s == 1) return hipSuccess;
  ts.k_splits = s;
  ts.tile0 = (int)(ntiles - R);
  ts.ntiles = (int)R;
  ts.ws = ws;
  hipLaunchKernelGGL((gemm_kernel<T, Cfg, LA, LB, Epi>), dim3((unsigned)(R * s)), dim3(Cfg::NT), 0, stream, la,
                     lb, epi, K, ts);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_fixup_kernel<Cfg, Epi>), dim3((unsigned)R), dim3(Cfg::NT), 0, stream, epi, ts);
  return hipGetLastError();
}

}  // namespace mtp
