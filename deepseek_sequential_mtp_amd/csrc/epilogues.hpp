// GEMM epilogues.  Each receives the wave's accumulators acc[MB][NB] in the
// 32x32 MFMA result layout (lane l, register r -> row 8*(r/4)+4*(l/32)+r%4,
// column l%32 of block (i, j)) plus the tile origin.
#pragma once

#include <type_traits>

#include "gemm.hpp"

namespace mtp {

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
#pragma unroll
        for (int r = 0; r < 16; ++r) buf_store_elem(rc, oc[r], v[r], OutT{});
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
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i) {
      int p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p[r] = (int)__builtin_amdgcn_raw_buffer_load_b32(rp, (unsigned)(acc_row<Cfg>(wm, i, r, lane) * 4), 0, 0);
#pragma unroll
      for (int j = 0; j < Cfg::NB; ++j) {
        const int col = n0 + acc_col<Cfg>(wn, j, lane);
        const int jh = col % HD;
        const bool lo = jh < HALF;
        const int jj = lo ? jh : jh - HALF;
        // 2A is a multiple of 32: the whole block column is q/k or v
        const int col0 = n0 + acc_col<Cfg>(wn, j, 0);
        const bool rot = rope != nullptr && __builtin_amdgcn_readfirstlane(col0) < 2 * A;
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = acc[i][j][r];
          float partner;
          if constexpr (HALF >= 32) {
            constexpr int PB = HALF / 32;
            partner = acc[i][j ^ PB][r];
          } else {
            partner = __shfl_xor(x, HALF);
          }
          v[r] = x;
          if (rot) {
            const float2 cs = rope[(long)p[r] * HALF + jj];
            v[r] = lo ? (x * cs.x - partner * cs.y) : (x * cs.x + partner * cs.y);
          }
        }
        const bool cok = col < N;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = acc_row<Cfg>(wm, i, r, lane);
          buf_store_elem(rc, cok ? (unsigned)(((long)rl * ldc + col) * sizeof(OutT)) : kOOB, v[r], OutT{});
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
  template <class Cfg>
  __device__ __forceinline__ void apply(f32x16 (&acc)[Cfg::MB][Cfg::NB], int m0, int n0, int wm,
                                        int wn, int lane, int, char *, char *) const {
    constexpr int NBh = Cfg::NB / 2;
    const int tile_n = n0 / Cfg::BN;
    const long rows = M - m0 < Cfg::BM ? M - m0 : Cfg::BM;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(C + (long)m0 * ldc, rows * ldc * (long)sizeof(OutT));
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
      for (int j = 0; j < NBh; ++j) {
        const int feat = tile_n * (Cfg::BN / 2) + wn * (Cfg::WN / 2) + j * 32 + (lane & 31);
        const bool fok = feat < f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = acc_row<Cfg>(wm, i, r, lane);
          const float g = acc[i][j][r], u = acc[i][j + NBh][r];
          const float sw = __fdividef(g, 1.f + __expf(-g));
          buf_store_elem(rc, fok ? (unsigned)(((long)rl * ldc + feat) * sizeof(OutT)) : kOOB, sw * u, OutT{});
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
// ---------------------------------------------------------------------------
struct EpiCEFwd {
  const int *labels; float2 *part; float *target; float *zout; int M, V, nt;
  template <class Cfg>
  __device__ __forceinline__ void apply(f32x16 (&acc)[Cfg::MB][Cfg::NB], int m0, int n0, int wm,
                                        int wn, int lane, int, char *lds, char *) const {
    // The 32 lanes of a half-wave hold one row (per accumulator register) in
    // 32 different columns: reduce across them with lane shuffles, then over
    // the WGN = 2 column waves through LDS ([WGN][BM] floats per quantity).
    static_assert(Cfg::WGN == 2, "two column waves per row");
    float *redm = reinterpret_cast<float *>(lds);          // [2][BM] row max per column wave
    float *reds = redm + 2 * Cfg::BM;                        // [2][BM] row sum-exp per column wave
    const bool writer = (lane & 31) == 0;
    const long rows = M - m0 < Cfg::BM ? M - m0 : Cfg::BM;
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(zout + (long)m0 * V, rows * V * 4L);
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
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        if (writer) redm[wn * Cfg::BM + acc_row<Cfg>(wm, i, r, lane)] = mx;
      }
    __syncthreads();
    // 2) sum of exp(z - m_row) over this wave's columns; target logit; logits
#pragma unroll
    for (int i = 0; i < Cfg::MB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = acc_row<Cfg>(wm, i, r, lane);
        const float nm = -fmaxf(redm[rr], redm[Cfg::BM + rr]) * kLog2e;
        const int lab0 = (int)__builtin_amdgcn_raw_buffer_load_b32(rl, (unsigned)(rr * 4), 0, 0);
        const int lab = rr < rows ? lab0 : -1;
        float s = 0.f, tv = 0.f;
        bool has = false;
#pragma unroll
        for (int j = 0; j < Cfg::NB; ++j) {
          const float z = acc[i][j][r];
          s += cok[j] ? __builtin_amdgcn_exp2f(fmaf(z, kLog2e, nm)) : 0.f;
          buf_store_elem(rz, cok[j] ? (unsigned)(((long)rr * V + col[j]) * 4) : kOOB, z, float{});
          const bool hit = col[j] == lab;
          tv = hit ? z : tv;
          has = has || hit;
        }
        if (__builtin_amdgcn_ballot_w64(has) != 0)
          buf_store_elem(rt, has ? (unsigned)(rr * 4) : kOOB, tv, float{});
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if (writer) reds[wn * Cfg::BM + rr] = s;
      }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < Cfg::BM && m0 + t < M)
      part[(long)(m0 + t) * nt + n0 / Cfg::BN] =
          make_float2(fmaxf(redm[t], redm[Cfg::BM + t]), reds[t] + reds[Cfg::BM + t]);
  }
};

// Whether a loader stages its operand in 128-byte pair rows.
template <class L, class = void>
struct PairRows : std::false_type {};
template <class L>
struct PairRows<L, std::void_t<decltype(L::kPairRows)>> : std::bool_constant<L::kPairRows> {};

template <typename T, class Cfg, class LA, class LB, class Epi>
__global__ __launch_bounds__(Cfg::NT) void gemm_kernel(LA la, LB lb, Epi epi, int K, TileSched ts) {
  if constexpr (PairRows<LA>::value) {
    __shared__ __attribute__((aligned(1024))) char a0[Cfg::BM * 128];
    __shared__ __attribute__((aligned(1024))) char a1[Cfg::BM * 128];
    __shared__ __attribute__((aligned(1024))) char a2[Cfg::BM * 128];
    __shared__ __attribute__((aligned(1024))) char b0[Cfg::BN * 64];
    __shared__ __attribute__((aligned(1024))) char b1[Cfg::BN * 64];
    __shared__ __attribute__((aligned(1024))) char b2[Cfg::BN * 64];
    __shared__ __attribute__((aligned(1024))) char b3[Cfg::BN * 64];
    char *const sa[3] = {a0, a1, a2};
    char *const sb[4] = {b0, b1, b2, b3};
    gemm_body_pairs<T, Cfg>(la, lb, epi, K, ts, sa, sb);
  } else {
    __shared__ __attribute__((aligned(1024))) char st0[Cfg::LDS_STAGE];
    __shared__ __attribute__((aligned(1024))) char st1[Cfg::LDS_STAGE];
    __shared__ __attribute__((aligned(1024))) char st2[Cfg::LDS_STAGE];
    __shared__ __attribute__((aligned(1024))) char st3[Cfg::LDS_STAGE];
    if constexpr (Cfg::NS == 5) {
      __shared__ __attribute__((aligned(1024))) char st4[Cfg::LDS_STAGE];
      char *const st[5] = {st0, st1, st2, st3, st4};
      gemm_body<T, Cfg>(la, lb, epi, K, ts, st);
    } else {
      char *const st[4] = {st0, st1, st2, st3};
      gemm_body<T, Cfg>(la, lb, epi, K, ts, st);
    }
  }
}

// Host-side launch helper (grid = tiles * K splits, one block per tile).
template <typename T, class Cfg, class LA, class LB, class Epi>
inline hipError_t launch_gemm(const LA &la, const LB &lb, const Epi &epi, int M, int N, int K,
                              int group_m, int k_splits, hipStream_t stream) {
  TileSched ts;
  ts.mt = (M + Cfg::BM - 1) / Cfg::BM;
  ts.nt = (N + Cfg::BN - 1) / Cfg::BN;
  ts.group_m = group_m < 1 ? 1 : (group_m > ts.mt ? ts.mt : group_m);
  ts.k_splits = k_splits < 1 ? 1 : k_splits;
  const long tiles = (long)ts.mt * ts.nt * ts.k_splits;
  if (tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<T, Cfg, LA, LB, Epi>), dim3((unsigned)tiles), dim3(Cfg::NT), 0,
                     stream, la, lb, epi, K, ts);
  return hipGetLastError();
}

}  // namespace mtp
