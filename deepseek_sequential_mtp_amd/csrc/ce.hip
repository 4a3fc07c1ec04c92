// Reductions of the fused linear cross-entropy (M7.6 0x05, 0x05A):
// merging the per-tile online log-sum-exp partials of each row, the per-depth
// loss sums and counts, the backward scale lambda / (D * denom_k), and the
// final L^(k) and L_MTP.  The vocabulary GEMMs themselves live in
// mtp_api.hip (GEMM core + CE epilogues).
#include "kernels.hpp"

namespace mtp {

// One wave per row: lse = M + log(sum_t s_t exp(m_t - M)) over the nt tile
// partials; row loss = lse - z[label] on labelled rows, else 0.  With pred
// (top-1 accuracy requested) the row maximum M is kept and pred is seeded
// with V on labelled rows (the softmax-gradient pass lowers it to the argmax)
// and -1 on the others.
__global__ __launch_bounds__(256) void ce_combine_kernel(const float2 *__restrict__ part, int nt,
                                                         const float *__restrict__ target,
                                                         const int32_t *__restrict__ labels,
                                                         float *__restrict__ lse, float *__restrict__ lse_out,
                                                         float *__restrict__ row_loss, float *__restrict__ rowmax,
                                                         int32_t *__restrict__ pred, int V, int N) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;
  const float2 *p = part + (long)row * nt;
  float mx = -INFINITY;
  for (int i = lane; i < nt; i += 64) mx = fmaxf(mx, p[i].x);
  mx = warp_max(mx);
  float s = 0.f;
  for (int i = lane; i < nt; i += 64) {
    const float2 v = p[i];
    s += v.y * expf(v.x - mx);
  }
  s = warp_sum(s);
  if (lane == 0) {
    const float l = mx + logf(s);
    lse[row] = l;
    if (lse_out != nullptr) lse_out[row] = l;
    const int lab = labels[row];
    row_loss[row] = lab >= 0 ? l - target[row] : 0.f;
    if (pred != nullptr) {
      rowmax[row] = mx;
      pred[row] = lab >= 0 ? V : -1;
    }
  }
}

// dz = softmax(z) - onehot(label) on labelled rows, 0 on the others, from the
// stored logits and the row's log-sum-exp; stored unscaled in T (the
// depth's scale lambda / (D * denom) is applied by the consuming GEMMs).
// The logits are either fp32 (ZT = float) or fp16 offsets z - m_t from the
// row max of their vocabulary tile (ZT = _Float16; m_t is the first member of
// part[row * nt + col / tile_cols]).  Each thread handles W consecutive
// columns of one tile, 16 bytes of kept logits (W = 8 fp16 offsets or 4
// fp32 logits; V is a multiple of W and the tile width of 8).
// With pred, the same pass finds each labelled row's argmax: a column is a
// maximum when its logit equals the row maximum rowmax (fp16 offsets: its
// tile's maximum is the row's and its offset is 0); atomicMin keeps the
// lowest such column.
constexpr int kDzChunksPerThread = 4;

template <typename T, typename ZT>
__global__ __launch_bounds__(256) void ce_dz_kernel(const ZT *__restrict__ z, const float2 *__restrict__ part,
                                                    int nt, int tile_cols, const float *__restrict__ lse,
                                                    const int32_t *__restrict__ labels, T *__restrict__ dz,
                                                    const float *__restrict__ rowmax, int32_t *__restrict__ pred,
                                                    int V, int N) {
  constexpr int W = 16 / (int)sizeof(ZT);
  constexpr int U = kDzChunksPerThread;
  // column blocks on x, rows on y (a row stride covers N > 65535); a thread
  // takes U chunks 256 apart, all loaded before any is used, so that U 16-byte
  // loads per thread are in flight
  for (long row = blockIdx.y; row < N; row += gridDim.y) {
    const int lab = labels[row];
    const float nl = -lse[row] * kLog2e;
    const float rmax = (pred != nullptr && lab >= 0) ? rowmax[row] : 0.f;
    const ZT *zr = z + row * V;
    T *dr = dz + row * V;
    for (int cw0 = blockIdx.x * 256 * U + threadIdx.x; cw0 < V / W; cw0 += gridDim.x * 256 * U) {
      float zz[U][W];
      if (lab >= 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int cw = cw0 + 256 * u;
          if (cw < V / W) {
            if constexpr (sizeof(ZT) == 4) {
              const float4 v = reinterpret_cast<const float4 *>(zr)[cw];
              zz[u][0] = v.x; zz[u][1] = v.y; zz[u][2] = v.z; zz[u][3] = v.w;
            } else {
              typedef _Float16 h8 __attribute__((ext_vector_type(8)));
              const h8 v = reinterpret_cast<const h8 *>(zr)[cw];
#pragma unroll
              for (int e = 0; e < W; ++e) zz[u][e] = (float)v[e];
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int cw = cw0 + 256 * u;
        if (cw >= V / W) break;
        float g[W];
#pragma unroll
        for (int e = 0; e < W; ++e) g[e] = 0.f;
        if (lab >= 0) {
          float off = nl;
          float top = rmax;            // the value a maximal column holds
          if constexpr (sizeof(ZT) == 2) {
            const float mt = part[row * nt + (W * cw) / tile_cols].x;
            off = fmaf(mt, kLog2e, nl);
            top = mt == rmax ? 0.f : 1.f;  // offsets are <= 0: 1 matches none
          }
          if (pred != nullptr) {
            int first = -1;
#pragma unroll
            for (int e = W - 1; e >= 0; --e) first = zz[u][e] == top ? W * cw + e : first;
            if (first >= 0) atomicMin(pred + row, first);
          }
          // softmax = 2^(z log2 e - lse log2 e): one FMA and the hardware exp2
          // (probabilities below 2^-126 flush to zero)
#pragma unroll
          for (int e = 0; e < W; ++e)
            g[e] = __builtin_amdgcn_exp2f(fmaf(zz[u][e], kLog2e, off)) - (W * cw + e == lab ? 1.f : 0.f);
        }
        if constexpr (sizeof(T) == 2 && W == 8) {
          reinterpret_cast<uint4 *>(dr)[cw] = f32_to_chunk(g, T{});
        } else {
#pragma unroll
          for (int q = 0; q < W; q += 4) store4(dr + W * cw + q, *reinterpret_cast<const float(*)[4]>(g + q));
        }
      }
    }
  }
}

// xT[c, r] = x[r, c] for an [R, C] bf16 matrix (C % 8 == 0); xT has leading
// dimension ldT >= R rounded up to 8 (the pad columns are written as 0).
// 64 x 64 tiles through LDS: 16-byte reads along C, 16-byte writes along R.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t *__restrict__ x, int R, int C,
                                                             bf16_t *__restrict__ xT, long ldT) {
  __shared__ uint16_t tile[64][64 + 2];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;   // row tiles on x (no 65535 limit)
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int rr = q >> 3, cc = (q & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < R && c < C) v = *reinterpret_cast<const uint4 *>(x + (long)r * C + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[rr][cc + 2 * e] = (uint16_t)(w[e] & 0xffffu);
      tile[rr][cc + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 512; q += 256) {
    const int cc = q >> 3, rr = (q & 7) * 8;
    const int c = c0 + cc, r = r0 + rr;
    if (c >= C || r >= ldT) continue;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = r + 2 * e < R ? tile[rr + 2 * e][cc] : 0u;
      const uint32_t hi = r + 2 * e + 1 < R ? tile[rr + 2 * e + 1][cc] : 0u;
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4 *>(xT + (long)c * ldT + r) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_transpose_bf16(const bf16_t *x, int R, int C, bf16_t *xT, long ldT, hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((R + 63) / 64, (C + 63) / 64), dim3(256), 0, s, x, R, C, xT, ldT);
  return hipGetLastError();
}

template <typename T, typename ZT>
hipError_t launch_ce_dz(const ZT *z, const float2 *part, int nt, int tile_cols, const float *lse,
                        const int32_t *labels, T *dz, const float *rowmax, int32_t *pred, int N, int V,
                        hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int per_block = 256 * kDzChunksPerThread;
  const int bx = min((V / (16 / (int)sizeof(ZT)) + per_block - 1) / per_block, 65535);
  hipLaunchKernelGGL((ce_dz_kernel<T, ZT>), dim3(bx, min(N, 65535)), dim3(256), 0, s, z, part, nt, tile_cols,
                     lse, labels, dz, rowmax, pred, V, N);
  return hipGetLastError();
}
template hipError_t launch_ce_dz<bf16_t, _Float16>(const _Float16 *, const float2 *, int, int, const float *,
                                                    const int32_t *, bf16_t *, const float *, int32_t *, int, int,
                                                    hipStream_t);
template hipError_t launch_ce_dz<float, float>(const float *, const float2 *, int, int, const float *,
                                               const int32_t *, float *, const float *, int32_t *, int, int,
                                               hipStream_t);

// One block: sum of the row losses of depth k (double, fixed order) and the
// count of labelled rows; scale[k] = lambda / (D * denom_k) for the backward
// (0 for an empty depth under the valid-row mean).  With row_loss = nullptr
// only the count and the scale are produced (they depend on the labels alone).
// With pred: the count of labelled rows whose argmax is the label goes to
// acc_correct[k], and pred is copied to pred_out when that is given.
__global__ __launch_bounds__(1024) void ce_reduce_kernel(const float *__restrict__ row_loss,
                                                         const int32_t *__restrict__ labels, int N, int k,
                                                         int D, int valid_mean, double denom, float lambda,
                                                         double *acc_sum, int32_t *acc_cnt, float *scale,
                                                         const int32_t *__restrict__ pred,
                                                         int32_t *__restrict__ pred_out, int32_t *acc_correct) {
  __shared__ double shs[16];
  __shared__ int shc[16], shh[16];
  const int t = threadIdx.x;
  double s = 0.0;
  int c = 0, hits = 0;
  for (int i = t; i < N; i += 1024) {
    if (row_loss != nullptr) s += (double)row_loss[i];
    const int lab = labels[i];
    c += lab >= 0 ? 1 : 0;
    if (pred != nullptr) {
      const int p = pred[i];
      hits += (lab >= 0 && p == lab) ? 1 : 0;
      if (pred_out != nullptr) pred_out[i] = p;
    }
  }
  s = warp_sum(s);
  for (int o = 32; o > 0; o >>= 1) {
    c += __shfl_xor(c, o);
    hits += __shfl_xor(hits, o);
  }
  if ((t & 63) == 0) { shs[t >> 6] = s; shc[t >> 6] = c; shh[t >> 6] = hits; }
  __syncthreads();
  if (t == 0) {
    double ts = 0.0;
    int tc = 0, th = 0;
    for (int w = 0; w < 16; ++w) { ts += shs[w]; tc += shc[w]; th += shh[w]; }
    if (row_loss != nullptr) acc_sum[k] = ts;
    if (pred != nullptr) acc_correct[k] = th;
    acc_cnt[k] = tc;
    const double den = valid_mean ? (double)tc : denom;
    scale[k] = den > 0.0 ? (float)((double)lambda / ((double)D * den)) : 0.f;
  }
}

__global__ void ce_finalize_kernel(const double *acc_sum, const int32_t *acc_cnt, int D, int valid_mean,
                                   double denom, float lambda, float *loss_sum, int32_t *counts,
                                   float *loss, float *loss_mtp, const int32_t *acc_correct, int32_t *correct,
                                   float *accuracy) {
  if (threadIdx.x != 0) return;
  double total = 0.0;
  for (int k = 0; k < D; ++k) {
    const double den = valid_mean ? (double)acc_cnt[k] : denom;
    const double lk = den > 0.0 ? acc_sum[k] / den : 0.0;
    loss_sum[k] = (float)acc_sum[k];
    counts[k] = acc_cnt[k];
    loss[k] = (float)lk;
    total += lk;
    if (correct != nullptr) correct[k] = acc_correct[k];
    if (accuracy != nullptr)
      accuracy[k] = acc_cnt[k] > 0 ? (float)((double)acc_correct[k] / (double)acc_cnt[k]) : 0.f;
  }
  loss_mtp[0] = (float)((double)lambda / D * total);
}

hipError_t launch_ce_combine(const float2 *part, int nt, const float *target, const int32_t *labels,
                             float *lse, float *lse_out, float *row_loss, float *rowmax, int32_t *pred, int V,
                             int N, hipStream_t s) {
  hipLaunchKernelGGL(ce_combine_kernel, dim3((N + 3) / 4), dim3(256), 0, s, part, nt, target, labels, lse,
                     lse_out, row_loss, rowmax, pred, V, N);
  return hipGetLastError();
}
hipError_t launch_ce_reduce(const float *row_loss, const int32_t *labels, int N, int k, int D,
                            int valid_mean, double denom, float lambda, double *acc_sum, int32_t *acc_cnt,
                            float *scale, const int32_t *pred, int32_t *pred_out, int32_t *acc_correct,
                            hipStream_t s) {
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(1), dim3(1024), 0, s, row_loss, labels, N, k, D, valid_mean,
                     denom, lambda, acc_sum, acc_cnt, scale, pred, pred_out, acc_correct);
  return hipGetLastError();
}
hipError_t launch_ce_finalize(const double *acc_sum, const int32_t *acc_cnt, int D, int valid_mean,
                              double denom, float lambda, float *loss_sum, int32_t *counts, float *loss,
                              float *loss_mtp, const int32_t *acc_correct, int32_t *correct, float *accuracy,
                              hipStream_t s) {
  hipLaunchKernelGGL(ce_finalize_kernel, dim3(1), dim3(64), 0, s, acc_sum, acc_cnt, D, valid_mean, denom,
                     lambda, loss_sum, counts, loss, loss_mtp, acc_correct, correct, accuracy);
  return hipGetLastError();
}

// out[i] = sum over s of part[s * n + i] (+ res[i]): the partial products of
// a GEMM split over K, summed in split order, with the residual of the
// product's epilogue.
template <typename TO>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float *__restrict__ part, int splits, long n,
                                                         const float *__restrict__ res, TO *__restrict__ out) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
    float v = res != nullptr ? res[i] : 0.f;
    float acc = 0.f;
    for (int sp = 0; sp < splits; ++sp) acc += part[(long)sp * n + i];
    store_elem(out, i, acc + v);
  }
}
template <typename TO>
hipError_t launch_splitk_sum(const float *part, int splits, long n, const float *res, TO *out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL((splitk_sum_kernel<TO>), dim3((unsigned)blocks), dim3(256), 0, s, part, splits, n, res, out);
  return hipGetLastError();
}
template hipError_t launch_splitk_sum<float>(const float *, int, long, const float *, float *, hipStream_t);
template hipError_t launch_splitk_sum<bf16_t>(const float *, int, long, const float *, bf16_t *, hipStream_t);

__global__ void fill_i32_kernel(int32_t *p, long n, int32_t v) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void fill_f32_kernel(float *p, long n, float v) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
hipError_t fill_i32(int32_t *p, long n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}
hipError_t fill_f32(float *p, long n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace mtp
