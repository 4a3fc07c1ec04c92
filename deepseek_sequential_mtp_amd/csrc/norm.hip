// Bandwidth-bound row kernels: the dual RMSNorm + concat that feeds eh_proj,
// the block pre-norms, the shared output norm and its backward.
//
// RMSNorm_g(z) = g * z / sqrt(mean(z^2) + eps) (M7.6 0x03C); statistics in
// float32.  One 256-thread block per row, 16-byte chunk accesses.  Rows of
// up to 8 chunks per thread (d <= 8192 for f32 input) are held in registers
// between the sum of squares and the scaling, so each row is read once.
#include "kernels.hpp"

namespace mtp {

namespace {
constexpr int kNormThreads = 256;

__device__ __forceinline__ float block_sum(float v, float *sh) {
  v = warp_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / 64; ++i) s += sh[i];
  return s;
}

template <typename T>
__device__ float row_sumsq(const T *row, int d) {
  constexpr int E = Elem<T>::kPerChunk;
  float acc = 0.f;
  for (int c = threadIdx.x; c < d / E; c += kNormThreads) {
    float v[E];
    chunk_to_f32(reinterpret_cast<const uint4 *>(row)[c], v, T{});
#pragma unroll
    for (int e = 0; e < E; ++e) acc += v[e] * v[e];
  }
  return acc;
}

template <typename TI, typename TO>
__device__ void row_scale_store(const TI *row, const float *g, float s, TO *out, int d) {
  constexpr int E = Elem<TI>::kPerChunk;
  for (int c = threadIdx.x; c < d / E; c += kNormThreads) {
    float v[E];
    chunk_to_f32(reinterpret_cast<const uint4 *>(row)[c], v, TI{});
#pragma unroll
    for (int e = 0; e < E; ++e) store_elem(out, (long)c * E + e, g[c * E + e] * v[e] * s);
  }
}

// One row's chunks: CPT > 0 holds chunk threadIdx.x + k * kNormThreads in
// register k (zeros past the row); CPT == 0 reads the row again for each pass.
template <typename TI, int CPT>
struct RowCache {
  static constexpr int E = Elem<TI>::kPerChunk;
  uint4 c[CPT > 0 ? CPT : 1];
  const TI *row;
  int d;
  __device__ __forceinline__ RowCache(const TI *r, int d_) : row(r), d(d_) {
    if constexpr (CPT > 0) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int idx = threadIdx.x + k * kNormThreads;
        c[k] = idx < d / E ? reinterpret_cast<const uint4 *>(row)[idx] : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ float sumsq() const {
    if constexpr (CPT > 0) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        float v[E];
        chunk_to_f32(c[k], v, TI{});
#pragma unroll
        for (int e = 0; e < E; ++e) acc += v[e] * v[e];
      }
      return acc;
    } else {
      return row_sumsq(row, d);
    }
  }
  // out = g * row * s, one vector store per chunk
  template <typename TO>
  __device__ __forceinline__ void scale_store(const float *g, float s, TO *out) const {
    if constexpr (CPT > 0) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int idx = threadIdx.x + k * kNormThreads;
        if (idx >= d / E) break;
        float v[E];
        chunk_to_f32(c[k], v, TI{});
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const float4 gq = reinterpret_cast<const float4 *>(g)[idx * (E / 4) + q];
          const float w[4] = {gq.x * v[4 * q] * s, gq.y * v[4 * q + 1] * s, gq.z * v[4 * q + 2] * s,
                              gq.w * v[4 * q + 3] * s};
          store4(out + (long)idx * E + 4 * q, w);
        }
      }
    } else {
      row_scale_store(row, g, s, out, d);
    }
  }
};

// Chunks per thread for a row of d elements of T: 1, 2, 4 or 8, or 0 (too
// long to hold: two reads).
template <typename T>
inline int row_cpt(int d) {
  const int c = (d / Elem<T>::kPerChunk + kNormThreads - 1) / kNormThreads;
  return c <= 1 ? 1 : c <= 2 ? 2 : c <= 4 ? 4 : c <= 8 ? 8 : 0;
}
template <typename T, class F>
inline void with_cpt(int d, F &&f) {
  switch (row_cpt<T>(d)) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    default: f(std::integral_constant<int, 0>{}); break;
  }
}
}  // namespace

// c[n] = [ g_h * h[n] * s_h ; g_e * E[x(b, i+k)] * s_e ]  (he order)
template <typename T, int CPT>
__global__ __launch_bounds__(kNormThreads) void dual_norm_concat_kernel(
    const T *__restrict__ h, const T *__restrict__ E, const int32_t *__restrict__ tokens,
    const float *__restrict__ g_h, const float *__restrict__ g_e, T *__restrict__ c, int T_len, int d,
    int V, int depth, float eps) {
  __shared__ float sh[kNormThreads / 64];
  const long n = blockIdx.x;
  const int b = (int)(n / T_len), i = (int)(n % T_len);
  int ti = i + depth;
  ti = ti < T_len ? ti : T_len - 1;              // rows with no x_(i+k): any valid id
  int tok = tokens[(long)b * T_len + ti];
  tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);
  const RowCache<T, CPT> hr(h + n * d, d);
  const RowCache<T, CPT> er(E + (long)tok * d, d);
  const float sh_h = block_sum(hr.sumsq(), sh);
  const float sh_e = block_sum(er.sumsq(), sh);
  const float s_h = rsqrtf(sh_h / d + eps);
  const float s_e = rsqrtf(sh_e / d + eps);
  T *cr = c + n * 2 * (long)d;
  hr.scale_store(g_h, s_h, cr);
  er.scale_store(g_e, s_e, cr + d);
}

// out[n] = g * z[n] / rms(z[n]); optionally r[n] = 1 / rms.
template <typename TI, typename TO, int CPT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const TI *__restrict__ z,
                                                              const float *__restrict__ g,
                                                              TO *__restrict__ out, float *__restrict__ r,
                                                              int d, float eps) {
  __shared__ float sh[kNormThreads / 64];
  const long n = blockIdx.x;
  const RowCache<TI, CPT> zr(z + n * d, d);
  const float s = rsqrtf(block_sum(zr.sumsq(), sh) / d + eps);
  if (r != nullptr && threadIdx.x == 0) r[n] = s;
  zr.scale_store(g, s, out + n * d);
}

// Shared output norm for one depth plus label sanitising: labels outside
// [-1, V) become -1 and raise the error flag.
template <typename T, int CPT>
__global__ __launch_bounds__(kNormThreads) void out_norm_kernel(
    const T *__restrict__ h, const float *__restrict__ g, T *__restrict__ xhat, float *__restrict__ r,
    const int32_t *__restrict__ labels_in, int32_t *__restrict__ labels_out, int32_t *__restrict__ err,
    int d, int V, float eps) {
  __shared__ float sh[kNormThreads / 64];
  const long n = blockIdx.x;
  const RowCache<T, CPT> hr(h + n * d, d);
  const float s = rsqrtf(block_sum(hr.sumsq(), sh) / d + eps);
  if (threadIdx.x == 0) {
    r[n] = s;
    int lab = labels_in[n];
    if (lab < -1 || lab >= V) {
      if (err != nullptr) atomicOr(err, 1);
      lab = -1;
    }
    labels_out[n] = lab;
  }
  hr.scale_store(g, s, xhat + n * d);
}

// RMSNorm backward through the output norm:
//   dh = r (g * dx - x_n * mean(x_n * g * dx)),  x_n = r h,
// with dx = sum of `splits` partial slabs (stride slab).
template <typename T>
__global__ __launch_bounds__(kNormThreads) void out_norm_bwd_kernel(
    const float *__restrict__ dx, int splits, long slab, const T *__restrict__ h,
    const float *__restrict__ r, const float *__restrict__ g, float *__restrict__ dh, int d, int dh_acc) {
  __shared__ float sh[kNormThreads / 64];
  const long n = blockIdx.x;
  const float rn = r[n];
  const T *hr = h + n * d;
  float acc = 0.f;
  for (int j = threadIdx.x; j < d; j += kNormThreads) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += dx[s * slab + n * d + j];
    acc += rn * load_elem(hr, j) * g[j] * v;
  }
  const float mean = block_sum(acc, sh) / d;
  for (int j = threadIdx.x; j < d; j += kNormThreads) {
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += dx[s * slab + n * d + j];
    const float xn = rn * load_elem(hr, j);
    const float o = rn * (g[j] * v - xn * mean);
    dh[n * d + j] = dh_acc ? dh[n * d + j] + o : o;
  }
}

// Four consecutive elements of a row as floats (d is a multiple of 4).
__device__ __forceinline__ float4 load4(const float *p, int c) { return reinterpret_cast<const float4 *>(p)[c]; }
__device__ __forceinline__ float4 load4(const bf16_t *p, int c) {
  const uint2 w = reinterpret_cast<const uint2 *>(p)[c];
  return make_float4(bf16_lo_f32(w.x), bf16_hi_f32(w.x), bf16_lo_f32(w.y), bf16_hi_f32(w.y));
}

// Output-norm backward over a block of rows, with its dg partial: for each
// row n, x = r_n h_n, dh_n = r_n (g * v - x * mean(g * v * x)) with v the
// sum of the dx_hat split slabs; part[block][j] = sum over the block's rows
// of v[j] x[j].  Thread t owns the 4-column chunks t, t + 256, ... (CPT of
// them), so the row is read once into registers and the dg partial stays in
// registers across the rows.
template <typename T, int CPT>
__global__ __launch_bounds__(kNormThreads) void out_norm_bwd_rows_kernel(
    const float *__restrict__ dx, int splits, long slab, const T *__restrict__ h, const float *__restrict__ r,
    const float *__restrict__ g, float *__restrict__ dh, float *__restrict__ part, int N, int d,
    int rows_per_block, int dh_acc) {
  __shared__ float sh[kNormThreads / 64];
  const int t = threadIdx.x;
  const int nch = d >> 2;
  const int n0 = blockIdx.x * rows_per_block;
  const int n1 = min(N, n0 + rows_per_block);
  float4 gg[CPT], dg[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = t + i * kNormThreads;
    gg[i] = c < nch ? load4(g, c) : make_float4(0.f, 0.f, 0.f, 0.f);
    dg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int n = n0; n < n1; ++n) {
    const float rn = r[n];
    float4 v[CPT], x[CPT];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + i * kNormThreads;
      if (c < nch) {
        float4 a = load4(dx + (long)n * d, c);
        for (int sp = 1; sp < splits; ++sp) {
          const float4 b = load4(dx + sp * slab + (long)n * d, c);
          a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        const float4 hv = load4(h + (long)n * d, c);
        v[i] = a;
        x[i] = make_float4(rn * hv.x, rn * hv.y, rn * hv.z, rn * hv.w);
        acc += gg[i].x * a.x * x[i].x + gg[i].y * a.y * x[i].y + gg[i].z * a.z * x[i].z + gg[i].w * a.w * x[i].w;
      }
    }
    const float mean = block_sum(acc, sh) / d;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + i * kNormThreads;
      if (c < nch) {
        float4 o = make_float4(rn * (gg[i].x * v[i].x - x[i].x * mean), rn * (gg[i].y * v[i].y - x[i].y * mean),
                               rn * (gg[i].z * v[i].z - x[i].z * mean), rn * (gg[i].w * v[i].w - x[i].w * mean));
        float4 *dp = reinterpret_cast<float4 *>(dh + (long)n * d) + c;
        if (dh_acc) {
          const float4 prev = *dp;
          o.x += prev.x; o.y += prev.y; o.z += prev.z; o.w += prev.w;
        }
        *dp = o;
        dg[i].x += v[i].x * x[i].x;
        dg[i].y += v[i].y * x[i].y;
        dg[i].z += v[i].z * x[i].z;
        dg[i].w += v[i].w * x[i].w;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = t + i * kNormThreads;
    if (c < nch) reinterpret_cast<float4 *>(part + (long)blockIdx.x * d)[c] = dg[i];
  }
}

// dg partials: part[rb][j] = sum over rows in row block rb of dx[n][j] * x_n[n][j].
template <typename T>
__global__ __launch_bounds__(kNormThreads) void dg_partial_kernel(
    const float *__restrict__ dx, int splits, long slab, const T *__restrict__ h,
    const float *__restrict__ r, float *__restrict__ part, int N, int d, int rows_per_block) {
  const int j = blockIdx.y * 64 + (threadIdx.x & 63);   // row blocks on x, column blocks on y
  const int rg = threadIdx.x >> 6;
  const int n0 = blockIdx.x * rows_per_block;
  const int n1 = min(N, n0 + rows_per_block);
  __shared__ float sh[4][64];
  float acc = 0.f;
  if (j < d) {
    for (int n = n0 + rg; n < n1; n += 4) {
      float v = 0.f;
      for (int s = 0; s < splits; ++s) v += dx[s * slab + (long)n * d + j];
      acc += v * r[n] * load_elem(h, (long)n * d + j);
    }
  }
  sh[rg][threadIdx.x & 63] = acc;
  __syncthreads();
  if (rg == 0 && j < d)
    part[(long)blockIdx.x * d + j] = sh[0][threadIdx.x] + sh[1][threadIdx.x] + sh[2][threadIdx.x] +
                                     sh[3][threadIdx.x];
}

// dg[j] (+)= sum_rb part[rb][j].  A block covers 64 columns with 16 row
// groups; group q sums the row blocks q, q + 16, ... in ascending order and
// the groups are added in order, so the result does not depend on timing.
constexpr int kDgGroups = 16;
__global__ __launch_bounds__(64 * kDgGroups) void dg_reduce_kernel(const float *__restrict__ part, int nrb, int d,
                                                                   float *__restrict__ dg, int accumulate) {
  __shared__ float sh[kDgGroups][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (j < d) {
#pragma unroll 4
    for (int b = q; b < nrb; b += kDgGroups) s += part[(long)b * d + j];
  }
  sh[q][lane] = s;
  __syncthreads();
  if (q == 0 && j < d) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kDgGroups; ++i) t += sh[i][lane];
    dg[j] = accumulate ? dg[j] + t : t;
  }
}

hipError_t launch_dg_reduce(const float *part, int nrb, int d, float *dg, int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(dg_reduce_kernel, dim3((d + 63) / 64), dim3(64 * kDgGroups), 0, s, part, nrb, d, dg, accumulate);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_dual_norm_concat(const T *h, const T *E, const int32_t *tokens, const float *g_h,
                                   const float *g_e, T *c, int B, int T_len, int d, int V, int depth,
                                   float eps, hipStream_t s) {
  with_cpt<T>(d, [&](auto cpt) {
    hipLaunchKernelGGL((dual_norm_concat_kernel<T, decltype(cpt)::value>), dim3(B * T_len), dim3(kNormThreads), 0,
                       s, h, E, tokens, g_h, g_e, c, T_len, d, V, depth, eps);
  });
  return hipGetLastError();
}
template <typename TI, typename TO>
hipError_t launch_rmsnorm(const TI *z, const float *g, TO *out, float *r, long rows, int d, float eps,
                          hipStream_t s) {
  with_cpt<TI>(d, [&](auto cpt) {
    hipLaunchKernelGGL((rmsnorm_kernel<TI, TO, decltype(cpt)::value>), dim3(rows), dim3(kNormThreads), 0, s, z, g,
                       out, r, d, eps);
  });
  return hipGetLastError();
}
template <typename T>
hipError_t launch_out_norm(const T *h, const float *g, T *xhat, float *r, const int32_t *labels_in,
                           int32_t *labels_out, int32_t *err, long rows, int d, int V, float eps,
                           hipStream_t s) {
  with_cpt<T>(d, [&](auto cpt) {
    hipLaunchKernelGGL((out_norm_kernel<T, decltype(cpt)::value>), dim3(rows), dim3(kNormThreads), 0, s, h, g, xhat,
                       r, labels_in, labels_out, err, d, V, eps);
  });
  return hipGetLastError();
}
template <typename T>
hipError_t launch_out_norm_bwd(const float *dx, int splits, long slab, const T *h, const float *r,
                               const float *g, float *dh, float *dg_part, float *dg, int accumulate,
                               int N, int d, int dh_acc, hipStream_t s) {
  const int nrb = dg_row_blocks(N);
  const int rpb = (N + nrb - 1) / nrb;
  const int cpt = (d / 4 + kNormThreads - 1) / kNormThreads;
  if (cpt <= 8) {
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(nrb), dim3(kNormThreads), 0, s, dx, splits, slab, h, r, g, dh, dg_part, N, d,
                         rpb, dh_acc);
    };
    if (cpt <= 1) go(out_norm_bwd_rows_kernel<T, 1>);
    else if (cpt <= 2) go(out_norm_bwd_rows_kernel<T, 2>);
    else if (cpt <= 4) go(out_norm_bwd_rows_kernel<T, 4>);
    else go(out_norm_bwd_rows_kernel<T, 8>);
  } else {
    hipLaunchKernelGGL(out_norm_bwd_kernel<T>, dim3(N), dim3(kNormThreads), 0, s, dx, splits, slab, h, r, g,
                       dh, d, dh_acc);
    hipLaunchKernelGGL(dg_partial_kernel<T>, dim3(nrb, (d + 63) / 64), dim3(kNormThreads), 0, s, dx, splits,
                       slab, h, r, dg_part, N, d, rpb);
  }
  hipLaunchKernelGGL(dg_reduce_kernel, dim3((d + 63) / 64), dim3(64 * kDgGroups), 0, s, dg_part, nrb, d, dg,
                     accumulate);
  return hipGetLastError();
}

#define MTP_NORM_INST(T)                                                                                  \
  template hipError_t launch_dual_norm_concat<T>(const T *, const T *, const int32_t *, const float *,    \
                                                 const float *, T *, int, int, int, int, int, float,      \
                                                 hipStream_t);                                            \
  template hipError_t launch_out_norm<T>(const T *, const float *, T *, float *, const int32_t *,         \
                                         int32_t *, int32_t *, long, int, int, float, hipStream_t);       \
  template hipError_t launch_out_norm_bwd<T>(const float *, int, long, const T *, const float *,          \
                                             const float *, float *, float *, float *, int, int, int,     \
                                             int, hipStream_t);
MTP_NORM_INST(bf16_t)
MTP_NORM_INST(float)
template hipError_t launch_rmsnorm<bf16_t, bf16_t>(const bf16_t *, const float *, bf16_t *, float *, long,
                                                   int, float, hipStream_t);
template hipError_t launch_rmsnorm<float, bf16_t>(const float *, const float *, bf16_t *, float *, long,
                                                  int, float, hipStream_t);
template hipError_t launch_rmsnorm<float, float>(const float *, const float *, float *, float *, long, int,
                                                 float, hipStream_t);

}  // namespace mtp
