// Row kernels of the chain's reverse pass (M7.6 0x05A: the MTP gradient
// reaches hnorm, enorm, the block's norms, the shared embedding and h^(0)):
// the RMSNorm backward with its gain gradient, and the embedding gradient,
// a scatter-add of the enorm input gradient into the rows of E that the
// module read.
//
// RMSNorm_g(z) = g z r, r = 1 / sqrt(mean(z^2) + eps), x_n = z r:
//   dz = r (g dy - x_n mean(x_n g dy)),   dg = sum over rows of dy x_n.
#include <rocprim/device/device_radix_sort.hpp>

#include "kernels.hpp"

namespace mtp {

namespace {
constexpr int kThreads = 256;

__device__ __forceinline__ float block_sum256(float v, float *sh) {
  v = warp_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

__device__ __forceinline__ float4 ld4(const float *p, int c) { return reinterpret_cast<const float4 *>(p)[c]; }
__device__ __forceinline__ float4 ld4(const bf16_t *p, int c) {
  const uint2 w = reinterpret_cast<const uint2 *>(p)[c];
  return make_float4(bf16_lo_f32(w.x), bf16_hi_f32(w.x), bf16_lo_f32(w.y), bf16_hi_f32(w.y));
}
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }
}  // namespace

// One block of rows: for each row n (input row zrow[n] of z when zrow is
// set), dz[n] = resid[n] + (rowmask[n] ? RMSNorm backward : 0), optional
// bf16 copy dzb[n]; part[block] = this block's rows' dg contribution.
// Thread t owns the 4-column chunks t, t + 256, ... (CPT of them), so each
// row is read once into registers and the dg partial stays in registers.
template <typename TZ, int CPT>
__global__ __launch_bounds__(kThreads) void rms_bwd_kernel(
    const float *__restrict__ dy, long ldy, const TZ *__restrict__ z, const int32_t *__restrict__ zrow,
    const float *__restrict__ g, float eps, const float *__restrict__ resid, const uint8_t *__restrict__ rowmask,
    float *__restrict__ dz, bf16_t *__restrict__ dzb, float *__restrict__ part, int N, int d, int rows_per_block) {
  __shared__ float sh[4];
  const int t = threadIdx.x;
  const int nch = d >> 2;
  const int n0 = blockIdx.x * rows_per_block;
  const int n1 = min(N, n0 + rows_per_block);
  float4 gg[CPT], dg[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = t + i * kThreads;
    gg[i] = c < nch ? ld4(g, c) : make_float4(0.f, 0.f, 0.f, 0.f);
    dg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int n = n0; n < n1; ++n) {
    const bool on = rowmask == nullptr || rowmask[n] != 0;
    const TZ *zr = z + (long)(zrow != nullptr ? zrow[n] : n) * d;
    float4 v[CPT], x[CPT];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + i * kThreads;
      if (c < nch) {
        x[i] = ld4(zr, c);
        v[i] = ld4(dy + (long)n * ldy, c);
        ss += dot4(x[i], x[i]);
      }
    }
    const float rn = rsqrtf(block_sum256(ss, sh) / d + eps);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + i * kThreads;
      if (c < nch) {
        x[i] = make_float4(rn * x[i].x, rn * x[i].y, rn * x[i].z, rn * x[i].w);
        acc += gg[i].x * v[i].x * x[i].x + gg[i].y * v[i].y * x[i].y + gg[i].z * v[i].z * x[i].z +
               gg[i].w * v[i].w * x[i].w;
      }
    }
    const float mean = block_sum256(acc, sh) / d;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = t + i * kThreads;
      if (c < nch) {
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (on) {
          o = make_float4(rn * (gg[i].x * v[i].x - x[i].x * mean), rn * (gg[i].y * v[i].y - x[i].y * mean),
                          rn * (gg[i].z * v[i].z - x[i].z * mean), rn * (gg[i].w * v[i].w - x[i].w * mean));
          dg[i].x += v[i].x * x[i].x;
          dg[i].y += v[i].y * x[i].y;
          dg[i].z += v[i].z * x[i].z;
          dg[i].w += v[i].w * x[i].w;
        }
        if (resid != nullptr) {
          const float4 rr = ld4(resid + (long)n * d, c);
          o.x += rr.x; o.y += rr.y; o.z += rr.z; o.w += rr.w;
        }
        reinterpret_cast<float4 *>(dz + (long)n * d)[c] = o;
        if (dzb != nullptr)
          reinterpret_cast<uint2 *>(dzb + (long)n * d)[c] = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = t + i * kThreads;
    if (c < nch) reinterpret_cast<float4 *>(part + (long)blockIdx.x * d)[c] = dg[i];
  }
}

template <typename TZ>
hipError_t launch_rms_bwd(const float *dy, long ldy, const TZ *z, const int32_t *zrow, const float *g, float eps,
                          const float *resid, const uint8_t *rowmask, float *dz, bf16_t *dzb, float *part,
                          float *dg, int accumulate, int N, int d, hipStream_t s) {
  const int nrb = dg_row_blocks(N);
  const int rpb = (N + nrb - 1) / nrb;
  const int cpt = (d / 4 + kThreads - 1) / kThreads;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(nrb), dim3(kThreads), 0, s, dy, ldy, z, zrow, g, eps, resid, rowmask, dz, dzb,
                       part, N, d, rpb);
  };
  if (cpt <= 1) go(rms_bwd_kernel<TZ, 1>);
  else if (cpt <= 2) go(rms_bwd_kernel<TZ, 2>);
  else if (cpt <= 4) go(rms_bwd_kernel<TZ, 4>);
  else if (cpt <= 8) go(rms_bwd_kernel<TZ, 8>);
  else return hipErrorInvalidValue;      // d > 8192: rejected on the host
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dg_reduce(part, nrb, d, dg, accumulate, s);
}
template hipError_t launch_rms_bwd<float>(const float *, long, const float *, const int32_t *, const float *, float,
                                          const float *, const uint8_t *, float *, bf16_t *, float *, float *, int,
                                          int, int, hipStream_t);
template hipError_t launch_rms_bwd<bf16_t>(const float *, long, const bf16_t *, const int32_t *, const float *,
                                           float, const float *, const uint8_t *, float *, bf16_t *, float *,
                                           float *, int, int, int, hipStream_t);

// Shifted-token rows of depth k: tok[n] = x[b, i + k] clamped as the forward
// gathers it; key[n] = tok[n] on state rows, V elsewhere (sorted last and
// skipped by the embedding gradient); val[n] = n.
__global__ void shifted_rows_kernel(const int32_t *__restrict__ tokens, const uint8_t *__restrict__ state, int B,
                                    int T_len, int V, int depth, int32_t *__restrict__ tok,
                                    int32_t *__restrict__ key, int32_t *__restrict__ val) {
  const long n = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= (long)B * T_len) return;
  const int b = (int)(n / T_len), i = (int)(n % T_len);
  int ti = i + depth;
  ti = ti < T_len ? ti : T_len - 1;
  int x = tokens[(long)b * T_len + ti];
  x = x < 0 ? 0 : (x >= V ? V - 1 : x);
  tok[n] = x;
  key[n] = state[n] ? x : V;
  val[n] = (int32_t)n;
}

// dE[t] += sum of de over the rows whose shifted token is t, in ascending
// row order (the stable sort keeps it): the block at sorted position p
// starts a run of equal keys; it sums the run for its column range.
__global__ __launch_bounds__(kThreads) void embed_grad_kernel(const int32_t *__restrict__ keys,
                                                             const int32_t *__restrict__ rows, int N,
                                                             const float *__restrict__ de, int d, int V,
                                                             float *__restrict__ dE) {
  const int p = blockIdx.x;
  const int k = keys[p];
  if (k >= V || (p > 0 && keys[p - 1] == k)) return;
  const int nch = d >> 2;
  for (int c = blockIdx.y * kThreads + threadIdx.x; c < nch; c += gridDim.y * kThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q = p; q < N && keys[q] == k; ++q) {
      const float4 v = ld4(de + (long)rows[q] * d, c);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    float4 *dst = reinterpret_cast<float4 *>(dE + (long)k * d) + c;
    float4 o = *dst;
    o.x += acc.x; o.y += acc.y; o.z += acc.z; o.w += acc.w;
    *dst = o;
  }
}

static unsigned key_bits(int V) {
  unsigned b = 1;
  while ((1L << b) <= (long)V) ++b;     // keys run to V (the sentinel)
  return b;
}

size_t embed_grad_sort_bytes(int N, int V) {
  size_t bytes = 0;
  if (rocprim::radix_sort_pairs(nullptr, bytes, (const int32_t *)nullptr, (int32_t *)nullptr,
                                (const int32_t *)nullptr, (int32_t *)nullptr, (size_t)N, 0u, key_bits(V)) !=
      hipSuccess)
    return 0;
  return bytes;
}

hipError_t launch_shifted_rows(const int32_t *tokens, const uint8_t *state, int B, int T_len, int V, int depth,
                               int32_t *tok, int32_t *key, int32_t *val, hipStream_t s) {
  const long N = (long)B * T_len;
  hipLaunchKernelGGL(shifted_rows_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, tokens, state, B,
                     T_len, V, depth, tok, key, val);
  return hipGetLastError();
}

hipError_t launch_embed_grad(const int32_t *key, const int32_t *val, int32_t *key_sorted, int32_t *val_sorted,
                             void *sort_tmp, size_t sort_bytes, int N, int V, const float *de, int d, float *dE,
                             hipStream_t s) {
  size_t bytes = sort_bytes;
  hipError_t e = rocprim::radix_sort_pairs(sort_tmp, bytes, key, key_sorted, val, val_sorted, (size_t)N, 0u,
                                           key_bits(V), s);
  if (e != hipSuccess) return e;
  const int ny = ((d >> 2) + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(embed_grad_kernel, dim3(N, ny), dim3(kThreads), 0, s, key_sorted, val_sorted, N, de, d, V, dE);
  return hipGetLastError();
}

}  // namespace mtp
