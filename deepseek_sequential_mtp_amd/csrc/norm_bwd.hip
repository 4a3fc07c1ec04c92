// Row kernels of the chain's reverse pass (M7.6 0x05A: the MTP gradient
// reaches hnorm, enorm, the block's norms, the shared embedding and h^(0)):
// the RMSNorm backward with its gain gradient, and the embedding gradient,
// a scatter-add of the enorm input gradient into the rows of E that the
// module read.
//
// RMSNorm_g(z) = g z r, r = 1 / sqrt(mean(z^2) + eps), x_n = z r:
//   dz = r (g dy - x_n mean(x_n g dy)),   dg = sum over rows of dy x_n.
#include <rocprim/device/device_radix_sort.hpp>
#include <rocprim/device/device_run_length_encode.hpp>
#include <rocprim/device/device_scan.hpp>

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

// dE[t] += sum of de over the rows whose shifted token is t.  The sorted
// (key, row) pairs form one run per distinct key (the stable sort keeps the
// rows ascending); run r holds counts[r] rows from offsets[r].  A fixed grid
// walks the runs; the block's kEmbWaves waves share a run's rows, wave w
// taking positions 4 (w + kEmbWaves i) + u, u = 0..3, into accumulator u,
// and the partial sums are added in wave order, so the result does not
// depend on timing (no atomics).  Lane l of grid column y owns the 16-byte
// chunk 64 y + l of the row.  Zipf-distributed tokens give a few long runs
// (the most frequent token appears in thousands of rows), which all the
// block's waves split instead of one thread walking them.
constexpr int kEmbWaves = 16;
__global__ __launch_bounds__(64 * kEmbWaves) void embed_grad_kernel(
    const int32_t *__restrict__ unique, const uint32_t *__restrict__ counts, const uint32_t *__restrict__ offsets,
    const uint32_t *__restrict__ nruns, const int32_t *__restrict__ rows, const float *__restrict__ de, int d,
    int V, float *__restrict__ dE) {
  __shared__ float4 part[kEmbWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int nch = d >> 2;
  const int c = blockIdx.y * 64 + lane;
  const bool cok = c < nch;
  const int R = (int)nruns[0];
  for (int r = blockIdx.x; r < R; r += gridDim.x) {
    const int k = unique[r];
    if (k >= V) continue;                       // the rows without a gathered embedding
    const int off = (int)offsets[r], len = (int)counts[r];
    float4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = 4 * w; q0 < len; q0 += 4 * kEmbWaves) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = q0 + u < len && cok ? ld4(de + (long)rows[off + q0 + u] * d, c) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[u].x += v[u].x; acc[u].y += v[u].y; acc[u].z += v[u].z; acc[u].w += v[u].w;
      }
    }
    float4 t = acc[0];
#pragma unroll
    for (int u = 1; u < 4; ++u) { t.x += acc[u].x; t.y += acc[u].y; t.z += acc[u].z; t.w += acc[u].w; }
    part[w][lane] = t;
    __syncthreads();
    if (w == 0 && cok) {
      float4 sum = part[0][lane];
#pragma unroll
      for (int i = 1; i < kEmbWaves; ++i) {
        const float4 x = part[i][lane];
        sum.x += x.x; sum.y += x.y; sum.z += x.z; sum.w += x.w;
      }
      float4 *dst = reinterpret_cast<float4 *>(dE + (long)k * d) + c;
      float4 o = *dst;
      o.x += sum.x; o.y += sum.y; o.z += sum.z; o.w += sum.w;
      *dst = o;
    }
    __syncthreads();
  }
}

static unsigned key_bits(int V) {
  unsigned b = 1;
  while ((1L << b) <= (long)V) ++b;     // keys run to V (the sentinel)
  return b;
}

// Scratch of launch_embed_grad: the library routines' temporary storage (the
// largest of the sort's, the run-length encoding's and the scan's), then the
// runs' keys, counts and offsets (N each) and the run count.
namespace {
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }
size_t embed_tmp_bytes(int N, int V) {
  size_t sort_b = 0, rle_b = 0, scan_b = 0;
  if (rocprim::radix_sort_pairs(nullptr, sort_b, (const int32_t *)nullptr, (int32_t *)nullptr,
                                (const int32_t *)nullptr, (int32_t *)nullptr, (size_t)N, 0u, key_bits(V)) !=
      hipSuccess)
    return 0;
  if (rocprim::run_length_encode(nullptr, rle_b, (const int32_t *)nullptr, (unsigned)N, (int32_t *)nullptr,
                                 (uint32_t *)nullptr, (uint32_t *)nullptr) != hipSuccess)
    return 0;
  if (rocprim::exclusive_scan(nullptr, scan_b, (const uint32_t *)nullptr, (uint32_t *)nullptr, 0u, (size_t)N,
                              rocprim::plus<uint32_t>()) != hipSuccess)
    return 0;
  return align256(std::max(sort_b, std::max(rle_b, scan_b)));
}
}  // namespace

size_t embed_grad_sort_bytes(int N, int V) {
  const size_t tmp = embed_tmp_bytes(N, V);
  if (tmp == 0) return 0;
  return tmp + 3 * align256((size_t)N * 4) + 256;
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
  const size_t tmp = embed_tmp_bytes(N, V);
  if (tmp == 0 || sort_bytes < embed_grad_sort_bytes(N, V)) return hipErrorInvalidValue;
  char *base = static_cast<char *>(sort_tmp);
  int32_t *unique = reinterpret_cast<int32_t *>(base + tmp);
  uint32_t *counts = reinterpret_cast<uint32_t *>(base + tmp + align256((size_t)N * 4));
  uint32_t *offsets = reinterpret_cast<uint32_t *>(base + tmp + 2 * align256((size_t)N * 4));
  uint32_t *nruns = reinterpret_cast<uint32_t *>(base + tmp + 3 * align256((size_t)N * 4));
  size_t bytes = tmp;
  hipError_t e = rocprim::radix_sort_pairs(sort_tmp, bytes, key, key_sorted, val, val_sorted, (size_t)N, 0u,
                                           key_bits(V), s);
  if (e != hipSuccess) return e;
  bytes = tmp;
  e = rocprim::run_length_encode(sort_tmp, bytes, (const int32_t *)key_sorted, (unsigned)N, unique, counts, nruns, s);
  if (e != hipSuccess) return e;
  bytes = tmp;
  // runs past nruns hold stale counts; their offsets are never read
  e = rocprim::exclusive_scan(sort_tmp, bytes, (const uint32_t *)counts, offsets, 0u, (size_t)N,
                              rocprim::plus<uint32_t>(), s);
  if (e != hipSuccess) return e;
  const int ny = ((d >> 2) + 63) / 64;
  const int gx = N < 1024 ? N : 1024;
  hipLaunchKernelGGL(embed_grad_kernel, dim3(gx, ny), dim3(64 * kEmbWaves), 0, s, unique, counts, offsets, nruns,
                     val_sorted, de, d, V, dE);
  return hipGetLastError();
}

// Reverse of SwiGLU from saved pre-activations (the recompute GEMM's
// epilogue without the GEMM): pre [N, 2f] f32 (gate | up) and dgsw [N, f]
// bf16 give gsw = silu(gate) up [N, f] and dgu = [d gate | d up] [N, 2f], in
// bf16.  One thread per row and 4 features (f % 4 == 0).
__global__ void swiglu_bwd_kernel(const float *__restrict__ pre, const bf16_t *__restrict__ dgsw,
                                  bf16_t *__restrict__ gsw, bf16_t *__restrict__ dgu, long N, int f) {
  const int f4 = f >> 2;
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * f4) return;
  const long row = i / f4;
  const int j = 4 * (int)(i - row * f4);
  const float4 g = *reinterpret_cast<const float4 *>(pre + row * 2 * f + j);
  const float4 u = *reinterpret_cast<const float4 *>(pre + row * 2 * f + f + j);
  const uint2 dw = *reinterpret_cast<const uint2 *>(dgsw + row * f + j);
  const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
  const float dv[4] = {bf16_lo_f32(dw.x), bf16_hi_f32(dw.x), bf16_lo_f32(dw.y), bf16_hi_f32(dw.y)};
  float sw[4], dg[4], du[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) swiglu_bwd_elem(gv[e], uv[e], dv[e], sw[e], dg[e], du[e]);
  *reinterpret_cast<uint2 *>(gsw + row * f + j) = make_uint2(pack_bf16x2(sw[0], sw[1]), pack_bf16x2(sw[2], sw[3]));
  *reinterpret_cast<uint2 *>(dgu + row * 2 * f + j) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
  *reinterpret_cast<uint2 *>(dgu + row * 2 * f + f + j) =
      make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
}

hipError_t launch_swiglu_bwd(const float *pre, const bf16_t *dgsw, bf16_t *gsw, bf16_t *dgu, long N, int f,
                             hipStream_t s) {
  if (f % 4 != 0) return hipErrorInvalidValue;
  const long n = N * (f / 4);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, pre, dgsw, gsw, dgu, N,
                     f);
  return hipGetLastError();
}

}  // namespace mtp
