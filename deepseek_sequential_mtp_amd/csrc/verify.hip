// Exact speculative verification (M7.6 0x09 for one proposal; the
// speculative-decoding explainer page for gamma proposals).
//
// Pass 1 (one block per logit row, all rows of all requests): log-sum-exp of
// z / tau in float64 (exponentials and sums), plus a finiteness flag.  A
// float32 exponential would leave a ~1e-7 relative error in p / q and in the
// CDF, the size of one token's mass at V ~ 1e5; float64 keeps every decision
// exact up to ~1e-13.  Pass 2 (one block per request): the left-to-right ratio tests in
// float64, then the draw from the normalised residual (p_A - q_A)+ or from
// p_gamma by inverse CDF over ascending token ids (smallest t with
// cdf(t) > u * mass), the CDF summed in float64 chunk by chunk.
#include "kernels.hpp"

namespace mtp {

namespace {
constexpr int kVThreads = 256;

__device__ __forceinline__ float logit(const void *z, int bf16, long i) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t *>(z)[i]) : static_cast<const float *>(z)[i];
}
}  // namespace

// ws layout per request r and row index j in [0, 2G+1):
//   ws[(r*(2G+1) + j)*2 + 0] = lse (double), [.. + 1] = 1.0 if finite else 0.0
// rows j <= G are target rows, j > G draft rows (j - G - 1).
__global__ __launch_bounds__(kVThreads) void verify_lse_kernel(const void *zt, const void *zd, int bf16,
                                                              int G, int V, float tau, double *ws) {
  __shared__ float shm[kVThreads / 64];
  __shared__ double shs[kVThreads / 64];
  __shared__ int shb[kVThreads / 64];
  const int nrow = 2 * G + 1;
  const long rid = blockIdx.x;
  const int r = (int)(rid / nrow), j = (int)(rid % nrow);
  const void *base;
  long off;
  if (j <= G) { base = zt; off = ((long)r * (G + 1) + j) * V; }
  else { base = zd; off = ((long)r * G + (j - G - 1)) * V; }
  const float inv_tau = 1.f / tau;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  float mx = -INFINITY;
  int bad = 0;
  for (int v = t; v < V; v += kVThreads) {
    const float x = logit(base, bf16, off + v) * inv_tau;
    if (isnan(x) || x == INFINITY) bad = 1;
    mx = fmaxf(mx, x);
  }
  mx = warp_max(mx);
  for (int o = 32; o > 0; o >>= 1) bad |= __shfl_xor(bad, o);
  if (lane == 0) { shm[w] = mx; shb[w] = bad; }
  __syncthreads();
  mx = shm[0];
  bad = shb[0];
  for (int i = 1; i < kVThreads / 64; ++i) { mx = fmaxf(mx, shm[i]); bad |= shb[i]; }
  if (mx == -INFINITY || isnan(mx)) bad = 1;
  double part = 0.0;
  const double dtau = 1.0 / (double)tau, dmx = (double)mx;
  if (!bad)
    for (int v = t; v < V; v += kVThreads) part += exp((double)logit(base, bf16, off + v) * dtau - dmx);
  double s = warp_sum(part);
  if (lane == 0) shs[w] = s;
  __syncthreads();
  if (t == 0) {
    double tot = 0.0;
    for (int i = 0; i < kVThreads / 64; ++i) tot += shs[i];
    ws[rid * 2] = bad ? 0.0 : (double)mx + log(tot);
    ws[rid * 2 + 1] = bad ? 0.0 : 1.0;
  }
}

__global__ __launch_bounds__(kVThreads) void verify_decide_kernel(
    const void *zt, const void *zd, int bf16, const int32_t *__restrict__ y, const float *__restrict__ ua,
    const float *__restrict__ us, int G, int V, float tau, const double *__restrict__ ws,
    int32_t *__restrict__ A_out, int32_t *__restrict__ tok_out, int32_t *__restrict__ st_out,
    float *__restrict__ margin_out) {
  __shared__ int sA, sSt;
  __shared__ double sMargin;
  __shared__ double sPre[kVThreads + 1];
  __shared__ int sTok;
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const int nrow = 2 * G + 1;
  const double *wr = ws + (long)r * nrow * 2;
  const double itau = 1.0 / (double)tau;

  if (t == 0) {
    int st = 0;
    int A = G;
    double margin = INFINITY;
    for (int j = 0; j < G && st == 0; ++j) {
      const float u = ua[(long)r * G + j];
      if (!(u >= 0.f && u < 1.f)) st = 1;
    }
    for (int j = 0; j <= G && st == 0; ++j) {
      const float u = us[(long)r * (G + 1) + j];
      if (!(u >= 0.f && u < 1.f)) st = 1;
    }
    for (int j = 0; j < G && st == 0; ++j) {
      const int yj = y[(long)r * G + j];
      if (yj < 0 || yj >= V) st = 2;
    }
    if (st == 0) {
      for (int j = 0; j < G; ++j) {
        if (wr[2 * j + 1] == 0.0 || wr[2 * (G + 1 + j) + 1] == 0.0) { st = 5; break; }
        const int yj = y[(long)r * G + j];
        const double p = exp((double)logit(zt, bf16, ((long)r * (G + 1) + j) * V + yj) * itau - wr[2 * j]);
        const double q =
            exp((double)logit(zd, bf16, ((long)r * G + j) * V + yj) * itau - wr[2 * (G + 1 + j)]);
        if (!(q > 0.0)) { st = 3; break; }
        const double ratio = p / q;
        const double u = (double)ua[(long)r * G + j];
        margin = fmin(margin, fabs(u - ratio));
        if (u < ratio) continue;
        A = j;
        break;
      }
      if (st == 0 && A == G && wr[2 * G + 1] == 0.0) st = 5;
    }
    sA = A;
    sSt = st;
    sMargin = margin;
    sTok = -1;
  }
  __syncthreads();
  const int A = sA;
  if (sSt != 0) {
    if (t == 0) {
      A_out[r] = 0;
      tok_out[r] = -1;
      st_out[r] = sSt;
      if (margin_out != nullptr) margin_out[r] = 0.f;
    }
    return;
  }
  // weights of the emission distribution
  const bool resid = A < G;
  const long offp = ((long)r * (G + 1) + A) * V;
  const long offq = resid ? ((long)r * G + A) * V : 0;
  const double lp = wr[2 * A];
  const double lq = resid ? wr[2 * (G + 1 + A)] : 0.0;
  const int chunk = (V + kVThreads - 1) / kVThreads;
  const int v0 = min(V, t * chunk), v1 = min(V, v0 + chunk);
  auto weight = [&](int v) -> double {
    const double p = exp((double)logit(zt, bf16, offp + v) * itau - lp);
    if (!resid) return p;
    const double q = exp((double)logit(zd, bf16, offq + v) * itau - lq);
    return p > q ? p - q : 0.0;
  };
  double sum = 0.0;
  for (int v = v0; v < v1; ++v) sum += weight(v);
  sPre[t + 1] = sum;
  __syncthreads();
  if (t == 0) {
    sPre[0] = 0.0;
    for (int i = 1; i <= kVThreads; ++i) sPre[i] += sPre[i - 1];
  }
  __syncthreads();
  const double W = sPre[kVThreads];
  if (!(W > 0.0)) {
    if (t == 0) {
      A_out[r] = 0;
      tok_out[r] = -1;
      st_out[r] = 4;
      if (margin_out != nullptr) margin_out[r] = 0.f;
    }
    return;
  }
  const double u = (double)us[(long)r * (G + 1) + A];
  const double target = u * W;
  const double pre = sPre[t];
  if (pre <= target && target < sPre[t + 1]) {
    double c = pre;
    int tok = -1, last = -1;
    double m = 0.0;
    for (int v = v0; v < v1; ++v) {
      const double wv = weight(v);
      if (wv > 0.0) last = v;
      const double cn = c + wv;
      if (cn > target) {
        tok = v;
        m = fmin(target - c, cn - target) / W;
        break;
      }
      c = cn;
    }
    if (tok < 0) { tok = last; m = 0.0; }   // crossing lost to rounding: flagged by margin 0
    sTok = tok;
    sMargin = fmin(sMargin, m);
  }
  __syncthreads();
  if (t == 0) {
    int tok = sTok;
    if (tok < 0) {   // target beyond the total (rounding): last positive weight
      for (int v = V - 1; v >= 0; --v)
        if (weight(v) > 0.0) { tok = v; break; }
      sMargin = 0.0;
    }
    A_out[r] = A;
    tok_out[r] = tok;
    st_out[r] = 0;
    if (margin_out != nullptr) margin_out[r] = (float)sMargin;
  }
}

hipError_t launch_verify(const void *zt, const void *zd, int bf16, const int32_t *y, const float *ua,
                         const float *us, int R, int G, int V, float tau, int32_t *A, int32_t *tok,
                         int32_t *status, float *margin, double *ws, hipStream_t s) {
  const long rows = (long)R * (2 * G + 1);
  hipLaunchKernelGGL(verify_lse_kernel, dim3((unsigned)rows), dim3(kVThreads), 0, s, zt, zd, bf16, G, V, tau,
                     ws);
  hipLaunchKernelGGL(verify_decide_kernel, dim3(R), dim3(kVThreads), 0, s, zt, zd, bf16, y, ua, us, G, V, tau,
                     ws, A, tok, status, margin);
  return hipGetLastError();
}

}  // namespace mtp
