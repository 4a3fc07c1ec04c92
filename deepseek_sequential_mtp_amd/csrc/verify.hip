// Exact speculative verification (M7.6 0x09 for one proposal; the
// speculative-decoding explainer page for gamma proposals).
//
// Pass 1 (one block per logit row, all rows of all requests): log-sum-exp of
// z / tau in float64 (exponentials and sums), plus a finiteness flag.  A
// float32 exponential would leave a ~1e-7 relative error in p / q and in the
// CDF, the size of one token's mass at V ~ 1e5; float64 keeps every decision
// exact up to ~1e-13.  The row is read once: each lane keeps a running max
// (float) and a float64 sum rescaled when its max rises, and the lanes' pairs
// are merged at the end.  Pass 2 (one block per request): the left-to-right
// ratio tests in float64, then the draw from the normalised residual
// (p_A - q_A)+ or from p_gamma by inverse CDF over ascending token ids
// (smallest t with cdf(t) > u * mass): chunk and tile sums of the weights
// first (across the chip), then per request the crossing tile from the tile
// sums and the crossing chunk from one block-wide prefix sum.
//
// Rows are read in chunks of E consecutive logits per lane (16 bytes: E = 8
// for bf16, 4 for f32) when V is a multiple of E, so every row starts on a
// chunk; otherwise element by element (E = 1).
#include "kernels.hpp"

namespace mtp {

namespace {
constexpr int kVThreads = 256;

// exp(x) in float64 by Tang's table-driven method (ACM TOMS 15(2), 1989),
// with a 256-entry table: x = (256 m + j) ln2/256 + r with |r| <= ln2/512,
// exp(x) = 2^m 2^(j/256) exp(r), exp(r) by its Taylor polynomial of degree 3
// (truncation |r|^4/24 below 1.4e-13 relative: the decisions built on these
// sums need far less than their 1e-9 tie window, and degree 4 costs one more
// float64 FMA per logit).  k = 256 m + j is rounded by adding 1.5 * 2^52
// (the integer then sits in the low mantissa bits), and r = x - k ln2/256
// takes one fused multiply-add with ln2/256 rounded to a double: the error
// |k| * 2^-64 is below 1e-16 relative for x >= -1 and smaller than the
// value's own rounding for every x where exp(x) still counts against a sum
// >= 1.  The values 2^(j/256) are correctly rounded doubles (a 60-digit
// decimal evaluation).  x <= -746 (and -inf) gives 0; the callers' arguments
// are <= 0 and not NaN (finiteness is checked apart).
__constant__ double kExp2Frac[256] = {
    0x1.0000000000000p+0, 0x1.00b1afa5abcbfp+0, 0x1.0163da9fb3335p+0, 0x1.02168143b0281p+0,
    0x1.02c9a3e778061p+0, 0x1.037d42e11bbccp+0, 0x1.04315e86e7f85p+0, 0x1.04e5f72f654b1p+0,
    0x1.059b0d3158574p+0, 0x1.0650a0e3c1f89p+0, 0x1.0706b29ddf6dep+0, 0x1.07bd42b72a836p+0,
    0x1.0874518759bc8p+0, 0x1.092bdf66607e0p+0, 0x1.09e3ecac6f383p+0, 0x1.0a9c79b1f3919p+0,
    0x1.0b5586cf9890fp+0, 0x1.0c0f145e46c85p+0, 0x1.0cc922b7247f7p+0, 0x1.0d83b23395decp+0,
    0x1.0e3ec32d3d1a2p+0, 0x1.0efa55fdfa9c5p+0, 0x1.0fb66affed31bp+0, 0x1.1073028d7233ep+0,
    0x1.11301d0125b51p+0, 0x1.11edbab5e2ab6p+0, 0x1.12abdc06c31ccp+0, 0x1.136a814f204abp+0,
    0x1.1429aaea92de0p+0, 0x1.14e95934f312ep+0, 0x1.15a98c8a58e51p+0, 0x1.166a45471c3c2p+0,
    0x1.172b83c7d517bp+0, 0x1.17ed48695bbc0p+0, 0x1.18af9388c8deap+0, 0x1.1972658375d2fp+0,
    0x1.1a35beb6fcb75p+0, 0x1.1af99f8138a1cp+0, 0x1.1bbe084045cd4p+0, 0x1.1c82f95281c6bp+0,
    0x1.1d4873168b9aap+0, 0x1.1e0e75eb44027p+0, 0x1.1ed5022fcd91dp+0, 0x1.1f9c18438ce4dp+0,
    0x1.2063b88628cd6p+0, 0x1.212be3578a819p+0, 0x1.21f49917ddc96p+0, 0x1.22bdda27912d1p+0,
    0x1.2387a6e756238p+0, 0x1.2451ffb82140ap+0, 0x1.251ce4fb2a63fp+0, 0x1.25e85711ece75p+0,
    0x1.26b4565e27cddp+0, 0x1.2780e341ddf29p+0, 0x1.284dfe1f56381p+0, 0x1.291ba7591bb70p+0,
    0x1.29e9df51fdee1p+0, 0x1.2ab8a66d10f13p+0, 0x1.2b87fd0dad990p+0, 0x1.2c57e39771b2fp+0,
    0x1.2d285a6e4030bp+0, 0x1.2df961f641589p+0, 0x1.2ecafa93e2f56p+0, 0x1.2f9d24abd886bp+0,
    0x1.306fe0a31b715p+0, 0x1.31432edeeb2fdp+0, 0x1.32170fc4cd831p+0, 0x1.32eb83ba8ea32p+0,
    0x1.33c08b26416ffp+0, 0x1.3496266e3fa2dp+0, 0x1.356c55f929ff1p+0, 0x1.36431a2de883bp+0,
    0x1.371a7373aa9cbp+0, 0x1.37f26231e754ap+0, 0x1.38cae6d05d866p+0, 0x1.39a401b7140efp+0,
    0x1.3a7db34e59ff7p+0, 0x1.3b57fbfec6cf4p+0, 0x1.3c32dc313a8e5p+0, 0x1.3d0e544ede173p+0,
    0x1.3dea64c123422p+0, 0x1.3ec70df1c5175p+0, 0x1.3fa4504ac801cp+0, 0x1.40822c367a024p+0,
    0x1.4160a21f72e2ap+0, 0x1.423fb2709468ap+0, 0x1.431f5d950a897p+0, 0x1.43ffa3f84b9d4p+0,
    0x1.44e086061892dp+0, 0x1.45c2042a7d232p+0, 0x1.46a41ed1d0057p+0, 0x1.4786d668b3237p+0,
    0x1.486a2b5c13cd0p+0, 0x1.494e1e192aed2p+0, 0x1.4a32af0d7d3dep+0, 0x1.4b17dea6db7d7p+0,
    0x1.4bfdad5362a27p+0, 0x1.4ce41b817c114p+0, 0x1.4dcb299fddd0dp+0, 0x1.4eb2d81d8abffp+0,
    0x1.4f9b2769d2ca7p+0, 0x1.508417f4531eep+0, 0x1.516daa2cf6642p+0, 0x1.5257de83f4eefp+0,
    0x1.5342b569d4f82p+0, 0x1.542e2f4f6ad27p+0, 0x1.551a4ca5d920fp+0, 0x1.56070dde910d2p+0,
    0x1.56f4736b527dap+0, 0x1.57e27dbe2c4cfp+0, 0x1.58d12d497c7fdp+0, 0x1.59c0827ff07ccp+0,
    0x1.5ab07dd485429p+0, 0x1.5ba11fba87a03p+0, 0x1.5c9268a5946b7p+0, 0x1.5d84590998b93p+0,
    0x1.5e76f15ad2148p+0, 0x1.5f6a320dceb71p+0, 0x1.605e1b976dc09p+0, 0x1.6152ae6cdf6f4p+0,
    0x1.6247eb03a5585p+0, 0x1.633dd1d1929fdp+0, 0x1.6434634ccc320p+0, 0x1.652b9febc8fb7p+0,
    0x1.6623882552225p+0, 0x1.671c1c70833f6p+0, 0x1.68155d44ca973p+0, 0x1.690f4b19e9538p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6b052fa75173ep+0, 0x1.6c012750bdabfp+0, 0x1.6cfdcddd47645p+0,
    0x1.6dfb23c651a2fp+0, 0x1.6ef9298593ae5p+0, 0x1.6ff7df9519484p+0, 0x1.70f7466f42e87p+0,
    0x1.71f75e8ec5f74p+0, 0x1.72f8286ead08ap+0, 0x1.73f9a48a58174p+0, 0x1.74fbd35d7cbfdp+0,
    0x1.75feb564267c9p+0, 0x1.77024b1ab6e09p+0, 0x1.780694fde5d3fp+0, 0x1.790b938ac1cf6p+0,
    0x1.7a11473eb0187p+0, 0x1.7b17b0976cfdbp+0, 0x1.7c1ed0130c132p+0, 0x1.7d26a62ff86f0p+0,
    0x1.7e2f336cf4e62p+0, 0x1.7f3878491c491p+0, 0x1.80427543e1a12p+0, 0x1.814d2add106d9p+0,
    0x1.82589994cce13p+0, 0x1.8364c1eb941f7p+0, 0x1.8471a4623c7adp+0, 0x1.857f4179f5b21p+0,
    0x1.868d99b4492edp+0, 0x1.879cad931a436p+0, 0x1.88ac7d98a6699p+0, 0x1.89bd0a478580fp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8be05bad61778p+0, 0x1.8cf3216b5448cp+0, 0x1.8e06a5e0866d9p+0,
    0x1.8f1ae99157736p+0, 0x1.902fed0282c8ap+0, 0x1.9145b0b91ffc6p+0, 0x1.925c353aa2fe2p+0,
    0x1.93737b0cdc5e5p+0, 0x1.948b82b5f98e5p+0, 0x1.95a44cbc8520fp+0, 0x1.96bdd9a7670b3p+0,
    0x1.97d829fde4e50p+0, 0x1.98f33e47a22a2p+0, 0x1.9a0f170ca07bap+0, 0x1.9b2bb4d53fe0dp+0,
    0x1.9c49182a3f090p+0, 0x1.9d674194bb8d5p+0, 0x1.9e86319e32323p+0, 0x1.9fa5e8d07f29ep+0,
    0x1.a0c667b5de565p+0, 0x1.a1e7aed8eb8bbp+0, 0x1.a309bec4a2d33p+0, 0x1.a42c980460ad8p+0,
    0x1.a5503b23e255dp+0, 0x1.a674a8af46052p+0, 0x1.a799e1330b358p+0, 0x1.a8bfe53c12e59p+0,
    0x1.a9e6b5579fdbfp+0, 0x1.ab0e521356ebap+0, 0x1.ac36bbfd3f37ap+0, 0x1.ad5ff3a3c2774p+0,
    0x1.ae89f995ad3adp+0, 0x1.afb4ce622f2ffp+0, 0x1.b0e07298db666p+0, 0x1.b20ce6c9a8952p+0,
    0x1.b33a2b84f15fbp+0, 0x1.b468415b749b1p+0, 0x1.b59728de5593ap+0, 0x1.b6c6e29f1c52ap+0,
    0x1.b7f76f2fb5e47p+0, 0x1.b928cf22749e4p+0, 0x1.ba5b030a1064ap+0, 0x1.bb8e0b79a6f1fp+0,
    0x1.bcc1e904bc1d2p+0, 0x1.bdf69c3f3a207p+0, 0x1.bf2c25bd71e09p+0, 0x1.c06286141b33dp+0,
    0x1.c199bdd85529cp+0, 0x1.c2d1cd9fa652cp+0, 0x1.c40ab5fffd07ap+0, 0x1.c544778fafb22p+0,
    0x1.c67f12e57d14bp+0, 0x1.c7ba88988c933p+0, 0x1.c8f6d9406e7b5p+0, 0x1.ca3405751c4dbp+0,
    0x1.cb720dcef9069p+0, 0x1.ccb0f2e6d1675p+0, 0x1.cdf0b555dc3fap+0, 0x1.cf3155b5bab74p+0,
    0x1.d072d4a07897cp+0, 0x1.d1b532b08c968p+0, 0x1.d2f87080d89f2p+0, 0x1.d43c8eacaa1d6p+0,
    0x1.d5818dcfba487p+0, 0x1.d6c76e862e6d3p+0, 0x1.d80e316c98398p+0, 0x1.d955d71ff6075p+0,
    0x1.da9e603db3285p+0, 0x1.dbe7cd63a8315p+0, 0x1.dd321f301b460p+0, 0x1.de7d5641c0658p+0,
    0x1.dfc97337b9b5fp+0, 0x1.e11676b197d17p+0, 0x1.e264614f5a129p+0, 0x1.e3b333b16ee12p+0,
    0x1.e502ee78b3ff6p+0, 0x1.e653924676d76p+0, 0x1.e7a51fbc74c83p+0, 0x1.e8f7977cdb740p+0,
    0x1.ea4afa2a490dap+0, 0x1.eb9f4867cca6ep+0, 0x1.ecf482d8e67f1p+0, 0x1.ee4aaa2188510p+0,
    0x1.efa1bee615a27p+0, 0x1.f0f9c1cb6412ap+0, 0x1.f252b376bba97p+0, 0x1.f3ac948dd7274p+0,
    0x1.f50765b6e4540p+0, 0x1.f6632798844f8p+0, 0x1.f7bfdad9cbe14p+0, 0x1.f91d802243c89p+0,
    0x1.fa7c1819e90d8p+0, 0x1.fbdba3692d514p+0, 0x1.fd3c22b8f71f1p+0, 0x1.fe9d96b2a23d9p+0};
constexpr double kInvLn2_256 = 0x1.71547652b82fep+8;  // 256 / ln 2
constexpr double kLn2_256 = 0x1.62e42fefa39efp-9;     // ln 2 / 256
constexpr double kRoundShift = 0x1.8p52;

// The block's copy of kExp2Frac in LDS (indexed per lane).
__device__ __forceinline__ void load_exp_table(double *tab) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) tab[i] = kExp2Frac[i];
  __syncthreads();
}

__device__ __forceinline__ double exp_tang(double x, const double *tab) {
  x = fmax(x, -746.0);
  const double t = fma(x, kInvLn2_256, kRoundShift);
  const double k = t - kRoundShift;
  const int ki = __double2loint(t);   // k as a 32-bit integer
  const double r = fma(-k, kLn2_256, x);
  double p = fma(r, 1.0 / 6.0, 0.5);                 // 1 + r + r^2/2 + r^3/6
  p = fma(r, p, 1.0);
  p = fma(r, p, 1.0);
  return ldexp(tab[ki & 255] * p, ki >> 8);
}

// exp_tang for the log-sum-exp loop, whose arguments the caller keeps at or
// above -700 (so the power of two 2^m, m >= -1011, stays a normal number):
// the scaling is an integer add to the exponent field of the table value,
// which gives the same bits as ldexp of the product (a power-of-two scaling
// of a normal number is exact either way).  NaN and +inf arguments give NaN.
__device__ __forceinline__ double exp_tang_ge700(double x, const double *tab) {
  const double t = fma(x, kInvLn2_256, kRoundShift);
  const double k = t - kRoundShift;
  const int ki = __double2loint(t);
  const double r = fma(-k, kLn2_256, x);
  double p = fma(r, 1.0 / 6.0, 0.5);
  p = fma(r, p, 1.0);
  p = fma(r, p, 1.0);
  const double e = tab[ki & 255];
  const double es = __hiloint2double(__double2hiint(e) + ((ki >> 8) << 20), __double2loint(e));
  return es * p;
}

// 1 if any of the chunk's logits is NaN or +inf (bf16: from the raw bits).
template <typename T, int E>
__device__ __forceinline__ int chunk_bad(const T *p, const float (&v)[E]) {
  int bad = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) bad |= (isnan(v[e]) || v[e] == INFINITY) ? 1 : 0;
  return bad;
}

template <typename T, int E>
__device__ __forceinline__ void load_chunk(const T *p, float (&v)[E]) {
  if constexpr (E == 8) {
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo_f32(a[i]);
      v[2 * i + 1] = bf16_hi_f32(a[i]);
    }
  } else if constexpr (E == 4) {
    const float4 w = *reinterpret_cast<const float4 *>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  } else {
    v[0] = load_elem(p, 0);
  }
}

// Block-wide reductions over the kVThreads lanes (sh: kVThreads / 64 slots).
__device__ __forceinline__ double block_sum(double v, double *sh) {
  v = warp_sum(v);
  const int t = threadIdx.x;
  __syncthreads();
  if ((t & 63) == 0) sh[t >> 6] = v;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < kVThreads / 64; ++i) tot += sh[i];
  return tot;
}
}  // namespace

// ws layout per request r and row index j in [0, 2G+1):
//   ws[(r*(2G+1) + j)*2 + 0] = lse (double), [.. + 1] = 1.0 if finite else 0.0
// rows j <= G are target rows, j > G draft rows (j - G - 1).
template <typename T, int E>
__global__ __launch_bounds__(kVThreads) void verify_lse_kernel(const T *zt, const T *zd, int G, int V, float tau,
                                                              double *ws) {
  __shared__ float shm[kVThreads / 64];
  __shared__ double shs[kVThreads / 64];
  __shared__ int shb[kVThreads / 64];
  __shared__ double tab[256];
  load_exp_table(tab);
  const int nrow = 2 * G + 1;
  const long rid = blockIdx.x;
  const int r = (int)(rid / nrow), j = (int)(rid % nrow);
  const T *row = j <= G ? zt + ((long)r * (G + 1) + j) * V : zd + ((long)r * G + (j - G - 1)) * V;
  const float inv_tau = 1.f / tau;
  const double dtau = 1.0 / (double)tau;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  // lane-private running max (float, of z / tau) and sum of exp(z / tau - max)
  float m = -INFINITY;
  double s = 0.0;
  int bad = 0;
  const int nchunk = V / E;
  // z / tau > max(z) / tau for finite z: the max is taken on raw logits
  // (tau > 0 keeps the order), the finiteness test once per chunk; NaN and
  // +inf poison the row, -inf contributes exp(-inf) = 0
  // A NaN or +inf logit needs no test of its own once the lane has a finite
  // running max: it turns the lane's sum into NaN (exp_tang_ge700 of NaN, or
  // of +inf - inf once the running max is +inf), which the merge below flags.  Arguments are kept
  // at or above -700 by clamping the logit in float before the conversion
  // (lo: the logit whose argument is -700 at this max); the comparison keeps
  // NaN, and a clamped term is below e^-700 of the max's term.
  float lo = -INFINITY;
  auto consume = [&](const float (&v)[E]) {
    float cm = v[0];
#pragma unroll
    for (int e = 1; e < E; ++e) cm = fmaxf(cm, v[e]);
    cm *= inv_tau;
    if (cm > m) {
      if (m != -INFINITY) s *= exp_tang((double)m - (double)cm, tab);
      m = cm;
      // below -FLT_MAX every finite logit already meets the bound; -inf is
      // then lifted to -FLT_MAX, which meets it too
      lo = (float)fmax((-700.0 + (double)m) * (double)tau, -3.4028234663852886e38);
    }
    if (m == -INFINITY) {
      // no finite logit yet: this chunk holds only -inf (nothing to add) or NaN
      bad |= chunk_bad<T, E>(nullptr, v);
      return;
    }
    const double nm = -(double)m;
    double cs = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float vc = v[e] < lo ? lo : v[e];
      cs += exp_tang_ge700(fma((double)vc, dtau, nm), tab);
    }
    s += cs;
  };
  // four chunks in flight per lane, then their arithmetic
  constexpr int U = 4;
  int c = t;
  for (; c + (U - 1) * kVThreads < nchunk; c += U * kVThreads) {
    float v[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) load_chunk<T, E>(row + (long)(c + u * kVThreads) * E, v[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) consume(v[u]);
  }
  for (; c < nchunk; c += kVThreads) {
    float v[E];
    load_chunk<T, E>(row + (long)c * E, v);
    consume(v);
  }
  // merge the lanes' (max, sum) pairs
  bad |= (isnan(s) || m == INFINITY) ? 1 : 0;
  float mx = warp_max(m);
  for (int o = 32; o > 0; o >>= 1) bad |= __shfl_xor(bad, o);
  if (lane == 0) { shm[w] = mx; shb[w] = bad; }
  __syncthreads();
  mx = shm[0];
  bad = shb[0];
  for (int i = 1; i < kVThreads / 64; ++i) { mx = fmaxf(mx, shm[i]); bad |= shb[i]; }
  if (mx == -INFINITY || isnan(mx)) bad = 1;
  const double part = (!bad && m != -INFINITY) ? s * exp_tang((double)m - (double)mx, tab) : 0.0;
  const double tot = block_sum(part, shs);
  if (t == 0) {
    ws[rid * 2] = bad ? 0.0 : (double)mx + log(tot);
    ws[rid * 2 + 1] = bad ? 0.0 : 1.0;
  }
}

// Outcome of the ratio tests of one request.
struct VerifyState {
  int A, st;
  double margin;
};

// One thread per request: uniform and token checks, then the left-to-right
// ratio tests in float64 (A = first rejection, gamma if none).
template <typename T>
__global__ __launch_bounds__(kVThreads) void verify_tests_kernel(
    const T *zt, const T *zd, const int32_t *__restrict__ y, const float *__restrict__ ua,
    const float *__restrict__ us, int R, int G, int V, float tau, const double *__restrict__ ws,
    VerifyState *__restrict__ vs) {
  const int r = blockIdx.x * kVThreads + threadIdx.x;
  if (r >= R) return;
  const double *wr = ws + (long)r * (2 * G + 1) * 2;
  const double itau = 1.0 / (double)tau;
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
      const double p = exp((double)load_elem(zt, ((long)r * (G + 1) + j) * V + yj) * itau - wr[2 * j]);
      const double q = exp((double)load_elem(zd, ((long)r * G + j) * V + yj) * itau - wr[2 * (G + 1 + j)]);
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
  vs[r] = VerifyState{A, st, margin};
}

// Weights of the emission distribution of request r (p_A, or (p_A - q_A)+
// after a rejection) for the E tokens of chunk c.
template <typename T, int E>
struct Emission {
  const T *rowp, *rowq;
  const double *tab;
  double lp, lq, itau;
  bool resid;
  __device__ __forceinline__ Emission(const T *zt, const T *zd, const double *ws, int r, int A, int G, int V,
                                      float tau, const double *tab_) : tab(tab_) {
    const double *wr = ws + (long)r * (2 * G + 1) * 2;
    resid = A < G;
    rowp = zt + ((long)r * (G + 1) + A) * V;
    rowq = zd + (resid ? ((long)r * G + A) * V : 0);
    lp = wr[2 * A];
    lq = resid ? wr[2 * (G + 1 + A)] : 0.0;
    itau = 1.0 / (double)tau;
  }
  __device__ __forceinline__ void weights(int c, double (&wv)[E]) const {
    float pv[E], qv[E];
    load_chunk<T, E>(rowp + (long)c * E, pv);
    if (resid) load_chunk<T, E>(rowq + (long)c * E, qv);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double p = exp_tang(fma((double)pv[e], itau, -lp), tab);
      if (resid) {
        const double q = exp_tang(fma((double)qv[e], itau, -lq), tab);
        wv[e] = p > q ? p - q : 0.0;
      } else {
        wv[e] = p;
      }
    }
  }
};

// Chunk sums of the emission weights, csum[r * nchunk + c]; grid (chunk
// blocks, R): the whole chip works on the requests' rows at once.
// Block x covers the kVThreads chunks of tile x and also writes their sum,
// tsum[r * ntile + x].
template <typename T, int E>
__global__ __launch_bounds__(kVThreads) void verify_mass_kernel(const T *zt, const T *zd, int G, int V, float tau,
                                                               const double *__restrict__ ws,
                                                               const VerifyState *__restrict__ vs,
                                                               double *__restrict__ csum,
                                                               double *__restrict__ tsum) {
  __shared__ double tab[256];
  __shared__ double sRed[kVThreads / 64];
  const int r = blockIdx.y;
  const VerifyState v = vs[r];
  if (v.st != 0) return;
  load_exp_table(tab);
  const int nchunk = V / E;
  const int c = blockIdx.x * kVThreads + threadIdx.x;
  double sum = 0.0;
  if (c < nchunk) {
    const Emission<T, E> em(zt, zd, ws, r, v.A, G, V, tau, tab);
    double wv[E];
    em.weights(c, wv);
#pragma unroll
    for (int e = 0; e < E; ++e) sum += wv[e];
    csum[(long)r * nchunk + c] = sum;
  }
  const double tile = block_sum(sum, sRed);
  if (threadIdx.x == 0) tsum[(long)r * gridDim.x + blockIdx.x] = tile;
}

// One block per request: the total mass from the tile sums, the crossing
// tile by a running sum over the tiles in ascending order, then one
// block-wide prefix sum over that tile's chunk sums and the token inside the
// crossing chunk.
template <typename T, int E>
__global__ __launch_bounds__(kVThreads) void verify_pick_kernel(
    const T *zt, const T *zd, const float *__restrict__ us, int G, int V, float tau,
    const double *__restrict__ ws, const VerifyState *__restrict__ vs, const double *__restrict__ csum,
    const double *__restrict__ tsum, int32_t *__restrict__ A_out, int32_t *__restrict__ tok_out,
    int32_t *__restrict__ st_out, float *__restrict__ margin_out) {
  __shared__ int sTile, sTok;
  __shared__ double sBase, sW, sMargin;
  __shared__ double sScan[kVThreads];
  __shared__ double tab[256];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  const VerifyState v = vs[r];
  load_exp_table(tab);
  auto finish = [&](int A, int tok, int st, double margin) {
    A_out[r] = A;
    tok_out[r] = tok;
    st_out[r] = st;
    if (margin_out != nullptr) margin_out[r] = (float)margin;
  };
  if (v.st != 0) {
    if (t == 0) finish(0, -1, v.st, 0.0);
    return;
  }
  const int nchunk = V / E;
  const int ntile = (nchunk + kVThreads - 1) / kVThreads;
  const double *cs_r = csum + (long)r * nchunk;
  const double *ts_r = tsum + (long)r * ntile;
  const double u = (double)us[(long)r * (G + 1) + v.A];
  if (t == 0) {
    double W = 0.0;
    for (int k = 0; k < ntile; ++k) W += ts_r[k];
    const double target = u * W;
    double base = 0.0;
    int tile = -1;
    for (int k = 0; k < ntile; ++k) {
      const double nb = base + ts_r[k];
      if (ts_r[k] > 0.0 && base <= target && target < nb) { tile = k; break; }
      base = nb;
    }
    sW = W;
    sTile = tile;
    sBase = base;
    sTok = -1;
    sMargin = v.margin;
  }
  __syncthreads();
  const double W = sW;
  if (!(W > 0.0)) {
    if (t == 0) finish(0, -1, 4, 0.0);
    return;
  }
  const double target = u * W;
  const int tile = sTile;
  const Emission<T, E> em(zt, zd, ws, r, v.A, G, V, tau, tab);
  if (tile >= 0) {
    const int c = tile * kVThreads + t;
    const double cs = c < nchunk ? cs_r[c] : 0.0;
    // inclusive prefix sum of the tile's chunk sums (Hillis-Steele)
    sScan[t] = cs;
    __syncthreads();
    for (int o = 1; o < kVThreads; o <<= 1) {
      const double add = t >= o ? sScan[t - o] : 0.0;
      __syncthreads();
      sScan[t] += add;
      __syncthreads();
    }
    const double incl = sBase + sScan[t];
    const double excl = incl - cs;
    if (c < nchunk && cs > 0.0 && excl <= target && target < incl) {
      double wv[E];
      em.weights(c, wv);
      double cc = excl;
      int tok = -1, last = -1;
      double mg = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double cn = cc + wv[e];
        if (wv[e] > 0.0) last = c * E + e;
        if (tok < 0 && wv[e] > 0.0 && cn > target) {
          tok = c * E + e;
          mg = fmin(target - cc, cn - target) / W;
        }
        cc = cn;
      }
      if (tok < 0) { tok = last; mg = 0.0; }   // crossing lost to rounding: flagged by margin 0
      sTok = tok;
      sMargin = fmin(sMargin, mg);
    }
    __syncthreads();
  }
  if (t == 0) {
    int tok = sTok;
    double margin = sMargin;
    if (tok < 0) {   // target at or beyond the summed mass (rounding): last positive weight
      for (int c = nchunk - 1; c >= 0 && tok < 0; --c) {
        if (!(cs_r[c] > 0.0)) continue;
        double wv[E];
        em.weights(c, wv);
        for (int e = E - 1; e >= 0; --e)
          if (wv[e] > 0.0) { tok = c * E + e; break; }
      }
      margin = 0.0;
    }
    finish(v.A, tok, 0, margin);
  }
}

namespace {
template <typename T, int E>
void launch_verify_t(const T *zt, const T *zd, const int32_t *y, const float *ua, const float *us, int R, int G,
                     int V, float tau, int32_t *A, int32_t *tok, int32_t *status, float *margin, double *ws,
                     hipStream_t s) {
  const long rows = (long)R * (2 * G + 1);
  VerifyState *vs = reinterpret_cast<VerifyState *>(ws + rows * 2);
  double *csum = reinterpret_cast<double *>(vs + R);
  const int nchunk = V / E;
  const int ntile = (nchunk + kVThreads - 1) / kVThreads;
  double *tsum = csum + (long)R * nchunk;
  hipLaunchKernelGGL((verify_lse_kernel<T, E>), dim3((unsigned)rows), dim3(kVThreads), 0, s, zt, zd, G, V, tau,
                     ws);
  hipLaunchKernelGGL((verify_tests_kernel<T>), dim3((R + kVThreads - 1) / kVThreads), dim3(kVThreads), 0, s, zt,
                     zd, y, ua, us, R, G, V, tau, ws, vs);
  hipLaunchKernelGGL((verify_mass_kernel<T, E>), dim3(ntile, R), dim3(kVThreads), 0, s, zt, zd, G, V, tau, ws, vs,
                     csum, tsum);
  hipLaunchKernelGGL((verify_pick_kernel<T, E>), dim3(R), dim3(kVThreads), 0, s, zt, zd, us, G, V, tau, ws, vs,
                     csum, tsum, A, tok, status, margin);
}
}  // namespace

// Workspace of launch_verify: the row log-sum-exps, the test outcomes, the
// emission chunk sums and their tile sums.
size_t verify_workspace_bytes(int R, int G, int V, int bf16) {
  const int E = bf16 ? (V % 8 == 0 ? 8 : 1) : (V % 4 == 0 ? 4 : 1);
  const size_t nchunk = V / E, ntile = (nchunk + kVThreads - 1) / kVThreads;
  return (size_t)R * (2 * G + 1) * 2 * sizeof(double) + (size_t)R * sizeof(VerifyState) +
         (size_t)R * (nchunk + ntile) * sizeof(double);
}

hipError_t launch_verify(const void *zt, const void *zd, int bf16, const int32_t *y, const float *ua,
                         const float *us, int R, int G, int V, float tau, int32_t *A, int32_t *tok,
                         int32_t *status, float *margin, double *ws, hipStream_t s) {
  if (bf16) {
    const bf16_t *a = static_cast<const bf16_t *>(zt), *b = static_cast<const bf16_t *>(zd);
    if (V % 8 == 0) launch_verify_t<bf16_t, 8>(a, b, y, ua, us, R, G, V, tau, A, tok, status, margin, ws, s);
    else launch_verify_t<bf16_t, 1>(a, b, y, ua, us, R, G, V, tau, A, tok, status, margin, ws, s);
  } else {
    const float *a = static_cast<const float *>(zt), *b = static_cast<const float *>(zd);
    if (V % 4 == 0) launch_verify_t<float, 4>(a, b, y, ua, us, R, G, V, tau, A, tok, status, margin, ws, s);
    else launch_verify_t<float, 1>(a, b, y, ua, us, R, G, V, tau, A, tok, status, margin, ws, s);
  }
  return hipGetLastError();
}

// Proposer step, before any other launch: tokens and positions clamped into
// range for the kernels (a bad request still runs, on in-range values), the
// request's status for them, and iota[r] = r (the row index through which
// the QKV epilogue reads each request's rotary row).
__global__ void propose_prepare_kernel(const int32_t *__restrict__ tokens, const int32_t *__restrict__ positions,
                                       int R, int V, int L_max, int32_t *__restrict__ tok_s,
                                       int32_t *__restrict__ pos_s, int32_t *__restrict__ st,
                                       int32_t *__restrict__ iota) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  iota[r] = r;
  const int tk = tokens[r], ps = positions[r];
  const bool badp = ps < 0 || ps >= L_max;
  const bool badt = tk < 0 || tk >= V;
  tok_s[r] = badt ? 0 : tk;
  pos_s[r] = badp ? 0 : ps;
  st[r] = badp ? 6 : (badt ? 2 : 0);
}

// After the draw: a status from the preparation wins over the draw's.
__global__ void propose_finish_kernel(const int32_t *__restrict__ st_prep, const int32_t *__restrict__ st_draw,
                                      int R, int32_t *__restrict__ tok, int32_t *__restrict__ st_out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int sp = st_prep[r];
  const int st = sp != 0 ? sp : st_draw[r];
  st_out[r] = st;
  if (st != 0) tok[r] = -1;
}

// Round bookkeeping, one thread per request (the rules are in mtp.h).
__global__ void round_commit_kernel(int R, int G, int eos, const int32_t *__restrict__ drafts,
                                    const int32_t *__restrict__ A_in, const int32_t *__restrict__ tok_in,
                                    const int32_t *__restrict__ st_in, const int32_t *__restrict__ rem_in,
                                    int32_t *__restrict__ out_tok, int32_t *__restrict__ n_new,
                                    int32_t *__restrict__ keep, int32_t *__restrict__ pending,
                                    int32_t *__restrict__ stopped) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  const int A = A_in[r], rem = rem_in[r], t = tok_in[r];
  int32_t *o = out_tok + (long)r * (G + 1);
  int n = 0, pend = -1, stop = 1, kp = 0;
  if (st_in[r] == 0 && rem >= 1 && A >= 0 && A <= G) {
    kp = A + 1;
    stop = 0;
    for (int j = 0; j < A && !stop; ++j) {
      const int y = drafts[(long)r * G + j];
      o[n++] = y;
      stop = (n == rem || (eos >= 0 && y == eos)) ? 1 : 0;
    }
    if (!stop) {
      o[n++] = t;
      pend = t;
      stop = (n == rem || (eos >= 0 && t == eos)) ? 1 : 0;
    }
  }
  for (int j = n; j <= G; ++j) o[j] = -1;
  n_new[r] = n;
  keep[r] = kp;
  pending[r] = pend;
  stopped[r] = stop;
}

hipError_t launch_round_commit(int R, int G, int eos, const int32_t *drafts, const int32_t *A, const int32_t *tok,
                               const int32_t *st, const int32_t *rem, int32_t *out_tok, int32_t *n_new,
                               int32_t *keep, int32_t *pending, int32_t *stopped, hipStream_t s) {
  hipLaunchKernelGGL(round_commit_kernel, dim3((R + 255) / 256), dim3(256), 0, s, R, G, eos, drafts, A, tok, st,
                     rem, out_tok, n_new, keep, pending, stopped);
  return hipGetLastError();
}

hipError_t launch_propose_prepare(const int32_t *tokens, const int32_t *positions, int R, int V, int L_max,
                                  int32_t *tok_s, int32_t *pos_s, int32_t *st, int32_t *iota, hipStream_t s) {
  hipLaunchKernelGGL(propose_prepare_kernel, dim3((R + 255) / 256), dim3(256), 0, s, tokens, positions, R, V,
                     L_max, tok_s, pos_s, st, iota);
  return hipGetLastError();
}
hipError_t launch_propose_finish(const int32_t *st_prep, const int32_t *st_draw, int R, int32_t *tok,
                                 int32_t *st_out, hipStream_t s) {
  hipLaunchKernelGGL(propose_finish_kernel, dim3((R + 255) / 256), dim3(256), 0, s, st_prep, st_draw, R, tok,
                     st_out);
  return hipGetLastError();
}

}  // namespace mtp
