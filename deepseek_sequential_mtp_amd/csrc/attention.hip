// Segment-causal multi-head attention of the MTP block (M7.6 0x03C: the
// block attends under a causal mask; 0x04C: the segment rule shapes the
// attention graph, not only the loss).  Query row i of a batch row sees keys
// j with run_start(i) <= j <= i (a padding row: itself only); scores are
// scaled by 1/sqrt(hd), softmax in float32 with an online max.
//
// Layout: qkv [B*T, 3*A] (q | k | v, head h at columns h*hd), out [B*T, A].
// One block = 4 waves = 128 queries of one (batch row, head); each wave owns
// 32 queries (two 16-query MFMA blocks).  Per key tile the wave computes
// S^T = K Q^T (keys on MFMA rows, queries on columns), so every softmax
// statistic of a query lives in one lane column: 16 values in-lane plus a
// reduction over the 4 lane groups.  P^T goes straight from the result
// registers into the B operand of O^T = V^T P^T; V is staged transposed in
// LDS with the key order permuted to match the result layout.
#include "kernels.hpp"

namespace mtp {

namespace {
constexpr int kAttnThreads = 256;
constexpr int kQW = 32;                       // queries per wave
constexpr int kQT = 4 * kQW;                  // queries per block

template <typename T> struct AttnCfg {
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int KT = 128 / Elem<T>::kBytes;   // keys per tile (V^T rows = 128 B)
};

// Physical position of key k (0 <= k < KT) inside a V^T row.  The O^T MFMA
// consumes, in lane group g and chunk element e, key 16*(e/4) + 4*g + e%4 of a
// 32-key step (bf16) or key 4*g + e of a 16-key step (f32); those keys are
// placed contiguously.
__device__ __forceinline__ int vt_pos(int k, bf16_t) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}
__device__ __forceinline__ int vt_pos(int k, float) { return k; }
// The key held by element e of physical chunk c (inverse of vt_pos).
__device__ __forceinline__ int vt_key(int c, int e, bf16_t) {
  return 32 * (c >> 2) + 16 * (e >> 2) + 4 * (c & 3) + (e & 3);
}
__device__ __forceinline__ int vt_key(int c, int e, float) { return 4 * c + e; }

template <int CPR>
__device__ __forceinline__ int swz(int row, int chunk) {
  constexpr int m = (CPR < 8 ? CPR : 8) - 1;
  return row * (CPR * 16) + ((chunk ^ (row & m)) << 4);
}

// P in bf16 for the O^T MFMA as hi + lo: hi = bf16(p), lo = bf16(p - hi), so
// the product carries ~16 mantissa bits of p instead of 8 (the probabilities
// are not a stored tensor of the method and get no bf16 rounding point).
__device__ __forceinline__ void pack_p2(const f32x4 &a, const f32x4 &b, uint4 &hi, uint4 &lo) {
  const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  hi = f32_to_chunk(v, bf16_t{});
  float r[8];
  const uint32_t w[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = v[2 * i] - bf16_to_f32(static_cast<uint16_t>(w[i] & 0xffff));
    r[2 * i + 1] = v[2 * i + 1] - bf16_to_f32(static_cast<uint16_t>(w[i] >> 16));
  }
  lo = f32_to_chunk(r, bf16_t{});
}
__device__ __forceinline__ uint4 pack_p(const f32x4 &a, const f32x4 &, float) {
  return make_uint4(__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                    __float_as_uint(a[3]));
}
}  // namespace

template <typename T, int HD>
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(const T *__restrict__ qkv,
                                                                T *__restrict__ out,
                                                                const int32_t *__restrict__ run_start,
                                                                int B, int T_len, int H, float scale_log2) {
  using C = AttnCfg<T>;
  constexpr int E = C::E, KT = C::KT;
  constexpr int CPR_K = HD * Elem<T>::kBytes / 16;   // chunks per K row
  constexpr int SK = HD / (4 * E);                   // MFMA steps over head dim
  constexpr int MBK = KT / 16;                       // key blocks per tile
  constexpr int MBD = HD / 16;                       // head-dim blocks
  constexpr int SV = KT / (4 * E);                   // MFMA steps over keys
  constexpr int K_BYTES = KT * HD * Elem<T>::kBytes;
  constexpr int V_BYTES = HD * 128;
  constexpr int O_BYTES = kQT * HD * Elem<T>::kBytes;
  constexpr int LDS = (K_BYTES + V_BYTES) > O_BYTES ? (K_BYTES + V_BYTES) : O_BYTES;
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  char *ldsK = lds;
  char *ldsV = lds + K_BYTES;

  const int A = H * HD;
  const long ld = 3L * A;
  const int nqt = (T_len + kQT - 1) / kQT;
  const int total = nqt * H * B;
  const int logical = xcd_remap(blockIdx.x, total);
  const int qt = nqt - 1 - (logical % nqt);          // long query tiles first
  const int h = (logical / nqt) % H;
  const int b = logical / (nqt * H);
  const int q0 = qt * kQT;
  const long rowbase = (long)b * T_len;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, c16 = lane & 15;

  // this lane's queries and their windows
  int qi[2], rsq[2];
  uint4 qreg[2][SK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qi[qb] = q0 + wave * kQW + qb * 16 + c16;
    const bool ok = qi[qb] < T_len;
    rsq[qb] = ok ? run_start[rowbase + qi[qb]] : 0;
    const T *qp = qkv + (rowbase + (ok ? qi[qb] : 0)) * ld + (long)h * HD;
#pragma unroll
    for (int s = 0; s < SK; ++s)
      qreg[qb][s] = ok ? reinterpret_cast<const uint4 *>(qp)[4 * s + g] : make_uint4(0, 0, 0, 0);
  }
  const int qlast = min(q0 + kQT, T_len) - 1;
  const int kbeg = run_start[rowbase + q0] / KT * KT;
  // wave bounds: smallest window start and largest query of the wave
  const int wq_lo = q0 + wave * kQW;
  const int wq_hi = min(wq_lo + kQW, T_len) - 1;
  const int w_rs = wq_lo < T_len ? run_start[rowbase + wq_lo] : 0;

  f32x4 o[MBD][2];
#pragma unroll
  for (int i = 0; i < MBD; ++i)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[i][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

  const T *kbase = qkv + rowbase * ld + A + (long)h * HD;
  const T *vbase = qkv + rowbase * ld + 2L * A + (long)h * HD;

  for (int k0 = kbeg; k0 <= qlast; k0 += KT) {
    // ---- stage K (row-major, swizzled) and V^T (permuted keys) in LDS
    for (int cidx = t; cidx < KT * CPR_K; cidx += kAttnThreads) {
      const int kr = cidx / CPR_K, ch = cidx % CPR_K;
      const int key = k0 + kr;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < T_len) v = reinterpret_cast<const uint4 *>(kbase + (long)key * ld)[ch];
      *reinterpret_cast<uint4 *>(ldsK + swz<CPR_K>(kr, ch)) = v;
    }
    {
      constexpr int NCH = KT / E;                     // physical chunks per V^T row
      constexpr int NBLK = NCH * (HD / E);
      for (int blk = t; blk < NBLK; blk += kAttnThreads) {
        const int c = blk % NCH, db = blk / NCH;
        uint4 r[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int key = k0 + vt_key(c, e, T{});
          r[e] = key < T_len ? reinterpret_cast<const uint4 *>(vbase + (long)key * ld)[db]
                             : make_uint4(0, 0, 0, 0);
        }
        transpose_chunks(r, T{});
#pragma unroll
        for (int j = 0; j < E; ++j) *reinterpret_cast<uint4 *>(ldsV + lds_off128(db * E + j, c)) = r[j];
      }
    }
    __syncthreads();

    const bool active = wq_lo < T_len && k0 <= wq_hi && k0 + KT - 1 >= w_rs;
    if (active) {
      // ---- S^T = K Q^T
      f32x4 s[MBK][2];
#pragma unroll
      for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) s[mb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < SK; ++st) {
#pragma unroll
        for (int mb = 0; mb < MBK; ++mb) {
          const uint4 a = *reinterpret_cast<const uint4 *>(ldsK + swz<CPR_K>(mb * 16 + c16, 4 * st + g));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) mma16(a, qreg[qb][st], s[mb][qb], T{});
        }
      }
      // ---- mask, online softmax
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = k0 + mb * 16 + 4 * g + r;
            const bool ok = qi[qb] < T_len && key <= qi[qb] && key >= rsq[qb];
            const float x = ok ? s[mb][qb][r] * scale_log2 : -INFINITY;
            s[mb][qb][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m[qb], mx);
        const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(m[qb] - mnew);
        float ls = 0.f;
#pragma unroll
        for (int mb = 0; mb < MBK; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = (mnew == -INFINITY) ? 0.f : exp2f(s[mb][qb][r] - mnew);
            s[mb][qb][r] = p;
            ls += p;
          }
        l[qb] = l[qb] * alpha + ls;
        m[qb] = mnew;
#pragma unroll
        for (int db = 0; db < MBD; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[db][qb][r] *= alpha;
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int sv = 0; sv < SV; ++sv) {
        uint4 pb[2], pl[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if constexpr (E == 8) pack_p2(s[2 * sv][qb], s[2 * sv + 1][qb], pb[qb], pl[qb]);
          else pb[qb] = pack_p(s[sv][qb], s[sv][qb], T{});
        }
#pragma unroll
        for (int db = 0; db < MBD; ++db) {
          const uint4 a = *reinterpret_cast<const uint4 *>(ldsV + lds_off128(db * 16 + c16, 4 * sv + g));
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            mma16(a, pb[qb], o[db][qb], T{});
            if constexpr (E == 8) mma16(a, pl[qb], o[db][qb], T{});
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- normalise, stage [query][dh] in LDS, coalesced stores
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float lt = l[qb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int ql = wave * kQW + qb * 16 + c16;
    T *orow = reinterpret_cast<T *>(lds) + (long)ql * HD;
#pragma unroll
    for (int db = 0; db < MBD; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) store_elem(orow, db * 16 + 4 * g + r, o[db][qb][r] * inv);
  }
  __syncthreads();
  constexpr int OCH = HD / E;   // chunks per output row
  for (int cidx = t; cidx < kQT * OCH; cidx += kAttnThreads) {
    const int ql = cidx / OCH, ch = cidx % OCH;
    const int q = q0 + ql;
    if (q >= T_len) continue;
    const uint4 v = reinterpret_cast<const uint4 *>(lds + (long)ql * HD * Elem<T>::kBytes)[ch];
    reinterpret_cast<uint4 *>(out + (rowbase + q) * (long)A + (long)h * HD)[ch] = v;
  }
}

template <typename T, int HD>
static hipError_t attn_launch(const T *qkv, T *out, const int32_t *rs, int B, int T_len, int H,
                              hipStream_t s) {
  const int nqt = (T_len + kQT - 1) / kQT;
  const long blocks = (long)nqt * H * B;
  const float scale_log2 = kLog2e / sqrtf((float)HD);
  hipLaunchKernelGGL((attention_kernel<T, HD>), dim3((unsigned)blocks), dim3(kAttnThreads), 0, s, qkv, out,
                     rs, B, T_len, H, scale_log2);
  return hipGetLastError();
}

template <>
hipError_t launch_attention<bf16_t>(const bf16_t *qkv, bf16_t *out, const int32_t *rs, int B, int T_len,
                                    int H, int hd, hipStream_t s) {
  switch (hd) {
    case 32: return attn_launch<bf16_t, 32>(qkv, out, rs, B, T_len, H, s);
    case 64: return attn_launch<bf16_t, 64>(qkv, out, rs, B, T_len, H, s);
    case 128: return attn_launch<bf16_t, 128>(qkv, out, rs, B, T_len, H, s);
    case 256: return attn_launch<bf16_t, 256>(qkv, out, rs, B, T_len, H, s);
    default: return hipErrorInvalidValue;
  }
}
template <>
hipError_t launch_attention<float>(const float *qkv, float *out, const int32_t *rs, int B, int T_len, int H,
                                   int hd, hipStream_t s) {
  switch (hd) {
    case 16: return attn_launch<float, 16>(qkv, out, rs, B, T_len, H, s);
    case 32: return attn_launch<float, 32>(qkv, out, rs, B, T_len, H, s);
    case 64: return attn_launch<float, 64>(qkv, out, rs, B, T_len, H, s);
    case 128: return attn_launch<float, 128>(qkv, out, rs, B, T_len, H, s);
    default: return hipErrorInvalidValue;
  }
}

// RoPE table: table[p][j] = (cos(p w_j), sin(p w_j)), w_j = theta^(-2j/hd),
// evaluated in double precision, p < max_pos, j < half.
__global__ void rope_table_kernel(float2 *table, int max_pos, int half, double theta) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)max_pos * half) return;
  const int p = (int)(i / half), j = (int)(i % half);
  const double w = pow(theta, -2.0 * j / (2.0 * half));
  double sn, cs;
  sincos((double)p * w, &sn, &cs);
  table[i] = make_float2((float)cs, (float)sn);
}

hipError_t rope_table(float2 *table, int max_pos, int half, float theta, hipStream_t s) {
  const long n = (long)max_pos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, table, max_pos,
                     half, (double)theta);
  return hipGetLastError();
}

}  // namespace mtp
