// Segment-causal multi-head attention of the MTP block (M7.6 0x03C: the
// block attends under a causal mask; 0x04C: the segment rule shapes the
// attention graph, not only the loss).  Query row i of a batch row sees keys
// j with run_start(i) <= j <= i (a padding row: itself only); scores are
// scaled by 1/sqrt(hd), softmax in float32 with an online max.
//
// Layout: qkv [B*T, 3*A] (q | k | v, head h at columns h*hd), out [B*T, A].
//
// One block = 256 queries of one (batch row, head); each wave owns 32 kNBQ
// queries (kNBQ 32-query MFMA column blocks) held in registers.  Key tiles
// of 64 keys (K and V, row-major as stored) move global -> LDS by direct
// loads into two stages; the loads of tile t+1 are issued as soon as tile
// t-1 has been consumed.  Per tile each wave computes
//   S^T = K Q^T     (keys on MFMA rows, queries on columns: every softmax
//                    statistic of a query lives in one lane column, 16 values
//                    in-lane plus the partner lane 32 away),
//   O^T += V^T P^T  (P^T taken straight from the S^T result registers: the
//                    MFMA's K-slots are mapped to the keys those registers
//                    hold, and V^T is read with the transposing LDS read at
//                    the same key order).
// P enters the bf16 product rounded to bf16 once (an unmirrored rounding:
// the probabilities are no stored tensor of the method; relative error at
// most 2^-9 per weight).
#include "gemm.hpp"
#include "kernels.hpp"

namespace mtp {

namespace {
constexpr int kQT = 256;                      // queries per block
constexpr int kKT = 64;                       // keys per tile
constexpr int kNBQ = 1;                       // 32-query column blocks per wave
constexpr int kQW = 32 * kNBQ;                // queries per wave
constexpr int kWaves = kQT / kQW;             // waves per block
constexpr int kAttnThreads = 64 * kWaves;
// The running max is raised (and the accumulators rescaled) only when a tile's
// max exceeds it by more than this (log2 units): probabilities stay <= 2^8.
constexpr float kRescale = 8.f;

template <typename T, int HD>
struct AttnCfg {
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int ROWB = HD * (int)sizeof(T);     // bytes per K / V row
  static constexpr int CPR = ROWB / 16;                // 16-byte chunks per row
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "row of 64, 128 or 256 bytes");
  static constexpr int RPL = 1024 / ROWB;              // rows per 1 KB load block
  static constexpr int TILE_BYTES = kKT * ROWB;        // K (or V) tile
  static constexpr int STAGE = 2 * TILE_BYTES;         // K then V
  static_assert((2 * kKT / RPL) % kWaves == 0, "load blocks per wave");
  static constexpr int LOADS = 2 * kKT / RPL / kWaves; // load instructions per wave and tile
  static constexpr int SK = HD / (2 * E);              // S^T MFMA steps over the head dim
  static constexpr int MD = HD >= 32 ? HD / 32 : 1;    // O^T row blocks (head dim)
  static constexpr int KPS = 2 * E;                    // keys per O^T MFMA step
};

// K tile: chunk c of key row r at physical chunk c ^ kswz(r) -- a 16-lane
// fragment read (16 consecutive rows, one logical chunk) covers all banks.
template <int CPR>
__device__ __forceinline__ int kswz(int r) {
  return (r / (16 / CPR)) & (CPR - 1);
}
// V tile: chunk c of key row k at physical chunk c ^ vswz(k) -- the four
// consecutive rows of a transposing read land in distinct 64-byte groups.
template <int CPR>
__device__ __forceinline__ int vswz(int k) {
  return CPR == 16 ? 4 * (k & 3) : (CPR == 8 ? 4 * ((k >> 1) & 1) : 0);
}
}  // namespace

template <typename T, int HD>
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(const T *__restrict__ qkv,
                                                                T *__restrict__ out,
                                                                const int32_t *__restrict__ run_start,
                                                                float *__restrict__ lse2_out, int B,
                                                                int T_len, int H, float scale_log2) {
  using C = AttnCfg<T, HD>;
  constexpr int E = C::E, CPR = C::CPR, ROWB = C::ROWB, SK = C::SK, MD = C::MD, KPS = C::KPS;
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE];

  const int A = H * HD;
  const long ld = 3L * A;
  const int ldb = (int)(ld * sizeof(T));
  const int nqt = (T_len + kQT - 1) / kQT;
  const int total = nqt * H * B;
  const int logical = xcd_remap(blockIdx.x, total);
  const int qt = nqt - 1 - (logical % nqt);          // long query tiles first
  const int h = (logical / nqt) % H;
  const int b = logical / (nqt * H);
  const int q0 = qt * kQT;
  const long rowbase = (long)b * T_len;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int hl = lane >> 5, c32 = lane & 31;

  // ---- this lane's queries (NBQ column blocks) and their Q fragments
  const int qw0 = q0 + wave * kQW;
  constexpr int NBQ = kNBQ;
  int qi[NBQ], rsq[NBQ];
  uint4 qreg[NBQ][SK];
#pragma unroll
  for (int nb = 0; nb < NBQ; ++nb) {
    qi[nb] = qw0 + 32 * nb + c32;
    const bool ok = qi[nb] < T_len;
    rsq[nb] = ok ? run_start[rowbase + qi[nb]] : 0;
    const T *qp = qkv + (rowbase + (ok ? qi[nb] : 0)) * ld + (long)h * HD;
#pragma unroll
    for (int s = 0; s < SK; ++s)
      qreg[nb][s] = ok ? reinterpret_cast<const uint4 *>(qp)[2 * s + hl] : make_uint4(0, 0, 0, 0);
  }
  // block key range: windows start no earlier than the first query's
  const int qlast = min(q0 + kQT, T_len) - 1;
  const int kbeg = run_start[rowbase + q0] / kKT * kKT;
  const int ntiles = (qlast - kbeg) / kKT + 1;
  // wave bounds: smallest window start and largest query of the wave; the
  // latest window start (window starts never decrease along a row)
  const int wq_hi = min(qw0 + kQW, T_len) - 1;
  const int w_rs = qw0 < T_len ? run_start[rowbase + qw0] : 0;
  const int w_rs_hi = qw0 < T_len ? run_start[rowbase + wq_hi] : 0;

  // ---- direct loads of key tile `it` (relative to kbeg) into a stage; tiles
  // past the range become all-out-of-range loads (no traffic)
  const long kv_bytes = (long)(T_len - 1) * ldb + ROWB;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(qkv + rowbase * ld + A + (long)h * HD, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(qkv + rowbase * ld + 2L * A + (long)h * HD, kv_bytes);
  const int rl = lane / CPR, pc = lane % CPR;
  auto issue = [&](int it, char *stage) {
    const bool valid = it < ntiles;
    const int k0 = kbeg + it * kKT;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int q = wave * C::LOADS + i;               // load block: K blocks first, then V
      const bool isv = q >= kKT / C::RPL;
      const int qb = isv ? q - kKT / C::RPL : q;
      const int row = qb * C::RPL + rl;                // key row inside the tile
      const int c = pc ^ (isv ? vswz<CPR>(row) : kswz<CPR>(row));
      const unsigned voff = valid ? (unsigned)(rl * ldb + c * 16) : kOOB;
      dma16(isv ? rv : rk, stage + (isv ? C::TILE_BYTES : 0) + qb * 1024, voff,
            valid ? (k0 + qb * C::RPL) * ldb : 0);
    }
  };

  f32x16 o[MD][NBQ];
  float m[NBQ], l[NBQ];
#pragma unroll
  for (int nb = 0; nb < NBQ; ++nb) {
    m[nb] = -INFINITY;
    l[nb] = 0.f;
#pragma unroll
    for (int i = 0; i < MD; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][nb][r] = 0.f;
  }

  // one key tile on stage sk (K at sk, V at sk + TILE_BYTES)
  auto tile = [&](int it, const char *sk) {
    const int k0 = kbeg + it * kKT;
    const bool active = qw0 < T_len && k0 <= wq_hi && k0 + kKT - 1 >= w_rs;
    if (!active) return;
    const char *sv = sk + C::TILE_BYTES;
    // every key of the tile visible to every query of the wave: no masking
    const bool full = k0 + kKT - 1 <= qw0 && k0 >= w_rs_hi && wq_hi == qw0 + kQW - 1;
    // ---- S^T = K Q^T: two 32-key row blocks x NBQ 32-query column blocks
    f32x16 s[2][NBQ];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][nb][r] = 0.f;
#pragma unroll
    for (int st = 0; st < SK; ++st) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * mb + c32, ch = 2 * st + hl;
        const uint4 a = *reinterpret_cast<const uint4 *>(sk + row * ROWB + ((ch ^ kswz<CPR>(row)) << 4));
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) mma32(a, qreg[nb][st], s[mb][nb], T{});
      }
    }
    // ---- mask, online softmax (base 2) with a lazily raised running max.
    // The max is taken on the raw scores (scale_log2 > 0 keeps the order) and
    // each probability is one FMA and one hardware exp2 (results below 2^-126
    // flush to zero).  `full` is the same for the whole wave: a tile visible
    // to every query of the wave skips the mask arithmetic.
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
      float mraw = -INFINITY;
      if (full) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mraw = fmaxf(mraw, s[mb][nb][r]);
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3);
            const bool ok = (qi[nb] < T_len) & (key <= qi[nb]) & (key >= rsq[nb]);
            const float x = ok ? s[mb][nb][r] : -INFINITY;
            s[mb][nb][r] = x;
            mraw = fmaxf(mraw, x);
          }
      }
      mraw = fmaxf(mraw, __shfl_xor(mraw, 32));
      const float mx = mraw * scale_log2;                 // -inf stays -inf
      const bool raise = mx > m[nb] + kRescale;          // same in both lanes of a query
      const float mnew = raise ? mx : m[nb];
      if (__builtin_amdgcn_read_exec() & __ballot(raise)) {
        const float alpha = raise ? exp2f(m[nb] - mnew) : 1.f;   // m = -inf: alpha = 0
        l[nb] *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[md][nb][r] *= alpha;
      }
      m[nb] = mnew;
      // no visible key yet: every score is -inf and every p must be 0
      const float neg = mnew == -INFINITY ? 0.f : -mnew;
      float ls = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][nb][r], scale_log2, neg));
          s[mb][nb][r] = p;
          ls += p;
        }
      l[nb] += ls;
    }
    // ---- O^T += V^T P^T.  Step j of 32-key block mb covers KPS keys; lane
    // half hl supplies the E registers E*j .. E*j+E-1 of s[mb], i.e. keys
    // 32 mb + 8 c + 4 hl + (0..3) for the register groups c of the step.
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int j = 0; j < 32 / KPS; ++j) {
        uint4 pb[NBQ];
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
          float v[E];
#pragma unroll
          for (int e = 0; e < E; ++e) v[e] = s[mb][nb][E * j + e];
          pb[nb] = f32_to_chunk(v, T{});
        }
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          uint4 a;
          if constexpr (sizeof(T) == 2) {
            // transposing reads: 16-lane group g reads head-dim rows M0 .. M0+15
            // at keys K0 .. K0+3 (first read) and K0+8 .. K0+11 (second read)
            typedef short v4s __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4s lds_v4s;
            const int g = lane >> 4, jj = lane & 15;
            const int kr = 32 * mb + 16 * j + 4 * (g >> 1) + (jj >> 2);      // key row of this lane's address
            const int dm = 32 * md + 16 * (g & 1) + 4 * (jj & 3);           // first head-dim element
            const int ch = dm / E, within = (dm % E) * (int)sizeof(T);
            const char *p0 = sv + kr * ROWB + ((ch ^ vswz<CPR>(kr)) << 4) + within;
            const char *p1 = sv + (kr + 8) * ROWB + ((ch ^ vswz<CPR>(kr + 8)) << 4) + within;
            const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)to_lds(const_cast<char *>(p0)));
            const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)to_lds(const_cast<char *>(p1)));
            const uint2 ua = __builtin_bit_cast(uint2, x0), ub = __builtin_bit_cast(uint2, x1);
            a = make_uint4(ua.x, ua.y, ub.x, ub.y);
          } else {
            // f32: element e of the chunk is key 32 mb + 8 j + 4 hl + e, head-dim row 32 md + c32
            const int dm = 32 * md + c32;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int kr = 32 * mb + 8 * j + 4 * hl + e;
              w[e] = dm < HD ? *reinterpret_cast<const uint32_t *>(
                                   sv + kr * ROWB + (((dm / E) ^ vswz<CPR>(kr)) << 4) + (dm % E) * 4)
                             : 0u;
            }
            a = make_uint4(w[0], w[1], w[2], w[3]);
          }
#pragma unroll
          for (int nb = 0; nb < NBQ; ++nb) mma32(a, pb[nb], o[md][nb], T{});
        }
      }
  };

  // ---- pipeline over the key tiles: tile it lives in stage it & 1; after a
  // tile is consumed, wait for the next one and refill the consumed stage
  issue(0, st0);
  issue(1, st1);
  wait_vm_lds_barrier<C::LOADS>();             // tile 0 landed (tile 1 may be in flight)
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    tile(it, st0);
    wait_vm_lds_barrier<0>();                  // tile it+1 landed, stage 0 retired
    issue(it + 2, st0);
    tile(it + 1, st1);
    wait_vm_lds_barrier<0>();                  // tile it+2 landed, stage 1 retired
    issue(it + 3, st1);
  }
  if (it < ntiles) tile(it, st0);
  wait_vm_lds_barrier<0>();                    // no load in flight into the stages

  // ---- normalise, stage [query][hd] in LDS (queries 0-127: stage 0,
  // 128-255: stage 1), coalesced stores
#pragma unroll
  for (int nb = 0; nb < NBQ; ++nb) {
    const float lt = l[nb] + __shfl_xor(l[nb], 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // base-2 log-sum-exp of the query's scaled scores (for the reverse pass)
    if (lse2_out != nullptr && hl == 0 && qi[nb] < T_len)
      lse2_out[2 * (rowbase * H + (long)h * T_len + qi[nb])] = m[nb] + __log2f(lt);
    const int qb = wave * kQW + 32 * nb + c32;            // query inside the block
    char *ostage = qb < kQT / 2 ? st0 : st1;
    T *orow = reinterpret_cast<T *>(ostage) + (long)(qb % (kQT / 2)) * HD;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dd = 32 * md + 8 * (r >> 2) + 4 * hl + (r & 3);
        if (dd < HD) store_elem(orow, dd, o[md][nb][r] * inv);
      }
  }
  __syncthreads();
  constexpr int OCH = HD / E;   // chunks per output row
  for (int cidx = t; cidx < kQT * OCH; cidx += kAttnThreads) {
    const int ql = cidx / OCH, ch = cidx % OCH;
    const int q = q0 + ql;
    if (q >= T_len) continue;
    const char *src = (ql < kQT / 2 ? st0 : st1) + (long)(ql % (kQT / 2)) * HD * sizeof(T);
    const uint4 v = reinterpret_cast<const uint4 *>(src)[ch];
    reinterpret_cast<uint4 *>(out + (rowbase + q) * (long)A + (long)h * HD)[ch] = v;
  }
}

template <typename T, int HD>
static hipError_t attn_launch(const T *qkv, T *out, const int32_t *rs, float *lse2, int B, int T_len, int H,
                              hipStream_t s) {
  const int nqt = (T_len + kQT - 1) / kQT;
  const long blocks = (long)nqt * H * B;
  const float scale_log2 = kLog2e / sqrtf((float)HD);
  hipLaunchKernelGGL((attention_kernel<T, HD>), dim3((unsigned)blocks), dim3(kAttnThreads), 0, s, qkv, out,
                     rs, lse2, B, T_len, H, scale_log2);
  return hipGetLastError();
}

template <>
hipError_t launch_attention<bf16_t>(const bf16_t *qkv, bf16_t *out, const int32_t *rs, float *lse2, int B,
                                    int T_len, int H, int hd, hipStream_t s) {
  switch (hd) {
    case 32: return attn_launch<bf16_t, 32>(qkv, out, rs, lse2, B, T_len, H, s);
    case 64: return attn_launch<bf16_t, 64>(qkv, out, rs, lse2, B, T_len, H, s);
    case 128: return attn_launch<bf16_t, 128>(qkv, out, rs, lse2, B, T_len, H, s);
    default: return hipErrorInvalidValue;
  }
}
template <>
hipError_t launch_attention<float>(const float *qkv, float *out, const int32_t *rs, float *lse2, int B,
                                   int T_len, int H, int hd, hipStream_t s) {
  switch (hd) {
    case 16: return attn_launch<float, 16>(qkv, out, rs, lse2, B, T_len, H, s);
    case 32: return attn_launch<float, 32>(qkv, out, rs, lse2, B, T_len, H, s);
    case 64: return attn_launch<float, 64>(qkv, out, rs, lse2, B, T_len, H, s);
    default: return hipErrorInvalidValue;
  }
}

// Attention of one decode step of the retained-module proposer (M7.6 0x09A:
// the module serves from its own K/V cache; 0x09D: one module rolled out over
// several draft steps).  One block of four waves per (request, head); wave w
// takes a contiguous quarter of the slots 0..pos.  A key row of HD elements
// is CPK 16-byte chunks: CPK lanes hold one key (lane c holds chunk c of the
// query), so one load instruction brings G = 64 / CPK keys (1 KB), and U of
// them are in flight per iteration.  Each lane group keeps its own online
// (max, sum, output chunk) over the keys it sees; the groups of a wave are
// merged with lane shuffles and the four waves through LDS.  The step's key
// (after RoPE) and value are read from the QKV activation for slot pos and
// copied to that slot of the cache.  Cache layout per request r: K of slot j
// at cache[((r * 2 + 0) * L_max + j) * A + h * HD ...], V at
// cache[((r * 2 + 1) * L_max + j) * A + ...].
template <typename T, int HD>
__global__ __launch_bounds__(256) void decode_attention_kernel(const T *__restrict__ qkv, T *__restrict__ cache,
                                                              T *__restrict__ out,
                                                              const int32_t *__restrict__ pos,
                                                              const int32_t *__restrict__ skip, int H, long L_max,
                                                              float scale_log2) {
  constexpr int E = 16 / (int)sizeof(T);       // elements per chunk
  constexpr int CPK = HD / E;                  // lanes (chunks) per key
  constexpr int G = 64 / CPK;                  // keys per load instruction
  constexpr int U = 4;                         // load instructions per iteration
  static_assert(CPK >= 1 && 64 % CPK == 0, "head row of 16-byte chunks");
  __shared__ float sm[4], sl[4];
  __shared__ float so[4][HD];
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const long A = (long)H * HD;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c = lane % CPK, g = lane / CPK;
  const int p = pos[r];                        // 0 <= p < L_max (checked before the launch)
  const T *qrow = qkv + (long)r * 3 * A + (long)h * HD;
  const T *knew = qrow + A, *vnew = qrow + 2 * A;
  T *kc = cache + (long)r * 2 * L_max * A + (long)h * HD;
  T *vc = kc + L_max * A;
  // a request flagged in skip (a rejected position or token) leaves its cache untouched
  if (w == 0 && lane < CPK && (skip == nullptr || skip[r] == 0)) {
    *reinterpret_cast<uint4 *>(kc + (long)p * A + c * E) = *reinterpret_cast<const uint4 *>(knew + c * E);
    *reinterpret_cast<uint4 *>(vc + (long)p * A + c * E) = *reinterpret_cast<const uint4 *>(vnew + c * E);
  }
  float q[E], o[E];
  chunk_to_f32(*reinterpret_cast<const uint4 *>(qrow + c * E), q, T{});
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int n = p + 1, per = (n + 3) / 4;
  const int k0 = w * per, k1 = min(n, k0 + per);
  for (int base = k0; base < k1; base += G * U) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + u * G + g;
      ok[u] = key < k1;
      const int kk = ok[u] ? key : k0;         // a valid slot of this wave
      const T *kp = kk == p ? knew : kc + (long)kk * A;
      const T *vp = kk == p ? vnew : vc + (long)kk * A;
      kr[u] = *reinterpret_cast<const uint4 *>(kp + c * E);
      vr[u] = *reinterpret_cast<const uint4 *>(vp + c * E);
    }
    float sc[U];
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kv[E];
      chunk_to_f32(kr[u], kv, T{});
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(q[e], kv[e], acc);
#pragma unroll
      for (int off = 1; off < CPK; off <<= 1) acc += __shfl_xor(acc, off);
      sc[u] = ok[u] ? acc * scale_log2 : -INFINITY;
      cm = fmaxf(cm, sc[u]);
    }
    const float mn = fmaxf(m, cm);
    const float corr = mn == -INFINITY ? 1.f : exp2f(m - mn);   // m = -inf, mn finite: 0
    l *= corr;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= corr;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = ok[u] ? exp2f(sc[u] - mn) : 0.f;
      float vv[E];
      chunk_to_f32(vr[u], vv, T{});
      l += pu;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmaf(pu, vv[e], o[e]);
    }
    m = mn;
  }
  // merge the lane groups of the wave (same chunk c, different keys)
#pragma unroll
  for (int off = CPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    const float M = fmaxf(m, m2);
    const float fa = m == -INFINITY ? 0.f : exp2f(m - M);
    const float fb = m2 == -INFINITY ? 0.f : exp2f(m2 - M);
    l = l * fa + l2 * fb;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float o2 = __shfl_xor(o[e], off);
      o[e] = o[e] * fa + o2 * fb;
    }
    m = M;
  }
  if (lane == 0) { sm[w] = m; sl[w] = l; }
  if (lane < CPK) {
#pragma unroll
    for (int e = 0; e < E; ++e) so[w][c * E + e] = o[e];
  }
  __syncthreads();
  if (w == 0 && lane < CPK) {
    float M = sm[0];
    for (int k = 1; k < 4; ++k) M = fmaxf(M, sm[k]);
    float f[4], L = 0.f;
    for (int k = 0; k < 4; ++k) {
      f[k] = sm[k] == -INFINITY ? 0.f : exp2f(sm[k] - M);      // a wave with no slot contributes 0
      L += sl[k] * f[k];
    }
    const float inv = 1.f / L;                                  // the maximal slot gives L >= 1
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float acc = 0.f;
      for (int k = 0; k < 4; ++k) acc = fmaf(so[k][c * E + e], f[k], acc);
      v[e] = acc * inv;
    }
    *reinterpret_cast<uint4 *>(out + (long)r * A + (long)h * HD + c * E) = f32_to_chunk(v, T{});
  }
}

template <typename T, int HD>
hipError_t decode_launch(const T *qkv, T *cache, T *out, const int32_t *pos, const int32_t *skip, int R, int H,
                         long L_max, hipStream_t s) {
  const float scale_log2 = kLog2e / sqrtf((float)HD);
  hipLaunchKernelGGL((decode_attention_kernel<T, HD>), dim3((unsigned)((long)R * H)), dim3(256), 0, s, qkv, cache,
                     out, pos, skip, H, L_max, scale_log2);
  return hipGetLastError();
}

template <>
hipError_t launch_decode_attention<bf16_t>(const bf16_t *qkv, bf16_t *cache, bf16_t *out, const int32_t *pos,
                                           const int32_t *skip, int R, int H, int hd, long L_max, hipStream_t s) {
  switch (hd) {
    case 32: return decode_launch<bf16_t, 32>(qkv, cache, out, pos, skip, R, H, L_max, s);
    case 64: return decode_launch<bf16_t, 64>(qkv, cache, out, pos, skip, R, H, L_max, s);
    case 128: return decode_launch<bf16_t, 128>(qkv, cache, out, pos, skip, R, H, L_max, s);
    default: return hipErrorInvalidValue;
  }
}
template <>
hipError_t launch_decode_attention<float>(const float *qkv, float *cache, float *out, const int32_t *pos,
                                          const int32_t *skip, int R, int H, int hd, long L_max, hipStream_t s) {
  switch (hd) {
    case 16: return decode_launch<float, 16>(qkv, cache, out, pos, skip, R, H, L_max, s);
    case 32: return decode_launch<float, 32>(qkv, cache, out, pos, skip, R, H, L_max, s);
    case 64: return decode_launch<float, 64>(qkv, cache, out, pos, skip, R, H, L_max, s);
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

// Rotary rows of the proposer's requests: table[r][j] = (cos, sin) of
// pos[r] w_j, as rope_table_kernel computes them.
__global__ void rope_rows_kernel(float2 *table, const int32_t *__restrict__ pos, int R, int half, double theta) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)R * half) return;
  const int r = (int)(i / half), j = (int)(i % half);
  const double w = pow(theta, -2.0 * j / (2.0 * half));
  double sn, cs;
  sincos((double)pos[r] * w, &sn, &cs);
  table[i] = make_float2((float)cs, (float)sn);
}

hipError_t rope_rows(float2 *table, const int32_t *pos, int R, int half, float theta, hipStream_t s) {
  const long n = (long)R * half;
  hipLaunchKernelGGL(rope_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, table, pos, R, half,
                     (double)theta);
  return hipGetLastError();
}

hipError_t rope_table(float2 *table, int max_pos, int half, float theta, hipStream_t s) {
  const long n = (long)max_pos * half;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, table, max_pos,
                     half, (double)theta);
  return hipGetLastError();
}

}  // namespace mtp
