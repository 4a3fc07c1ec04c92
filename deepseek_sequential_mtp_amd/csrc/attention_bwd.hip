// Reverse of the block's segment-causal attention (M7.6 0x05A: the MTP
// gradient reaches the module's Transformer block; 0x03C / 0x04C: the
// block's attention is causal inside a segment run).
//
// With S_ij = q_i . k_j, the forward's probabilities are
// P_ij = 2^(S_ij c - lse2_i) on visible pairs (run_start(i) <= j <= i; a
// padding row sees itself), c = log2(e) / sqrt(hd), lse2 the base-2
// log-sum-exp the forward kept per (row, head).  Given dO:
//   dV_j = sum_i P_ij dO_i,         dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i),     D_i = dO_i . o_i,
//   dQ_i = sum_j dS_ij k_j / sqrt(hd),   dK_j = sum_i dS_ij q_i / sqrt(hd),
// and dq, dk are rotated back through RoPE (the opposite angle at their
// positions).  q, k are the stored (RoPE'd) values, o the stored output.
//
// lse2 and D live side by side per (batch row, head, position): lsed
// [B, H, T] x float2, so that a tile of consecutive queries reads one
// contiguous run of them.
//
// Three passes, no atomics (the result does not depend on timing):
//   dV and dK (one kernel template, two launches: each pass keeps only its
//   own accumulators, so that two waves fit each SIMD; the scores are
//   computed in both): a block owns 128 keys of one (batch row, head), four
//   waves of 32;
//     each wave keeps its keys' K and V fragments in registers and walks the
//     query tiles that can see them (64 queries per tile; Q and dO, and the
//     tile's (lse2, D) pairs and run starts, staged in LDS by direct loads,
//     double-buffered).  Per 32 x 32 (query, key) block:
//     S = Q K^T and dP = dO V^T (queries on MFMA rows, keys on columns, so a
//     lane holds one key), then dV += P^T dO and dK += dS^T Q with P^T, dS^T
//     taken straight from those result registers (the MFMA K-slots are the
//     queries the registers hold) and dO, Q read with the transposing LDS
//     read in that query order.
//   dQ: a block owns 128 queries, four waves of 32, Q and dO fragments in
//     registers; key tiles of 64 (K and V in LDS, double-buffered).  Per key
//     block: S^T = K Q^T, dP^T = V dO^T (a lane holds one query), then
//     dQ^T += K^T dS^T with K^T by the transposing read.
// P and dS enter their bf16 products rounded to bf16 once.
#include "gemm.hpp"
#include "kernels.hpp"

namespace mtp {

namespace {
constexpr int kBwdThreads = 256;       // four waves
constexpr int kBwdKeys = 128;          // keys per dK/dV block (32 per wave)
constexpr int kBwdQT = 64;             // queries per staged tile of the dK/dV kernel
constexpr int kBwdQueries = 128;       // queries per dQ block (32 per wave)
constexpr int kBwdKT = 64;             // keys per staged tile of the dQ kernel

template <int HD>
struct BwdCfg {
  static constexpr int E = 8;                        // bf16 per 16-byte chunk
  static constexpr int ROWB = HD * 2;                // bytes per head row
  static constexpr int CPR = ROWB / 16;              // chunks per head row
  static_assert(CPR == 8 || CPR == 16, "head_dim 64 or 128");
  static constexpr int RPL = 1024 / ROWB;            // rows per 1 KB direct load
  static constexpr int TILE = 64 * ROWB;             // one 64-row tile
  static constexpr int STAGE = 2 * TILE;             // two tiles (Q + dO, or K + V)
  // dK/dV stage: Q + dO, then one 1 KB direct-load region per wave for the
  // tile's per-query scalars: (lse2, D) of queries 0-31 and 32-63, run
  // starts of queries 0-63 (the fourth region is unused)
  static constexpr int XSTAGE = 2 * TILE + 4 * 1024;
  static constexpr int LOADS = 2 * 64 / RPL / 4;     // load instructions per wave and stage
  static constexpr int SK = HD / 16;                 // MFMA steps over the head dim
  static constexpr int MD = HD / 32;                 // 32-wide head-dim blocks
};

// Tile rows: chunk ch of row r at physical chunk ch ^ swz(r), so that a
// 16-lane fragment read of 16 consecutive rows at one logical chunk covers
// every bank group.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  return (r / (16 / CPR)) & (CPR - 1);
}

// Fragment (16 bytes) of tile row `row`, logical chunk ch.
template <int CPR>
__device__ __forceinline__ uint4 tile_frag(const char *tile, int row, int ch) {
  constexpr int ROWB = CPR * 16;
  return *reinterpret_cast<const uint4 *>(tile + row * ROWB + ((ch ^ swz<CPR>(row)) << 4));
}

// Transposing read of a 32 x 32 (row, head-dim) block as an MFMA operand
// whose K-slots are rows: 16-lane group g reads head-dim columns
// 32 md + 16 (g & 1) + 0..15 at rows base + 0..3 and base + 8..11, base =
// r0 + 16 j + 4 (g >> 1).  Lane l then holds column 32 md + (l & 31) at rows
// r0 + 16 j + 4 (l >> 5) + {0..3, 8..11}: the rows that registers 8 j .. 8 j + 7
// of a 32x32 result hold for lane half l >> 5.
template <int CPR>
__device__ __forceinline__ uint4 tile_tr(const char *tile, int r0, int j, int md, int lane) {
  constexpr int ROWB = CPR * 16;
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const int g = lane >> 4, jj = lane & 15;
  const int kr = r0 + 16 * j + 4 * (g >> 1) + (jj >> 2);
  const int dm = 32 * md + 16 * (g & 1) + 4 * (jj & 3);
  const int ch = dm >> 3, within = (dm & 7) * 2;
  const char *p0 = tile + kr * ROWB + ((ch ^ swz<CPR>(kr)) << 4) + within;
  const char *p1 = tile + (kr + 8) * ROWB + ((ch ^ swz<CPR>(kr + 8)) << 4) + within;
  const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)to_lds(const_cast<char *>(p0)));
  const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)to_lds(const_cast<char *>(p1)));
  const uint2 a = __builtin_bit_cast(uint2, x0), b = __builtin_bit_cast(uint2, x1);
  return make_uint4(a.x, a.y, b.x, b.y);
}

__device__ __forceinline__ uint4 pack8(const float *v) {
  return make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                    pack_bf16x2(v[6], v[7]));
}

// Direct loads of a 64-row tile pair (rows row0 .. row0 + 63 of two
// tensors with row strides lda_b / ldb_b bytes) into stage; the wave's
// share of the 2 * 64 / RPL load blocks.  Rows past the resources read 0.
template <int HD>
__device__ __forceinline__ void load_tile_pair(__amdgpu_buffer_rsrc_t ra, int lda_b, __amdgpu_buffer_rsrc_t rb,
                                               int ldb_b, int row0, bool valid, char *stage, int wave, int lane) {
  using C = BwdCfg<HD>;
  const int rl = lane / C::CPR, pc = lane % C::CPR;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int q = wave * C::LOADS + i;                 // first tensor's blocks, then the second's
    const bool second = q >= 64 / C::RPL;
    const int qb = second ? q - 64 / C::RPL : q;
    const int row = qb * C::RPL + rl;
    const int c = pc ^ swz<C::CPR>(row);
    const int ldx = second ? ldb_b : lda_b;
    const unsigned voff = valid ? (unsigned)(rl * ldx + c * 16) : kOOB;
    dma16(second ? rb : ra, stage + (second ? C::TILE : 0) + qb * 1024, voff,
          valid ? (row0 + qb * C::RPL) * ldx : 0);
  }
}

// The per-query scalars of the 64-query tile at row0 into the wave's 1 KB
// region after the two tiles: wave 0 the (lse2, D) pairs of queries
// row0 .. row0 + 31, wave 1 those of row0 + 32 .. row0 + 63, wave 2 the run
// starts of all 64 (16 lanes x 16 B each; queries past the row read 0); wave
// 3 loads nothing (every lane past the resource) so that each wave issues
// one load per tile.
template <int HD>
__device__ __forceinline__ void load_query_scalars(__amdgpu_buffer_rsrc_t rld, __amdgpu_buffer_rsrc_t rrs,
                                                   int row0, int T_len, bool valid, char *stage, int wave,
                                                   int lane) {
  using C = BwdCfg<HD>;
  const int q0 = row0 + (wave == 1 ? 32 : 0);
  const bool ok = valid && wave < 3 && q0 < T_len && lane < 16;
  const int soff = valid && wave < 3 && q0 < T_len ? q0 * (wave == 2 ? 4 : 8) : 0;
  dma16(wave == 2 ? rrs : rld, stage + 2 * C::TILE + wave * 1024, ok ? (unsigned)(lane * 16) : kOOB, soff);
}
}  // namespace

// D = dO[n, h, :] . o[n, h, :] in float32 into element 1 of the (b, h, t)
// pair of lsed.  One block per row; lane groups of HD / 8 lanes hold one
// head's chunks.
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_dot_kernel(const bf16_t *__restrict__ dout,
                                                          const bf16_t *__restrict__ o, float2 *__restrict__ lsed,
                                                          int T_len, int H) {
  constexpr int CPH = HD / 8;                        // chunks per head
  const long n = blockIdx.x;
  const long brow = n / T_len, tpos = n % T_len;
  const int A = H * HD;
  for (int c = threadIdx.x; c < A / 8; c += 256) {
    float a[8], b[8];
    chunk_to_f32(reinterpret_cast<const uint4 *>(dout + n * A)[c], a, bf16_t{});
    chunk_to_f32(reinterpret_cast<const uint4 *>(o + n * A)[c], b, bf16_t{});
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(a[e], b[e], s);
#pragma unroll
    for (int off = 1; off < CPH; off <<= 1) s += __shfl_xor(s, off);
    if ((c % CPH) == 0) lsed[(brow * H + c / CPH) * T_len + tpos].y = s;
  }
}

template <int HD, bool DK>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_dkdv_kernel(
    const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout, const float2 *__restrict__ lsed,
    const int32_t *__restrict__ run_start, const int32_t *__restrict__ pos, const float2 *__restrict__ rope,
    bf16_t *__restrict__ dqkv, int B, int T_len, int H, float c2, float scale) {
  using C = BwdCfg<HD>;
  constexpr int CPR = C::CPR, ROWB = C::ROWB, SK = C::SK, MD = C::MD;
  __shared__ __attribute__((aligned(1024))) char st0[C::XSTAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::XSTAGE];

  const int A = H * HD;
  const long ld = 3L * A;
  const int ldq_b = (int)(ld * 2), ldo_b = A * 2;
  const int nkt = (T_len + kBwdKeys - 1) / kBwdKeys;
  const int logical = xcd_remap(blockIdx.x, nkt * H * B);
  const int kt = logical % nkt;                      // early keys (the most queries) first
  const int h = (logical / nkt) % H;
  const int b = logical / (nkt * H);
  const long rowbase = (long)b * T_len;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int hl = lane >> 5, c32 = lane & 31;
  const int j0 = kt * kBwdKeys;
  const int jlast = min(j0 + kBwdKeys, T_len) - 1;
  const int kw0 = j0 + 32 * wave;                    // the wave's first key
  const int key = kw0 + c32;                         // this lane's key (result column)
  const bool kok = key < T_len;

  // the wave's K (and, for dK, V) fragments (MFMA B operands: column = key,
  // K = head dim)
  uint4 kreg[SK], vreg[DK ? SK : 1];
  {
    const bf16_t *kp = qkv + (rowbase + (kok ? key : 0)) * ld + A + (long)h * HD;
#pragma unroll
    for (int s = 0; s < SK; ++s) {
      kreg[s] = kok ? reinterpret_cast<const uint4 *>(kp)[2 * s + hl] : make_uint4(0, 0, 0, 0);
      if constexpr (DK) vreg[s] = kok ? reinterpret_cast<const uint4 *>(kp + A)[2 * s + hl] : make_uint4(0, 0, 0, 0);
    }
  }
  // query tiles from j0 while their first query's window can reach the
  // block's keys (window starts never decrease along a row)
  // (a binary search over the tile starts: run starts never decrease along a
  // row, so the tiles that qualify are a prefix; the first always does)
  int ntiles = 0;
  {
    int hi = (T_len - j0 + kBwdQT - 1) / kBwdQT;     // tiles starting inside the row
    while (ntiles < hi) {
      const int mid = (ntiles + hi) >> 1;
      if (run_start[rowbase + j0 + mid * kBwdQT] <= jlast) ntiles = mid + 1;
      else hi = mid;
    }
  }

  const __amdgpu_buffer_rsrc_t rq =
      make_rsrc(qkv + rowbase * ld + (long)h * HD, (long)(T_len - 1) * ldq_b + ROWB);
  const __amdgpu_buffer_rsrc_t rdo =
      make_rsrc(dout + rowbase * A + (long)h * HD, (long)(T_len - 1) * ldo_b + ROWB);
  const __amdgpu_buffer_rsrc_t rld = make_rsrc(lsed + ((long)b * H + h) * T_len, (long)T_len * 8);
  const __amdgpu_buffer_rsrc_t rrs = make_rsrc(run_start + rowbase, (long)T_len * 4);
  auto issue = [&](int it, char *stage) {
    load_tile_pair<HD>(rq, ldq_b, rdo, ldo_b, j0 + it * kBwdQT, it < ntiles, stage, wave, lane);
    load_query_scalars<HD>(rld, rrs, j0 + it * kBwdQT, T_len, it < ntiles, stage, wave, lane);
  };

  f32x16 acc[MD];                                    // dK or dV of the wave's keys
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[md][r] = 0.f;

  auto tile = [&](int it, const char *sq) {
    const char *sdo = sq + C::TILE;
    const int i0 = j0 + it * kBwdQT;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int i0s = i0 + 32 * sub;
      // the sub-tile's first run start, from the tile's staged run starts
      const int rs_first = __builtin_amdgcn_readfirstlane(
          *reinterpret_cast<const int *>(sq + 2 * C::TILE + 2 * 1024 + (32 * sub) * 4));
      if (!(kw0 < T_len && i0s < T_len && i0s + 31 >= kw0 && rs_first <= kw0 + 31)) continue;
      f32x16 S, dP;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.f;
#pragma unroll
      for (int st = 0; st < SK; ++st) {
        mma32(tile_frag<CPR>(sq, 32 * sub + c32, 2 * st + hl), kreg[st], S, bf16_t{});
        if constexpr (DK) mma32(tile_frag<CPR>(sdo, 32 * sub + c32, 2 * st + hl), vreg[st], dP, bf16_t{});
      }
      // register r: query i0s + 8 (r / 4) + 4 hl + r % 4, key `key`; the four
      // queries of r / 4 read their (lse2, D) pairs and run starts from the
      // stage (one address per lane half: broadcast reads)
      // The block is fully visible when every query follows every key and
      // the last query's run starts at or before the first key (run starts
      // never decrease): then no mask arithmetic (wave-uniform branch).
      const int rs_last = __builtin_amdgcn_readfirstlane(
          *reinterpret_cast<const int *>(sq + 2 * C::TILE + 2 * 1024 + (32 * sub + 31) * 4));
      const bool full = i0s >= kw0 + 31 && i0s + 31 < T_len && kw0 + 31 < T_len && rs_last <= kw0;
      float P[16], dS[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = 32 * sub + 8 * g + 4 * hl;                // first of the four queries in the tile
        const float4 *px = reinterpret_cast<const float4 *>(sq + 2 * C::TILE + (ql >> 5) * 1024 + (ql & 31) * 8);
        const float4 x01 = px[0], x23 = px[1];
        const float lq[4] = {x01.x, x01.z, x23.x, x23.z}, dq[4] = {x01.y, x01.w, x23.y, x23.w};
        if (full) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            P[r] = __builtin_amdgcn_exp2f(fmaf(S[r], c2, -lq[e]));
            dS[r] = P[r] * (dP[r] - dq[e]);
          }
        } else {
          const int4 rs4 = *reinterpret_cast<const int4 *>(sq + 2 * C::TILE + 2 * 1024 + ql * 4);
          const int rq4[4] = {rs4.x, rs4.y, rs4.z, rs4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            const int qi = i0s + 8 * g + 4 * hl + e;
            const bool vis = kok && qi < T_len && key <= qi && key >= rq4[e];
            const float p = vis ? __builtin_amdgcn_exp2f(fmaf(S[r], c2, -lq[e])) : 0.f;
            P[r] = p;
            dS[r] = p * (dP[r] - dq[e]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (DK) {
          const uint4 sa = pack8(dS + 8 * j);
#pragma unroll
          for (int md = 0; md < MD; ++md) mma32(sa, tile_tr<CPR>(sq, 32 * sub, j, md, lane), acc[md], bf16_t{});
        } else {
          const uint4 pa = pack8(P + 8 * j);
#pragma unroll
          for (int md = 0; md < MD; ++md) mma32(pa, tile_tr<CPR>(sdo, 32 * sub, j, md, lane), acc[md], bf16_t{});
        }
      }
    }
  };

  issue(0, st0);
  issue(1, st1);
  wait_vm_lds_barrier<C::LOADS + 1>();             // tile 0 landed
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    tile(it, st0);
    wait_vm_lds_barrier<0>();                      // tile it+1 landed, stage 0 retired
    issue(it + 2, st0);
    tile(it + 1, st1);
    wait_vm_lds_barrier<0>();
    issue(it + 3, st1);
  }
  if (it < ntiles) tile(it, st0);
  wait_vm_lds_barrier<0>();                        // no load in flight into the stages

  // dK: scale, then back through RoPE at each key's position.  Register r of
  // block md holds key kw0 + 8 (r / 4) + 4 hl + r % 4, head-dim 32 md + c32;
  // the rotation partner of block md < MD / 2 is block md + MD / 2.
  if constexpr (DK) {
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[md][r] *= scale;
    if (rope != nullptr) {
      constexpr int HALF = HD / 2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = kw0 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const int p = kr < T_len ? pos[rowbase + kr] : 0;
#pragma unroll
        for (int md = 0; md < MD / 2; ++md) {
          const float2 cs = rope[(long)p * HALF + 32 * md + c32];
          const float d1 = acc[md][r], d2 = acc[md + MD / 2][r];
          acc[md][r] = d1 * cs.x + d2 * cs.y;
          acc[md + MD / 2][r] = d2 * cs.x - d1 * cs.y;
        }
      }
    }
  }
  // stage [key][head dim] in LDS, then 16-byte stores into the dk (or dv) columns
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kl = 32 * wave + 8 * (r >> 2) + 4 * hl + (r & 3);
      const int dd = 32 * md + c32;
      reinterpret_cast<bf16_t *>(st0 + kl * ROWB)[dd].bits = f32_to_bf16(acc[md][r]);
    }
  __syncthreads();
  for (int cidx = t; cidx < kBwdKeys * CPR; cidx += kBwdThreads) {
    const int kl = cidx / CPR, ch = cidx % CPR;
    const int kr = j0 + kl;
    if (kr >= T_len) continue;
    bf16_t *dst = dqkv + (rowbase + kr) * ld + (DK ? A : 2L * A) + (long)h * HD + ch * 8;
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(st0 + kl * ROWB + ch * 16);
  }
}

// Two waves per SIMD (at most 256 registers): the second wave hides the
// first's waits.
template <int HD>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_bwd_dq_kernel(
    const bf16_t *__restrict__ qkv, const bf16_t *__restrict__ dout, const float2 *__restrict__ lsed,
    const int32_t *__restrict__ run_start, const int32_t *__restrict__ pos, const float2 *__restrict__ rope,
    bf16_t *__restrict__ dqkv, int B, int T_len, int H, float c2, float scale) {
  using C = BwdCfg<HD>;
  constexpr int CPR = C::CPR, ROWB = C::ROWB, SK = C::SK, MD = C::MD;
  __shared__ __attribute__((aligned(1024))) char st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[C::STAGE];

  const int A = H * HD;
  const long ld = 3L * A;
  const int ldq_b = (int)(ld * 2);
  const int nqt = (T_len + kBwdQueries - 1) / kBwdQueries;
  const int logical = xcd_remap(blockIdx.x, nqt * H * B);
  const int qt = nqt - 1 - (logical % nqt);          // late queries (the most keys) first
  const int h = (logical / nqt) % H;
  const int b = logical / (nqt * H);
  const long rowbase = (long)b * T_len;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int hl = lane >> 5, c32 = lane & 31;
  const int q0 = qt * kBwdQueries;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c32;                          // this lane's query (result column)
  const bool qok = qi < T_len;

  uint4 qreg[SK], doreg[SK];
  {
    const bf16_t *qp = qkv + (rowbase + (qok ? qi : 0)) * ld + (long)h * HD;
    const bf16_t *dp = dout + (rowbase + (qok ? qi : 0)) * A + (long)h * HD;
#pragma unroll
    for (int s = 0; s < SK; ++s) {
      qreg[s] = qok ? reinterpret_cast<const uint4 *>(qp)[2 * s + hl] : make_uint4(0, 0, 0, 0);
      doreg[s] = qok ? reinterpret_cast<const uint4 *>(dp)[2 * s + hl] : make_uint4(0, 0, 0, 0);
    }
  }
  const float2 lq = lsed[((long)b * H + h) * T_len + (qok ? qi : 0)];
  const float l2 = lq.x, Dq = lq.y;
  const int rsq = run_start[rowbase + (qok ? qi : 0)];

  const int qlast = min(q0 + kBwdQueries, T_len) - 1;
  const int kbeg = run_start[rowbase + q0] / kBwdKT * kBwdKT;
  const int ntiles = (qlast - kbeg) / kBwdKT + 1;
  const int wq_hi = min(qw0 + 32, T_len) - 1;
  const int w_rs = qw0 < T_len ? run_start[rowbase + qw0] : 0;
  const int w_rs_hi = qw0 < T_len ? run_start[rowbase + wq_hi] : 0;    // the wave's largest run start

  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(qkv + rowbase * ld + A + (long)h * HD, (long)(T_len - 1) * ldq_b + ROWB);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(qkv + rowbase * ld + 2L * A + (long)h * HD, (long)(T_len - 1) * ldq_b + ROWB);
  auto issue = [&](int it, char *stage) {
    load_tile_pair<HD>(rk, ldq_b, rv, ldq_b, kbeg + it * kBwdKT, it < ntiles, stage, wave, lane);
  };

  f32x16 dQ[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) dQ[md][r] = 0.f;

  auto tile = [&](int it, const char *sk) {
    const char *sv = sk + C::TILE;
    const int k0 = kbeg + it * kBwdKT;
    if (!(qw0 < T_len && k0 <= wq_hi && k0 + kBwdKT - 1 >= w_rs)) return;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 S, dP;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = dP[r] = 0.f;
#pragma unroll
      for (int st = 0; st < SK; ++st) {
        mma32(tile_frag<CPR>(sk, 32 * mb + c32, 2 * st + hl), qreg[st], S, bf16_t{});
        mma32(tile_frag<CPR>(sv, 32 * mb + c32, 2 * st + hl), doreg[st], dP, bf16_t{});
      }
      // register r: key k0 + 32 mb + 8 (r / 4) + 4 hl + r % 4, query qi.  The
      // block is fully visible to the wave when its last key precedes the
      // wave's first query, its first key is at or after the wave's largest
      // run start, and all 32 queries exist (wave-uniform branch).
      const int kb0 = k0 + 32 * mb;
      const bool full = kb0 + 31 <= qw0 && kb0 >= w_rs_hi && qw0 + 31 < T_len;
      float dS[16];
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dS[r] = __builtin_amdgcn_exp2f(fmaf(S[r], c2, -l2)) * (dP[r] - Dq);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kj = kb0 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool vis = qok && kj <= qi && kj >= rsq;
          const float p = vis ? __builtin_amdgcn_exp2f(fmaf(S[r], c2, -l2)) : 0.f;
          dS[r] = p * (dP[r] - Dq);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 sb = pack8(dS + 8 * j);
#pragma unroll
        for (int md = 0; md < MD; ++md) mma32(tile_tr<CPR>(sk, 32 * mb, j, md, lane), sb, dQ[md], bf16_t{});
      }
    }
  };

  issue(0, st0);
  issue(1, st1);
  wait_vm_lds_barrier<C::LOADS>();
  int it = 0;
  for (; it + 1 < ntiles; it += 2) {
    tile(it, st0);
    wait_vm_lds_barrier<0>();
    issue(it + 2, st0);
    tile(it + 1, st1);
    wait_vm_lds_barrier<0>();
    issue(it + 3, st1);
  }
  if (it < ntiles) tile(it, st0);
  wait_vm_lds_barrier<0>();

  // dQ^T: register r of block md holds head-dim 32 md + 8 (r / 4) + 4 hl + r % 4
  // of query qi; scale and rotate back at the query's position
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int r = 0; r < 16; ++r) dQ[md][r] *= scale;
  if (rope != nullptr) {
    constexpr int HALF = HD / 2;
    const int p = qok ? pos[rowbase + qi] : 0;
#pragma unroll
    for (int md = 0; md < MD / 2; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float2 cs = rope[(long)p * HALF + 32 * md + 8 * (r >> 2) + 4 * hl + (r & 3)];
        const float d1 = dQ[md][r], d2 = dQ[md + MD / 2][r];
        dQ[md][r] = d1 * cs.x + d2 * cs.y;
        dQ[md + MD / 2][r] = d2 * cs.x - d1 * cs.y;
      }
  }
  // stage [query][head dim] (queries 0-63 in st0, 64-127 in st1), 16-byte stores
  {
    const int ql = 32 * wave + c32;
    char *sq = ql < 64 ? st0 : st1;
    bf16_t *row = reinterpret_cast<bf16_t *>(sq + (ql % 64) * ROWB);
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int r = 0; r < 16; ++r) row[32 * md + 8 * (r >> 2) + 4 * hl + (r & 3)].bits = f32_to_bf16(dQ[md][r]);
  }
  __syncthreads();
  for (int cidx = t; cidx < kBwdQueries * CPR; cidx += kBwdThreads) {
    const int ql = cidx / CPR, ch = cidx % CPR;
    const int q = q0 + ql;
    if (q >= T_len) continue;
    const char *src = (ql < 64 ? st0 : st1) + (ql % 64) * ROWB + ch * 16;
    *reinterpret_cast<uint4 *>(dqkv + (rowbase + q) * ld + (long)h * HD + ch * 8) =
        *reinterpret_cast<const uint4 *>(src);
  }
}

template <int HD>
static hipError_t attn_bwd_launch(const bf16_t *qkv, const bf16_t *o, const bf16_t *dout, float2 *lsed,
                                  const int32_t *rs, const int32_t *pos, const float2 *rope, bf16_t *dqkv, int B,
                                  int T_len, int H, hipStream_t s) {
  const float scale = 1.f / sqrtf((float)HD);
  const float c2 = kLog2e * scale;
  hipLaunchKernelGGL((attn_bwd_dot_kernel<HD>), dim3((unsigned)((long)B * T_len)), dim3(256), 0, s, dout, o, lsed,
                     T_len, H);
  const long nk = (long)(T_len + kBwdKeys - 1) / kBwdKeys * H * B;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<HD, false>), dim3((unsigned)nk), dim3(kBwdThreads), 0, s, qkv, dout, lsed,
                     rs, pos, rope, dqkv, B, T_len, H, c2, scale);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<HD, true>), dim3((unsigned)nk), dim3(kBwdThreads), 0, s, qkv, dout, lsed,
                     rs, pos, rope, dqkv, B, T_len, H, c2, scale);
  const long nq = (long)(T_len + kBwdQueries - 1) / kBwdQueries * H * B;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<HD>), dim3((unsigned)nq), dim3(kBwdThreads), 0, s, qkv, dout, lsed, rs,
                     pos, rope, dqkv, B, T_len, H, c2, scale);
  return hipGetLastError();
}

hipError_t launch_attention_bwd(const bf16_t *qkv, const bf16_t *o, const bf16_t *dout, float2 *lsed,
                                const int32_t *run_start, const int32_t *pos, const float2 *rope, bf16_t *dqkv,
                                int B, int T_len, int H, int hd, hipStream_t s) {
  switch (hd) {
    case 64: return attn_bwd_launch<64>(qkv, o, dout, lsed, run_start, pos, rope, dqkv, B, T_len, H, s);
    case 128: return attn_bwd_launch<128>(qkv, o, dout, lsed, run_start, pos, rope, dqkv, B, T_len, H, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
