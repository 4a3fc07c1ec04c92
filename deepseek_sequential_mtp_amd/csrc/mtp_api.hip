// C ABI of the library (declared in include/mtp.h): argument checks,
// workspace layout and the launch sequence of each entry point.  All
// launches go to the caller's stream; nothing here synchronises the host.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/mtp.h"
#include "epilogues.hpp"
#include "kernels.hpp"

using namespace mtp;

// Scratch of mtp_verify_noalloc: one copy per device (the code object's
// storage), held until the process ends.  Host code never passes `scratch`
// itself to a kernel -- on the host it only names the symbol; its device
// address comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) char scratch[MTP_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, resolved once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_address(hipStream_t s, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MTP_ERR_HIP;
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return MTP_ERR_HIP;
    if ((int)sdev != dev) return MTP_ERR_ARG;   // the stream must belong to the current device
  }
  if (dev < 0 || dev >= kMaxDevices) return MTP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MTP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MTP_OK;
}

constexpr size_t kAlign = 256;

struct Carve {
  char *base;
  size_t off = 0;
  explicit Carve(void *b) : base(static_cast<char *>(b)) {}
  template <typename P>
  P *take(size_t count) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    P *p = base ? reinterpret_cast<P *>(base + off) : nullptr;
    off += count * sizeof(P);
    return p;
  }
};

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

#define MTP_TRY(expr)                        \
  do {                                       \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return MTP_ERR_HIP; \
  } while (0)

// ---------------------------------------------------------------------------
// Stage instrumentation (mtp_profile_stage): caller events recorded around
// every launch of the armed stage.
// ---------------------------------------------------------------------------
struct Profile {
  int stage = -1;
  bool all = false;            // every stage (mtp_profile_all)
  int *ids = nullptr;          // [host] stage of each slot (mtp_profile_all)
  hipEvent_t *start = nullptr, *stop = nullptr;
  int n = 0, count = 0;
};
Profile g_prof;

struct StageScope {
  hipStream_t s;
  bool on;
  int slot;
  StageScope(int stage, hipStream_t st)
      : s(st), on((g_prof.all || g_prof.stage == stage) && g_prof.n > 0), slot(0) {
    if (on) {
      slot = g_prof.count % g_prof.n;
      if (g_prof.ids != nullptr) g_prof.ids[slot] = stage;
      (void)hipEventRecord(g_prof.start[slot], s);
    }
  }
  ~StageScope() {
    if (on) {
      (void)hipEventRecord(g_prof.stop[slot], s);
      ++g_prof.count;
    }
  }
};
#define MTP_STAGE(id) StageScope stage_scope_##__LINE__((id), s)

// ---------------------------------------------------------------------------
// GEMM dispatch.  The 256x256 tile is used when it still yields at least one
// tile per compute unit; otherwise 128x128.
// ---------------------------------------------------------------------------
using Big = Tile<256, 256, 4, 2>;
using Small = Tile<128, 128>;
// GEMMs of a few rows (the proposer's R <= 64 requests) stream the weights:
// a 64-row tile wastes no MFMA work on absent rows, its 80 KB of LDS lets two
// blocks share a compute unit, and each block keeps three 16 KB weight slices
// in flight (the 256x256 tile streamed the vocabulary head at 3.8 TB/s, this
// one at 4.8 TB/s; QKV 3.3 -> 4.3 TB/s, gate/up 2.8 -> 3.5 TB/s, where 192
// and 144 tiles leave part of the chip idle; a 64x128 tile was slower).
using Few = Tile<64, 256, 2, 2, 4>;
// A 256 x 224 tile (eight waves of 32 x 224 each; B staged in the 256-row
// layout, its last 32 rows empty) for NT GEMMs whose 256 x 256 tiles would
// leave the last round partly idle: at M 4096, N 7168 (eh_proj, O-proj, down
// at V3 width) 448 tiles of 256 x 256 take two rounds, 512 tiles of 256 x 224
// two rounds of 7/8 the work.
using Wide = Tile<256, 224, 8, 1, 4, 256>;
template <typename T> using KBW = DmaKMajor<T, Wide::BNL, Wide::NT, Wide::BN>;

// Operand loaders for a tile shape: K-major / MN-major A (BM rows) and B (BN rows).
template <typename T, class Cfg> using KA = DmaKMajor<T, Cfg::BM, Cfg::NT>;
template <typename T, class Cfg> using KB = DmaKMajor<T, Cfg::BN, Cfg::NT>;
template <typename T, class Cfg> using MA = DmaMNMajor<T, Cfg::BM, Cfg::NT>;
template <typename T, class Cfg> using MB_ = DmaMNMajor<T, Cfg::BN, Cfg::NT>;
// A operand of the GEMMs whose B is K-major too: the 256x256 bf16 tile stages
// it in 128-byte pair rows (whole 128-byte lines per load).
template <typename T, class Cfg>
using PA = std::conditional_t<sizeof(T) == 2 && Cfg::BM == 256, DmaKMajor128<T, Cfg::BM, Cfg::NT>,
                              DmaKMajor<T, Cfg::BM, Cfg::NT>>;

inline bool use_big(long M, long N) { return (long)ceil_div(M, 256) * ceil_div(N, 256) >= 256; }

// One GEMM without K splits: the 256x256 tile (one block per compute unit)
// on the balanced schedule (skws: tail_ws_bytes<Big>() of scratch) when it
// has at least kBalancedRounds rounds of tiles or a long K
// (kBalancedK elements), else one block per tile (the 128x128 tile always).
// With few rounds and a short K, the split tail's short partial tiles cost
// more than the idle compute units of a plain last round: the chip is
// power-limited and runs a partly filled round at a higher clock (measured
// at M 4096, N 7168: K 14336 8% faster plain, K 18432 even, K 129280 5%
// faster balanced).
constexpr long kBalancedRounds = 4;
constexpr int kBalancedK = 65536;
// The 256 x 224 tile replaces a plain (unbalanced) 256 x 256 launch when its
// rounds of 7/8-size tiles take at most 95% of the 256 x 256 rounds.
inline bool use_wide(long M, long N, long K) {
  const long big = (long)ceil_div(M, 256) * ceil_div(N, 256);
  if (big >= kBalancedRounds * kGemmSlots || K >= kBalancedK) return false;
  const long wide = (long)ceil_div(M, 256) * ceil_div(N, 224);
  return 0.875 * (double)ceil_div(wide, kGemmSlots) <= 0.95 * (double)ceil_div(big, kGemmSlots);
}
template <typename T, class Cfg, class LA, class LB, class Epi>
hipError_t run_gemm(const LA &la, const LB &lb, const Epi &epi, int M, int N, int K, int group_m, float *skws,
                    hipStream_t s) {
  if constexpr (std::is_same_v<Cfg, Big>) {
    if ((long)ceil_div(M, Cfg::BM) * ceil_div(N, Cfg::BN) >= kBalancedRounds * kGemmSlots || K >= kBalancedK)
      return launch_gemm_balanced<T, Cfg>(la, lb, epi, M, N, K, group_m, skws, s);
  }
  return launch_gemm<T, Cfg>(la, lb, epi, M, N, K, group_m, 1, s);
}

template <typename T, typename OutT, typename ResT>
int gemm_nt_store(const T *A, long lda, const T *Bm, long ldb, OutT *C, long ldc, const ResT *R, long ldr,
                  int M, int N, int K, float alpha, const float *alpha_dev, int accumulate, float *skws,
                  hipStream_t s) {
  EpiStore<OutT, ResT> epi{C, ldc, M, N, alpha, alpha_dev, R, ldr, accumulate, 0};
  if constexpr (sizeof(T) == 2) {
    if (M <= Few::BM) {
      PA<T, Few> la{A, lda, M, K};
      KB<T, Few> lb{Bm, ldb, N, K};
      MTP_TRY((launch_gemm<T, Few>(la, lb, epi, M, N, K, 8, 1, s)));
      return MTP_OK;
    }
    if (use_big(M, N)) {
      if (use_wide(M, N, K)) {
        PA<T, Wide> la{A, lda, M, K};
        KBW<T> lb{Bm, ldb, N, K};
        MTP_TRY((launch_gemm<T, Wide>(la, lb, epi, M, N, K, 8, 1, s)));
        return MTP_OK;
      }
      PA<T, Big> la{A, lda, M, K};
      KB<T, Big> lb{Bm, ldb, N, K};
      MTP_TRY((run_gemm<T, Big>(la, lb, epi, M, N, K, 8, skws, s)));
      return MTP_OK;
    }
  }
  {
    PA<T, Small> la{A, lda, M, K};
    KB<T, Small> lb{Bm, ldb, N, K};
    MTP_TRY((launch_gemm<T, Small>(la, lb, epi, M, N, K, 8, 1, s)));
  }
  return MTP_OK;
}

template <typename T, int HALF, class Cfg>
int gemm_qkv_rope_cfg(const T *xa, const T *W, T *qkv, const int *pos, const float2 *rope, int M, int d,
                      int A, float *skws, hipStream_t s) {
  const int N = 3 * A;
  EpiRope<T, HALF> epi{qkv, (long)N, M, N, A, pos, rope};
  PA<T, Cfg> la{xa, (long)d, M, d};
  KB<T, Cfg> lb{W, (long)d, N, d};
  MTP_TRY((run_gemm<T, Cfg>(la, lb, epi, M, N, d, 8, skws, s)));
  return MTP_OK;
}

template <typename T>
int gemm_qkv_rope(const T *xa, const T *W, T *qkv, const int *pos, const float2 *rope, int M, int d, int A,
                  int hd, float *skws, hipStream_t s) {
  // The wave's column range (WN) must cover whole heads for HALF >= 32.
  if constexpr (sizeof(T) == 2) {
    if (M <= Few::BM) switch (hd) {
      case 32: return gemm_qkv_rope_cfg<T, 16, Few>(xa, W, qkv, pos, rope, M, d, A, skws, s);
      case 64: return gemm_qkv_rope_cfg<T, 32, Few>(xa, W, qkv, pos, rope, M, d, A, skws, s);
      case 128: return gemm_qkv_rope_cfg<T, 64, Few>(xa, W, qkv, pos, rope, M, d, A, skws, s);
      default: return MTP_ERR_UNSUPPORTED;
    }
    switch (hd) {
      case 32: return gemm_qkv_rope_cfg<T, 16, Big>(xa, W, qkv, pos, rope, M, d, A, skws, s);
      case 64: return gemm_qkv_rope_cfg<T, 32, Big>(xa, W, qkv, pos, rope, M, d, A, skws, s);
      case 128: return gemm_qkv_rope_cfg<T, 64, Big>(xa, W, qkv, pos, rope, M, d, A, skws, s);
      default: return MTP_ERR_UNSUPPORTED;
    }
  } else switch (hd) {
    case 16: return gemm_qkv_rope_cfg<T, 8, Small>(xa, W, qkv, pos, rope, M, d, A, skws, s);
    case 32: return gemm_qkv_rope_cfg<T, 16, Small>(xa, W, qkv, pos, rope, M, d, A, skws, s);
    case 64: return gemm_qkv_rope_cfg<T, 32, Small>(xa, W, qkv, pos, rope, M, d, A, skws, s);
    default: return MTP_ERR_UNSUPPORTED;
  }
}

template <typename T>
int gemm_swiglu(const T *y, const T *Wg, const T *Wu, T *out, int M, int d, int f, float *skws, hipStream_t s,
                float *pre = nullptr) {
  if constexpr (sizeof(T) == 2) {
    if (M <= Few::BM) {
      EpiSwiGLU<T> epi{out, (long)f, M, f, pre};
      PA<T, Few> la{y, (long)d, M, d};
      DmaKMajorSwiGLU<T, Few> lb{Wg, Wu, (long)d, f, d};
      MTP_TRY((launch_gemm<T, Few>(la, lb, epi, M, 2 * ceil_div(f, Few::BN / 2) * (Few::BN / 2), d, 8, 1, s)));
      return MTP_OK;
    }
    if (use_big(M, 2L * f)) {
      EpiSwiGLU<T> epi{out, (long)f, M, f, pre};
      PA<T, Big> la{y, (long)d, M, d};
      DmaKMajorSwiGLU<T, Big> lb{Wg, Wu, (long)d, f, d};
      MTP_TRY((run_gemm<T, Big>(la, lb, epi, M, 2 * ceil_div(f, Big::BN / 2) * (Big::BN / 2), d, 8, skws, s)));
      return MTP_OK;
    }
  }
  {
    EpiSwiGLU<T> epi{out, (long)f, M, f, pre};
    PA<T, Small> la{y, (long)d, M, d};
    DmaKMajorSwiGLU<T, Small> lb{Wg, Wu, (long)d, f, d};
    MTP_TRY((launch_gemm<T, Small>(la, lb, epi, M, 2 * ceil_div(f, Small::BN / 2) * (Small::BN / 2), d, 8,
                                   1, s)));
  }
  return MTP_OK;
}

// Storage of the kept logits: bf16 runs keep fp16 offsets from the tile max,
// f32 runs keep fp32 logits.
template <typename T>
using LogitT = std::conditional_t<sizeof(T) == 2, _Float16, float>;

template <typename T, class Cfg>
int gemm_ce_fwd_cfg(const T *xhat, const T *W, const int *lab, float2 *part, float *target, LogitT<T> *z, int M,
                    int V, int d, float *skws, hipStream_t s) {
  const int nt = ceil_div(V, Cfg::BN);
  EpiCEFwd<LogitT<T>> epi{lab, part, target, z, M, V, nt};
  PA<T, Cfg> la{xhat, (long)d, M, d};
  KB<T, Cfg> lb{W, (long)d, V, d};
  // all row tiles of one vocabulary tile run next to each other: W is read once
  MTP_TRY((run_gemm<T, Cfg>(la, lb, epi, M, V, d, 1 << 30, skws, s)));
  return MTP_OK;
}

// Transposed tile (bf16): z^T = W_out x_hat^T with W_out the pair-row A
// operand and x_hat^T [d, ldT] the MN-major B operand (whole 128-byte lines
// for both).  Raster: groups of 4 vocabulary tiles, the 4 tiles of a group
// running next to each other for each token tile, so that an XCD's 32 tiles
// in flight are 4 vocabulary x 8 token tiles and read 12 operand tiles.
template <typename T, class Cfg>
int gemm_ce_fwd_t_cfg(const T *xhatT, long ldT, const T *W, const int *lab, float2 *part, float *target,
                      _Float16 *z, int rows, int V, int d, float *skws, hipStream_t s) {
  const int nt = ceil_div(V, Cfg::BM);
  EpiCEFwdT epi{lab, part, target, z, V, V, rows, nt};
  PA<T, Cfg> la{W, (long)d, V, d};
  MB_<T, Cfg> lb{xhatT, ldT, rows, d};
  MTP_TRY((run_gemm<T, Cfg>(la, lb, epi, V, rows, d, 4, skws, s)));
  return MTP_OK;
}

// dx[split] = scale * dz[:, split range] W_out[split range, :]  (B operand MN-major)
template <typename T, class Cfg>
int gemm_dx_cfg(const T *dz, const T *W, float *dxs, long slab, int M, int V, int d, const float *scale,
                int splits, float *skws, hipStream_t s) {
  EpiStore<float, float> epi{dxs, (long)d, M, d, 1.f, scale, nullptr, 0, 0, slab};
  KA<T, Cfg> la{dz, (long)V, M, V};
  MB_<T, Cfg> lb{W, (long)d, d, V};
  if (splits == 1) MTP_TRY((run_gemm<T, Cfg>(la, lb, epi, M, d, V, 8, skws, s)));
  else MTP_TRY((launch_gemm<T, Cfg>(la, lb, epi, M, d, V, 8, splits, s)));
  return MTP_OK;
}

// dW (+)= scale * dz^T xhat  (both operands MN-major)
template <typename T, class Cfg>
int gemm_dw_cfg(const T *dz, const T *xhat, float *dW, int M, int V, int d, const float *scale, int accumulate,
                float *skws, hipStream_t s) {
  EpiStore<float, float> epi{dW, (long)d, V, d, 1.f, scale, nullptr, 0, accumulate, 0};
  MA<T, Cfg> la{dz, (long)V, V, M};
  MB_<T, Cfg> lb{xhat, (long)d, d, M};
  MTP_TRY((run_gemm<T, Cfg>(la, lb, epi, V, d, M, 8, skws, s)));
  return MTP_OK;
}

// Run f with the 256x256 tile (bf16 and `big`) or the 128x128 tile.
template <typename T, class F>
int pick(bool big, F &&f) {
  if constexpr (sizeof(T) == 2) {
    if (big) return f(Big{});
  }
  return f(Small{});
}

// K-split count for the dx GEMM: fill the 256 compute units with whole waves
// of tiles while keeping each split long.  Cost in units of one K step: a
// wave of tiles takes its K range plus a fixed ~10^4 for the tile's start,
// epilogue and partial-sum traffic (measured on the 256x256 tile: one
// unsplit pass over K = 129280 beats 2 or 4 splits even when it leaves the
// second wave of tiles a quarter empty).
inline int dx_splits(int M, int d, int V, bool big) {
  const long tiles = (long)ceil_div(M, big ? 256 : 128) * ceil_div(d, big ? 256 : 128);
  int best = 1;
  double best_cost = 1e300;
  for (int s = 1; s <= 8; s *= 2) {
    const double waves = ceil((double)tiles * s / 256.0);
    const double cost = waves * ((double)V / s + 1e4) + 0.02 * V * s;   // + split-sum traffic
    if (cost < best_cost - 1e-9) { best_cost = cost; best = s; }
  }
  return best;
}

// ---------------------------------------------------------------------------
// argument checks
// ---------------------------------------------------------------------------
int check_chain(const mtp_chain_args *a) {
  if (a == nullptr) return MTP_ERR_NULL;
  if (a->D < 1) return MTP_ERR_DEPTH;
  if (a->dtype != MTP_F32 && a->dtype != MTP_BF16) return MTP_ERR_DTYPE;
  if (a->B < 1 || a->T < 1 || a->d < 1 || a->n_heads < 1 || a->head_dim < 2 || a->ffn < 1 || a->V < 1)
    return MTP_ERR_SHAPE;
  if (a->head_dim % 2) return MTP_ERR_SHAPE;
  const int E = a->dtype == MTP_BF16 ? 8 : 4;
  const int A = a->n_heads * a->head_dim;
  if (a->d % E || a->ffn % E || A % E) return MTP_ERR_SHAPE;
  if ((long)a->B * a->T > (1L << 30) || (long)a->V * a->d > (1L << 40)) return MTP_ERR_SHAPE;
  // attention addresses one batch row's keys and values through a 32-bit
  // buffer range: T rows of the [q | k | v] activation must span < 2 GiB
  if ((long)a->T * 3 * A * (a->dtype == MTP_BF16 ? 2 : 4) >= (1L << 31) - 4096) return MTP_ERR_UNSUPPORTED;
  if (a->dtype == MTP_BF16 && a->head_dim != 32 && a->head_dim != 64 && a->head_dim != 128)
    return MTP_ERR_UNSUPPORTED;
  if (a->dtype == MTP_F32 && a->head_dim != 16 && a->head_dim != 32 && a->head_dim != 64)
    return MTP_ERR_UNSUPPORTED;
  if (!(a->eps >= 0.f) || !(a->rope_theta >= 0.f)) return MTP_ERR_ARG;
  return MTP_OK;
}

// Kernels access tensors in 16-byte vectors: every device pointer (NULL
// aside) must be 16-byte aligned.
inline bool al16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
template <typename... P>
bool all_al16(const P *...p) { return (al16(p) && ...); }

int check_chain_ptrs(const mtp_chain_args *a) {
  if (!a->tokens || !a->segment_ids || !a->h0 || !a->embed || !a->w || !a->h_out || !a->state_mask ||
      !a->loss_mask || !a->labels || !a->counts || !a->device_error)
    return MTP_ERR_NULL;
  for (int k = 0; k < a->D; ++k) {
    const mtp_depth_weights &w = a->w[k];
    if (!w.g_h || !w.g_e || !w.g_attn || !w.g_ffn || !w.M || !w.Wqkv || !w.Wo || !w.Wgate || !w.Wup ||
        !w.Wdown || !a->h_out[k])
      return MTP_ERR_NULL;
  }
  if (!all_al16(a->tokens, a->segment_ids, a->h0, a->embed, a->state_mask, a->loss_mask, a->labels, a->counts,
                a->device_error, a->workspace))
    return MTP_ERR_ARG;
  for (int k = 0; k < a->D; ++k) {
    const mtp_depth_weights &w = a->w[k];
    if (!all_al16(w.g_h, w.g_e, w.g_attn, w.g_ffn, w.M, w.Wqkv, w.Wo, w.Wgate, w.Wup, w.Wdown, a->h_out[k]))
      return MTP_ERR_ARG;
  }
  return MTP_OK;
}

constexpr int kChainParts = 14;  // workspace regions of the chain call

// ---------------------------------------------------------------------------
// Saved activations (bf16 chain, optional): per depth, the activations of
// the forward that the reverse pass reads, so that it need not recompute
// them.  Depth k's record starts at k * saved_depth_bytes(...).
// ---------------------------------------------------------------------------
struct SavedDepth {
  bf16_t *c, *xa, *qkv, *o, *y;
  float *u, *a;
  float *gu;                                        // gate | up before SwiGLU [N, 2 ffn]
  float2 *lsed;
};
inline size_t saved_depth_layout(long N, int d, int A, int H, int f, Carve &c, SavedDepth &r) {
  r.c = c.take<bf16_t>(N * 2 * d);
  r.u = c.take<float>(N * d);
  r.xa = c.take<bf16_t>(N * d);
  r.qkv = c.take<bf16_t>(N * 3 * (long)A);
  r.o = c.take<bf16_t>(N * (long)A);
  r.lsed = c.take<float2>(N * H);
  r.a = c.take<float>(N * d);
  r.y = c.take<bf16_t>(N * d);
  r.gu = c.take<float>(N * 2 * (long)f);
  c.take<char>(0);                                  // the record ends aligned
  return c.off;
}
inline size_t saved_depth_bytes(long N, int d, int A, int H, int f) {
  Carve c(nullptr);
  SavedDepth r;
  return saved_depth_layout(N, d, A, H, f, c, r);
}
inline SavedDepth saved_depth(const void *base, int k, long N, int d, int A, int H, int f) {
  Carve c(static_cast<char *>(const_cast<void *>(base)) + (size_t)k * saved_depth_bytes(N, d, A, H, f));
  SavedDepth r;
  saved_depth_layout(N, d, A, H, f, c, r);
  return r;
}

template <typename T>
size_t chain_layout(const mtp_chain_args *a, Carve &c, void **parts) {
  const long N = (long)a->B * a->T;
  const int d = a->d, A = a->n_heads * a->head_dim, f = a->ffn;
  parts[0] = c.take<int32_t>(N);                              // run_start
  parts[1] = c.take<int32_t>(N);                              // pos
  parts[2] = c.take<int32_t>((size_t)a->D * a->B);             // cnt_part
  parts[3] = c.take<int32_t>(a->B);                            // err_part
  parts[4] = c.take<float2>((size_t)a->T * (a->head_dim / 2)); // rope table
  parts[5] = c.take<T>(N * 2 * d);                             // c
  parts[6] = c.take<float>(N * d);                             // u (residual stream, f32)
  parts[7] = c.take<T>(N * d);                                 // x_a
  parts[8] = c.take<T>(N * 3 * (long)A);                       // qkv
  parts[9] = c.take<T>(N * (long)A);                           // o
  parts[10] = c.take<float>(N * d);                            // a (residual stream, f32)
  parts[11] = c.take<T>(N * d);                                // y
  parts[12] = c.take<T>(N * (long)f);                          // silu(gate) * up
  parts[13] = c.take<float>(sizeof(T) == 2 ? tail_ws_bytes<Big>() / 4 : 0);  // partial tiles of split tail GEMM tiles
  return c.off;
}

template <typename T>
int chain_run(const mtp_chain_args *a, hipStream_t s) {
  void *p[kChainParts];
  Carve c(a->workspace);
  chain_layout<T>(a, c, p);
  const int B = a->B, Tl = a->T, d = a->d, H = a->n_heads, hd = a->head_dim, f = a->ffn, V = a->V;
  const int A = H * hd;
  const int N = B * Tl;
  int32_t *run_start = (int32_t *)p[0], *pos = (int32_t *)p[1];
  float2 *rope = (float2 *)p[4];
  T *cbuf = (T *)p[5], *xa = (T *)p[7], *qkv = (T *)p[8], *o = (T *)p[9];
  float *u = (float *)p[6];
  float *abuf = (float *)p[10];
  T *ybuf = (T *)p[11], *gsw = (T *)p[12];
  float *skws = sizeof(T) == 2 ? (float *)p[13] : nullptr;

  {
  MTP_STAGE(MTP_STAGE_ROWS);
  MTP_TRY(launch_rows(a->tokens, a->segment_ids, B, Tl, V, a->D, run_start, pos, a->state_mask, a->loss_mask,
                      a->labels, a->counts, a->device_error, (int32_t *)p[2], (int32_t *)p[3], s));
  }
  const bool use_rope = a->rope_theta > 0.f;
  if (use_rope) MTP_TRY(rope_table(rope, Tl, hd / 2, a->rope_theta, s));

  const T *h_prev = static_cast<const T *>(a->h0);
  const T *E = static_cast<const T *>(a->embed);
  float *lse2 = nullptr;                           // kept only with saved activations
  float *pre = nullptr;                            // gate | up before SwiGLU, likewise
  for (int k = 1; k <= a->D; ++k) {
    const mtp_depth_weights &w = a->w[k - 1];
    T *h_out = static_cast<T *>(a->h_out[k - 1]);
    int st = 0;
    if constexpr (std::is_same_v<T, bf16_t>) {
      if (a->saved != nullptr) {
        const SavedDepth sd = saved_depth(a->saved, k - 1, N, d, A, H, f);
        cbuf = sd.c; u = sd.u; xa = sd.xa; qkv = sd.qkv; o = sd.o; abuf = sd.a; ybuf = sd.y;
        lse2 = (float *)sd.lsed;
        pre = sd.gu;
      }
    }
    {
      MTP_STAGE(MTP_STAGE_DUAL_NORM);
      MTP_TRY(launch_dual_norm_concat<T>(h_prev, E, a->tokens, w.g_h, w.g_e, cbuf, B, Tl, d, V, k, a->eps, s));
    }
    {
      MTP_STAGE(MTP_STAGE_EH_PROJ);
      st = gemm_nt_store<T, float, float>(cbuf, 2L * d, (const T *)w.M, 2L * d, u, d, nullptr, 0, N, d, 2 * d, 1.f,
                                          nullptr, 0, skws, s);
    }
    if (st) return st;
    {
      MTP_STAGE(MTP_STAGE_NORM_A);
      MTP_TRY((launch_rmsnorm<float, T>(u, w.g_attn, xa, nullptr, N, d, a->eps, s)));
    }
    {
      MTP_STAGE(MTP_STAGE_QKV);
      st = gemm_qkv_rope<T>(xa, (const T *)w.Wqkv, qkv, pos, use_rope ? rope : nullptr, N, d, A, hd, skws, s);
    }
    if (st) return st;
    {
      MTP_STAGE(MTP_STAGE_ATTN);
      MTP_TRY(launch_attention<T>(qkv, o, run_start, lse2, B, Tl, H, hd, s));
    }
    {
      MTP_STAGE(MTP_STAGE_O_PROJ);
      st = gemm_nt_store<T, float, float>(o, A, (const T *)w.Wo, A, abuf, d, u, d, N, d, A, 1.f, nullptr, 0, skws,
                                          s);
    }
    if (st) return st;
    {
      MTP_STAGE(MTP_STAGE_NORM_F);
      MTP_TRY((launch_rmsnorm<float, T>(abuf, w.g_ffn, ybuf, nullptr, N, d, a->eps, s)));
    }
    {
      MTP_STAGE(MTP_STAGE_GATE_UP);
      st = gemm_swiglu<T>(ybuf, (const T *)w.Wgate, (const T *)w.Wup, gsw, N, d, f, skws, s, pre);
    }
    if (st) return st;
    {
      MTP_STAGE(MTP_STAGE_DOWN);
      st = gemm_nt_store<T, T, float>(gsw, f, (const T *)w.Wdown, f, h_out, d, abuf, d, N, d, f, 1.f, nullptr, 0,
                                      skws, s);
    }
    if (st) return st;
    h_prev = h_out;
  }
  return MTP_OK;
}

// ---------------------------------------------------------------------------
// Reverse pass of the chain (bf16)
// ---------------------------------------------------------------------------
// C[M, N] (+)= A[M, K] B[K, N] with B stored [K, N] (N contiguous).
template <typename T, typename OutT>
int gemm_nn(const T *A, long lda, const T *Bm, long ldb, OutT *C, long ldc, int M, int N, int K, int accumulate,
            float *skws, hipStream_t s) {
  EpiStore<OutT, float> epi{C, ldc, M, N, 1.f, nullptr, nullptr, 0, accumulate, 0};
  return pick<T>(use_big(M, N), [&](auto cfg) -> int {
    using Cfg = decltype(cfg);
    KA<T, Cfg> la{A, lda, M, K};
    MB_<T, Cfg> lb{Bm, ldb, N, K};
    MTP_TRY((run_gemm<T, Cfg>(la, lb, epi, M, N, K, 8, skws, s)));
    return (int)MTP_OK;
  });
}

// C[M, N] (+)= At^T Bt with At stored [K, M] and Bt stored [K, N] (the
// weight gradient dW = dY^T X of y = x W^T: At = dY, Bt = X, K = rows).
template <typename T>
int gemm_tn(const T *At, long lda, const T *Bt, long ldb, float *C, long ldc, int M, int N, int K, int accumulate,
            float *skws, hipStream_t s) {
  EpiStore<float, float> epi{C, ldc, M, N, 1.f, nullptr, nullptr, 0, accumulate, 0};
  return pick<T>(use_big(M, N), [&](auto cfg) -> int {
    using Cfg = decltype(cfg);
    MA<T, Cfg> la{At, lda, M, K};
    MB_<T, Cfg> lb{Bt, ldb, N, K};
    MTP_TRY((run_gemm<T, Cfg>(la, lb, epi, M, N, K, 8, skws, s)));
    return (int)MTP_OK;
  });
}

// Recomputed gate/up products of y with the SwiGLU reverse in the epilogue.
template <typename T>
int gemm_swiglu_bwd(const T *y, const T *Wg, const T *Wu, const T *dgsw, T *gsw, T *dgu, int M, int d, int f,
                    float *skws, hipStream_t s) {
  EpiSwiGLUBwd<T> epi{dgsw, gsw, dgu, M, f};
  return pick<T>(use_big(M, 2L * f), [&](auto cfg) -> int {
    using Cfg = decltype(cfg);
    PA<T, Cfg> la{y, (long)d, M, d};
    DmaKMajorSwiGLU<T, Cfg> lb{Wg, Wu, (long)d, f, d};
    MTP_TRY((run_gemm<T, Cfg>(la, lb, epi, M, 2 * ceil_div(f, Cfg::BN / 2) * (Cfg::BN / 2), d, 8, skws, s)));
    return (int)MTP_OK;
  });
}

int check_chain_bwd(const mtp_chain_bwd_args *a) {
  if (a == nullptr) return MTP_ERR_NULL;
  mtp_chain_args f{};
  f.B = a->B; f.T = a->T; f.d = a->d; f.n_heads = a->n_heads; f.head_dim = a->head_dim; f.ffn = a->ffn;
  f.V = a->V; f.D = a->D; f.dtype = a->dtype; f.eps = a->eps; f.rope_theta = a->rope_theta;
  const int st = check_chain(&f);
  if (st) return st;
  if (a->dtype != MTP_BF16) return MTP_ERR_UNSUPPORTED;
  if (a->head_dim != 64 && a->head_dim != 128) return MTP_ERR_UNSUPPORTED;
  if (a->d > 8192) return MTP_ERR_UNSUPPORTED;
  return MTP_OK;
}

int check_chain_bwd_ptrs(const mtp_chain_bwd_args *a) {
  if (!a->tokens || !a->segment_ids || !a->h0 || !a->embed || !a->w || !a->h || !a->dh || !a->dh0 || !a->dE ||
      !a->dw)
    return MTP_ERR_NULL;
  for (int k = 0; k < a->D; ++k) {
    const mtp_depth_weights &w = a->w[k];
    const mtp_depth_grads &g = a->dw[k];
    if (!w.g_h || !w.g_e || !w.g_attn || !w.g_ffn || !w.M || !w.Wqkv || !w.Wo || !w.Wgate || !w.Wup || !w.Wdown ||
        !g.g_h || !g.g_e || !g.g_attn || !g.g_ffn || !g.M || !g.Wqkv || !g.Wo || !g.Wgate || !g.Wup || !g.Wdown ||
        !a->dh[k] || (k + 1 < a->D && !a->h[k]))
      return MTP_ERR_NULL;
    if (!all_al16(w.g_h, w.g_e, w.g_attn, w.g_ffn, w.M, w.Wqkv, w.Wo, w.Wgate, w.Wup, w.Wdown) ||
        !all_al16(g.g_h, g.g_e, g.g_attn, g.g_ffn, g.M, g.Wqkv, g.Wo, g.Wgate, g.Wup, g.Wdown) ||
        !all_al16(a->dh[k], a->h[k]))
      return MTP_ERR_ARG;
  }
  if (!all_al16(a->tokens, a->segment_ids, a->h0, a->embed, a->dh0, a->dE, a->device_error, a->workspace))
    return MTP_ERR_ARG;
  return MTP_OK;
}

constexpr int kBwdParts = 40;     // workspace regions of the reverse pass

size_t chain_bwd_layout(const mtp_chain_bwd_args *a, Carve &c, void **p) {
  using T = bf16_t;
  const long N = (long)a->B * a->T;
  const int d = a->d, A = a->n_heads * a->head_dim, f = a->ffn, H = a->n_heads, D = a->D;
  p[0] = c.take<int32_t>(N);                      // run_start
  p[1] = c.take<int32_t>(N);                      // pos
  p[2] = c.take<int32_t>((size_t)D * a->B);       // count partials
  p[3] = c.take<int32_t>(a->B);                   // error partials
  p[4] = c.take<uint8_t>((size_t)D * N);          // state masks
  p[5] = c.take<uint8_t>((size_t)D * N);          // loss masks
  p[6] = c.take<int32_t>((size_t)D * N);          // labels
  p[7] = c.take<int32_t>(D);                      // counts
  p[8] = c.take<int32_t>(1);                      // error flag (when the caller passes none)
  p[9] = c.take<float2>((size_t)a->T * (a->head_dim / 2));   // RoPE table
  p[10] = c.take<T>(N * 2 * d);                   // c
  p[11] = c.take<float>(N * d);                   // u
  p[12] = c.take<T>(N * d);                       // x_a
  p[13] = c.take<T>(N * 3 * (long)A);             // qkv
  p[14] = c.take<T>(N * (long)A);                 // o
  p[15] = c.take<float2>(N * H);                  // (lse2, D) per (batch row, head, position)
  p[16] = c.take<float>(N * d);                   // a
  p[17] = c.take<T>(N * d);                       // y
  p[18] = c.take<T>(N * (long)f);                 // silu(gate) * up
  p[19] = c.take<float>(N * d);                   // gradient arriving at h^(k) (carry)
  p[20] = c.take<T>(N * d);                       // its bf16 copy
  p[21] = c.take<T>(N * (long)f);                 // d(silu(gate) * up)
  p[22] = c.take<T>(N * 2 * (long)f);             // [d gate | d up]
  p[23] = c.take<float>(N * d);                   // dy
  p[24] = c.take<float>(N * d);                   // da
  p[25] = c.take<T>(N * d);                       // da (bf16)
  p[26] = c.take<T>(N * (long)A);                 // dO
  p[27] = c.take<char>(0);                        // (D lives beside lse2)
  p[28] = c.take<T>(N * 3 * (long)A);             // dqkv
  p[29] = c.take<float>(N * d);                   // dx_a
  p[30] = c.take<float>(N * d);                   // du
  p[31] = c.take<T>(N * d);                       // du (bf16)
  p[32] = c.take<float>(N * 2 * d);               // dc
  p[33] = c.take<float>(N * d);                   // de
  p[34] = c.take<int32_t>(5 * N);                 // shifted tokens, keys, rows, sorted keys, sorted rows
  p[35] = c.take<char>(embed_grad_sort_bytes((int)N, a->V));   // radix sort scratch
  p[36] = c.take<float>((size_t)dg_row_blocks((int)N) * d);    // gain-gradient partials
  p[37] = c.take<float>(tail_ws_bytes<Big>() / 4);            // partial tiles of split tail GEMM tiles
  p[38] = c.take<char>(0);
  p[39] = c.take<char>(0);
  return c.off;
}

// One Transformer block's reverse (bf16): buffers, weights and gradients.
struct BlockBufs {
  bf16_t *xa, *qkv, *o, *y, *gsw;       // stored activations (x_a, q|k|v after RoPE, o, y, SwiGLU product)
  float2 *lsed;                         // (lse2, D) pairs [B, H, T]: attention log-sum-exps and dO . o
  float *a;                             // residual after attention
  bf16_t *gb, *dgsw, *dgu, *dab, *dO, *dqkv, *dub;
  float *dy, *da, *dxa, *du;
  float *part, *skws;
  const int32_t *run_start, *pos;
  const float2 *rope;                   // NULL: no RoPE
  const float *gu;                      // gate | up before SwiGLU [N, 2f] f32, or NULL: recomputed
};
struct BlockW {
  const float *g_attn, *g_ffn;
  const bf16_t *Wqkv, *Wo, *Wgate, *Wup, *Wdown;
};
struct BlockG {
  float *g_attn, *g_ffn, *Wqkv, *Wo, *Wgate, *Wup, *Wdown;
};

// Reverse of out = a + FFN(Norm_f(a)), a = u + Attn(Norm_a(u)) from the
// stored activations, given dL/dout = gcur (f32) and its bf16 copy in
// b.gb: every weight and gain gradient of the block (written, or added
// with acc) and du = dL/du in b.du (f32) and b.dub (bf16).  The block input
// u is TU (f32: the module's residual stream; bf16: a trunk state).
template <typename TU>
int block_bwd(const BlockBufs &b, const BlockW &w, const BlockG &g, const TU *u, const float *gcur, int acc, int B,
              int Tl, int d, int H, int hd, int f, float eps, hipStream_t s) {
  using T = bf16_t;
  const int A = H * hd, N = B * Tl;
  int st = 0;
  float *skws = b.skws;
  // ---- out = a + gsw W_down^T: the MLP's reverse and Norm_f's
  {
    MTP_STAGE(MTP_STAGE_BWD_MLP);
    if ((st = gemm_nn<T, T>(b.gb, d, w.Wdown, f, b.dgsw, f, N, f, d, 0, skws, s))) return st;
    // with the forward's pre-activations kept, their reverse is elementwise;
    // else the gate/up product runs again with the reverse as its epilogue
    if (b.gu != nullptr) MTP_TRY(launch_swiglu_bwd(b.gu, b.dgsw, b.gsw, b.dgu, N, f, s));
    else if ((st = gemm_swiglu_bwd<T>(b.y, w.Wgate, w.Wup, b.dgsw, b.gsw, b.dgu, N, d, f, skws, s))) return st;
    if ((st = gemm_tn<T>(b.gb, d, b.gsw, f, g.Wdown, f, d, f, N, acc, skws, s))) return st;
    if ((st = gemm_nn<T, float>(b.dgu, 2L * f, w.Wgate, d, b.dy, d, N, d, f, 0, skws, s))) return st;
    if ((st = gemm_nn<T, float>(b.dgu + f, 2L * f, w.Wup, d, b.dy, d, N, d, f, 1, skws, s))) return st;
    if ((st = gemm_tn<T>(b.dgu, 2L * f, b.y, d, g.Wgate, d, f, d, N, acc, skws, s))) return st;
    if ((st = gemm_tn<T>(b.dgu + f, 2L * f, b.y, d, g.Wup, d, f, d, N, acc, skws, s))) return st;
    MTP_TRY(launch_rms_bwd<float>(b.dy, d, b.a, nullptr, w.g_ffn, eps, gcur, nullptr, b.da, b.dab, b.part, g.g_ffn,
                                  acc, N, d, s));
  }
  // ---- a = u + o W_o^T
  {
    MTP_STAGE(MTP_STAGE_BWD_ATTN_PROJ);
    if ((st = gemm_nn<T, T>(b.dab, d, w.Wo, A, b.dO, A, N, A, d, 0, skws, s))) return st;
    if ((st = gemm_tn<T>(b.dab, d, b.o, A, g.Wo, A, d, A, N, acc, skws, s))) return st;
  }
  {
    MTP_STAGE(MTP_STAGE_BWD_ATTN);
    MTP_TRY(launch_attention_bwd(b.qkv, b.o, b.dO, b.lsed, b.run_start, b.pos, b.rope, b.dqkv, B, Tl, H, hd, s));
  }
  // ---- qkv = x_a W_qkv^T, x_a = Norm_a(u)
  {
    MTP_STAGE(MTP_STAGE_BWD_QKV);
    if ((st = gemm_nn<T, float>(b.dqkv, 3L * A, w.Wqkv, d, b.dxa, d, N, d, 3 * A, 0, skws, s))) return st;
    if ((st = gemm_tn<T>(b.dqkv, 3L * A, b.xa, d, g.Wqkv, d, 3 * A, d, N, acc, skws, s))) return st;
    MTP_TRY(launch_rms_bwd<TU>(b.dxa, d, u, nullptr, w.g_attn, eps, b.da, nullptr, b.du, b.dub, b.part, g.g_attn,
                               acc, N, d, s));
  }
  return MTP_OK;
}

__global__ void to_bf16_kernel(const float *__restrict__ x, bf16_t *__restrict__ y, long n4) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4 *>(x)[i];
  reinterpret_cast<uint2 *>(y)[i] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

int chain_bwd_run(const mtp_chain_bwd_args *a, hipStream_t s) {
  using T = bf16_t;
  void *p[kBwdParts];
  Carve c(a->workspace);
  chain_bwd_layout(a, c, p);
  const int B = a->B, Tl = a->T, d = a->d, H = a->n_heads, hd = a->head_dim, f = a->ffn, V = a->V, D = a->D;
  const int A = H * hd;
  const int N = B * Tl;
  int32_t *run_start = (int32_t *)p[0], *pos = (int32_t *)p[1];
  uint8_t *state = (uint8_t *)p[4];
  float2 *rope = (float2 *)p[9];
  T *cbuf = (T *)p[10], *xa = (T *)p[12], *qkv = (T *)p[13], *o = (T *)p[14], *ybuf = (T *)p[17];
  T *gsw = (T *)p[18];
  float *u = (float *)p[11], *abuf = (float *)p[16];
  float2 *lsed = (float2 *)p[15];
  float *gbuf = (float *)p[19];
  T *gb = (T *)p[20], *dgsw = (T *)p[21], *dgu = (T *)p[22];
  float *dy = (float *)p[23], *da = (float *)p[24];
  T *dab = (T *)p[25], *dO = (T *)p[26];
  T *dqkv = (T *)p[28];
  float *dxa = (float *)p[29], *du = (float *)p[30];
  T *dub = (T *)p[31];
  float *dc = (float *)p[32], *de = (float *)p[33];
  int32_t *ids = (int32_t *)p[34];
  int32_t *tok = ids, *key = ids + N, *val = ids + 2L * N, *key_s = ids + 3L * N, *val_s = ids + 4L * N;
  void *sort_tmp = p[35];
  const size_t sort_bytes = embed_grad_sort_bytes(N, V);
  float *part = (float *)p[36];
  float *skws = (float *)p[37];
  const int acc = a->accumulate ? 1 : 0;
  const T *E = static_cast<const T *>(a->embed);
  const bool use_rope = a->rope_theta > 0.f;

  MTP_TRY(launch_rows(a->tokens, a->segment_ids, B, Tl, V, D, run_start, pos, state, (uint8_t *)p[5],
                      (int32_t *)p[6], (int32_t *)p[7], a->device_error ? a->device_error : (int32_t *)p[8],
                      (int32_t *)p[2], (int32_t *)p[3], s));
  if (use_rope) MTP_TRY(rope_table(rope, Tl, hd / 2, a->rope_theta, s));

  for (int k = D; k >= 1; --k) {
    const mtp_depth_weights &w = a->w[k - 1];
    const mtp_depth_grads &g = a->dw[k - 1];
    const T *hprev = static_cast<const T *>(k == 1 ? a->h0 : a->h[k - 2]);
    const uint8_t *st_k = state + (long)(k - 1) * N;
    const float *gcur = k == D ? a->dh[D - 1] : gbuf;
    int st = 0;
    // this depth's forward activations: the caller's saved record, or the
    // module's forward run again here (as chain_run), keeping lse2
    T *cbk = cbuf, *xak = xa, *qkvk = qkv, *ok = o, *yk = ybuf;
    float *uk = u, *ak = abuf;
    const float *guk = nullptr;
    float2 *lsk = lsed;
    if (a->saved != nullptr) {
      const SavedDepth sd = saved_depth(a->saved, k - 1, N, d, A, H, f);
      cbk = sd.c; xak = sd.xa; qkvk = sd.qkv; ok = sd.o; yk = sd.y; uk = sd.u; ak = sd.a; lsk = sd.lsed;
      guk = sd.gu;
    } else {
      MTP_STAGE(MTP_STAGE_BWD_RECOMPUTE);
      MTP_TRY(launch_dual_norm_concat<T>(hprev, E, a->tokens, w.g_h, w.g_e, cbk, B, Tl, d, V, k, a->eps, s));
      if ((st = gemm_nt_store<T, float, float>(cbk, 2L * d, (const T *)w.M, 2L * d, uk, d, nullptr, 0, N, d, 2 * d,
                                               1.f, nullptr, 0, skws, s)))
        return st;
      MTP_TRY((launch_rmsnorm<float, T>(uk, w.g_attn, xak, nullptr, N, d, a->eps, s)));
      if ((st = gemm_qkv_rope<T>(xak, (const T *)w.Wqkv, qkvk, pos, use_rope ? rope : nullptr, N, d, A, hd, skws, s)))
        return st;
      MTP_TRY(launch_attention<T>(qkvk, ok, run_start, (float *)lsk, B, Tl, H, hd, s));
      if ((st = gemm_nt_store<T, float, float>(ok, A, (const T *)w.Wo, A, ak, d, uk, d, N, d, A, 1.f, nullptr, 0,
                                               skws, s)))
        return st;
      MTP_TRY((launch_rmsnorm<float, T>(ak, w.g_ffn, yk, nullptr, N, d, a->eps, s)));
    }
    // ---- the block (MLP, attention, their norms), down to du
    if (k == D) {
      const long n4 = (long)N * d / 4;
      hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, gcur, gb, n4);
      MTP_TRY(hipGetLastError());
    }
    {
      const BlockBufs bb{xak, qkvk, ok, yk, gsw, lsk, ak, gb, dgsw, dgu, dab, dO, dqkv, dub, dy, da, dxa, du,
                         part, skws, run_start, pos, use_rope ? rope : nullptr, guk};
      const BlockW bw{w.g_attn, w.g_ffn, (const T *)w.Wqkv, (const T *)w.Wo, (const T *)w.Wgate, (const T *)w.Wup,
                      (const T *)w.Wdown};
      const BlockG bg{g.g_attn, g.g_ffn, g.Wqkv, g.Wo, g.Wgate, g.Wup, g.Wdown};
      if ((st = block_bwd<float>(bb, bw, bg, uk, gcur, acc, B, Tl, d, H, hd, f, a->eps, s))) return st;
    }
    // ---- u = M [h_bar; e_bar]: eh_proj, enorm (into dE) and hnorm (the
    // gradient carried to depth k-1, or dh0)
    {
      MTP_STAGE(MTP_STAGE_BWD_EH);
      if ((st = gemm_nn<T, float>(dub, d, (const T *)w.M, 2L * d, dc, 2L * d, N, 2 * d, d, 0, skws, s))) return st;
      if ((st = gemm_tn<T>(dub, d, cbk, 2L * d, g.M, 2L * d, d, 2 * d, N, acc, skws, s))) return st;
      MTP_TRY(launch_shifted_rows(a->tokens, st_k, B, Tl, V, k, tok, key, val, s));
      MTP_TRY(launch_rms_bwd<T>(dc + d, 2L * d, E, tok, w.g_e, a->eps, nullptr, st_k, de, nullptr, part, g.g_e, acc,
                                N, d, s));
      MTP_TRY(launch_embed_grad(key, val, key_s, val_s, sort_tmp, sort_bytes, N, V, de, d, a->dE, s));
      MTP_TRY(launch_rms_bwd<T>(dc, 2L * d, hprev, nullptr, w.g_h, a->eps, k > 1 ? a->dh[k - 2] : nullptr, st_k,
                                k > 1 ? gbuf : a->dh0, k > 1 ? gb : nullptr, part, g.g_h, acc, N, d, s));
    }
  }
  return MTP_OK;
}

// ---------------------------------------------------------------------------
// Independent horizon heads (block heads, sequential per-head schedule)
// ---------------------------------------------------------------------------
// labels[n] = x[b, t + k] where t and t + k lie in one run, else -1 (tokens
// outside [0, V) pass through: the head CE flags and drops them).
__global__ void horizon_labels_kernel(const int32_t *__restrict__ tokens, const int32_t *__restrict__ seg,
                                      const int32_t *__restrict__ run_start, int B, int T_len, int k,
                                      int32_t *__restrict__ labels) {
  const long n = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= (long)B * T_len) return;
  const int t = (int)(n % T_len);
  int lab = -1;
  if (seg[n] >= 0 && t + k < T_len && run_start[n + k] == run_start[n]) lab = tokens[n + k];
  labels[n] = lab;
}

// y = x (first head) or y += x, 4 floats per thread
__global__ void add_rows_kernel(float *__restrict__ y, const float *__restrict__ x, long n4, int first) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4 *>(x)[i];
  float4 *py = reinterpret_cast<float4 *>(y) + i;
  if (first) {
    *py = v;
  } else {
    float4 o = *py;
    o.x += v.x; o.y += v.y; o.z += v.z; o.w += v.w;
    *py = o;
  }
}

// Per-head CE outputs (slot k at index 4 k) -> the caller's arrays; the
// total objective summed in head order; error flags or-ed.
__global__ void horizon_finalize_kernel(const float *__restrict__ hl_loss, const int32_t *__restrict__ hl_counts,
                                        const float *__restrict__ hl_mtp, const int32_t *__restrict__ hl_err,
                                        const int32_t *__restrict__ rows_err, int K, float *loss, int32_t *counts,
                                        float *loss_total, int32_t *device_error) {
  if (threadIdx.x != 0) return;
  float tot = 0.f;
  int err = rows_err[0];
  for (int k = 0; k < K; ++k) {
    loss[k] = hl_loss[4 * k];
    counts[k] = hl_counts[4 * k];
    tot += hl_mtp[4 * k];
    err |= hl_err[4 * k];
  }
  loss_total[0] = tot;
  if (device_error != nullptr) device_error[0] = err ? 1 : 0;
}

int check_horizon(const mtp_horizon_args *a) {
  if (a == nullptr) return MTP_ERR_NULL;
  if (a->K < 1) return MTP_ERR_DEPTH;
  mtp_chain_bwd_args c{};
  c.B = a->B; c.T = a->T; c.d = a->d; c.n_heads = a->n_heads; c.head_dim = a->head_dim; c.ffn = a->ffn;
  c.V = a->V; c.D = 1; c.dtype = a->dtype; c.eps = a->eps; c.rope_theta = a->rope_theta;
  const int st = check_chain_bwd(&c);
  if (st) return st;
  if (a->V % 8 || a->V >= (1 << 21)) return MTP_ERR_SHAPE;
  if (!isfinite(a->lambda)) return MTP_ERR_ARG;
  return MTP_OK;
}

constexpr int kHorParts = 36;     // workspace regions of the horizon heads

// The head CE arguments of head k (D = 1) over the given workspace.
mtp_ce_args horizon_ce_args(const mtp_horizon_args *a, void *const *hptr, void *const *dhptr, const int32_t *labels,
                            float *hl_sum, int32_t *hl_counts, float *hl_loss, float *hl_mtp, int32_t *hl_err, int k,
                            void *ws, size_t ws_bytes) {
  mtp_ce_args c{};
  c.B = a->B; c.T = a->T; c.d = a->d; c.V = a->V; c.D = 1; c.dtype = a->dtype; c.eps = a->eps;
  c.lambda = a->lambda / (float)a->K;
  c.reduce = MTP_REDUCE_FIXED;
  c.denom = 0.0;
  c.h = hptr;
  c.labels = labels;
  c.W_out = a->W_out;
  c.g_out = a->g_out;
  c.loss_sum = hl_sum + 4 * k; c.counts = hl_counts + 4 * k; c.loss = hl_loss + 4 * k; c.loss_mtp = hl_mtp + 4 * k;
  c.lse = nullptr;
  c.dh = dhptr;
  c.dW_out = a->dW_out; c.dg_out = a->dg_out;
  c.accumulate = (k > 0 || a->accumulate) ? 1 : 0;
  c.device_error = hl_err + 4 * k;
  c.logit_slab_bytes = 0;
  c.dh_accumulate = 0;
  c.pred = nullptr; c.correct = nullptr; c.accuracy = nullptr;
  c.workspace = ws;
  c.workspace_bytes = ws_bytes;
  return c;
}

size_t horizon_layout(const mtp_horizon_args *a, Carve &c, void **p) {
  using T = bf16_t;
  const long N = (long)a->B * a->T;
  const int d = a->d, A = a->n_heads * a->head_dim, f = a->ffn, H = a->n_heads, K = a->K;
  p[0] = c.take<int32_t>(N);                      // run_start
  p[1] = c.take<int32_t>(N);                      // pos
  p[2] = c.take<int32_t>(a->B);                   // count partials (rows kernel, one depth)
  p[3] = c.take<int32_t>(a->B);                   // error partials
  p[4] = c.take<uint8_t>(N);                      // state mask (unused)
  p[5] = c.take<uint8_t>(N);                      // loss mask (unused)
  p[6] = c.take<int32_t>(N);                      // chain labels (unused)
  p[7] = c.take<int32_t>(1);                      // chain count (unused)
  p[8] = c.take<int32_t>(1);                      // token error flag
  p[9] = c.take<float2>((size_t)a->T * (a->head_dim / 2));   // RoPE table
  p[10] = c.take<T>(N * d);                       // x_a
  p[11] = c.take<T>(N * 3 * (long)A);             // qkv
  p[12] = c.take<T>(N * (long)A);                 // o
  p[13] = c.take<float2>(N * H);                  // (lse2, D) per (batch row, head, position)
  p[14] = c.take<float>(N * d);                   // a
  p[15] = c.take<T>(N * d);                       // y
  p[16] = c.take<T>(N * (long)f);                 // silu(gate) * up
  p[17] = c.take<T>(N * d);                       // the head output u^(k)
  p[18] = c.take<T>(N * d);                       // dL/du^(k) (bf16)
  p[19] = c.take<T>(N * (long)f);                 // d(silu(gate) * up)
  p[20] = c.take<T>(N * 2 * (long)f);             // [d gate | d up]
  p[21] = c.take<float>(N * d);                   // dy
  p[22] = c.take<float>(N * d);                   // da
  p[23] = c.take<T>(N * d);                       // da (bf16)
  p[24] = c.take<T>(N * (long)A);                 // dO
  p[25] = c.take<float>(N * 2 * (long)f);         // gate | up before SwiGLU (f32), for the reverse
  p[26] = c.take<T>(N * 3 * (long)A);             // dqkv
  p[27] = c.take<float>(N * d);                   // dx_a
  p[28] = c.take<float>(N * d);                   // du (the head's share of dh)
  p[29] = c.take<T>(N * d);                       // du (bf16)
  p[30] = c.take<int32_t>(N);                     // horizon labels
  p[31] = c.take<float>(N * d);                   // dL/du^(k) (f32, from the head CE)
  p[32] = c.take<float>((size_t)dg_row_blocks((int)N) * d);   // gain-gradient partials
  p[33] = c.take<float>(tail_ws_bytes<Big>() / 4);            // partial tiles of split tail GEMM tiles
  p[34] = c.take<float>(5 * 4 * (size_t)K);       // per-head CE scalars (sum, counts, loss, objective, error)
  mtp_ce_args ce = horizon_ce_args(a, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                                   nullptr, 0);
  p[35] = c.take<char>(mtp_ce_workspace_size(&ce));            // the head CE's workspace
  return c.off;
}

int horizon_run(const mtp_horizon_args *a, hipStream_t s) {
  using T = bf16_t;
  void *p[kHorParts];
  Carve c(a->workspace);
  const size_t total = horizon_layout(a, c, p);
  const int B = a->B, Tl = a->T, d = a->d, H = a->n_heads, hd = a->head_dim, f = a->ffn, V = a->V, K = a->K;
  const int A = H * hd;
  const int N = B * Tl;
  int32_t *run_start = (int32_t *)p[0], *pos = (int32_t *)p[1];
  float2 *rope = (float2 *)p[9];
  const bool use_rope = a->rope_theta > 0.f;
  T *xa = (T *)p[10], *qkv = (T *)p[11], *o = (T *)p[12], *ybuf = (T *)p[15], *gsw = (T *)p[16], *out = (T *)p[17];
  float2 *lsed = (float2 *)p[13];
  float *abuf = (float *)p[14];
  float *dhk = (float *)p[31];
  int32_t *hlab = (int32_t *)p[30];
  float *small = (float *)p[34];
  float *hl_sum = small, *hl_loss = small + 8 * K, *hl_mtp = small + 12 * K;
  int32_t *hl_counts = (int32_t *)(small + 4 * K), *hl_err = (int32_t *)(small + 16 * K);
  const T *h = static_cast<const T *>(a->h);
  const BlockBufs bb{xa, qkv, o, ybuf, gsw, lsed, abuf, (T *)p[18], (T *)p[19], (T *)p[20], (T *)p[23],
                     (T *)p[24], (T *)p[26], (T *)p[29], (float *)p[21], (float *)p[22], (float *)p[27],
                     (float *)p[28], (float *)p[32], (float *)p[33], run_start, pos, use_rope ? rope : nullptr,
                     (const float *)p[25]};
  const size_t ce_bytes = total - (size_t)((char *)p[35] - (char *)a->workspace);
  const int acc = a->accumulate ? 1 : 0;

  MTP_TRY(launch_rows(a->tokens, a->segment_ids, B, Tl, V, 1, run_start, pos, (uint8_t *)p[4], (uint8_t *)p[5],
                      (int32_t *)p[6], (int32_t *)p[7], (int32_t *)p[8], (int32_t *)p[2], (int32_t *)p[3], s));
  if (use_rope) MTP_TRY(rope_table(rope, Tl, hd / 2, a->rope_theta, s));
  void *hptr[1] = {out};
  void *dhptr[1] = {dhk};
  for (int k = 0; k < K; ++k) {
    const mtp_block_weights &w = a->w[k];
    const mtp_block_grads &g = a->dw[k];
    const BlockW bw{w.g_attn, w.g_ffn, (const T *)w.Wqkv, (const T *)w.Wo, (const T *)w.Wgate, (const T *)w.Wup,
                    (const T *)w.Wdown};
    const BlockG bg{g.g_attn, g.g_ffn, g.Wqkv, g.Wo, g.Wgate, g.Wup, g.Wdown};
    int st = 0;
    // ---- head k's block forward: u^(k) = Block_k(h)
    {
      MTP_STAGE(MTP_STAGE_BWD_RECOMPUTE);
      MTP_TRY((launch_rmsnorm<T, T>(h, w.g_attn, xa, nullptr, N, d, a->eps, s)));
      if ((st = gemm_qkv_rope<T>(xa, bw.Wqkv, qkv, pos, use_rope ? rope : nullptr, N, d, A, hd, (float *)p[33], s)))
        return st;
      MTP_TRY(launch_attention<T>(qkv, o, run_start, (float *)lsed, B, Tl, H, hd, s));
      if ((st = gemm_nt_store<T, float, T>(o, A, bw.Wo, A, abuf, d, h, d, N, d, A, 1.f, nullptr, 0, (float *)p[33],
                                           s)))
        return st;
      MTP_TRY((launch_rmsnorm<float, T>(abuf, w.g_ffn, ybuf, nullptr, N, d, a->eps, s)));
      if ((st = gemm_swiglu<T>(ybuf, bw.Wgate, bw.Wup, gsw, N, d, f, (float *)p[33], s, (float *)p[25]))) return st;
      if ((st = gemm_nt_store<T, T, float>(gsw, f, bw.Wdown, f, out, d, abuf, d, N, d, f, 1.f, nullptr, 0,
                                           (float *)p[33], s)))
        return st;
    }
    // ---- the shared head on u^(k): labels x[t + k + 1] (horizon k + 1), loss and dL/du^(k)
    hipLaunchKernelGGL(horizon_labels_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, a->tokens,
                       a->segment_ids, run_start, B, Tl, k + 1, hlab);
    MTP_TRY(hipGetLastError());
    const mtp_ce_args ce = horizon_ce_args(a, hptr, dhptr, hlab, hl_sum, hl_counts, hl_loss, hl_mtp, hl_err, k,
                                           p[35], ce_bytes);
    if ((st = mtp_head_ce_fwd_bwd(&ce, s))) return st;
    // ---- head k's block backward; its share of the trunk gradient into dh
    const long n4 = (long)N * d / 4;
    hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, dhk, bb.gb, n4);
    MTP_TRY(hipGetLastError());
    if ((st = block_bwd<T>(bb, bw, bg, h, dhk, acc, B, Tl, d, H, hd, f, a->eps, s))) return st;
    hipLaunchKernelGGL(add_rows_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, a->dh, bb.du, n4,
                       k == 0 ? 1 : 0);
    MTP_TRY(hipGetLastError());
  }
  hipLaunchKernelGGL(horizon_finalize_kernel, dim3(1), dim3(64), 0, s, hl_loss, hl_counts, hl_mtp, hl_err,
                     (const int32_t *)p[8], K, a->loss, a->counts, a->loss_total, a->device_error);
  return hipGetLastError() == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}

int check_ce(const mtp_ce_args *a) {
  if (a == nullptr) return MTP_ERR_NULL;
  if (a->D < 1) return MTP_ERR_DEPTH;
  if (a->dtype != MTP_F32 && a->dtype != MTP_BF16) return MTP_ERR_DTYPE;
  if (a->B < 1 || a->T < 1 || a->d < 1 || a->V < 1) return MTP_ERR_SHAPE;
  const int E = a->dtype == MTP_BF16 ? 8 : 4;
  if (a->d % E || a->V % E) return MTP_ERR_SHAPE;
  if ((long)a->B * a->T > (1L << 30)) return MTP_ERR_SHAPE;
  if (a->V >= (1 << 21)) return MTP_ERR_SHAPE;   // a 256-row logit tile spans < 2 GiB
  if (a->reduce != MTP_REDUCE_FIXED && a->reduce != MTP_REDUCE_VALID_MEAN) return MTP_ERR_ARG;
  if (a->reduce == MTP_REDUCE_FIXED && !(a->denom >= 0.0)) return MTP_ERR_ARG;
  if (!(a->eps >= 0.f) || !isfinite(a->lambda)) return MTP_ERR_ARG;
  return MTP_OK;
}

int check_ce_ptrs(const mtp_ce_args *a) {
  if (!a->h || !a->labels || !a->W_out || !a->g_out || !a->loss_sum || !a->counts || !a->loss ||
      !a->loss_mtp || !a->dh || !a->dW_out || !a->dg_out)
    return MTP_ERR_NULL;
  for (int k = 0; k < a->D; ++k)
    if (!a->h[k] || !a->dh[k]) return MTP_ERR_NULL;
  if (!all_al16(a->labels, a->W_out, a->g_out, a->loss_sum, a->counts, a->loss, a->loss_mtp, a->lse, a->dW_out,
                a->dg_out, a->device_error, a->workspace) ||
      !all_al16(a->pred, a->correct, a->accuracy))
    return MTP_ERR_ARG;
  for (int k = 0; k < a->D; ++k)
    if (!all_al16(a->h[k], a->dh[k])) return MTP_ERR_ARG;
  return MTP_OK;
}

struct CeDims {
  long N, ldT; int d, V, nt, splits; bool big, big_dx;
  long slab;          // rows per logit slab (logits kept as LogitT)
  long group;         // rows per dz buffer: a whole number of slabs (or all N rows)
};

constexpr size_t kDefaultLogitSlab = size_t(1) << 30;

template <typename T>
CeDims ce_dims(const mtp_ce_args *a) {
  CeDims c;
  c.N = (long)a->B * a->T;
  c.d = a->d;
  c.V = a->V;
  const size_t budget = a->logit_slab_bytes ? a->logit_slab_bytes : kDefaultLogitSlab;
  // a slab keeps its logits as LogitT (fp16 offsets for bf16 runs): the more
  // rows a slab holds, the fewer times the forward GEMM streams W_out from
  // HBM and the fewer partly filled rounds of tiles it runs
  long r = (long)(budget / ((size_t)c.V * sizeof(LogitT<T>)));
  if (a->logit_slab_bytes == 0 && c.N > 1) {
    // under the default bound a slab never keeps the logits of the whole
    // batch: at most half of its rows (rounded up to a multiple of 256 from
    // 256 rows on, which stays below the row count)
    long half = (c.N + 1) / 2;
    if (half >= 256) half = (half + 255) / 256 * 256;
    r = r < half ? r : half;
  }
  if (r >= 256) r -= r % 256;
  c.slab = r < 1 ? 1 : (r > c.N ? c.N : r);
  // dz is stored in T (as wide as LogitT): the dx_hat / dW_out GEMMs run once
  // per group of G rows with G * V * sizeof(T) within the same budget
  long g = (long)(budget / ((size_t)c.V * sizeof(T)));
  g -= g % c.slab;
  c.group = g < c.slab ? c.slab : (g > c.N ? c.N : g);
  c.big = sizeof(T) == 2 && use_big(c.slab, c.V);
  c.nt = ceil_div(c.V, c.big ? 256 : 128);
  c.ldT = (c.N + 7) / 8 * 8;                    // x_hat^T leading dimension (bf16 runs)
  // the dx_hat GEMM (group rows x d, K = V) may also fill the chip with K splits
  c.big_dx = sizeof(T) == 2 && (long)ceil_div(c.group, 256) * ceil_div(c.d, 256) * 8 >= 256;
  // with a round of 256x256 tiles or more the dx GEMM needs no K splits of
  // its own: the balanced schedule splits only the last partial round
  const bool dx_balanced = c.big_dx && (long)ceil_div(c.group, 256) * ceil_div(c.d, 256) >= kGemmSlots;
  c.splits = dx_balanced ? 1 : dx_splits((int)c.group, c.d, c.V, c.big_dx);
  return c;
}

constexpr int kCeParts = 19;     // workspace regions of the CE call

template <typename T>
size_t ce_layout(const mtp_ce_args *a, Carve &c, void **p) {
  const CeDims m = ce_dims<T>(a);
  p[0] = c.take<T>(m.N * m.d);                   // x_hat
  p[1] = c.take<float>(m.N);                     // r = 1 / rms
  p[2] = c.take<int32_t>(m.N);                   // sanitised labels
  p[3] = c.take<float2>(m.slab * m.nt);          // (max, sumexp) per slab row and vocab tile
  p[4] = c.take<float>(m.N);                     // target logit
  p[5] = c.take<float>(m.N);                     // lse
  p[6] = c.take<float>(m.N);                     // row loss
  p[7] = c.take<double>(a->D);                   // loss sums
  p[8] = c.take<int32_t>(a->D);                  // counts
  p[9] = c.take<float>(a->D);                    // backward scales
  p[10] = c.take<T>(m.group * m.V);              // dz = softmax - onehot of the row group
  p[11] = c.take<float>((size_t)m.splits * m.N * m.d);   // dx_hat split partials
  p[12] = c.take<float>((size_t)dg_row_blocks((int)m.N) * m.d);  // dg partials
  p[13] = c.take<LogitT<T>>(m.slab * m.V);       // logits of the slab (LogitT)
  p[14] = c.take<float>(sizeof(T) == 2 ? tail_ws_bytes<Big>() / 4 : 0);  // partial tiles of split tail GEMM tiles
  // top-1 accuracy: row maxima of the slab, argmax per row, hits per depth
  const bool acc = a->pred || a->correct || a->accuracy;
  p[15] = c.take<float>(acc ? m.slab : 0);
  p[16] = c.take<int32_t>(acc ? m.N : 0);
  p[17] = c.take<int32_t>(acc ? a->D : 0);
  p[18] = c.take<T>(sizeof(T) == 2 ? (size_t)m.d * m.ldT : 0);   // x_hat^T (bf16 runs)
  return c.off;
}

template <typename T>
int ce_run(const mtp_ce_args *a, hipStream_t s) {
  void *p[kCeParts];
  Carve c(a->workspace);
  ce_layout<T>(a, c, p);
  const CeDims m = ce_dims<T>(a);
  const int N = (int)m.N, d = m.d, V = m.V, D = a->D;
  T *xhat = (T *)p[0];
  float *r = (float *)p[1];
  int32_t *lab = (int32_t *)p[2];
  float2 *part = (float2 *)p[3];
  float *target = (float *)p[4], *lse = (float *)p[5], *row_loss = (float *)p[6];
  double *acc_sum = (double *)p[7];
  int32_t *acc_cnt = (int32_t *)p[8];
  float *scale = (float *)p[9];
  T *dz = (T *)p[10];
  float *dxs = (float *)p[11];
  float *dg_part = (float *)p[12];
  LogitT<T> *zbuf = (LogitT<T> *)p[13];
  T *xhatT = (T *)p[18];
  float *skws = sizeof(T) == 2 ? (float *)p[14] : nullptr;
  const bool want_acc = a->pred || a->correct || a->accuracy;
  float *rowmax = want_acc ? (float *)p[15] : nullptr;
  int32_t *pred = want_acc ? (int32_t *)p[16] : nullptr;
  int32_t *acc_correct = want_acc ? (int32_t *)p[17] : nullptr;
  const bool valid_mean = a->reduce == MTP_REDUCE_VALID_MEAN;
  const double denom = valid_mean ? 0.0 : (a->denom > 0.0 ? a->denom : (double)N);
  const long sstride = m.N * m.d;                // stride of the dx_hat split partials
  if (a->device_error) MTP_TRY(fill_i32(a->device_error, 1, 0, s));
  const bool big_dw = sizeof(T) == 2 && use_big(V, d);

  for (int k = 0; k < D; ++k) {
    const T *h = static_cast<const T *>(a->h[k]);
    const int dw_acc0 = (k > 0 || a->accumulate) ? 1 : 0;
    int st = 0;
    {
      MTP_STAGE(MTP_STAGE_OUT_NORM);
      MTP_TRY(launch_out_norm<T>(h, a->g_out, xhat, r, a->labels + (long)k * N, lab, a->device_error, N, d, V,
                                 a->eps, s));
      if constexpr (sizeof(T) == 2)
        if (m.big) MTP_TRY(launch_transpose_bf16(reinterpret_cast<const bf16_t *>(xhat), N, d, xhatT, m.ldT, s));
    }
    {
      // the backward scale depends on the labels only: known before any slab
      MTP_STAGE(MTP_STAGE_CE_REDUCE);
      MTP_TRY(launch_ce_reduce(nullptr, lab, N, k, D, valid_mean, denom, a->lambda, acc_sum, acc_cnt, scale,
                               nullptr, nullptr, nullptr, s));
    }
    for (long g0 = 0; g0 < m.N; g0 += m.group) {
      const int gn = (int)(m.N - g0 < m.group ? m.N - g0 : m.group);
      for (long r0 = g0; r0 < g0 + gn; r0 += m.slab) {
        const int nr = (int)(g0 + gn - r0 < m.slab ? g0 + gn - r0 : m.slab);
        const int32_t *ls = lab + r0;
        {
          MTP_STAGE(MTP_STAGE_CE_FWD);
          if constexpr (sizeof(T) == 2) {
            // the transposed tile on 256 x 256 tiles; small problems keep the row tile
            if (m.big)
              st = gemm_ce_fwd_t_cfg<T, Big>(xhatT + r0, m.ldT, (const T *)a->W_out, ls, part, target + r0, zbuf,
                                             nr, V, d, skws, s);
            else
              st = gemm_ce_fwd_cfg<T, Small>(xhat + r0 * d, (const T *)a->W_out, ls, part, target + r0, zbuf, nr,
                                             V, d, skws, s);
          } else {
            st = gemm_ce_fwd_cfg<T, Small>(xhat + r0 * d, (const T *)a->W_out, ls, part, target + r0, zbuf, nr, V,
                                           d, skws, s);
          }
        }
        if (st) return st;
        {
          MTP_STAGE(MTP_STAGE_CE_REDUCE);
          MTP_TRY(launch_ce_combine(part, m.nt, target + r0, ls, lse + r0,
                                    a->lse ? a->lse + (long)k * N + r0 : nullptr, row_loss + r0, rowmax,
                                    want_acc ? pred + r0 : nullptr, V, nr, s));
        }
        {
          MTP_STAGE(MTP_STAGE_CE_GRAD);
          MTP_TRY((launch_ce_dz<T, LogitT<T>>(zbuf, part, m.nt, m.big ? Big::BM : Small::BM, lse + r0, ls,
                                              dz + (r0 - g0) * V, rowmax, want_acc ? pred + r0 : nullptr, nr,
                                              V, s)));
        }
      }
      {
        MTP_STAGE(MTP_STAGE_CE_DX);
        st = pick<T>(m.big_dx, [&](auto cfg) {
          return gemm_dx_cfg<T, decltype(cfg)>(dz, (const T *)a->W_out, dxs + g0 * d, sstride, gn, V, d, scale + k,
                                               m.splits, skws, s);
        });
      }
      if (st) return st;
      {
        MTP_STAGE(MTP_STAGE_CE_DW);
        st = pick<T>(big_dw, [&](auto cfg) {
          return gemm_dw_cfg<T, decltype(cfg)>(dz, xhat + g0 * d, a->dW_out, gn, V, d, scale + k,
                                               dw_acc0 || g0 > 0, skws, s);
        });
      }
      if (st) return st;
    }
    {
      MTP_STAGE(MTP_STAGE_CE_REDUCE);
      MTP_TRY(launch_ce_reduce(row_loss, lab, N, k, D, valid_mean, denom, a->lambda, acc_sum, acc_cnt, scale,
                               pred, a->pred ? a->pred + (long)k * N : nullptr, acc_correct, s));
    }
    {
      MTP_STAGE(MTP_STAGE_CE_NORM_BWD);
      MTP_TRY(launch_out_norm_bwd<T>(dxs, m.splits, sstride, h, r, a->g_out, static_cast<float *>(a->dh[k]),
                                     dg_part, a->dg_out, dw_acc0, N, d, a->dh_accumulate ? 1 : 0, s));
    }
  }
  MTP_TRY(launch_ce_finalize(acc_sum, acc_cnt, D, valid_mean, denom, a->lambda, a->loss_sum, a->counts, a->loss,
                             a->loss_mtp, acc_correct, a->correct, a->accuracy, s));
  return MTP_OK;
}

int check_verify(const mtp_verify_args *a) {
  if (a == nullptr) return MTP_ERR_NULL;
  if (a->logits_dtype != MTP_F32 && a->logits_dtype != MTP_BF16) return MTP_ERR_DTYPE;
  if (a->R < 1 || a->gamma < 1 || a->V < 1) return MTP_ERR_SHAPE;
  if ((long)a->R * (2 * a->gamma + 1) > (1L << 31) - 1) return MTP_ERR_SHAPE;
  if (a->R > 65535) return MTP_ERR_UNSUPPORTED;   // requests are a grid dimension of the mass pass
  if (!(a->temperature > 0.f) || !isfinite(a->temperature)) return MTP_ERR_ARG;
  return MTP_OK;
}

size_t verify_bytes(const mtp_verify_args *a) {
  return verify_workspace_bytes(a->R, a->gamma, a->V, a->logits_dtype == MTP_BF16 ? 1 : 0);
}

int check_propose(const mtp_propose_args *a) {
  if (a == nullptr) return MTP_ERR_NULL;
  if (a->dtype != MTP_F32 && a->dtype != MTP_BF16) return MTP_ERR_DTYPE;
  if (a->R < 1 || a->L_max < 1 || a->d < 1 || a->n_heads < 1 || a->head_dim < 2 || a->ffn < 1 || a->V < 1)
    return MTP_ERR_SHAPE;
  const int E = a->dtype == MTP_BF16 ? 8 : 4;
  const long A = (long)a->n_heads * a->head_dim;
  if (a->head_dim % 2 || a->d % E || a->ffn % E || A % E || a->V % E) return MTP_ERR_SHAPE;
  if (a->L_max > (1 << 20) || a->V >= (1 << 21) || (long)a->V * a->d > (1L << 40)) return MTP_ERR_SHAPE;
  if (a->R > 65535) return MTP_ERR_UNSUPPORTED;   // requests are a grid dimension of the draw's mass pass
  if (a->dtype == MTP_BF16 && a->head_dim != 32 && a->head_dim != 64 && a->head_dim != 128)
    return MTP_ERR_UNSUPPORTED;
  if (a->dtype == MTP_F32 && a->head_dim != 16 && a->head_dim != 32 && a->head_dim != 64)
    return MTP_ERR_UNSUPPORTED;
  if (!(a->eps >= 0.f) || !(a->rope_theta >= 0.f) || !(a->temperature > 0.f) || !isfinite(a->temperature))
    return MTP_ERR_ARG;
  return MTP_OK;
}

int check_propose_ptrs(const mtp_propose_args *a) {
  if (!a->w || !a->embed || !a->W_out || !a->g_out || !a->h_prev || !a->tokens || !a->positions ||
      !a->u_sample || !a->kv_cache || !a->h_out || !a->logits || !a->draft_token || !a->status)
    return MTP_ERR_NULL;
  const mtp_depth_weights &w = a->w[0];
  if (!w.g_h || !w.g_e || !w.g_attn || !w.g_ffn || !w.M || !w.Wqkv || !w.Wo || !w.Wgate || !w.Wup || !w.Wdown)
    return MTP_ERR_NULL;
  if (!all_al16(a->embed, a->W_out, a->g_out, a->h_prev, a->tokens, a->positions, a->u_sample, a->kv_cache,
                a->h_out, a->logits, a->draft_token, a->status, a->margin, a->workspace) ||
      !all_al16(w.g_h, w.g_e, w.g_attn, w.g_ffn, w.M, w.Wqkv, w.Wo, w.Wgate, w.Wup, w.Wdown))
    return MTP_ERR_ARG;
  return MTP_OK;
}

// K splits of a GEMM with few rows (the proposer's R requests) and N = d:
// enough blocks to stream the weights with most compute units, at least 8 K
// slices of 32 per split.
constexpr int kMaxSplits = 16;
template <class Cfg>
inline int few_row_splits(int M, int N, int K) {
  const long tiles = (long)ceil_div(M, Cfg::BM) * ceil_div(N, Cfg::BN);
  long sp = 512 / (tiles > 0 ? tiles : 1);
  const long by_k = K / (32 * 8);
  sp = sp < by_k ? sp : by_k;
  sp = sp < kMaxSplits ? sp : kMaxSplits;
  return sp < 1 ? 1 : (int)sp;
}

// C = A B^T (+ res) for few rows: K-split partial products into part, then
// summed with the residual into out.
template <typename T, typename TO>
int gemm_few_rows(const T *A, long lda, const T *Bm, long ldb, float *part, TO *out, const float *res, int M, int N,
                  int K, hipStream_t s) {
  // (the 128x128 tile: with K splits it fills the chip; the 64-row tile
  // measured slower here)
  const int sp = few_row_splits<Small>(M, N, K);
  EpiStore<float, float> epi{part, (long)N, M, N, 1.f, nullptr, nullptr, 0, 0, (long)M * N};
  PA<T, Small> la{A, lda, M, K};
  KB<T, Small> lb{Bm, ldb, N, K};
  MTP_TRY((launch_gemm<T, Small>(la, lb, epi, M, N, K, 8, sp, s)));
  MTP_TRY(launch_splitk_sum<TO>(part, sp, (long)M * N, res, out, s));
  return MTP_OK;
}

constexpr int kProposeParts = 19;  // workspace regions of the proposer step

template <typename T>
size_t propose_layout(const mtp_propose_args *a, Carve &c, void **p) {
  const long R = a->R;
  const int d = a->d, f = a->ffn, half = a->head_dim / 2;
  const long A = (long)a->n_heads * a->head_dim;
  for (int i = 0; i < 6; ++i) p[i] = c.take<int32_t>(R);  // tokens, positions, status (checked), iota, A, status (draw)
  p[6] = c.take<float2>(R * half);                          // rotary rows
  p[7] = c.take<T>(R * 2 * d);                              // c
  p[8] = c.take<float>(R * d);                              // u (f32)
  p[9] = c.take<T>(R * d);                                  // x_a
  p[10] = c.take<T>(R * 3 * A);                             // qkv
  p[11] = c.take<T>(R * A);                                 // o
  p[12] = c.take<float>(R * d);                             // a (f32)
  p[13] = c.take<T>(R * d);                                 // y
  p[14] = c.take<T>(R * f);                                 // silu(gate) * up
  p[15] = c.take<T>(R * d);                                 // x_hat
  p[16] = c.take<float>(sizeof(T) == 2 ? tail_ws_bytes<Big>() / 4 : 0);  // partial tiles of split tail GEMM tiles
  p[17] = c.take<double>(verify_workspace_bytes(a->R, 0, a->V, sizeof(T) == 2 ? 1 : 0) / sizeof(double) + 1);
  p[18] = c.take<float>((size_t)kMaxSplits * R * d);      // K-split partial products (N = d GEMMs)
  return c.off;
}

template <typename T>
int propose_run(const mtp_propose_args *a, hipStream_t s) {
  void *p[kProposeParts];
  Carve c(a->workspace);
  propose_layout<T>(a, c, p);
  const int R = a->R, d = a->d, H = a->n_heads, hd = a->head_dim, f = a->ffn, V = a->V;
  const int A = H * hd;
  int32_t *tok_s = (int32_t *)p[0], *pos_s = (int32_t *)p[1], *st_prep = (int32_t *)p[2];
  int32_t *iota = (int32_t *)p[3], *vA = (int32_t *)p[4], *st_draw = (int32_t *)p[5];
  float2 *rope = (float2 *)p[6];
  T *cbuf = (T *)p[7], *xa = (T *)p[9], *qkv = (T *)p[10], *o = (T *)p[11], *ybuf = (T *)p[13];
  T *gsw = (T *)p[14], *xhat = (T *)p[15];
  float *u = (float *)p[8], *abuf = (float *)p[12];
  float *skws = sizeof(T) == 2 ? (float *)p[16] : nullptr;
  double *vws = (double *)p[17];
  const mtp_depth_weights &w = a->w[0];
  const T *E = static_cast<const T *>(a->embed);
  T *h_out = static_cast<T *>(a->h_out);
  T *logits = static_cast<T *>(a->logits);
  const bool use_rope = a->rope_theta > 0.f;

  MTP_TRY(launch_propose_prepare(a->tokens, a->positions, R, V, a->L_max, tok_s, pos_s, st_prep, iota, s));
  if (use_rope) MTP_TRY(rope_rows(rope, pos_s, R, hd / 2, a->rope_theta, s));
  // one row per request: B = R rows of length 1, the token of the row itself
  MTP_TRY(launch_dual_norm_concat<T>(static_cast<const T *>(a->h_prev), E, tok_s, w.g_h, w.g_e, cbuf, R, 1, d, V,
                                     0, a->eps, s));
  float *part = (float *)p[18];
  int st = gemm_few_rows<T, float>(cbuf, 2L * d, (const T *)w.M, 2L * d, part, u, nullptr, R, d, 2 * d, s);
  if (st) return st;
  MTP_TRY((launch_rmsnorm<float, T>(u, w.g_attn, xa, nullptr, R, d, a->eps, s)));
  st = gemm_qkv_rope<T>(xa, (const T *)w.Wqkv, qkv, iota, use_rope ? rope : nullptr, R, d, A, hd, skws, s);
  if (st) return st;
  MTP_TRY(launch_decode_attention<T>(qkv, static_cast<T *>(a->kv_cache), o, pos_s, st_prep, R, H, hd, a->L_max, s));
  st = gemm_few_rows<T, float>(o, A, (const T *)w.Wo, A, part, abuf, u, R, d, A, s);
  if (st) return st;
  MTP_TRY((launch_rmsnorm<float, T>(abuf, w.g_ffn, ybuf, nullptr, R, d, a->eps, s)));
  st = gemm_swiglu<T>(ybuf, (const T *)w.Wgate, (const T *)w.Wup, gsw, R, d, f, skws, s);
  if (st) return st;
  st = gemm_few_rows<T, T>(gsw, f, (const T *)w.Wdown, f, part, h_out, abuf, R, d, f, s);
  if (st) return st;
  MTP_TRY((launch_rmsnorm<T, T>(h_out, a->g_out, xhat, nullptr, R, d, a->eps, s)));
  st = gemm_nt_store<T, T, float>(xhat, d, (const T *)a->W_out, d, logits, V, nullptr, 0, R, V, d, 1.f, nullptr, 0,
                                  skws, s);
  if (st) return st;
  // the draw: verify's emission pass with no drafts (A = 0: p_0 from the stored logits)
  MTP_TRY(launch_verify(logits, nullptr, sizeof(T) == 2 ? 1 : 0, nullptr, nullptr, a->u_sample, R, 0, V,
                        a->temperature, vA, a->draft_token, st_draw, a->margin, vws, s));
  MTP_TRY(launch_propose_finish(st_prep, st_draw, R, a->draft_token, a->status, s));
  return MTP_OK;
}

}  // namespace

extern "C" {

int mtp_abi_version(void) { return MTP_ABI_VERSION; }

int mtp_profile_stage(int stage, void *const *start_events, void *const *stop_events, int n) {
  if (stage < 0) {
    g_prof = Profile();
    return MTP_OK;
  }
  if (stage >= MTP_STAGE_COUNT || n < 1) return MTP_ERR_ARG;
  if (!start_events || !stop_events) return MTP_ERR_NULL;
  g_prof.stage = stage;
  g_prof.start = reinterpret_cast<hipEvent_t *>(const_cast<void **>(start_events));
  g_prof.stop = reinterpret_cast<hipEvent_t *>(const_cast<void **>(stop_events));
  g_prof.n = n;
  g_prof.count = 0;
  return MTP_OK;
}

int mtp_profile_all(void *const *start_events, void *const *stop_events, int *stage_ids, int n) {
  if (n < 1) return MTP_ERR_ARG;
  if (!start_events || !stop_events || !stage_ids) return MTP_ERR_NULL;
  g_prof = Profile();
  g_prof.all = true;
  g_prof.ids = stage_ids;
  g_prof.start = reinterpret_cast<hipEvent_t *>(const_cast<void **>(start_events));
  g_prof.stop = reinterpret_cast<hipEvent_t *>(const_cast<void **>(stop_events));
  g_prof.n = n;
  return MTP_OK;
}

int mtp_profile_count(void) { return g_prof.count; }

const char *mtp_strerror(int status) {
  switch (status) {
    case MTP_OK: return "ok";
    case MTP_ERR_NULL: return "a required pointer is NULL";
    case MTP_ERR_SHAPE: return "invalid or unsupported shape";
    case MTP_ERR_DEPTH: return "depth must be positive";
    case MTP_ERR_DTYPE: return "unknown dtype";
    case MTP_ERR_WORKSPACE: return "workspace missing or too small";
    case MTP_ERR_ARG: return "invalid argument";
    case MTP_ERR_HIP: return "HIP launch failed";
    case MTP_ERR_UNSUPPORTED: return "configuration not supported by the kernels";
    case MTP_ERR_TOO_LARGE: return "request needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

size_t mtp_chain_workspace_size(const mtp_chain_args *a) {
  if (check_chain(a) != MTP_OK) return 0;
  Carve c(nullptr);
  void *p[kChainParts];
  return a->dtype == MTP_BF16 ? chain_layout<bf16_t>(a, c, p) : chain_layout<float>(a, c, p);
}

size_t mtp_chain_saved_bytes(const mtp_chain_args *a) {
  if (check_chain(a) != MTP_OK || a->dtype != MTP_BF16) return 0;
  return (size_t)a->D * saved_depth_bytes((long)a->B * a->T, a->d, a->n_heads * a->head_dim, a->n_heads, a->ffn);
}

int mtp_chain_forward(const mtp_chain_args *a, void *stream) {
  int st = check_chain(a);
  if (st) return st;
  if ((st = check_chain_ptrs(a))) return st;
  if (!a->workspace || a->workspace_bytes < mtp_chain_workspace_size(a)) return MTP_ERR_WORKSPACE;
  if (a->saved != nullptr) {
    if (a->dtype != MTP_BF16) return MTP_ERR_UNSUPPORTED;
    if (!al16(a->saved)) return MTP_ERR_ARG;
    if (a->saved_bytes < mtp_chain_saved_bytes(a)) return MTP_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return a->dtype == MTP_BF16 ? chain_run<bf16_t>(a, s) : chain_run<float>(a, s);
}

size_t mtp_chain_backward_workspace_size(const mtp_chain_bwd_args *a) {
  if (check_chain_bwd(a) != MTP_OK) return 0;
  Carve c(nullptr);
  void *p[kBwdParts];
  return chain_bwd_layout(a, c, p);
}

int mtp_chain_backward(const mtp_chain_bwd_args *a, void *stream) {
  int st = check_chain_bwd(a);
  if (st) return st;
  if ((st = check_chain_bwd_ptrs(a))) return st;
  if (!a->workspace || a->workspace_bytes < mtp_chain_backward_workspace_size(a)) return MTP_ERR_WORKSPACE;
  if (a->saved != nullptr) {
    if (!al16(a->saved)) return MTP_ERR_ARG;
    if (a->saved_bytes < (size_t)a->D * saved_depth_bytes((long)a->B * a->T, a->d, a->n_heads * a->head_dim,
                                                           a->n_heads, a->ffn))
      return MTP_ERR_WORKSPACE;
  }
  return chain_bwd_run(a, static_cast<hipStream_t>(stream));
}

size_t mtp_horizon_heads_workspace_size(const mtp_horizon_args *a) {
  if (check_horizon(a) != MTP_OK) return 0;
  Carve c(nullptr);
  void *p[kHorParts];
  return horizon_layout(a, c, p);
}

int mtp_horizon_heads(const mtp_horizon_args *a, void *stream) {
  int st = check_horizon(a);
  if (st) return st;
  if (!a->tokens || !a->segment_ids || !a->h || !a->w || !a->W_out || !a->g_out || !a->loss || !a->counts ||
      !a->loss_total || !a->dh || !a->dW_out || !a->dg_out || !a->dw)
    return MTP_ERR_NULL;
  for (int k = 0; k < a->K; ++k) {
    const mtp_block_weights &w = a->w[k];
    const mtp_block_grads &g = a->dw[k];
    if (!w.g_attn || !w.g_ffn || !w.Wqkv || !w.Wo || !w.Wgate || !w.Wup || !w.Wdown || !g.g_attn || !g.g_ffn ||
        !g.Wqkv || !g.Wo || !g.Wgate || !g.Wup || !g.Wdown)
      return MTP_ERR_NULL;
    if (!all_al16(w.g_attn, w.g_ffn, w.Wqkv, w.Wo, w.Wgate, w.Wup, w.Wdown) ||
        !all_al16(g.g_attn, g.g_ffn, g.Wqkv, g.Wo, g.Wgate, g.Wup, g.Wdown))
      return MTP_ERR_ARG;
  }
  if (!all_al16(a->tokens, a->segment_ids, a->h, a->W_out, a->g_out, a->dh, a->dW_out, a->dg_out, a->device_error,
                a->workspace))
    return MTP_ERR_ARG;
  if (!a->workspace || a->workspace_bytes < mtp_horizon_heads_workspace_size(a)) return MTP_ERR_WORKSPACE;
  return horizon_run(a, static_cast<hipStream_t>(stream));
}

size_t mtp_ce_workspace_size(const mtp_ce_args *a) {
  if (check_ce(a) != MTP_OK) return 0;
  Carve c(nullptr);
  void *p[kCeParts];
  return a->dtype == MTP_BF16 ? ce_layout<bf16_t>(a, c, p) : ce_layout<float>(a, c, p);
}

int mtp_head_ce_fwd_bwd(const mtp_ce_args *a, void *stream) {
  int st = check_ce(a);
  if (st) return st;
  if ((st = check_ce_ptrs(a))) return st;
  if (!a->workspace || a->workspace_bytes < mtp_ce_workspace_size(a)) return MTP_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return a->dtype == MTP_BF16 ? ce_run<bf16_t>(a, s) : ce_run<float>(a, s);
}

size_t mtp_verify_workspace_size(const mtp_verify_args *a) {
  if (check_verify(a) != MTP_OK) return 0;
  return verify_bytes(a);
}

namespace {
int check_verify_ptrs(const mtp_verify_args *a, const void *ws) {
  if (!a->target_logits || !a->draft_logits || !a->draft_tokens || !a->u_accept || !a->u_sample ||
      !a->accepted_len || !a->next_token || !a->status)
    return MTP_ERR_NULL;
  if (!all_al16(a->target_logits, a->draft_logits, a->draft_tokens, a->u_accept, a->u_sample, a->accepted_len,
                a->next_token, a->status, a->margin, ws))
    return MTP_ERR_ARG;
  return MTP_OK;
}

int verify_run(const mtp_verify_args *a, double *ws, hipStream_t s) {
  MTP_STAGE(MTP_STAGE_VERIFY);
  MTP_TRY(launch_verify(a->target_logits, a->draft_logits, a->logits_dtype == MTP_BF16 ? 1 : 0, a->draft_tokens,
                        a->u_accept, a->u_sample, a->R, a->gamma, a->V, a->temperature, a->accepted_len,
                        a->next_token, a->status, a->margin, ws, s));
  return MTP_OK;
}
}  // namespace

int mtp_verify(const mtp_verify_args *a, void *stream) {
  int st = check_verify(a);
  if (st) return st;
  if ((st = check_verify_ptrs(a, a->workspace))) return st;
  if (!a->workspace || a->workspace_bytes < verify_bytes(a)) return MTP_ERR_WORKSPACE;
  return verify_run(a, static_cast<double *>(a->workspace), static_cast<hipStream_t>(stream));
}

int mtp_verify_noalloc(const mtp_verify_args *a, void *stream) {
  int st = check_verify(a);
  if (st) return st;
  if ((st = check_verify_ptrs(a, nullptr))) return st;
  if (verify_bytes(a) > (size_t)MTP_NOALLOC_SCRATCH_BYTES) return MTP_ERR_TOO_LARGE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void *ws = nullptr;
  if ((st = scratch_address(s, &ws))) return st;
  // every workspace entry the verify kernels read is written earlier in the
  // same call: nothing needs clearing between calls
  return verify_run(a, static_cast<double *>(ws), s);
}

int mtp_round_commit(const mtp_round_args *a, void *stream) {
  if (a == nullptr) return MTP_ERR_NULL;
  if (a->R < 1 || a->gamma < 1 || (long)a->R * (a->gamma + 1) > (1L << 31) - 1) return MTP_ERR_SHAPE;
  if (!a->draft_tokens || !a->accepted_len || !a->next_token || !a->status || !a->remaining || !a->new_tokens ||
      !a->n_new || !a->rows_to_keep || !a->pending_frontier || !a->stopped)
    return MTP_ERR_NULL;
  if (!all_al16(a->draft_tokens, a->accepted_len, a->next_token, a->status, a->remaining, a->new_tokens, a->n_new,
                a->rows_to_keep, a->pending_frontier, a->stopped))
    return MTP_ERR_ARG;
  MTP_TRY(launch_round_commit(a->R, a->gamma, a->eos, a->draft_tokens, a->accepted_len, a->next_token, a->status,
                              a->remaining, a->new_tokens, a->n_new, a->rows_to_keep, a->pending_frontier,
                              a->stopped, static_cast<hipStream_t>(stream)));
  return MTP_OK;
}

size_t mtp_propose_workspace_size(const mtp_propose_args *a) {
  if (check_propose(a) != MTP_OK) return 0;
  Carve c(nullptr);
  void *p[kProposeParts];
  return a->dtype == MTP_BF16 ? propose_layout<bf16_t>(a, c, p) : propose_layout<float>(a, c, p);
}

int mtp_propose_step(const mtp_propose_args *a, void *stream) {
  int st = check_propose(a);
  if (st) return st;
  if ((st = check_propose_ptrs(a))) return st;
  if (!a->workspace || a->workspace_bytes < mtp_propose_workspace_size(a)) return MTP_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return a->dtype == MTP_BF16 ? propose_run<bf16_t>(a, s) : propose_run<float>(a, s);
}

}  // extern "C"
