// Internal launch interface of the kernels (host side).  Not part of the
// public ABI; mtp_api.hip is the only caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mtp {

// rows / masks / labels / counts
hipError_t launch_rows(const int32_t *tokens, const int32_t *seg, int B, int T, int V, int D,
                       int32_t *run_start, int32_t *pos, uint8_t *state_mask, uint8_t *loss_mask,
                       int32_t *labels, int32_t *counts, int32_t *device_error, int32_t *cnt_part,
                       int32_t *err_part, hipStream_t s);

// norms
template <typename T>
hipError_t launch_dual_norm_concat(const T *h, const T *E, const int32_t *tokens, const float *g_h,
                                   const float *g_e, T *c, int B, int T_len, int d, int V, int depth,
                                   float eps, hipStream_t s);
template <typename TI, typename TO>
hipError_t launch_rmsnorm(const TI *z, const float *g, TO *out, float *r, long rows, int d, float eps,
                          hipStream_t s);
template <typename T>
hipError_t launch_out_norm(const T *h, const float *g, T *xhat, float *r, const int32_t *labels_in,
                           int32_t *labels_out, int32_t *err, long rows, int d, int V, float eps,
                           hipStream_t s);
template <typename T>
hipError_t launch_out_norm_bwd(const float *dx, int splits, long slab, const T *h, const float *r,
                               const float *g, float *dh, float *dg_part, float *dg, int accumulate,
                               int N, int d, int dh_acc, hipStream_t s);
// Row blocks of the output-norm backward (8 rows each); one dg partial row per block.
inline int dg_row_blocks(int N) { int b = (N + 7) / 8; return b < 1 ? 1 : b; }
// dg[j] (+)= sum over the nrb partial rows, in a fixed order
hipError_t launch_dg_reduce(const float *part, int nrb, int d, float *dg, int accumulate, hipStream_t s);

// reverse pass of the chain (bf16 runs)
// RMSNorm backward over rows (z row zrow[n] when zrow is set; d <= 8192):
// dz = resid + (rowmask ? backward : 0), optional bf16 copy; gain gradient
// into dg via part (dg_row_blocks(N) x d floats)
template <typename TZ>
hipError_t launch_rms_bwd(const float *dy, long ldy, const TZ *z, const int32_t *zrow, const float *g, float eps,
                          const float *resid, const uint8_t *rowmask, float *dz, bf16_t *dzb, float *part,
                          float *dg, int accumulate, int N, int d, hipStream_t s);
// shifted tokens of depth k (tok), sort keys (token on state rows, V
// elsewhere) and row indices
hipError_t launch_shifted_rows(const int32_t *tokens, const uint8_t *state, int B, int T_len, int V, int depth,
                               int32_t *tok, int32_t *key, int32_t *val, hipStream_t s);
// reverse of SwiGLU from saved pre-activations pre [N, 2f] f32 (gate | up):
// gsw = silu(gate) up [N, f] and dgu = [d gate | d up] [N, 2f] (bf16), from
// dgsw [N, f] (bf16); f % 4 == 0
hipError_t launch_swiglu_bwd(const float *pre, const bf16_t *dgsw, bf16_t *gsw, bf16_t *dgu, long N, int f,
                             hipStream_t s);
// dE[t] += sum of de rows whose key is t (stable sort by key, then one sum per run)
size_t embed_grad_sort_bytes(int N, int V);
hipError_t launch_embed_grad(const int32_t *key, const int32_t *val, int32_t *key_sorted, int32_t *val_sorted,
                             void *sort_tmp, size_t sort_bytes, int N, int V, const float *de, int d, float *dE,
                             hipStream_t s);
// attention reverse: dqkv [B*T, 3A] (dq, dk after the inverse RoPE; dv) from
// qkv, o, dO [B*T, A] and the per-query pairs lsed [B, H, T] x float2 whose
// first element the forward wrote (lse2); the second receives D = dO . o
hipError_t launch_attention_bwd(const bf16_t *qkv, const bf16_t *o, const bf16_t *dout, float2 *lsed,
                                const int32_t *run_start, const int32_t *pos, const float2 *rope, bf16_t *dqkv,
                                int B, int T_len, int H, int hd, hipStream_t s);

// attention
// lse2 (may be NULL): per (batch row, head, position) pairs of floats,
// [B, H, T, 2]; element 0 of each pair receives the base-2 log-sum-exp of the
// query's scores scaled by log2(e)/sqrt(hd), for the reverse pass (element 1
// is the reverse pass's)
template <typename T>
hipError_t launch_attention(const T *qkv, T *out, const int32_t *run_start, float *lse2, int B, int T_len,
                            int H, int hd, hipStream_t s);
hipError_t rope_table(float2 *table, int max_pos, int half, float theta, hipStream_t s);
template <typename T>
// skip (may be NULL): requests with skip[r] != 0 do not write their cache slot
hipError_t launch_decode_attention(const T *qkv, T *cache, T *out, const int32_t *pos, const int32_t *skip, int R,
                                   int H, int hd, long L_max, hipStream_t s);

// CE reductions
// xT[c, r] = x[r, c] (bf16 [R, C], C % 8 == 0; ldT >= R rounded up to 8, pad written 0)
hipError_t launch_transpose_bf16(const bf16_t *x, int R, int C, bf16_t *xT, long ldT, hipStream_t s);
template <typename T, typename ZT>
hipError_t launch_ce_dz(const ZT *z, const float2 *part, int nt, int tile_cols, const float *lse,
                        const int32_t *labels, T *dz, const float *rowmax, int32_t *pred, int N, int V,
                        hipStream_t s);
template <typename TO>
hipError_t launch_splitk_sum(const float *part, int splits, long n, const float *res, TO *out, hipStream_t s);
hipError_t launch_ce_combine(const float2 *part, int nt, const float *target, const int32_t *labels,
                             float *lse, float *lse_out, float *row_loss, float *rowmax, int32_t *pred, int V,
                             int N, hipStream_t s);
hipError_t launch_ce_reduce(const float *row_loss, const int32_t *labels, int N, int k, int D,
                            int reduce_valid_mean, double denom, float lambda, double *acc_sum,
                            int32_t *acc_cnt, float *scale, const int32_t *pred, int32_t *pred_out,
                            int32_t *acc_correct, hipStream_t s);
hipError_t launch_ce_finalize(const double *acc_sum, const int32_t *acc_cnt, int D,
                              int reduce_valid_mean, double denom, float lambda, float *loss_sum,
                              int32_t *counts, float *loss, float *loss_mtp, const int32_t *acc_correct,
                              int32_t *correct, float *accuracy, hipStream_t s);

// verify
size_t verify_workspace_bytes(int R, int G, int V, int bf16);
hipError_t launch_propose_prepare(const int32_t *tokens, const int32_t *positions, int R, int V, int L_max,
                                  int32_t *tok_s, int32_t *pos_s, int32_t *st, int32_t *iota, hipStream_t s);
hipError_t rope_rows(float2 *table, const int32_t *pos, int R, int half, float theta, hipStream_t s);
hipError_t launch_round_commit(int R, int G, int eos, const int32_t *drafts, const int32_t *A, const int32_t *tok,
                               const int32_t *st, const int32_t *rem, int32_t *out_tok, int32_t *n_new,
                               int32_t *keep, int32_t *pending, int32_t *stopped, hipStream_t s);
hipError_t launch_propose_finish(const int32_t *st_prep, const int32_t *st_draw, int R, int32_t *tok,
                                 int32_t *st_out, hipStream_t s);
hipError_t launch_verify(const void *zt, const void *zd, int bf16, const int32_t *y, const float *ua,
                         const float *us, int R, int G, int V, float tau, int32_t *A, int32_t *tok,
                         int32_t *status, float *margin, double *ws, hipStream_t s);

// small utilities
hipError_t fill_i32(int32_t *p, long n, int32_t v, hipStream_t s);
hipError_t fill_f32(float *p, long n, float v, hipStream_t s);

}  // namespace mtp
