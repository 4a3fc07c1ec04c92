// Runs, state/loss masks, labels and counts of every depth
// (M7.6 0x02 depth contract, 0x04 alignment, 0x04C row compiler restated on
// the dense [B, T] layout).
//
// A run is a maximal stretch of one non-negative segment id in a batch row.
// For i in run [r0, r1]: state(k, i) = i + k <= r1, loss(k, i) = i + k + 1 <= r1,
// label(k, i) = tokens[i + k + 1] when loss, else -1.  Padding rows (id < 0)
// are their own one-row window (r0 = r1 = i) and are never state rows.
#include "kernels.hpp"

namespace mtp {

namespace {
constexpr int kRowThreads = 1024;

// Inclusive scan of one int per thread over the block: prefix max
// (REVERSE = false, over threads <= t) or suffix min (REVERSE = true, over
// threads >= t).  Leaves the scanned values in sh.
template <bool REVERSE>
__device__ int block_scan(int v, int *sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int off = 1; off < kRowThreads; off <<= 1) {
    int o;
    if (REVERSE) o = (t + off < kRowThreads) ? sh[t + off] : INT_MAX;
    else o = (t >= off) ? sh[t - off] : INT_MIN;
    __syncthreads();
    v = REVERSE ? min(v, o) : max(v, o);
    sh[t] = v;
    __syncthreads();
  }
  return v;
}

__device__ __forceinline__ bool run_starts_at(const int32_t *sg, int i) {
  return sg[i] >= 0 && (i == 0 || sg[i - 1] != sg[i]);
}
__device__ __forceinline__ bool run_ends_at(const int32_t *sg, int i, int T) {
  return sg[i] >= 0 && (i == T - 1 || sg[i + 1] != sg[i]);
}
}  // namespace

// One block per batch row; thread t owns a contiguous chunk of positions.
// Writes run_start / pos (= i - run_start) to the workspace, masks and labels
// for all depths, and per-row partial counts and error flags.
__global__ __launch_bounds__(kRowThreads) void rows_kernel(
    const int32_t *__restrict__ tokens, const int32_t *__restrict__ seg, int B, int T, int V, int D,
    int32_t *__restrict__ run_start, int32_t *__restrict__ pos, uint8_t *__restrict__ state_mask,
    uint8_t *__restrict__ loss_mask, int32_t *__restrict__ labels, int32_t *__restrict__ cnt_part,
    int32_t *__restrict__ err_part) {
  __shared__ int sh[kRowThreads];
  __shared__ int red[kRowThreads / 64];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int chunk = (T + kRowThreads - 1) / kRowThreads;
  const int lo = min(T, t * chunk), hi = min(T, lo + chunk);
  const int32_t *sg = seg + (long)b * T;
  const int32_t *tk = tokens + (long)b * T;
  int32_t *rs_out = run_start + (long)b * T;

  // last run start before the chunk / first run end after it
  int last = INT_MIN, first = INT_MAX;
  for (int i = lo; i < hi; ++i) {
    if (run_starts_at(sg, i)) last = i;
    if (first == INT_MAX && run_ends_at(sg, i, T)) first = i;
  }
  block_scan<false>(last, sh);
  const int before = (t > 0) ? sh[t - 1] : INT_MIN;
  __syncthreads();
  block_scan<true>(first, sh);
  const int after = (t + 1 < kRowThreads) ? sh[t + 1] : INT_MAX;
  __syncthreads();

  // forward pass: run starts
  int cur = before;
  for (int i = lo; i < hi; ++i) {
    if (run_starts_at(sg, i)) cur = i;
    const int rs = sg[i] >= 0 ? cur : i;
    rs_out[i] = rs;
    pos[(long)b * T + i] = i - rs;
  }
  // backward pass: run ends, masks, labels, counts
  int err = 0;
  int cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int cur_end = after;
  for (int i = hi - 1; i >= lo; --i) {
    if (run_ends_at(sg, i, T)) cur_end = i;
    const bool active = sg[i] >= 0;
    const int r1 = active ? cur_end : i;
    const int tok = tk[i];
    if (active && (tok < 0 || tok >= V)) err = 1;
    for (int k = 1; k <= D; ++k) {
      const long o = ((long)(k - 1) * B + b) * T + i;
      const bool st = active && i + k <= r1;
      const bool ls = active && i + k + 1 <= r1;
      state_mask[o] = st ? 1 : 0;
      loss_mask[o] = ls ? 1 : 0;
      int lab = -1;
      if (ls) {
        lab = tk[i + k + 1];
        lab = lab < 0 ? 0 : (lab >= V ? V - 1 : lab);   // out of range: flagged above
      }
      labels[o] = lab;
      if (ls) {
        if (k <= 8) cnt[k - 1]++;
        else atomicAdd(&cnt_part[(long)(k - 1) * B + b], 1);
      }
    }
  }
  // block reductions of the counts (first 8 depths) and of the error flag
  const int lane = t & 63, wv = t >> 6;
  for (int k = 1; k <= min(D, 8); ++k) {
    int v = cnt[k - 1];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[wv] = v;
    __syncthreads();
    if (t == 0) {
      int s = 0;
      for (int w = 0; w < kRowThreads / 64; ++w) s += red[w];
      cnt_part[(long)(k - 1) * B + b] += s;
    }
    __syncthreads();
  }
  int v = err;
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o);
  if (lane == 0) red[wv] = v;
  __syncthreads();
  if (t == 0) {
    int s = 0;
    for (int w = 0; w < kRowThreads / 64; ++w) s |= red[w];
    err_part[b] = s;
  }
}

__global__ void rows_zero_kernel(int32_t *cnt_part, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) cnt_part[i] = 0;
}

// Sums the per-row partials in a fixed order.
__global__ void rows_finalize_kernel(const int32_t *cnt_part, const int32_t *err_part, int B, int D,
                                     int32_t *counts, int32_t *device_error) {
  const int t = threadIdx.x;
  for (int k = t; k < D; k += blockDim.x) {
    int s = 0;
    for (int b = 0; b < B; ++b) s += cnt_part[(long)k * B + b];
    counts[k] = s;
  }
  if (t == 0) {
    int e = 0;
    for (int b = 0; b < B; ++b) e |= err_part[b];
    device_error[0] = e;
  }
}

hipError_t launch_rows(const int32_t *tokens, const int32_t *seg, int B, int T, int V, int D,
                       int32_t *run_start, int32_t *pos, uint8_t *state_mask, uint8_t *loss_mask,
                       int32_t *labels, int32_t *counts, int32_t *device_error, int32_t *cnt_part,
                       int32_t *err_part, hipStream_t s) {
  const int n = D * B;
  hipLaunchKernelGGL(rows_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, cnt_part, n);
  hipLaunchKernelGGL(rows_kernel, dim3(B), dim3(kRowThreads), 0, s, tokens, seg, B, T, V, D, run_start,
                     pos, state_mask, loss_mask, labels, cnt_part, err_part);
  hipLaunchKernelGGL(rows_finalize_kernel, dim3(1), dim3(64), 0, s, cnt_part, err_part, B, D, counts,
                     device_error);
  return hipGetLastError();
}

}  // namespace mtp
