// leank_build_mask: stage-2 channel mask of the LeanK page, section 2.2.
// leank_build_mask_host computes the same mask on the host from host
// memory (the offline conversion of that section, with no device involved).
//
// Kernel 1 (one workgroup) finds the global threshold: the order statistic
// of all alpha values at ascending rank ceil((n-1)*p/100), by a 4-pass
// 8-bit radix select over order-preserving 32-bit keys.  Kernel 2 (one
// workgroup per (layer, head)) counts the head's channels at or above the
// threshold, floors the count to the alignment and keeps the channels of
// rank below that count in the head's (alpha desc, channel asc) order.

#include <math.h>

#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"

namespace leank {
namespace {

// Arguments both forms check before any work.  The kept counts a mask can
// give are multiples of `align`; the cache plan takes multiples of
// LEANK_CHANNEL_QUANTUM, so an align that is not one is refused here rather
// than by the plan one call later.
int check_mask_args(const void* alpha, int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                    int32_t prune_pct, int32_t align, const void* mask_out,
                    const void* kept_count_out, const void* kept_idx_out) {
  if (!alpha || !mask_out || !kept_count_out || !kept_idx_out) return LEANK_EINVAL;
  if (n_layers < 1 || n_kv_heads < 1 || head_dim < 1 || head_dim > 1024) return LEANK_EINVAL;
  if (prune_pct < 0 || prune_pct > 100) return LEANK_EINVAL;
  if (align < 1 || head_dim % align) return LEANK_EINVAL;
  if (align % LEANK_CHANNEL_QUANTUM) return LEANK_EUNSUPPORTED;
  const int64_t heads = static_cast<int64_t>(n_layers) * n_kv_heads;
  if (heads > INT32_MAX || heads * head_dim > INT32_MAX) return LEANK_EINVAL;
  return LEANK_OK;
}

constexpr uint32_t kNanKey = 0xFFFFFFFFu;  // a NaN was seen (no finite/inf key is this large)

// Order-preserving map of a float to an unsigned key; -0.0 and +0.0 share a key.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelectThreads = 1024;

__global__ __launch_bounds__(kSelectThreads) void threshold_select_kernel(
    const float* __restrict__ alpha, int64_t n, int64_t rank, uint32_t* __restrict__ key_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_rank, s_nan;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_prefix = 0;
    s_rank = static_cast<uint32_t>(rank);
    s_nan = 0;
  }
  __syncthreads();
  uint32_t prefix_mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    bool nan_here = false;
    for (int64_t i = tid; i < n; i += kSelectThreads) {
      const float x = alpha[i];
      if (shift == 24 && x != x) nan_here = true;
      const uint32_t k = order_key(x);
      if ((k & prefix_mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    if (nan_here) atomicOr(&s_nan, 1u);
    __syncthreads();
    if (tid == 0) {
      uint32_t r = s_rank, below = 0;
      int bin = 0;
      for (; bin < 255; ++bin) {
        if (below + hist[bin] > r) break;
        below += hist[bin];
      }
      s_rank = r - below;
      s_prefix = prefix | (static_cast<uint32_t>(bin) << shift);
    }
    prefix_mask |= 255u << shift;
    __syncthreads();
  }
  if (tid == 0) *key_out = s_nan ? kNanKey : s_prefix;
}

__global__ void head_mask_kernel(const float* __restrict__ alpha, int head_dim, int align,
                                 uint32_t threshold_key, uint8_t* __restrict__ mask,
                                 int32_t* __restrict__ kept_count, int16_t* __restrict__ kept_idx) {
  extern __shared__ uint32_t keys[];  // [head_dim] keys, then [head_dim] keep flags
  uint32_t* keep_flag = keys + head_dim;
  __shared__ uint32_t s_count;
  const int64_t head = blockIdx.x;
  const float* a = alpha + head * head_dim;
  if (threadIdx.x == 0) s_count = 0;
  for (int c = threadIdx.x; c < head_dim; c += blockDim.x) keys[c] = order_key(a[c]);
  __syncthreads();
  uint32_t mine = 0;
  for (int c = threadIdx.x; c < head_dim; c += blockDim.x) mine += keys[c] >= threshold_key ? 1u : 0u;
  if (mine) atomicAdd(&s_count, mine);
  __syncthreads();
  const int n_keep = static_cast<int>(s_count) / align * align;
  for (int c = threadIdx.x; c < head_dim; c += blockDim.x) {
    const uint32_t kc = keys[c];
    int rank = 0;
    for (int o = 0; o < head_dim; ++o) {
      const uint32_t ko = keys[o];
      rank += (ko > kc || (ko == kc && o < c)) ? 1 : 0;
    }
    const bool keep = rank < n_keep;
    keep_flag[c] = keep ? 1u : 0u;
    mask[head * head_dim + c] = keep ? 1 : 0;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < head_dim; c += blockDim.x) {
    int pos = 0;
    for (int o = 0; o < c; ++o) pos += static_cast<int>(keep_flag[o]);
    if (keep_flag[c]) kept_idx[head * head_dim + pos] = static_cast<int16_t>(c);
    if (c >= n_keep) kept_idx[head * head_dim + c] = -1;
  }
  if (threadIdx.x == 0) kept_count[head] = n_keep;
}

}  // namespace
}  // namespace leank

using namespace leank;

extern "C" int leank_build_mask(const float* alpha, int32_t n_layers, int32_t n_kv_heads,
                                int32_t head_dim, int32_t prune_pct, int32_t align,
                                uint8_t* mask_out, int32_t* kept_count_out,
                                int16_t* kept_idx_out, void* stream) {
  const int st = check_mask_args(alpha, n_layers, n_kv_heads, head_dim, prune_pct, align, mask_out,
                                 kept_count_out, kept_idx_out);
  if (st != LEANK_OK) return st;
  const int64_t heads = static_cast<int64_t>(n_layers) * n_kv_heads;
  const int64_t n = heads * head_dim;
  const int64_t rank = ((n - 1) * prune_pct + 99) / 100;  // ceil((n-1) p / 100)
  hipStream_t s = static_cast<hipStream_t>(stream);

  // kept_count_out[0] briefly carries the threshold key back to the host.
  uint32_t* key_slot = reinterpret_cast<uint32_t*>(kept_count_out);
  hipLaunchKernelGGL(threshold_select_kernel, dim3(1), dim3(kSelectThreads), 0, s, alpha, n, rank,
                     key_slot);
  LEANK_HIP_TRY(hipGetLastError());
  uint32_t key = 0;
  LEANK_HIP_TRY(hipMemcpyAsync(&key, key_slot, sizeof(key), hipMemcpyDeviceToHost, s));
  LEANK_HIP_TRY(hipStreamSynchronize(s));
  if (key == kNanKey) return LEANK_EINVAL;

  const int threads = std::min(1024, (head_dim + 63) / 64 * 64);
  const size_t lds = static_cast<size_t>(head_dim) * 2 * sizeof(uint32_t);
  hipLaunchKernelGGL(head_mask_kernel, dim3(static_cast<unsigned>(heads)), dim3(threads), lds, s,
                     alpha, head_dim, align, key, mask_out, kept_count_out, kept_idx_out);
  LEANK_HIP_TRY(hipGetLastError());
  LEANK_HIP_TRY(hipStreamSynchronize(s));
  return LEANK_OK;
}

extern "C" int leank_build_mask_host(const float* alpha, int32_t n_layers, int32_t n_kv_heads,
                                     int32_t head_dim, int32_t prune_pct, int32_t align,
                                     uint8_t* mask_out, int32_t* kept_count_out,
                                     int16_t* kept_idx_out) {
  const int st = check_mask_args(alpha, n_layers, n_kv_heads, head_dim, prune_pct, align, mask_out,
                                 kept_count_out, kept_idx_out);
  if (st != LEANK_OK) return st;
  const int64_t heads = static_cast<int64_t>(n_layers) * n_kv_heads;
  const int64_t n = heads * head_dim;
  for (int64_t i = 0; i < n; ++i)
    if (isnan(alpha[i])) return LEANK_EINVAL;
  // the global threshold: the value at ascending rank ceil((n - 1) p / 100)
  // (-0.0 and +0.0 compare equal, as in the float order)
  const int64_t rank = ((n - 1) * prune_pct + 99) / 100;
  std::vector<float> sorted(alpha, alpha + n);
  std::nth_element(sorted.begin(), sorted.begin() + rank, sorted.end());
  const float threshold = sorted[static_cast<size_t>(rank)];
  // per head: channels at or above the threshold, floored to the alignment;
  // that many of the head's largest alpha are kept, ties to the lower channel
  std::vector<int> order(static_cast<size_t>(head_dim));
  for (int64_t hd = 0; hd < heads; ++hd) {
    const float* a = alpha + hd * head_dim;
    int passing = 0;
    for (int c = 0; c < head_dim; ++c) passing += a[c] >= threshold ? 1 : 0;
    const int n_keep = passing / align * align;
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [a](int x, int y) { return a[x] > a[y]; });
    std::sort(order.begin(), order.begin() + n_keep);
    uint8_t* m = mask_out + hd * head_dim;
    int16_t* idx = kept_idx_out + hd * head_dim;
    std::fill(m, m + head_dim, uint8_t{0});
    for (int j = 0; j < head_dim; ++j) idx[j] = j < n_keep ? static_cast<int16_t>(order[j]) : int16_t{-1};
    for (int j = 0; j < n_keep; ++j) m[order[j]] = 1;
    kept_count_out[hd] = n_keep;
  }
  return LEANK_OK;
}
