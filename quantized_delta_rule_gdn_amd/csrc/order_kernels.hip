// order_kernels.hip -- gfx950 kernel of damp_batch_order: the batch positions listed by
// ascending slot bucket, so that a step launched with that order streams blocks that lie close
// together in the pool. One workgroup: a counting sort in LDS (histogram of the buckets, an
// exclusive prefix sum, then each position takes the next free place of its bucket). The
// atomics make every place unique, so the result is a permutation of [0, B) for any slot
// indices (repeated or out of range ones included); positions of one bucket come in no fixed
// order, which no step result depends on.
#include "launch.h"

namespace damp {
namespace {

constexpr int kOrderThreads = 1024;
constexpr int kOrderPer = kOrderBuckets / kOrderThreads;   // buckets per thread in the prefix sum

__device__ __forceinline__ int bucket_of(int32_t s, int32_t num_slots, int shift) {
  const int32_t c = s < 0 ? 0 : (s >= num_slots ? num_slots - 1 : s);
  return c >> shift;
}

__global__ __launch_bounds__(kOrderThreads) void batch_order_kernel(const int32_t* __restrict__ slot_idx,
                                                                    int32_t B, int32_t num_slots, int shift,
                                                                    int32_t* __restrict__ order) {
  __shared__ int cnt[kOrderBuckets];
  __shared__ int wave_sum[kOrderThreads / 64];
  const int t = __builtin_amdgcn_workitem_id_x();
  const int lane = t & 63, wv = t >> 6;
  for (int i = t; i < kOrderBuckets; i += kOrderThreads) cnt[i] = 0;
  __syncthreads();
  for (int64_t b = t; b < B; b += kOrderThreads) atomicAdd(&cnt[bucket_of(slot_idx[b], num_slots, shift)], 1);
  __syncthreads();
  // exclusive prefix sum: thread t owns buckets kOrderPer t .. kOrderPer (t + 1) - 1
  int c[kOrderPer], own = 0;
#pragma unroll
  for (int i = 0; i < kOrderPer; ++i) {
    c[i] = cnt[kOrderPer * t + i];
    own += c[i];
  }
  int incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_sum[wv] = incl;
  __syncthreads();
  int base = incl - own;
  for (int i = 0; i < wv; ++i) base += wave_sum[i];
#pragma unroll
  for (int i = 0; i < kOrderPer; ++i) {
    cnt[kOrderPer * t + i] = base;
    base += c[i];
  }
  __syncthreads();
  // (pos < B holds whenever slot_idx is not written meanwhile; the test keeps a racing writer
  // from making this kernel store out of bounds)
  for (int64_t b = t; b < B; b += kOrderThreads) {
    const int pos = atomicAdd(&cnt[bucket_of(slot_idx[b], num_slots, shift)], 1);
    if (pos < B) order[pos] = static_cast<int32_t>(b);
  }
}

}  // namespace

int order_shift(int32_t num_slots) {
  int shift = 0;
  while (((num_slots - 1) >> shift) >= kOrderBuckets) ++shift;
  return shift;
}

hipError_t launch_batch_order(const int32_t* slot_idx, int32_t B, int32_t num_slots, int32_t* order,
                              hipStream_t s) {
  hipLaunchKernelGGL(batch_order_kernel, dim3(1), dim3(kOrderThreads), 0, s, slot_idx, B, num_slots,
                     order_shift(num_slots), order);
  return hipGetLastError();
}

}  // namespace damp
