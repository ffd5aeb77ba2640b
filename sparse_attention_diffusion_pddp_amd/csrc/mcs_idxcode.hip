// Compact form of the cached KV indices for host offload (research
// walkthrough page, method step 5; paper landing page, Table 8, which
// offloads the selected KV indices beside the residuals): one bit per key.
// A group's ascending index list of K entries becomes ceil(N/32) words, bit j
// of the row set iff key j is selected. At the densities the method uses
// (K >= N/32) this is smaller than K 4-byte indices (4.8x at 15%).
//
// encode: one workgroup per (b, h, g) row; the row's words are built in LDS
//         with atomic ORs (order-free, so deterministic) and written once.
// decode: one workgroup per row; each thread takes a contiguous run of
//         words, a block-wide exclusive scan of their popcounts gives every
//         thread its first output position, and set bits are written in
//         ascending key order.
#include "mcs_common.hpp"
#include "mcs_internal.hpp"

namespace mcs {

namespace {

constexpr int kCodeThreads = 256;

__global__ __launch_bounds__(kCodeThreads) void idx_encode_kernel(const int32_t *idx, int K, int N, int W,
                                                                  uint32_t *bitmap) {
  extern __shared__ uint32_t words[];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  for (int w = tid; w < W; w += kCodeThreads) words[w] = 0u;
  __syncthreads();
  const int32_t *in = idx + row * K;
  for (int i = tid; i < K; i += kCodeThreads) {
    const int j = in[i];
    if (j >= 0 && j < N) atomicOr(&words[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  uint32_t *out = bitmap + row * W;
  for (int w = tid; w < W; w += kCodeThreads) out[w] = words[w];
}

__global__ __launch_bounds__(kCodeThreads) void idx_decode_kernel(const uint32_t *bitmap, int K, int W,
                                                                  int32_t *idx) {
  __shared__ uint32_t wave_sum[kCodeThreads / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (W + kCodeThreads - 1) / kCodeThreads;  // words per thread
  const int w0 = tid * per < W ? tid * per : W;
  const int w1 = w0 + per < W ? w0 + per : W;
  const uint32_t *in = bitmap + row * W;
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += (uint32_t)__popc(in[w]);
  // exclusive scan of the threads' counts in thread order
  uint32_t x = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_sum[wave] = x;
  __syncthreads();
  uint32_t pos = x - cnt;
  for (int q = 0; q < wave; ++q) pos += wave_sum[q];
  int32_t *out = idx + row * K;
  for (int w = w0; w < w1; ++w) {
    uint32_t bits = in[w];
    while (bits) {
      const int b = __ffs(bits) - 1;
      if (pos < (uint32_t)K) out[pos] = 32 * w + b;
      ++pos;
      bits &= bits - 1u;
    }
  }
}

}  // namespace

size_t idx_bitmap_words(int N) { return (size_t)((N + 31) / 32); }

hipError_t launch_idx_encode(const int32_t *idx, int64_t rows, int K, int N, uint32_t *bitmap, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int W = (int)idx_bitmap_words(N);
  hipLaunchKernelGGL(idx_encode_kernel, dim3((unsigned)rows), dim3(kCodeThreads), (size_t)W * 4, s, idx, K, N, W,
                     bitmap);
  return hipGetLastError();
}

hipError_t launch_idx_decode(const uint32_t *bitmap, int64_t rows, int K, int N, int32_t *idx, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int W = (int)idx_bitmap_words(N);
  hipLaunchKernelGGL(idx_decode_kernel, dim3((unsigned)rows), dim3(kCodeThreads), 0, s, bitmap, K, W, idx);
  return hipGetLastError();
}

}  // namespace mcs
