// Internal launcher interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mcs {

enum AttnMode { kModeDense = 0, kModeSparse = 1, kModeResidual = 2 };

struct AttnArgs {
  const uint16_t *q, *k, *v;
  const uint16_t *aux;  // sparse: R (nullable); residual: O_dense
  uint16_t *out;        // O (dense, sparse) or R (residual)
  float *lse;           // dense only, nullable
  const int32_t *perm;  // sparse / residual
  const int32_t *idx;   // sparse / residual
  int64_t sb, sn, sh;
  int32_t B, H, N;
  int32_t rows;   // query rows per workgroup (group size T, or the dense tile)
  int32_t G;      // workgroups per head
  int32_t K;      // selected keys per group (sparse / residual)
  float scale_log2;
};

// head_dim in {64,128}; rows in {64,128}
hipError_t launch_attention(int mode, int head_dim, const AttnArgs &a, hipStream_t s);

struct SelectArgs {
  const uint16_t *q, *k;
  const float *lse;
  const int32_t *perm;
  float *mass;  // [B][H][G][N]
  int32_t *idx; // [B][H][G][K]
  int64_t sb, sn, sh;
  int32_t B, H, N, T, G, K;
  float scale_log2;
};
hipError_t launch_select(int head_dim, const SelectArgs &a, hipStream_t s);

// block-granularity selection over mass rows: block sums, top-nb blocks,
// expansion to ascending key indices; ws holds the sums and the block ids
size_t select_blocks_bsum_bytes(int64_t rows, int N, int blk);
size_t select_blocks_ws_bytes(int64_t rows, int N, int blk, int nb);
hipError_t launch_select_blocks(const float *mass, int64_t rows, int N, int blk, int nb, int32_t *kv_idx, void *ws,
                                hipStream_t s);

// bitmap form of the KV indices: ceil(N/32) words per (b, h, g) row
size_t idx_bitmap_words(int N);
hipError_t launch_idx_encode(const int32_t *idx, int64_t rows, int K, int N, uint32_t *bitmap, hipStream_t s);
hipError_t launch_idx_decode(const uint32_t *bitmap, int64_t rows, int K, int N, int32_t *idx, hipStream_t s);

// Device scratch owned by the library (mcs_scratch.hip): kScratchBytes on
// each GPU, whose address scratch_address() returns for the current device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_address(void **out);

size_t pddp_workspace_bytes(int B, int H, int N, int D, int T);
hipError_t run_pddp(const uint16_t *q, int64_t sb, int64_t sn, int64_t sh, int B, int H, int N,
                    int D, int T, int power_iters, bool whiten, int32_t *perm, void *ws,
                    size_t ws_bytes, hipStream_t s);

}  // namespace mcs
