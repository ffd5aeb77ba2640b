// Anchor selection on gfx950: the second QK pass that recovers exact
// probabilities P_ij = exp(scale * q_i . k_j - L_i), their sum over each query
// group, A[g][j] = sum_{i in g} P_ij, and the per-group top-K of single keys
// (ties -> lower key index), stored ascending.
//
// mass_kernel: one workgroup per (b, h, g). Each wave holds 32 of the group's
// query rows as MFMA A-operands; 64-key tiles of K arrive by LDS-DMA (16
// bytes per lane straight into LDS, chunks XOR-swizzled per row) in two
// stages, the next tile loading while the current one is used. S = Q . K^T
// via v_mfma_f32_32x32x16_bf16 leaves every lane with 16 query rows of ONE
// key, so the column sum over the wave is 16 local adds plus one
// cross-half add; the 4 (or 2) waves' partial sums meet in LDS and are added
// in a fixed order (no atomics).
//
// topk_kernel: one workgroup per (b, h, g). Radix select (4 passes of 8 bits,
// most significant first) finds the K-th largest mass; a single ordered pass
// with ballot prefix counts then keeps every key above it and the
// lowest-index keys equal to it, writing their indices in ascending order.
#include <type_traits>

#include "mcs_common.hpp"
#include "mcs_internal.hpp"
#include "mcs_lds.hpp"
#include "mcs_radix.hpp"

namespace mcs {

template <int D, int NW>
struct MassCfg {
  static constexpr int NT = 64 * NW;
  static constexpr int KT = 64;                  // keys per tile
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int TILEB = KT * D * 2;       // bytes of one K tile
  static constexpr int LPW = TILEB / 1024 / NW;  // 1 KB LDS-DMA loads per wave
  static_assert(LPW >= 1 && LPW * NW * 1024 == TILEB, "loader mapping");
};

template <int D, int NW>
// four workgroups per CU (34.5 KB of LDS each at d = 128): at 128 VGPRs the
// waves' exponentials and MFMAs overlap better than at two workgroups
__global__ __launch_bounds__(64 * NW, 4) void mass_kernel(SelectArgs a) {
  using C = MassCfg<D, NW>;
  // two stages as separate LDS objects, so the compiler can tell the stage
  // being filled by DMA from the one being read
  __shared__ __attribute__((aligned(1024))) bf16_t st0[C::KT * D];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[C::KT * D];
  __shared__ float partial[2][NW][C::KT];

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / a.G;
  const int g = work - bh * a.G;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;

  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const bf16_t *qb = a.q + head_off;
  const int32_t *pr = a.perm + (int64_t)bh * a.N;
  const float *lse = a.lse + (int64_t)bh * a.N;
  const int row0 = g * a.T;
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const uint32_t extent = (uint32_t)(a.N - 1) * row_bytes + D * 2;
  const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(a.k + head_off, extent);

  // A-operand rows: query wave*32 + l32 of the group
  bf16x8 qf[D / 16];
  {
    const int r = wave * 32 + l32;
    const int pos = row0 + r;
    const bool ok = r < a.T && pos < a.N;
    const bf16_t *qrow = qb + (int64_t)pr[ok ? pos : row0] * a.sn + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *(const bf16x8 *)(qrow + 16 * s);
  }
  // accumulator rows held by this lane: wave*32 + 8*(v/4) + 4*hh + (v%4)
  float l2[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = wave * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
    const int pos = row0 + r;
    const bool ok = r < a.T && pos < a.N;
    l2[v] = ok ? lse[pr[pos]] * kLog2e : 1.0e30f;  // invalid row: P = 0
  }
  const float c2 = a.scale_log2;

  const int ntiles = (a.N + C::KT - 1) / C::KT;
  // DMA of tile t's K rows: slot S of the stage is row S / CH, stored chunk
  // S % CH, holding logical chunk (S % CH) ^ swz(row); rows past N repeat
  // the last key (their sums are not written)
  auto issue = [&](int t, bf16_t *stage) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int slot = (wave * C::LPW + i) * 64 + lane;
      const int row = slot / C::CH;
      const int chunk = (slot % C::CH) ^ swz<C::CH>(row);
      const int key = t * C::KT + row;
      const uint32_t off = (uint32_t)(key < a.N ? key : a.N - 1) * row_bytes + chunk * 16;
      buffer_load_lds16(rk, (char *)stage + (wave * C::LPW + i) * 1024, off);
    }
  };

  float *mass_row = a.mass + ((int64_t)bh * a.G + g) * a.N;
  auto finish = [&](int t) {  // tile t's column sums over the waves, fixed order
    if (tid < C::KT) {
      const int key = t * C::KT + tid;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += partial[t & 1][w][tid];
      if (key < a.N) mass_row[key] = s;
    }
  };
  auto tile = [&](int t, const bf16_t *cur, bf16_t *nxt, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    if (!LAST) issue(t + 1, nxt);
    if (t > 0) finish(t - 1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 st = f32x16{};
      const int r = 32 * kb + l32;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 kf = *(const bf16x8 *)(cur + r * D + (((2 * s + hh) ^ swz<C::CH>(r)) << 3));
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[s], kf, st, 0, 0, 0);
      }
      float cs = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) cs += fast_exp2(__builtin_fmaf(st[v], c2, -l2[v]));
      float lo, hi;
      cross_half(cs, lo, hi);
      if (hh == 0) partial[t & 1][wave][r] = lo + hi;
    }
    // this wave's DMA into `nxt` has landed; then every wave's, and every
    // wave's partial sums are in LDS
    if (!LAST) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };

  issue(0, st0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  int t = 0;
  for (; t + 2 < ntiles; t += 2) {
    tile(t, st0, st1, std::false_type{});
    tile(t + 1, st1, st0, std::false_type{});
  }
  if (ntiles - t == 2) {
    tile(t, st0, st1, std::false_type{});
    tile(t + 1, st1, st0, std::true_type{});
  } else {
    tile(t, st0, st1, std::true_type{});
  }
  finish(ntiles - 1);
}

// ---------------------------------------------------------------------------
// top-K
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 512;

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);  // -0 and +0 are equal masses
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_cnt[2][kTopkThreads / 64];
  __shared__ uint32_t sel_digit, sel_above;

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int row = work;  // (bh, g) flattened
  const float *A = a.mass + (int64_t)row * a.N;
  int32_t *out = a.idx + (int64_t)row * a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N;

  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)a.K;  // how many of the largest are still to be placed
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < N; j += kTopkThreads) {
      const uint32_t u = order_key(A[j]);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) radix_pick<true>(hist, remaining, &sel_digit, &sel_above);
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= 255u << shift;
    remaining -= sel_above;
    __syncthreads();
  }
  // prefix is the K-th largest key; take all larger keys and `remaining`
  // keys equal to it, lowest index first.
  const uint32_t tau = prefix;
  const uint32_t need = remaining;
  uint32_t written = 0, ties = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < N; base += kTopkThreads) {
    const int j = base + tid;
    uint32_t u = 0;
    if (j < N) u = order_key(A[j]);
    const bool gt = j < N && u > tau;
    const bool eq = j < N && u == tau;
    const uint64_t beq = __ballot(eq);
    const uint64_t bgt = __ballot(gt);
    if (lane == 0) {
      wave_cnt[0][wave] = (uint32_t)__popcll(beq);
      wave_cnt[1][wave] = (uint32_t)__popcll(bgt);
    }
    __syncthreads();
    uint32_t eq_before = 0, eq_total = 0;
    for (int w = 0; w < kTopkThreads / 64; ++w) {
      const uint32_t ce = wave_cnt[0][w];
      eq_before += (w < wave) ? ce : 0u;
      eq_total += ce;
    }
    const uint32_t tie_rank = ties + eq_before + (uint32_t)__popcll(beq & lt_mask);
    const bool sel = gt || (eq && tie_rank < need);
    const uint64_t bsel = __ballot(sel);
    __syncthreads();
    if (lane == 0) wave_cnt[0][wave] = (uint32_t)__popcll(bsel);
    __syncthreads();
    uint32_t sel_before = 0, sel_total = 0;
    for (int w = 0; w < kTopkThreads / 64; ++w) {
      const uint32_t cs = wave_cnt[0][w];
      sel_before += (w < wave) ? cs : 0u;
      sel_total += cs;
    }
    if (sel) out[written + sel_before + (uint32_t)__popcll(bsel & lt_mask)] = j;
    written += sel_total;
    ties += eq_total;
    __syncthreads();
  }
}

template <int D, int NW>
static hipError_t launch_mass(const SelectArgs &a, hipStream_t s) {
  const int nblocks = a.B * a.H * a.G;
  hipLaunchKernelGGL((mass_kernel<D, NW>), dim3(nblocks), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(int head_dim, const SelectArgs &a, hipStream_t s) {
  const int nblocks = a.B * a.H * a.G;
  if (nblocks <= 0) return hipSuccess;
  hipError_t e;
  if (head_dim == 128 && a.T == 128) e = launch_mass<128, 4>(a, s);
  else if (head_dim == 128 && a.T == 64) e = launch_mass<128, 2>(a, s);
  else if (head_dim == 64 && a.T == 128) e = launch_mass<64, 4>(a, s);
  else if (head_dim == 64 && a.T == 64) e = launch_mass<64, 2>(a, s);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3(nblocks), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mcs
