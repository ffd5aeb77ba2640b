// Anchor selection on gfx950: the second QK pass that recovers exact
// probabilities P_ij = exp(scale * q_i . k_j - L_i), their sum over each query
// group, A[g][j] = sum_{i in g} P_ij, and the per-group top-K of single keys
// (ties -> lower key index), stored ascending.
//
// mass_kernel / mass_wide_kernel: one workgroup per GPW groups of one head.
// Each wave holds 32 (or, in the wide form, 64) of a group's query rows as
// MFMA A-operands; K tiles arrive by LDS-DMA (16 bytes per lane straight
// into LDS, chunks XOR-swizzled per row) in two stages, the next tile
// loading while the current one is used. S = Q . K^T via
// v_mfma_f32_32x32x16_bf16 leaves every lane with 16 query rows of ONE key,
// so the column sum over 32 rows is 16 local adds plus one cross-half add;
// the 32-row blocks' partial sums meet in LDS and are added in a fixed order
// (no atomics), so both forms give the same bits.
//
// Top-K: one workgroup per (b, h, g). A radix select, most significant
// digit first, finds the K-th largest mass; an ordered pass with ballot
// prefix counts then keeps every key above it and the lowest-index keys equal
// to it, writing their indices in ascending order.
//   topk_reg_kernel (rows up to 98304 keys): the row is read once into
//     registers and every digit and the partition work from there;
//   topk_kernel (longer rows): the first digit from the row, the rest from
//     that digit's bin compacted into LDS (or from the row again when the
//     bin does not fit), then the partition reads the row once more.
#include <type_traits>

#include "mcs_common.hpp"
#include "mcs_internal.hpp"
#include "mcs_lds.hpp"
#include "mcs_radix.hpp"

namespace mcs {

template <int D, int NW, int KT_ = 64>
struct MassCfg {
  static constexpr int NT = 64 * NW;
  static constexpr int KT = KT_;                 // keys per tile
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int TILEB = KT * D * 2;       // bytes of one K tile
  static constexpr int LPW = TILEB / 1024 / NW;  // 1 KB LDS-DMA loads per wave
  static_assert(LPW >= 1 && LPW * NW * 1024 == TILEB, "loader mapping");
};

// GPW groups per workgroup, WPG waves (32 rows each) per group. 128-row
// groups run two to a workgroup: the eight waves share each K tile's DMA,
// and at 128 VGPRs two such workgroups fill a CU (four waves per SIMD):
// select 4.6% faster than one group per workgroup at the same occupancy,
// identical indices (randomised-order A/B in one process); four groups per
// workgroup (one per CU) were 1.9% slower than one. 64-row groups run four
// to a workgroup, the same eight waves and 256 rows per K tile: select 5.04
// -> 3.80 ms at wan480p with T = 64 against one 2-wave group per workgroup,
// identical indices and masses.
template <int D, int WPG, int GPW>
__global__ __launch_bounds__(64 * WPG * GPW, WPG * GPW >= 4 ? 4 : 2) void mass_kernel(SelectArgs a) {
  constexpr int NW = WPG * GPW;
  using C = MassCfg<D, NW>;
  static_assert(C::NT >= GPW * C::KT, "one finishing thread per key of each group");
  // two stages as separate LDS objects, so the compiler can tell the stage
  // being filled by DMA from the one being read
  __shared__ __attribute__((aligned(1024))) bf16_t st0[C::KT * D];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[C::KT * D];
  __shared__ float partial[2][NW][C::KT];

  const int sets = (a.G + GPW - 1) / GPW;  // workgroups per head
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / sets;
  const int gs = work - bh * sets;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = wave % WPG;               // wave within its group
  const int g = GPW * gs + wave / WPG;     // this wave's group (past G: none, rows masked)
  const bool gvalid = g < a.G;
  const int l32 = lane & 31, hh = lane >> 5;

  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const bf16_t *qb = a.q + head_off;
  const int32_t *pr = a.perm + (int64_t)bh * a.N;
  const float *lse = a.lse + (int64_t)bh * a.N;
  const int row0 = (gvalid ? g : 0) * a.T;
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const uint32_t extent = (uint32_t)(a.N - 1) * row_bytes + D * 2;
  const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(a.k + head_off, extent);

  // A-operand rows: query wg*32 + l32 of the group
  bf16x8 qf[D / 16];
  {
    const int r = wg * 32 + l32;
    const int pos = row0 + r;
    const bool ok = r < a.T && pos < a.N;
    const bf16_t *qrow = qb + (int64_t)pr[ok ? pos : row0] * a.sn + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *(const bf16x8 *)(qrow + 16 * s);
  }
  // accumulator rows held by this lane: wg*32 + 8*(v/4) + 4*hh + (v%4)
  float l2[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = wg * 32 + 8 * (v >> 2) + 4 * hh + (v & 3);
    const int pos = row0 + r;
    const bool ok = gvalid && r < a.T && pos < a.N;
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

  // thread fg * KT + fk finishes key fk of the tile for group GPW*gs + fg
  const int fg = tid / C::KT;
  const int fk = tid - fg * C::KT;
  const bool fval = fg < GPW && GPW * gs + fg < a.G;
  float *mass_row = a.mass + ((int64_t)bh * a.G + (GPW * gs + fg)) * a.N;
  auto finish = [&](int t) {  // tile t's column sums over the group's waves, fixed order
    if (fval) {
      const int key = t * C::KT + fk;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WPG; ++w) s += partial[t & 1][WPG * fg + w][fk];
      if (key < a.N) mass_row[key] = s;
    }
  };
  auto tile = [&](int t, const bf16_t *cur, bf16_t *nxt, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
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
      // the next tile's DMA once the first half's K reads are out, so its
      // LDS writes do not compete with them (3% faster than issuing it first)
      if (kb == 0 && !LAST) issue(t + 1, nxt);
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

// The same sweep with 64 query rows per wave (WPG waves per group, GPW
// groups per workgroup, KT-key tiles): each K fragment read from LDS feeds
// two MFMAs (rows 0-31 and 32-63 of the wave), at two waves per SIMD. For
// 128-row groups at d = 128 it runs four groups per workgroup, eight waves
// sharing each 128-key tile's DMA (512 rows), one workgroup per CU: select
// 1.6-2.4% faster than two groups per workgroup of mass_kernel at wan480p
// on three boxes (3% at longvideo with 64-key tiles), identical masses and
// indices.
template <int D, int WPG, int GPW, int KT>
__global__ __launch_bounds__(64 * WPG * GPW, 2) void mass_wide_kernel(SelectArgs a) {
  constexpr int NW = WPG * GPW;
  using C = MassCfg<D, NW, KT>;
  static_assert(C::NT >= GPW * C::KT, "one finishing thread per key of each group");
  // two stages as separate LDS objects, so the compiler can tell the stage
  // being filled by DMA from the one being read
  __shared__ __attribute__((aligned(1024))) bf16_t st0[C::KT * D];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[C::KT * D];
  __shared__ float partial[2][2 * NW][C::KT];  // one row per 32-row half of a wave

  const int sets = (a.G + GPW - 1) / GPW;  // workgroups per head
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = work / sets;
  const int gs = work - bh * sets;
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = wave % WPG;               // wave within its group
  const int g = GPW * gs + wave / WPG;     // this wave's group (past G: none, rows masked)
  const bool gvalid = g < a.G;
  const int l32 = lane & 31, hh = lane >> 5;

  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const bf16_t *qb = a.q + head_off;
  const int32_t *pr = a.perm + (int64_t)bh * a.N;
  const float *lse = a.lse + (int64_t)bh * a.N;
  const int row0 = (gvalid ? g : 0) * a.T;
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const uint32_t extent = (uint32_t)(a.N - 1) * row_bytes + D * 2;
  const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(a.k + head_off, extent);

  // A-operand rows: query 64*wg + 32*m + l32 of the group
  bf16x8 qf[2][D / 16];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int r = 64 * wg + 32 * m + l32;
    const int pos = row0 + r;
    const bool ok = r < a.T && pos < a.N;
    const bf16_t *qrow = qb + (int64_t)pr[ok ? pos : row0] * a.sn + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[m][s] = *(const bf16x8 *)(qrow + 16 * s);
  }
  // accumulator rows held by this lane: 64*wg + 32*m + 8*(v/4) + 4*hh + (v%4)
  float l2[2][16];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 64 * wg + 32 * m + 8 * (v >> 2) + 4 * hh + (v & 3);
      const int pos = row0 + r;
      const bool ok = gvalid && r < a.T && pos < a.N;
      l2[m][v] = ok ? lse[pr[pos]] * kLog2e : 1.0e30f;  // invalid row: P = 0
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

  // thread fg * KT + fk finishes key fk of the tile for group GPW*gs + fg
  const int fg = tid / C::KT;
  const int fk = tid - fg * C::KT;
  const bool fval = fg < GPW && GPW * gs + fg < a.G;
  float *mass_row = a.mass + ((int64_t)bh * a.G + (GPW * gs + fg)) * a.N;
  auto finish = [&](int t) {  // tile t's column sums over the group's 32-row blocks, fixed order
    if (fval) {
      const int key = t * C::KT + fk;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < 2 * WPG; ++w) s += partial[t & 1][2 * WPG * fg + w][fk];
      if (key < a.N) mass_row[key] = s;
    }
  };
  auto tile = [&](int t, const bf16_t *cur, bf16_t *nxt, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    if (t > 0) finish(t - 1);
#pragma unroll
    for (int kb = 0; kb < C::KT / 32; ++kb) {
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      const int r = 32 * kb + l32;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 kf = *(const bf16x8 *)(cur + r * D + (((2 * s + hh) ^ swz<C::CH>(r)) << 3));
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], kf, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][s], kf, s1, 0, 0, 0);
      }
      // the next tile's DMA once the first half's K reads are out, so its
      // LDS writes do not compete with them
      if (kb == 0 && !LAST) issue(t + 1, nxt);
      float c0 = 0.f, c1 = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) c0 += fast_exp2(__builtin_fmaf(s0[v], c2, -l2[0][v]));
#pragma unroll
      for (int v = 0; v < 16; ++v) c1 += fast_exp2(__builtin_fmaf(s1[v], c2, -l2[1][v]));
      float lo0, hi0, lo1, hi1;
      cross_half(c0, lo0, hi0);
      cross_half(c1, lo1, hi1);
      if (hh == 0) {
        partial[t & 1][2 * wave][r] = lo0 + hi0;
        partial[t & 1][2 * wave + 1][r] = lo1 + hi1;
      }
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
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kCandCap = 15360;  // keys of the first digit's bin kept in LDS (two workgroups per CU)
constexpr int kHCopies = 8;      // private histogram copies (lane % 8)
constexpr int kILP = 8;          // keys loaded per thread before they are used

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);  // -0 and +0 are equal masses
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// radix_pick over 512 descending bins (one wave): the upper 256 bins first.
__device__ __forceinline__ void pick512_desc(const uint32_t *hist, uint32_t remaining, uint32_t *digit_out,
                                             uint32_t *before_out) {
  const int lane = threadIdx.x & 63;
  uint32_t up = hist[256 + 4 * lane] + hist[257 + 4 * lane] + hist[258 + 4 * lane] + hist[259 + 4 * lane];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) up += __shfl_xor(up, off);
  if (remaining <= up) radix_pick<true>(hist + 256, remaining, digit_out, before_out, 256u, 0u);
  else radix_pick<true>(hist, remaining - up, digit_out, before_out, 0u, up);
}

// One workgroup per (b, h, g) row of A. Keys are the masses' order-preserving
// 32-bit images. The K-th largest key is found digit by digit, most
// significant first: bits 31..23 over the whole row; then, when the chosen
// bin's keys fit, they are compacted into LDS and bits 22..15, 14..7 and 6..0
// are resolved there (otherwise from the row again). A last ordered pass keeps
// every key above it and the lowest-index keys equal to it, writing their
// indices in ascending order. Histograms are kept in kHCopies copies, picked
// by lane % 8 at a bank-shifting stride, so equal digits within a wave
// contend at most 8-way; the copies are added in a fixed order.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  __shared__ uint32_t hc[kHCopies * 513];
  __shared__ uint32_t hist[512];
  __shared__ uint32_t cand[kCandCap];
  __shared__ uint32_t eq_cnt[kTopkWaves], sel_cnt[kTopkWaves];
  __shared__ uint32_t sel_digit, sel_above, ncand;

  const int row = xcd_remap(blockIdx.x, gridDim.x);  // (bh, g) flattened
  const float *A = a.mass + (int64_t)row * a.N;
  int32_t *out = a.idx + (int64_t)row * a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  auto clear = [&](int nb) {
    for (int i = tid; i < kHCopies * (nb + 1); i += kTopkThreads) hc[i] = 0;
  };
  auto merge = [&](int nb) {
    for (int b = tid; b < nb; b += kTopkThreads) {
      uint32_t s = 0;
#pragma unroll
      for (int c = 0; c < kHCopies; ++c) s += hc[c * (nb + 1) + b];
      hist[b] = s;
    }
  };
  // the row's keys, kILP per thread in flight: f(j, key) for j < N
  auto scan_row = [&](auto f) {
    for (int base = 0; base < N; base += kTopkThreads * kILP) {
      uint32_t u[kILP];
#pragma unroll
      for (int k = 0; k < kILP; ++k) {
        const int j = base + k * kTopkThreads + tid;
        u[k] = order_key(A[j < N ? j : N - 1]);
      }
#pragma unroll
      for (int k = 0; k < kILP; ++k) f(base + k * kTopkThreads + tid, u[k]);
    }
  };

  // digit 1: bits 31..23 of every key
  clear(512);
  if (tid == 0) ncand = 0;
  __syncthreads();
  scan_row([&](int j, uint32_t u) {
    if (j < N) atomicAdd(&hc[(lane & (kHCopies - 1)) * 513 + (u >> 23)], 1u);
  });
  __syncthreads();
  merge(512);
  __syncthreads();
  if (wave == 0) pick512_desc(hist, (uint32_t)a.K, &sel_digit, &sel_above);
  __syncthreads();
  uint32_t prefix = sel_digit << 23, mask = 0xff800000u;
  uint32_t remaining = (uint32_t)a.K - sel_above;  // of the largest, still to be placed
  const bool in_lds = hist[sel_digit] <= (uint32_t)kCandCap;
  if (in_lds) {  // compact the chosen bin's keys (any order: only values matter)
    scan_row([&](int j, uint32_t u) {
      const bool m = j < N && (u & mask) == prefix;
      const uint64_t b = __ballot(m);
      if (b != 0) {
        uint32_t at = 0;
        if (lane == 0) at = atomicAdd(&ncand, (uint32_t)__popcll(b));
        at = __shfl(at, 0);
        const uint32_t slot = at + (uint32_t)__popcll(b & lt_mask);
        if (m && slot < (uint32_t)kCandCap) cand[slot] = u;
      }
    });
    __syncthreads();
  }
  const int nc = in_lds ? (int)(ncand < (uint32_t)kCandCap ? ncand : (uint32_t)kCandCap) : 0;
  // digits 2..4: bits 22..15, 14..7, 6..0
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 15 : (pass == 1 ? 7 : 0);
    const uint32_t dm = pass == 2 ? 127u : 255u;
    clear(256);
    __syncthreads();
    auto add = [&](uint32_t u) {
      if ((u & mask) == prefix) atomicAdd(&hc[(lane & (kHCopies - 1)) * 257 + ((u >> shift) & dm)], 1u);
    };
    if (in_lds) {
      for (int i = tid; i < nc; i += kTopkThreads) add(cand[i]);
    } else {
      scan_row([&](int j, uint32_t u) {
        if (j < N) add(u);
      });
    }
    __syncthreads();
    merge(256);
    __syncthreads();
    if (wave == 0) radix_pick<true>(hist, remaining, &sel_digit, &sel_above);
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= dm << shift;
    remaining -= sel_above;
    __syncthreads();
  }
  // prefix is the K-th largest key; take all larger keys and `remaining`
  // keys equal to it, lowest index first.
  const uint32_t tau = prefix;
  const uint32_t need = remaining;
  // Per 512-key chunk, two barriers: a wave rewrites eq_cnt only after the
  // previous chunk's second barrier, by which every wave has read it, and
  // sel_cnt only after this chunk's first barrier, by which every wave has
  // read the previous chunk's.
  uint32_t written = 0, ties = 0;
  scan_row([&](int j, uint32_t u) {
    const bool ok = j < N;
    const bool gt = ok && u > tau;
    const bool eq = ok && u == tau;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) eq_cnt[wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_before = 0, eq_total = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const uint32_t ce = eq_cnt[w];
      eq_before += (w < wave) ? ce : 0u;
      eq_total += ce;
    }
    const uint32_t tie_rank = ties + eq_before + (uint32_t)__popcll(beq & lt_mask);
    const bool sel = gt || (eq && tie_rank < need);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) sel_cnt[wave] = (uint32_t)__popcll(bsel);
    __syncthreads();
    uint32_t sel_before = 0, sel_total = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      const uint32_t cs = sel_cnt[w];
      sel_before += (w < wave) ? cs : 0u;
      sel_total += cs;
    }
    const uint32_t pos = written + sel_before + (uint32_t)__popcll(bsel & lt_mask);
    if (sel && pos < (uint32_t)a.K) out[pos] = j;
    written += sel_total;
    ties += eq_total;
  });
}

// Indices staged in LDS before the row's output is written: the whole row
// (K <= N) for the smaller kernels, else 12,288 indices (48 KB, two 512-thread
// workgroups per CU), or 16,384 (64 KB) for the 768-thread kernel, which runs
// one workgroup per CU.
template <int NTH, int KPT>
constexpr int topk_stage_cap() {
  return NTH == 768 ? 16384 : (NTH * KPT < 12288 ? NTH * KPT : 12288);
}

// Rows of up to NTH * KPT keys: the whole row is read once into registers
// (wave w holds the contiguous segment [w * 64 * KPT, (w + 1) * 64 * KPT),
// lane l the keys at l, l + 64, ...), every digit is resolved from the
// registers, and each wave writes its own segment's selected indices after a
// single barrier that gives it the counts of the segments before it.
template <int NTH, int KPT>
__global__ __launch_bounds__(NTH) void topk_reg_kernel(SelectArgs a) {
  constexpr int NW = NTH / 64;
  constexpr int SEG = 64 * KPT;
  constexpr int SCAP = topk_stage_cap<NTH, KPT>();
  __shared__ uint32_t hc[kHCopies * 513];
  __shared__ uint32_t hist[512];
  __shared__ uint32_t gt_cnt[NW], eq_cnt[NW];
  __shared__ uint32_t sel_digit, sel_above;
  __shared__ int32_t stage[SCAP];

  const int row = xcd_remap(blockIdx.x, gridDim.x);  // (bh, g) flattened
  const float *A = a.mass + (int64_t)row * a.N;
  int32_t *out = a.idx + (int64_t)row * a.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N;
  const int j0 = wave * SEG + lane;  // key k of this lane: j0 + 64 k
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t *hcl = hc + (lane & (kHCopies - 1)) * 513;

  // Masses are sums of exponentials, so every key of the row has bit 31 set
  // (a negative value, which cannot occur, would rank as +0). Slots past the
  // row hold key 0: no digit prefix matches it and it is never above the
  // threshold, so no per-key validity test is needed. Buffer loads: the
  // whole byte offset of key j0 + 64 k is in the VGPR offset (the range check
  // covers the VGPR and instruction offsets, not the SGPR offset), so a read
  // past the row's N keys returns 0 and never touches memory after it.
  const __amdgpu_buffer_rsrc_t ra = uniform_rsrc(A, (uint32_t)N * 4u);
  const int nv = N - j0 <= 0 ? 0 : (N - j0 + 63) / 64;  // valid keys of this lane
  uint32_t u[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const uint32_t voff = (uint32_t)(j0 + 64 * k) * 4u;
    const uint32_t key = order_key(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, voff, 0, 0)));
    u[k] = k < nv ? (key > 0x80000000u ? key : 0x80000000u) : 0u;
  }

  // digit 1: bits 31..23
  for (int i = tid; i < kHCopies * 513; i += NTH) hc[i] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < KPT; ++k) atomicAdd(&hcl[u[k] >> 23], 1u);  // key 0 lands in bin 0, never reached
  __syncthreads();
  for (int b = tid; b < 512; b += NTH) {
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < kHCopies; ++c) s += hc[c * 513 + b];
    hist[b] = s;
  }
  __syncthreads();
  if (wave == 0) pick512_desc(hist, (uint32_t)a.K, &sel_digit, &sel_above);
  __syncthreads();
  uint32_t prefix = sel_digit << 23, mask = 0xff800000u;
  uint32_t remaining = (uint32_t)a.K - sel_above;
  // digits 2..4: bits 22..15, 14..7, 6..0
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 15 : (pass == 1 ? 7 : 0);
    const uint32_t dm = pass == 2 ? 127u : 255u;
    for (int i = tid; i < kHCopies * 257; i += NTH) hc[i] = 0;
    __syncthreads();
    uint32_t *hcl2 = hc + (lane & (kHCopies - 1)) * 257;
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if ((u[k] & mask) == prefix) atomicAdd(&hcl2[(u[k] >> shift) & dm], 1u);
    __syncthreads();
    for (int b = tid; b < 256; b += NTH) {
      uint32_t s = 0;
#pragma unroll
      for (int c = 0; c < kHCopies; ++c) s += hc[c * 257 + b];
      hist[b] = s;
    }
    __syncthreads();
    if (wave == 0) radix_pick<true>(hist, remaining, &sel_digit, &sel_above);
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= dm << shift;
    remaining -= sel_above;
  }
  const uint32_t tau = prefix;
  const uint32_t need = remaining;
  // the segments' counts above and equal to tau (tau through an empty asm:
  // the partitions below then make their own comparisons instead of keeping
  // these 2 * KPT flags live across the barrier)
  uint32_t tau_cnt = tau;
  asm volatile("" : "+v"(tau_cnt));
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    gt += u[k] > tau_cnt ? 1u : 0u;
    eq += u[k] == tau_cnt ? 1u : 0u;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) {
    gt_cnt[wave] = gt;
    eq_cnt[wave] = eq;
  }
  __syncthreads();
  uint32_t written = 0, ties = 0;  // before this wave's segment
  for (int w = 0; w < wave; ++w) {
    const uint32_t e = eq_cnt[w];
    const uint32_t room = need > ties ? need - ties : 0u;
    written += gt_cnt[w] + (e < room ? e : room);
    ties += e;
  }
  uint32_t eq_all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) eq_all += eq_cnt[w];
  if (eq_all == need) {
    // Every key equal to tau is kept (the usual case: the K-th largest mass
    // is unique), so the selection is simply u >= tau, K keys in all. A
    // key's position is its wave's offset plus the selected keys before it
    // in (k, lane) order. With K <= SCAP the indices gather in LDS and the
    // row is written by all threads in order, 256 contiguous bytes a wave.
    // (tau passes through an empty asm so that these comparisons are not
    // merged with the counts' above, whose 128 flags would then stay live.)
    uint32_t tau_ge = tau;
    asm volatile("" : "+v"(tau_ge));
    if (a.K <= SCAP) {
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        const bool sel = u[k] >= tau_ge;
        const uint64_t m = __ballot(sel);
        const uint32_t pos = written + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (sel && pos < (uint32_t)a.K) stage[pos] = j0 + 64 * k;
        written += (uint32_t)__popcll(m);
      }
      __syncthreads();
      for (int i = tid; i < a.K; i += NTH) out[i] = stage[i];
    } else {
#pragma unroll
      for (int k = 0; k < KPT; ++k) {
        const bool sel = u[k] >= tau_ge;
        const uint64_t m = __ballot(sel);
        const uint32_t pos = written + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (sel && pos < (uint32_t)a.K) out[pos] = j0 + 64 * k;
        written += (uint32_t)__popcll(m);
      }
    }
    return;
  }
  // Some keys equal to tau are left out: they are taken in ascending index
  // order until `need` of them are in.
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool g = u[k] > tau;
    const bool e = u[k] == tau;
    const uint64_t beq = __ballot(e);
    const bool sel = g || (e && ties + (uint32_t)__popcll(beq & lt_mask) < need);
    const uint64_t bsel = __ballot(sel);
    const uint32_t pos = written + (uint32_t)__popcll(bsel & lt_mask);
    if (sel && pos < (uint32_t)a.K) out[pos] = j0 + 64 * k;
    written += (uint32_t)__popcll(bsel);
    ties += (uint32_t)__popcll(beq);
  }
}

template <int D, int WPG, int GPW, int KT>
static hipError_t launch_mass_wide(const SelectArgs &a, hipStream_t s) {
  const int nblocks = a.B * a.H * ((a.G + GPW - 1) / GPW);
  hipLaunchKernelGGL((mass_wide_kernel<D, WPG, GPW, KT>), dim3(nblocks), dim3(64 * WPG * GPW), 0, s, a);
  return hipGetLastError();
}

template <int D, int WPG, int GPW>
static hipError_t launch_mass(const SelectArgs &a, hipStream_t s) {
  const int nblocks = a.B * a.H * ((a.G + GPW - 1) / GPW);
  hipLaunchKernelGGL((mass_kernel<D, WPG, GPW>), dim3(nblocks), dim3(64 * WPG * GPW), 0, s, a);
  return hipGetLastError();
}

// top-K of every row of a.mass (a.B * a.H * a.G rows of a.N keys) into a.idx
static hipError_t launch_topk(const SelectArgs &a, hipStream_t s) {
  const dim3 grid(a.B * a.H * a.G);
  if (a.N <= 512 * 8) hipLaunchKernelGGL((topk_reg_kernel<512, 8>), grid, dim3(512), 0, s, a);
  else if (a.N <= 512 * 16) hipLaunchKernelGGL((topk_reg_kernel<512, 16>), grid, dim3(512), 0, s, a);
  else if (a.N <= 512 * 32) hipLaunchKernelGGL((topk_reg_kernel<512, 32>), grid, dim3(512), 0, s, a);
  else if (a.N <= 512 * 64) hipLaunchKernelGGL((topk_reg_kernel<512, 64>), grid, dim3(512), 0, s, a);
  else if (a.N <= 512 * 128) hipLaunchKernelGGL((topk_reg_kernel<512, 128>), grid, dim3(512), 0, s, a);
  // 12 waves, three per SIMD: up to 168 VGPRs, room for 128 keys a lane
  else if (a.N <= 768 * 128) hipLaunchKernelGGL((topk_reg_kernel<768, 128>), grid, dim3(768), 0, s, a);
  else hipLaunchKernelGGL(topk_kernel, grid, dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(int head_dim, const SelectArgs &a, hipStream_t s) {
  const int nblocks = a.B * a.H * a.G;
  if (nblocks <= 0) return hipSuccess;
  hipError_t e;
  if (head_dim == 128 && a.T == 128) e = launch_mass_wide<128, 2, 4, 128>(a, s);
  else if (head_dim == 128 && a.T == 64) e = launch_mass<128, 2, 4>(a, s);
  else if (head_dim == 64 && a.T == 128) e = launch_mass<64, 4, 2>(a, s);
  else if (head_dim == 64 && a.T == 64) e = launch_mass<64, 2, 4>(a, s);
  else return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  return launch_topk(a, s);
}

// ---------------------------------------------------------------------------
// Block-granularity selection (the granularity ablation of the paper landing
// page, Tables 3-4): a block is `blk` consecutive keys; its mass is the sum
// of its keys' exact group mass. Only the N / blk full blocks are candidates.
// ---------------------------------------------------------------------------

// One workgroup per mass row, each wave one block at a time: lane l adds the
// block's keys l, l + 64, ... in order, then a fixed butterfly over the wave.
__global__ __launch_bounds__(256) void block_sum_kernel(const float *mass, int N, int blk, int nfull,
                                                        float *bsum) {
  const int64_t row = blockIdx.x;
  const float *A = mass + row * N;
  float *out = bsum + row * nfull;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int b = wave; b < nfull; b += 4) {
    float x = 0.f;
    for (int j = lane; j < blk; j += 64) x += A[(int64_t)b * blk + j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if (lane == 0) out[b] = x;
  }
}

// kv_idx row = the chosen blocks' keys, block by block (blocks ascending);
// one workgroup per row (a 1-D grid: rows may exceed a grid's y extent)
__global__ __launch_bounds__(256) void block_expand_kernel(const int32_t *bidx, int nb, int blk, int32_t *kv_idx) {
  const int64_t row = blockIdx.x;
  const int K = nb * blk;
  for (int i = threadIdx.x; i < K; i += 256) kv_idx[row * K + i] = bidx[row * nb + i / blk] * blk + i % blk;
}

hipError_t launch_select_blocks(const float *mass, int64_t rows, int N, int blk, int nb, int32_t *kv_idx, void *ws,
                                hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int nfull = N / blk;
  float *bsum = (float *)ws;
  int32_t *bidx = (int32_t *)((char *)ws + select_blocks_bsum_bytes(rows, N, blk));
  hipLaunchKernelGGL(block_sum_kernel, dim3((unsigned)rows), dim3(256), 0, s, mass, N, blk, nfull, bsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SelectArgs a{};
  a.mass = bsum;
  a.idx = bidx;
  a.B = 1;
  a.H = 1;
  a.G = (int32_t)rows;
  a.N = nfull;
  a.K = nb;
  e = launch_topk(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(block_expand_kernel, dim3((unsigned)rows), dim3(256), 0, s, bidx, nb, blk, kv_idx);
  return hipGetLastError();
}

size_t select_blocks_bsum_bytes(int64_t rows, int N, int blk) {
  return ((size_t)rows * (size_t)(N / blk) * sizeof(float) + 255) & ~(size_t)255;
}

size_t select_blocks_ws_bytes(int64_t rows, int N, int blk, int nb) {
  return select_blocks_bsum_bytes(rows, N, blk) + (size_t)rows * nb * sizeof(int32_t);
}

}  // namespace mcs
