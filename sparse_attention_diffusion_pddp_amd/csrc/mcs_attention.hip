// Attention kernels on gfx950: anchor dense attention with LSE, reuse-step
// sparse attention over gathered KV (+ cached residual), and the anchor
// residual R = O_dense - O_sparse.
//
// One workgroup owns one tile of query rows: a PDDP query group (sparse,
// residual) or a run of consecutive tokens (dense). Each of its waves owns 32
// query rows. The key loop walks 64-key tiles; a tile's K rows and V rows are
// gathered by index (or read contiguously, dense) with 16-byte loads, staged
// in LDS (K row-major, V transposed so keys are contiguous) with one tile of
// prefetch in registers, and consumed by v_mfma_f32_32x32x16_bf16:
//   S^T (keys x queries) = K . Q^T        -- D/16 MFMAs per 32-key block
//   O^T (dims x queries) += V^T . P^T     -- P^T comes straight from S^T's
//                                            accumulator layout, no shuffle.
// Online softmax in base 2 (scale * log2 e folded in), fp32 statistics.
//
// MFMA operand layout used (32x32x16): lane l holds row/col (l % 32) and the
// 8 reduction elements of half h = l / 32; accumulator value v of lane l is
// row 8*(v/4) + 4*h + (v%4), col l % 32.
#include <type_traits>

#include "mcs_common.hpp"
#include "mcs_internal.hpp"

namespace mcs {

template <int D, int NW>
struct AttnCfg {
  static constexpr int TQ = 32 * NW;          // query rows per workgroup
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int KT = 64;               // keys per tile
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int KPT = KT * CH / NT;    // keys gathered per thread per tile (K and V each)
  static constexpr int KROW = D + 8;          // LDS K row stride (bf16), +16 B pad
  static constexpr int VROW = KT + 8;         // LDS V^T row stride (bf16), +16 B pad
  static constexpr int KTILE = KT * KROW;
  static constexpr int VTILE = D * VROW;
  static constexpr int STAGE = KTILE + VTILE;
  static_assert(NT % CH == 0 && (NT / CH) * KPT == KT, "loader mapping");
  static_assert(KPT == 2 || KPT == 4 || KPT == 8, "transpose width");
};

// The running max is only moved (and O, l rescaled) when a tile's max
// exceeds it by more than this many powers of two; until then the
// exponentials may reach 2^8, which fp32 and bf16 hold exactly as well as 1.
constexpr float kRescaleLog2 = 8.0f;

// Column of key k (0..63) in the V^T tile: inside each 16-key block the
// quads (4 keys) are stored in the order 0, 2, 1, 3, so that the 8 keys one
// lane feeds to a 16-key MFMA step (keys 4h..4h+3 and 8+4h..8+4h+3) are
// contiguous and one 16-byte LDS read fetches them.
__device__ __forceinline__ int vt_col(int k) {
  const int q = (k >> 2) & 3;
  return (k & ~15) | ((((q & 1) << 1) | (q >> 1)) << 2) | (k & 3);
}

template <int D, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, (D == 128 && NW == 2) ? 1 : 2) void attention_kernel(AttnArgs a) {
  using C = AttnCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * C::STAGE];
  __shared__ __attribute__((aligned(16))) uint32_t idx_s[2][C::KT];  // key rows of the next tiles

  const int nblocks = gridDim.x;
  const int work = xcd_remap(blockIdx.x, nblocks);
  const int bh = work / a.G;
  const int g = work - bh * a.G;
  const int b = bh / a.H;
  const int h = bh - b * a.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const bf16_t *qb = a.q + head_off;
  // byte extent of this head's rows; buffer loads past it return zeros
  const uint32_t row_bytes = (uint32_t)a.sn * 2u;
  const uint32_t extent = (uint32_t)(a.N - 1) * row_bytes + D * 2;
  const __amdgpu_buffer_rsrc_t rk = uniform_rsrc(a.k + head_off, extent);
  const __amdgpu_buffer_rsrc_t rv = uniform_rsrc(a.v + head_off, extent);

  // ---- this lane's query row -------------------------------------------
  const int row0 = g * a.rows;
  const int rloc = wave * 32 + l32;
  const int my_pos = row0 + rloc;
  const bool row_valid = (rloc < a.rows) && (my_pos < a.N);
  int token;
  if (MODE == kModeDense) {
    token = row_valid ? my_pos : (a.N - 1);
  } else {
    const int32_t *pr = a.perm + (int64_t)bh * a.N;
    token = pr[row_valid ? my_pos : row0];
  }
  bf16x8 qf[D / 16];
  {
    const bf16_t *qrow = qb + (int64_t)token * a.sn + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = *(const bf16x8 *)(qrow + 16 * s);
  }

  // ---- key list ---------------------------------------------------------
  const int nkeys = (MODE == kModeDense) ? a.N : a.K;
  const int ntiles = (nkeys + C::KT - 1) / C::KT;
  const int32_t *idx_row = (MODE == kModeDense) ? a.idx : a.idx + ((int64_t)bh * a.G + g) * a.K;
  // past the list the index buffer reads 0 (a valid row, masked later)
  const __amdgpu_buffer_rsrc_t ri = uniform_rsrc(idx_row, (MODE == kModeDense) ? 0u : (uint32_t)a.K * 4u);

  // Loader mappings (KPT consecutive keys x one 16-byte chunk per thread):
  //  K: chunk-minor, so 16 lanes fill one contiguous K row in LDS;
  //  V: key-minor, so 16 lanes fill one contiguous V^T row in LDS
  //     (conflict-free transposed writes).
  const int kc = tid % C::CH, kk = (tid / C::CH) * C::KPT;
  const int vq = tid % (C::KT / C::KPT), vc = tid / (C::KT / C::KPT);
  const int vk = vq * C::KPT;

  u32x4 kreg[C::KPT], vreg[C::KPT];
  uint32_t next_idx = 0;  // wave 0: key row of tile t+2 for this lane

  auto key_row = [&](int t, int j) -> uint32_t {  // rows of tile t: LDS (sparse) or arithmetic (dense)
    if (MODE == kModeDense) {
      const int pos = t * C::KT + j;
      return (uint32_t)(pos < a.N ? pos : a.N - 1);
    }
    return idx_s[t & 1][j];
  };
  auto fetch_idx = [&](int t) {  // wave 0 lane l: index of key t*KT + l
    if (MODE != kModeDense && wave == 0)
      next_idx = __builtin_amdgcn_raw_buffer_load_b32(ri, (t * C::KT + lane) * 4, 0, 0);
  };
  auto store_idx = [&](int t) {
    if (MODE != kModeDense && wave == 0) idx_s[t & 1][lane] = next_idx;
  };
  auto issue = [&](int t) {
#pragma unroll
    for (int j = 0; j < C::KPT; ++j) {
      kreg[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, key_row(t, kk + j) * row_bytes + kc * 16, 0, 0);
      vreg[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, key_row(t, vk + j) * row_bytes + vc * 16, 0, 0);
    }
  };
  auto commit = [&](int buf) {
    bf16_t *ks = smem + buf * C::STAGE;
    bf16_t *vs = ks + C::KTILE;
#pragma unroll
    for (int j = 0; j < C::KPT; ++j)
      *(u32x4 *)(ks + (kk + j) * C::KROW + kc * 8) = kreg[j];
    // transpose into V^T[8*vc + e][vt_col(key)]
#pragma unroll
    for (int m = 0; m < 4; ++m) {  // dim pair (8vc+2m, 8vc+2m+1)
      uint32_t lo[C::KPT / 2], hi[C::KPT / 2];
#pragma unroll
      for (int j = 0; j < C::KPT / 2; ++j) {
        const uint32_t x0 = vreg[2 * j][m], x1 = vreg[2 * j + 1][m];
        lo[j] = (x0 & 0xffffu) | (x1 << 16);
        hi[j] = (x0 >> 16) | (x1 & 0xffff0000u);
      }
      bf16_t *d0 = vs + (8 * vc + 2 * m) * C::VROW;
      bf16_t *d1 = d0 + C::VROW;
      if (C::KPT == 2) {
        const int col = vt_col(vk);
        *(uint32_t *)(d0 + col) = lo[0];
        *(uint32_t *)(d1 + col) = hi[0];
      } else {
#pragma unroll
        for (int j = 0; j < C::KPT / 2; j += 2) {  // one quad of keys per 8-byte write
          const int col = vt_col(vk + 2 * j);
          *(u32x2 *)(d0 + col) = u32x2{lo[j], lo[j + 1]};
          *(u32x2 *)(d1 + col) = u32x2{hi[j], hi[j + 1]};
        }
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = kNegBig;  // running max, log2 units
  float l_run = 0.f;
  const float c2 = a.scale_log2;
  const bool ragged = (nkeys % C::KT) != 0;

  // prologue: indices of tiles 0 and 1 into LDS, tile 0 into stage 0
  fetch_idx(0);
  store_idx(0);
  fetch_idx(1);
  store_idx(1);
  __syncthreads();
  issue(0);
  commit(0);
  __syncthreads();

  // one 64-key tile: S^T = K Q^T, online softmax, O^T += V^T P^T; the key
  // mask exists only in the instantiation for the last tile
  auto tile = [&](int t, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    if (!LAST) issue(t + 1);  // rows from idx_s[(t+1)&1]
    if (t + 2 < ntiles) fetch_idx(t + 2);
    const bf16_t *ks = smem + (t & 1) * C::STAGE;
    const bf16_t *vs = ks + C::KTILE;

    f32x16 st[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      st[kb2] = f32x16{};
      const bf16_t *krow = ks + (32 * kb2 + l32) * C::KROW + 8 * hh;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 kf = *(const bf16x8 *)(krow + 16 * s);
        st[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[kb2], 0, 0, 0);
      }
    }
    if (LAST && ragged) {
      const int kbase = t * C::KT + 4 * hh;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kbase + 32 * kb2 + 8 * (v >> 2) + (v & 3) >= nkeys) st[kb2][v] = kNegBig;
    }

    // online softmax, base 2; every value of this lane belongs to query l32
    float mx = fmaxf(st[0][0], st[1][0]);
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(st[0][v], st[1][v]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_tile = mx * c2;
    if (__any(m_tile > m_run + kRescaleLog2)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
    }
    const float neg_m = -m_run;

    bf16x8 pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(__builtin_fmaf(st[s >> 1][8 * (s & 1) + e], c2, neg_m));
        l_run += p;
        pf[s][e] = (__bf16)p;
      }
    }

#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16_t *vrow = vs + (32 * db + l32) * C::VROW + 8 * hh;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 vf = *(const bf16x8 *)(vrow + 16 * s);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s], oacc[db], 0, 0, 0);
      }
    }

    if (!LAST) commit((t + 1) & 1);
    // idx_s[t&1] (tile t's rows) was last read by issue(t) one tile ago
    if (t + 2 < ntiles) store_idx(t + 2);
    __syncthreads();
  };
  for (int t = 0; t < ntiles - 1; ++t) tile(t, std::false_type{});
  tile(ntiles - 1, std::true_type{});

  // ---- epilogue -----------------------------------------------------------
  l_run += __shfl_xor(l_run, 32);
  if (!row_valid) return;
  const float inv = 1.0f / l_run;
  const int64_t row_off = head_off + (int64_t)token * a.sn;
  bf16_t *orow = a.out + row_off;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = 32 * db + 8 * qd + 4 * hh;
      float o0 = oacc[db][4 * qd + 0] * inv, o1 = oacc[db][4 * qd + 1] * inv;
      float o2 = oacc[db][4 * qd + 2] * inv, o3 = oacc[db][4 * qd + 3] * inv;
      if (MODE == kModeSparse) {
        if (a.aux) {
          const u32x2 r = *(const u32x2 *)(a.aux + row_off + d0);
          o0 += bf16_to_f32(r[0] & 0xffffu);
          o1 += bf16_to_f32(r[0] >> 16);
          o2 += bf16_to_f32(r[1] & 0xffffu);
          o3 += bf16_to_f32(r[1] >> 16);
        }
      } else if (MODE == kModeResidual) {
        const u32x2 od = *(const u32x2 *)(a.aux + row_off + d0);
        o0 = bf16_to_f32(od[0] & 0xffffu) - o0;
        o1 = bf16_to_f32(od[0] >> 16) - o1;
        o2 = bf16_to_f32(od[1] & 0xffffu) - o2;
        o3 = bf16_to_f32(od[1] >> 16) - o3;
      }
      *(u32x2 *)(orow + d0) = u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
    }
  }
  if (MODE == kModeDense && a.lse != nullptr && hh == 0) {
    a.lse[(int64_t)bh * a.N + my_pos] = (m_run + __log2f(l_run)) * kLn2;
  }
}

template <int D, int NW, int MODE>
static hipError_t launch_one(const AttnArgs &a, hipStream_t s) {
  const int nblocks = a.B * a.H * a.G;
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((attention_kernel<D, NW, MODE>), dim3(nblocks), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_mode(int head_dim, const AttnArgs &a, hipStream_t s) {
  if (head_dim == 128 && a.rows == 128) return launch_one<128, 4, MODE>(a, s);
  if (head_dim == 128 && a.rows == 64) return launch_one<128, 2, MODE>(a, s);
  if (head_dim == 64 && a.rows == 128) return launch_one<64, 4, MODE>(a, s);
  if (head_dim == 64 && a.rows == 64) return launch_one<64, 2, MODE>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_attention(int mode, int head_dim, const AttnArgs &a, hipStream_t s) {
  switch (mode) {
    case kModeDense: return launch_mode<kModeDense>(head_dim, a, s);
    case kModeSparse: return launch_mode<kModeSparse>(head_dim, a, s);
    case kModeResidual: return launch_mode<kModeResidual>(head_dim, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mcs
