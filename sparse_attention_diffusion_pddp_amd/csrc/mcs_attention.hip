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
#include "mcs_common.hpp"
#include "mcs_internal.hpp"

namespace mcs {

template <int D, int NW>
struct AttnCfg {
  static constexpr int TQ = 32 * NW;          // query rows per workgroup
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int KT = 64;               // keys per tile
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int KPT = KT * CH / NT;    // keys gathered per thread per tile
  static constexpr int KROW = D + 8;          // LDS K row stride (bf16), +16 B pad
  static constexpr int VROW = KT + 4;         // LDS V^T row stride (bf16), +8 B pad
  static constexpr int KTILE = KT * KROW;
  static constexpr int VTILE = D * VROW;
  static constexpr int STAGE = KTILE + VTILE;
  static_assert(NT % CH == 0 && (NT / CH) * KPT == KT, "loader mapping");
  static_assert(KPT == 2 || KPT == 4 || KPT == 8, "transpose width");
};

template <int D, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, (D == 128 && NW == 2) ? 1 : 2) void attention_kernel(AttnArgs a) {
  using C = AttnCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * C::STAGE];

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
  const bf16_t *kb = a.k + head_off;
  const bf16_t *vb = a.v + head_off;

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
  const int32_t *kidx = (MODE == kModeDense) ? nullptr : a.idx + ((int64_t)bh * a.G + g) * a.K;
  const int ntiles = (nkeys + C::KT - 1) / C::KT;

  // loader: thread owns 16-byte chunk column c of keys kg*KPT .. kg*KPT+KPT-1
  const int c = tid % C::CH;
  const int kg = tid / C::CH;

  int ids[C::KPT], ids_next[C::KPT];
  u32x4 kreg[C::KPT], vreg[C::KPT];

  auto load_ids = [&](int t, int *out) {
#pragma unroll
    for (int j = 0; j < C::KPT; ++j) {
      int pos = t * C::KT + kg * C::KPT + j;
      pos = pos < nkeys ? pos : nkeys - 1;  // tail: repeat a valid key, masked later
      out[j] = (MODE == kModeDense) ? pos : kidx[pos];
    }
  };
  auto issue = [&](const int *id) {
#pragma unroll
    for (int j = 0; j < C::KPT; ++j) {
      const int64_t off = (int64_t)id[j] * a.sn + c * 8;
      kreg[j] = *(const u32x4 *)(kb + off);
      vreg[j] = *(const u32x4 *)(vb + off);
    }
  };
  auto commit = [&](int buf) {
    bf16_t *ks = smem + buf * C::STAGE;
    bf16_t *vs = ks + C::KTILE;
#pragma unroll
    for (int j = 0; j < C::KPT; ++j)
      *(u32x4 *)(ks + (kg * C::KPT + j) * C::KROW + c * 8) = kreg[j];
    // transpose: V^T[8c + e][kg*KPT + j]
#pragma unroll
    for (int m = 0; m < 4; ++m) {  // dim pair (8c+2m, 8c+2m+1)
      uint32_t lo[C::KPT / 2], hi[C::KPT / 2];
#pragma unroll
      for (int j = 0; j < C::KPT / 2; ++j) {
        const uint32_t x0 = vreg[2 * j][m], x1 = vreg[2 * j + 1][m];
        lo[j] = (x0 & 0xffffu) | (x1 << 16);
        hi[j] = (x0 >> 16) | (x1 & 0xffff0000u);
      }
      bf16_t *d0 = vs + (8 * c + 2 * m) * C::VROW + kg * C::KPT;
      bf16_t *d1 = d0 + C::VROW;
      if (C::KPT == 2) {
        *(uint32_t *)d0 = lo[0];
        *(uint32_t *)d1 = hi[0];
      } else {
#pragma unroll
        for (int j = 0; j < C::KPT / 2; j += 2) {
          *(u32x2 *)(d0 + 2 * j) = u32x2{lo[j], lo[j + 1]};
          *(u32x2 *)(d1 + 2 * j) = u32x2{hi[j], hi[j + 1]};
        }
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float m_run = kNegBig;
  float l_run = 0.f;

  load_ids(0, ids);
  issue(ids);
  if (ntiles > 1) load_ids(1, ids_next);
  commit(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const bool more = (t + 1) < ntiles;
    if (more) {
      issue(ids_next);
      if (t + 2 < ntiles) load_ids(t + 2, ids_next);
    }
    const bf16_t *ks = smem + (t & 1) * C::STAGE;
    const bf16_t *vs = ks + C::KTILE;

    // S^T = K . Q^T for two 32-key blocks
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

    // online softmax (base 2); this lane's values all belong to query l32
    const int kbase = t * C::KT + 4 * hh;
    float mt = kNegBig;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kbase + 32 * kb2 + 8 * (v >> 2) + (v & 3);
        float x = st[kb2][v] * a.scale_log2;
        x = key < nkeys ? x : kNegBig;
        st[kb2][v] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;

    bf16x8 pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(st[s >> 1][8 * (s & 1) + e] - m_new);
        l_run += p;
        pf[s][e] = (__bf16)p;
      }
    }

    // O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const bf16_t *vrow = vs + (32 * db + l32) * C::VROW + 4 * hh;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x2 lo = *(const u32x2 *)(vrow + 16 * s);
        const u32x2 hi = *(const u32x2 *)(vrow + 16 * s + 8);
        const u32x4 vv = u32x4{lo[0], lo[1], hi[0], hi[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vv), pf[s],
                                                           oacc[db], 0, 0, 0);
      }
    }

    if (more) commit((t + 1) & 1);
    __syncthreads();
  }

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
