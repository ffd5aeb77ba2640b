// Attention kernels on gfx950: anchor dense attention with LSE, reuse-step
// sparse attention over gathered KV (+ cached residual), and the anchor
// residual R = O_dense - O_sparse.
//
// One workgroup owns one tile of query rows: a PDDP query group (sparse,
// residual) or a run of 256 consecutive tokens (dense: eight waves share each
// K/V tile). Each of its waves owns 32 query rows. The key loop walks 64-key
// tiles (128-key tiles on the dense path, 32-key tiles for 64-row groups);
// a tile's K rows and V rows are gathered by index (or read contiguously,
// dense) with LDS-DMA buffer loads straight into one of two LDS stages (the
// next tile fills one stage while the current one is consumed), and consumed
// by v_mfma_f32_32x32x16_bf16:
//   S^T (keys x queries) = K . Q^T        -- D/16 MFMAs per 32-key block
//   O^T (dims x queries) += V^T . P^T     -- P^T comes straight from S^T's
//                                            accumulator layout, no shuffle;
//                                            V^T through transposing LDS reads.
// Online softmax in base 2 (scale * log2 e folded in), fp32 statistics.
// The group modes' R (or O_dense) rows reach LDS by DMA during the last key
// tile, into the stage that tile leaves free, and the epilogue reads them
// from there in the accumulator layout.
//
// MFMA operand layout used (32x32x16): lane l holds row/col (l % 32) and the
// 8 reduction elements of half h = l / 32; accumulator value v of lane l is
// row 8*(v/4) + 4*h + (v%4), col l % 32.
#include <type_traits>

#include "mcs_common.hpp"
#include "mcs_internal.hpp"
#include "mcs_lds.hpp"

namespace mcs {

template <int D, int NW, int KT_>
struct AttnCfg {
  static constexpr int TQ = 32 * NW;           // query rows per workgroup
  static constexpr int NT = 64 * NW;           // threads
  static constexpr int KT = KT_;               // keys per tile
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int ROWB = D * 2;           // bytes per K or V row
  static constexpr int TILEB = KT * ROWB;      // bytes of one K (or V) tile
  static constexpr int LPW = TILEB / 1024 / NW;  // 1 KB LDS-DMA loads per wave per tensor
  static_assert(LPW >= 1 && LPW * NW * 1024 == TILEB, "loader mapping");
};

// The running max is only moved (and O, l rescaled) when a tile's max
// exceeds it by more than this many powers of two; until then the
// exponentials may reach 2^8, which fp32 and bf16 hold exactly as well as 1.
constexpr float kRescaleLog2 = 8.0f;

// Keys per tile: 128 on the 256-row dense path, 32 for the 2-wave (64-row)
// group modes, 64 elsewhere.
template <int NW, int MODE>
constexpr int attn_key_tile() { return MODE == kModeDense && NW >= 8 ? 128 : (MODE != kModeDense && NW == 2 ? 32 : 64); }

// Waves per SIMD the LDS allows: one 8-wave (dense, 256-row) workgroup per
// CU; two 4-wave ones (65 KB each); four 2-wave ones for 64-row groups
// (33 KB each: two 16 KB stages of 32-key tiles); two per CU for the 2-wave
// dense form (32 KB stages), one wave per SIMD.
template <int NW, int MODE>
constexpr int attn_waves_per_simd() { return NW == 4 || (NW == 2 && MODE != kModeDense) ? 2 : 1; }

template <int D, int NW, int MODE>
__global__ __launch_bounds__(64 * NW, (attn_waves_per_simd<NW, MODE>())) void attention_kernel(AttnArgs a) {
  // 128-key tiles on the 256-row dense path (one barrier and DMA wait per
  // 128 keys; its single workgroup per CU has the LDS for them), 64 keys
  // elsewhere
  using C = AttnCfg<D, NW, attn_key_tile<NW, MODE>()>;
  static_assert(MODE == kModeDense || C::KT <= 64, "one index per lane of wave 0 covers a tile");
  // two pipeline stages as separate LDS objects, so the compiler can tell
  // the stage being filled by DMA from the one being read
  __shared__ __attribute__((aligned(1024))) bf16_t st0[2 * C::TILEB / 2];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[2 * C::TILEB / 2];
  __shared__ __attribute__((aligned(16))) uint32_t idx_s[2][C::KT];  // key rows of upcoming tiles
  // group modes: the group's row tokens, for the DMA of R (O_dense) rows
  __shared__ int32_t tok_s[MODE == kModeDense ? 1 : C::TQ];

  const int nblocks = gridDim.x;
  const int work = xcd_remap(blockIdx.x, nblocks);
  const int bh = work / a.G;
  const int g = work - bh * a.G;
  const int b = bh / a.H;
  const int h = bh - b * a.H;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  if (MODE != kModeDense && hh == 0) tok_s[rloc] = token;
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

  uint32_t next_idx = 0;  // wave 0: key row of tile t+2 for this lane
  auto key_row = [&](int t, int j) -> uint32_t {
    if (MODE == kModeDense) {
      const int pos = t * C::KT + j;
      return (uint32_t)(pos < a.N ? pos : a.N - 1);
    }
    return idx_s[t & 1][j];
  };
  auto fetch_idx = [&](int t) {  // wave 0 lane l < KT: index of key t*KT + l
    if (MODE != kModeDense && wave == 0 && lane < C::KT)
      next_idx = __builtin_amdgcn_raw_buffer_load_b32(ri, (t * C::KT + lane) * 4, 0, 0);
  };
  auto store_idx = [&](int t) {
    if (MODE != kModeDense && wave == 0 && lane < C::KT) idx_s[t & 1][lane] = next_idx;
  };
  // DMA tile t's K and V rows into a stage: wave w fills LDS slots
  // [(w*LPW + i)*64, +64) of 16 bytes; slot S is row S/CH, stored chunk S%CH,
  // which holds logical chunk (S%CH) ^ swz(row)
  auto issue = [&](int t, bf16_t *stage) {
#pragma unroll
    for (int i = 0; i < C::LPW; ++i) {
      const int slot = (wave * C::LPW + i) * 64 + lane;
      const int row = slot / C::CH;
      const int chunk = (slot % C::CH) ^ swz<C::CH>(row);
      const uint32_t off = key_row(t, row) * row_bytes + chunk * 16;
      char *kdst = (char *)stage + (wave * C::LPW + i) * 1024;
      buffer_load_lds16(rk, kdst, off);
      buffer_load_lds16(rv, kdst + C::TILEB, off);
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  const bool has_aux = (MODE == kModeResidual) || (MODE == kModeSparse && a.aux != nullptr);
  u32x2 aux[D / 32][4];
  // DMA of the group's R (O_dense) rows into a stage: row r = slot / CH at
  // chunk (slot % CH) ^ swz(r), as the K rows; rows past the group take
  // the first row's token (loaded, never used)
  auto issue_aux = [&](bf16_t *stage) {
    const __amdgpu_buffer_rsrc_t ra = uniform_rsrc(a.aux + head_off, extent);
    constexpr int LPA = C::TQ * C::ROWB / 1024 / NW;  // 1 KB loads per wave
#pragma unroll
    for (int i = 0; i < LPA; ++i) {
      const int slot = (wave * LPA + i) * 64 + lane;
      const int row = slot / C::CH;
      const int chunk = (slot % C::CH) ^ swz<C::CH>(row);
      const uint32_t off = (uint32_t)tok_s[row] * row_bytes + chunk * 16;
      buffer_load_lds16(ra, (char *)stage + (wave * LPA + i) * 1024, off);
    }
  };
  auto read_aux = [&](const bf16_t *stage) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int c = 4 * db + qd;
        aux[db][qd] = *(const u32x2 *)((const char *)stage + rloc * C::ROWB + ((c ^ swz<C::CH>(rloc)) << 4) + 8 * hh);
      }
  };
  float m_run = kNegBig;  // running max, log2 units
  // running row sum, compensated (Kahan): over tens of thousands of keys
  // the mass of the many small probabilities would otherwise fall below
  // half an ulp of the sum and be lost, biasing the LSE low. l_cmp holds
  // minus the part of the added values that l_run could not take up.
  float l_run = 0.f, l_cmp = 0.f;
  const float c2 = a.scale_log2;
  const bool ragged = (nkeys % C::KT) != 0;

  // one key tile on `cur` while `nxt` fills with tile t+1:
  // S^T = K Q^T, online softmax, O^T += V^T P^T
  auto tile = [&](int t, const bf16_t *cur, bf16_t *nxt, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    if (t + 2 < ntiles) fetch_idx(t + 2);
    const bf16_t *ks = cur;
    const bf16_t *vs = cur + C::TILEB / 2;

    // halves A (keys 0..31) and B (32..63): QK(B) is issued next to A's
    // exponentials and PV(A) next to B's max, so MFMA and VALU work of one
    // wave interleave
    f32x16 st[C::KT / 32];
    const int grp = lane >> 4, j = lane & 15;
    const int dim = 16 * (grp & 1) + 4 * (j & 3);
    auto qkh = [&](int kb2) {
      st[kb2] = f32x16{};
      const int r = 32 * kb2 + l32;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 kf = *(const bf16x8 *)(ks + r * D + (((2 * s + hh) ^ swz<C::CH>(r)) << 3));
        st[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[kb2], 0, 0, 0);
      }
      if (LAST && ragged) {
        const int kbase = t * C::KT + 4 * hh + 32 * kb2;
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kbase + 8 * (v >> 2) + (v & 3) >= nkeys) st[kb2][v] = kNegBig;
      }
    };
    auto rescale = [&](int kb2) {
      float mx = st[kb2][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, st[kb2][v]);
      float mlo, mhi;
      cross_half(mx, mlo, mhi);
      const float m_tile = fmaxf(mlo, mhi) * c2;
      if (__any(m_tile > m_run + kRescaleLog2)) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        l_cmp *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      }
    };
    auto exps = [&](int kb2, bf16x8 *pf) {
      const float neg_m = -m_run;
      float lt = 0.f;  // this half tile's 16 values
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(__builtin_fmaf(st[kb2][8 * s2 + e], c2, neg_m));
          lt += p;
          pf[s2][e] = (__bf16)p;
        }
      const float y = lt - l_cmp;
      const float sum = l_run + y;
      l_cmp = (sum - l_run) - y;
      l_run = sum;
    };
    auto pvh = [&](int kb2, const bf16x8 *pf) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int s = 2 * kb2 + s2;
        const int key0 = 16 * s + 4 * hh + (j >> 2);
        const int k1 = key0 + 8;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int dd = 32 * db + dim;
          const s16x4 lo = lds_read_tr16(vs + key0 * D + ((((dd >> 3) ^ swz<C::CH>(key0)) << 3) | (dd & 7)));
          const s16x4 hi = lds_read_tr16(vs + k1 * D + ((((dd >> 3) ^ swz<C::CH>(k1)) << 3) | (dd & 7)));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                                           lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s2], oacc[db], 0, 0, 0);
        }
      }
    };
    if constexpr (C::KT == 32) {
      // 64-row groups: one 32-key half per tile, so that four 2-wave
      // workgroups (two waves per SIMD) fit a CU's LDS; 16-21% faster than
      // 64-key tiles at one wave per SIMD, outputs bitwise equal (the same
      // halves in the same order)
      bf16x8 pfa[2];
      qkh(0);
      if (!LAST) issue(t + 1, nxt);
      if (LAST && MODE != kModeDense && has_aux) issue_aux(nxt);
      rescale(0);
      exps(0, pfa);
      pvh(0, pfa);
    } else if constexpr (C::KT == 64) {
      bf16x8 pfa[2], pfb[2];
      qkh(0);
      // the next tile's DMA (rows from idx_s[(t+1)&1]) goes out once the
      // first half's K reads are issued: its LDS writes then do not compete
      // with them (2% faster than issuing it first); in the last tile the
      // free stage takes the group's R rows instead
      if (!LAST) issue(t + 1, nxt);
      if (LAST && MODE != kModeDense && has_aux) issue_aux(nxt);
      rescale(0);
      qkh(1);
      exps(0, pfa);
      pvh(0, pfa);
      rescale(1);
      exps(1, pfb);
      pvh(1, pfb);
    } else {
      // the same pairing over four 32-key quarters
      bf16x8 pf[C::KT / 32][2];
      qkh(0);
      rescale(0);
#pragma unroll
      for (int k = 1; k < C::KT / 32; ++k) {
        qkh(k);
        // here the next tile's DMA goes out after the third quarter's QK
        // (1% faster than at the tile start; half a tile still hides it)
        if (k == 2 && !LAST) issue(t + 1, nxt);
        exps(k - 1, pf[k - 1]);
        pvh(k - 1, pf[k - 1]);
        rescale(k);
      }
      exps(C::KT / 32 - 1, pf[C::KT / 32 - 1]);
      pvh(C::KT / 32 - 1, pf[C::KT / 32 - 1]);
    }

    if (!LAST) {
      // idx_s[t&1] (tile t's rows) was last read by issue(t) one tile ago
      if (t + 2 < ntiles) store_idx(t + 2);
      // this wave's DMA into `nxt` has landed (vmcnt(0)); then every wave's
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    } else if (MODE != kModeDense && has_aux) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      read_aux(nxt);
    }
  };

  // prologue: rows of tiles 0 and 1, tile 0 into stage 0
  fetch_idx(0);
  store_idx(0);
  fetch_idx(1);
  store_idx(1);
  __syncthreads();
  issue(0, st0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  // stages alternate st0 / st1; unrolled by two so each tile's stage is static
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

  // ---- epilogue -----------------------------------------------------------
  {
    float llo, lhi;
    cross_half(l_run - l_cmp, llo, lhi);
    l_run = llo + lhi;
  }
  if (!row_valid) return;
  const float inv = 1.0f / l_run;
  const int64_t row_off = head_off + (int64_t)token * a.sn;
  bf16_t *orow = a.out + row_off;
  // group modes: R / O_dense came through LDS in the last tile
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = 32 * db + 8 * qd + 4 * hh;
      float o0 = oacc[db][4 * qd + 0] * inv, o1 = oacc[db][4 * qd + 1] * inv;
      float o2 = oacc[db][4 * qd + 2] * inv, o3 = oacc[db][4 * qd + 3] * inv;
      if (has_aux) {
        const u32x2 r = aux[db][qd];
        const float a0 = bf16_to_f32(r[0] & 0xffffu), a1 = bf16_to_f32(r[0] >> 16);
        const float a2 = bf16_to_f32(r[1] & 0xffffu), a3 = bf16_to_f32(r[1] >> 16);
        if (MODE == kModeSparse) {  // O + R
          o0 += a0; o1 += a1; o2 += a2; o3 += a3;
        } else {                    // R = O_dense - O
          o0 = a0 - o0; o1 = a1 - o1; o2 = a2 - o2; o3 = a3 - o3;
        }
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
  // dense: 256-row tiles, so eight waves share each K/V tile's DMA
  if constexpr (MODE == kModeDense) {
    if (head_dim == 128 && a.rows == 256) return launch_one<128, 8, MODE>(a, s);
    if (head_dim == 64 && a.rows == 256) return launch_one<64, 8, MODE>(a, s);
  }
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
