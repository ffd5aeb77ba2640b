// Fast PDDP query grouping on gfx950 (research walkthrough page, method
// step 1, Figure 6 left): recursive principal-direction splits at the
// tile-aligned median until every node holds at most T queries.
//
// The tree's shape depends only on (N, T): a node of n tokens with
// G_S = ceil(n/T) > 1 sends its first floor(G_S/2)*T tokens (in projection
// order) left. So the node ranges of every level are planned up front and
// `perm` itself is the working array: it starts as the identity and each
// level stably partitions every active node's range in place, which keeps
// every node (and finally every group) in ascending token order.
//
// Second moments are additive, so a split's children need only one pass:
// the moments of the left child (never larger than the right one) are
// accumulated from its tokens and the right child's are the parent's minus
// the left's. Every moment is taken about one fixed point per head, the
// head's token 0 (c), so that x - c is exact and the moments stay small for
// data with a common offset: s = sum (x - c), S = sum (x - c)(x - c)^T, and a
// node's covariance is S/n - m m^T with m = s/n, its mean c + m.
//
// Per level, over all heads and nodes at once:
//   moment   per chunk of a unit (a range whose moments are accumulated):
//            s and the upper-triangle 16x16 tiles of S on the fp64 MFMA
//            (v_mfma_f64_16x16x4_f64)                            -> partials
//            (its accumulator: lane l, register i holds row l/16 + 4i,
//            column l % 16; operands: lane l holds row/col l % 16, k = l/16)
//   reduce   (levels whose units span more than 4 chunks) partials of a
//            unit added in chunk order, sliced over many blocks
//   power    per node: its moments (unit, or parent minus unit), kept for
//            the next level when its right child is split again; the
//            covariance, power iteration from e_{argmax diag}, orientation
//            -> mu, u
//   project  per chunk of a node: p_i = (q_i - mu) . u in float64
//   split    per node: radix select of the floor(G_S/2)*T-th smallest
//            (p, position) and a stable partition of the node's range.
// Whitened grouping (an open item of the authors on the news page; read as
// per-dimension standardization) runs the same tree on the queries scaled by
// w_d = 1/sigma_d of the root: every node's covariance becomes w_i C_ij w_j,
// its direction is reported as w_d u_d in the queries' own coordinates, and
// the root's start index is the lowest dimension of nonzero variance.
//
// All sums run in a fixed order, so the result is bitwise reproducible, and
// decisions are taken on float64 values so the split does not hinge on fp32
// rounding. Level 0 needs neither the plan nor perm (its one unit is the
// whole sequence in token order): its moment kernel writes the identity perm
// and one extra block builds the plan tables meanwhile.
#include <vector>

#include "mcs_common.hpp"
#include "mcs_internal.hpp"
#include "mcs_radix.hpp"

namespace mcs {

namespace {

constexpr int kChunk0 = 512;     // tokens per moment chunk at level 0
constexpr int kChunk = 256;      // tokens per moment chunk below level 0
constexpr int kChunk0Shift = 9, kChunkShift = 8;
static_assert((1 << kChunk0Shift) == kChunk0 && (1 << kChunkShift) == kChunk, "chunk sizes are powers of two");
constexpr int kPChunk = 256;     // tokens per projection chunk
constexpr int kDirectChunks = 4; // a unit of at most this many chunks is summed by the power kernel
constexpr int kMaxLevels = 40;
constexpr int kSplitThreads = 512;

struct PLevel {
  int node0, nnodes;     // nodes (more than T tokens) split at this level
  int unit0, nunits;     // units whose moments this level accumulates
  int mchunk0, nmchunks; // moment chunks (over units)
  int pchunk0, npchunks; // projection chunks (over nodes)
  int reduced;           // 1: a reduce pass adds the units' partials
  int maxn;              // largest node of the level (tokens)
};
struct PNode {
  int off, n, nl;
  int unit;      // level-local unit: the node's own range, or its left sibling's
  int derived;   // 1: moments = parent's - unit's (a right child)
  int kid_unit;  // next-level unit of its children when the right child is split again, else -1
};
struct PUnit {
  int off, n, chunk0, nchunks;  // chunk0: level-local index of its first moment chunk
};
struct PChunk {
  int owner, off, len;  // owner: level-local unit (moment) or node (projection)
};

struct PlanCounts {
  int levels, nodes, units, mchunks, pchunks;
  int max_nodes, max_units, max_runits, max_mchunks, max_pchunks;
};

// Builds the level / node / unit / chunk tables. `nd` and `un` must hold at
// least 2*G + 2 entries; `lv`, `mc` and `pc` may be null to only count.
__host__ __device__ PlanCounts plan_tree(int N, int T, PLevel *lv, PNode *nd, PUnit *un, PChunk *mc,
                                         PChunk *pc) {
  PlanCounts k{};
  if (N <= T) return k;
  // T and the chunk sizes are powers of two: shifts instead of divisions,
  // which on the GPU are long instruction sequences in a serial walk
  int tsh = 0;
  while ((1 << tsh) < T) ++tsh;
  // active nodes (more than T tokens) are appended level by level, so the
  // nodes of one level are contiguous; so are the units; level 0 is the root
  nd[0] = PNode{0, N, 0, 0, 0, -1};
  un[0] = PUnit{0, N, 0, 0};
  int lb = 0, le = 1, ub = 0, ue = 1;
  while (lb < le) {
    const int cs = k.levels == 0 ? kChunk0 : kChunk;
    const int csh = k.levels == 0 ? kChunk0Shift : kChunkShift;
    int nm = 0, most = 0;
    for (int u = ub; u < ue; ++u) {
      PUnit x = un[u];
      x.chunk0 = nm;
      x.nchunks = (x.n + cs - 1) >> csh;
      if (mc)
        for (int c = 0; c < x.nchunks; ++c) {
          const int rest = x.n - c * cs;
          mc[k.mchunks + nm + c] = PChunk{u - ub, x.off + c * cs, rest < cs ? rest : cs};
        }
      nm += x.nchunks;
      most = most > x.nchunks ? most : x.nchunks;
      un[u] = x;
    }
    int np = 0, nle = le, nue = ue, maxn = 0;
    for (int i = lb; i < le; ++i) {
      PNode x = nd[i];
      maxn = maxn > x.n ? maxn : x.n;
      const int G = (x.n + T - 1) >> tsh;
      x.nl = (G >> 1) << tsh;
      const int nr = x.n - x.nl;  // nr >= nl: the right child is the larger
      const int npc = (x.n + kPChunk - 1) / kPChunk;
      if (pc)
        for (int c = 0; c < npc; ++c) {
          const int rest = x.n - c * kPChunk;
          pc[k.pchunks + np + c] = PChunk{i - lb, x.off + c * kPChunk, rest < kPChunk ? rest : kPChunk};
        }
      np += npc;
      x.kid_unit = -1;
      if (nr > T) {
        x.kid_unit = nue - ue;
        un[nue++] = PUnit{x.off, x.nl, 0, 0};
        if (x.nl > T) nd[nle++] = PNode{x.off, x.nl, 0, x.kid_unit, 0, -1};
        nd[nle++] = PNode{x.off + x.nl, nr, 0, x.kid_unit, 1, -1};
      }
      nd[i] = x;
    }
    const int red = most > kDirectChunks ? 1 : 0;
    if (lv) lv[k.levels] = PLevel{lb, le - lb, ub, ue - ub, k.mchunks, nm, k.pchunks, np, red, maxn};
    const int nn = le - lb, nu = ue - ub;
    k.max_nodes = k.max_nodes > nn ? k.max_nodes : nn;
    k.max_units = k.max_units > nu ? k.max_units : nu;
    if (red) k.max_runits = k.max_runits > nu ? k.max_runits : nu;
    k.max_mchunks = k.max_mchunks > nm ? k.max_mchunks : nm;
    k.max_pchunks = k.max_pchunks > np ? k.max_pchunks : np;
    k.mchunks += nm;
    k.pchunks += np;
    k.levels++;
    lb = le;
    le = nle;
    ub = ue;
    ue = nue;
  }
  k.nodes = le;
  k.units = ue;
  return k;
}

// Stores of the parallel plan builder, and its per-level sanity check: a
// checked build (the plan is compared with the serial walk on many shapes)
// redefines both to bounds-check every store and stop a runaway walk.
#ifndef MCS_PLAN_STORE
#define MCS_PLAN_STORE(arr, idx, val) ((arr)[idx] = (val))
#endif
#ifndef MCS_PLAN_BAD
#define MCS_PLAN_BAD(le, ue, level) false
#endif

// Block-wide exclusive sum of one int per thread of a 256-thread block; the
// total goes to *total. sh holds 4 ints and is free again on return.
__device__ __forceinline__ int block_excl_scan(int v, int *total, int *sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = sh[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

__device__ __forceinline__ int block_max(int v, int *sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  const int m = max(max(sh[0], sh[1]), max(sh[2], sh[3]));
  __syncthreads();
  return m;
}

// plan_tree's tables built by a 256-thread block, one level at a time: every
// unit and node of the level is handled by its own thread, and block scans
// place their chunks and children exactly where the serial walk puts them
// (same tables, same order). The lists nd / un may be in LDS or in global
// memory; counts[0], counts[1] receive the numbers of nodes and units.
// Requires N > T, T a power of two, and nd / un of 2G + 2 entries.
__device__ void plan_tree_par(int N, int T, PLevel *lv, PNode *nd, PUnit *un, PChunk *mc, PChunk *pc,
                              int *counts) {
  __shared__ int sh[4];
  const int tid = threadIdx.x;
  int tsh = 0;
  while ((1 << tsh) < T) ++tsh;
  if (tid == 0) {
    nd[0] = PNode{0, N, 0, 0, 0, -1};
    un[0] = PUnit{0, N, 0, 0};
  }
  __syncthreads();
  int lb = 0, le = 1, ub = 0, ue = 1, level = 0, mtot = 0, ptot = 0;
  while (lb < le) {
    if (MCS_PLAN_BAD(le, ue, level)) break;
    const int cs = level == 0 ? kChunk0 : kChunk;
    const int csh = level == 0 ? kChunk0Shift : kChunkShift;
    int nm = 0, most = 0;
    for (int base = ub; base < ue; base += 256) {
      const int u = base + tid;
      const bool ok = u < ue;
      PUnit x = ok ? un[u] : PUnit{0, 0, 0, 0};
      const int nch = ok ? (x.n + cs - 1) >> csh : 0;
      int tot;
      const int ex = block_excl_scan(nch, &tot, sh);
      if (ok) {
        x.chunk0 = nm + ex;
        x.nchunks = nch;
        un[u] = x;
        for (int c = 0; c < nch; ++c) {
          const int rest = x.n - c * cs;
          MCS_PLAN_STORE(mc, mtot + nm + ex + c, (PChunk{u - ub, x.off + c * cs, rest < cs ? rest : cs}));
        }
      }
      most = max(most, block_max(nch, sh));
      nm += tot;
    }
    int np = 0, nu_new = 0, nn_new = 0, maxn = 0;
    for (int base = lb; base < le; base += 256) {
      const int i = base + tid;
      const bool ok = i < le;
      PNode x = ok ? nd[i] : PNode{0, 0, 0, 0, 0, -1};
      const int G = (x.n + T - 1) >> tsh;
      x.nl = (G >> 1) << tsh;
      const int nr = x.n - x.nl;
      const int npc = ok ? (x.n + kPChunk - 1) / kPChunk : 0;
      const int kid = (ok && nr > T) ? 1 : 0;
      const int left = (kid && x.nl > T) ? 1 : 0;
      int tp, tu, tn;
      const int ep = block_excl_scan(npc, &tp, sh);
      const int eu = block_excl_scan(kid, &tu, sh);
      const int en = block_excl_scan(kid + left, &tn, sh);
      const int mx = block_max(ok ? x.n : 0, sh);
      if (ok) {
        for (int c = 0; c < npc; ++c) {
          const int rest = x.n - c * kPChunk;
          MCS_PLAN_STORE(pc, ptot + np + ep + c, (PChunk{i - lb, x.off + c * kPChunk, rest < kPChunk ? rest : kPChunk}));
        }
        x.kid_unit = -1;
        if (kid) {
          x.kid_unit = nu_new + eu;
          MCS_PLAN_STORE(un, ue + x.kid_unit, (PUnit{x.off, x.nl, 0, 0}));
          int pos = le + nn_new + en;
          if (left) MCS_PLAN_STORE(nd, pos++, (PNode{x.off, x.nl, 0, x.kid_unit, 0, -1}));
          MCS_PLAN_STORE(nd, pos, (PNode{x.off + x.nl, nr, 0, x.kid_unit, 1, -1}));
        }
        nd[i] = x;
      }
      np += tp;
      nu_new += tu;
      nn_new += tn;
      maxn = max(maxn, mx);
    }
    if (tid == 0) MCS_PLAN_STORE(lv, level, (PLevel{lb, le - lb, ub, ue - ub, mtot, nm, ptot, np, most > kDirectChunks ? 1 : 0, maxn}));
    mtot += nm;
    ptot += np;
    ++level;
    lb = le;
    le += nn_new;
    ub = ue;
    ue += nu_new;
    __syncthreads();
  }
  if (tid == 0) {
    counts[0] = le;
    counts[1] = ue;
  }
}

inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// doubles per moment block: the upper-triangle tiles of S, then s
constexpr int moment_doubles(int D) { return (D / 16) * (D / 16 + 1) / 2 * 256 + D; }

// Upper-triangle tile t (row-major over (bi, bj), bi <= bj) of an NB x NB
// grid of 16-wide dim blocks: its row block bi and column block bj.
constexpr int tile_bi(int t, int NB) {
  int bi = 0;
  while (bi < NB && t >= NB - bi) {
    t -= NB - bi;
    ++bi;
  }
  return bi < NB ? bi : 0;
}
constexpr int tile_bj(int t, int NB) {
  int bi = 0;
  while (bi < NB && t >= NB - bi) {
    t -= NB - bi;
    ++bi;
  }
  return bi < NB ? bi + t : 0;
}

struct WsLayout {
  size_t levels, nodes, units, mchunks, pchunks, part, ured, nodem, mu, dir, proj, tmp, wscale, total;
};

WsLayout ws_layout(const PlanCounts &pc, int BH, int N, int D) {
  WsLayout w{};
  const size_t MB = (size_t)moment_doubles(D);
  auto at_least1 = [](int x) { return (size_t)(x > 0 ? x : 1); };
  size_t o = 0;
  w.levels = o; o = align_up(o + sizeof(PLevel) * kMaxLevels);
  w.nodes = o; o = align_up(o + sizeof(PNode) * at_least1(pc.nodes));
  w.units = o; o = align_up(o + sizeof(PUnit) * at_least1(pc.units));
  w.mchunks = o; o = align_up(o + sizeof(PChunk) * at_least1(pc.mchunks));
  w.pchunks = o; o = align_up(o + sizeof(PChunk) * at_least1(pc.pchunks));
  w.part = o; o = align_up(o + sizeof(double) * (size_t)BH * at_least1(pc.max_mchunks) * MB);
  w.ured = o; o = align_up(o + sizeof(double) * (size_t)BH * at_least1(pc.max_runits) * MB);
  w.nodem = o; o = align_up(o + sizeof(double) * 2 * (size_t)BH * at_least1(pc.max_units) * MB);
  w.mu = o; o = align_up(o + sizeof(double) * (size_t)BH * at_least1(pc.max_nodes) * D);
  w.dir = o; o = align_up(o + sizeof(double) * (size_t)BH * at_least1(pc.max_nodes) * D);
  w.proj = o; o = align_up(o + sizeof(double) * (size_t)BH * N);
  w.tmp = o; o = align_up(o + sizeof(int32_t) * (size_t)BH * N);
  w.wscale = o; o = align_up(o + sizeof(double) * (size_t)BH * D);
  w.total = o;
  return w;
}

// Host-side plan with real node / unit arrays (counting needs the ranges).
PlanCounts host_plan(int N, int T, PLevel *lv) {
  if (N <= T) return PlanCounts{};
  const int G = (N + T - 1) / T;
  std::vector<PNode> nd(2 * G + 2);
  std::vector<PUnit> un(2 * G + 2);
  return plan_tree(N, T, lv, nd.data(), un.data(), nullptr, nullptr);
}

struct PddpArgs {
  const uint16_t *q;
  int64_t sb, sn, sh;
  int B, H, N, T;
  int32_t *perm;
  PLevel *levels;
  PNode *nodes;
  PUnit *units;
  PChunk *mchunks, *pchunks;
  double *part, *ured, *nodem, *mu, *dir, *proj;
  double *wscale;  // whitening: per-head 1/sigma_d of the root (1 where sigma_d = 0)
  int32_t *tmp;
  int max_mchunks, max_runits, max_units, max_nodes;
  int level;
  int power_iters;
  int whiten;
  int plan_in_lds;  // the level-0 plan block keeps its node / unit lists in dynamic LDS
};

// bytes of the plan's node and unit lists (2G + 2 entries each)
__host__ __device__ inline size_t plan_list_bytes(int N, int T) {
  const size_t n = 2 * (size_t)((N + T - 1) / T) + 2;
  return ((n * sizeof(PNode) + 15) & ~(size_t)15) + n * sizeof(PUnit);
}

// The level-0 plan block: plan_tree_par on the node and unit lists in LDS
// (copied out by the whole block at the end) when they fit in the dynamic
// LDS the launch gave it, else on the global lists.
__device__ void build_plan(const PddpArgs &a, char *lds) {
  __shared__ int counts[2];
  if (!a.plan_in_lds) {
    plan_tree_par(a.N, a.T, a.levels, a.nodes, a.units, a.mchunks, a.pchunks, counts);
    return;
  }
  const size_t n = 2 * (size_t)((a.N + a.T - 1) / a.T) + 2;
  PNode *nd = (PNode *)lds;
  PUnit *un = (PUnit *)(lds + ((n * sizeof(PNode) + 15) & ~(size_t)15));
  plan_tree_par(a.N, a.T, a.levels, nd, un, a.mchunks, a.pchunks, counts);
  __syncthreads();
  for (int i = threadIdx.x; i < counts[0]; i += blockDim.x) a.nodes[i] = nd[i];
  for (int i = threadIdx.x; i < counts[1]; i += blockDim.x) a.units[i] = un[i];
}

__global__ void init_perm_kernel(int32_t *perm, int N, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) perm[i] = (int32_t)(i % N);
}

__device__ __forceinline__ const uint16_t *head_q(const PddpArgs &a, int bh) {
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  return a.q + (int64_t)b * a.sb + (int64_t)h * a.sh;
}

// ---- moment partials: grid (chunks [+1 at level 0], BH), 256 threads ----------
// Tokens are staged through LDS as float64 (x - c), SUB at a time, the next
// SUB rows already loaded into registers while the MFMAs run on these.
template <int D, bool L0>
__global__ __launch_bounds__(256, 2) void moment_kernel(PddpArgs a) {
  constexpr int NB = D / 16;                 // 16-wide dim blocks
  constexpr int NT = NB * (NB + 1) / 2;      // upper-triangle tiles
  constexpr int TPW = (NT + 3) / 4;          // tiles per wave (at most)
  constexpr int MB = moment_doubles(D);
  constexpr int SUB = 32;                    // tokens staged per step
  // LDS row stride (doubles): D + 16 puts consecutive token rows 32 banks
  // apart, so the two 16-lane row groups of a 32-lane half of an operand
  // read hit disjoint banks (D + 1 shifted rows by 2 banks: 1.70 -> 1.62 ms
  // per wan480p call with D + 16, identical groups)
  constexpr int XS = D + 16;
  constexpr int CH = D / 8;                  // 16-byte pieces per row
  constexpr int TL = 256 / CH;               // token lanes
  constexpr int RPT = SUB / TL;              // staged rows per thread
  static_assert(RPT >= 1 && SUB % TL == 0 && TL <= SUB, "staging shape");
  __shared__ double X[SUB * XS];
  extern __shared__ __attribute__((aligned(16))) char plan_lds[];  // level 0: the plan's lists

  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int32_t *cur = a.perm + (int64_t)bh * a.N;
  int off, len;
  if (L0) {
    const int nch = (a.N + kChunk0 - 1) / kChunk0;
    if ((int)blockIdx.x == nch) {
      if (bh == 0) build_plan(a, plan_lds);
      return;
    }
    off = blockIdx.x * kChunk0;
    len = a.N - off < kChunk0 ? a.N - off : kChunk0;
    for (int i = tid; i < len; i += 256) cur[off + i] = off + i;
  } else {
    const PChunk c = a.mchunks[a.levels[a.level].mchunk0 + blockIdx.x];
    off = c.off;
    len = c.len;
  }
  const uint16_t *qh = head_q(a, bh);
  const int col = tid % CH, tl = tid / CH;

  float cv[8];  // token 0 of the head (bf16 values: exact as float)
  {
    const u32x4 v = *(const u32x4 *)(qh + col * 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      cv[2 * m] = bf16_to_f32(v[m] & 0xffffu);
      cv[2 * m + 1] = bf16_to_f32(v[m] >> 16);
    }
  }
  double sx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // wave w owns the upper-triangle tiles t = 4k + w (t enumerates (bi, bj),
  // bi <= bj, row-major); acc[k] accumulates tile 4k + w (fixed
  // accumulators, no branches in the MFMA loop)
  f64x4 acc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) acc[k] = f64x4{0, 0, 0, 0};

  u32x4 pre[RPT];
  bool ok[RPT];
  auto fetch = [&](int base) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = base + tl + TL * r;
      ok[r] = i < len;
      const int tok = L0 ? off + (ok[r] ? i : 0) : cur[off + (ok[r] ? i : 0)];
      pre[r] = *(const u32x4 *)(qh + (int64_t)tok * a.sn + col * 8);
    }
  };
  fetch(0);
  for (int base = 0; base < len; base += SUB) {
    // stage x - c for SUB tokens; rows past the chunk are zero
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      double x[8];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[2 * m] = ok[r] ? (double)bf16_to_f32(pre[r][m] & 0xffffu) - (double)cv[2 * m] : 0.0;
        x[2 * m + 1] = ok[r] ? (double)bf16_to_f32(pre[r][m] >> 16) - (double)cv[2 * m + 1] : 0.0;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sx[e] += x[e];
        X[(tl + TL * r) * XS + col * 8 + e] = x[e];
      }
    }
    __syncthreads();
    if (base + SUB < len) fetch(base + SUB);
    const int steps = (len - base) < SUB ? ((len - base + 3) / 4) : SUB / 4;
    // A tile's A operand (dims 16 bi.., 4 tokens) and B operand (dims
    // 16 bj..) are the same lane values as the one-block operand of block
    // bi or bj: lane l holds x[token l / 16][16 b + l % 16]. So a step reads
    // the NB blocks once and each of the wave's tiles takes two of them. The
    // wave's tile list is made static per wave (a uniform switch), so the
    // operands are fixed registers.
    auto run = [&](auto wtag) {
      constexpr int W = decltype(wtag)::value;
      for (int s = 0; s < steps; ++s) {
        const double *xr = X + (4 * s + (lane >> 4)) * XS + (lane & 15);
        double v[NB];
#pragma unroll
        for (int bk = 0; bk < NB; ++bk) v[bk] = xr[16 * bk];
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
          if (4 * k + W < NT)
            acc[k] = __builtin_amdgcn_mfma_f64_16x16x4f64(v[tile_bi(4 * k + W, NB)], v[tile_bj(4 * k + W, NB)],
                                                          acc[k], 0, 0, 0);
        }
      }
    };
    switch (wave) {
      case 0: run(std::integral_constant<int, 0>{}); break;
      case 1: run(std::integral_constant<int, 1>{}); break;
      case 2: run(std::integral_constant<int, 2>{}); break;
      default: run(std::integral_constant<int, 3>{}); break;
    }
    __syncthreads();
  }
  // s: add the token lanes' sums in lane order
#pragma unroll
  for (int e = 0; e < 8; ++e) X[tl * XS + col * 8 + e] = sx[e];
  __syncthreads();
  double *out = a.part + ((int64_t)bh * a.max_mchunks + blockIdx.x) * MB;
  if (tid < D) {
    double s = 0.0;
    for (int t = 0; t < TL; ++t) s += X[t * XS + tid];
    out[NT * 256 + tid] = s;
  }
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = 4 * k + wave;
    if (t < NT) {
#pragma unroll
      for (int i = 0; i < 4; ++i)  // f64 MFMA: row = lane/16 + 4*i, column = lane % 16
        out[t * 256 + ((lane >> 4) + 4 * i) * 16 + (lane & 15)] = acc[k][i];
    }
  }
}

// ---- unit moments: grid (units * slices, BH), 256 threads -------------------
// Entry e of a unit's moments = its chunks' partials added in chunk order.
template <int D>
__global__ __launch_bounds__(256) void reduce_kernel(PddpArgs a) {
  constexpr int MB = moment_doubles(D);
  constexpr int NSL = (MB + 255) / 256;
  const PLevel L = a.levels[a.level];
  const int u = blockIdx.x / NSL, e = (blockIdx.x - u * NSL) * 256 + threadIdx.x;
  const int bh = blockIdx.y;
  if (e >= MB) return;
  const PUnit U = a.units[L.unit0 + u];
  const double *src = a.part + ((int64_t)bh * a.max_mchunks + U.chunk0) * MB + e;
  double s = 0.0;
  int k = 0;
  for (; k + 8 <= U.nchunks; k += 8) {
    double v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = src[(int64_t)(k + i) * MB];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
  }
  for (; k < U.nchunks; ++k) s += src[(int64_t)k * MB];
  a.ured[((int64_t)bh * a.max_runits + u) * MB + e] = s;
}

// ---- node direction: grid (nnodes, BH), 256 threads -------------------------
// A double moved across lanes by a DPP pattern (two 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long bits = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)bits, CTRL, 0xF, 0xF, false);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(bits >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const unsigned long long bits = (unsigned long long)__double_as_longlong(x);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)bits, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(bits >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}
// Sum over the 64 lanes of a wave, returned to every lane: the quads by two
// DPP quad permutes, the 16-lane rows by two DPP rotations (VALU steps, no
// LDS round trip like a shuffle's), then the rows' sums read from lanes 0,
// 16, 32 and 48 and added in a fixed order, so every lane and wave of equal
// data gets the same bits.
__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp_f64<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f64<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f64<0x124>(x);  // row_ror:4
  x += dpp_f64<0x128>(x);  // row_ror:8
  return (readlane_f64(x, 0) + readlane_f64(x, 16)) + (readlane_f64(x, 32) + readlane_f64(x, 48));
}

// (value, index) max over a wave, lowest index among equal values
__device__ __forceinline__ void wave_argmax(double &v, int &j) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) {
    const double ov = __shfl_xor(v, s);
    const int oj = __shfl_xor(j, s);
    if (ov > v || (ov == v && oj < j)) {
      v = ov;
      j = oj;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void power_kernel(PddpArgs a) {
  constexpr int NB = D / 16;
  constexpr int NT = NB * (NB + 1) / 2;
  constexpr int MB = moment_doubles(D);
  constexpr int PARTS = 256 / D;    // threads per column in the matrix-vector product
  constexpr int JPP = D / PARTS;    // rows per part
  constexpr int CS = 33;            // row stride (doubles) of the 32-column exchange buffer
  __shared__ double Cb[D * CS];
  __shared__ double u[D], wpart[PARTS][D], mvec[D], diag[D], wsc[D];
  __shared__ int jstar;
  const PLevel L = a.levels[a.level];
  const int bh = blockIdx.y;
  const int ln = blockIdx.x;
  const PNode nd = a.nodes[L.node0 + ln];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  double creg[JPP];  // this thread's rows of one column of C (filled below)
  // the node's moments: its unit's (partials added in chunk order, or the
  // reduce pass's sum), minus from the parent's for a right child; entry
  // m * 256 + tid of the moment block is this thread's, m <= NT (m == NT: s)
  {
    double val[NT + 1];
    const bool has_s = tid < D;
    if (L.reduced) {
      const double *src = a.ured + ((int64_t)bh * a.max_runits + nd.unit) * MB + tid;
#pragma unroll
      for (int m = 0; m < NT; ++m) val[m] = src[m * 256];
      val[NT] = has_s ? src[NT * 256] : 0.0;
    } else {
      const PUnit U = a.units[L.unit0 + nd.unit];
      const double *src = a.part + ((int64_t)bh * a.max_mchunks + U.chunk0) * MB + tid;
#pragma unroll
      for (int m = 0; m <= NT; ++m) val[m] = 0.0;
      for (int k = 0; k < U.nchunks; ++k) {
        const double *p = src + (int64_t)k * MB;
        double v[NT + 1];
#pragma unroll
        for (int m = 0; m < NT; ++m) v[m] = p[m * 256];
        v[NT] = has_s ? p[NT * 256] : 0.0;
#pragma unroll
        for (int m = 0; m <= NT; ++m) val[m] += v[m];
      }
    }
    if (nd.derived) {
      const double *par = a.nodem + (((int64_t)(a.level & 1) * a.B * a.H + bh) * a.max_units + nd.unit) * MB + tid;
      double v[NT + 1];
#pragma unroll
      for (int m = 0; m < NT; ++m) v[m] = par[m * 256];
      v[NT] = has_s ? par[NT * 256] : 0.0;
#pragma unroll
      for (int m = 0; m <= NT; ++m) val[m] = v[m] - val[m];
    }
    if (nd.kid_unit >= 0) {
      double *dst = a.nodem + (((int64_t)((a.level + 1) & 1) * a.B * a.H + bh) * a.max_units + nd.kid_unit) * MB + tid;
#pragma unroll
      for (int m = 0; m < NT; ++m) dst[m * 256] = val[m];
      if (has_s) dst[NT * 256] = val[NT];
    }
    const double inv_n = 1.0 / (double)nd.n;
    if (has_s) mvec[tid] = val[NT] * inv_n;
    __syncthreads();
    // covariance S/n - m m^T, upper tiles, in place
    const int r = tid >> 4, c = tid & 15;
    int m = 0;
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
#pragma unroll
      for (int bj = bi; bj < NB; ++bj, ++m) {
        const int gi = 16 * bi + r, gj = 16 * bj + c;
        val[m] = val[m] * inv_n - mvec[gi] * mvec[gj];
        if (bi == bj && r == c) diag[gi] = val[m];
      }
    }
    // the node's mean for the projection kernel: c + m
    if (has_s) {
      const uint16_t *qh = head_q(a, bh);
      a.mu[((int64_t)bh * a.max_nodes + ln) * D + tid] = (double)bf16_to_f32(qh[tid]) + mvec[tid];
    }
    __syncthreads();
    if (a.whiten) {
      // per-dimension standardization: the root's variances give
      // w_d = 1/sigma_d (1 for a zero variance), kept for the deeper levels;
      // the node's covariance becomes w_i C_ij w_j
      if (tid < D) {
        double w;
        if (a.level == 0) {
          const double v = diag[tid];
          w = v > 0.0 ? 1.0 / sqrt(v) : 1.0;
          a.wscale[(int64_t)bh * D + tid] = w;
        } else {
          w = a.wscale[(int64_t)bh * D + tid];
        }
        wsc[tid] = w;
      }
      __syncthreads();
      int mw = 0;
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
#pragma unroll
        for (int bj = bi; bj < NB; ++bj, ++mw) {
          const int gi = 16 * bi + r, gj = 16 * bj + c;
          val[mw] *= wsc[gi] * wsc[gj];
          if (bi == bj && r == c) diag[gi] = val[mw];
        }
      }
      __syncthreads();
    }
    // start vector: e_j for the largest diagonal entry (lowest j on ties).
    // Whitened root: every standardized variance is 1 in exact arithmetic,
    // so the tie rule's answer, the lowest dimension of nonzero variance, is
    // taken exactly (0 when every variance is 0).
    if (wave == 0) {
      if (a.whiten && a.level == 0) {
        const uint64_t nz0 = __ballot(diag[lane] > 0.0);
        const uint64_t nz1 = D > 64 ? __ballot(diag[(lane + 64) % D] > 0.0) : 0ull;
        if (lane == 0) jstar = nz0 ? __ffsll((unsigned long long)nz0) - 1
                                   : (nz1 ? 64 + __ffsll((unsigned long long)nz1) - 1 : 0);
      } else {
        double v = diag[lane];
        int j = lane;
        if (D > 64) {
          const double v2 = diag[lane + 64];
          if (v2 > v) {
            v = v2;
            j = lane + 64;
          }
        }
        wave_argmax(v, j);
        if (lane == 0) jstar = j;
      }
    }
    // thread (part, col) keeps rows part, part + PARTS, ... of column col of
    // C in registers for all iterations (C is symmetric: column = row). C
    // reaches them 32 columns at a time through Cb: the upper tiles as they
    // are, the lower ones mirrored, so a block needs 33 KB of LDS, not
    // 128 KB, and two blocks share a CU.
#pragma unroll
    for (int pc = 0; pc < D / 32; ++pc) {
      int mt = 0;
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
#pragma unroll
        for (int bj = bi; bj < NB; ++bj, ++mt) {
          const int gi = 16 * bi + r, gj = 16 * bj + c;
          if ((bj >> 1) == pc) Cb[gi * CS + (gj - 32 * pc)] = val[mt];
          if (bi != bj && (bi >> 1) == pc) Cb[gj * CS + (gi - 32 * pc)] = val[mt];
        }
      }
      __syncthreads();
      if (((tid % D) >> 5) == pc) {
#pragma unroll
        for (int mm = 0; mm < JPP; ++mm) creg[mm] = Cb[(tid / D + PARTS * mm) * CS + (tid % D - 32 * pc)];
      }
      __syncthreads();
    }
  }
  if (tid < D) u[tid] = (tid == jstar) ? 1.0 : 0.0;
  __syncthreads();
  const int col = tid % D, part = tid / D;
  for (int it = 0; it < a.power_iters; ++it) {
    // w = C u, this thread's rows; two accumulators for ILP
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int m = 0; m < JPP; m += 2) {
      s0 += creg[m] * u[part + PARTS * m];
      s1 += creg[m + 1] * u[part + PARTS * (m + 1)];
    }
    wpart[part][col] = s0 + s1;
    __syncthreads();
    // every wave forms all of w and its norm (entries lane + 64 q; the
    // same sums in the same order in every wave), so no second exchange is
    // needed; wave 0 writes the new u
    double wq[(D + 63) / 64], sq = 0.0;
#pragma unroll
    for (int q = 0; q < (D + 63) / 64; ++q) {
      double w = 0.0;
#pragma unroll
      for (int p = 0; p < PARTS; ++p) w += wpart[p][lane + 64 * q];
      wq[q] = w;
      sq += w * w;
    }
    const double nrm2 = wave_sum_f64(sq);
    if (nrm2 == 0.0) {  // all queries equal: every projection will be 0
      if (wave == 0) {
#pragma unroll
        for (int q = 0; q < (D + 63) / 64; ++q) u[lane + 64 * q] = 0.0;
      }
      break;
    }
    if (wave == 0) {
#pragma unroll
      for (int q = 0; q < (D + 63) / 64; ++q) u[lane + 64 * q] = wq[q] / sqrt(nrm2);
    }
    __syncthreads();
  }
  __syncthreads();
  // orientation: the largest-magnitude component positive (lowest j on ties)
  if (wave == 0) {
    double v = fabs(u[lane]);
    int j = lane;
    if (D > 64) {
      const double v2 = fabs(u[lane + 64]);
      if (v2 > v) {
        v = v2;
        j = lane + 64;
      }
    }
    wave_argmax(v, j);
    if (lane == 0) jstar = j;
  }
  __syncthreads();
  // the direction in the queries' own coordinates (whitened: w_d u_d, so
  // the projection of x - mu equals that of the standardized queries)
  if (tid < D) {
    const double sgn = (u[jstar] < 0.0) ? -1.0 : 1.0;
    a.dir[((int64_t)bh * a.max_nodes + ln) * D + tid] = sgn * u[tid] * (a.whiten ? wsc[tid] : 1.0);
  }
}

// ---- projection: grid (nchunks, BH), 256 threads -----------------------------
template <int D>
__global__ __launch_bounds__(256) void project_kernel(PddpArgs a) {
  constexpr int LPT = D / 8;       // lanes per token
  constexpr int TPW = 64 / LPT;    // tokens per wave step
  const PLevel L = a.levels[a.level];
  const int bh = blockIdx.y;
  const PChunk c = a.pchunks[L.pchunk0 + blockIdx.x];
  const uint16_t *qh = head_q(a, bh);
  const int32_t *cur = a.perm + (int64_t)bh * a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT, tw = lane / LPT;
  const double *mu = a.mu + ((int64_t)bh * a.max_nodes + c.owner) * D + sub * 8;
  const double *dv = a.dir + ((int64_t)bh * a.max_nodes + c.owner) * D + sub * 8;
  double m8[8], u8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m8[e] = mu[e];
    u8[e] = dv[e];
  }
  double *proj = a.proj + (int64_t)bh * a.N;
  int32_t *tmp = a.tmp + (int64_t)bh * a.N;
  // the chunk's tokens in one coalesced read, then UNR rows in flight per
  // lane group: the row loads no longer wait one by one behind index loads
  __shared__ int32_t toks[kPChunk];
  for (int i = tid; i < c.len; i += 256) toks[i] = cur[c.off + i];
  __syncthreads();
  constexpr int TPB = 4 * TPW;  // tokens per block step
  constexpr int UNR = 4;
  for (int i0 = wave * TPW; i0 < c.len; i0 += UNR * TPB) {
    u32x4 v[UNR];
    int tk[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + u * TPB + tw;
      tk[u] = toks[i < c.len ? i : 0];
      v[u] = *(const u32x4 *)(qh + (int64_t)tk[u] * a.sn + sub * 8);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + u * TPB + tw;
      double p = 0.0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        p += ((double)bf16_to_f32(v[u][m] & 0xffffu) - m8[2 * m]) * u8[2 * m];
        p += ((double)bf16_to_f32(v[u][m] >> 16) - m8[2 * m + 1]) * u8[2 * m + 1];
      }
      // the sum over the token's LPT lanes on DPP, each a VALU step instead
      // of a shuffle through LDS: LPT = 16 (a whole 16-lane row) rotates the
      // row by 8 and by 4; LPT = 8 (half a row) mirrors each half. Then the
      // two quad permutes. The lane with sub == 0, the only one that stores,
      // adds in a fixed order.
      if (LPT == 16) {
        p += dpp_f64<0x128>(p);  // row_ror:8
        p += dpp_f64<0x124>(p);  // row_ror:4
      } else {
        p += dpp_f64<0x141>(p);  // row_half_mirror: lane i and 7 - i of each 8
      }
      p += dpp_f64<0x4E>(p);  // quad_perm [2,3,0,1]
      p += dpp_f64<0xB1>(p);  // quad_perm [1,0,3,2]
      if (i < c.len && sub == 0) {
        proj[c.off + i] = p;
        tmp[c.off + i] = tk[u];
      }
    }
  }
}

__device__ __forceinline__ uint64_t order_key64(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x == 0.0 ? 0.0 : x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// ---- split: grid (nnodes, BH), 512 threads ----------------------------------
__global__ __launch_bounds__(kSplitThreads) void split_kernel(PddpArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wcnt[kSplitThreads / 64];
  __shared__ uint32_t sel_digit, sel_below;
  const PLevel L = a.levels[a.level];
  const int bh = blockIdx.y;
  const PNode nd = a.nodes[L.node0 + blockIdx.x];
  const double *p = a.proj + (int64_t)bh * a.N + nd.off;
  const int32_t *src = a.tmp + (int64_t)bh * a.N + nd.off;
  int32_t *dst = a.perm + (int64_t)bh * a.N + nd.off;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)nd.nl;  // smallest keys still to place left
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < 256; i += kSplitThreads) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < nd.n; i += kSplitThreads) {
      const uint64_t k = order_key64(p[i]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) radix_pick<false>(hist, remaining, &sel_digit, &sel_below);
    __syncthreads();
    prefix |= (uint64_t)sel_digit << shift;
    mask |= (uint64_t)255 << shift;
    remaining -= sel_below;
    __syncthreads();
  }
  const uint64_t tau = prefix;
  const uint32_t need = remaining;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t nleft = 0, ties = 0;
  for (int base = 0; base < nd.n; base += kSplitThreads) {
    const int i = base + tid;
    const bool ok = i < nd.n;
    const uint64_t k = ok ? order_key64(p[i]) : 0;
    const bool eq = ok && k == tau;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wcnt[wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_before = 0, eq_total = 0;
    for (int w = 0; w < kSplitThreads / 64; ++w) {
      eq_before += (w < wave) ? wcnt[w] : 0u;
      eq_total += wcnt[w];
    }
    const bool left = ok && (k < tau || (eq && ties + eq_before + (uint32_t)__popcll(beq & lt_mask) < need));
    const uint64_t bl = __ballot(left);
    __syncthreads();
    if (lane == 0) wcnt[wave] = (uint32_t)__popcll(bl);
    __syncthreads();
    uint32_t l_before = 0, l_total = 0;
    for (int w = 0; w < kSplitThreads / 64; ++w) {
      l_before += (w < wave) ? wcnt[w] : 0u;
      l_total += wcnt[w];
    }
    if (ok) {
      const uint32_t lrank = nleft + l_before + (uint32_t)__popcll(bl & lt_mask);
      const int tok = src[i];
      if (left) dst[lrank] = tok;
      else dst[nd.nl + (i - (int)lrank)] = tok;
    }
    nleft += l_total;
    ties += eq_total;
    __syncthreads();
  }
}

// ---- split of nodes up to 512 * KPT tokens: grid (nnodes, BH), 512 threads --
// The node's keys are read once into registers (wave w holds the contiguous
// positions [w * 64 * KPT, (w + 1) * 64 * KPT), lane l the positions l,
// l + 64, ...); the radix passes count them into kSplitCopies private
// histograms (lane % 8, bank-shifting stride), so equal digits within a wave
// contend at most 8-way; and each wave partitions its own positions after a
// single barrier that gives it the counts of the positions before it.
constexpr int kSplitCopies = 8;

template <int NTH, int KPT>
__global__ __launch_bounds__(NTH) void split_reg_kernel(PddpArgs a) {
  constexpr int NW = NTH / 64;
  constexpr int SEG = 64 * KPT;
  __shared__ uint32_t hc[kSplitCopies * 257];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t lt_cnt[NW], eq_cnt[NW];
  __shared__ uint32_t sel_digit, sel_below;
  __shared__ unsigned long long tau_s;
  const PLevel L = a.levels[a.level];
  const int bh = blockIdx.y;
  const PNode nd = a.nodes[L.node0 + blockIdx.x];
  const double *p = a.proj + (int64_t)bh * a.N + nd.off;
  const int32_t *src = a.tmp + (int64_t)bh * a.N + nd.off;
  int32_t *dst = a.perm + (int64_t)bh * a.N + nd.off;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = wave * SEG + lane;  // position of key k: i0 + 64 k
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t *hcl = hc + (lane & (kSplitCopies - 1)) * 257;

  // positions past the node hold the largest key: never below the
  // threshold, which is a key of the node (the nl-th smallest, nl < n)
  uint64_t key[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = i0 + 64 * k;
    key[k] = i < nd.n ? order_key64(p[i]) : ~0ull;
  }
  uint64_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)nd.nl;  // smallest keys still to place left
#pragma unroll 1
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = tid; i < kSplitCopies * 257; i += NTH) hc[i] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if ((key[k] & mask) == prefix) atomicAdd(&hcl[(uint32_t)(key[k] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0;
#pragma unroll
      for (int cc = 0; cc < kSplitCopies; ++cc) c += hc[cc * 257 + tid];
      hist[tid] = c;
    }
    __syncthreads();
    if (wave == 0) radix_pick<false>(hist, remaining, &sel_digit, &sel_below);
    __syncthreads();
    prefix |= (uint64_t)sel_digit << shift;
    mask |= (uint64_t)255 << shift;
    remaining -= sel_below;
    // a bin holding one key: that key is the threshold (and remaining is 1),
    // so the low digits need no more passes
    if (pass < 7 && hist[sel_digit] == 1u) {
#pragma unroll
      for (int k = 0; k < KPT; ++k)
        if ((key[k] & mask) == prefix) tau_s = key[k];
      __syncthreads();
      prefix = tau_s;
      break;
    }
  }
  const uint64_t tau = prefix;
  const uint32_t need = remaining;
  uint32_t lt = 0, eq = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    lt += key[k] < tau ? 1u : 0u;
    eq += key[k] == tau ? 1u : 0u;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lt += __shfl_xor(lt, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) {
    lt_cnt[wave] = lt;
    eq_cnt[wave] = eq;
  }
  __syncthreads();
  uint32_t nleft = 0, ties = 0;  // before this wave's positions
  for (int w = 0; w < wave; ++w) {
    const uint32_t e = eq_cnt[w];
    const uint32_t room = need > ties ? need - ties : 0u;
    nleft += lt_cnt[w] + (e < room ? e : room);
    ties += e;
  }
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const int i = i0 + 64 * k;
    const bool e = key[k] == tau;
    const uint64_t beq = __ballot(e);
    const bool left = key[k] < tau || (e && ties + (uint32_t)__popcll(beq & lt_mask) < need);
    const uint64_t bl = __ballot(left);
    const uint32_t lrank = nleft + (uint32_t)__popcll(bl & lt_mask);
    if (i < nd.n) {
      const int tok = src[i];
      if (left) dst[lrank] = tok;
      else dst[nd.nl + (i - (int)lrank)] = tok;
    }
    nleft += (uint32_t)__popcll(bl);
    ties += (uint32_t)__popcll(beq);
  }
}

// the split of one level: register keys when its largest node fits. The
// top levels have few nodes (one or two per head), so nodes above 8192
// tokens get more threads (fewer keys per thread, more waves hiding each
// pass's latency) as far as the registers allow without spilling: 1024
// threads of 16 keys, then 768 threads of 43; the result does not depend
// on the count.
hipError_t launch_split(const PddpArgs &a, const PLevel &L, int BH, hipStream_t s) {
  const dim3 g(L.nnodes, BH), b(kSplitThreads);
  if (L.maxn <= 512) hipLaunchKernelGGL((split_reg_kernel<kSplitThreads, 1>), g, b, 0, s, a);
  else if (L.maxn <= 512 * 2) hipLaunchKernelGGL((split_reg_kernel<kSplitThreads, 2>), g, b, 0, s, a);
  else if (L.maxn <= 512 * 4) hipLaunchKernelGGL((split_reg_kernel<kSplitThreads, 4>), g, b, 0, s, a);
  else if (L.maxn <= 512 * 8) hipLaunchKernelGGL((split_reg_kernel<kSplitThreads, 8>), g, b, 0, s, a);
  else if (L.maxn <= 1024 * 16) hipLaunchKernelGGL((split_reg_kernel<1024, 16>), g, dim3(1024), 0, s, a);
  else if (L.maxn <= 768 * 43) hipLaunchKernelGGL((split_reg_kernel<768, 43>), g, dim3(768), 0, s, a);
  else if (L.maxn <= 512 * 64) hipLaunchKernelGGL((split_reg_kernel<kSplitThreads, 64>), g, b, 0, s, a);
  else hipLaunchKernelGGL(split_kernel, g, b, 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t run_levels(PddpArgs &a, const PlanCounts &pc, const std::vector<PLevel> &host_levels,
                      hipStream_t s) {
  constexpr int NSL = (moment_doubles(D) + 255) / 256;
  const int BH = a.B * a.H;
  for (int l = 0; l < pc.levels; ++l) {
    a.level = l;
    const PLevel &L = host_levels[l];
    if (l == 0)  // one more block builds the plan tables
      hipLaunchKernelGGL((moment_kernel<D, true>), dim3(L.nmchunks + 1, BH), dim3(256),
                         a.plan_in_lds ? plan_list_bytes(a.N, a.T) : 0, s, a);
    else
      hipLaunchKernelGGL((moment_kernel<D, false>), dim3(L.nmchunks, BH), dim3(256), 0, s, a);
    if (L.reduced) hipLaunchKernelGGL(reduce_kernel<D>, dim3(L.nunits * NSL, BH), dim3(256), 0, s, a);
    hipLaunchKernelGGL(power_kernel<D>, dim3(L.nnodes, BH), dim3(256), 0, s, a);
    hipLaunchKernelGGL(project_kernel<D>, dim3(L.npchunks, BH), dim3(256), 0, s, a);
    const hipError_t e = launch_split(a, L, BH, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t pddp_workspace_bytes(int B, int H, int N, int D, int T) {
  const PlanCounts pc = host_plan(N, T, nullptr);
  return ws_layout(pc, B * H, N, D).total;
}

hipError_t run_pddp(const uint16_t *q, int64_t sb, int64_t sn, int64_t sh, int B, int H, int N,
                    int D, int T, int power_iters, bool whiten, int32_t *perm, void *ws,
                    size_t ws_bytes, hipStream_t s) {
  const int BH = B * H;
  const int64_t total = (int64_t)BH * N;
  std::vector<PLevel> hl(kMaxLevels);
  const PlanCounts pc = host_plan(N, T, hl.data());
  const WsLayout wl = ws_layout(pc, BH, N, D);
  if (ws_bytes < wl.total || pc.levels > kMaxLevels || (D != 64 && D != 128)) return hipErrorInvalidValue;
  if (N <= T) {  // one group per head: the identity
    hipLaunchKernelGGL(init_perm_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, perm,
                       N, total);
    return hipGetLastError();
  }
  char *base = (char *)ws;
  PddpArgs a{};
  a.q = q;
  a.sb = sb;
  a.sn = sn;
  a.sh = sh;
  a.B = B;
  a.H = H;
  a.N = N;
  a.T = T;
  a.perm = perm;
  a.levels = (PLevel *)(base + wl.levels);
  a.nodes = (PNode *)(base + wl.nodes);
  a.units = (PUnit *)(base + wl.units);
  a.mchunks = (PChunk *)(base + wl.mchunks);
  a.pchunks = (PChunk *)(base + wl.pchunks);
  a.part = (double *)(base + wl.part);
  a.ured = (double *)(base + wl.ured);
  a.nodem = (double *)(base + wl.nodem);
  a.mu = (double *)(base + wl.mu);
  a.dir = (double *)(base + wl.dir);
  a.proj = (double *)(base + wl.proj);
  a.tmp = (int32_t *)(base + wl.tmp);
  a.wscale = (double *)(base + wl.wscale);
  a.whiten = whiten ? 1 : 0;
  a.max_mchunks = pc.max_mchunks;
  a.max_runits = pc.max_runits > 0 ? pc.max_runits : 1;
  a.max_units = pc.max_units;
  a.max_nodes = pc.max_nodes;
  a.power_iters = power_iters;
  // the level-0 blocks run two per CU (registers), so LDS up to half the
  // CU's 160 KB each, the moment staging buffer included, costs no
  // occupancy; 72 KB leaves room for allocation granules and small arrays
  const size_t staging = (size_t)32 * (D + 16) * sizeof(double);
  a.plan_in_lds = plan_list_bytes(N, T) + staging <= (size_t)72 * 1024 ? 1 : 0;
  if (D == 128) return run_levels<128>(a, pc, hl, s);
  return run_levels<64>(a, pc, hl, s);
}

}  // namespace mcs
