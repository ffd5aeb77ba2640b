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
// Every level runs five kernels over all heads and nodes at once:
//   mean     per chunk of a node: sum of q (float64)           -> partials
//   cov      per chunk: sum of (q-mu)(q-mu)^T on the fp64 MFMA
//            (v_mfma_f64_16x16x4_f64, upper-triangle tiles)      -> partials
//            (its accumulator: lane l, register i holds row l/16 + 4i,
//            column l % 16; operands: lane l holds row/col l % 16, k = l/16)
//   power    per node: add the partials in chunk order (fixed, no atomics),
//            power iteration from e_{argmax diag}, orientation    -> mu, u
//   project  per chunk: p_i = (q_i - mu) . u in float64
//   split    per node: radix select of the floor(G_S/2)*T-th smallest
//            (p, position) and a stable partition of the node's range.
// Decisions are taken on float64 values so the split does not hinge on
// fp32 rounding.
#include <vector>

#include "mcs_common.hpp"
#include "mcs_internal.hpp"
#include "mcs_radix.hpp"

namespace mcs {

namespace {

constexpr int kChunk = 1024;       // tokens per chunk of the per-chunk kernels
constexpr int kMaxLevels = 40;
constexpr int kSplitThreads = 512;

struct PLevel {
  int node0, nnodes, chunk0, nchunks;
};
struct PNode {
  int off, n, nl, chunk0, nchunks;  // chunk0: level-local index of its first chunk
};
struct PChunk {
  int node, off, len;  // node: level-local node index; off: absolute position
};

struct PlanCounts {
  int levels, nodes, chunks, max_nodes, max_chunks;
};

// Builds the level / node / chunk tables. `nd` must hold at least 2*G nodes;
// `lv` and `ch` may be null to only count.
__host__ __device__ PlanCounts plan_tree(int N, int T, PLevel *lv, PNode *nd, PChunk *ch) {
  PlanCounts pc{0, 0, 0, 0, 0};
  if (N <= T) return pc;
  // active nodes (more than T tokens) are appended level by level, so the
  // nodes of one level are contiguous; level 0 is the root
  nd[0] = PNode{0, N, 0, 0, 0};
  int lvl_begin = 0, lvl_end = 1;
  while (lvl_begin < lvl_end) {
    int level_chunks = 0;
    int next_end = lvl_end;
    for (int i = lvl_begin; i < lvl_end; ++i) {
      PNode x = nd[i];
      const int G = (x.n + T - 1) / T;
      x.nl = (G / 2) * T;
      x.chunk0 = level_chunks;
      x.nchunks = (x.n + kChunk - 1) / kChunk;
      for (int c = 0; c < x.nchunks; ++c) {
        const int rest = x.n - c * kChunk;
        if (ch) ch[pc.chunks + level_chunks + c] = PChunk{i - lvl_begin, x.off + c * kChunk,
                                                          rest < kChunk ? rest : kChunk};
      }
      level_chunks += x.nchunks;
      nd[i] = x;
      const int nr = x.n - x.nl;
      if (x.nl > T) nd[next_end++] = PNode{x.off, x.nl, 0, 0, 0};
      if (nr > T) nd[next_end++] = PNode{x.off + x.nl, nr, 0, 0, 0};
    }
    if (lv) lv[pc.levels] = PLevel{lvl_begin, lvl_end - lvl_begin, pc.chunks, level_chunks};
    const int nn = lvl_end - lvl_begin;
    pc.max_nodes = pc.max_nodes > nn ? pc.max_nodes : nn;
    pc.max_chunks = pc.max_chunks > level_chunks ? pc.max_chunks : level_chunks;
    pc.chunks += level_chunks;
    pc.levels++;
    lvl_begin = lvl_end;
    lvl_end = next_end;
  }
  pc.nodes = lvl_end;
  return pc;
}

inline size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t levels, nodes, chunks, mean_part, cov_part, mu, dir, proj, tmp, total;
};

WsLayout ws_layout(const PlanCounts &pc, int BH, int N, int D) {
  WsLayout w{};
  size_t o = 0;
  w.levels = o; o = align_up(o + sizeof(PLevel) * kMaxLevels);
  w.nodes = o; o = align_up(o + sizeof(PNode) * (size_t)(pc.nodes > 0 ? pc.nodes : 1));
  w.chunks = o; o = align_up(o + sizeof(PChunk) * (size_t)(pc.chunks > 0 ? pc.chunks : 1));
  w.mean_part = o; o = align_up(o + sizeof(double) * (size_t)BH * pc.max_chunks * D);
  w.cov_part = o; o = align_up(o + sizeof(double) * (size_t)BH * pc.max_chunks * D * D);
  w.mu = o; o = align_up(o + sizeof(double) * (size_t)BH * pc.max_nodes * D);
  w.dir = o; o = align_up(o + sizeof(double) * (size_t)BH * pc.max_nodes * D);
  w.proj = o; o = align_up(o + sizeof(double) * (size_t)BH * N);
  w.tmp = o; o = align_up(o + sizeof(int32_t) * (size_t)BH * N);
  w.total = o;
  return w;
}

// Host-side plan with real arrays (the counting needs the node ranges).
PlanCounts host_plan(int N, int T) {
  if (N <= T) return PlanCounts{0, 0, 0, 0, 0};
  const int G = (N + T - 1) / T;
  std::vector<PNode> nd(2 * G + 2);
  return plan_tree(N, T, nullptr, nd.data(), nullptr);
}

struct PddpArgs {
  const uint16_t *q;
  int64_t sb, sn, sh;
  int B, H, N;
  int32_t *perm;
  const PLevel *levels;
  const PNode *nodes;
  const PChunk *chunks;
  double *mean_part, *cov_part, *mu, *dir, *proj;
  int32_t *tmp;
  int max_chunks, max_nodes;
  int level;
  int power_iters;
};

__global__ void plan_kernel(int N, int T, PLevel *lv, PNode *nd, PChunk *ch) {
  if (threadIdx.x == 0 && blockIdx.x == 0) plan_tree(N, T, lv, nd, ch);
}

__global__ void init_perm_kernel(int32_t *perm, int N, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) perm[i] = (int32_t)(i % N);
}

__device__ __forceinline__ const uint16_t *head_q(const PddpArgs &a, int bh) {
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  return a.q + (int64_t)b * a.sb + (int64_t)h * a.sh;
}

// ---- mean partials: grid (nchunks, BH), 256 threads -------------------------
template <int D>
__global__ __launch_bounds__(256) void mean_kernel(PddpArgs a) {
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int TL = 256 / CH;    // token lanes
  __shared__ double red[TL][D + 1];
  const PLevel L = a.levels[a.level];
  const int bh = blockIdx.y;
  const PChunk c = a.chunks[L.chunk0 + blockIdx.x];
  const uint16_t *qh = head_q(a, bh);
  const int32_t *cur = a.perm + (int64_t)bh * a.N;
  const int col = threadIdx.x % CH, tl = threadIdx.x / CH;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i = tl; i < c.len; i += TL) {
    const int tok = cur[c.off + i];
    const u32x4 v = *(const u32x4 *)(qh + (int64_t)tok * a.sn + col * 8);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[2 * m] += (double)bf16_to_f32(v[m] & 0xffffu);
      acc[2 * m + 1] += (double)bf16_to_f32(v[m] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tl][col * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
    for (int t = 0; t < TL; ++t) s += red[t][threadIdx.x];
    a.mean_part[((int64_t)bh * a.max_chunks + blockIdx.x) * D + threadIdx.x] = s;
  }
}

// ---- covariance partials: grid (nchunks, BH), 256 threads ------------------
template <int D>
__global__ __launch_bounds__(256) void cov_kernel(PddpArgs a) {
  constexpr int NB = D / 16;                 // 16-wide dim blocks
  constexpr int NTILES = NB * (NB + 1) / 2;  // upper-triangle tiles
  constexpr int TPW = (NTILES + 3) / 4;      // tiles per wave (at most)
  constexpr int SUB = 64;                    // tokens staged per step
  constexpr int XS = D + 1;                  // LDS row stride (doubles)
  constexpr int CH = D / 8;
  constexpr int TL = 256 / CH;
  __shared__ double X[SUB * XS];
  __shared__ double mu_s[D];

  const PLevel L = a.levels[a.level];
  const int bh = blockIdx.y;
  const PChunk c = a.chunks[L.chunk0 + blockIdx.x];
  const PNode nd = a.nodes[L.node0 + c.node];
  const uint16_t *qh = head_q(a, bh);
  const int32_t *cur = a.perm + (int64_t)bh * a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (tid < D) {
    double s = 0.0;
    const double *mp = a.mean_part + ((int64_t)bh * a.max_chunks + nd.chunk0) * D + tid;
    for (int k = 0; k < nd.nchunks; ++k) s += mp[(int64_t)k * D];
    mu_s[tid] = s / (double)nd.n;
  }
  __syncthreads();

  // wave w owns the upper-triangle tiles t with t % 4 == w (t enumerates
  // (bi, bj), bi <= bj, row-major); acc[t / 4] is its accumulator
  f64x4 acc[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) acc[k] = f64x4{0, 0, 0, 0};

  const int col = tid % CH, tl = tid / CH;
  double muc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) muc[e] = mu_s[col * 8 + e];

  for (int base = 0; base < c.len; base += SUB) {
    // stage (q - mu) for SUB tokens; rows past the chunk are zero
    for (int r = tl; r < SUB; r += TL) {
      double x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (base + r < c.len) {
        const int tok = cur[c.off + base + r];
        const u32x4 v = *(const u32x4 *)(qh + (int64_t)tok * a.sn + col * 8);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          x[2 * m] = (double)bf16_to_f32(v[m] & 0xffffu) - muc[2 * m];
          x[2 * m + 1] = (double)bf16_to_f32(v[m] >> 16) - muc[2 * m + 1];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) X[r * XS + col * 8 + e] = x[e];
    }
    __syncthreads();
    const int steps = (c.len - base) < SUB ? ((c.len - base + 3) / 4) : SUB / 4;
    for (int s = 0; s < steps; ++s) {
      const int row = 4 * s + (lane >> 4);
      double fr[NB];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) fr[bb] = X[row * XS + 16 * bb + (lane & 15)];
      int t = 0;
#pragma unroll
      for (int bi = 0; bi < NB; ++bi) {
#pragma unroll
        for (int bj = bi; bj < NB; ++bj, ++t) {
          if ((t & 3) == wave)
            acc[t >> 2] = __builtin_amdgcn_mfma_f64_16x16x4f64(fr[bi], fr[bj], acc[t >> 2], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  double *out = a.cov_part + ((int64_t)bh * a.max_chunks + blockIdx.x) * D * D;
  int t = 0;
#pragma unroll
  for (int bi = 0; bi < NB; ++bi) {
#pragma unroll
    for (int bj = bi; bj < NB; ++bj, ++t) {
      if ((t & 3) == wave) {
        const int colj = 16 * bj + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rowi = 16 * bi + (lane >> 4) + 4 * i;  // f64 MFMA: row = lane/16 + 4*i
          out[(int64_t)rowi * D + colj] = acc[t >> 2][i];
        }
      }
    }
  }
}

// ---- node direction: grid (nnodes, BH), 256 threads -------------------------
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
  constexpr int EPT = D * D / 256;  // covariance entries per thread
  constexpr int PARTS = 256 / D;    // threads per column in the matrix-vector product
  constexpr int JPP = D / PARTS;    // rows per part
  __shared__ double C[D * D];
  __shared__ double u[D], wpart[PARTS][D], red[4];
  __shared__ int jstar;
  const PLevel L = a.levels[a.level];
  const int bh = blockIdx.y;
  const int ln = blockIdx.x;
  const PNode nd = a.nodes[L.node0 + ln];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // covariance: add the chunk partials (upper tiles) in chunk order, every
  // entry of this thread accumulating at once so its loads overlap. The
  // loads are unconditional (a partial's lower tiles are in the buffer but
  // never written) and the lower-tile values are dropped by a select, so no
  // branch serialises them.
  {
    const double *cp = a.cov_part + ((int64_t)bh * a.max_chunks + nd.chunk0) * D * D;
    double acc[EPT];
#pragma unroll
    for (int m = 0; m < EPT; ++m) acc[m] = 0.0;
    for (int k = 0; k < nd.nchunks; ++k) {
      const double *src = cp + (int64_t)k * D * D;
      double v[EPT];
#pragma unroll
      for (int m = 0; m < EPT; ++m) v[m] = src[tid + 256 * m];
#pragma unroll
      for (int m = 0; m < EPT; ++m) {
        const int e = tid + 256 * m;
        acc[m] += (((e / D) >> 4) <= ((e % D) >> 4)) ? v[m] : 0.0;
      }
    }
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
      const int e = tid + 256 * m;
      if (((e / D) >> 4) <= ((e % D) >> 4)) C[e] = acc[m] / (double)nd.n;
    }
  }
  __syncthreads();
  for (int e = tid; e < D * D; e += 256) {
    const int i = e / D, j = e - (e / D) * D;
    if ((i >> 4) > (j >> 4)) C[e] = C[j * D + i];
  }
  // mean of the node for the projection kernel, partials in chunk order
  if (tid < D) {
    const double *mp = a.mean_part + ((int64_t)bh * a.max_chunks + nd.chunk0) * D + tid;
    double s = 0.0;
    int k = 0;
    for (; k + 8 <= nd.nchunks; k += 8) {
      double v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = mp[(int64_t)(k + i) * D];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; k < nd.nchunks; ++k) s += mp[(int64_t)k * D];
    a.mu[((int64_t)bh * a.max_nodes + ln) * D + tid] = s / (double)nd.n;
  }
  __syncthreads();
  // start vector: e_j for the largest diagonal entry (lowest j on ties)
  if (wave == 0) {
    double v = C[lane * D + lane];
    int j = lane;
    if (D > 64) {
      const double v2 = C[(lane + 64) * D + lane + 64];
      if (v2 > v) {
        v = v2;
        j = lane + 64;
      }
    }
    wave_argmax(v, j);
    if (lane == 0) jstar = j;
  }
  __syncthreads();
  if (tid < D) u[tid] = (tid == jstar) ? 1.0 : 0.0;
  __syncthreads();
  // thread (part, col) keeps rows part, part + PARTS, ... of column col of
  // C in registers for all iterations (C is symmetric: column = row)
  const int col = tid % D, part = tid / D;
  double creg[JPP];
#pragma unroll
  for (int m = 0; m < JPP; ++m) creg[m] = C[(part + PARTS * m) * D + col];
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
    double w = 0.0, sq = 0.0;
    if (tid < D) {
#pragma unroll
      for (int p = 0; p < PARTS; ++p) w += wpart[p][tid];
      sq = w * w;
    }
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) sq += __shfl_xor(sq, s);
    if (lane == 0) red[wave] = sq;
    __syncthreads();
    double nrm2 = 0.0;
#pragma unroll
    for (int q = 0; q < (D + 63) / 64; ++q) nrm2 += red[q];
    if (nrm2 == 0.0) {  // all queries equal: every projection will be 0
      if (tid < D) u[tid] = 0.0;
      break;
    }
    if (tid < D) u[tid] = w / sqrt(nrm2);
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
  if (tid < D) {
    const double sgn = (u[jstar] < 0.0) ? -1.0 : 1.0;
    a.dir[((int64_t)bh * a.max_nodes + ln) * D + tid] = sgn * u[tid];
  }
}

// ---- projection: grid (nchunks, BH), 256 threads -----------------------------
template <int D>
__global__ __launch_bounds__(256) void project_kernel(PddpArgs a) {
  constexpr int LPT = D / 8;       // lanes per token
  constexpr int TPW = 64 / LPT;    // tokens per wave step
  const PLevel L = a.levels[a.level];
  const int bh = blockIdx.y;
  const PChunk c = a.chunks[L.chunk0 + blockIdx.x];
  const uint16_t *qh = head_q(a, bh);
  const int32_t *cur = a.perm + (int64_t)bh * a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPT, tw = lane / LPT;
  const double *mu = a.mu + ((int64_t)bh * a.max_nodes + c.node) * D + sub * 8;
  const double *dv = a.dir + ((int64_t)bh * a.max_nodes + c.node) * D + sub * 8;
  double m8[8], u8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m8[e] = mu[e];
    u8[e] = dv[e];
  }
  double *proj = a.proj + (int64_t)bh * a.N;
  int32_t *tmp = a.tmp + (int64_t)bh * a.N;
  for (int i0 = wave * TPW; i0 < c.len; i0 += 4 * TPW) {
    const int i = i0 + tw;
    const bool ok = i < c.len;
    const int pos = c.off + (ok ? i : 0);
    const int tok = cur[pos];
    const u32x4 v = *(const u32x4 *)(qh + (int64_t)tok * a.sn + sub * 8);
    double p = 0.0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      p += ((double)bf16_to_f32(v[m] & 0xffffu) - m8[2 * m]) * u8[2 * m];
      p += ((double)bf16_to_f32(v[m] >> 16) - m8[2 * m + 1]) * u8[2 * m + 1];
    }
#pragma unroll
    for (int s = LPT / 2; s > 0; s >>= 1) p += __shfl_xor(p, s);
    if (ok && sub == 0) {
      proj[pos] = p;
      tmp[pos] = tok;
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

template <int D>
hipError_t run_levels(PddpArgs &a, const PlanCounts &pc, const std::vector<PLevel> &host_levels,
                      hipStream_t s) {
  const int BH = a.B * a.H;
  for (int l = 0; l < pc.levels; ++l) {
    a.level = l;
    const PLevel &L = host_levels[l];
    const dim3 gc(L.nchunks, BH), gn(L.nnodes, BH);
    hipLaunchKernelGGL(mean_kernel<D>, gc, dim3(256), 0, s, a);
    hipLaunchKernelGGL(cov_kernel<D>, gc, dim3(256), 0, s, a);
    hipLaunchKernelGGL(power_kernel<D>, gn, dim3(256), 0, s, a);
    hipLaunchKernelGGL(project_kernel<D>, gc, dim3(256), 0, s, a);
    hipLaunchKernelGGL(split_kernel, gn, dim3(kSplitThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t pddp_workspace_bytes(int B, int H, int N, int D, int T) {
  const PlanCounts pc = host_plan(N, T);
  return ws_layout(pc, B * H, N, D).total;
}

hipError_t run_pddp(const uint16_t *q, int64_t sb, int64_t sn, int64_t sh, int B, int H, int N,
                    int D, int T, int power_iters, int32_t *perm, void *ws, size_t ws_bytes,
                    hipStream_t s) {
  const int BH = B * H;
  const int64_t total = (int64_t)BH * N;
  const int G = (N + T - 1) / T;
  std::vector<PNode> hn(2 * G + 2);
  std::vector<PLevel> hl(kMaxLevels);
  const PlanCounts pc = plan_tree(N, T, hl.data(), hn.data(), nullptr);
  const WsLayout wl = ws_layout(pc, BH, N, D);
  if (ws_bytes < wl.total || pc.levels > kMaxLevels) return hipErrorInvalidValue;
  hipLaunchKernelGGL(init_perm_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, perm,
                     N, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || N <= T) return e;
  char *base = (char *)ws;
  PddpArgs a{};
  a.q = q;
  a.sb = sb;
  a.sn = sn;
  a.sh = sh;
  a.B = B;
  a.H = H;
  a.N = N;
  a.perm = perm;
  a.levels = (const PLevel *)(base + wl.levels);
  a.nodes = (const PNode *)(base + wl.nodes);
  a.chunks = (const PChunk *)(base + wl.chunks);
  a.mean_part = (double *)(base + wl.mean_part);
  a.cov_part = (double *)(base + wl.cov_part);
  a.mu = (double *)(base + wl.mu);
  a.dir = (double *)(base + wl.dir);
  a.proj = (double *)(base + wl.proj);
  a.tmp = (int32_t *)(base + wl.tmp);
  a.max_chunks = pc.max_chunks;
  a.max_nodes = pc.max_nodes;
  a.power_iters = power_iters;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(64), 0, s, N, T, (PLevel *)(base + wl.levels),
                     (PNode *)(base + wl.nodes), (PChunk *)(base + wl.chunks));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D == 128) return run_levels<128>(a, pc, hl, s);
  if (D == 64) return run_levels<64>(a, pc, hl, s);
  return hipErrorInvalidValue;
}

}  // namespace mcs
