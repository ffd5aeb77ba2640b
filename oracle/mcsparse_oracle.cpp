// CPU oracle for MC-Sparse's meta-cached token-level sparse attention, in
// plain C++17 with float64 arithmetic.
//
// TEST INFRASTRUCTURE ONLY. It is loaded by tests/, by the smoke check of the
// package's entry module and by the CPU-baseline leg of the benchmark. The
// library it checks (libmcsparse) never links or loads it, and it includes
// nothing from that library: no header, helper, table or constant is shared.
//
// It works on ONE (batch, head) slice at a time: arrays are row-major [N][d]
// float64 holding the stored bf16 (or fp32) input values widened exactly.
// Units of work that the method keeps independent -- the query rows of a
// dense pass, the key columns of a group's mass, the groups of a head, the
// nodes of one PDDP tree level -- are spread over std::thread workers; each
// unit is computed by the same sequential loop whatever the thread count, so
// results do not depend on it.
//
// Sources (MC-Sparse, arXiv 2610.06801, as summarised on the pages):
//  * paper landing page, Abstract: the cached metadata is query groups, KV
//    indices chosen from exact attention probabilities, and dense-minus-
//    sparse residuals, reused over the following denoising steps;
//  * research walkthrough page, method steps 1-4 (Figure 6): step 1 Fast
//    PDDP grouping (project the queries on the principal direction, split at
//    the median, recurse until the groups are tile-sized); step 2 dense
//    attention with per-row log-sum-exp, a second QK pass recovering the
//    exact probabilities, their sum per query group and a top-K of single KV
//    tokens; step 3 residual R = dense output minus sparse output at the
//    anchor; step 4 the reuse step: sparse attention over the cached indices
//    with fresh Q/K/V, plus R.
//
// Readings where the pages are silent (each one stated where it is used):
// softmax scale given by the caller, no mask; principal direction = leading
// eigenvector of the node's centred covariance by a fixed number of power
// iterations from the unit vector of the largest diagonal entry (lowest index
// on ties), oriented so its largest-magnitude component is positive (lowest
// index on ties); median = a rank split at floor(G_S/2)*T tokens in
// (projection, token index) order, lower-projection child first, rows of a
// group ascending; group accumulation = plain sum over the group's rows;
// top-K order (-A, j), stored ascending; sparse softmax renormalised over the
// selected keys; R and the reuse output rounded to bf16 (nearest, ties to
// even); whitening = per-dimension standardization of the head's queries.
//
// Parity status: every function is pinned by tests/test_oracle_pins.py
// (exact decimal brute force, closed forms, library routines, invariants),
// run against this file and against an independent numpy transcription of
// the same steps; planted mistakes built from this file (ORC_MUTANT) fail
// those pins. Unpinned: that this reading of "Fast PDDP" reproduces the
// authors' groups (the pages print none).
#include <algorithm>
#include <atomic>
#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

#ifndef ORC_MUTANT
#define ORC_MUTANT 0
#endif

namespace {

// ---------------------------------------------------------------------------
// a tiny work splitter: units [0, n) handed out one at a time
// ---------------------------------------------------------------------------
template <class F>
void parallel_for(int64_t n, int threads, F f) {
  if (n <= 0) return;
  if (threads < 1) threads = 1;
  if (threads > n) threads = (int)n;
  if (threads == 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> pool;
  pool.reserve(threads);
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&] {
      for (int64_t i = next.fetch_add(1); i < n; i = next.fetch_add(1)) f(i);
    });
  for (auto &th : pool) th.join();
}

inline double dot(const double *a, const double *b, int d) {
  double s = 0.0;
  for (int c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

// ---------------------------------------------------------------------------
// storage rounding: float64 -> nearest bfloat16 (8 significant bits, fp32's
// exponent range), ties to even, straight from float64
// ---------------------------------------------------------------------------
constexpr double kBf16Max = 3.3895313892515355e38;  // (2 - 2^-7) * 2^127

double round_bf16_one(double x) {
  if (!std::isfinite(x) || x == 0.0) return x;
  int e;
  std::frexp(x, &e);  // |x| = f * 2^e, f in [0.5, 1): the leading bit is 2^(e-1)
  // 8 significant bits: the last kept bit is 2^(e-8); below bf16's smallest
  // normal the spacing stays at the subnormal step 2^-133
  const int ulp_exp = std::max(e - 8, -133);
  const double scaled = std::ldexp(x, -ulp_exp);  // exact (power-of-two scaling)
#if ORC_MUTANT == 12
  const double r = std::ldexp(std::trunc(scaled), ulp_exp);  // planted: truncation
#else
  const double r = std::ldexp(std::nearbyint(scaled), ulp_exp);  // current mode: nearest, ties to even
#endif
  if (std::fabs(r) > kBf16Max) return std::copysign(INFINITY, x);
  return r;
}

// ---------------------------------------------------------------------------
// step 1: PDDP
// ---------------------------------------------------------------------------

// Leading eigenvector of the symmetric d x d matrix C: start at e_start (or
// at the largest diagonal entry, lowest index on ties, when start < 0), then
// exactly `iters` steps u <- C u / |C u|; if C u vanishes the direction is 0.
// Oriented so the largest-magnitude component is positive (lowest index on
// ties).
void principal_direction(const double *C, int d, int iters, int start, double *u) {
  int j0 = start;
  if (j0 < 0) {
    j0 = 0;
    for (int j = 1; j < d; ++j)
      if (C[(int64_t)j * d + j] > C[(int64_t)j0 * d + j0]) j0 = j;
  }
  std::vector<double> w(d);
  std::fill(u, u + d, 0.0);
  u[j0] = 1.0;
#if ORC_MUTANT == 7
  iters -= 1;  // planted: one power iteration short
#endif
  for (int it = 0; it < iters; ++it) {
    for (int i = 0; i < d; ++i) w[i] = dot(C + (int64_t)i * d, u, d);
    const double nrm = std::sqrt(dot(w.data(), w.data(), d));
    if (nrm == 0.0) {
      std::fill(u, u + d, 0.0);
      return;
    }
    for (int i = 0; i < d; ++i) u[i] = w[i] / nrm;
  }
  int jm = 0;
  for (int j = 1; j < d; ++j)
    if (std::fabs(u[j]) > std::fabs(u[jm])) jm = j;
#if ORC_MUTANT == 8
  const bool flip = u[jm] > 0;  // planted: orientation reversed
#else
  const bool flip = u[jm] < 0;
#endif
  if (flip)
    for (int j = 0; j < d; ++j) u[j] = -u[j];
}

// Per-dimension standardization over the N rows: z = (x - mu) / sigma with
// the population variance; a zero-variance dimension is centred only.
void standardize(const double *q, int N, int d, double *z, double *var) {
  std::vector<double> mu(d, 0.0);
  for (int i = 0; i < N; ++i)
    for (int c = 0; c < d; ++c) mu[c] += q[(int64_t)i * d + c];
  for (int c = 0; c < d; ++c) mu[c] /= N;
  for (int c = 0; c < d; ++c) var[c] = 0.0;
  for (int i = 0; i < N; ++i)
    for (int c = 0; c < d; ++c) {
      const double x = q[(int64_t)i * d + c] - mu[c];
      var[c] += x * x;
    }
  for (int c = 0; c < d; ++c) var[c] /= N;
  for (int i = 0; i < N; ++i)
    for (int c = 0; c < d; ++c) {
      const double x = q[(int64_t)i * d + c] - mu[c];
#if ORC_MUTANT == 10
      z[(int64_t)i * d + c] = x;  // planted: never scaled
#else
      z[(int64_t)i * d + c] = var[c] > 0.0 ? x * (1.0 / std::sqrt(var[c])) : x;
#endif
    }
}

// One split of a node (its member tokens, any order): centre, covariance,
// principal direction, projection of every centred member, and the first
// n_left members in (projection, token) order to the left child. Both
// children come back ascending. The covariance's rows are computed by up to
// `threads` workers (rows are independent; each is the same loop).
void split_node(const double *q, int d, const std::vector<int64_t> &members, int64_t n_left, int iters,
                int start, int threads, std::vector<int64_t> &left, std::vector<int64_t> &right) {
  const int64_t n = (int64_t)members.size();
  std::vector<double> mu(d, 0.0);
  for (int64_t t = 0; t < n; ++t) {
    const double *x = q + members[t] * d;
    for (int c = 0; c < d; ++c) mu[c] += x[c];
  }
  for (int c = 0; c < d; ++c) mu[c] /= (double)n;
  std::vector<double> xc((size_t)n * d);
  for (int64_t t = 0; t < n; ++t) {
    const double *x = q + members[t] * d;
    for (int c = 0; c < d; ++c) xc[(size_t)t * d + c] = x[c] - mu[c];
  }
  // C_ab = (1/n) sum_t xc_ta xc_tb
  std::vector<double> C((size_t)d * d, 0.0);
  parallel_for(d, threads, [&](int64_t a) {
    std::vector<double> row(d, 0.0);
    for (int64_t t = 0; t < n; ++t) {
      const double *x = &xc[(size_t)t * d];
      const double xa = x[a];
      for (int b = 0; b < d; ++b) row[b] += xa * x[b];
    }
    for (int b = 0; b < d; ++b) C[(size_t)a * d + b] = row[b] / (double)n;
  });
  std::vector<double> u(d);
  principal_direction(C.data(), d, iters, start, u.data());
  std::vector<double> p(n);
  for (int64_t t = 0; t < n; ++t) p[t] = dot(&xc[(size_t)t * d], u.data(), d);
  std::vector<int64_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    if (p[a] != p[b]) return p[a] < p[b];
    return members[a] < members[b];  // equal projections: lower token index first
  });
  left.clear();
  right.clear();
  for (int64_t r = 0; r < n; ++r) (r < n_left ? left : right).push_back(members[order[r]]);
  std::sort(left.begin(), left.end());
  std::sort(right.begin(), right.end());
}

struct Node {
  std::vector<int64_t> members;  // ascending
};

// Whole tree, level by level: the nodes of one level are independent, so
// they are split by separate workers; a level with fewer nodes than workers
// gives the spare workers to each node's covariance rows. The left child's
// groups come first, so children are kept in order.
void pddp_group(const double *q_in, int N, int d, int T, int iters, bool whiten, int threads, int64_t *perm) {
  std::vector<double> zbuf;
  const double *q = q_in;
  int root_start = -1;
  if (whiten) {
    zbuf.resize((size_t)N * d);
    std::vector<double> var(d);
    standardize(q_in, N, d, zbuf.data(), var.data());
    q = zbuf.data();
    // exact arithmetic ties every standardized root variance at 1: the root
    // starts at the lowest dimension of nonzero variance
    root_start = 0;
    for (int c = 0; c < d; ++c)
      if (var[c] > 0.0) {
        root_start = c;
        break;
      }
  }
  std::vector<Node> level(1);
  level[0].members.resize(N);
  std::iota(level[0].members.begin(), level[0].members.end(), 0);
  bool root = true;
  std::vector<int64_t> out;
  out.reserve(N);
  for (;;) {
    bool any_split = false;
    for (const Node &nd : level)
      if ((int64_t)nd.members.size() > T) any_split = true;
    if (!any_split) break;
    std::vector<Node> next(2 * level.size());
    const int inner = std::max(1, threads / (int)level.size());
    const int start = root ? root_start : -1;
    parallel_for((int64_t)level.size(), threads, [&](int64_t i) {
      const std::vector<int64_t> &m = level[i].members;
      const int64_t n = (int64_t)m.size();
      const int64_t G = (n + T - 1) / T;
      if (G <= 1) {  // a leaf: it moves down unchanged
        next[2 * i].members = m;
        return;
      }
#if ORC_MUTANT == 9
      const int64_t n_left = ((G + 1) / 2) * T;  // planted: the larger half left
#else
      const int64_t n_left = (G / 2) * T;
#endif
      split_node(q, d, m, n_left, iters, start, inner, next[2 * i].members, next[2 * i + 1].members);
    });
    root = false;
    std::vector<Node> kept;
    kept.reserve(next.size());
    for (auto &nd : next)
      if (!nd.members.empty()) kept.push_back(std::move(nd));
    level.swap(kept);
  }
  for (const Node &nd : level) out.insert(out.end(), nd.members.begin(), nd.members.end());
  std::copy(out.begin(), out.end(), perm);
}

// ---------------------------------------------------------------------------
// step 2: dense attention with per-row log-sum-exp
// ---------------------------------------------------------------------------
// s_ij = scale q_i.k_j; L_i = max_j s_ij + ln sum_j exp(s_ij - max);
// O_i = sum_j exp(s_ij - L_i) v_j. Rows are independent.
void dense_lse(const double *qr, int M, const double *k, const double *v, int N, int d, double scale,
               int threads, double *o, double *lse) {
  parallel_for(M, threads, [&](int64_t i) {
    std::vector<double> s(N);
    double m = -INFINITY;
    for (int j = 0; j < N; ++j) {
#if ORC_MUTANT == 1
      s[j] = dot(qr + i * d, k + (int64_t)j * d, d);  // planted: scale dropped
#else
      s[j] = scale * dot(qr + i * d, k + (int64_t)j * d, d);
#endif
      m = std::max(m, s[j]);
    }
    double z = 0.0;
    for (int j = 0; j < N; ++j) z += std::exp(s[j] - m);
#if ORC_MUTANT == 2
    const double L = std::log(z);  // planted: the max term dropped
#else
    const double L = m + std::log(z);
#endif
    std::vector<double> acc(d, 0.0);
    for (int j = 0; j < N; ++j) {
      const double p = std::exp(s[j] - L);
#if ORC_MUTANT == 3
      const double *vj = v + (int64_t)(N - 1 - j) * d;  // planted: values paired with the wrong keys
#else
      const double *vj = v + (int64_t)j * d;
#endif
      for (int c = 0; c < d; ++c) acc[c] += p * vj[c];
    }
    for (int c = 0; c < d; ++c) o[i * d + c] = acc[c];
    lse[i] = L;
  });
}

// ---------------------------------------------------------------------------
// step 2 (cont.): exact probabilities summed over a group, top-K
// ---------------------------------------------------------------------------
// A_j = sum_i exp(scale q_i.k_j - L_i) over the group's rows i, in row order.
// Key columns are independent.
void group_mass(const double *qg, int M, const double *k, int N, int d, const double *lse, double scale,
                int threads, double *A) {
  const int64_t chunk = 256;
  parallel_for((N + chunk - 1) / chunk, threads, [&](int64_t cb) {
    const int64_t j1 = std::min<int64_t>(N, (cb + 1) * chunk);
    for (int64_t j = cb * chunk; j < j1; ++j) {
      double a = 0.0;
      for (int i = 0; i < M; ++i) {
#if ORC_MUTANT == 4
        a += std::exp(scale * dot(qg + (int64_t)i * d, k + j * d, d) + lse[i]);  // planted: wrong sign
#else
        a += std::exp(scale * dot(qg + (int64_t)i * d, k + j * d, d) - lse[i]);
#endif
      }
      A[j] = a;
    }
  });
}

// The K keys of largest mass, equal mass -> lower index first; ascending.
void topk_select(const double *A, int N, int K, int64_t *idx) {
  std::vector<int64_t> order(N);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    if (A[a] != A[b]) return A[a] > A[b];
#if ORC_MUTANT == 5
    return a > b;  // planted: ties to the higher index
#else
    return a < b;
#endif
  });
  std::vector<int64_t> sel(order.begin(), order.begin() + K);
  std::sort(sel.begin(), sel.end());
  std::copy(sel.begin(), sel.end(), idx);
}

// ---------------------------------------------------------------------------
// steps 3-4: sparse attention, residual, reuse
// ---------------------------------------------------------------------------
// Softmax over the selected keys only (renormalised), keys in ascending order.
void sparse_attention(const double *qr, int M, const double *k, const double *v, int d, const int64_t *idx,
                      int K, double scale, double *o) {
  std::vector<double> s(K);
  std::vector<double> acc(d);
  for (int i = 0; i < M; ++i) {
    double m = -INFINITY;
    for (int t = 0; t < K; ++t) {
      s[t] = scale * dot(qr + (int64_t)i * d, k + idx[t] * d, d);
      m = std::max(m, s[t]);
    }
    double z = 0.0;
    for (int t = 0; t < K; ++t) {
      s[t] = std::exp(s[t] - m);
      z += s[t];
    }
    std::fill(acc.begin(), acc.end(), 0.0);
    for (int t = 0; t < K; ++t) {
      const double *vj = v + idx[t] * d;
      for (int c = 0; c < d; ++c) acc[c] += s[t] * vj[c];
    }
    for (int c = 0; c < d; ++c)
#if ORC_MUTANT == 6
      o[(int64_t)i * d + c] = acc[c];  // planted: not renormalised
#else
      o[(int64_t)i * d + c] = acc[c] / z;
#endif
  }
}

// R = bf16(O_dense_stored - O_sparse)
void residual(const double *od, const double *osp, int64_t n, double *r) {
  for (int64_t e = 0; e < n; ++e)
#if ORC_MUTANT == 11
    r[e] = round_bf16_one(osp[e] - od[e]);  // planted: flipped difference
#else
    r[e] = round_bf16_one(od[e] - osp[e]);
#endif
}

}  // namespace

extern "C" {

int orc_version(void) { return 1; }
int orc_mutant(void) { return ORC_MUTANT; }

void orc_round_bf16(const double *x, int64_t n, double *out) {
  for (int64_t e = 0; e < n; ++e) out[e] = round_bf16_one(x[e]);
}

void orc_principal_direction(const double *C, int32_t d, int32_t iters, int32_t start, double *u) {
  principal_direction(C, d, iters, start, u);
}

void orc_standardize(const double *q, int32_t N, int32_t d, double *z, double *var) { standardize(q, N, d, z, var); }

void orc_pddp_group(const double *q, int32_t N, int32_t d, int32_t T, int32_t iters, int32_t whiten,
                    int32_t threads, int64_t *perm) {
  pddp_group(q, N, d, T, iters, whiten != 0, threads, perm);
}

void orc_dense_lse(const double *q_rows, int32_t M, const double *k, const double *v, int32_t N, int32_t d,
                   double scale, int32_t threads, double *o, double *lse) {
  dense_lse(q_rows, M, k, v, N, d, scale, threads, o, lse);
}

void orc_group_mass(const double *q_group, int32_t M, const double *k, int32_t N, int32_t d, const double *lse,
                    double scale, int32_t threads, double *A) {
  group_mass(q_group, M, k, N, d, lse, scale, threads, A);
}

void orc_topk_select(const double *A, int32_t N, int32_t K, int64_t *idx) { topk_select(A, N, K, idx); }

void orc_sparse_attention(const double *q_rows, int32_t M, const double *k, const double *v, int32_t d,
                          const int64_t *idx, int32_t K, double scale, double *o) {
  sparse_attention(q_rows, M, k, v, d, idx, K, scale, o);
}

void orc_residual(const double *o_dense, const double *o_sparse, int64_t n, double *r) {
  residual(o_dense, o_sparse, n, r);
}

// bf16(SparseAttn(fresh Q, K, V; cached idx) + cached R)
void orc_reuse_output(const double *q_rows, int32_t M, const double *k, const double *v, int32_t d,
                      const int64_t *idx, int32_t K, const double *r, double scale, double *o) {
  sparse_attention(q_rows, M, k, v, d, idx, K, scale, o);
  for (int64_t e = 0; e < (int64_t)M * d; ++e) o[e] = round_bf16_one(o[e] + r[e]);
}

// Block granularity (paper landing page, Tables 3-4, the granularity
// ablation): block b holds keys [b*block, (b+1)*block); its mass is the sum
// of its keys' group mass, in key order. Only the floor(N/block) full blocks
// compete; the `nblocks` of largest mass win, equal mass -> lower block. The
// winners' keys are written block by block, ascending.
void orc_block_select(const double *A, int32_t N, int32_t block, int32_t nblocks, int64_t *idx) {
#if ORC_MUTANT == 13
  const int64_t nfull = (N + block - 1) / block;  // planted: the short last block competes
#else
  const int64_t nfull = N / block;
#endif
  std::vector<double> bm(nfull, 0.0);
  for (int64_t b = 0; b < nfull; ++b)
    for (int64_t t = 0; t < block && b * block + t < N; ++t) bm[b] += A[b * block + t];
  std::vector<int64_t> sel(nblocks);
  topk_select(bm.data(), (int)nfull, nblocks, sel.data());
  for (int64_t i = 0; i < nblocks; ++i)
    for (int64_t t = 0; t < block; ++t) idx[i * block + t] = std::min<int64_t>(sel[i] * block + t, N - 1);
}

// Recall of a selection: the mean over the group's n_rows query rows of the
// probability mass its selected keys carry, (1/n_rows) sum_{j in idx} A_j.
double orc_group_recall(const double *A, const int64_t *idx, int32_t K, int32_t n_rows) {
  double s = 0.0;
  for (int32_t t = 0; t < K; ++t) s += A[idx[t]];
#if ORC_MUTANT == 14
  return s / K;  // planted: divided by the key count
#else
  return s / n_rows;
#endif
}

// Relative L1 error: sum |x - ref| / sum |ref|.
double orc_rel_l1(const double *x, const double *ref, int64_t n) {
  double num = 0.0, den = 0.0;
  for (int64_t e = 0; e < n; ++e) {
    num += std::fabs(x[e] - ref[e]);
    den += std::fabs(ref[e]);
  }
  return num / den;
}

// A head's reuse step over groups: entry e of `gids` (or e itself when gids
// is NULL) names group g, whose rows are perm[g*T : min((g+1)*T, N)] and
// whose indices are idx[e]; each entry on its own worker. q, k, v, r and out
// are [N][d] by token; only the named groups' rows of out are written.
void orc_reuse_head(const double *q, const double *k, const double *v, int32_t N, int32_t d, const int64_t *perm,
                    int32_t T, const int64_t *gids, int64_t n_groups, const int64_t *idx, int32_t K,
                    const double *r, double scale, int32_t threads, double *out) {
  parallel_for(n_groups, threads, [&](int64_t e) {
    const int64_t g = gids ? gids[e] : e;
    const int64_t r0 = g * T, r1 = std::min<int64_t>(N, r0 + T), M = r1 - r0;
    std::vector<double> qg((size_t)M * d), rg((size_t)M * d), og((size_t)M * d);
    for (int64_t t = 0; t < M; ++t) {
      std::memcpy(&qg[(size_t)t * d], q + perm[r0 + t] * d, sizeof(double) * d);
      std::memcpy(&rg[(size_t)t * d], r + perm[r0 + t] * d, sizeof(double) * d);
    }
    orc_reuse_output(qg.data(), (int32_t)M, k, v, d, idx + e * K, K, rg.data(), scale, og.data());
    for (int64_t t = 0; t < M; ++t) std::memcpy(out + perm[r0 + t] * d, &og[(size_t)t * d], sizeof(double) * d);
  });
}

// A whole head's anchor step on given groups: dense O (stored bf16) and L of
// every row, then per group the mass row, its top-K and R, each group on its
// own worker. perm is the caller's (e.g. from orc_pddp_group). Outputs by
// token: o_dense, r [N][d], lse [N]; per group: idx [G][K], mass [G][N]
// (mass may be NULL).
void orc_anchor_head(const double *q, const double *k, const double *v, int32_t N, int32_t d, const int64_t *perm,
                     int32_t T, int32_t K, double scale, int32_t threads, double *o_dense, double *lse,
                     int64_t *idx, double *mass, double *r) {
  dense_lse(q, N, k, v, N, d, scale, threads, o_dense, lse);
  for (int64_t e = 0; e < (int64_t)N * d; ++e) o_dense[e] = round_bf16_one(o_dense[e]);
  const int64_t G = (N + T - 1) / T;
  parallel_for(G, threads, [&](int64_t g) {
    const int64_t r0 = g * T, r1 = std::min<int64_t>(N, r0 + T), M = r1 - r0;
    std::vector<double> qg((size_t)M * d), lg(M), A(N), osp((size_t)M * d), odg((size_t)M * d), rg((size_t)M * d);
    for (int64_t t = 0; t < M; ++t) {
      std::memcpy(&qg[(size_t)t * d], q + perm[r0 + t] * d, sizeof(double) * d);
      std::memcpy(&odg[(size_t)t * d], o_dense + perm[r0 + t] * d, sizeof(double) * d);
      lg[t] = lse[perm[r0 + t]];
    }
    group_mass(qg.data(), (int)M, k, N, d, lg.data(), scale, 1, A.data());
    topk_select(A.data(), N, K, idx + g * K);
    sparse_attention(qg.data(), (int)M, k, v, d, idx + g * K, K, scale, osp.data());
    residual(odg.data(), osp.data(), M * d, rg.data());
    for (int64_t t = 0; t < M; ++t) std::memcpy(r + perm[r0 + t] * d, &rg[(size_t)t * d], sizeof(double) * d);
    if (mass) std::memcpy(mass + g * N, A.data(), sizeof(double) * N);
  });
}

}  // extern "C"
