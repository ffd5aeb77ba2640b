// C-ABI of libmcsparse: argument validation, dispatch to the gfx950 kernels,
// error reporting. Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "mcs_internal.hpp"
#include "mcsparse.h"

namespace {

thread_local std::string g_last_error;

mcs_status_t fail(mcs_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mcs_status_t ok() { return MCS_OK; }

mcs_status_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return MCS_OK;
  return fail(MCS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// extent in elements of a [B,N,H,d] tensor under the descriptor's strides
// (check_desc has bounded it, so this does not overflow)
int64_t extent(const mcs_attn_desc_t *d) {
  return (int64_t)(d->batch - 1) * d->stride_b + (int64_t)(d->seqlen - 1) * d->stride_n +
         (int64_t)(d->heads - 1) * d->stride_h + d->head_dim;
}

// [a, a + a_bytes) and [b, b + b_bytes) share a byte
bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)b_bytes && y < x + (uintptr_t)a_bytes;
}

// Rows of a [B,N,H,d] layout do not overlap when, taking the dimensions of
// size > 1 by increasing stride, each stride is at least the span of the
// dimensions inside it (a row of d elements innermost). The span is kept
// below 2^56 elements so the extent arithmetic stays in range.
bool rows_disjoint(const mcs_attn_desc_t *d, bool *too_large) {
  struct Dim { int64_t count, stride; } dims[3] = {
      {d->batch, d->stride_b}, {d->seqlen, d->stride_n}, {d->heads, d->stride_h}};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (dims[j].stride < dims[i].stride) std::swap(dims[i], dims[j]);
  constexpr int64_t kMaxSpan = (int64_t)1 << 56;
  int64_t span = d->head_dim;
  *too_large = false;
  for (const Dim &x : dims) {
    if (x.count <= 1) continue;
    if (x.stride < span) return false;
    int64_t more;
    if (__builtin_mul_overflow(x.count - 1, x.stride, &more) || __builtin_add_overflow(span, more, &span) ||
        span > kMaxSpan) {
      *too_large = true;
      return true;
    }
  }
  return true;
}

constexpr int32_t kMaxSeqlen = 1 << 28;

mcs_status_t check_desc(const mcs_attn_desc_t *d) {
  if (!d) return fail(MCS_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 1 || d->heads < 1 || d->seqlen < 1)
    return fail(MCS_ERR_INVALID_ARGUMENT, "batch, heads and seqlen must be >= 1 (got %d, %d, %d)",
                d->batch, d->heads, d->seqlen);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MCS_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->seqlen > kMaxSeqlen) return fail(MCS_ERR_UNSUPPORTED, "seqlen %d above %d", d->seqlen, kMaxSeqlen);
  if ((int64_t)d->batch * d->heads > (((int64_t)1 << 31) - 1) / d->seqlen)
    return fail(MCS_ERR_INVALID_ARGUMENT, "batch*heads*seqlen exceeds 2^31-1");
  if (d->stride_b < 0 || d->stride_n < 0 || d->stride_h < 0 || d->stride_b % 8 || d->stride_n % 8 ||
      d->stride_h % 8)
    return fail(MCS_ERR_INVALID_ARGUMENT, "strides must be non-negative multiples of 8 elements");
  bool too_large;
  if (!rows_disjoint(d, &too_large))
    return fail(MCS_ERR_INVALID_ARGUMENT, "strides make rows of the [B,N,H,d] layout overlap");
  if (too_large) return fail(MCS_ERR_INVALID_ARGUMENT, "strides span more than 2^56 elements");
  if (!std::isfinite(d->scale)) return fail(MCS_ERR_INVALID_ARGUMENT, "scale is not finite");
  // the kernels address one head's rows with 32-bit byte offsets
  if ((int64_t)(d->seqlen - 1) * d->stride_n * 2 + d->head_dim * 2 > (int64_t)UINT32_MAX)
    return fail(MCS_ERR_UNSUPPORTED, "one head's rows span more than 4 GiB ((N-1)*stride_n too large)");
  return ok();
}

mcs_status_t check_tensor(const void *p, const char *name) {
  if (!p) return fail(MCS_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(MCS_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return ok();
}

mcs_status_t check_ptr(const void *p, const char *name) {
  if (!p) return fail(MCS_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (((uintptr_t)p & 3u) != 0) return fail(MCS_ERR_INVALID_ARGUMENT, "%s is not 4-byte aligned", name);
  return ok();
}

// the grouping kernels run a grid row per (batch, head): at most 65535
constexpr int64_t kMaxPddpHeads = 65535;

mcs_status_t check_pddp_heads(const mcs_attn_desc_t *d) {
  if ((int64_t)d->batch * d->heads > kMaxPddpHeads)
    return fail(MCS_ERR_UNSUPPORTED, "batch*heads %lld above the grouping's %lld",
                (long long)d->batch * d->heads, (long long)kMaxPddpHeads);
  return ok();
}

mcs_status_t check_group(int32_t T) {
  if (T != 64 && T != 128) return fail(MCS_ERR_UNSUPPORTED, "group_size %d not supported (64 or 128)", T);
  return ok();
}

mcs_status_t check_topk(const mcs_attn_desc_t *d, int32_t K) {
  if (K < 1 || K > d->seqlen) return fail(MCS_ERR_INVALID_ARGUMENT, "topk %d outside [1, %d]", K, d->seqlen);
  return ok();
}

#define MCS_TRY(x)                   \
  do {                               \
    const mcs_status_t _st = (x);    \
    if (_st != MCS_OK) return _st;   \
  } while (0)

mcs::AttnArgs attn_args(const mcs_attn_desc_t *d) {
  mcs::AttnArgs a{};
  a.sb = d->stride_b;
  a.sn = d->stride_n;
  a.sh = d->stride_h;
  a.B = d->batch;
  a.H = d->heads;
  a.N = d->seqlen;
  a.scale_log2 = d->scale * 1.4426950408889634f;
  return a;
}

int32_t groups_of(const mcs_attn_desc_t *d, int32_t T) { return (d->seqlen + T - 1) / T; }

struct Buf {
  const void *p;
  int64_t bytes;
  const char *name;
};

// an output must share no byte with any other buffer of the call (NULL
// entries are skipped)
mcs_status_t check_disjoint(Buf out, std::initializer_list<Buf> others) {
  if (!out.p) return ok();
  for (const Buf &b : others)
    if (b.p && overlaps(out.p, out.bytes, b.p, b.bytes))
      return fail(MCS_ERR_INVALID_ARGUMENT, "%s overlaps %s", out.name, b.name);
  return ok();
}

// byte extents of the call's buffers
int64_t tensor_bytes(const mcs_attn_desc_t *d) { return extent(d) * 2; }
int64_t per_token_bytes(const mcs_attn_desc_t *d) { return (int64_t)d->batch * d->heads * d->seqlen * 4; }
int64_t per_group_bytes(const mcs_attn_desc_t *d, int32_t T, int64_t per_row) {
  return (int64_t)d->batch * d->heads * groups_of(d, T) * per_row * 4;
}

}  // namespace

namespace mcs {
void set_last_error(const char *msg) { g_last_error = msg; }
}  // namespace mcs

extern "C" {

int32_t mcs_version(void) { return 100; }

const char *mcs_last_error(void) { return g_last_error.c_str(); }

mcs_status_t mcs_pddp_group_workspace_size(const mcs_attn_desc_t *desc, int32_t group_size,
                                           size_t *bytes) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_pddp_heads(desc));
  MCS_TRY(check_group(group_size));
  if (!bytes) return fail(MCS_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = mcs::pddp_workspace_bytes(desc->batch, desc->heads, desc->seqlen, desc->head_dim, group_size);
  return ok();
}

mcs_status_t mcs_pddp_group_ex(const mcs_attn_desc_t *desc, const void *q, int32_t group_size,
                               int32_t power_iters, uint32_t flags, int32_t *perm, void *ws,
                               size_t ws_bytes, mcs_stream_t stream) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_pddp_heads(desc));
  MCS_TRY(check_group(group_size));
  MCS_TRY(check_tensor(q, "q"));
  MCS_TRY(check_ptr(perm, "perm"));
  if (power_iters < 1 || power_iters > 64)
    return fail(MCS_ERR_INVALID_ARGUMENT, "power_iters %d outside [1, 64]", power_iters);
  if (flags & ~MCS_PDDP_WHITEN) return fail(MCS_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags);
  const size_t need = mcs::pddp_workspace_bytes(desc->batch, desc->heads, desc->seqlen, desc->head_dim, group_size);
  if (ws_bytes < need) return fail(MCS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!ws || !aligned16(ws)) return fail(MCS_ERR_INVALID_ARGUMENT, "ws is NULL or not 16-byte aligned");
  const int64_t tb = tensor_bytes(desc), pb = per_token_bytes(desc);
  MCS_TRY(check_disjoint({perm, pb, "perm"}, {{q, tb, "q"}, {ws, (int64_t)need, "ws"}}));
  MCS_TRY(check_disjoint({ws, (int64_t)need, "ws"}, {{q, tb, "q"}}));
  return hip_status(mcs::run_pddp((const uint16_t *)q, desc->stride_b, desc->stride_n, desc->stride_h,
                                  desc->batch, desc->heads, desc->seqlen, desc->head_dim, group_size,
                                  power_iters, (flags & MCS_PDDP_WHITEN) != 0, perm, ws, ws_bytes,
                                  (hipStream_t)stream),
                    "mcs_pddp_group");
}

mcs_status_t mcs_pddp_group_noalloc(const mcs_attn_desc_t *desc, const void *q, int32_t group_size,
                                    int32_t power_iters, uint32_t flags, int32_t *perm, mcs_stream_t stream) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_pddp_heads(desc));
  MCS_TRY(check_group(group_size));
  MCS_TRY(check_tensor(q, "q"));
  MCS_TRY(check_ptr(perm, "perm"));
  if (power_iters < 1 || power_iters > 64)
    return fail(MCS_ERR_INVALID_ARGUMENT, "power_iters %d outside [1, 64]", power_iters);
  if (flags & ~MCS_PDDP_WHITEN) return fail(MCS_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags);
  const int N = desc->seqlen, D = desc->head_dim, H = desc->heads;
  // heads are independent: run them in chunks whose workspace fits the
  // library's scratch (the plan tables are shared by a chunk's heads)
  const size_t one = mcs::pddp_workspace_bytes(1, 1, N, D, group_size);
  if (one > mcs::kScratchBytes)
    return fail(MCS_ERR_UNSUPPORTED, "one head needs %zu bytes of PDDP scratch, above the library's %zu",
                one, mcs::kScratchBytes);
  const size_t per_head = mcs::pddp_workspace_bytes(1, 2, N, D, group_size) - one;
  int chunk = per_head == 0 ? H : (int)std::min<size_t>((size_t)H, 1 + (mcs::kScratchBytes - one) / per_head);
  while (chunk > 1 && mcs::pddp_workspace_bytes(1, chunk, N, D, group_size) > mcs::kScratchBytes) --chunk;
  MCS_TRY(check_disjoint({perm, per_token_bytes(desc), "perm"}, {{q, tensor_bytes(desc), "q"}}));
  void *ws = nullptr;
  const hipError_t e = mcs::scratch_address(&ws);
  if (e != hipSuccess) return hip_status(e, "mcs_pddp_group_noalloc (scratch address)");
  const uint16_t *qb = (const uint16_t *)q;
  for (int b = 0; b < desc->batch; ++b)
    for (int h0 = 0; h0 < H; h0 += chunk) {
      const int nh = std::min(chunk, H - h0);
      const uint16_t *qc = qb + (int64_t)b * desc->stride_b + (int64_t)h0 * desc->stride_h;
      int32_t *pc = perm + ((int64_t)b * H + h0) * N;
      const hipError_t le = mcs::run_pddp(qc, desc->stride_b, desc->stride_n, desc->stride_h, 1, nh, N, D,
                                          group_size, power_iters, (flags & MCS_PDDP_WHITEN) != 0, pc, ws,
                                          mcs::kScratchBytes, (hipStream_t)stream);
      if (le != hipSuccess) return hip_status(le, "mcs_pddp_group_noalloc");
    }
  return ok();
}

mcs_status_t mcs_pddp_group(const mcs_attn_desc_t *desc, const void *q, int32_t group_size,
                            int32_t power_iters, int32_t *perm, void *ws, size_t ws_bytes,
                            mcs_stream_t stream) {
  return mcs_pddp_group_ex(desc, q, group_size, power_iters, 0u, perm, ws, ws_bytes, stream);
}

mcs_status_t mcs_anchor_dense_lse(const mcs_attn_desc_t *desc, const void *q, const void *k,
                                  const void *v, void *o, float *lse, mcs_stream_t stream) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_tensor(q, "q"));
  MCS_TRY(check_tensor(k, "k"));
  MCS_TRY(check_tensor(v, "v"));
  MCS_TRY(check_tensor(o, "o"));
  if (lse) MCS_TRY(check_ptr(lse, "lse"));
  const int64_t tb = tensor_bytes(desc), lb = per_token_bytes(desc);
  MCS_TRY(check_disjoint({o, tb, "o"}, {{q, tb, "q"}, {k, tb, "k"}, {v, tb, "v"}, {lse, lb, "lse"}}));
  MCS_TRY(check_disjoint({lse, lb, "lse"}, {{q, tb, "q"}, {k, tb, "k"}, {v, tb, "v"}}));
  mcs::AttnArgs a = attn_args(desc);
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.out = (uint16_t *)o;
  a.lse = lse;
  a.rows = 256;  // dense tile: 8 waves x 32 rows
  a.G = groups_of(desc, a.rows);
  return hip_status(mcs::launch_attention(mcs::kModeDense, desc->head_dim, a, (hipStream_t)stream),
                    "mcs_anchor_dense_lse");
}

mcs_status_t mcs_anchor_select_topk_workspace_size(const mcs_attn_desc_t *desc, int32_t group_size,
                                                   int32_t topk, size_t *bytes) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_group(group_size));
  MCS_TRY(check_topk(desc, topk));
  if (!bytes) return fail(MCS_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = (size_t)desc->batch * desc->heads * groups_of(desc, group_size) * desc->seqlen * sizeof(float);
  return ok();
}

mcs_status_t mcs_anchor_select_topk(const mcs_attn_desc_t *desc, const void *q, const void *k,
                                    const float *lse, const int32_t *perm, int32_t group_size,
                                    int32_t topk, int32_t *kv_idx, float *group_mass, void *ws,
                                    size_t ws_bytes, mcs_stream_t stream) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_group(group_size));
  MCS_TRY(check_topk(desc, topk));
  MCS_TRY(check_tensor(q, "q"));
  MCS_TRY(check_tensor(k, "k"));
  MCS_TRY(check_ptr(lse, "lse"));
  MCS_TRY(check_ptr(perm, "perm"));
  MCS_TRY(check_ptr(kv_idx, "kv_idx"));
  float *mass = group_mass;
  if (mass) {
    MCS_TRY(check_ptr(mass, "group_mass"));
  } else {
    const size_t need = (size_t)desc->batch * desc->heads * groups_of(desc, group_size) * desc->seqlen * sizeof(float);
    if (ws_bytes < need) return fail(MCS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    MCS_TRY(check_ptr(ws, "ws"));
    mass = (float *)ws;
  }
  {
    const int64_t tb = tensor_bytes(desc), lb = per_token_bytes(desc);
    const int64_t mb = per_group_bytes(desc, group_size, desc->seqlen), ib = per_group_bytes(desc, group_size, topk);
    MCS_TRY(check_disjoint({mass, mb, group_mass ? "group_mass" : "ws"},
                           {{q, tb, "q"}, {k, tb, "k"}, {lse, lb, "lse"}, {perm, lb, "perm"}, {kv_idx, ib, "kv_idx"}}));
    MCS_TRY(check_disjoint({kv_idx, ib, "kv_idx"}, {{q, tb, "q"}, {k, tb, "k"}, {lse, lb, "lse"}, {perm, lb, "perm"}}));
  }
  mcs::SelectArgs a{};
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.lse = lse;
  a.perm = perm;
  a.mass = mass;
  a.idx = kv_idx;
  a.sb = desc->stride_b;
  a.sn = desc->stride_n;
  a.sh = desc->stride_h;
  a.B = desc->batch;
  a.H = desc->heads;
  a.N = desc->seqlen;
  a.T = group_size;
  a.G = groups_of(desc, group_size);
  a.K = topk;
  a.scale_log2 = desc->scale * 1.4426950408889634f;
  return hip_status(mcs::launch_select(desc->head_dim, a, (hipStream_t)stream), "mcs_anchor_select_topk");
}

namespace {
mcs_status_t check_block_args(const mcs_attn_desc_t *desc, int32_t group_size, int32_t block, int32_t nblocks) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_group(group_size));
  if (block < 64 || block > 4096 || block % 64)
    return fail(MCS_ERR_UNSUPPORTED, "block %d not supported (a multiple of 64 in [64, 4096])", block);
  const int32_t nfull = desc->seqlen / block;
  if (nfull < 1) return fail(MCS_ERR_INVALID_ARGUMENT, "seqlen %d holds no full block of %d keys", desc->seqlen, block);
  if (nblocks < 1 || nblocks > nfull)
    return fail(MCS_ERR_INVALID_ARGUMENT, "nblocks %d outside [1, %d] (full blocks)", nblocks, nfull);
  return ok();
}
}  // namespace

mcs_status_t mcs_select_blocks_workspace_size(const mcs_attn_desc_t *desc, int32_t group_size, int32_t block,
                                              int32_t nblocks, size_t *bytes) {
  MCS_TRY(check_block_args(desc, group_size, block, nblocks));
  if (!bytes) return fail(MCS_ERR_INVALID_ARGUMENT, "bytes is NULL");
  const int64_t rows = (int64_t)desc->batch * desc->heads * groups_of(desc, group_size);
  *bytes = mcs::select_blocks_ws_bytes(rows, desc->seqlen, block, nblocks);
  return ok();
}

mcs_status_t mcs_select_blocks(const mcs_attn_desc_t *desc, const float *group_mass, int32_t group_size,
                               int32_t block, int32_t nblocks, int32_t *kv_idx, void *ws, size_t ws_bytes,
                               mcs_stream_t stream) {
  MCS_TRY(check_block_args(desc, group_size, block, nblocks));
  MCS_TRY(check_ptr(group_mass, "group_mass"));
  MCS_TRY(check_ptr(kv_idx, "kv_idx"));
  const int64_t rows = (int64_t)desc->batch * desc->heads * groups_of(desc, group_size);
  const size_t need = mcs::select_blocks_ws_bytes(rows, desc->seqlen, block, nblocks);
  if (ws_bytes < need) return fail(MCS_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!ws || !aligned16(ws)) return fail(MCS_ERR_INVALID_ARGUMENT, "ws is NULL or not 16-byte aligned");
  const int64_t mb = per_group_bytes(desc, group_size, desc->seqlen);
  const int64_t ib = per_group_bytes(desc, group_size, (int64_t)nblocks * block);
  MCS_TRY(check_disjoint({kv_idx, ib, "kv_idx"}, {{group_mass, mb, "group_mass"}, {ws, (int64_t)need, "ws"}}));
  MCS_TRY(check_disjoint({ws, (int64_t)need, "ws"}, {{group_mass, mb, "group_mass"}}));
  return hip_status(mcs::launch_select_blocks(group_mass, rows, desc->seqlen, block, nblocks, kv_idx, ws,
                                              (hipStream_t)stream),
                    "mcs_select_blocks");
}

mcs_status_t mcs_residual(const mcs_attn_desc_t *desc, const void *q, const void *k, const void *v,
                          const void *o_dense, const int32_t *perm, int32_t group_size,
                          const int32_t *kv_idx, int32_t topk, void *r, mcs_stream_t stream) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_group(group_size));
  MCS_TRY(check_topk(desc, topk));
  MCS_TRY(check_tensor(q, "q"));
  MCS_TRY(check_tensor(k, "k"));
  MCS_TRY(check_tensor(v, "v"));
  MCS_TRY(check_tensor(o_dense, "o_dense"));
  MCS_TRY(check_tensor(r, "r"));
  MCS_TRY(check_ptr(perm, "perm"));
  MCS_TRY(check_ptr(kv_idx, "kv_idx"));
  const int64_t tb = tensor_bytes(desc);
  MCS_TRY(check_disjoint({r, tb, "r"}, {{q, tb, "q"}, {k, tb, "k"}, {v, tb, "v"}, {o_dense, tb, "o_dense"},
                                        {perm, per_token_bytes(desc), "perm"},
                                        {kv_idx, per_group_bytes(desc, group_size, topk), "kv_idx"}}));
  mcs::AttnArgs a = attn_args(desc);
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.aux = (const uint16_t *)o_dense;
  a.out = (uint16_t *)r;
  a.perm = perm;
  a.idx = kv_idx;
  a.rows = group_size;
  a.G = groups_of(desc, group_size);
  a.K = topk;
  return hip_status(mcs::launch_attention(mcs::kModeResidual, desc->head_dim, a, (hipStream_t)stream),
                    "mcs_residual");
}

mcs_status_t mcs_sparse_apply(const mcs_attn_desc_t *desc, const void *q, const void *k,
                              const void *v, const int32_t *perm, int32_t group_size,
                              const int32_t *kv_idx, int32_t topk, const void *r, void *o,
                              mcs_stream_t stream) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_group(group_size));
  MCS_TRY(check_topk(desc, topk));
  MCS_TRY(check_tensor(q, "q"));
  MCS_TRY(check_tensor(k, "k"));
  MCS_TRY(check_tensor(v, "v"));
  MCS_TRY(check_tensor(o, "o"));
  if (r) MCS_TRY(check_tensor(r, "r"));
  MCS_TRY(check_ptr(perm, "perm"));
  MCS_TRY(check_ptr(kv_idx, "kv_idx"));
  const int64_t tb = tensor_bytes(desc);
  MCS_TRY(check_disjoint({o, tb, "o"}, {{q, tb, "q"}, {k, tb, "k"}, {v, tb, "v"}, {r, tb, "r"},
                                        {perm, per_token_bytes(desc), "perm"},
                                        {kv_idx, per_group_bytes(desc, group_size, topk), "kv_idx"}}));
  mcs::AttnArgs a = attn_args(desc);
  a.q = (const uint16_t *)q;
  a.k = (const uint16_t *)k;
  a.v = (const uint16_t *)v;
  a.aux = (const uint16_t *)r;
  a.out = (uint16_t *)o;
  a.perm = perm;
  a.idx = kv_idx;
  a.rows = group_size;
  a.G = groups_of(desc, group_size);
  a.K = topk;
  return hip_status(mcs::launch_attention(mcs::kModeSparse, desc->head_dim, a, (hipStream_t)stream),
                    "mcs_sparse_apply");
}

mcs_status_t mcs_kv_idx_bitmap_bytes(const mcs_attn_desc_t *desc, int32_t group_size, size_t *bytes) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_group(group_size));
  if (!bytes) return fail(MCS_ERR_INVALID_ARGUMENT, "bytes is NULL");
  *bytes = (size_t)desc->batch * desc->heads * groups_of(desc, group_size) * mcs::idx_bitmap_words(desc->seqlen) * 4;
  return ok();
}

namespace {
// the encoder builds one row's words in LDS (64 KB at most)
constexpr int32_t kMaxBitmapKeys = 64 * 1024 * 8;

mcs_status_t check_code_args(const mcs_attn_desc_t *desc, int32_t group_size, int32_t topk, const void *idx,
                             const void *bitmap) {
  MCS_TRY(check_desc(desc));
  MCS_TRY(check_group(group_size));
  MCS_TRY(check_topk(desc, topk));
  if (desc->seqlen > kMaxBitmapKeys)
    return fail(MCS_ERR_UNSUPPORTED, "seqlen %d above the bitmap codec's %d keys", desc->seqlen, kMaxBitmapKeys);
  MCS_TRY(check_ptr(idx, "kv_idx"));
  MCS_TRY(check_ptr(bitmap, "bitmap"));
  const int64_t rows = (int64_t)desc->batch * desc->heads * groups_of(desc, group_size);
  if (overlaps(idx, rows * topk * 4, bitmap, rows * (int64_t)mcs::idx_bitmap_words(desc->seqlen) * 4))
    return fail(MCS_ERR_INVALID_ARGUMENT, "kv_idx and bitmap overlap");
  return ok();
}
}  // namespace

mcs_status_t mcs_kv_idx_encode(const mcs_attn_desc_t *desc, int32_t group_size, const int32_t *kv_idx,
                               int32_t topk, uint32_t *bitmap, mcs_stream_t stream) {
  MCS_TRY(check_code_args(desc, group_size, topk, kv_idx, bitmap));
  const int64_t rows = (int64_t)desc->batch * desc->heads * groups_of(desc, group_size);
  return hip_status(mcs::launch_idx_encode(kv_idx, rows, topk, desc->seqlen, bitmap, (hipStream_t)stream),
                    "mcs_kv_idx_encode");
}

mcs_status_t mcs_kv_idx_decode(const mcs_attn_desc_t *desc, int32_t group_size, const uint32_t *bitmap,
                               int32_t topk, int32_t *kv_idx, mcs_stream_t stream) {
  MCS_TRY(check_code_args(desc, group_size, topk, kv_idx, bitmap));
  const int64_t rows = (int64_t)desc->batch * desc->heads * groups_of(desc, group_size);
  return hip_status(mcs::launch_idx_decode(bitmap, rows, topk, desc->seqlen, kv_idx, (hipStream_t)stream),
                    "mcs_kv_idx_decode");
}

}  // extern "C"
