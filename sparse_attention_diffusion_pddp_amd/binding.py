"""ctypes binding of libmcsparse (include/mcsparse.h).

Argument marshalling only: torch tensors supply device memory, their
``data_ptr()`` is passed through, and torch's current stream is the HIP
stream. Every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmcsparse.so")

MCS_OK = 0
STATUS_NAMES = {0: "MCS_OK", 1: "MCS_ERR_INVALID_ARGUMENT", 2: "MCS_ERR_UNSUPPORTED",
                3: "MCS_ERR_WORKSPACE", 4: "MCS_ERR_HIP", 5: "MCS_ERR_STATE"}

# (name, restype, argtypes) for every symbol the header declares
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
SIGNATURES = [
    ("mcs_version", _i32, []),
    ("mcs_last_error", ctypes.c_char_p, []),
    ("mcs_pddp_group_workspace_size", _i32, [_p, _i32, ctypes.POINTER(_sz)]),
    ("mcs_pddp_group", _i32, [_p, _p, _i32, _i32, _p, _p, _sz, _p]),
    ("mcs_pddp_group_ex", _i32, [_p, _p, _i32, _i32, ctypes.c_uint32, _p, _p, _sz, _p]),
    ("mcs_pddp_group_noalloc", _i32, [_p, _p, _i32, _i32, ctypes.c_uint32, _p, _p]),
    ("mcs_anchor_dense_lse", _i32, [_p, _p, _p, _p, _p, _p, _p]),
    ("mcs_anchor_select_topk_workspace_size", _i32, [_p, _i32, _i32, ctypes.POINTER(_sz)]),
    ("mcs_anchor_select_topk", _i32, [_p, _p, _p, _p, _p, _i32, _i32, _p, _p, _p, _sz, _p]),
    ("mcs_select_blocks_workspace_size", _i32, [_p, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    ("mcs_select_blocks", _i32, [_p, _p, _i32, _i32, _i32, _p, _p, _sz, _p]),
    ("mcs_residual", _i32, [_p, _p, _p, _p, _p, _p, _i32, _p, _i32, _p, _p]),
    ("mcs_sparse_apply", _i32, [_p, _p, _p, _p, _p, _i32, _p, _i32, _p, _p, _p]),
    ("mcs_kv_idx_bitmap_bytes", _i32, [_p, _i32, ctypes.POINTER(_sz)]),
    ("mcs_kv_idx_encode", _i32, [_p, _i32, _p, _i32, _p, _p]),
    ("mcs_kv_idx_decode", _i32, [_p, _i32, _p, _i32, _p, _p]),
    ("mcs_rcache_create", _i32, [_i32, _sz, ctypes.POINTER(_p)]),
    ("mcs_rcache_store", _i32, [_p, _i32, _p, _p]),
    ("mcs_rcache_prefetch", _i32, [_p, _i32, _p]),
    ("mcs_rcache_acquire", _i32, [_p, _i32, _p, ctypes.POINTER(_p)]),
    ("mcs_rcache_host_ptr", _i32, [_p, _i32, ctypes.POINTER(_p)]),
    ("mcs_rcache_destroy", _i32, [_p]),
]


class Desc(ctypes.Structure):
    """mcs_attn_desc_t"""
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("stride_b", ctypes.c_int64), ("stride_n", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("scale", ctypes.c_float)]


class McsError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmcsparse.so (built by ``python -m sparse_attention_diffusion_pddp_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_attention_diffusion_pddp_amd.build`")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(fn, status):
    if status != MCS_OK:
        raise McsError(fn, status, _lib.mcs_last_error().decode())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t, name, dtype=None, numel=None, contiguous=False):
    """The library takes bare device pointers and cannot see a tensor's
    device, dtype or size: check them here, before the call."""
    if t is None:
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} must hold at least {numel} elements, got {t.numel()}")


def _tensors(*named):
    for name, t in named:
        _dev(t, name, torch.bfloat16)


def _groups(desc: Desc, group_size: int) -> int:
    return (desc.seqlen + group_size - 1) // group_size


def _idx_numel(desc: Desc, group_size: int, topk: int):
    """Elements of a [B][H][G][topk] index array; None when the library will
    reject group_size or topk itself (it then reports its own status)."""
    if group_size not in (64, 128) or not 1 <= topk <= desc.seqlen:
        return None
    return desc.batch * desc.heads * _groups(desc, group_size) * topk


def _per_token(desc: Desc) -> int:
    return desc.batch * desc.heads * desc.seqlen


def desc_for(q: torch.Tensor, scale: float | None = None) -> Desc:
    """Descriptor of a [B, N, H, d] tensor (d contiguous); k, v, o, r share its strides."""
    if q.dim() != 4:
        raise ValueError("expected a [B, N, H, d] tensor")
    if q.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    B, N, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Desc(B, H, N, d, q.stride(0), q.stride(1), q.stride(2), scale)


def _same_layout(ref, *ts):
    for t in ts:
        if t is not None and (t.shape != ref.shape or t.stride() != ref.stride()):
            raise ValueError("q, k, v, o, r must share shape and strides")


def pddp_workspace_size(desc: Desc, group_size: int) -> int:
    lib = load()
    n = ctypes.c_size_t()
    _check("mcs_pddp_group_workspace_size", lib.mcs_pddp_group_workspace_size(ctypes.byref(desc), group_size, ctypes.byref(n)))
    return n.value


def select_workspace_size(desc: Desc, group_size: int, topk: int) -> int:
    lib = load()
    n = ctypes.c_size_t()
    _check("mcs_anchor_select_topk_workspace_size",
           lib.mcs_anchor_select_topk_workspace_size(ctypes.byref(desc), group_size, topk, ctypes.byref(n)))
    return n.value


PDDP_WHITEN = 1  # MCS_PDDP_WHITEN


def pddp_group(q, group_size, perm, ws, power_iters=16, desc=None, stream=None, whiten=False):
    lib = load()
    desc = desc or desc_for(q)
    _tensors(("q", q))
    _dev(perm, "perm", torch.int32, _per_token(desc), contiguous=True)
    _dev(ws, "ws", contiguous=True)
    if whiten:
        _check("mcs_pddp_group_ex", lib.mcs_pddp_group_ex(ctypes.byref(desc), _ptr(q), group_size, power_iters,
                                                          PDDP_WHITEN, _ptr(perm), _ptr(ws),
                                                          ws.numel() * ws.element_size(), _stream(stream)))
        return
    _check("mcs_pddp_group", lib.mcs_pddp_group(ctypes.byref(desc), _ptr(q), group_size, power_iters, _ptr(perm),
                                                _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def pddp_group_noalloc(q, group_size, perm, power_iters=16, desc=None, stream=None, whiten=False):
    """mcs_pddp_group_noalloc: the grouping with the library's own device
    scratch, no workspace argument and no allocation."""
    lib = load()
    desc = desc or desc_for(q)
    _tensors(("q", q))
    _dev(perm, "perm", torch.int32, _per_token(desc), contiguous=True)
    _check("mcs_pddp_group_noalloc",
           lib.mcs_pddp_group_noalloc(ctypes.byref(desc), _ptr(q), group_size, power_iters,
                                      PDDP_WHITEN if whiten else 0, _ptr(perm), _stream(stream)))


def anchor_dense_lse(q, k, v, o, lse=None, desc=None, stream=None):
    lib = load()
    _same_layout(q, k, v, o)
    desc = desc or desc_for(q)
    _tensors(("q", q), ("k", k), ("v", v), ("o", o))
    _dev(lse, "lse", torch.float32, _per_token(desc), contiguous=True)
    _check("mcs_anchor_dense_lse", lib.mcs_anchor_dense_lse(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                                            _ptr(lse), _stream(stream)))


def anchor_select_topk(q, k, lse, perm, group_size, topk, kv_idx, group_mass=None, ws=None, desc=None, stream=None):
    lib = load()
    _same_layout(q, k)
    desc = desc or desc_for(q)
    _tensors(("q", q), ("k", k))
    _dev(lse, "lse", torch.float32, _per_token(desc), contiguous=True)
    _dev(perm, "perm", torch.int32, _per_token(desc), contiguous=True)
    _dev(kv_idx, "kv_idx", torch.int32, _idx_numel(desc, group_size, topk), contiguous=True)
    mass_numel = _idx_numel(desc, group_size, desc.seqlen)
    _dev(group_mass, "group_mass", torch.float32, mass_numel, contiguous=True)
    _dev(ws, "ws", contiguous=True)
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    _check("mcs_anchor_select_topk",
           lib.mcs_anchor_select_topk(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(lse), _ptr(perm), group_size, topk,
                                      _ptr(kv_idx), _ptr(group_mass), _ptr(ws), wsb, _stream(stream)))


def select_blocks_workspace_size(desc: Desc, group_size: int, block: int, nblocks: int) -> int:
    lib = load()
    n = ctypes.c_size_t()
    _check("mcs_select_blocks_workspace_size",
           lib.mcs_select_blocks_workspace_size(ctypes.byref(desc), group_size, block, nblocks, ctypes.byref(n)))
    return n.value


def select_blocks(desc: Desc, group_mass, group_size, block, nblocks, kv_idx, ws=None, stream=None):
    """mcs_select_blocks: the `nblocks` full blocks of `block` keys with the
    largest summed group mass, expanded to ascending key indices
    [B][H][G][nblocks * block]. Allocates the workspace when none is given."""
    lib = load()
    G = _groups(desc, group_size)
    rows = desc.batch * desc.heads * G
    _dev(group_mass, "group_mass", torch.float32, rows * desc.seqlen, contiguous=True)
    _dev(kv_idx, "kv_idx", torch.int32, rows * nblocks * block, contiguous=True)
    if ws is None:
        ws = torch.empty(select_blocks_workspace_size(desc, group_size, block, nblocks), dtype=torch.uint8,
                         device=group_mass.device)
    _dev(ws, "ws", contiguous=True)
    _check("mcs_select_blocks", lib.mcs_select_blocks(ctypes.byref(desc), _ptr(group_mass), group_size, block,
                                                      nblocks, _ptr(kv_idx), _ptr(ws),
                                                      ws.numel() * ws.element_size(), _stream(stream)))


def residual(q, k, v, o_dense, perm, group_size, kv_idx, topk, r, desc=None, stream=None):
    lib = load()
    _same_layout(q, k, v, o_dense, r)
    desc = desc or desc_for(q)
    _tensors(("q", q), ("k", k), ("v", v), ("o_dense", o_dense), ("r", r))
    _dev(perm, "perm", torch.int32, _per_token(desc), contiguous=True)
    _dev(kv_idx, "kv_idx", torch.int32, _idx_numel(desc, group_size, topk), contiguous=True)
    _check("mcs_residual", lib.mcs_residual(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o_dense), _ptr(perm),
                                            group_size, _ptr(kv_idx), topk, _ptr(r), _stream(stream)))


def sparse_apply(q, k, v, perm, group_size, kv_idx, topk, r, o, desc=None, stream=None):
    lib = load()
    _same_layout(q, k, v, r, o)
    desc = desc or desc_for(q)
    _tensors(("q", q), ("k", k), ("v", v), ("r", r), ("o", o))
    _dev(perm, "perm", torch.int32, _per_token(desc), contiguous=True)
    _dev(kv_idx, "kv_idx", torch.int32, _idx_numel(desc, group_size, topk), contiguous=True)
    _check("mcs_sparse_apply", lib.mcs_sparse_apply(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(perm),
                                                    group_size, _ptr(kv_idx), topk, _ptr(r), _ptr(o), _stream(stream)))


def kv_idx_bitmap_bytes(desc: Desc, group_size: int) -> int:
    lib = load()
    n = ctypes.c_size_t()
    _check("mcs_kv_idx_bitmap_bytes", lib.mcs_kv_idx_bitmap_bytes(ctypes.byref(desc), group_size, ctypes.byref(n)))
    return n.value


def _codec_args(desc, group_size, kv_idx, topk, bitmap):
    _dev(kv_idx, "kv_idx", torch.int32, _idx_numel(desc, group_size, topk), contiguous=True)
    _dev(bitmap, "bitmap", contiguous=True)
    if group_size in (64, 128) and (bitmap.element_size() != 4 or
                                    bitmap.numel() * 4 < kv_idx_bitmap_bytes(desc, group_size)):
        raise ValueError("bitmap must be a 4-byte tensor of at least kv_idx_bitmap_bytes() bytes")


def kv_idx_encode(desc: Desc, group_size, kv_idx, topk, bitmap, stream=None):
    """kv_idx int32 [B][H][G][topk] -> bitmap uint32 [B][H][G][ceil(N/32)] (any 4-byte tensor)."""
    lib = load()
    _codec_args(desc, group_size, kv_idx, topk, bitmap)
    _check("mcs_kv_idx_encode", lib.mcs_kv_idx_encode(ctypes.byref(desc), group_size, _ptr(kv_idx), topk,
                                                      _ptr(bitmap), _stream(stream)))


def kv_idx_decode(desc: Desc, group_size, bitmap, topk, kv_idx, stream=None):
    """bitmap -> kv_idx, ascending (each row must hold exactly topk set bits)."""
    lib = load()
    _codec_args(desc, group_size, kv_idx, topk, bitmap)
    _check("mcs_kv_idx_decode", lib.mcs_kv_idx_decode(ctypes.byref(desc), group_size, _ptr(bitmap), topk,
                                                      _ptr(kv_idx), _stream(stream)))


class RCache:
    """Per-layer host cache of R with a one-layer-ahead prefetch (mcs_rcache_*)."""

    def __init__(self, n_layers: int, bytes_per_layer: int):
        self.lib = load()
        h = ctypes.c_void_p()
        _check("mcs_rcache_create", self.lib.mcs_rcache_create(n_layers, bytes_per_layer, ctypes.byref(h)))
        self.h = h
        self.bytes = bytes_per_layer

    def store(self, layer: int, src: torch.Tensor, stream=None):
        _dev(src, "src")
        if src.numel() * src.element_size() < self.bytes:
            raise ValueError(f"src holds fewer than the cache's {self.bytes} bytes per layer")
        _check("mcs_rcache_store", self.lib.mcs_rcache_store(self.h, layer, _ptr(src), _stream(stream)))

    def prefetch(self, layer: int, stream=None):
        _check("mcs_rcache_prefetch", self.lib.mcs_rcache_prefetch(self.h, layer, _stream(stream)))

    def acquire(self, layer: int, stream=None) -> int:
        p = ctypes.c_void_p()
        _check("mcs_rcache_acquire", self.lib.mcs_rcache_acquire(self.h, layer, _stream(stream), ctypes.byref(p)))
        return p.value

    def host_ptr(self, layer: int) -> int:
        p = ctypes.c_void_p()
        _check("mcs_rcache_host_ptr", self.lib.mcs_rcache_host_ptr(self.h, layer, ctypes.byref(p)))
        return p.value

    def close(self):
        if self.h:
            _check("mcs_rcache_destroy", self.lib.mcs_rcache_destroy(self.h))
            self.h = None
