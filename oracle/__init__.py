"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package. The library and its binding
never do.

The package's functions are those of the C++ oracle (``mcsparse_oracle.cpp``
through ``oracle.cpp``), float64 throughout, with std::thread workers over
independent units. ``oracle.mcsparse_ref`` is an independent numpy
transcription of the same steps; the pins run on both, and the two are
cross-checked against each other.
"""
from . import cpp as _cpp

__all__ = [
    "round_bf16",
    "topk_count",
    "pddp_group",
    "principal_direction",
    "standardize",
    "dense_lse",
    "group_mass",
    "topk_select",
    "sparse_attention",
    "residual",
    "reuse_output",
    "block_select",
    "group_recall",
    "rel_l1",
    "reuse_head",
    "anchor_head",
]


def _bind(name):
    def call(*args, **kwargs):
        return getattr(_cpp.default(), name)(*args, **kwargs)

    call.__name__ = name
    call.__doc__ = getattr(_cpp.CppOracle, name).__doc__
    return call


for _name in __all__:
    globals()[_name] = _bind(_name)
del _name
