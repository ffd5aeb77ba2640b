"""The oracle and the HIP path share no code: the oracle imports nothing from
the package, and nothing in the package imports the oracle. Outside tests/,
only __graft_entry__.smoke() and bench.py's cpu_baseline leg may use it."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_diffusion_pddp_amd")


def _imports(path):
    """(module name, enclosing top-level function or None) for every import."""
    tree = ast.parse(open(path).read(), path)
    out = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) and fn is None else fn
            if isinstance(child, ast.Import):
                out.extend((a.name, fn) for a in child.names)
            elif isinstance(child, ast.ImportFrom):
                out.append(("." * child.level + (child.module or ""), fn))
            visit(child, f)

    visit(tree, None)
    return out


def _py_files(d):
    for base, _, files in os.walk(d):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(base, f)


def test_oracle_imports_nothing_from_the_package():
    for path in _py_files(os.path.join(ROOT, "oracle")):
        for mod, _ in _imports(path):
            assert "sparse_attention_diffusion_pddp_amd" not in mod and mod not in ("binding", "synth"), (path, mod)


def test_cpp_oracle_includes_nothing_from_the_library():
    """The C++ oracle includes only the standard library: no header of the
    HIP library, no HIP, nothing from the package."""
    import re
    src = open(os.path.join(ROOT, "oracle", "mcsparse_oracle.cpp")).read()
    for inc in re.findall(r'#\s*include\s*[<"]([^>"]+)[>"]', src):
        assert "/" not in inc and "." not in inc, inc  # standard headers only (<vector>, <cmath>, ...)
    assert "hip" not in src.lower()


def test_package_does_not_load_the_oracle_library():
    for base, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                assert "libmcsoracle" not in open(os.path.join(base, f)).read(), f


def test_package_does_not_import_the_oracle():
    for path in _py_files(PKG):
        for mod, _ in _imports(path):
            assert not mod.split(".")[0] == "oracle", (path, mod)


def test_oracle_use_outside_tests_is_confined():
    """bench.py's cpu_baseline and the entry module's smoke() may use the
    oracle; the entry module's build() may only compile it (oracle.build)."""
    for name, allowed in (("bench.py", {"cpu_baseline"}), ("__graft_entry__.py", {"smoke"})):
        for mod, fn in _imports(os.path.join(ROOT, name)):
            if mod.split(".")[0] == "oracle":
                assert fn in allowed or (name == "__graft_entry__.py" and fn == "build" and mod == "oracle"), (name, fn)
    src = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    build_src = src[src.index("def build("):src.index("def smoke(")]
    lines = [ln.strip() for ln in build_src.splitlines() if "oracle" in ln and not ln.strip().startswith(("#", "\"", "("))]
    assert lines == ["from oracle import build as _oracle_build", "_oracle_build.build()"], lines
