"""The oracle and the product path stay apart: the package and its HIP
sources never import or include anything of the oracle, the oracle never
imports the package or includes its sources, importing the package loads no
oracle module, and bench.py touches the oracle only inside its CPU-baseline
functions. bench.py also refuses to run on more than one GPU."""
import ast
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "paged_kv_cache_209_amd")
ORACLE = os.path.join(ROOT, "oracle")


def files(top, exts):
    for d, _, names in os.walk(top):
        if "__pycache__" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def python_imports(path):
    tree = ast.parse(open(path).read(), path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom) and node.module:
            yield node.module


def test_package_never_imports_the_oracle():
    for path in files(PKG, (".py",)):
        for mod in python_imports(path):
            assert mod.split(".")[0] != "oracle", f"{path} imports {mod}"
    for path in files(PKG, (".hip", ".cpp", ".h")):
        text = open(path).read()
        assert not re.search(r'#include\s*["<][^">]*oracle', text), f"{path} includes oracle code"


def test_oracle_never_imports_the_package():
    for path in files(ORACLE, (".py",)):
        for mod in python_imports(path):
            assert not mod.startswith("paged_kv_cache_209_amd"), f"{path} imports {mod}"
    for path in files(ORACLE, (".c", ".h", ".cpp")):
        text = open(path).read()
        assert "paged_kv_cache_209_amd" not in text and "paged_attn.h" not in text, path


def test_importing_the_package_loads_no_oracle_module():
    code = ("import sys; sys.path.insert(0, %r); import paged_kv_cache_209_amd; "
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd="/")
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "[]", out.stdout


def test_bench_uses_the_oracle_only_in_its_cpu_baseline():
    path = os.path.join(ROOT, "bench.py")
    tree = ast.parse(open(path).read(), path)
    allowed = {"cpu_baseline", "cpu_baseline_prefill", "block_manager_oracle_step_us"}
    for node in tree.body:
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
            assert all(m.split(".")[0] != "oracle" for m in mods), "bench.py imports the oracle at top level"
        if isinstance(node, ast.FunctionDef) and node.name not in allowed:
            for sub in ast.walk(node):
                if isinstance(sub, (ast.Import, ast.ImportFrom)):
                    mods = [a.name for a in sub.names] if isinstance(sub, ast.Import) else [sub.module or ""]
                    assert all(m.split(".")[0] != "oracle" for m in mods), f"{node.name} imports the oracle"


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says
    so, before touching a device."""
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert out.returncode == 2
    assert "one GPU only" in out.stderr
