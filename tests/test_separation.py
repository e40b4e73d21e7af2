"""The oracle and the HIP path share no code and the product path never uses
the oracle: no import, include or link in either direction, and importing
the binding loads nothing from oracle/."""
import ast
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "progressive_kv_transfer_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _files(top, exts):
    for d, _, fs in os.walk(top):
        if "__pycache__" in d:
            continue
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(d, f)


def _imports(path):
    tree = ast.parse(open(path, encoding="utf-8").read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield ("." * node.level) + (node.module or "")


def test_product_python_never_imports_the_oracle():
    for path in _files(PKG, (".py",)):
        for mod in _imports(path):
            assert not mod.split(".")[0] == "oracle", (path, mod)


def test_oracle_python_imports_no_product_code():
    for path in _files(ORACLE, (".py",)):
        for mod in _imports(path):
            top = mod.lstrip(".").split(".")[0]
            assert top not in ("progressive_kv_transfer_amd", "bench"), (path, mod)


def test_no_include_crosses_the_boundary():
    inc = re.compile(r'^\s*#\s*include\s*[<"]([^>"]+)[>"]', re.M)
    for path in _files(PKG, (".hip", ".cpp", ".h", ".c")):
        for h in inc.findall(open(path, encoding="utf-8").read()):
            assert "oracle" not in h, (path, h)
    for path in _files(ORACLE, (".c", ".h")):
        for h in inc.findall(open(path, encoding="utf-8").read()):
            # the C library only: no header of the product (lynx.h, csrc/)
            assert "lynx" not in h and "hip" not in h, (path, h)


def test_library_does_not_link_the_oracle():
    lib = os.path.join(PKG, "liblynx.so")
    if not os.path.exists(lib) or not shutil.which("readelf"):
        pytest.skip("liblynx.so not built or readelf missing")
    out = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True).stdout
    needed = re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out)
    assert needed and not any("oracle" in n for n in needed), needed


def test_importing_the_binding_loads_no_oracle():
    code = ("import sys; import progressive_kv_transfer_amd.lynx, "
            "progressive_kv_transfer_amd.kvgen; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip() == "False"
