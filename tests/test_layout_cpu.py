"""Source-layout rules checked on the CPU: the product (the package and its
HIP/C++ sources) never imports, links or reads the oracle, and no file the
GPU runs (package, tests, bench, entry point) refers to the pages' copy."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dynamic_top_sparse_amd")


def _files(top, exts):
    for d, _, names in os.walk(top):
        if "__pycache__" in d or os.sep + "lib" in d[len(top):]:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def test_product_never_touches_the_oracle():
    pat = re.compile(r"\boracle\b")
    bad = []
    for p in _files(PKG, (".py", ".hip", ".cpp", ".h")):
        for i, line in enumerate(open(p, encoding="utf-8"), 1):
            code = line.split("#")[0] if p.endswith(".py") else line.split("//")[0]
            if pat.search(code) and ("import" in code or "include" in code or "open(" in code):
                bad.append(f"{os.path.relpath(p, ROOT)}:{i}: {line.strip()}")
    assert not bad, bad


def test_nothing_run_on_the_gpu_reads_the_pages_copy():
    needle = "/root/" + "reference"
    paths = list(_files(PKG, (".py", ".hip", ".cpp", ".h")))
    paths += list(_files(os.path.join(ROOT, "tests"), (".py",)))
    paths += [os.path.join(ROOT, n) for n in ("bench.py", "__graft_entry__.py")]
    bad = [os.path.relpath(p, ROOT) for p in paths if needle in open(p, encoding="utf-8").read()]
    assert not bad, bad
