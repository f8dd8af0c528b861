"""The oracle and the product share no code, and the product has no CPU path.

* No product source (Python binding, C ABI, HIP kernels, header) refers to the
  oracle, and no oracle module imports the product.
* Importing the product pulls in no oracle module; importing bench.py pulls in
  none either (its CPU-baseline leg imports the oracle only when it runs).
* Without the compiled library, importing the product raises: nothing can fall
  back to running elsewhere.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "orthogonalized_optimizer_step_amd")


def sources(top, exts):
    for d, _, files in os.walk(top):
        if "__pycache__" in d:
            continue
        for f in files:
            if f.endswith(exts):
                yield os.path.join(d, f)


def test_product_sources_do_not_refer_to_the_oracle():
    pat = re.compile(r"import\s+oracle|from\s+oracle|oracle/|dion_oracle|orthdion_oracle")
    files = list(sources(PKG, (".py", ".cpp", ".hip", ".h"))) + list(sources(os.path.join(ROOT, "include"), (".h",)))
    assert files
    for f in files:
        text = open(f, encoding="utf-8").read()
        assert not pat.search(text), f


def test_oracle_does_not_import_the_product():
    pat = re.compile(r"orthogonalized_optimizer_step_amd|libdion|csrc")
    files = list(sources(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")))
    assert files
    for f in files:
        code = [l for l in open(f, encoding="utf-8") if not l.lstrip().startswith("#")]
        assert not pat.search("".join(code)), f


def run(code, env=None):
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_importing_the_product_and_bench_loads_no_oracle_module():
    code = ("import sys; import orthogonalized_optimizer_step_amd, bench; "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "assert not bad, bad; print('ok')")
    r = run(code)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]


def test_missing_library_raises_on_import(tmp_path):
    # a copy of the Python package without libdion.so
    dst = tmp_path / "orthogonalized_optimizer_step_amd"
    dst.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            (dst / f).write_text(open(os.path.join(PKG, f), encoding="utf-8").read())
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import orthogonalized_optimizer_step_amd\nexcept ImportError as e:\n    print('raised', e)\n"
            "else:\n    print('imported')") % str(tmp_path)
    r = run(code)
    assert "raised" in r.stdout, r.stdout + r.stderr[-2000:]
