"""The library and the oracle share nothing, and the library has no fallback (CPU).

* Importing the package loads only its own modules: neither ``oracle`` nor ``synth``
  (the seeded input generators) comes along.
* No library source (Python binding, HIP kernels, C ABI host code, headers) names the
  oracle, and no oracle code imports or names the library's entry points.
* With the shared library missing, importing the package raises instead of falling back.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_decode_amd")
SRC_EXT = (".py", ".hip", ".cpp", ".h", ".map")


def _sources(top, exts):
    for d, dirs, files in os.walk(top):
        dirs[:] = [x for x in dirs if not x.startswith(("_build", "__pycache__"))]
        for f in files:
            if f.endswith(exts):
                yield os.path.join(d, f)


def _run(code, env=None, cwd=ROOT):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, "-c", code], cwd=cwd, env=e, capture_output=True, text=True,
                          timeout=120)


def test_package_import_pulls_in_neither_oracle_nor_synth():
    r = _run("import sys, long_context_decode_amd; "
             "print(sorted(m for m in sys.modules if m.split('.')[0] in ('oracle', 'synth')))")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "[]"


def test_library_sources_never_name_the_oracle():
    files = list(_sources(PKG, SRC_EXT)) + list(_sources(os.path.join(ROOT, "include"), (".h",)))
    assert files
    for f in files:
        text = open(f, encoding="utf-8").read()
        assert not re.search(r"\boracle\b", text), f


def test_oracle_never_uses_the_library():
    files = list(_sources(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")))
    assert files
    for f in files:
        text = open(f, encoding="utf-8").read()
        assert not re.search(r"^\s*(import|from)\s+long_context_decode_amd", text, flags=re.M), f
        assert not re.search(r"\blcd_[a-z0-9_]+\s*\(", text), f
        assert "liblcd" not in text, f


def test_missing_library_fails_loudly(tmp_path):
    """A copy of the package's Python files without liblcd.so next to them: the import
    raises and names the missing library (the binding loads only the in-tree build)."""
    import shutil

    dst = tmp_path / "long_context_decode_amd"
    dst.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), dst / f)
    r = _run("import long_context_decode_amd", cwd=str(tmp_path), env={"PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "liblcd.so is missing" in r.stderr
