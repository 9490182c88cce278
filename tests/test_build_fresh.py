"""build() must work on a checkout that holds no built library.

The package's __init__ loads libzero_mi355x.so and raises when it is missing,
so build() has to reach the build scripts without importing the package first.
This copies the sources (no built files) to a temporary directory and runs
build() there in a fresh interpreter."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ignored_dirs():
    """The directories .gitignore lists (caches, build outputs, working
    folders), plus the repository metadata and the parts build() does not read."""
    out = {".git", "profiles", "tests"}
    with open(os.path.join(ROOT, ".gitignore")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#") and line.endswith("/"):
                out.add(line.strip("/"))
    return out


def _ignore(_dir, names, _dirs=_ignored_dirs()):
    return [n for n in names if n.endswith((".so", ".tmp", ".pyc")) or n in _dirs]


def test_build_from_a_tree_without_libraries(tmp_path):
    dst = tmp_path / "repo"
    shutil.copytree(ROOT, dst, ignore=_ignore)
    assert not any(p.suffix == ".so" for p in dst.rglob("*"))
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"], cwd=dst,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert (dst / "zero_partitioned_mixed_flatten_amd" / "libzero_mi355x.so").exists()
    assert (dst / "oracle" / "liboracle_zero.so").exists()
