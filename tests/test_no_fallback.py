"""The product path has no CPU fallback: a copy of the package without
libmoeq.so imports, but its first call into the library raises ImportError
instead of computing anything."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = """
import quantized_expert_gemv_router_amd as q
try:
    q.moeq_abi_version()
except ImportError as e:
    print("IMPORTERROR", e)
else:
    print("CALLED")
"""


def test_missing_library_fails_loudly(tmp_path):
    src = os.path.join(ROOT, "quantized_expert_gemv_router_amd")
    dst = tmp_path / "quantized_expert_gemv_router_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    assert not any(p.suffix == ".so" for p in dst.rglob("*"))
    env = {**os.environ, "PYTHONPATH": str(tmp_path)}
    r = subprocess.run([sys.executable, "-c", PROBE], cwd=tmp_path, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "IMPORTERROR" in r.stdout and "libmoeq.so is missing" in r.stdout, r.stdout
