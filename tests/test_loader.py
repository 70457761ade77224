"""The binding fails loudly when its library is absent: importing the package raises
ImportError naming the missing libmxq.so (there is no fallback path).  CPU only."""

import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mxfp4_microscaled_quantization_amd")


def test_import_without_the_library_raises(tmp_path):
    pkg = tmp_path / "mxfp4_microscaled_quantization_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(PKG, "__init__.py"), pkg / "__init__.py")       # the binding, no libmxq.so
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    r = subprocess.run([sys.executable, "-c", "import mxfp4_microscaled_quantization_amd"], cwd=tmp_path,
                       env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libmxq.so not found" in r.stderr
