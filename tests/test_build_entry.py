"""The build entry point the round-end check calls: compiles every HIP source for gfx950,
links libmxq.so in place and checks that the loaded library's ABI version is the binding's
(no GPU needed: hipcc cross-compiles)."""

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def test_graft_entry_build_compiles_and_loads():
    import __graft_entry__
    import mxfp4_microscaled_quantization_amd as mxq
    __graft_entry__.build()
    assert os.path.exists(mxq.LIB_PATH)
    assert mxq.lib.mxq_abi_version() == mxq.ABI_VERSION
