import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_built():
    """Tests load the in-tree libmdt.so; build it once if nothing is built yet."""
    lib = os.path.join(ROOT, "medusa_tree_verification_heads_amd", "libmdt.so")
    if not os.path.exists(lib):
        from __graft_entry__ import _builder
        _builder().build(verbose=False)


_ensure_built()
