import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Tests load what is built; they build only when nothing is.
if not os.path.exists(os.path.join(ROOT, "memory_hierarchy_optimisation_amd", "libmhgemm.so")) or \
        not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
    import __graft_entry__
    __graft_entry__.build()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
