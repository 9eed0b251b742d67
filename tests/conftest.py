import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")
LIB = os.path.join(ROOT, "combine_router_topk_amd", "libmoe_route.so")

# Tests load what is built; they build only when nothing is.
C_CHECK_LIB = os.path.join(ROOT, "tests", "c_abi", "libcheck_abi.so")
if not os.path.exists(LIB) or not os.path.exists(C_CHECK_LIB):
    import importlib.util
    _spec = importlib.util.spec_from_file_location(
        "_moe_build", os.path.join(ROOT, "combine_router_topk_amd", "build.py"))
    _mod = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(_mod)
    if not os.path.exists(LIB):
        _mod.build()
    _mod.build_c_check()


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def load_golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)
