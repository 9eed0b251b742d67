import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")
LIB = os.path.join(ROOT, "combine_router_topk_amd", "libmoe_route.so")

# Tests load what is built; they build only when nothing is. A library built
# from other sources than those in the tree is refused, never run.
C_CHECK_LIB = os.path.join(ROOT, "tests", "c_abi", "libcheck_abi.so")


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_moe_build", os.path.join(ROOT, "combine_router_topk_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_BUILD = _build_module()
if not os.path.exists(LIB) or not os.path.exists(C_CHECK_LIB):
    if not os.path.exists(LIB):
        _BUILD.build()
    _BUILD.build_c_check()
import ctypes as _ct  # noqa: E402

# torch first: it loads the HIP runtime it ships, and the library then binds
# to that same runtime (same soname). Loading the library first would pull
# in the system runtime under that name and torch would run on it.
import torch  # noqa: E402,F401

_id_fn = _ct.CDLL(LIB).moe_build_id
_id_fn.restype = _ct.c_char_p
BUILD_ID = _id_fn().decode()
if BUILD_ID != _BUILD.source_digest():
    raise RuntimeError(f"{LIB} is stale: built from sources with id {BUILD_ID}, the tree's sources "
                       f"have id {_BUILD.source_digest()}; run `python combine_router_topk_amd/build.py`")
print(f"libmoe_route.so build id {BUILD_ID}", flush=True)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def load_golden(name):
    import json
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)
