"""The library driven from plain C (tests/c_abi/check_abi.c): device memory
from the HIP runtime's C API, the forward path through include/moe_route.h,
and host-side invariants (top-k order, weights summing to 1, the demand
vector, the permutation and its inverse, send rows as bit copies, the
(expert, token) row order, the refused NULL argument)."""
import ctypes

import pytest

from conftest import C_CHECK_LIB
from pathcheck import say

pytestmark = pytest.mark.gpu


def test_plain_c_caller():
    say("[case] plain C caller of the C ABI")
    lib = ctypes.CDLL(C_CHECK_LIB)
    lib.moe_c_abi_check.restype = ctypes.c_int
    assert lib.moe_c_abi_check() == 0
