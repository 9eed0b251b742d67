"""The library driven from plain C (tests/c_abi/check_abi.c): device memory
from the HIP runtime's C API, every entry point through include/moe_route.h,
and host-side invariants.

- The forward path: top-k order, weights summing to 1, the demand vector,
  the permutation and its inverse, send rows as bit copies, the (expert,
  token) row order, the refused NULL argument, the one-call plan equal to
  the three calls.
- The rest: the one-call single-send plan and the allocation-free plan equal
  to the separate calls; one single-send row per (token, rank) in token
  order; the single-send dispatch and fan-out equal to the plain dispatch;
  dy, dw and dx within their rounding bounds; the send-counts matrix and
  co-selection histogram exact and the four summaries from the same
  integers; the token-balanced split without a replica table."""
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


def test_plain_c_caller_every_other_entry_point():
    say("[case] plain C caller: single-send, backward, statistics, split, one-call and no-alloc plans")
    lib = ctypes.CDLL(C_CHECK_LIB)
    lib.moe_c_abi_check_rest.restype = ctypes.c_int
    assert lib.moe_c_abi_check_rest() == 0
