"""Seeded synthetic workloads shared by the HIP path's tests/bench and the
CPU oracle. No routing arithmetic lives here."""
from .configs import (BF16, BY_NAME, DECODE, F16, LARGE, TINY, TRAIN_TOP2,  # noqa: F401
                      TRAIN_TOP6, WORKLOADS, Workload, replica_table, scaled)
from .gen import digest, make_grad, make_logits, make_x  # noqa: F401
