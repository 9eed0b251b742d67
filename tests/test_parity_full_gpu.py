"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: every index output compared whole with the oracle, rows and
combine outputs on seeded samples the oracle computes one by one, plus the
dispatch identity send[r] == x[src[r] / k] checked on every row on the GPU."""
import numpy as np
import pytest
import torch

import oracle
import synth
from pathcheck import check_meta, check_rows, run_gpu, say

pytestmark = pytest.mark.gpu


def sample(rng, n, m):
    s = rng.choice(n, size=min(m, n), replace=False)
    return np.unique(np.concatenate([s, [0, n - 1]])).astype(np.int64)


def dispatch_identity_all_rows(b, k):
    rows = b.send.shape[0]
    step = 1 << 16
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        tok = (b.src[r0:r1].long() // k)
        assert torch.equal(b.send[r0:r1].view(torch.int16), b.x.index_select(0, tok).view(torch.int16)), r0


@pytest.mark.parametrize("w", [synth.DECODE, synth.TRAIN_TOP2, synth.TRAIN_TOP6, synth.LARGE],
                         ids=lambda w: w.name)
def test_full_size(w):
    seed = 0
    say(f"[case] full {w.name}")
    logits = synth.make_logits(w, seed)
    x = synth.make_x(w, seed)
    rep = synth.replica_table(w)
    ref = oracle.route_and_layout(w.T, w.E, w.k, w.R, logits, rep)
    b = run_gpu(w, logits, x, rep)
    check_meta(b, ref, w.T, w.k)
    rng = np.random.default_rng(1234)
    check_rows(b, ref, x, w, sample(rng, w.T * w.k, 512), sample(rng, w.T, 256), out_f32=False)
    dispatch_identity_all_rows(b, w.k)
    assert int(b.counts.sum()) == w.T * w.k
