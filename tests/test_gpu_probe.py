"""Pin the gfx950 matrix-instruction operand maps against the hardware.

The pages give SM80 thread/value tables only; for the CDNA4 instructions the
oracle states closed forms (oracle/layout.py).  Here one wave executes one
instruction with slots filled from random small-integer matrices through
those maps; every output slot must equal C + A B^T at the (m, n) the oracle
map assigns to it, bit for bit.  A wrong row/column map, or a K pairing that
is not shared by A and B, fails."""
import itertools

import numpy as np
import pytest
import torch

import mma_fragment_layouts_tn_amd as mfl
from oracle import layout as L
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("op", sorted(L.MFMA_OPS))
def test_mfma_operand_maps(op):
    M, N, K, nv, nacc = L.MFMA_OPS[op]
    rng = np.random.default_rng(sorted(L.MFMA_OPS).index(op) + 40)
    A = rng.integers(-2, 3, (M, K)).astype(np.float16)
    B = rng.integers(-2, 3, (N, K)).astype(np.float16)
    C = rng.integers(-8, 9, (M, N)).astype(np.float32)
    a = np.zeros((64, nv), np.float16)
    b = np.zeros((64, nv), np.float16)
    c = np.zeros((64, nacc), np.float32)
    for l, v in itertools.product(range(64), range(nv)):
        r, k = L.mfma_ab_coord(op, l, v)
        a[l, v] = A[r, k]
        b[l, v] = B[r, k]
    for l, v in itertools.product(range(64), range(nacc)):
        m, n = L.mfma_c_coord(op, l, v)
        c[l, v] = C[m, n]
    say(f"[gpu] probe {op}")
    d = mfl.probe_mfma(op, torch.from_numpy(a.view(np.int16).copy()).cuda(),
                       torch.from_numpy(b.view(np.int16).copy()).cuda(),
                       torch.from_numpy(c).cuda())
    torch.cuda.synchronize()
    d = d.cpu().numpy()
    want = C.astype(np.float64) + A.astype(np.float64) @ B.astype(np.float64).T
    bad = []
    for l, v in itertools.product(range(64), range(nacc)):
        m, n = L.mfma_c_coord(op, l, v)
        if d[l, v] != want[m, n]:
            bad.append((l, v, m, n, float(d[l, v]), want[m, n]))
    assert not bad, bad[:8]
