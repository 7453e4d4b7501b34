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


def _tr16_rule(offsets, values):
    """The regrouping the kernels assume for ds_read_b64_tr_b16: in each
    block of 16 lanes, lane i receives element e from lane 4e + i//4 of the
    block, element i % 4 (each lane reads 4 halves at its own offset)."""
    out = np.empty((64, 4), np.int16)
    for l in range(64):
        b, i = divmod(l, 16)
        for e in range(4):
            out[l, e] = values[offsets[16 * b + 4 * e + i // 4] + i % 4]
    return out


@pytest.mark.parametrize("pattern", ["contiguous", "rows", "random", "kernel"])
def test_lds_transposing_read(pattern):
    rng = np.random.default_rng(7)
    values = rng.permutation(4096).astype(np.int16)      # distinct: each output names its source
    if pattern == "contiguous":
        offs = [4 * l for l in range(64)]
    elif pattern == "rows":
        offs = [32 * l for l in range(64)]
    elif pattern == "random":
        offs = [int(v) * 4 for v in rng.choice(1024, 64, replace=False)]
    else:
        # the kernel's own first read of A fragment (wave 0, repeat 0, K
        # sub-step 0) in the 256-wide M-contiguous tile
        lay = mfl.lds_tile_offsets("lds256", "A_mmajor")          # [k, m]
        src = mfl.fragment_coords("lds256", "A_tr")[:64, 0]         # (m, k) per lane
        offs = [int(lay[k, m]) for m, k in src]
    say(f"[gpu] probe tr16 {pattern}")
    got = mfl.probe_lds_tr16(offs, torch.from_numpy(values).cuda()).cpu().numpy()
    assert np.array_equal(got, _tr16_rule(offs, values))
    if pattern == "kernel":
        # and the values are the MFMA operand: lane l gets (m, k) = (l%32, 8(l/32) + e)
        lay = mfl.lds_tile_offsets("lds256", "A_mmajor")
        for l in range(64):
            for e in range(4):
                m, k = l % 32, 8 * (l // 32) + e
                assert got[l, e] == values[lay[k, m]], (l, e)


def test_workgroups_dealt_round_robin_over_xcds():
    """The kernels' tile order (tile_of_block) assumes that workgroup b runs
    on XCD b % 8: the 8 dies are dealt workgroups in turn, so renumbering
    gives each die a contiguous run of tiles whose operand rows share its
    L2.  A launch of 4096 small workgroups records where each one ran."""
    n = 4096
    x = mfl.probe_xcc(n).cpu().numpy()
    counts = np.bincount(x[x >= 0], minlength=8)
    match = float(np.mean(x == np.arange(n) % 8))
    say(f"[gpu] XCD of workgroup b: first 16 {x[:16].tolist()}, per die {counts.tolist()}, "
        f"b % 8 matches {100 * match:.1f} %")
    assert ((x >= 0) & (x < 8)).all()
    assert np.array_equal(x, np.arange(n) % 8)
