"""dq2k's two key-split variants under each mask form, against the fp64 oracle.

At head dim 128 the dS-panel route's dq2k comes in two forms: 4 q tiles per workgroup (two
workgroups per CU) and 8 q tiles per workgroup (16 waves, one per CU).  The 4-q-tile form runs
when a mask makes the key ranges of a group's q tiles differ (causal, window, per-batch lengths)
and a grid of 8-q-tile groups would hold fewer than two workgroups per CU (512 on the 256 CUs);
the 8-q-tile form runs otherwise.  Every mask form below runs on a small grid and on a large one
(B*Hq*ceil(n_q_tiles/8) below and above 512), so each form meets each mask, with a ragged tail
(S = 260: eight full q tiles and a 4-row one, alone in its group).  dQ, dK and dV are compared
with the oracle element by element.
"""
import pytest

from attention_backward_sdpa_amd import synth
from tests import _common as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N_CUS = 256
MASKS = {
    "none": dict(causal=False),
    "causal": dict(causal=True),
    "causal_window": dict(causal=True, window_left=70),
    "lengths": dict(causal=False, padded=True, len_lo=90),
    "lengths_causal_window": dict(causal=True, window_left=45, padded=True, len_lo=90),
}
GRIDS = {"small": dict(B=2, Hq=4, Hkv=2), "large": dict(B=2, Hq=256, Hkv=64)}


def _workload(mask, grid):
    base = synth.WORKLOADS["gqa_causal_s4096_d128"]
    fields = dict(name=f"dq2k_{mask}_{grid}", Sq=260, Skv=260, window_left=-1, padded=False,
                  len_lo=0, seed=11, **GRIDS[grid])
    fields.update(MASKS[mask])
    return synth.small_variant(base, **fields)


@pytest.mark.parametrize("grid", list(GRIDS))
@pytest.mark.parametrize("mask", list(MASKS))
def test_dq2k_variant_parity(mask, grid):
    w = _workload(mask, grid)
    groups = w.B * w.Hq * (((w.Sq + 31) // 32 + 7) // 8)
    uneven = w.causal or w.window_left >= 0 or w.padded
    form = "4 q tiles" if uneven and groups < 2 * N_CUS else "8 q tiles"
    C.log(f"dq2k {form} per workgroup, mask {mask}, {groups} groups of 8: {w}")
    case = C.make_case(w)
    got = C.run_gpu(case, torch, deterministic=2)
    ref = C.oracle_backward(case)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        C.assert_close(f"{w.name} {name}", g, r)
