"""GPU check of sdpa_bwd_noalloc, the allocation-free variant of sdpa_bwd_ex for callers that
cannot allocate (its workspace is the library's static device scratch).

Two calls in a row, the second on a smaller problem, each compared with sdpa_bwd_ex on the same
inputs and route: bitwise on the deterministic routes (same kernels, same fixed summation order),
within the parity tolerance against the oracle on the fp32-atomic route.  The second call finds
the first call's contents in the scratch, so it also shows that the chain clears what it
accumulates into.
"""
import ctypes

import numpy as np
import pytest

from attention_backward_sdpa_amd import synth
from tests import _common as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
V = synth.small_variant

BIG = V(W["gqa_causal_s4096_d128"], Hq=8, Hkv=2, Sq=333, Skv=333)
SMALL = V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=1, Sq=150, Skv=150, window_left=60,
          len_lo=40)


def _outputs(t):
    outs = [torch.empty_like(t[x]) for x in ("q", "k", "v")]
    for x in outs:
        x.view(torch.int16).fill_(0x7FC0)  # NaN poison: every element must be written
    return outs


def _run_noalloc(case, t, det):
    import attention_backward_sdpa_amd as lib
    w = case["w"]
    outs = _outputs(t)
    lib.sdpa_bwd_noalloc(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], *outs,
                         scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
                         deterministic=det, seq_q_lens=t["lens"], seq_kv_lens=t["lens"])
    torch.cuda.synchronize()
    return tuple(C.bf16_tensor_to_f32(x) for x in outs)


@pytest.mark.parametrize("det", [3, 2, 0], ids=["dqpartials", "dspanels", "atomic"])
def test_noalloc_matches_workspace_entry_point(det):
    for w in (BIG, SMALL):  # the second call is the smaller problem
        case = C.make_case(w)
        t = C.to_device(case, torch)
        C.log(f"noalloc {w.name} B={w.B} Hq={w.Hq} S={w.Sq} route {det}")
        got = _run_noalloc(case, t, det)
        ref_ws = C.run_gpu(case, torch, deterministic=det, dev_inputs=t)
        if det != 0:
            for name, a, b in zip(("dQ", "dK", "dV"), got, ref_ws):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
                    f"{w.name} {name}: sdpa_bwd_noalloc differs from sdpa_bwd_ex"
        else:
            # dK / dV are deterministic on every route; dQ's atomics may round differently
            for a, b in zip(got[1:], ref_ws[1:]):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
            ref = C.oracle_backward(case)
            for name, a, r in zip(("dQ", "dK", "dV"), got, ref):
                C.assert_close(f"noalloc {w.name} {name}", a, r)
                C.assert_close(f"noalloc vs ex {w.name} {name}", a,
                               ref_ws[("dQ", "dK", "dV").index(name)].astype(np.float64))


def test_noalloc_declines_problems_beyond_the_scratch():
    import attention_backward_sdpa_amd as lib
    so = lib.library()
    p = ctypes.c_void_p(4096)  # never dereferenced: the call is declined before any GPU work
    # fp32 dQ accumulator of 64 heads x 16384 rows x 128 floats = 512 MiB > 256 MiB
    st = so.sdpa_bwd_noalloc(*([p] * 9), 1, 64, 64, 16384, 16384, 128, 128, -1.0, 1, -1, 0,
                             None, None, 0, 0, None)
    assert st == lib.SCRATCH_TOO_SMALL
    assert lib.workspace_size(1, 64, 64, 16384, 16384, 128, 128) > lib.NOALLOC_SCRATCH_BYTES
