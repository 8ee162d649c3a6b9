"""The backward chain captured in a HIP graph (torch.cuda.CUDAGraph) and replayed; and two
independent calls enqueued on two streams at once.

Every step of the chain is a kernel launched on the caller's stream (the library issues no memset,
copy or allocation), so one captured call replays the whole chain: the preprocess clears what the
main kernel accumulates into on every replay.  Both the workspace entry point (its workspace
allocated before the capture) and the allocation-free one are captured.  Three replays, with the
outputs poisoned eagerly and the device synchronised between them, are each compared with the
eager call on the same inputs: bitwise on the deterministic routes (and for dK/dV on every route),
and dQ of the fp32-atomic route within the parity tolerance of the oracle.
"""
import numpy as np
import pytest

from attention_backward_sdpa_amd import synth
from tests import _common as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASE = synth.small_variant(W["gqa_causal_s4096_d128"], Hq=8, Hkv=2, Sq=333, Skv=333)


@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_graph_replays_match_eager(entry, det):
    import attention_backward_sdpa_amd as lib
    w = CASE
    case = C.make_case(w)
    t = C.to_device(case, torch)
    C.log(f"graph capture: {entry} entry point, route {det}, {w}")
    outs = [torch.empty_like(t[x]) for x in ("q", "k", "v")]
    ws = None
    if entry == "workspace":
        n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, w.causal,
                               w.window_left, det, False)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    kw = dict(scale=w.softmax_scale, causal=w.causal, window_left=w.window_left, deterministic=det)

    def call():
        if entry == "workspace":
            lib.sdpa_bwd_ex(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], *outs, workspace=ws, **kw)
        else:
            lib.sdpa_bwd_noalloc(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], *outs, **kw)

    def poison():
        for x in outs:
            x.view(torch.int16).fill_(0x7FC0)

    # the eager reference (it also raises the kernels' LDS limits before the capture)
    poison()
    call()
    torch.cuda.synchronize()
    ref = [C.bf16_tensor_to_f32(x) for x in outs]

    # a warm-up call on a side stream, then the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    oracle_ref = C.oracle_backward(case) if det == 0 else None
    for rep in range(3):
        poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [C.bf16_tensor_to_f32(x) for x in outs]
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            if det != 0 or name != "dQ":
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
                    f"replay {rep}: {name} differs from the eager call"
        if det == 0:
            C.assert_close(f"graph replay {rep} ({entry}, atomic) dQ", got[0], oracle_ref[0])


@pytest.mark.parametrize("det", [0, 2, 4], ids=["atomic", "dspanels", "relay"])
def test_two_streams_at_once(det):
    # two independent calls, each with its own workspace, enqueued on two streams at once: both
    # equal their sequential results (bitwise on the deterministic routes; dK/dV on every route)
    import attention_backward_sdpa_amd as lib
    cases = [C.make_case(CASE), C.make_case(synth.small_variant(
        W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=1, Sq=260, Skv=260, window_left=70, len_lo=90))]
    ts = [C.to_device(c, torch) for c in cases]
    seq = [C.run_gpu(c, torch, deterministic=det, dev_inputs=t) for c, t in zip(cases, ts)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, wss = [], []
    for c, t in zip(cases, ts):
        w = c["w"]
        o = [torch.empty_like(t[x]) for x in ("q", "k", "v")]
        for x in o:
            x.view(torch.int16).fill_(0x7FC0)
        n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, w.causal,
                               w.window_left, det, t["lens"] is not None)
        outs.append(o)
        wss.append(torch.empty(max(n, 256), dtype=torch.uint8, device="cuda"))
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())  # inputs, poison and workspaces are ready
    for c, t, o, ws, s in zip(cases, ts, outs, wss, streams):
        w = c["w"]
        lib.sdpa_bwd_ex(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], *o,
                        scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
                        deterministic=det, seq_q_lens=t["lens"], seq_kv_lens=t["lens"],
                        workspace=ws, stream=s)
    torch.cuda.synchronize()
    for c, o, ref in zip(cases, outs, seq):
        got = [C.bf16_tensor_to_f32(x) for x in o]
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            if det != 0 or name != "dQ":
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
                    f"{c['w'].name} {name}: concurrent call differs from the sequential one"
            else:
                C.assert_close(f"{c['w'].name} concurrent dQ", a, C.oracle_backward(c)[0])
