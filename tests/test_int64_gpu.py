"""64-bit addressing on the GPU ("cudnn-frontend python/cudnn/sdpa AGENTS.md", the Int64 rule: a
physical stride above 2**32 and offsets past 2**31 elements must be exercised, not assumed).

  * A batch stride above 2**31 elements on Q, dQ and dO (a strided "dense_flex" view over one
    large allocation, through sdpa_bwd_flex): the second batch entry's rows sit more than 4 GiB
    past the base pointer.  Full outputs against the oracle, on three dQ routes.
  * A deterministic call whose dS workspace holds more than 2**31 elements (B*Hq*S*S bf16 with
    Hq = 36, S = 8192, head dim 128: 4.5 GiB): the explicit dS-panel route, whose main kernel and
    dq2k address the panels of the last heads past 2**31 elements, and the library's deterministic
    choice, which takes the relay there because the panels exceed the 4 GiB bound.  Sampled dQ rows
    and dK/dV key rows against the oracle, which recomputes them from exactly the tensors the GPU
    received; O and LSE come from a float32 forward on the GPU (input preparation: the fp64 oracle
    forward over 36 heads at S = 8192 would take minutes, and this case is about addressing).
"""
import numpy as np
import pytest

import oracle
from attention_backward_sdpa_amd import synth
from tests import _common as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
BIG = (1 << 31) + (1 << 20)  # elements between batch entries: more than 2**31, a multiple of 8


def _bf(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def _strided(shape, stride_b):
    """A (B, H, S, D) bf16 view whose batch entries are stride_b elements apart."""
    B, H, S, D = shape
    flat = torch.empty((B - 1) * stride_b + H * S * D, dtype=torch.bfloat16, device="cuda")
    return flat.as_strided(shape, (stride_b, S * D, D, 1))


@pytest.mark.parametrize("det", [0, 2, 3], ids=["atomic", "dspanels", "dqpartials"])
def test_batch_stride_above_2_pow_31(det):
    import attention_backward_sdpa_amd as lib
    w = synth.small_variant(W["gqa_causal_s4096_d128"], B=2, Hq=4, Hkv=2, Sq=300, Skv=300)
    case = C.make_case(w)
    C.log(f"int64 batch stride {BIG} elements, route {det}")
    q = _strided((w.B, w.Hq, w.Sq, w.Dqk), BIG)
    do = _strided((w.B, w.Hq, w.Sq, w.Dv), BIG)
    dq = _strided((w.B, w.Hq, w.Sq, w.Dqk), BIG)
    q.copy_(_bf(case["q"]))
    do.copy_(_bf(case["do"]))
    dq.view(torch.int16).fill_(0x7FC0)
    k, v, o = _bf(case["k"]), _bf(case["v"]), _bf(case["o"])
    lse = torch.from_numpy(case["lse"]).cuda()
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, w.causal, -1, det)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_ex(q, k, v, o, do, lse, dq, dk, dv, scale=w.softmax_scale, causal=w.causal,
                    deterministic=det, workspace=ws)
    torch.cuda.synchronize()
    assert dq.stride(0) > (1 << 31)
    ref = C.oracle_backward(case)
    got = [C.bf16_tensor_to_f32(x.contiguous()) for x in (dq, dk, dv)]
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        C.assert_close(f"int64 batch stride route {det} {name}", g, r)
    del q, do, dq
    torch.cuda.empty_cache()


_BIGWS = {}


def _bigws_case():
    # MHA, causal, head dim 128: 36 heads x 8192 x 8192 bf16 dS panels = 4.5 GiB (2.4e9 elements)
    if not _BIGWS:
        import bench
        w = synth.small_variant(W["gqa_causal_s4096_d128"], B=1, Hq=36, Hkv=36, Sq=8192,
                                Skv=8192, seed=21)
        C.log("int64 workspace case: drawing inputs and a float32 GPU forward (36 heads, S=8192)")
        inp = synth.draw_inputs(w)
        t = dict(q=_bf(inp.q), k=_bf(inp.k), v=_bf(inp.v))
        o, lse = bench.gpu_forward_inputs(torch, t["q"], t["k"], t["v"], w, None)
        torch.cuda.synchronize()
        _BIGWS.update(w=w, inp=inp, o=o.cpu().view(torch.int16).numpy().view(np.uint16),
                      lse=lse.cpu().numpy())
    return _BIGWS


@pytest.mark.parametrize("det", [2, 1], ids=["dspanels", "deterministic-choice"])
def test_deterministic_workspace_above_2_pow_31(det):
    import attention_backward_sdpa_amd as lib
    c = _bigws_case()
    w, inp = c["w"], c["inp"]
    dims = (w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv)
    route = lib.dq_route(*dims, det)
    assert route == (lib.DQ_DS_PANELS if det == 2 else lib.DQ_RELAY)
    n = lib.workspace_size(*dims, True, -1, det)
    if det == 2:
        assert n > (1 << 32)  # more than 2**31 bf16 dS elements
    C.log(f"int64 workspace: route {route}, {n / 2**30:.2f} GiB")
    t = dict(q=_bf(inp.q), k=_bf(inp.k), v=_bf(inp.v), o=_bf(c["o"]), do=_bf(inp.do),
             lse=torch.from_numpy(c["lse"]).cuda())
    outs = [torch.empty_like(t[x]) for x in ("q", "k", "v")]
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_ex(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], *outs,
                    scale=w.softmax_scale, causal=True, deterministic=det, workspace=ws)
    torch.cuda.synchronize()
    del ws
    dq, dk, dv = (C.bf16_tensor_to_f32(x) for x in outs)
    f = C.f64
    q, k, v, o, do = f(inp.q), f(inp.k), f(inp.v), f(c["o"]), f(inp.do)
    lse = c["lse"].astype(np.float64)
    # the last heads' panels lie past 2**31 elements (head 35 starts at 35 * 8192 * 8192)
    rows = [0, 1, 255, 256, 4095, 4096, 8000, 8191]
    got_q, ref_q, got_k, ref_k, got_v, ref_v = [], [], [], [], [], []
    for h in (0, 33, 35):
        ref_q.append(oracle.backward_dq_rows(q, k, v, o, do, lse, w.softmax_scale, 0, h, rows,
                                             causal=True))
        got_q.append(dq[0, h, rows])
        rk, rv = oracle.backward_dkdv_rows(q, k, v, o, do, lse, w.softmax_scale, 0, h, rows,
                                           causal=True)
        ref_k.append(rk)
        ref_v.append(rv)
        got_k.append(dk[0, h, rows])
        got_v.append(dv[0, h, rows])
    for name, g, r in (("dQ", got_q, ref_q), ("dK", got_k, ref_k), ("dV", got_v, ref_v)):
        C.assert_close(f"int64 workspace det={det} {name} sampled rows", np.concatenate(g),
                       np.concatenate(r))
    torch.cuda.empty_cache()
