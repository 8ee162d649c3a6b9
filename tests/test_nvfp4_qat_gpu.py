"""GPU parity of the NVFP4 attention-QAT backward ("NVFP4 Attention QAT Backward", "Overview")
through sdpa_bwd_nvfp4_qat, against the fp64 oracle of oracle.nvfp4_qat.

Inputs: Q, K, V, dO ~ N(0, 1) rounded to bf16 (MHA, head dim 128); O_hp and LSE from the oracle's
QAT forward (softmax of the fake-quantised inputs), rounded to bf16 / fp32.  The fake-quantised
copies of Q, K, V the library leaves at the start of the workspace must equal the oracle's bit for
bit (the quantisation is exact integer work once the fp32 divisions are correctly rounded); dQ,
dK, dV must match the oracle to max|err| <= 1e-2 * max|ref| per tensor on every dQ route.
"""
import numpy as np
import pytest

import oracle
from attention_backward_sdpa_amd import synth
from tests import _common as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
V = synth.small_variant

# (workload, causal): MHA, head dim 128
CASES = {
    "causal_s300": V(W["mha_causal_s2048_d128"], B=1, Hq=2, Hkv=2, Sq=300, Skv=300),
    "causal_s640": V(W["mha_causal_s2048_d128"], B=1, Hq=1, Hkv=1, Sq=640, Skv=640),
    "cross_s200x333": V(W["mha_causal_s2048_d128"], B=2, Hq=2, Hkv=2, Sq=200, Skv=333, causal=False),
    "s128": V(W["mha_causal_s2048_d128"], B=1, Hq=2, Hkv=2, Sq=128, Skv=128, causal=False),
}


def _al(n):
    return (n + 255) // 256 * 256


def _case(w):
    inp = synth.draw_inputs(w)
    f32 = lambda bits: synth.bf16_to_f32(bits)
    q, k, v, do = (f32(x) for x in (inp.q, inp.k, inp.v, inp.do))
    o64, lse64 = oracle.qat_forward(q, k, v, w.softmax_scale, causal=w.causal)
    o_bits = synth.bf16_bits(o64.astype(np.float32))
    lse = lse64.astype(np.float32)
    ref = oracle.qat_backward(q, k, v, synth.bf16_to_f32(o_bits), do, lse, w.softmax_scale,
                              causal=w.causal)
    return inp, o_bits, lse, ref


def _run(w, inp, o_bits, lse, det):
    import attention_backward_sdpa_amd as lib
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, o, do = bf(inp.q), bf(inp.k), bf(inp.v), bf(o_bits), bf(inp.do)
    outs = [torch.empty_like(x) for x in (q, k, v)]
    for x in outs:
        x.view(torch.int16).fill_(0x7FC0)
    n = lib.nvfp4_qat_workspace_size(w.B, w.Hq, w.Sq, w.Skv, 128, w.causal, det)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_nvfp4_qat(q, k, v, o, do, torch.from_numpy(lse).cuda(), *outs,
                           scale=w.softmax_scale, causal=w.causal, deterministic=det, workspace=ws)
    torch.cuda.synchronize()
    return [C.bf16_tensor_to_f32(x) for x in outs], ws


@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
@pytest.mark.parametrize("name", list(CASES))
def test_nvfp4_qat_parity(name, det):
    w = CASES[name]
    C.log(f"nvfp4 qat case {name} route {det}: {w}")
    inp, o_bits, lse, ref = _case(w)
    got, _ = _run(w, inp, o_bits, lse, det)
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        C.assert_close(f"qat {name} route {det} {tname}", g, r)


def test_nvfp4_qat_quantised_inputs_bit_exact():
    w = CASES["cross_s200x333"]
    inp, o_bits, lse, _ = _case(w)
    _, ws = _run(w, inp, o_bits, lse, 0)
    raw = ws.cpu().numpy()
    nq = w.B * w.Hq * w.Sq * 128
    nk = w.B * w.Hq * w.Skv * 128
    offs = [(0, nq, inp.q), (_al(2 * nq), nk, inp.k), (_al(2 * nq) + _al(2 * nk), nk, inp.v)]
    for off, n, bits in offs:
        got = raw[off:off + 2 * n].view(np.uint16).reshape(bits.shape)
        want = synth.bf16_bits(oracle.fake_nvfp4(synth.bf16_to_f32(bits)))
        assert np.array_equal(got, want)


def test_nvfp4_qat_dv_uses_quantised_probability():
    # the parity bound separates the QAT dV from the plain P^T dO on these inputs, so a missing
    # probability quantisation could not pass test_nvfp4_qat_parity
    w = CASES["causal_s300"]
    inp, o_bits, lse, ref = _case(w)
    f = lambda bits: oracle.fake_nvfp4(synth.bf16_to_f32(bits)).astype(np.float64)
    plain = oracle.backward(f(inp.q), f(inp.k), f(inp.v), synth.bf16_to_f32(o_bits).astype(np.float64),
                            synth.bf16_to_f32(inp.do).astype(np.float64), lse.astype(np.float64),
                            w.softmax_scale, causal=True)
    assert C.max_rel_err(plain[2].astype(np.float32), ref[2]) > 5e-2
    got, _ = _run(w, inp, o_bits, lse, 0)
    assert C.max_rel_err(got[2], plain[2]) > 5e-2


@pytest.mark.parametrize("det", [0, 2], ids=["atomic", "dspanels"])
def test_nvfp4_qat_fullsize_sampled_rows(det):
    # the QAT page's example shape, B1 H16 S4096 D128 non-causal (and its causal variant on the
    # atomic route), in the launch configuration bench.py --qat times: sampled rows of three heads;
    # O_hp and LSE from the oracle's QAT forward
    from oracle import nvfp4_qat as Q
    w = W["qat_mha_s4096_d128"]
    for causal in ([False, True] if det == 0 else [False]):
        wc = V(w, causal=causal)
        C.log(f"qat full size causal={causal} route {det}: drawing inputs")
        inp = synth.draw_inputs(wc)
        f32 = lambda bits: synth.bf16_to_f32(bits)
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        C.log("qat full size: fp64 oracle QAT forward (O_hp and LSE of the fake-quantised inputs)")
        o64, lse64 = oracle.qat_forward(f32(inp.q), f32(inp.k), f32(inp.v), wc.softmax_scale,
                                        causal=causal)
        o = bf(synth.bf16_bits(o64.astype(np.float32)))
        lse = torch.from_numpy(lse64.astype(np.float32)).cuda()
        del o64, lse64
        q, k, v, do = bf(inp.q), bf(inp.k), bf(inp.v), bf(inp.do)
        outs = [torch.empty_like(x) for x in (q, k, v)]
        import attention_backward_sdpa_amd as lib
        n = lib.nvfp4_qat_workspace_size(w.B, w.Hq, w.Sq, w.Skv, 128, causal, det)
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        C.log("qat full size: GPU chain")
        lib.sdpa_bwd_nvfp4_qat(q, k, v, o, do, lse, *outs, scale=w.softmax_scale, causal=causal,
                               deterministic=det, workspace=ws)
        torch.cuda.synchronize()
        got = [C.bf16_tensor_to_f32(x) for x in outs]
        o_h = synth.bf16_to_f32(o.cpu().view(torch.int16).numpy().view(np.uint16))
        lse_h = lse.cpu().numpy()
        xs = [f32(inp.q), f32(inp.k), f32(inp.v)]
        rows = [0, 1, 15, 16, 31, 32, 127, 128, 2047, 4064, 4095]
        for h in (0, 7, 15):
            C.log(f"qat full size: oracle rows of head {h}")
            dq, dk, dv = Q.qat_backward_rows(*xs, o_h, f32(inp.do), lse_h, w.softmax_scale, 0, h,
                                             rows, rows, causal=causal)
            for tname, g, r in (("dQ", got[0][0, h, rows], dq), ("dK", got[1][0, h, rows], dk),
                                ("dV", got[2][0, h, rows], dv)):
                C.assert_close(f"qat full size causal={causal} route {det} head {h} {tname}", g, r)
