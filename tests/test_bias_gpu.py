"""GPU parity of the additive bias and its gradient ("SDPA Backward (SM120)", "API Usage"
bias_tensor, "Support surface" bias) through sdpa_bwd_run, against the fp64 oracle.

The bias (1 or B, Hq, Sq, Skv) is drawn N(0,1), rounded to the io type (or kept fp32); the oracle
forward folds it into O and LSE, and the GPU chain receives exactly those tensors.  dQ/dK/dV and
dBias must match the oracle to max|err| <= 1e-2 * max|ref| per tensor, on every dQ route; dBias
elements of masked pairs, padded rows and padded keys are exactly 0; a batch-1 bias with B > 1
sums dBias over the batch (fp32 atomics, the atomic route only).
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

CASES = {
    # causal GQA, ragged S, per-batch bias
    "gqa_causal_d128_s333": (V(W["gqa_causal_s4096_d128"], B=2, Hq=4, Hkv=2, Sq=333, Skv=333), "B"),
    # same shape, one bias shared by the batch (dBias summed over it)
    "gqa_causal_d128_s333_b1": (V(W["gqa_causal_s4096_d128"], B=2, Hq=4, Hkv=2, Sq=333, Skv=333), 1),
    # MLA 192/128, causal window and padding
    "mla_window_padded_s300": (V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=2, Sq=300, Skv=300,
                                 window_left=90, len_lo=100), "B"),
    # non-causal D = 64, S_q != S_kv
    "mha_d64_s200x330": (V(W["mha_s128_d64"], B=1, Hq=2, Hkv=2, Sq=200, Skv=330), "B"),
    # non-causal D = 256
    "det_d256_s200": (V(W["mha_det_s8192_d256"], Hq=2, Hkv=2, Sq=200, Skv=200), "B"),
    # S_kv a multiple of 8 with an io-type bias: the 8-wave layout, the bias tile staged in LDS
    # (the relay route keeps the 4-wave layout)
    "gqa_causal_d128_s320": (V(W["gqa_causal_s4096_d128"], B=2, Hq=4, Hkv=2, Sq=320, Skv=320), "B"),
    "gqa_causal_d128_s320_b1": (V(W["gqa_causal_s4096_d128"], B=2, Hq=4, Hkv=2, Sq=320, Skv=320), 1),
    "window_padded_d128_s296": (V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=2, Sq=296, Skv=296,
                                  window_left=90, len_lo=100, Dqk=128, Dv=128), "B"),
    "mha_d64_s200x328": (V(W["mha_s128_d64"], B=1, Hq=2, Hkv=2, Sq=200, Skv=328), "B"),
}


def _case(w, bias_batch, bias_f32, seed=11):
    inp = synth.draw_inputs(w)
    Bb = w.B if bias_batch == "B" else 1
    rng = np.random.default_rng(seed)
    bias32 = rng.standard_normal((Bb, w.Hq, w.Sq, w.Skv)).astype(np.float32)
    bias_bits = None if bias_f32 else synth.bf16_bits(bias32)
    bias64 = (bias32 if bias_f32 else synth.bf16_to_f32(bias_bits)).astype(np.float64)
    f = C.f64
    lens = None if inp.seq_q_lens is None else [int(x) for x in inp.seq_q_lens]
    kw = dict(causal=w.causal, window_left=w.window_left, seq_q_lens=lens, seq_kv_lens=lens)
    o64, lse64 = oracle.forward(f(inp.q), f(inp.k), f(inp.v), w.softmax_scale, bias=bias64, **kw)
    o_bits = synth.bf16_bits(o64.astype(np.float32))
    lse = lse64.astype(np.float32)
    ref = oracle.backward(f(inp.q), f(inp.k), f(inp.v), f(o_bits), f(inp.do),
                          lse.astype(np.float64), w.softmax_scale, bias=bias64,
                          return_dbias=True, **kw)
    return inp, o_bits, lse, bias32 if bias_f32 else bias_bits, lens, ref


def _run(w, inp, o_bits, lse, bias, lens, det, want_dbias=True, ws_fill=None, dbias_io=False):
    import attention_backward_sdpa_amd as lib
    dev = "cuda"
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v, o, do = bf(inp.q), bf(inp.k), bf(inp.v), bf(o_bits), bf(inp.do)
    tb = torch.from_numpy(bias).to(dev) if bias.dtype == np.float32 else bf(bias)
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=dev)
    outs = [torch.empty_like(x) for x in (q, k, v)]
    for x in outs:
        x.view(torch.int16).fill_(0x7FC0)
    dbias = torch.full(tuple(bias.shape), float("nan"), dtype=torch.bfloat16 if dbias_io else torch.float32,
                       device=dev) if want_dbias else None
    kw = dict(scale=w.softmax_scale, causal=w.causal, window_left=w.window_left, deterministic=det,
              seq_q_lens=tl, seq_kv_lens=tl, bias=tb, dbias=dbias)
    n = lib.run_workspace_size(q, k, v, **kw)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    if ws_fill is not None:
        ws.copy_(ws_fill(ws.numel()))
    lib.sdpa_bwd_run(q, k, v, o, do, torch.from_numpy(lse).to(dev), *outs, workspace=ws, **kw)
    torch.cuda.synchronize()
    got = [C.bf16_tensor_to_f32(x) for x in outs]
    if dbias is not None and dbias_io:
        return got, C.bf16_tensor_to_f32(dbias)
    return got, None if dbias is None else dbias.cpu().numpy()


@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
@pytest.mark.parametrize("name", list(CASES))
def test_bias_parity(name, det):
    import attention_backward_sdpa_amd as lib
    w, bias_batch = CASES[name]
    C.log(f"bias case {name} route {det}: {w}")
    inp, o_bits, lse, bias, lens, ref = _case(w, bias_batch, bias_f32=False)
    if bias_batch == 1 and w.B > 1 and det != 0:
        # a batch-summed dBias needs atomics: the deterministic routes decline before any launch
        with pytest.raises(lib.SdpaBwdError) as e:
            _run(w, inp, o_bits, lse, bias, lens, det)
        assert e.value.status == lib.UNSUPPORTED
        return
    got, dbias = _run(w, inp, o_bits, lse, bias, lens, det)
    for tname, g, r in zip(("dQ", "dK", "dV", "dBias"), got + [dbias], ref):
        C.assert_close(f"bias {name} route {det} {tname}", g, r)
    # masked pairs, padded rows and padded keys: exactly zero
    for bb in range(dbias.shape[0]):
        L = None if lens is None else lens[bb]
        vis = oracle.visible_mask(w.Sq, w.Skv, w.causal, w.window_left, L, L)
        if bias_batch == 1 and w.B > 1:
            vis = np.any([oracle.visible_mask(w.Sq, w.Skv, w.causal, w.window_left,
                                              None if lens is None else lens[x],
                                              None if lens is None else lens[x])
                          for x in range(w.B)], axis=0)
        assert np.all(dbias[bb][:, ~vis] == 0)


@pytest.mark.parametrize("det", [0, 3], ids=["atomic", "dqpartials"])
def test_fp32_bias_and_no_dbias(det):
    w, _ = CASES["gqa_causal_d128_s333"]
    inp, o_bits, lse, bias, lens, ref = _case(w, "B", bias_f32=True)
    got, dbias = _run(w, inp, o_bits, lse, bias, lens, det)
    for tname, g, r in zip(("dQ", "dK", "dV", "dBias"), got + [dbias], ref):
        C.assert_close(f"fp32 bias route {det} {tname}", g, r)
    # the bias alone (no dBias output) gives the same dQ/dK/dV
    got2, _ = _run(w, inp, o_bits, lse, bias, lens, det, want_dbias=False)
    for tname, g, r in zip(("dQ", "dK", "dV"), got2, ref):
        C.assert_close(f"fp32 bias, no dBias, route {det} {tname}", g, r)


@pytest.mark.parametrize("det", [2, 3], ids=["dspanels", "dqpartials"])
def test_bias_deterministic_bitwise(det):
    w, _ = CASES["mla_window_padded_s300"]
    inp, o_bits, lse, bias, lens, ref = _case(w, "B", bias_f32=False)
    gen = torch.Generator(device="cpu").manual_seed(0)
    fill = lambda n: torch.randint(0, 256, (n,), dtype=torch.uint8, generator=gen).cuda()
    first = None
    for _ in range(5):
        got, dbias = _run(w, inp, o_bits, lse, bias, lens, det, ws_fill=fill)
        bits = [x.view(np.uint32) for x in got + [dbias]]
        if first is None:
            first = bits
        else:
            assert all(np.array_equal(a, b) for a, b in zip(first, bits))


@pytest.mark.parametrize("det", [0, 2, 3], ids=["atomic", "dspanels", "dqpartials"])
@pytest.mark.parametrize("name", ["gqa_causal_d128_s333", "gqa_causal_d128_s333_b1", "mla_window_padded_s300",
                                  "mha_d64_s200x330", "gqa_causal_d128_s320", "gqa_causal_d128_s320_b1"])
def test_io_dtype_dbias(name, det):
    # "The kernel chain" dbias_cvt: a bf16 dBias output is the fp32 dBias rounded once; within the
    # parity tolerance of the oracle, masked pairs exactly 0, and the other gradients unchanged
    w, bias_batch = CASES[name]
    if bias_batch == 1 and w.B > 1 and det != 0:
        pytest.skip("a batch-summed dBias needs the atomic route")
    C.log(f"io-type dBias {name} route {det}")
    inp, o_bits, lse, bias, lens, ref = _case(w, bias_batch, bias_f32=False)
    got, dbias = _run(w, inp, o_bits, lse, bias, lens, det, dbias_io=True)
    for tname, g, r in zip(("dQ", "dK", "dV", "dBias"), got + [dbias], ref):
        C.assert_close(f"io dBias {name} route {det} {tname}", g, r)
    got32, dbias32 = _run(w, inp, o_bits, lse, bias, lens, det)
    # the io-type dBias is the fp32 one rounded to bf16 (exactly, on the deterministic routes)
    if det != 0:
        assert np.array_equal(dbias, C.synth.round_bf16(dbias32.astype(np.float32)))
        for a, b in zip(got, got32):
            assert np.array_equal(a, b)
    for bb in range(dbias.shape[0]):
        L = None if lens is None else lens[bb]
        vis = oracle.visible_mask(w.Sq, w.Skv, w.causal, w.window_left, L, L)
        if bias_batch == 1 and w.B > 1:
            vis = np.any([oracle.visible_mask(w.Sq, w.Skv, w.causal, w.window_left,
                                              None if lens is None else lens[x],
                                              None if lens is None else lens[x])
                          for x in range(w.B)], axis=0)
        assert np.all(dbias[bb][:, ~vis] == 0)


# fp16 io with a bias of the io type (S_kv a multiple of 8): the 8-wave layout with the bias tile
# staged in LDS as fp16 (the relay keeps the 4-wave layout).  Tolerance as for the other fp16
# cases: fp16 keeps 11 significant bits, so the error budget is 4 unit roundoffs (2e-3), which a
# bias or operand read in the wrong 16-bit format would exceed by far.
FP16_CASES = {
    "fp16_gqa_causal_d128_s320": V(W["gqa_causal_s4096_d128"], B=2, Hq=4, Hkv=2, Sq=320, Skv=320),
    "fp16_window_padded_d64_s264": V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=2, Sq=264,
                                     Skv=264, window_left=90, len_lo=100, Dqk=64, Dv=64),
    "fp16_d32_s200x328": V(W["mha_s128_d64"], B=1, Hq=2, Hkv=2, Sq=200, Skv=328, Dqk=32, Dv=32),
}
FP16_TOL = 2e-3


@pytest.mark.parametrize("dbias_io", [False, True], ids=["dbias_f32", "dbias_fp16"])
@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
@pytest.mark.parametrize("name", list(FP16_CASES))
def test_fp16_io_bias_parity(name, det, dbias_io):
    import attention_backward_sdpa_amd as lib
    w = FP16_CASES[name]
    C.log(f"fp16 io-type bias case {name} route {det}, fp16 dBias {dbias_io}: {w}")
    inp = synth.draw_inputs(w, dtype="fp16")
    f = lambda x: synth.fp16_to_f32(x).astype(np.float64)
    bias_bits = synth.fp16_bits(np.random.default_rng(23).standard_normal(
        (w.B, w.Hq, w.Sq, w.Skv)).astype(np.float32))
    bias64 = f(bias_bits)
    lens = None if inp.seq_q_lens is None else [int(x) for x in inp.seq_q_lens]
    kw = dict(causal=w.causal, window_left=w.window_left, seq_q_lens=lens, seq_kv_lens=lens)
    o64, lse64 = oracle.forward(f(inp.q), f(inp.k), f(inp.v), w.softmax_scale, bias=bias64, **kw)
    o_bits = synth.fp16_bits(o64.astype(np.float32))
    lse = lse64.astype(np.float32)
    ref = oracle.backward(f(inp.q), f(inp.k), f(inp.v), f(o_bits), f(inp.do),
                          lse.astype(np.float64), w.softmax_scale, bias=bias64,
                          return_dbias=True, **kw)
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).cuda()
    q, k, v, o, do = h(inp.q), h(inp.k), h(inp.v), h(o_bits), h(inp.do)
    outs = [torch.full_like(x, float("nan")) for x in (q, k, v)]
    dbias = torch.full((w.B, w.Hq, w.Sq, w.Skv), float("nan"), device="cuda",
                       dtype=torch.float16 if dbias_io else torch.float32)
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    args = dict(scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
                deterministic=det, seq_q_lens=tl, seq_kv_lens=tl, bias=h(bias_bits), dbias=dbias)
    n = lib.run_workspace_size(q, k, v, **args)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_run(q, k, v, o, do, torch.from_numpy(lse).cuda(), *outs, workspace=ws, **args)
    torch.cuda.synchronize()
    got = [x.float().cpu().numpy() for x in outs + [dbias]]
    for tname, g, r in zip(("dQ", "dK", "dV", "dBias"), got, ref):
        C.assert_close(f"fp16 bias {name} route {det} {tname}", g, r, tol=FP16_TOL)
    for bb in range(w.B):
        L = None if lens is None else lens[bb]
        vis = oracle.visible_mask(w.Sq, w.Skv, w.causal, w.window_left, L, L)
        assert np.all(got[3][bb][:, ~vis] == 0)


# An additive bias under the other mask forms: bottom-right causal with S_q < S_kv, a right band,
# and separate query / key lengths, with S_kv a multiple of 8 (the 8-wave layout with the bias tile
# in LDS, whose last key tile runs past the keys and whose bottom q tile past the queries) and not
# (the 4-wave layout).
MASK_CASES = {
    # name: (base workload, overrides, q lens, kv lens, bottom_right, window_right)
    "bottom_right_sq_lt_skv_d128": ("gqa_causal_s4096_d128", dict(B=2, Hq=4, Hkv=2, Sq=300, Skv=520),
                                    None, None, True, 0),
    "bottom_right_band_lens_d64": ("mha_s128_d64", dict(B=2, Hq=2, Hkv=2, Sq=260, Skv=392, causal=True,
                                                        window_left=100), [200, 260], [392, 300], True, 3),
    "bottom_right_lens_d128_skv_odd": ("gqa_causal_s4096_d128", dict(B=2, Hq=4, Hkv=2, Sq=300, Skv=517),
                                       [300, 211], [517, 400], True, 0),
}


@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
@pytest.mark.parametrize("name", list(MASK_CASES))
def test_bias_mask_forms(name, det):
    import attention_backward_sdpa_amd as lib
    base, ov, lq, lkv, br, wr = MASK_CASES[name]
    w = V(W[base], **ov)
    C.log(f"bias mask case {name} route {det}: {w}, lens {lq} / {lkv}, bottom_right {br}, band {wr}")
    inp = synth.draw_inputs(w)
    f = C.f64
    bias_bits = synth.bf16_bits(np.random.default_rng(31).standard_normal(
        (w.B, w.Hq, w.Sq, w.Skv)).astype(np.float32))
    bias64 = f(bias_bits)
    kw = dict(causal=w.causal, window_left=w.window_left, seq_q_lens=lq, seq_kv_lens=lkv,
              bottom_right=br, window_right=wr)
    o64, lse64 = oracle.forward(f(inp.q), f(inp.k), f(inp.v), w.softmax_scale, bias=bias64, **kw)
    o_bits = synth.bf16_bits(o64.astype(np.float32))
    lse = lse64.astype(np.float32)
    ref = oracle.backward(f(inp.q), f(inp.k), f(inp.v), f(o_bits), f(inp.do), lse.astype(np.float64),
                          w.softmax_scale, bias=bias64, return_dbias=True, **kw)
    dev = "cuda"
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v, o, do = bf(inp.q), bf(inp.k), bf(inp.v), bf(o_bits), bf(inp.do)
    outs = [torch.empty_like(x) for x in (q, k, v)]
    for x in outs:
        x.view(torch.int16).fill_(0x7FC0)
    dbias = torch.full((w.B, w.Hq, w.Sq, w.Skv), float("nan"), device=dev)
    tl = lambda L: None if L is None else torch.tensor(L, dtype=torch.int32, device=dev)
    args = dict(scale=w.softmax_scale, causal=w.causal, window_left=w.window_left, deterministic=det,
                seq_q_lens=tl(lq), seq_kv_lens=tl(lkv), causal_bottom_right=br, window_right=wr,
                bias=bf(bias_bits), dbias=dbias)
    n = lib.run_workspace_size(q, k, v, **args)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    lib.sdpa_bwd_run(q, k, v, o, do, torch.from_numpy(lse).to(dev), *outs, workspace=ws, **args)
    torch.cuda.synchronize()
    got = [C.bf16_tensor_to_f32(x) for x in outs] + [dbias.cpu().numpy()]
    for tname, g, r in zip(("dQ", "dK", "dV", "dBias"), got, ref):
        C.assert_close(f"bias mask {name} route {det} {tname}", g, r)
    for bb in range(w.B):
        vis = oracle.visible_mask(w.Sq, w.Skv, w.causal, w.window_left,
                                  None if lq is None else lq[bb], None if lkv is None else lkv[bb],
                                  br, wr)
        assert np.all(got[3][bb][:, ~vis] == 0)
