"""GPU parity of the HIP attention backward against the fp64 CPU oracle.

Reduced-size cases span several q/key tiles and end in ragged tails; every output buffer is
poisoned with NaN before the call so that an element the chain fails to write shows up.  The
tolerance is the stated one: max |err| <= 1e-2 * max |ref| per tensor.
"""
import numpy as np
import pytest

from attention_backward_sdpa_amd import synth
from tests import _common as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
V = synth.small_variant

SMALL_CASES = {
    # the tiny workload at its full size: non-causal MHA, D = 64
    "mha_s128_d64": W["mha_s128_d64"],
    # causal MHA, D = 128, ragged S (not a multiple of the 64-row q tile or the 128-key tile)
    "mha_causal_d128_s300": V(W["mha_causal_s2048_d128"], B=2, Hq=2, Hkv=2, Sq=300, Skv=300),
    # causal GQA group 4, D = 128
    "gqa_causal_d128_s333": V(W["gqa_causal_s4096_d128"], Hq=8, Hkv=2, Sq=333, Skv=333),
    # MQA, non-causal
    "mqa_d128_s200": V(W["gqa_causal_s4096_d128"], Hq=4, Hkv=1, Sq=200, Skv=200, causal=False),
    # deterministic non-causal D = 256, inputs 0.5 * N(0,1)
    "det_d256_s200": V(W["mha_det_s8192_d256"], Hq=2, Hkv=2, Sq=200, Skv=200),
    # MLA 192/128, causal + left window + padding
    "mla_window_padded_s400": V(W["mla_window_padded_s4096"], B=3, Hq=2, Hkv=2, Sq=400, Skv=400,
                                window_left=100, len_lo=100),
    # window without causal
    "window_only_d64_s260": V(W["mha_s128_d64"], Sq=260, Skv=260, window_left=70),
    # exact tile multiples
    "causal_d128_s256": V(W["mha_causal_s2048_d128"], B=1, Hq=2, Hkv=2, Sq=256, Skv=256),
    # a single query and key
    "s1_d128": V(W["mha_causal_s2048_d128"], B=1, Hq=2, Hkv=2, Sq=1, Skv=1),
    # deterministic GQA causal D = 128
    "det_gqa_causal_d128_s333": V(W["gqa_causal_s4096_d128"], Hq=8, Hkv=2, Sq=333, Skv=333,
                                  deterministic=True),
    # deterministic MLA with window + padding
    "det_mla_window_padded_s400": V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=1, Sq=400,
                                    Skv=400, window_left=100, len_lo=100, deterministic=True),
    # non-deterministic D = 256
    "nondet_d256_s200": V(W["mha_det_s8192_d256"], Hq=2, Hkv=2, Sq=200, Skv=200,
                          deterministic=False),
    # few workgroups per CU: every key tile's q-tile range is split in parts whose dK/dV
    # partials the reduction sums (causal MHA, 3 key tiles x 2 heads, 19 q tiles)
    "split_causal_d128_s600": V(W["mha_causal_s2048_d128"], B=1, Hq=2, Hkv=2, Sq=600, Skv=600),
    # split ranges under GQA on the deterministic route
    "det_gqa_split_d128_s700": V(W["gqa_causal_s4096_d128"], Hq=4, Hkv=2, Sq=700, Skv=700,
                                 deterministic=True),
    # head dim 32 (its own kernel: 16 x 16 GEMM4 blocks on four of the eight waves), causal GQA
    "d32_gqa_causal_s300": V(W["gqa_causal_s4096_d128"], Hq=4, Hkv=2, Sq=300, Skv=300, Dqk=32, Dv=32),
    # split ranges with the 4-wave MLA kernel, a window and padding
    "mla_split_window_padded_s900": V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=2, Sq=900,
                                      Skv=900, window_left=300, len_lo=500),
}


# dQ routes (the `deterministic` argument): None = the workload's own (False / True)
ROUTES = {"default": None, "dspanels": 2, "dqpartials": 3, "relay": 4}


@pytest.mark.parametrize("route", list(ROUTES))
@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_small_parity(name, route):
    w = SMALL_CASES[name]
    C.log(f"case {name} route {route}: {w}")
    case = C.make_case(w)
    ref = C.oracle_backward(case)
    got = C.run_gpu(case, torch, deterministic=ROUTES[route])
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        C.assert_close(f"{name} {tname}", g, r)
    # padded rows are exactly zero
    if case["lens"] is not None:
        for b, L in enumerate(case["lens"]):
            assert np.all(got[0][b, :, L:] == 0), "dQ rows past seq_q must be zero"
            assert np.all(got[1][b, :, L:] == 0) and np.all(got[2][b, :, L:] == 0)


@pytest.mark.parametrize("name,det", [("det_d256_s200", True), ("gqa_causal_d128_s333", 2),
                                      ("gqa_causal_d128_s333", 3), ("split_causal_d128_s600", 3),
                                      ("gqa_causal_d128_s333", 4), ("split_causal_d128_s600", 4),
                                      ("det_mla_window_padded_s400", 4), ("mha_s128_d64", 4),
                                      ("det_d256_s200", 4)])
def test_deterministic_bitwise_over_runs(name, det):
    # 10 runs over a workspace refilled with random bytes each time: identical bits
    w = SMALL_CASES[name]
    case = C.make_case(w)
    t = C.to_device(case, torch)
    gen = torch.Generator(device="cpu").manual_seed(0)

    def random_bytes(n):
        return torch.randint(0, 256, (n,), dtype=torch.uint8, generator=gen).cuda()

    first = None
    for run in range(10):
        out = C.run_gpu(case, torch, deterministic=det, dev_inputs=t, ws_fill=random_bytes)
        if first is None:
            first = out
        else:
            for a, b in zip(first, out):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"run {run} differs"


def test_routes_agree():
    w = SMALL_CASES["gqa_causal_d128_s333"]
    case = C.make_case(w)
    ref = C.oracle_backward(case)
    outs = {r: C.run_gpu(case, torch, deterministic=r) for r in (0, 1, 2, 3, 4)}
    for r, out in outs.items():
        for tname, x, rr in zip(("dQ", "dK", "dV"), out, ref):
            C.assert_close(f"route {r} {tname}", x, rr)
    # dK and dV are deterministic on every route and come from the same GEMM3/GEMM5 arithmetic
    for r in (1, 2, 3, 4):
        assert np.array_equal(outs[0][1], outs[r][1]) and np.array_equal(outs[0][2], outs[r][2])
    # at head dim 128 the deterministic choice is the dS-panel route
    for x, y in zip(outs[1], outs[2]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


@pytest.mark.parametrize("name", ["gqa_causal_d128_s333", "split_causal_d128_s600", "mha_s128_d64",
                                  "det_d256_s200", "mla_window_padded_s400",
                                  "mla_split_window_padded_s900", "window_only_d64_s260", "s1_d128"])
def test_relay_equals_dq_partials(name):
    # the relay adds the same fp32 GEMM4 blocks in the same ascending key-tile order as the
    # dQ-partial reduction (whose sum starts from 0, the relay's from the first block), with the
    # same final scaling: equal values
    w = SMALL_CASES[name]
    case = C.make_case(w)
    t = C.to_device(case, torch)
    a = C.run_gpu(case, torch, deterministic=3, dev_inputs=t)
    b = C.run_gpu(case, torch, deterministic=4, dev_inputs=t)
    for tname, x, y in zip(("dQ", "dK", "dV"), a, b):
        assert np.array_equal(x, y), f"{name} {tname}: relay differs from the dQ-partial route"


def test_linear_in_dO_bitwise():
    # doubling dO doubles every intermediate exactly in bf16/fp32, so the deterministic route
    # must return exactly twice the gradients
    w = SMALL_CASES["det_mla_window_padded_s400"]
    case = C.make_case(w)
    case2 = dict(case)
    do2 = C.synth.bf16_bits((C.synth.bf16_to_f32(case["do"]) * 2).astype(np.float32))
    case2["do"] = do2
    a = C.run_gpu(case, torch)
    b = C.run_gpu(case2, torch)
    for x, y in zip(a, b):
        assert np.array_equal(2 * x, y)


def test_non_default_stream():
    w = SMALL_CASES["mha_causal_d128_s300"]
    case = C.make_case(w)
    s = torch.cuda.Stream()
    got = C.run_gpu(case, torch, stream=s)
    ref = C.oracle_backward(case)
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        C.assert_close(f"stream {tname}", g, r)


def test_fully_masked_rows_and_zero_lengths():
    # one batch entry with length 0 (every row masked, LSE = -inf) next to a normal one
    w = V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=2, Sq=130, Skv=130, window_left=40,
          len_lo=0)
    case = dict(C.make_case(w))
    lens = np.array([0, 97], dtype=np.int32)
    case["lens"] = lens
    # recompute O / LSE for the forced lengths
    q, k, v = (C.f64(case[x]) for x in ("q", "k", "v"))
    o64, lse64 = C.oracle.forward(q, k, v, w.softmax_scale, causal=True, window_left=40,
                                  seq_q_lens=list(lens), seq_kv_lens=list(lens))
    case["o"] = C.synth.bf16_bits(o64.astype(np.float32))
    case["lse"] = lse64.astype(np.float32)
    ref = C.oracle_backward(case)
    got = C.run_gpu(case, torch)
    assert np.all(got[0][0] == 0) and np.all(got[1][0] == 0) and np.all(got[2][0] == 0)
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        C.assert_close(f"masked {tname}", g, r)


# ---- mask and shape surface: S_q != S_kv, bottom-right causal, right band, separate q / kv
# padding lengths ("SDPA Backward (SM120)", "API Usage" and "Causal, sliding-window, and padding
# masks").  Each case: (name, base workload, overrides, q lens, kv lens, bottom_right, window_right)
SURFACE_CASES = [
    ("sq_lt_skv_bottom_right", "gqa_causal_s4096_d128", dict(B=2, Hq=4, Hkv=2, Sq=300, Skv=520),
     [300, 180], [520, 260], True, 0),
    ("sq_gt_skv_top_left", "mha_causal_s2048_d128", dict(B=1, Hq=2, Hkv=2, Sq=520, Skv=300),
     None, None, False, 0),
    ("right_band_window", "mha_causal_s2048_d128", dict(B=1, Hq=2, Hkv=2, Sq=400, Skv=400,
                                                       window_left=90), None, None, False, 37),
    ("mla_bottom_right_window_lens", "mla_window_padded_s4096", dict(B=2, Hq=2, Hkv=2, Sq=330,
     Skv=610, window_left=150, padded=False), [330, 201], [610, 333], True, 0),
    ("det_d256_bottom_right_lens", "mha_det_s8192_d256", dict(B=2, Hq=2, Hkv=2, Sq=260, Skv=390,
     causal=True), [260, 99], [390, 150], True, 0),
]


@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
@pytest.mark.parametrize("case_def", SURFACE_CASES, ids=[c[0] for c in SURFACE_CASES])
def test_mask_and_shape_surface(case_def, det):
    import attention_backward_sdpa_amd as lib
    name, base, over, lq, lkv, br, wr = case_def
    w = V(W[base], **over)
    inp = synth.draw_inputs(w)
    f = C.f64
    q, k, v = f(inp.q), f(inp.k), f(inp.v)
    kw = dict(causal=w.causal, window_left=w.window_left, seq_q_lens=lq, seq_kv_lens=lkv,
              bottom_right=br, window_right=wr)
    o64, lse64 = C.oracle.forward(q, k, v, w.softmax_scale, **kw)
    o_bits = synth.bf16_bits(o64.astype(np.float32))
    lse = lse64.astype(np.float32)
    ref = C.oracle.backward(q, k, v, f(o_bits), f(inp.do), lse.astype(np.float64),
                            w.softmax_scale, **kw)
    dev = "cuda"
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    tq, tk, tv, to, tdo = bf(inp.q), bf(inp.k), bf(inp.v), bf(o_bits), bf(inp.do)
    tlse = torch.from_numpy(lse).to(dev)
    tlq = None if lq is None else torch.tensor(lq, dtype=torch.int32, device=dev)
    tlkv = None if lkv is None else torch.tensor(lkv, dtype=torch.int32, device=dev)
    outs = [torch.empty_like(x) for x in (tq, tk, tv)]
    for x in outs:
        x.view(torch.int16).fill_(0x7FC0)
    n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, w.causal, w.window_left,
                           det, lq is not None)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    C.log(f"surface case {name} deterministic={det}")
    lib.sdpa_bwd_ex(tq, tk, tv, to, tdo, tlse, *outs, scale=w.softmax_scale, causal=w.causal,
                    window_left=w.window_left, deterministic=det, seq_q_lens=tlq,
                    seq_kv_lens=tlkv, causal_bottom_right=br, window_right=wr, workspace=ws)
    torch.cuda.synchronize()
    got = [C.bf16_tensor_to_f32(x) for x in outs]
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        C.assert_close(f"{name} route {det} {tname}", g, r)
