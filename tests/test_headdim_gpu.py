"""GPU parity for head dims outside the native kernel sizes ("SDPA Backward (SM120)", "Support
surface": head dims that are multiples of 8 up to 256 run on the next larger native kernel, which
sees zeros beyond the actual head dim; d_qk >= d_v).  Each case runs the whole chain on tensors whose
head dim is the actual one (rows Dqk / Dv elements long, or strided views) and is compared with
the fp64 oracle on every dQ route, max|err| <= 1e-2 * max|ref| per tensor; every output element
is overwritten (outputs start as NaN)."""
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
    # (Dqk, Dv) -> kernel size: 96 -> 128, 40 -> 64, 32 native, 24 -> 32, 32/16 -> 32/32,
    # 72/56 -> 128/128, 176/104 -> 192/128,
    # 160 -> 256, 248 -> 256
    "d96_gqa_causal_s300": V(W["gqa_causal_s4096_d128"], Hq=4, Hkv=2, Sq=300, Skv=300, Dqk=96, Dv=96),
    "d40_s200": V(W["mha_s128_d64"], Sq=200, Skv=200, Dqk=40, Dv=40),
    "d32_causal_s257": V(W["mha_causal_s2048_d128"], B=1, Hq=2, Hkv=2, Sq=257, Skv=257, Dqk=32, Dv=32),
    "d24_s230": V(W["mha_s128_d64"], Sq=230, Skv=230, Dqk=24, Dv=24),
    "d32x16_window_padded_s280": V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=1, Sq=280, Skv=280,
                                   window_left=50, len_lo=120, Dqk=32, Dv=16),
    "d72x56_window_padded_s280": V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=1, Sq=280, Skv=280,
                                   window_left=70, len_lo=120, Dqk=72, Dv=56),
    "d176x104_causal_s300": V(W["mla_window_padded_s4096"], B=1, Hq=2, Hkv=2, Sq=300, Skv=300,
                              window_left=-1, padded=False, Dqk=176, Dv=104),
    "d160_s150": V(W["mha_det_s8192_d256"], Hq=2, Hkv=2, Sq=150, Skv=150, Dqk=160, Dv=160),
    "d248_causal_s130": V(W["mha_det_s8192_d256"], Hq=2, Hkv=1, Sq=130, Skv=130, causal=True,
                          Dqk=248, Dv=248),
    # native head dim 32 with each key tile's q range split into 4 parts (a grid of 16 workgroups:
    # 4 key tiles x 4 query heads), GQA: the staggered loop on partial ranges, the reduction over
    # (query head, part) slots
    "d32_gqa_split_causal_s1024": V(W["gqa_causal_s4096_d128"], B=1, Hq=4, Hkv=1, Sq=1024,
                                    Skv=1024, Dqk=32, Dv=32),
}


@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
@pytest.mark.parametrize("name", list(CASES))
def test_headdim_envelope_parity(name, det):
    w = CASES[name]
    C.log(f"head-dim case {name} route {det}: {w}")
    case = C.make_case(w)
    ref = C.oracle_backward(case)
    got = C.run_gpu(case, torch, deterministic=det)
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        C.assert_close(f"{name} route {det} {tname}", g, r)
    if case["lens"] is not None:
        for b, L in enumerate(case["lens"]):
            assert np.all(got[0][b, :, L:] == 0) and np.all(got[1][b, :, L:] == 0)
            assert np.all(got[2][b, :, L:] == 0)


@pytest.mark.parametrize("name", ["d96_gqa_causal_s300", "d32_causal_s257"])
def test_headdim_envelope_bshd_layout_and_gaps(name):
    # BSHD storage with a 16-element gap after each row: the gap columns of the inputs hold 7.0
    # and must not reach the result; those of the outputs hold NaN and must not be written
    import attention_backward_sdpa_amd as lib
    w = CASES[name]
    C.log(f"bshd layout with gaps: {name}")
    case = C.make_case(w)
    ref = C.oracle_backward(case)
    pad = 16

    def storage(shape, fill):
        B, H, S, D = shape
        return torch.full((B, S, H, D + pad), fill, dtype=torch.bfloat16, device="cuda")

    def view(st, D):
        return st[..., :D].permute(0, 2, 1, 3)  # (B, H, S, D), seq stride H * (D + pad)

    t = {}
    for x in ("q", "k", "v", "o", "do"):
        st = storage(case[x].shape, 7.0)
        D = case[x].shape[-1]
        st[..., :D] = torch.from_numpy(case[x].view(np.int16)).view(torch.bfloat16).cuda() \
            .permute(0, 2, 1, 3)
        t[x] = view(st, D)
    out_st = [storage(case[x].shape, float("nan")) for x in ("q", "k", "v")]
    outs = [view(st, case[x].shape[-1]) for st, x in zip(out_st, ("q", "k", "v"))]
    lse = torch.from_numpy(case["lse"]).cuda()
    kw = dict(scale=w.softmax_scale, causal=True, deterministic=3)
    n = lib.run_workspace_size(t["q"], t["k"], t["v"], **kw)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_run(t["q"], t["k"], t["v"], t["o"], t["do"], lse, *outs, workspace=ws, **kw)
    torch.cuda.synchronize()
    for tname, g, st, r in zip(("dQ", "dK", "dV"), outs, out_st, ref):
        C.assert_close(f"bshd {name} {tname}", g.float().cpu().numpy(), r)
        assert bool(torch.isnan(st[..., g.shape[-1]:].float()).all()), f"{tname} gap written"


BIAS_CASES = {
    "d72x56_window_padded_s280": CASES["d72x56_window_padded_s280"],
    # the native head-dim-32 kernel with bias, fp16, window and per-batch lengths
    "d32_window_padded_s200": V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=1, Sq=200, Skv=200,
                                window_left=50, len_lo=90, Dqk=32, Dv=32),
}


@pytest.mark.parametrize("name,det", [("d72x56_window_padded_s280", 0),
                                      ("d32_window_padded_s200", 0),
                                      ("d32_window_padded_s200", 3)])
def test_headdim_envelope_with_bias_fp16(name, det):
    import attention_backward_sdpa_amd as lib
    w = BIAS_CASES[name]
    C.log(f"bias fp16 case {name} route {det}: {w}")
    inp = synth.draw_inputs(w, dtype="fp16")
    f = lambda x: synth.bits_to_f32(x, "fp16").astype(np.float64)
    lens = [int(x) for x in inp.seq_q_lens]
    bias32 = np.random.default_rng(5).standard_normal((w.B, w.Hq, w.Sq, w.Skv)).astype(np.float32)
    kw = dict(causal=True, window_left=w.window_left, seq_q_lens=lens, seq_kv_lens=lens)
    o64, lse64 = oracle.forward(f(inp.q), f(inp.k), f(inp.v), w.softmax_scale,
                                bias=bias32.astype(np.float64), **kw)
    o_bits = synth.fp16_bits(o64.astype(np.float32))
    lse = lse64.astype(np.float32)
    ref = oracle.backward(f(inp.q), f(inp.k), f(inp.v), f(o_bits), f(inp.do),
                          lse.astype(np.float64), w.softmax_scale,
                          bias=bias32.astype(np.float64), return_dbias=True, **kw)
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).cuda()
    q, k, v, o, do = h(inp.q), h(inp.k), h(inp.v), h(o_bits), h(inp.do)
    outs = [torch.full_like(x, float("nan")) for x in (q, k, v)]
    dbias = torch.full((w.B, w.Hq, w.Sq, w.Skv), float("nan"), device="cuda")
    tl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    args = dict(scale=w.softmax_scale, causal=True, window_left=w.window_left, deterministic=det,
                seq_q_lens=tl, seq_kv_lens=tl, bias=torch.from_numpy(bias32).cuda(), dbias=dbias)
    n = lib.run_workspace_size(q, k, v, **args)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_run(q, k, v, o, do, torch.from_numpy(lse).cuda(), *outs, workspace=ws, **args)
    torch.cuda.synchronize()
    for tname, g, r in zip(("dQ", "dK", "dV", "dBias"), outs + [dbias], ref):
        C.assert_close(f"fp16 {name} bias route {det} {tname}", g.float().cpu().numpy(), r)
