"""GPU parity with fp16 io ("Support surface": FP16 / BF16, LSE fp32): Q, K, V, dO drawn as in the
bf16 cases but rounded to IEEE binary16; O and LSE from the fp64 oracle forward rounded to fp16 /
fp32; the expected gradients are the oracle's on exactly those values.  Outputs are poisoned with
an fp16 NaN first, so every element must be written.

Tolerance: fp16 keeps 11 significant bits (unit roundoff u = 2^-11 ~ 4.9e-4) against bf16's 8, so
the same arithmetic lands about 8x closer to the fp64 result.  The final rounding of each output
costs at most u/2 of max|ref|; the fp16 copies of P and dS that feed the products, and the fp16
GQA partials, add errors of the same order that mostly cancel over the contraction.  FP16_TOL =
4u bounds all of them with room, and it fails if any step silently ran in bf16 (~4e-3)."""
import numpy as np
import pytest

import oracle
from attention_backward_sdpa_amd import synth
from tests import _common as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
V = synth.small_variant
NAN16 = 0x7E00
FP16_TOL = 2e-3

CASES = {
    "gqa_causal_d128_s333": V(W["gqa_causal_s4096_d128"], Hq=8, Hkv=2, Sq=333, Skv=333),
    "mla_window_lens_s400": V(W["mla_window_padded_s4096"], B=2, Hq=2, Hkv=2, Sq=400, Skv=400,
                              window_left=100, len_lo=100),
    "d256_noncausal_s200": V(W["mha_det_s8192_d256"], Hq=2, Hkv=2, Sq=200, Skv=200),
    "d64_s128": W["mha_s128_d64"],
    # head dim 32 (staggered wave groups): GQA, causal window, padding lengths
    "d32_gqa_window_lens_s290": V(W["mla_window_padded_s4096"], B=2, Hq=4, Hkv=2, Sq=290, Skv=290,
                                  window_left=70, len_lo=130, Dqk=32, Dv=32),
}


def fp16_case(w):
    inp = synth.draw_inputs(w, dtype="fp16")
    f = lambda b: synth.fp16_to_f32(b).astype(np.float64)
    lens = None if inp.seq_q_lens is None else [int(x) for x in inp.seq_q_lens]
    kw = dict(causal=w.causal, window_left=w.window_left, seq_q_lens=lens, seq_kv_lens=lens)
    o64, lse64 = oracle.forward(f(inp.q), f(inp.k), f(inp.v), w.softmax_scale, **kw)
    o_bits = synth.fp16_bits(o64.astype(np.float32))
    lse = lse64.astype(np.float32)
    ref = oracle.backward(f(inp.q), f(inp.k), f(inp.v), f(o_bits), f(inp.do),
                          lse.astype(np.float64), w.softmax_scale, **kw)
    return inp, o_bits, lse, lens, ref


def to_half(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.float16)


@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
@pytest.mark.parametrize("name", list(CASES))
def test_fp16_parity(name, det):
    import attention_backward_sdpa_amd as lib
    w = CASES[name]
    C.log(f"fp16 case {name} (dQ route {det}): {w}")
    inp, o_bits, lse, lens, ref = fp16_case(w)
    q, k, v, o, do = (to_half(x) for x in (inp.q, inp.k, inp.v, o_bits, inp.do))
    outs = [torch.empty_like(x) for x in (q, k, v)]
    for x in outs:
        x.view(torch.int16).fill_(NAN16)
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, w.causal, w.window_left,
                           det, tl is not None)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_ex(q, k, v, o, do, torch.from_numpy(lse).to("cuda"), *outs,
                    scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
                    deterministic=det, seq_q_lens=tl, seq_kv_lens=tl, workspace=ws)
    torch.cuda.synchronize()
    for tname, g, r in zip(("dQ", "dK", "dV"), outs, ref):
        C.assert_close(f"fp16 {name} {tname}", g.float().cpu().numpy(), r, tol=FP16_TOL)
    if lens is not None:
        for b, L in enumerate(lens):
            for x in outs:
                assert bool((x[b, :, L:] == 0).all()), "rows past the length must be zero"


@pytest.mark.parametrize("det", [2, 3], ids=["dspanels", "dqpartials"])
def test_fp16_deterministic_bitwise(det):
    import attention_backward_sdpa_amd as lib
    w = CASES["gqa_causal_d128_s333"]
    inp, o_bits, lse, lens, _ = fp16_case(w)
    q, k, v, o, do = (to_half(x) for x in (inp.q, inp.k, inp.v, o_bits, inp.do))
    tlse = torch.from_numpy(lse).to("cuda")
    n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, w.causal, -1, det)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    first = None
    for _ in range(3):
        outs = [torch.empty_like(x) for x in (q, k, v)]
        lib.sdpa_bwd_ex(q, k, v, o, do, tlse, *outs, scale=w.softmax_scale, causal=True,
                        deterministic=det, workspace=ws)
        torch.cuda.synchronize()
        bits = [x.view(torch.int16).cpu() for x in outs]
        if first is None:
            first = bits
        else:
            assert all(bool((a == b).all()) for a, b in zip(first, bits))


@pytest.mark.parametrize("det", [0, 2, 3, 4], ids=["atomic", "dspanels", "dqpartials", "relay"])
def test_fp16_bshd_layout(det):
    """fp16 io through BSHD storage (strided views) on a GQA window case with padding lengths."""
    import attention_backward_sdpa_amd as lib
    w = V(W["gqa_causal_s4096_d128"], B=2, Hq=4, Hkv=2, Sq=230, Skv=230, window_left=90)
    C.log(f"fp16 bshd (dQ route {det}): {w}")
    inp, o_bits, lse, lens, ref = fp16_case(w)

    def bshd(bits):
        return to_half(np.ascontiguousarray(np.swapaxes(bits, 1, 2))).transpose(1, 2)

    q, k, v, o, do = (bshd(x) for x in (inp.q, inp.k, inp.v, o_bits, inp.do))
    outs = [torch.full((x.shape[0], x.shape[2], x.shape[1], x.shape[3]), float("nan"),
                       dtype=torch.float16, device="cuda").transpose(1, 2) for x in (q, k, v)]
    assert not q.is_contiguous()
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, w.causal, w.window_left,
                           det, tl is not None)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_ex(q, k, v, o, do, torch.from_numpy(lse).to("cuda"), *outs,
                    scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
                    deterministic=det, seq_q_lens=tl, seq_kv_lens=tl, workspace=ws)
    torch.cuda.synchronize()
    for tname, g, r in zip(("dQ", "dK", "dV"), outs, ref):
        C.assert_close(f"fp16 bshd {tname}", g.float().cpu().numpy(), r, tol=FP16_TOL)
