"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

The whole chain runs on the GPU at full size; the fp64 oracle then recomputes sampled rows one by
one (dQ rows and dK/dV key rows, including tile edges and padding boundaries) from exactly the
inputs the GPU received, and the parity tolerance max|err| <= 1e-2 * max|ref| is applied per
tensor over the samples.  Properties that hold at any size are checked on the full outputs: the
column sums of dV equal the summed dO of the rows that see a key (sum_j P_ij = 1), the column
sums of dK vanish (sum_j dS_ij = 0), padded rows are exactly zero, and the deterministic route is
bitwise identical over 10 runs.

O and LSE are the workloads' own inputs: the fp64 oracle forward on the drawn Q, K, V (and
lengths), rounded to bf16 / fp32, as for the reduced sizes.  Both the GPU path and the oracle
backward consume exactly these tensors.
"""
import hashlib

import numpy as np
import pytest

import oracle
from attention_backward_sdpa_amd import synth

from tests import _common as C

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu]

W = synth.WORKLOADS

# (workload, dQ route): None = the workload's own route, else the `deterministic` argument
# (0 fp32 atomics, 2 dS panels, 3 dQ partials)
CASES = [
    ("mha_causal_s2048_d128", None),
    ("mha_causal_s2048_d128", 3),
    ("gqa_causal_s4096_d128", 0),
    ("gqa_causal_s4096_d128", 2),
    ("gqa_causal_s4096_d128", 3),
    ("mha_det_s8192_d256", None),
    ("mla_window_padded_s4096", None),
    ("mla_window_padded_s4096", 3),
    ("gqa_causal_s4096_d128", 4),
    ("mha_det_s8192_d256", 4),
    ("mla_window_padded_s4096", 4),
    ("gqa_causal_s4096_d128_1of8", 0),
    ("gqa_causal_s4096_d128_1of8", 2),
    ("gqa_causal_s4096_d128_1of8", 3),
    ("gqa_causal_s4096_d128_1of8", 4),
]
ROUTE_NAMES = {0: "atomic", 1: "det", 2: "dspanels", 3: "dqpartials", 4: "relay", None: "default"}


def _prepare(w):
    C.log(f"full-size case {w.name}: drawing inputs")
    inp = synth.draw_inputs(w)
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    t = dict(q=bf(inp.q), k=bf(inp.k), v=bf(inp.v), do=bf(inp.do))
    lens = inp.seq_q_lens
    lens_l = None if lens is None else [int(x) for x in lens]
    C.log(f"full-size case {w.name}: fp64 oracle forward for O and LSE")
    o64, lse64 = oracle.forward(_f64(inp.q), _f64(inp.k), _f64(inp.v), w.softmax_scale,
                                causal=w.causal, window_left=w.window_left, seq_q_lens=lens_l,
                                seq_kv_lens=lens_l)
    o_bits = synth.bf16_bits(o64.astype(np.float32))
    lse = lse64.astype(np.float32)
    del o64, lse64
    t["o"], t["lse"] = bf(o_bits), torch.from_numpy(lse).to(dev)
    t["lens"] = None if lens is None else torch.from_numpy(lens).to(dev)
    torch.cuda.synchronize()
    C.log(f"full-size case {w.name}: inputs ready")
    host = dict(q=inp.q, k=inp.k, v=inp.v, do=inp.do, o=o_bits, lse=lse, lens=lens)
    return t, host


_PREP = {}


def prepared(name):
    if name not in _PREP:
        _PREP.clear()
        _PREP[name] = _prepare(W[name])
    return _PREP[name]


def _run(w, t, det):
    case = dict(w=w, lens=t["lens"])
    C.log(f"full-size case {w.name}: GPU chain (deterministic={det})")
    return C.run_gpu(case, torch, deterministic=det, dev_inputs=t)


def _edge_rows(S, L=None):
    rows = {0, 1, 31, 32, 33, 127, 128, 255, 256, 257, S // 2, S - 33, S - 32, S - 1}
    if L is not None:
        rows |= {L - 33, L - 1, L, L + 1}
    return sorted(r for r in rows if 0 <= r < S)


def _f64(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("name,det", CASES, ids=[f"{n}-{ROUTE_NAMES[d]}" for n, d in CASES])
def test_fullsize_sampled_rows(name, det):
    w = W[name]
    det = w.deterministic if det is None else det
    t, host = prepared(name)
    dq, dk, dv = _run(w, t, det)
    lens = host["lens"]
    lens_l = None if lens is None else [int(x) for x in lens]
    kw = dict(causal=w.causal, window_left=w.window_left, seq_q_lens=lens_l, seq_kv_lens=lens_l)
    q, k, v, o, do = (_f64(host[x]) for x in ("q", "k", "v", "o", "do"))
    lse = host["lse"].astype(np.float64)
    rng = np.random.default_rng(1234)
    # dQ rows
    got_q, ref_q = [], []
    heads = sorted({(0, 0), (w.B - 1, w.Hq - 1), (int(rng.integers(w.B)), int(rng.integers(w.Hq)))})
    for b, h in heads:
        L = None if lens is None else int(lens[b])
        rows = _edge_rows(w.Sq, L) + sorted(rng.choice(w.Sq, 4, replace=False).tolist())
        ref_q.append(oracle.backward_dq_rows(q, k, v, o, do, lse, w.softmax_scale, b, h, rows, **kw))
        got_q.append(dq[b, h, rows])
    # dK / dV key rows (summed over the query heads of the group)
    got_k, ref_k, got_v, ref_v = [], [], [], []
    kvheads = sorted({(0, 0), (w.B - 1, w.Hkv - 1)})
    for b, kh in kvheads:
        L = None if lens is None else int(lens[b])
        rows = _edge_rows(w.Skv, L) + sorted(rng.choice(w.Skv, 4, replace=False).tolist())
        rk, rv = oracle.backward_dkdv_rows(q, k, v, o, do, lse, w.softmax_scale, b, kh, rows, **kw)
        ref_k.append(rk)
        ref_v.append(rv)
        got_k.append(dk[b, kh, rows])
        got_v.append(dv[b, kh, rows])
    tag = f"{name} (dQ route {ROUTE_NAMES[int(det)]})"
    C.assert_close(f"{tag} dQ sampled rows", np.concatenate(got_q), np.concatenate(ref_q))
    C.assert_close(f"{tag} dK sampled rows", np.concatenate(got_k), np.concatenate(ref_k))
    C.assert_close(f"{tag} dV sampled rows", np.concatenate(got_v), np.concatenate(ref_v))

    # properties over the full outputs
    group = w.Hq // w.Hkv
    for b in range(w.B):
        L = w.Sq if lens is None else int(lens[b])
        vis = oracle.visible_mask(w.Sq, w.Skv, w.causal, w.window_left, L, L)
        has_key = vis.any(axis=1)
        for kh in range(w.Hkv):
            hs = slice(kh * group, (kh + 1) * group)
            lhs = dv[b, kh].astype(np.float64).sum(axis=0)
            rhs = do[b, hs][:, has_key].sum(axis=(0, 1))
            scale = max(float(np.abs(rhs).max()), float(np.abs(dv[b, kh]).max()))
            assert np.abs(lhs - rhs).max() <= 1e-2 * scale, f"{tag}: sum_j dV != sum_i dO (b={b})"
            colsum = np.abs(dk[b, kh].astype(np.float64).sum(axis=0)).max()
            assert colsum <= 1e-2 * np.abs(dk[b, kh]).astype(np.float64).sum(axis=0).max(), \
                f"{tag}: sum_j dK != 0 (b={b})"
        if lens is not None:
            assert np.all(dq[b, :, L:] == 0), f"{tag}: dQ rows past seq_q must be zero"
            assert np.all(dk[b, :, L:] == 0) and np.all(dv[b, :, L:] == 0)


@pytest.mark.parametrize("name,det", [("mha_det_s8192_d256", True), ("gqa_causal_s4096_d128", 3),
                                      ("gqa_causal_s4096_d128", 4)],
                         ids=["mha_det_s8192_d256-det", "gqa_causal_s4096_d128-dqpartials",
                              "gqa_causal_s4096_d128-relay"])
def test_fullsize_deterministic_bitwise(name, det):
    # 10 runs of a deterministic route at full size, identical bits
    w = W[name]
    t, _ = prepared(name)
    digests = set()
    for run in range(10):
        out = _run(w, t, det)
        h = hashlib.sha256()
        for x in out:
            h.update(np.ascontiguousarray(x).view(np.uint32).tobytes())
        digests.add(h.hexdigest())
    assert len(digests) == 1, f"{len(digests)} distinct results over 10 runs"


# The additive bias at the headline's full size (causal GQA B=1 Hq=32 Hkv=8 S=4096 D=128): a
# per-batch bf16 bias drawn N(0, 1) with its fp32 gradient ("API Usage" bias_tensor), on the fp32
# atomic and dS-panel routes (the 8-wave kernels with the bias tile staged in LDS).  O and LSE come
# from the fp64 oracle forward with that bias.  Sampled dQ rows, their dBias rows and dK/dV key
# rows against the oracle; over whole heads: dBias exactly 0 on masked pairs, and every dBias row
# sums to about 0 (sum_j dS_ij = sum_j P_ij dP_ij - delta_i, with sum_j P_ij = 1).
_BIAS_PREP = {}


def _prepare_bias():
    if "c3" not in _BIAS_PREP:
        w = W["gqa_causal_s4096_d128"]
        t, host = prepared("gqa_causal_s4096_d128")
        C.log("full-size bias case: drawing the bias")
        rng = np.random.default_rng(77)
        bias_bits = synth.bf16_bits(rng.standard_normal((w.B, w.Hq, w.Sq, w.Skv), dtype=np.float32))
        bias32 = synth.bf16_to_f32(bias_bits)
        C.log("full-size bias case: fp64 oracle forward with the bias")
        o64, lse64 = oracle.forward(_f64(host["q"]), _f64(host["k"]), _f64(host["v"]),
                                    w.softmax_scale, causal=True, bias=bias32)
        o_bits = synth.bf16_bits(o64.astype(np.float32))
        lse = lse64.astype(np.float32)
        del o64, lse64
        dev = torch.device("cuda:0")
        tb = dict(t)
        tb["o"] = torch.from_numpy(o_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        tb["lse"] = torch.from_numpy(lse).to(dev)
        tb["bias"] = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        hb = dict(host, o=o_bits, lse=lse, bias=bias32)
        torch.cuda.synchronize()
        C.log("full-size bias case: inputs ready")
        _BIAS_PREP["c3"] = (tb, hb)
    return _BIAS_PREP["c3"]


@pytest.mark.parametrize("det", [0, 2], ids=["atomic", "dspanels"])
def test_fullsize_bias_sampled_rows(det):
    import attention_backward_sdpa_amd as lib
    w = W["gqa_causal_s4096_d128"]
    t, host = _prepare_bias()
    C.log(f"full-size bias case: GPU chain (deterministic={det})")
    outs = [torch.empty_like(t[x]) for x in ("q", "k", "v")]
    for x in outs:
        x.view(torch.int16).fill_(0x7FC0)
    dbias = torch.full(tuple(t["bias"].shape), float("nan"), device="cuda")
    kw = dict(scale=w.softmax_scale, causal=True, deterministic=det, bias=t["bias"], dbias=dbias)
    n = lib.run_workspace_size(t["q"], t["k"], t["v"], **kw)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_run(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], *outs, workspace=ws, **kw)
    torch.cuda.synchronize()
    dq, dk, dv = (C.bf16_tensor_to_f32(x) for x in outs)
    heads = [0, 13, w.Hq - 1]
    db = {h: dbias[0, h].cpu().numpy() for h in heads}
    del dbias, ws
    q, k, v, o, do = (_f64(host[x]) for x in ("q", "k", "v", "o", "do"))
    lse = host["lse"].astype(np.float64)
    okw = dict(causal=True, bias=host["bias"])
    rng = np.random.default_rng(4321)
    got_q, ref_q, got_b, ref_b = [], [], [], []
    for h in heads:
        rows = _edge_rows(w.Sq) + sorted(rng.choice(w.Sq, 4, replace=False).tolist())
        r, ds = oracle.backward_dq_rows(q, k, v, o, do, lse, w.softmax_scale, 0, h, rows,
                                        return_ds=True, **okw)
        ref_q.append(r)
        got_q.append(dq[0, h, rows])
        ref_b.append(ds)
        got_b.append(db[h][rows])
    got_k, ref_k, got_v, ref_v = [], [], [], []
    for kh in (0, w.Hkv - 1):
        rows = _edge_rows(w.Skv) + sorted(rng.choice(w.Skv, 4, replace=False).tolist())
        rk, rv = oracle.backward_dkdv_rows(q, k, v, o, do, lse, w.softmax_scale, 0, kh, rows, **okw)
        ref_k.append(rk)
        ref_v.append(rv)
        got_k.append(dk[0, kh, rows])
        got_v.append(dv[0, kh, rows])
    tag = f"full-size bias (dQ route {ROUTE_NAMES[det]})"
    C.assert_close(f"{tag} dQ sampled rows", np.concatenate(got_q), np.concatenate(ref_q))
    C.assert_close(f"{tag} dBias sampled rows", np.concatenate(got_b), np.concatenate(ref_b))
    C.assert_close(f"{tag} dK sampled rows", np.concatenate(got_k), np.concatenate(ref_k))
    C.assert_close(f"{tag} dV sampled rows", np.concatenate(got_v), np.concatenate(ref_v))
    vis = oracle.visible_mask(w.Sq, w.Skv, True)
    for h in heads:
        assert np.all(db[h][~vis] == 0), f"{tag}: dBias on masked pairs must be zero (head {h})"
        rowsum = np.abs(db[h].astype(np.float64).sum(axis=1)).max()
        assert rowsum <= 1e-2 * np.abs(db[h]).astype(np.float64).sum(axis=1).max(), \
            f"{tag}: dBias rows do not sum to 0 (head {h})"


# fp16 io at the headline's full size ("Support surface": FP16 / BF16): the inputs drawn as for
# bf16 but rounded to binary16, O and LSE from the fp64 oracle forward rounded to fp16 / fp32, on
# the fp32-atomic and dS-panel routes.  Sampled rows against the oracle at the fp16 tolerance
# (4 unit roundoffs of binary16, as in tests/test_fp16_gpu.py), and the column-sum identities.
FP16_TOL = 2e-3
_FP16_PREP = {}


def _prepare_fp16():
    if "c3" not in _FP16_PREP:
        w = W["gqa_causal_s4096_d128"]
        C.log("full-size fp16 case: drawing inputs")
        inp = synth.draw_inputs(w, dtype="fp16")
        f = lambda bits: synth.fp16_to_f32(bits).astype(np.float64)
        C.log("full-size fp16 case: fp64 oracle forward for O and LSE")
        o64, lse64 = oracle.forward(f(inp.q), f(inp.k), f(inp.v), w.softmax_scale, causal=True)
        o_bits = synth.fp16_bits(o64.astype(np.float32))
        lse = lse64.astype(np.float32)
        del o64, lse64
        h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.float16).cuda()
        t = dict(q=h(inp.q), k=h(inp.k), v=h(inp.v), do=h(inp.do), o=h(o_bits),
                 lse=torch.from_numpy(lse).cuda())
        host = dict(q=f(inp.q), k=f(inp.k), v=f(inp.v), do=f(inp.do), o=f(o_bits),
                    lse=lse.astype(np.float64))
        torch.cuda.synchronize()
        C.log("full-size fp16 case: inputs ready")
        _FP16_PREP["c3"] = (t, host)
    return _FP16_PREP["c3"]


@pytest.mark.parametrize("det", [0, 2], ids=["atomic", "dspanels"])
def test_fullsize_fp16_sampled_rows(det):
    import attention_backward_sdpa_amd as lib
    w = W["gqa_causal_s4096_d128"]
    t, host = _prepare_fp16()
    C.log(f"full-size fp16 case: GPU chain (deterministic={det})")
    outs = [torch.empty_like(t[x]) for x in ("q", "k", "v")]
    for x in outs:
        x.view(torch.int16).fill_(0x7E00)  # fp16 NaN: every element must be written
    n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, True, -1, det, False)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lib.sdpa_bwd_ex(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], *outs,
                    scale=w.softmax_scale, causal=True, deterministic=det, workspace=ws)
    torch.cuda.synchronize()
    dq, dk, dv = (x.float().cpu().numpy() for x in outs)
    q, k, v, o, do, lse = (host[x] for x in ("q", "k", "v", "o", "do", "lse"))
    rng = np.random.default_rng(99)
    got_q, ref_q = [], []
    for h in (0, 17, w.Hq - 1):
        rows = _edge_rows(w.Sq) + sorted(rng.choice(w.Sq, 4, replace=False).tolist())
        ref_q.append(oracle.backward_dq_rows(q, k, v, o, do, lse, w.softmax_scale, 0, h, rows, causal=True))
        got_q.append(dq[0, h, rows])
    got_k, ref_k, got_v, ref_v = [], [], [], []
    for kh in (0, w.Hkv - 1):
        rows = _edge_rows(w.Skv) + sorted(rng.choice(w.Skv, 4, replace=False).tolist())
        rk, rv = oracle.backward_dkdv_rows(q, k, v, o, do, lse, w.softmax_scale, 0, kh, rows, causal=True)
        ref_k.append(rk)
        ref_v.append(rv)
        got_k.append(dk[0, kh, rows])
        got_v.append(dv[0, kh, rows])
    tag = f"full-size fp16 (dQ route {ROUTE_NAMES[det]})"
    C.assert_close(f"{tag} dQ sampled rows", np.concatenate(got_q), np.concatenate(ref_q), tol=FP16_TOL)
    C.assert_close(f"{tag} dK sampled rows", np.concatenate(got_k), np.concatenate(ref_k), tol=FP16_TOL)
    C.assert_close(f"{tag} dV sampled rows", np.concatenate(got_v), np.concatenate(ref_v), tol=FP16_TOL)
    group = w.Hq // w.Hkv
    for kh in range(w.Hkv):
        hs = slice(kh * group, (kh + 1) * group)
        lhs = dv[0, kh].astype(np.float64).sum(axis=0)
        rhs = do[0, hs].sum(axis=(0, 1))
        scale = max(float(np.abs(rhs).max()), float(np.abs(dv[0, kh]).max()))
        assert np.abs(lhs - rhs).max() <= 1e-2 * scale, f"{tag}: sum_j dV != sum_i dO (kv head {kh})"
        colsum = np.abs(dk[0, kh].astype(np.float64).sum(axis=0)).max()
        assert colsum <= 1e-2 * np.abs(dk[0, kh]).astype(np.float64).sum(axis=0).max(), \
            f"{tag}: sum_j dK != 0 (kv head {kh})"
