"""Helpers shared by the parity tests: case construction (synthetic inputs + oracle forward),
GPU invocation through the C ABI binding, and the tolerance check.

The oracle supplies O and LSE (its fp64 forward, rounded to bf16 / fp32) and the expected
gradients (its fp64 backward fed exactly the tensors the GPU receives).  Nothing expected ever
comes from the GPU path.
"""
import time

import numpy as np

import oracle
from attention_backward_sdpa_amd import synth

# parity tolerance: max |err| <= 1e-2 * max |ref|, per tensor
REL_TOL = 1e-2

_CACHE = {}


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def make_case(w: synth.Workload, seed=None):
    """Inputs of workload w: bf16 bit patterns of q, k, v, do, o, fp32 lse and optional lengths."""
    key = (w, seed)
    if key in _CACHE:
        return _CACHE[key]
    inp = synth.draw_inputs(w, seed)
    qf, kf, vf = (synth.bf16_to_f32(x).astype(np.float64) for x in (inp.q, inp.k, inp.v))
    lens = None if inp.seq_q_lens is None else [int(x) for x in inp.seq_q_lens]
    o64, lse64 = oracle.forward(qf, kf, vf, w.softmax_scale, causal=w.causal,
                                window_left=w.window_left, seq_q_lens=lens, seq_kv_lens=lens)
    case = dict(w=w, q=inp.q, k=inp.k, v=inp.v, do=inp.do,
                o=synth.bf16_bits(o64.astype(np.float32)), lse=lse64.astype(np.float32),
                lens=None if lens is None else np.asarray(lens, dtype=np.int32))
    if len(_CACHE) > 8:
        _CACHE.clear()
    _CACHE[key] = case
    return case


def f64(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def oracle_kwargs(case):
    w = case["w"]
    lens = None if case["lens"] is None else [int(x) for x in case["lens"]]
    return dict(causal=w.causal, window_left=w.window_left, seq_q_lens=lens, seq_kv_lens=lens)


def oracle_backward(case):
    """Full fp64 backward on exactly the GPU's inputs (bf16 q/k/v/o/do, fp32 lse)."""
    w = case["w"]
    return oracle.backward(f64(case["q"]), f64(case["k"]), f64(case["v"]), f64(case["o"]),
                           f64(case["do"]), case["lse"].astype(np.float64), w.softmax_scale,
                           **oracle_kwargs(case))


def to_device(case, torch):
    dev = "cuda"

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    t = dict(q=bf(case["q"]), k=bf(case["k"]), v=bf(case["v"]), o=bf(case["o"]),
             do=bf(case["do"]), lse=torch.from_numpy(case["lse"]).to(dev))
    t["lens"] = None if case["lens"] is None else torch.from_numpy(case["lens"]).to(dev)
    return t


def bf16_tensor_to_f32(t):
    return synth.bf16_to_f32(t.detach().cpu().view(dtypes_int16(t)).numpy().view(np.uint16))


def dtypes_int16(t):
    import torch
    return torch.int16


def run_gpu(case, torch, deterministic=None, stream=None, poison=True, ws_fill=None, dev_inputs=None):
    """Run sdpa_bwd_ex on the case; returns (dq, dk, dv) as float32 numpy arrays."""
    import attention_backward_sdpa_amd as lib
    w = case["w"]
    det = w.deterministic if deterministic is None else deterministic
    t = dev_inputs if dev_inputs is not None else to_device(case, torch)
    dq = torch.empty_like(t["q"])
    dk = torch.empty_like(t["k"])
    dv = torch.empty_like(t["v"])
    if poison:  # bf16 NaN everywhere: every element must be overwritten
        for x in (dq, dk, dv):
            x.view(torch.int16).fill_(0x7FC0)
    n = lib.workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.Dqk, w.Dv, w.causal, w.window_left,
                           det, t["lens"] is not None)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    if ws_fill is not None:
        ws.copy_(ws_fill(ws.numel()))
    if stream is not None:
        # the inputs, the NaN poison and the workspace fill were enqueued on the current stream
        stream.wait_stream(torch.cuda.current_stream())
        for x in (ws, dq, dk, dv):
            x.record_stream(stream)
    lib.sdpa_bwd_ex(t["q"], t["k"], t["v"], t["o"], t["do"], t["lse"], dq, dk, dv,
                    scale=w.softmax_scale, causal=w.causal, window_left=w.window_left,
                    deterministic=det, seq_q_lens=t["lens"], seq_kv_lens=t["lens"],
                    workspace=ws, stream=stream)
    torch.cuda.synchronize()
    return tuple(bf16_tensor_to_f32(x) for x in (dq, dk, dv))


def max_rel_err(got, ref):
    denom = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got.astype(np.float64) - ref)))
    return err / denom if denom > 0 else err


def assert_close(name, got, ref, tol=REL_TOL):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values in GPU output"
    r = max_rel_err(got, ref)
    log(f"{name}: max|err|/max|ref| = {r:.3e}")
    assert r <= tol, f"{name}: max|err|/max|ref| = {r:.3e} > {tol}"
