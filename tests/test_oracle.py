"""Pins of the fp64 CPU oracle against things other than itself.

* a hand-written mask fixture (tests/golden/masks_6x6.txt) derived from the pages' mask rules;
* torch's CPU scaled_dot_product_attention in float64 (a library routine) for the forward, and its
  autograd for the backward;
* scipy's logsumexp for the natural-log LSE;
* central finite differences of L = sum(dO * O(Q, K, V)) on tiny shapes, every mask combination;
* invariants: rows of dS sum to 0, sum over keys of dV equals the sum of dO over rows that see a
  key, sum over keys of dK is 0;
* closed forms: one key, a zero-width causal window, Q = 0;
* structure: GQA equals MHA on repeated K/V with group-summed dK/dV, padding equals the unpadded
  per-batch slice, linearity in dO;
* the row-sampled functions equal the full backward;
* mutation checks: deliberately broken backwards (planted here, on the CPU) fail the same checks;
* sink tokens: finite differences in the sink logits and in Q, K, V with the sink folded into the
  forward, a one-key closed form, the -inf limit (no sink) and the row sums of dS;
* additive bias: finite differences in every bias element (per-batch and batch-1 biases, whose
  gradient sums over the batch) and in Q, K, V, row-shift invariance, a causal mask written as a
  bias, zero bias = no bias, and planted dBias mistakes.
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import sdpa_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "masks_6x6.txt")


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


def _problem(seed, B=1, Hq=2, Hkv=2, Sq=7, Skv=7, Dqk=8, Dv=8, causal=False, W=-1, lens=None,
             br=False, R=0):
    rng = np.random.default_rng(seed)
    q = _rand(rng, B, Hq, Sq, Dqk)
    k = _rand(rng, B, Hkv, Skv, Dqk)
    v = _rand(rng, B, Hkv, Skv, Dv)
    do = _rand(rng, B, Hq, Sq, Dv)
    scale = 1.0 / math.sqrt(Dqk)
    kw = dict(causal=causal, window_left=W, seq_q_lens=lens, seq_kv_lens=lens, bottom_right=br,
              window_right=R)
    o, lse = oracle.forward(q, k, v, scale, **kw)
    return q, k, v, do, o, lse, scale, kw


MASKS = [
    dict(causal=False, W=-1),
    dict(causal=True, W=-1),
    dict(causal=True, W=2),
    dict(causal=False, W=2),
    dict(causal=True, W=0),
    dict(causal=True, W=-1, lens=[5]),
    dict(causal=True, W=1, lens=[4]),
    dict(causal=True, W=-1, br=True),
    dict(causal=True, W=-1, R=1),
]


# ----------------------------------------------------------------------------------------------
# mask semantics against the hand-written fixture
def _read_golden():
    cases = []
    with open(GOLDEN) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    i = 0
    while i < len(lines):
        parts = lines[i].split()
        assert parts[0] == "case"
        name = parts[1]
        Sq, Skv, causal, W, lq, lkv, br, R = map(int, parts[2:])
        rows = lines[i + 1:i + 1 + Sq]
        mask = np.array([[c == "1" for c in r] for r in rows])
        assert mask.shape == (Sq, Skv)
        cases.append((name, Sq, Skv, causal, W, lq, lkv, br, R, mask))
        i += 1 + Sq
    return cases


@pytest.mark.parametrize("case", _read_golden(), ids=lambda c: c[0])
def test_visible_mask_matches_golden(case):
    name, Sq, Skv, causal, W, lq, lkv, br, R, mask = case
    got = oracle.visible_mask(Sq, Skv, bool(causal), W, lq, lkv, bool(br), R)
    np.testing.assert_array_equal(got, mask, err_msg=name)


# ----------------------------------------------------------------------------------------------
# forward against torch's CPU SDPA and scipy's logsumexp
def _torch_reference(q, k, v, do, scale, kw, need_grad=True):
    """O and (optionally) dQ/dK/dV from torch's float64 CPU SDPA with an explicit boolean mask.

    Rows that see no key are given one dummy visible key and their output is multiplied by 0, so
    they contribute exactly nothing (torch would otherwise produce NaN for an all-masked row).
    """
    B, Hq, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    lens = kw["seq_q_lens"]
    masks = []
    for b in range(B):
        L = None if lens is None else lens[b]
        masks.append(oracle.visible_mask(Sq, Skv, kw["causal"], kw["window_left"], L, L,
                                         kw["bottom_right"], kw["window_right"]))
    vis = torch.tensor(np.stack(masks))[:, None]                 # (B,1,Sq,Skv)
    rows = vis.any(dim=-1, keepdim=True)                          # (B,1,Sq,1)
    safe = vis | (~rows & (torch.arange(Skv) == 0))
    tq = torch.tensor(q, requires_grad=need_grad)
    tk = torch.tensor(k, requires_grad=need_grad)
    tv = torch.tensor(v, requires_grad=need_grad)
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=safe, scale=scale, enable_gqa=(Hq != Hkv))
    out = out * rows
    if not need_grad:
        return out.detach().numpy()
    out.backward(torch.tensor(do))
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("mask", MASKS, ids=str)
@pytest.mark.parametrize("heads", [(2, 2), (4, 2), (4, 1)], ids=str)
def test_forward_matches_torch_sdpa(mask, heads):
    q, k, v, do, o, lse, scale, kw = _problem(11, Hq=heads[0], Hkv=heads[1], Sq=9, Skv=9,
                                              Dqk=8, Dv=6, **mask)
    ref = _torch_reference(q, k, v, do, scale, kw, need_grad=False)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mask", MASKS, ids=str)
def test_lse_is_natural_log_logsumexp(mask):
    q, k, v, do, o, lse, scale, kw = _problem(12, Hq=2, Hkv=1, Sq=9, Skv=9, **mask)
    lens = kw["seq_q_lens"]
    for h in range(2):
        vis = oracle.visible_mask(9, 9, kw["causal"], kw["window_left"],
                                  None if lens is None else lens[0],
                                  None if lens is None else lens[0], kw["bottom_right"],
                                  kw["window_right"])
        s = scale * q[0, h] @ k[0, 0].T
        s = np.where(vis, s, -np.inf)
        ref = logsumexp(s, axis=1)
        np.testing.assert_allclose(lse[0, h], ref, rtol=1e-13, atol=1e-13)
        # e-base statistic: the visible probabilities of every non-empty row sum to one
        p = np.where(vis, np.exp(s - np.where(np.isfinite(ref), ref, 0)[:, None]), 0)
        nonempty = vis.any(axis=1)
        np.testing.assert_allclose(p.sum(axis=1)[nonempty], 1.0, rtol=1e-13)


# ----------------------------------------------------------------------------------------------
# backward against torch autograd and finite differences
@pytest.mark.parametrize("mask", MASKS, ids=str)
@pytest.mark.parametrize("heads", [(2, 2), (4, 2), (3, 1)], ids=str)
def test_backward_matches_torch_autograd(mask, heads):
    q, k, v, do, o, lse, scale, kw = _problem(13, B=1, Hq=heads[0], Hkv=heads[1], Sq=9, Skv=9,
                                              Dqk=8, Dv=6, **mask)
    _, gq, gk, gv = _torch_reference(q, k, v, do, scale, kw)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    np.testing.assert_allclose(dq, gq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, gk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, gv, rtol=1e-10, atol=1e-12)


def _fd_check(backward_fn, q, k, v, do, scale, kw, h=1e-6):
    """Max relative error of backward_fn's gradients against central differences of sum(dO*O)."""
    o, lse = oracle.forward(q, k, v, scale, **kw)
    grads = backward_fn(q, k, v, o, do, lse, scale, **kw)
    worst = 0.0
    for idx, x in enumerate((q, k, v)):
        g = grads[idx]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            old = x[mi]
            x[mi] = old + h
            lp = np.sum(do * oracle.forward(q, k, v, scale, **kw)[0])
            x[mi] = old - h
            lm = np.sum(do * oracle.forward(q, k, v, scale, **kw)[0])
            x[mi] = old
            fd[mi] = (lp - lm) / (2 * h)
        denom = max(np.max(np.abs(fd)), 1e-2)  # an all-zero gradient is judged absolutely
        worst = max(worst, float(np.max(np.abs(g - fd)) / denom))
    return worst


@pytest.mark.parametrize("mask", MASKS, ids=str)
@pytest.mark.parametrize("shape", [(1, 2, 2, 5, 4), (1, 4, 2, 7, 8), (2, 2, 1, 6, 4)], ids=str)
def test_backward_finite_differences(mask, shape):
    B, Hq, Hkv, S, D = shape
    if mask.get("lens") is not None:
        mask = dict(mask, lens=[min(mask["lens"][0], S)] * B)
    q, k, v, do, o, lse, scale, kw = _problem(14, B=B, Hq=Hq, Hkv=Hkv, Sq=S, Skv=S, Dqk=D, Dv=D,
                                              **mask)
    err = _fd_check(oracle.backward, q, k, v, do, scale, kw)
    assert err < 1e-6, err


# ----------------------------------------------------------------------------------------------
# invariants (self-consistent inputs: the exact fp64 O and LSE of the forward)
@pytest.mark.parametrize("mask", MASKS, ids=str)
def test_invariants(mask):
    q, k, v, do, o, lse, scale, kw = _problem(15, B=1, Hq=4, Hkv=2, Sq=9, Skv=9, **mask)
    dq, dk, dv, delta, ds = oracle.backward(q, k, v, o, do, lse, scale, return_intermediates=True,
                                            **kw)
    # each row of dS sums to zero
    np.testing.assert_allclose(ds.sum(axis=-1), 0.0, atol=1e-12)
    # sum over keys of dV = sum over query rows that see a key of dO, summed over the group
    lens = kw["seq_q_lens"]
    L = None if lens is None else lens[0]
    vis = oracle.visible_mask(9, 9, kw["causal"], kw["window_left"], L, L, kw["bottom_right"],
                              kw["window_right"])
    rows = vis.any(axis=1)
    for kvh in range(2):
        ref = sum(do[0, h][rows].sum(axis=0) for h in (2 * kvh, 2 * kvh + 1))
        np.testing.assert_allclose(dv[0, kvh].sum(axis=0), ref, atol=1e-12)
    # sum over keys of dK is zero (it is scale * sum_i (sum_j dS_ij) Q_i)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# closed forms
def test_single_key():
    q, k, v, do, o, lse, scale, kw = _problem(16, B=1, Hq=4, Hkv=2, Sq=5, Skv=1)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    for kvh in range(2):
        np.testing.assert_allclose(dv[0, kvh, 0], do[0, 2 * kvh:2 * kvh + 2].sum(axis=(0, 1)),
                                   atol=1e-12)


def test_zero_width_causal_window_is_diagonal():
    q, k, v, do, o, lse, scale, kw = _problem(17, B=1, Hq=2, Hkv=2, Sq=8, Skv=8, causal=True, W=0)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv, do, atol=1e-14)
    np.testing.assert_allclose(o, v, atol=1e-14)


def test_zero_queries_give_uniform_attention():
    rng = np.random.default_rng(18)
    Sq, Skv, D = 6, 5, 4
    q = np.zeros((1, 1, Sq, D))
    k = rng.standard_normal((1, 1, Skv, D))
    v = rng.standard_normal((1, 1, Skv, D))
    do = rng.standard_normal((1, 1, Sq, D))
    scale = 0.5
    o, lse = oracle.forward(q, k, v, scale)
    np.testing.assert_allclose(o[0, 0], np.tile(v[0, 0].mean(axis=0), (Sq, 1)), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(Skv), atol=1e-14)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv[0, 0], np.tile(do[0, 0].sum(axis=0) / Skv, (Skv, 1)), atol=1e-13)
    vbar = v[0, 0].mean(axis=0)
    kmat = k[0, 0].T @ (v[0, 0] - vbar)           # sum_j K_j (V_j - Vbar)^T
    np.testing.assert_allclose(dq[0, 0], scale / Skv * (do[0, 0] @ kmat.T), atol=1e-13)


# ----------------------------------------------------------------------------------------------
# structural identities
def test_gqa_equals_repeated_mha():
    q, k, v, do, o, lse, scale, kw = _problem(19, B=2, Hq=6, Hkv=2, Sq=7, Skv=7, causal=True, W=3)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    o2, lse2 = oracle.forward(q, kr, vr, scale, **kw)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    dq2, dk2, dv2 = oracle.backward(q, kr, vr, o2, do, lse2, scale, **kw)
    np.testing.assert_allclose(dq2, dq, atol=1e-13)
    np.testing.assert_allclose(dk2.reshape(2, 2, 3, 7, 8).sum(axis=2), dk, atol=1e-13)
    np.testing.assert_allclose(dv2.reshape(2, 2, 3, 7, 8).sum(axis=2), dv, atol=1e-13)


def test_padding_equals_unpadded_slice():
    lens = [5, 9]
    q, k, v, do, o, lse, scale, kw = _problem(20, B=2, Hq=2, Hkv=1, Sq=9, Skv=9, causal=True,
                                              W=2, lens=lens)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    for b, L in enumerate(lens):
        ob, lb = oracle.forward(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L], scale,
                                causal=True, window_left=2)
        np.testing.assert_allclose(o[b, :, :L], ob[0], atol=1e-14)
        assert np.all(o[b, :, L:] == 0) and np.all(np.isneginf(lse[b, :, L:]))
        gq, gk, gv = oracle.backward(q[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L],
                                     ob, do[b:b + 1, :, :L], lb, scale, causal=True, window_left=2)
        np.testing.assert_allclose(dq[b, :, :L], gq[0], atol=1e-13)
        np.testing.assert_allclose(dk[b, :, :L], gk[0], atol=1e-13)
        np.testing.assert_allclose(dv[b, :, :L], gv[0], atol=1e-13)
        # rows past the length are exactly zero
        assert np.all(dq[b, :, L:] == 0) and np.all(dk[b, :, L:] == 0) and np.all(dv[b, :, L:] == 0)


def test_linear_in_dO():
    q, k, v, do, o, lse, scale, kw = _problem(21, Hq=2, Hkv=1, causal=True)
    g1 = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    g2 = oracle.backward(q, k, v, o, 2 * do, lse, scale, **kw)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(b, 2 * a, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------------------------
# row-sampled entry points equal the full backward
@pytest.mark.parametrize("mask", MASKS, ids=str)
def test_sampled_rows_match_full(mask):
    q, k, v, do, o, lse, scale, kw = _problem(22, B=2, Hq=4, Hkv=2, Sq=9, Skv=9, **dict(
        mask, lens=None if mask.get("lens") is None else [mask["lens"][0], 9]))
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    for b in range(2):
        for h in range(4):
            r = oracle.backward_dq_rows(q, k, v, o, do, lse, scale, b, h, [0, 3, 8], **kw)
            np.testing.assert_allclose(r, dq[b, h, [0, 3, 8]], atol=1e-13)
        for kvh in range(2):
            gk, gv = oracle.backward_dkdv_rows(q, k, v, o, do, lse, scale, b, kvh, [1, 4, 8], **kw)
            np.testing.assert_allclose(gk, dk[b, kvh, [1, 4, 8]], atol=1e-13)
            np.testing.assert_allclose(gv, dv[b, kvh, [1, 4, 8]], atol=1e-13)


@pytest.mark.parametrize("bias_batch", [1, 2])
def test_sampled_rows_match_full_with_bias(bias_batch):
    # the same with an additive bias: the rows' dQ, their dS (= dBias for a per-batch bias), and
    # the key rows' dK/dV equal the full backward's
    q, k, v, do, o, lse, scale, kw = _problem(23, B=2, Hq=4, Hkv=2, Sq=9, Skv=9, causal=True,
                                              lens=[7, 9])
    bias = np.random.default_rng(5).standard_normal((bias_batch, 4, 9, 9))
    o, lse = oracle.forward(q, k, v, scale, bias=bias, **kw)
    dq, dk, dv, dbias = oracle.backward(q, k, v, o, do, lse, scale, bias=bias, return_dbias=True, **kw)
    for b in range(2):
        for h in range(4):
            r, ds = oracle.backward_dq_rows(q, k, v, o, do, lse, scale, b, h, [0, 3, 8], bias=bias,
                                            return_ds=True, **kw)
            np.testing.assert_allclose(r, dq[b, h, [0, 3, 8]], atol=1e-13)
            if bias_batch == 2:
                np.testing.assert_allclose(ds, dbias[b, h, [0, 3, 8]], atol=1e-13)
        for kvh in range(2):
            gk, gv = oracle.backward_dkdv_rows(q, k, v, o, do, lse, scale, b, kvh, [1, 4, 8],
                                               bias=bias, **kw)
            np.testing.assert_allclose(gk, dk[b, kvh, [1, 4, 8]], atol=1e-13)
            np.testing.assert_allclose(gv, dv[b, kvh, [1, 4, 8]], atol=1e-13)


# ----------------------------------------------------------------------------------------------
# FLOP convention
def test_flop_count():
    # 10 * S^2 * D per head for D_qk = D_v, halved for causal
    assert oracle.attention_flops(1, 32, 4096, 4096, 128, 128, causal=True) == 10 * 4096 ** 2 * 128 * 32 / 2
    # windowed causal rows of length L >= W see min(i, W) + 1 keys: 1025 * L - 524800 pairs for W=1024
    L = 2000
    f = oracle.attention_flops(1, 1, 4096, 4096, 192, 128, causal=True, window_left=1024,
                               seq_q_lens=[L], seq_kv_lens=[L])
    assert f == 2 * (3 * 192 + 2 * 128) * (1025 * L - 524800)


# ----------------------------------------------------------------------------------------------
# mutation checks: a plausible mistake planted in a copy of the backward fails the pins above
def _mutant(kind):
    def bwd(q, k, v, o, do, lse, scale, **kw):
        dq, dk, dv, delta, ds = oracle.backward(q, k, v, o, do, lse, scale,
                                                return_intermediates=True, **kw)
        if kind == "no_delta":      # dS = P * dP (delta term dropped)
            B, Hq = q.shape[:2]
            group = Hq // k.shape[1]
            dq2 = np.zeros_like(dq)
            for b in range(B):
                for h in range(Hq):
                    p_ds = ds[b, h] + 0  # dS = P (dP - delta) -> add back P * delta
                    vis_p = np.exp(scale * q[b, h] @ k[b, h // group].T - lse[b, h][:, None])
                    vis_p = np.where(ds[b, h] != 0, vis_p, 0)
                    p_ds = p_ds + vis_p * delta[b, h][:, None]
                    dq2[b, h] = scale * p_ds @ k[b, h // group]
            return dq2, dk, dv
        if kind == "dk_unscaled":
            return dq, dk / scale, dv
        if kind == "dv_transposed_heads":
            return dq, dk, dv[:, ::-1].copy()
        raise ValueError(kind)
    return bwd


@pytest.mark.parametrize("kind", ["no_delta", "dk_unscaled", "dv_transposed_heads"])
def test_planted_mistakes_are_caught(kind):
    q, k, v, do, o, lse, scale, kw = _problem(23, B=1, Hq=2, Hkv=2, Sq=5, Skv=5, Dqk=4, Dv=4,
                                              causal=True)
    assert _fd_check(_mutant(kind), q, k, v, do, scale, kw) > 1e-3


# ----------------------------------------------------------------------------------------------
# sink tokens ("SDPA Backward (SM120)", "The kernel chain" (dsink) and "Support surface"):
# finite differences of L = sum(dO * O(Q, K, V, sink)), a closed form, the -inf limit and the
# row-sum identity with the sink's own softmax entry
SINK_MASKS = [dict(causal=False, W=-1), dict(causal=True, W=-1), dict(causal=True, W=1, lens=[4]),
              dict(causal=True, W=-1, br=True)]


def _sink_problem(seed, mask, B=1, Hq=2, Hkv=1, S=5, D=4):
    q, k, v, do, _, _, scale, kw = _problem(seed, B=B, Hq=Hq, Hkv=Hkv, Sq=S, Skv=S, Dqk=D, Dv=D,
                                            **dict(mask, lens=None if mask.get("lens") is None
                                                   else mask["lens"] * B))
    sink = np.random.default_rng(seed + 100).standard_normal(Hq) + 0.5
    o, lse = oracle.forward(q, k, v, scale, sink=sink, **kw)
    return q, k, v, do, o, lse, scale, kw, sink


@pytest.mark.parametrize("mask", SINK_MASKS, ids=str)
def test_sink_finite_differences(mask):
    q, k, v, do, o, lse, scale, kw, sink = _sink_problem(31, mask, B=2)
    h = 1e-6
    # dsink against central differences in each sink logit
    got = oracle.dsink(o, do, lse, sink, seq_q_lens=kw["seq_q_lens"])
    for hh in range(len(sink)):
        sp, sm = sink.copy(), sink.copy()
        sp[hh] += h
        sm[hh] -= h
        lp = np.sum(do * oracle.forward(q, k, v, scale, sink=sp, **kw)[0])
        lm = np.sum(do * oracle.forward(q, k, v, scale, sink=sm, **kw)[0])
        fd = (lp - lm) / (2 * h)
        assert abs(got[hh] - fd) <= 1e-6 * max(1.0, abs(fd)), (hh, got[hh], fd)
    # dQ/dK/dV need no sink term: the backward fed the sink-folded LSE matches the differences
    grads = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    for idx, x in enumerate((q, k, v)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            old = x[mi]
            x[mi] = old + h
            lp = np.sum(do * oracle.forward(q, k, v, scale, sink=sink, **kw)[0])
            x[mi] = old - h
            lm = np.sum(do * oracle.forward(q, k, v, scale, sink=sink, **kw)[0])
            x[mi] = old
            fd[mi] = (lp - lm) / (2 * h)
        assert np.max(np.abs(grads[idx] - fd)) <= 1e-6 * max(1.0, np.max(np.abs(fd)))


def test_sink_single_key_closed_form():
    # one key per row: P_key = 1 / (1 + exp(sink - x)), x = scale q.k; O = P_key v;
    # dL/dsink = -P_key (1 - P_key) (v . dO) per row, summed over rows and batch entries
    rng = np.random.default_rng(32)
    B, Sq, D = 2, 4, 3
    q = rng.standard_normal((B, 1, Sq, D))
    k = rng.standard_normal((B, 1, 1, D))
    v = rng.standard_normal((B, 1, 1, D))
    do = rng.standard_normal((B, 1, Sq, D))
    scale, sink = 0.7, np.array([0.3])
    o, lse = oracle.forward(q, k, v, scale, sink=sink)
    x = scale * np.einsum("bqd,bd->bq", q[:, 0], k[:, 0, 0])
    p_key = 1.0 / (1.0 + np.exp(sink[0] - x))
    np.testing.assert_allclose(o[:, 0], p_key[..., None] * v[:, 0, 0][:, None, :], atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], np.logaddexp(x, sink[0]), atol=1e-14)
    vdo = np.einsum("bd,bqd->bq", v[:, 0, 0], do[:, 0])
    ref = -np.sum(p_key * (1.0 - p_key) * vdo)
    np.testing.assert_allclose(oracle.dsink(o, do, lse, sink), [ref], rtol=1e-13)


def test_sink_at_minus_infinity_is_no_sink():
    q, k, v, do, o, lse, scale, kw = _problem(33, B=1, Hq=2, Hkv=1, Sq=6, Skv=6, causal=True)
    o2, lse2 = oracle.forward(q, k, v, scale, sink=np.array([-np.inf, -np.inf]), **kw)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(lse2, lse)
    assert np.all(oracle.dsink(o, do, lse, np.array([-np.inf, -np.inf])) == 0)


@pytest.mark.parametrize("mask", SINK_MASKS, ids=str)
def test_sink_row_sums(mask):
    # with the sink in the softmax, sum_j dS_ij over the keys equals minus the sink's own entry
    # P_sink (0 - delta): sum_j dS_ij = exp(sink - LSE_i) * delta_i; every row with a sink exists
    q, k, v, do, o, lse, scale, kw, sink = _sink_problem(34, mask, B=1, Hq=2, S=7)
    dq, dk, dv, delta, ds = oracle.backward(q, k, v, o, do, lse, scale, return_intermediates=True,
                                            **kw)
    L = 7 if kw["seq_q_lens"] is None else kw["seq_q_lens"][0]
    for h in range(2):
        p_sink = np.exp(sink[h] - lse[0, h, :L])
        np.testing.assert_allclose(ds[0, h, :L].sum(axis=1), p_sink * delta[0, h, :L], atol=1e-12)
        assert np.all(np.isneginf(lse[0, h, L:]))
    np.testing.assert_allclose(oracle.dsink(o, do, lse, sink, seq_q_lens=kw["seq_q_lens"]),
                               [-np.sum(np.exp(sink[h] - lse[0, h, :L]) * delta[0, h, :L])
                                for h in range(2)], rtol=1e-13)


@pytest.mark.parametrize("kind", ["sign", "no_delta", "rows_past_len"])
def test_planted_dsink_mistakes_are_caught(kind):
    q, k, v, do, o, lse, scale, kw, sink = _sink_problem(35, dict(causal=True, W=-1, lens=[3]),
                                                         B=1, Hq=2, S=5)
    o_bad = o.copy()
    if kind == "no_delta":
        o_bad = np.ones_like(o)          # delta from the wrong O
    got = oracle.dsink(o_bad, do, lse, sink, seq_q_lens=None if kind == "rows_past_len" else
                       kw["seq_q_lens"])
    if kind == "sign":
        got = -got
    if kind == "rows_past_len":          # padded rows given a finite LSE would leak in
        lse2 = np.where(np.isfinite(lse), lse, 0.0)
        got = oracle.dsink(o + 1.0, do, lse2, sink)
    h = 1e-6
    fd = []
    for hh in range(2):
        sp, sm = sink.copy(), sink.copy()
        sp[hh] += h
        sm[hh] -= h
        fd.append((np.sum(do * oracle.forward(q, k, v, scale, sink=sp, **kw)[0]) -
                   np.sum(do * oracle.forward(q, k, v, scale, sink=sm, **kw)[0])) / (2 * h))
    assert np.max(np.abs(np.asarray(got) - np.asarray(fd))) > 1e-3


# ----------------------------------------------------------------------------------------------
# additive bias ("SDPA Backward (SM120)", "API Usage" bias_tensor and "Support surface" bias):
# finite differences in every bias element (per-batch and batch-1 biases) and in Q, K, V with the
# bias in the forward, row-shift invariance, a mask written as a bias, and zero bias = no bias
BIAS_MASKS = [dict(causal=False, W=-1), dict(causal=True, W=-1), dict(causal=True, W=1, lens=[4])]


def _bias_problem(seed, mask, B=2, Hq=2, Hkv=1, S=5, D=4, bias_batch=None):
    q, k, v, do, _, _, scale, kw = _problem(seed, B=B, Hq=Hq, Hkv=Hkv, Sq=S, Skv=S, Dqk=D, Dv=D,
                                            **dict(mask, lens=None if mask.get("lens") is None
                                                   else mask["lens"] * B))
    bias = np.random.default_rng(seed + 200).standard_normal((bias_batch or B, Hq, S, S))
    o, lse = oracle.forward(q, k, v, scale, bias=bias, **kw)
    return q, k, v, do, o, lse, scale, kw, bias


@pytest.mark.parametrize("bias_batch", [None, 1], ids=["per_batch", "batch1"])
@pytest.mark.parametrize("mask", BIAS_MASKS, ids=str)
def test_bias_finite_differences(mask, bias_batch):
    q, k, v, do, o, lse, scale, kw, bias = _bias_problem(41, mask, bias_batch=bias_batch)
    dq, dk, dv, dbias = oracle.backward(q, k, v, o, do, lse, scale, bias=bias, return_dbias=True,
                                        **kw)
    h = 1e-6

    def loss():
        return np.sum(do * oracle.forward(q, k, v, scale, bias=bias, **kw)[0])

    for x, g in ((bias, dbias), (q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            old = x[mi]
            x[mi] = old + h
            lp = loss()
            x[mi] = old - h
            lm = loss()
            x[mi] = old
            fd[mi] = (lp - lm) / (2 * h)
        assert np.max(np.abs(g - fd)) <= 1e-6 * max(1.0, np.max(np.abs(fd)))


def test_bias_row_shift_invariance_and_row_sums():
    q, k, v, do, o, lse, scale, kw, bias = _bias_problem(42, dict(causal=True, W=-1), B=1, S=6)
    g1 = oracle.backward(q, k, v, o, do, lse, scale, bias=bias, return_dbias=True, **kw)
    shifted = bias + np.random.default_rng(3).standard_normal((1, 2, 6, 1)) * 5.0
    o2, lse2 = oracle.forward(q, k, v, scale, bias=shifted, **kw)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    g2 = oracle.backward(q, k, v, o2, do, lse2, scale, bias=shifted, return_dbias=True, **kw)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(b, a, atol=1e-12)
    # each row of dBias (= dS) sums to zero
    np.testing.assert_allclose(g1[3].sum(axis=-1), 0.0, atol=1e-12)


def test_causal_mask_as_bias():
    # a causal mask written as a bias of -inf above the diagonal, in a non-causal call
    q, k, v, do, o, lse, scale, kw = _problem(43, B=1, Hq=2, Hkv=1, Sq=6, Skv=6, causal=True)
    mask_bias = np.where(np.tril(np.ones((6, 6), dtype=bool)), 0.0, -np.inf)[None, None]
    mask_bias = np.repeat(mask_bias, 2, axis=1)
    o2, lse2 = oracle.forward(q, k, v, scale, bias=mask_bias)
    np.testing.assert_allclose(o2, o, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)
    ref = oracle.backward(q, k, v, o, do, lse, scale, return_intermediates=True, **kw)
    got = oracle.backward(q, k, v, o2, do, lse2, scale, bias=mask_bias, return_dbias=True)
    for a, b in zip(ref[:3], got[:3]):
        np.testing.assert_allclose(b, a, atol=1e-13)
    np.testing.assert_allclose(got[3], ref[4], atol=1e-13)   # dBias = dS of the causal call


def test_zero_bias_is_no_bias():
    q, k, v, do, o, lse, scale, kw = _problem(44, B=2, Hq=2, Hkv=2, Sq=5, Skv=7, causal=True, W=2)
    zb = np.zeros((1, 2, 5, 7))
    o2, lse2 = oracle.forward(q, k, v, scale, bias=zb, **kw)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(lse2, lse)
    a = oracle.backward(q, k, v, o, do, lse, scale, **kw)
    b = oracle.backward(q, k, v, o, do, lse, scale, bias=zb, return_dbias=True, **kw)
    for x, y in zip(a, b[:3]):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("kind", ["scaled", "no_batch_sum", "sign"])
def test_planted_dbias_mistakes_are_caught(kind):
    q, k, v, do, o, lse, scale, kw, bias = _bias_problem(45, dict(causal=True, W=-1), B=2, S=4,
                                                         bias_batch=1)
    dbias = oracle.backward(q, k, v, o, do, lse, scale, bias=bias, return_dbias=True, **kw)[3]
    if kind == "scaled":                 # dBias = scale * dS (scale applied like dK's)
        dbias = scale * dbias
    elif kind == "no_batch_sum":         # batch-1 bias given only batch entry 0's dS
        d0 = oracle.backward(q[:1], k[:1], v[:1], o[:1], do[:1], lse[:1], scale, bias=bias,
                             return_dbias=True, **kw)[3]
        dbias = d0
    else:
        dbias = -dbias
    h = 1e-6
    fd = np.zeros_like(bias)
    it = np.nditer(bias, flags=["multi_index"])
    for _ in it:
        mi = it.multi_index
        old = bias[mi]
        bias[mi] = old + h
        lp = np.sum(do * oracle.forward(q, k, v, scale, bias=bias, **kw)[0])
        bias[mi] = old - h
        lm = np.sum(do * oracle.forward(q, k, v, scale, bias=bias, **kw)[0])
        bias[mi] = old
        fd[mi] = (lp - lm) / (2 * h)
    assert np.max(np.abs(dbias - fd)) > 1e-3


@pytest.mark.parametrize("mask", [dict(causal=False, W=-1), dict(causal=True, W=-1),
                                  dict(causal=True, W=2)], ids=str)
@pytest.mark.parametrize("scale", [0.37, 2.5])
def test_bias_matches_torch_float_mask(mask, scale):
    # the bias's place relative to the softmax scale, pinned by a library routine: torch's fp64 CPU
    # SDPA with a float attn_mask adds the mask to the already scaled scores; at a scale other than
    # 1 (and 1/sqrt(D)) a bias applied before the scale, or scaled with it, would differ.  O, LSE
    # (through O), dQ, dK, dV and dBias (the mask's gradient) must agree.
    q, k, v, do, _, _, _, kw = _problem(46, B=2, Hq=2, Hkv=2, Sq=7, Skv=7, Dqk=8, Dv=6, **mask)
    bias = np.random.default_rng(47).standard_normal((2, 2, 7, 7)) * 1.5
    o, lse = oracle.forward(q, k, v, scale, bias=bias, **kw)
    dq, dk, dv, dbias = oracle.backward(q, k, v, o, do, lse, scale, bias=bias, return_dbias=True,
                                        **kw)
    vis = oracle.visible_mask(7, 7, kw["causal"], kw["window_left"])
    tb = torch.tensor(bias, requires_grad=True)
    attn_mask = tb + torch.tensor(np.where(vis, 0.0, -np.inf))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn_mask,
                                                           scale=scale)
    out.backward(torch.tensor(do))
    np.testing.assert_allclose(o, out.detach().numpy(), rtol=1e-12, atol=1e-12)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (dbias, tb.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)
    # the same mask placed before the scale is a different function (the pin discriminates)
    pre = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(k), torch.tensor(v),
        attn_mask=torch.tensor(bias * scale) + torch.tensor(np.where(vis, 0.0, -np.inf)),
        scale=scale)
    assert np.max(np.abs(pre.numpy() - o)) > 1e-3
