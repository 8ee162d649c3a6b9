"""Plain fp64 CPU oracle of scaled-dot-product attention: forward (to make inputs) and backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library imports this module and this module imports
nothing from the GPU library; the two share only the seeded input generator, which holds none of
the method's arithmetic.  Every array is processed whole, per (batch, head), in float64, with the
score matrix formed densely over all keys, so that each line can be checked against the equations
by eye.

Sources (cited by page title and section):
  * "SDPA Backward (SM120)", section "API Usage": the tensor contract (logical (B, H, S, D), LSE is
    the natural-log forward statistic of shape (B, H, S_q)), the default softmax scale 1/sqrt(D),
    the left-window rule (a key k is masked when k < q + diag - W) and the right band R
    (keep k <= q + diag + R), per-batch padding lengths.
  * same page, "The kernel chain": delta = rowsum(O * dO).
  * same page, "Main-kernel pipeline: KV-stationary, five chained GEMMs": S = Q K^T, P replayed from
    the natural-log LSE, dP = dO V^T, dS = P * (dP - delta), dV += P^T dO, dQ = dS K, dK += dS^T Q.
  * same page, "GQA/MQA group reduction": the KV head of query head h is h // (H_q / H_kv); dK and
    dV of a KV head are the sums over its group of query heads; dQ is unaffected.
  * same page, "Causal, sliding-window, and padding masks": top-left causal (diag = 0) or
    bottom-right (diag = seq_kv - seq_q, at the actual lengths under padding); rows at or past
    seq_q and keys at or past seq_kv carry no probability; a fully masked row has LSE = -inf and
    P = 0 (never NaN); dQ rows past seq_q and dK/dV rows past seq_kv are exactly zero.
  * "NVFP4 Attention QAT Backward", section "Overview": with the fake quantisation removed, the
    printed equations place the softmax scale as dQ = scale * dS K and dK = scale * dS^T Q, with dS
    the unscaled softmax vector-Jacobian product, and dV = P^T dO.

  * same page, "The kernel chain" (dsink) and "Support surface" (sink tokens): a per-query-head sink
    logit joins every row's softmax denominator without a value vector; the forward LSE folds it
    in, so dQ/dK/dV need no sink term, and the sink's gradient is
    dsink[h] = -sum over batch entries and query rows of exp(sink[h] - LSE) * delta.

  * same page, "API Usage" (bias_tensor) and "Support surface" (bias): an additive bias of shape
    (1 or B, H_q, S_q, S_kv) joins the scores after the softmax scale and before the softmax; its
    gradient is dBias = dS (the unscaled softmax VJP), summed over the batch entries when the bias
    has batch 1.

Readings taken where the pages leave a step open:
  * the default scale uses D_qk (the contraction length of Q K^T) when D_qk != D_v;
  * delta is formed from the O that is handed in (not re-derived as rowsum(P * dP));
  * the window bound is inclusive: W + 1 keys are visible on a causal row, the diagonal included;
  * with a sink, a query row below seq_q that sees no key still has the sink in its denominator
    (LSE = sink, O = 0); rows at or past seq_q do not exist (LSE = -inf, O = 0) and contribute
    nothing to dsink.
"""
import math

import numpy as np

LOG2E = 1.4426950408889634


def visible_mask(Sq, Skv, causal, window_left=-1, len_q=None, len_kv=None,
                 bottom_right=False, window_right=0):
    """Boolean (Sq, Skv) visibility of (query i, key j) for one batch entry.

    "SDPA Backward (SM120)", "API Usage" and "Causal, sliding-window, and padding masks":
      * padding: i < len_q and j < len_kv (lengths default to the full extents);
      * causal:  j <= i + diag + window_right, diag = 0 (top-left) or len_kv - len_q (bottom-right);
      * window:  j >= i + diag - window_left when window_left >= 0 (inclusive lower bound).
    """
    Lq = Sq if len_q is None else int(len_q)
    Lkv = Skv if len_kv is None else int(len_kv)
    diag = (Lkv - Lq) if bottom_right else 0
    i = np.arange(Sq)[:, None]
    j = np.arange(Skv)[None, :]
    vis = (i < Lq) & (j < Lkv)
    if causal:
        vis &= j <= i + diag + window_right
    if window_left is not None and window_left >= 0:
        vis &= j >= i + diag - window_left
    return vis


def _lens(B, S, lens):
    return [S] * B if lens is None else [int(x) for x in lens]


def _bias_for(bias, b, h):
    """The (S_q, S_kv) bias of batch entry b and query head h (batch-1 biases broadcast)."""
    if bias is None:
        return 0.0
    bias = np.asarray(bias)
    return np.asarray(bias[0 if bias.shape[0] == 1 else b, h], dtype=np.float64)


def forward(q, k, v, scale, causal=False, window_left=-1, seq_q_lens=None, seq_kv_lens=None,
            bottom_right=False, window_right=0, sink=None, bias=None):
    """Softmax-attention forward in fp64; returns (O, LSE), O (B,Hq,Sq,Dv), LSE (B,Hq,Sq) natural log.

    s_ij = scale * q_i . k_j on visible pairs and -inf elsewhere; LSE_i = log sum_j exp(s_ij) with
    LSE_i = -inf on a row that sees no key; P = exp(s - LSE); O = P V.  Rows with no visible key
    have O = 0.  With sink (Hq,) logits, every row below seq_q adds exp(sink[h]) to its
    denominator (the sink has no value vector).  With bias (1 or B, Hq, Sq, Skv), s_ij gains
    bias[b, h, i, j] on visible pairs.  (The forward is not the method; it produces the O and LSE
    the backward consumes.)
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Sq, _ = q.shape
    _, Hkv, Skv, Dv = v.shape
    group = Hq // Hkv
    Lq, Lkv = _lens(B, Sq, seq_q_lens), _lens(B, Skv, seq_kv_lens)
    O = np.zeros((B, Hq, Sq, Dv))
    LSE = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        vis = visible_mask(Sq, Skv, causal, window_left, Lq[b], Lkv[b], bottom_right, window_right)
        for h in range(Hq):
            kh = h // group
            s = scale * (q[b, h] @ k[b, kh].T) + _bias_for(bias, b, h)
            s = np.where(vis, s, -np.inf)
            if sink is not None and np.isfinite(sink[h]):
                # the sink is one more logit in the denominator of every existing row
                s_all = np.concatenate([s, np.where(np.arange(Sq) < Lq[b], float(sink[h]),
                                                    -np.inf)[:, None]], axis=1)
            else:
                s_all = s
            rows = np.isfinite(s_all).any(axis=1)
            m = np.where(rows, s_all.max(axis=1, initial=-np.inf), 0.0)
            denom = np.exp(s_all - m[:, None]).sum(axis=1)
            lse = np.where(rows, m + np.log(np.where(rows, denom, 1.0)), -np.inf)
            p = np.where(vis, np.exp(s - np.where(rows, lse, 0.0)[:, None]), 0.0)
            O[b, h] = p @ v[b, kh]
            LSE[b, h] = lse
    return O, LSE


def _probabilities(s_scaled, lse, vis):
    """P replayed from the natural-log LSE: P = exp(scale*S - LSE) on visible pairs, else 0.

    A row whose LSE is -inf (fully masked in the forward) yields P = 0 rather than NaN
    ("Causal, sliding-window, and padding masks").
    """
    finite = np.isfinite(lse)
    expo = s_scaled - np.where(finite, lse, 0.0)[:, None]
    return np.where(vis & finite[:, None], np.exp(np.where(vis, expo, 0.0)), 0.0)


def backward(q, k, v, o, do, lse, scale, causal=False, window_left=-1, seq_q_lens=None,
             seq_kv_lens=None, bottom_right=False, window_right=0, return_intermediates=False,
             bias=None, return_dbias=False):
    """Exact SDPA backward in fp64: returns (dQ, dK, dV) shaped like Q, K, V.

    Per (batch b, query head h), with K/V taken from KV head h // group ("SDPA Backward (SM120)",
    "The kernel chain" and "Main-kernel pipeline"; scale placement from "NVFP4 Attention QAT
    Backward", "Overview"):
        P     = exp(scale * Q K^T - LSE)   on visible pairs, 0 elsewhere
        delta = rowsum(O * dO)
        dP    = dO V^T
        dS    = P * (dP - delta)
        dV   += P^T dO
        dK   += scale * dS^T Q
        dQ    = scale * dS K
    dK and dV of a KV head are summed over its group of query heads ("GQA/MQA group reduction").
    With bias, P = exp(scale * Q K^T + bias - LSE) and, when return_dbias is set, dBias = dS
    (summed over the batch entries for a batch-1 bias) is appended to the results ("API Usage"
    bias_tensor, "Support surface" bias).
    With return_intermediates=True also returns delta (B,Hq,Sq) and dS (B,Hq,Sq,Skv).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    B, Hq, Sq, _ = q.shape
    _, Hkv, Skv, _ = k.shape
    group = Hq // Hkv
    Lq, Lkv = _lens(B, Sq, seq_q_lens), _lens(B, Skv, seq_kv_lens)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta_all = np.zeros((B, Hq, Sq)) if return_intermediates else None
    dbias = None
    if return_dbias:
        dbias = np.zeros((np.asarray(bias).shape[0], Hq, Sq, Skv))
    ds_all = np.zeros((B, Hq, Sq, Skv)) if return_intermediates else None
    for b in range(B):
        vis = visible_mask(Sq, Skv, causal, window_left, Lq[b], Lkv[b], bottom_right, window_right)
        for h in range(Hq):
            kh = h // group
            p = _probabilities(scale * (q[b, h] @ k[b, kh].T) + _bias_for(bias, b, h), lse[b, h],
                               vis)
            delta = np.sum(o[b, h] * do[b, h], axis=1)
            dp = do[b, h] @ v[b, kh].T
            ds = p * (dp - delta[:, None])
            if dbias is not None:
                dbias[0 if dbias.shape[0] == 1 else b, h] += ds
            dv[b, kh] += p.T @ do[b, h]
            dk[b, kh] += scale * (ds.T @ q[b, h])
            dq[b, h] = scale * (ds @ k[b, kh])
            if return_intermediates:
                delta_all[b, h] = delta
                ds_all[b, h] = ds
    out = (dq, dk, dv) + ((dbias,) if return_dbias else ())
    if return_intermediates:
        return out + (delta_all, ds_all)
    return out


def dsink(o, do, lse, sink, seq_q_lens=None):
    """Gradient of the sink logits, (Hq,): dsink[h] = -sum_{b, q} exp(sink[h] - LSE[b,h,q]) * delta[b,h,q].

    "SDPA Backward (SM120)", "The kernel chain" (dsink) and "Support surface" (sink tokens): the
    sink is a logit without a value vector, so its softmax VJP entry on row q is
    P_sink * (0 - delta) with P_sink = exp(sink - LSE) and delta = rowsum(O * dO); the sink is
    shared by every batch entry and row.  Rows at or past seq_q and rows whose LSE is -inf
    contribute nothing.
    """
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    B, Hq, Sq, _ = o.shape
    Lq = _lens(B, Sq, seq_q_lens)
    out = np.zeros(Hq)
    for h in range(Hq):
        total = 0.0
        for b in range(B):
            delta = np.sum(o[b, h] * do[b, h], axis=1)
            live = (np.arange(Sq) < Lq[b]) & np.isfinite(lse[b, h])
            p_sink = np.exp(float(sink[h]) - np.where(live, lse[b, h], 0.0))
            total += float(np.sum(np.where(live, p_sink * delta, 0.0)))
        out[h] = -total
    return out


def backward_dq_rows(q, k, v, o, do, lse, scale, b, h, rows, causal=False, window_left=-1,
                     seq_q_lens=None, seq_kv_lens=None, bottom_right=False, window_right=0,
                     bias=None, return_ds=False):
    """dQ[b, h, rows, :] alone, from the same equations restricted to the listed query rows.

    dQ_i = scale * sum_j dS_ij K_j with dS_ij = P_ij (dO_i . V_j - O_i . dO_i): only the rows' own
    scores are needed, so full-size tensors can be sampled row by row.  With bias the scores gain
    bias[b, h, rows] as in backward(); return_ds also returns the rows' dS, which is their dBias
    for a per-batch bias.
    """
    B, Hq, Sq, _ = q.shape
    _, Hkv, Skv, _ = k.shape
    kh = h // (Hq // Hkv)
    Lq, Lkv = _lens(B, Sq, seq_q_lens), _lens(B, Skv, seq_kv_lens)
    rows = np.asarray(rows)
    vis = visible_mask(Sq, Skv, causal, window_left, Lq[b], Lkv[b], bottom_right, window_right)[rows]
    qr = np.asarray(q[b, h, rows], dtype=np.float64)
    kb = np.asarray(k[b, kh], dtype=np.float64)
    vb = np.asarray(v[b, kh], dtype=np.float64)
    dor = np.asarray(do[b, h, rows], dtype=np.float64)
    s_rows = scale * (qr @ kb.T)
    if bias is not None:
        s_rows = s_rows + np.asarray(np.asarray(bias)[0 if np.asarray(bias).shape[0] == 1 else b, h, rows],
                                     dtype=np.float64)
    p = _probabilities(s_rows, np.asarray(lse[b, h, rows], dtype=np.float64), vis)
    delta = np.sum(np.asarray(o[b, h, rows], dtype=np.float64) * dor, axis=1)
    ds = p * (dor @ vb.T - delta[:, None])
    return (scale * (ds @ kb), ds) if return_ds else scale * (ds @ kb)


def backward_dkdv_rows(q, k, v, o, do, lse, scale, b, kv_head, rows, causal=False, window_left=-1,
                       seq_q_lens=None, seq_kv_lens=None, bottom_right=False, window_right=0,
                       bias=None):
    """(dK, dV)[b, kv_head, rows, :] alone: the listed key columns of P and dS over every query row.

    dV_j = sum_h sum_i P_ij dO_i and dK_j = scale * sum_h sum_i dS_ij Q_i, summed over the query
    heads h of the KV head's group; only the listed key columns of the score matrix are formed
    (with bias, the listed columns of bias[b, h] join the scores as in backward()).
    """
    B, Hq, Sq, _ = q.shape
    _, Hkv, Skv, _ = k.shape
    group = Hq // Hkv
    Lq, Lkv = _lens(B, Sq, seq_q_lens), _lens(B, Skv, seq_kv_lens)
    rows = np.asarray(rows)
    vis = visible_mask(Sq, Skv, causal, window_left, Lq[b], Lkv[b], bottom_right, window_right)[:, rows]
    kr = np.asarray(k[b, kv_head, rows], dtype=np.float64)
    vr = np.asarray(v[b, kv_head, rows], dtype=np.float64)
    dk = np.zeros_like(kr)
    dv = np.zeros_like(vr)
    for h in range(kv_head * group, (kv_head + 1) * group):
        qh = np.asarray(q[b, h], dtype=np.float64)
        doh = np.asarray(do[b, h], dtype=np.float64)
        s_cols = scale * (qh @ kr.T)
        if bias is not None:
            s_cols = s_cols + np.asarray(
                np.asarray(bias)[0 if np.asarray(bias).shape[0] == 1 else b, h][:, rows], dtype=np.float64)
        p = _probabilities(s_cols, np.asarray(lse[b, h], dtype=np.float64), vis)
        delta = np.sum(np.asarray(o[b, h], dtype=np.float64) * doh, axis=1)
        ds = p * (doh @ vr.T - delta[:, None])
        dv += p.T @ doh
        dk += scale * (ds.T @ qh)
    return dk, dv


def attention_flops(B, Hq, Sq, Skv, Dqk, Dv, causal=False, window_left=-1, seq_q_lens=None,
                    seq_kv_lens=None, exact=False):
    """Algorithmic FLOPs of one backward: 2*(3*Dqk + 2*Dv) per visible (query, key) pair per head.

    GEMM1 (S recompute) 2*Dqk, GEMM2 (dP) 2*Dv, GEMM3 (dV) 2*Dv, GEMM4 (dQ) 2*Dqk, GEMM5 (dK)
    2*Dqk per pair.  With exact=False a plain causal mask counts half the dense pairs (the stated
    convention); otherwise the visible pairs are counted one by one.
    """
    per_pair = 2 * (3 * Dqk + 2 * Dv)
    if not exact and window_left < 0 and seq_q_lens is None and seq_kv_lens is None:
        pairs = Sq * Skv * (0.5 if causal else 1.0)
        return per_pair * pairs * B * Hq
    Lq, Lkv = _lens(B, Sq, seq_q_lens), _lens(B, Skv, seq_kv_lens)
    pairs = 0
    for b in range(B):
        pairs += int(visible_mask(Sq, Skv, causal, window_left, Lq[b], Lkv[b]).sum())
    return per_pair * pairs * Hq
