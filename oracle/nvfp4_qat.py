"""CPU oracle of the NVFP4 attention-QAT backward ("NVFP4 Attention QAT Backward", "Overview").

TEST INFRASTRUCTURE ONLY, like the rest of this package: the GPU library never imports it.

What the page fixes:
  * Q, K and V are fake-quantised to NVFP4 and immediately dequantised: E2M1 values with one E4M3
    scale for every 16 values;
  * the converted value x / scale is formed with precise (correctly rounded) division, so exact
    E2M1 midpoints round to nearest even;
  * with Q^, K^, V^ the fake-quantised inputs and P = softmax(scale * Q^ K^T):
        dS = P * (dO V^T - rowsum(O_hp * dO)),   O_hp = P V^ (the pre-probability-quantisation
                                                 output saved by the forward, "high_precision_o")
        dQ = scale * dS K^,   dK = scale * dS^T Q^   (the unquantised P: straight-through estimator)
        dV = fake_nvfp4(P)^T dO                      (the fake-quantised probability)
  * MHA, head dimension 128, bf16 activations, fp32 LSE; causal only for self-attention.

Readings where the page is silent (the plainest ones; each is also listed in the design notes):
  * the 16-value groups run along the last (contiguous) axis: the head dim of Q, K, V, and the key
    axis of P (16 consecutive keys of one query row);
  * the group scale is amax / 6 rounded to nearest even in E4M3 (the OCP "fn" format: 4 exponent
    bits, bias 7, 3 mantissa bits, subnormals down to 2^-9, largest finite 448), saturating at 448;
    6 is the largest E2M1 magnitude; amax / 6 is an fp32 division;
  * E2M1 (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) is reached by round to nearest
    even of x / scale in fp32, saturating at 6; a group whose amax is 0 (scale 0) stays 0;
  * P is quantised from its fp32 value after masking (masked pairs are 0 and take part in their
    group's amax as zeros), and the dequantised values q * scale are formed in fp32, where they
    are exact.
Everything else is the fp64 oracle backward of sdpa_oracle on the fake-quantised inputs.
"""
import numpy as np

from . import sdpa_oracle as _sdpa

E2M1_MAX = 6.0
E4M3_MAX = 448.0
GROUP = 16


def e4m3_round(x):
    """Round float32 magnitudes (x >= 0) to the nearest E4M3 value, ties to even, saturating at
    448.  Normal range [2^-6, 448]: 3 mantissa bits, so the quantum is 2^(e-3) for x in
    [2^e, 2^(e+1)); below 2^-6 the quantum is the subnormal step 2^-9."""
    x = np.asarray(x, dtype=np.float32)
    out = np.zeros_like(x)
    pos = x > 0
    xp = x[pos].astype(np.float64)
    e = np.floor(np.log2(xp))
    e = np.maximum(e, -6.0)                     # subnormals share the 2^-9 quantum of 2^-6
    quantum = np.exp2(e - 3.0)
    r = np.round(xp / quantum) * quantum        # numpy rounds halves to even; x / quantum exact
    out[pos] = np.minimum(r, E4M3_MAX).astype(np.float32)
    return out


def e2m1_round(y):
    """Round float32 values to the nearest E2M1 value, ties to even (the even codes are 0, 1, 2, 4
    times the sign), saturating at +-6.  Quantum 0.5 below 2, 1 in [2, 4), 2 in [4, 6]."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    quantum = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.round(a / quantum) * quantum          # halves to even: the even integers are the
    r = np.minimum(r, E2M1_MAX)                  # even E2M1 codes in every binade
    return (np.sign(y) * r).astype(np.float32)


def fake_nvfp4(x):
    """Fake NVFP4 quantisation along the last axis in groups of 16 (a ragged last group is padded
    with zeros): returns float32 values q * scale, q in E2M1, scale in E4M3 per group."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    pad = (-n) % GROUP
    xp = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,), np.float32)], axis=-1) if pad else x
    g = xp.reshape(xp.shape[:-1] + (xp.shape[-1] // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1, keepdims=True)
    scale = e4m3_round(amax / np.float32(E2M1_MAX))            # fp32 division
    safe = np.where(scale > 0, scale, np.float32(1.0))
    q = e2m1_round(g / safe)                                    # fp32 (correctly rounded) division
    out = np.where(scale > 0, q * scale, np.float32(0.0)).astype(np.float32)
    return out.reshape(xp.shape)[..., :n]


def qat_forward(q, k, v, scale, causal=False):
    """The high-precision forward of the QAT recipe: O_hp = softmax(scale Q^ K^T) V^ and the
    natural-log LSE, in fp64 on the fake-quantised inputs (test-input generation)."""
    qh, kh, vh = (fake_nvfp4(t).astype(np.float64) for t in (q, k, v))
    return _sdpa.forward(qh, kh, vh, scale, causal=causal)


def qat_backward(q, k, v, o_hp, do, lse, scale, causal=False, quantize=True):
    """dQ, dK, dV of the QAT backward (equations above).  quantize=False replaces every fake
    quantisation by the identity, which must give the plain backward."""
    fq = fake_nvfp4 if quantize else (lambda t: np.asarray(t, dtype=np.float32))
    qh, kh, vh = (fq(t).astype(np.float64) for t in (q, k, v))
    # P is quantised from its fp32 value (without quantisation it stays fp64)
    fp = (lambda p: fake_nvfp4(p.astype(np.float32)).astype(np.float64)) if quantize else (lambda p: p)
    # dQ, dK: the plain backward on the fake-quantised inputs, delta from O_hp (unquantised P)
    dq, dk, _ = _sdpa.backward(qh, kh, vh, np.asarray(o_hp, np.float64),
                               np.asarray(do, np.float64), np.asarray(lse, np.float64), scale,
                               causal=causal)
    # dV from the fake-quantised probability of each (batch, head)
    B, H, Sq, _ = np.shape(q)
    Skv = np.shape(k)[2]
    vis = _sdpa.visible_mask(Sq, Skv, causal)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scale * (qh[b, h] @ kh[b, h].T)
            p = _sdpa._probabilities(s, np.asarray(lse, np.float64)[b, h], vis)
            dv[b, h] = fp(p).T @ np.asarray(do, np.float64)[b, h]
    return dq, dk, dv


def qat_backward_rows(q, k, v, o_hp, do, lse, scale, b, h, q_rows, kv_rows, causal=False):
    """Sampled rows of the QAT backward for one (batch, head): dQ[q_rows] and (dK, dV)[kv_rows].
    Only the score entries the equations need are formed: the listed query rows against all keys
    for dQ; for dK and dV every query row against the listed keys, and against the whole 16-key
    group of each listed key, since fake(P) of a key depends on its group's amax."""
    qh = fake_nvfp4(np.asarray(q[b, h], np.float32)).astype(np.float64)
    kh = fake_nvfp4(np.asarray(k[b, h], np.float32)).astype(np.float64)
    vh = fake_nvfp4(np.asarray(v[b, h], np.float32)).astype(np.float64)
    dob = np.asarray(do[b, h], np.float64)
    lseb = np.asarray(lse[b, h], np.float64)
    delta = np.sum(np.asarray(o_hp[b, h], np.float64) * dob, axis=1)
    Sq, Skv = qh.shape[0], kh.shape[0]
    vis = _sdpa.visible_mask(Sq, Skv, causal)
    q_rows = np.asarray(q_rows)
    p = _sdpa._probabilities(scale * (qh[q_rows] @ kh.T), lseb[q_rows], vis[q_rows])
    ds = p * (dob[q_rows] @ vh.T - delta[q_rows][:, None])
    dq = scale * (ds @ kh)
    dk = np.zeros((len(kv_rows), kh.shape[1]))
    dv = np.zeros((len(kv_rows), vh.shape[1]))
    for n, j in enumerate(kv_rows):
        g0 = (j // GROUP) * GROUP
        cols = np.arange(g0, min(g0 + GROUP, Skv))
        pg = _sdpa._probabilities(scale * (qh @ kh[cols].T), lseb, vis[:, cols])
        pq = fake_nvfp4(pg.astype(np.float32)).astype(np.float64)  # the group's fake(P), rows
        c = j - g0
        dv[n] = pq[:, c] @ dob
        dsj = pg[:, c] * (dob @ vh[j] - delta)
        dk[n] = scale * (dsj @ qh)
    return dq, dk, dv
