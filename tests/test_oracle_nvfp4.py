"""Pins of the NVFP4 attention-QAT oracle ("NVFP4 Attention QAT Backward", "Overview") against
things other than itself: torch's float8_e4m3fn cast, the E2M1 tie table, invariants of a
block-scaled quantiser, finite differences of the two forward outputs the gradients belong to, and
the reduction to the plain backward when quantisation is switched off."""
import numpy as np
import pytest

import oracle
from oracle import nvfp4_qat as Q

torch = pytest.importorskip("torch")

E2M1_GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(0)
    # every finite positive E4M3 value, the midpoints between neighbours, and random magnitudes
    codes = torch.arange(1, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = (codes[:-1].astype(np.float64) + codes[1:]) / 2
    rand = np.exp(rng.uniform(np.log(2.0 ** -11), np.log(448.0), 4000))
    x = np.concatenate([codes, mids, rand, [0.0, 2.0 ** -10, 3 * 2.0 ** -10]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    got = Q.e4m3_round(x)
    assert np.array_equal(got, ref)
    # every E4M3 value is a fixed point; beyond the largest finite value the scale saturates
    assert np.array_equal(Q.e4m3_round(codes), codes)
    assert Q.e4m3_round(np.float32(1000.0)) == 448.0


def test_e2m1_ties_and_grid():
    # the grid is fixed; ties go to the even code (0, 1, 2, 4), above 6 saturates
    assert np.array_equal(Q.e2m1_round(E2M1_GRID), E2M1_GRID)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert Q.e2m1_round(ties).tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert Q.e2m1_round(np.float32([0.26, 0.74, 1.26, 2.51, 3.49, 5.01, 7.0, 100.0])).tolist() == \
        [0.5, 0.5, 1.5, 3.0, 3.0, 6.0, 6.0, 6.0]
    assert np.array_equal(Q.e2m1_round(-ties), -Q.e2m1_round(ties))


def test_fake_nvfp4_ties_under_non_power_of_two_scale():
    # amax 9 gives the scale 1.5 (exact in E4M3); x / 1.5 hits the E2M1 midpoints exactly, which
    # the correctly rounded division keeps, and they go to the even neighbour
    g = np.array([9.0, 0.375, 1.125, 1.875, 3.75, 5.25, 7.5, -1.125] + [0.0] * 8, np.float32)
    out = Q.fake_nvfp4(g)
    assert out[:8].tolist() == [9.0, 0.0, 1.5, 1.5, 3.0, 6.0, 6.0, -1.5]


def test_fake_nvfp4_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 64)).astype(np.float32)
    y = Q.fake_nvfp4(x)
    # idempotent: a quantised group has amax = 6 * scale exactly or maps onto the same grid
    assert np.array_equal(Q.fake_nvfp4(y), y)
    # odd, and commutes with powers of two inside the E4M3 range
    assert np.array_equal(Q.fake_nvfp4(-x), -y)
    assert np.array_equal(Q.fake_nvfp4(4 * x), 4 * y)
    # every output is an E2M1 value times its group's E4M3 scale
    g = x.reshape(3, 5, 4, 16)
    scale = Q.e4m3_round(np.abs(g).max(-1, keepdims=True) / np.float32(6))
    ratio = np.abs(y.reshape(3, 5, 4, 16)) / scale
    assert np.all(np.isin(ratio, E2M1_GRID))
    # groups are independent; a zero group stays zero
    x2 = x.copy()
    x2[..., 16:32] *= 7
    x2[..., 48:64] = 0
    y2 = Q.fake_nvfp4(x2)
    assert np.array_equal(y2[..., :16], y[..., :16]) and np.array_equal(y2[..., 32:48], y[..., 32:48])
    assert np.all(y2[..., 48:64] == 0)
    # a group built from grid values and a representable scale (with +-6 in it) comes back exactly
    built = (rng.choice(E2M1_GRID, 16) * np.sign(rng.standard_normal(16))).astype(np.float32)
    built[3] = 6.0
    assert np.array_equal(Q.fake_nvfp4(built * np.float32(0.6875)), built * np.float32(0.6875))
    # a ragged last group is quantised as if padded with zeros
    r = rng.standard_normal((2, 37)).astype(np.float32)
    padded = np.concatenate([r, np.zeros((2, 11), np.float32)], axis=1)
    assert np.array_equal(Q.fake_nvfp4(r), Q.fake_nvfp4(padded)[:, :37])
    # the quantisation is not the identity on random data
    assert not np.array_equal(y, x)


def _softmax_out(q, k, v, scale, causal, p_transform=None):
    s = scale * np.einsum("bhqd,bhkd->bhqk", q, k)
    if causal:
        s = np.where(np.tril(np.ones(s.shape[-2:], bool)), s, -np.inf)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    if p_transform is not None:
        p = p_transform(p)
    return np.einsum("bhqk,bhkd->bhqd", p, v)


@pytest.mark.parametrize("causal", [False, True])
def test_qat_backward_finite_differences(causal):
    rng = np.random.default_rng(2)
    B, H, S, D = 1, 2, 20, 16
    q, k, v, do = (rng.standard_normal((B, H, S, D)).astype(np.float32) for _ in range(4))
    scale = 0.4
    o_hp, lse = oracle.qat_forward(q, k, v, scale, causal=causal)
    dq, dk, dv = oracle.qat_backward(q, k, v, o_hp, do, lse, scale, causal=causal)
    qh, kh, vh = (Q.fake_nvfp4(t).astype(np.float64) for t in (q, k, v))
    dO = do.astype(np.float64)
    eps = 1e-6
    # dQ, dK: gradients of <O_hp, dO> with respect to Q^ and K^ (the unquantised probability)
    for name, grad, which in (("dQ", dq, 0), ("dK", dk, 1)):
        for idx in [(0, 0, 3, 5), (0, 1, 17, 0), (0, 1, 9, 15)]:
            args = [qh.copy(), kh.copy(), vh]
            args[which][idx] += eps
            fp = np.sum(_softmax_out(*args, scale, causal) * dO)
            args[which][idx] -= 2 * eps
            fm = np.sum(_softmax_out(*args, scale, causal) * dO)
            assert abs((fp - fm) / (2 * eps) - grad[idx]) < 1e-5 * max(1.0, abs(grad[idx])), name
    # dV: gradient of <fake(P) V^, dO> with respect to V^ (fake(P) does not depend on V)
    fake_p = lambda p: Q.fake_nvfp4(p.astype(np.float32)).astype(np.float64)
    for idx in [(0, 0, 2, 7), (0, 1, 19, 3)]:
        vp = vh.copy()
        vp[idx] += eps
        fp = np.sum(_softmax_out(qh, kh, vp, scale, causal, fake_p) * dO)
        vp[idx] -= 2 * eps
        fm = np.sum(_softmax_out(qh, kh, vp, scale, causal, fake_p) * dO)
        assert abs((fp - fm) / (2 * eps) - dv[idx]) < 1e-6 * max(1.0, abs(dv[idx]))
    # and it is not the plain dV = P^T dO
    p_plain = oracle.backward(qh, kh, vh, o_hp, dO, lse, scale, causal=causal)[2]
    assert not np.allclose(dv, p_plain, rtol=1e-3, atol=1e-6)


def test_qat_backward_without_quantisation_is_plain_backward():
    rng = np.random.default_rng(3)
    B, H, Sq, Skv, D = 2, 2, 24, 40, 32
    q = rng.standard_normal((B, H, Sq, D)).astype(np.float32)
    k, v = (rng.standard_normal((B, H, Skv, D)).astype(np.float32) for _ in range(2))
    do = rng.standard_normal((B, H, Sq, D)).astype(np.float32)
    f = lambda t: t.astype(np.float64)
    o, lse = oracle.forward(f(q), f(k), f(v), 0.3)
    got = oracle.qat_backward(q, k, v, o, do, lse, 0.3, quantize=False)
    ref = oracle.backward(f(q), f(k), f(v), o, f(do), lse, 0.3)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal,Sq,Skv", [(True, 70, 70), (False, 50, 83)])
def test_qat_sampled_rows_match_full_backward(causal, Sq, Skv):
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 2, Sq, 32)).astype(np.float32)
    k, v = (rng.standard_normal((1, 2, Skv, 32)).astype(np.float32) for _ in range(2))
    do = rng.standard_normal((1, 2, Sq, 32)).astype(np.float32)
    o, lse = oracle.qat_forward(q, k, v, 0.3, causal=causal)
    full = oracle.qat_backward(q, k, v, o, do, lse, 0.3, causal=causal)
    qr, kr = [0, 17, Sq - 1], [0, 15, 16, Skv - 1]
    rows = Q.qat_backward_rows(q, k, v, o, do, lse, 0.3, 0, 1, qr, kr, causal=causal)
    for got, ref in zip(rows, (full[0][0, 1, qr], full[1][0, 1, kr], full[2][0, 1, kr])):
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
