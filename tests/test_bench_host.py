"""Host logic of bench.py, checked without a GPU: the count of fp32 dQ atomic adds that one
main-kernel launch makes on the atomic route (reported with the measured atomic rate as the
route's floor), against brute force over the element-wise visibility rule."""
import numpy as np

import bench
from attention_backward_sdpa_amd import synth

W = synth.WORKLOADS
V = synth.small_variant


def brute_force_adds(w, lens):
    """Every (key tile, q tile) pair with at least one visible (q, k) pair adds one dQ block:
    its rows below the query length times the kernel head dim, per query head."""
    kq, bc, br = bench.kernel_tiles(w)
    total = 0
    for b in range(w.B):
        L = w.Sq if lens is None else int(lens[b])
        q = np.arange(w.Sq)[:, None]
        k = np.arange(w.Skv)[None, :]
        vis = (q < L) & (k < L)
        if w.causal:
            vis &= k <= q
        if w.window_left >= 0:
            vis &= k >= q - w.window_left
        for k0 in range(0, w.Skv, bc):
            for q0 in range(0, w.Sq, br):
                if vis[q0:q0 + br, k0:k0 + bc].any():
                    total += min(br, L - q0) * w.Hq * kq
    return total


def test_headline_closed_form():
    # causal, 16 key tiles of 256 keys over 128 q tiles of 32 rows: key tile j sees 128 - 8 j
    # q tiles, 1088 in all, each a 32 x 128 block, for 32 query heads
    assert bench.dq_atomic_adds(W["gqa_causal_s4096_d128"], None) == 32 * 1088 * 32 * 128


def test_against_brute_force():
    cases = [
        V(W["gqa_causal_s4096_d128"], Hq=4, Hkv=1, Sq=600, Skv=600),
        V(W["mha_causal_s2048_d128"], Hq=2, Hkv=2, Sq=333, Skv=333, causal=False),
        V(W["mla_window_padded_s4096"], B=3, Hq=2, Hkv=2, Sq=700, Skv=700, window_left=90,
          len_lo=150),
        V(W["mha_det_s8192_d256"], Hq=1, Hkv=1, Sq=300, Skv=300),
        V(W["gqa_causal_s4096_d128"], Hq=2, Hkv=1, Sq=530, Skv=530, window_left=40, Dqk=64, Dv=64),
    ]
    for w in cases:
        lens = synth.draw_inputs(w).seq_q_lens if w.padded else None
        assert bench.dq_atomic_adds(w, lens) == brute_force_adds(w, lens), w



def test_kernel_tiles_match_the_library_plan():
    """bench.py's model of the main kernel's key tile (which sets its atomic-add count) agrees with
    the library's own layout choice, read from the dQ-partial workspace: statistics, then one
    32 x Dqk fp32 block per (head, key tile, q tile).  MHA with 8 q tiles keeps the grid unsplit,
    so there are no dK/dV partials in the carve."""
    import ctypes
    import attention_backward_sdpa_amd as lib
    so = lib.library()
    al = lambda n: (n + 255) // 256 * 256
    B, H, Sq = 1, 2, 256
    for D, Dv in ((32, 32), (64, 64), (128, 128), (192, 128), (256, 256)):
        for Skv in (512, 520, 516):
            for bias in (False, True):
                w = V(W["mha_s128_d64"], B=B, Hq=H, Hkv=H, Sq=Sq, Skv=Skv, Dqk=D, Dv=Dv)
                kq, bc, br = bench.kernel_tiles(w, bias)
                a = lib.Args()
                a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.Dqk, a.Dv = B, H, H, Sq, Skv, D, Dv
                a.window_left, a.deterministic, a.dtype = -1, 3, lib.BF16
                if bias:  # an io-type, 16-byte-aligned bias (the kind bench.py draws)
                    a.bias, a.bias_batch, a.bias_dtype = 8192, B, lib.BF16
                n_kv = -(-Skv // bc)
                expected = al(B * H * Sq * 2 * 4) + al(B * H * n_kv * Sq * kq * 4)
                assert so.sdpa_bwd_run_workspace_size(ctypes.byref(a)) == expected, (D, Skv, bias, bc)
