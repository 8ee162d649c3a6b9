"""Host-side checks of the C ABI (no GPU needed): the library loads and exports every function
declared in include/sdpa_bwd.h, the workspace size follows its carve rules, and every rejected call
returns its status before touching the GPU (validation precedes any HIP call)."""
import ctypes
import os
import re

import pytest

import attention_backward_sdpa_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa_bwd.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_bwd\w*)\s*\(", text)))


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(lib.LIB_PATH):
        pytest.fail("libsdpa_bwd.so is not built: run __graft_entry__.build()")
    return lib.library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("sdpa_bwd", "sdpa_bwd_ex", "sdpa_bwd_workspace_size", "sdpa_bwd_status_string",
              "sdpa_bwd_ex_events", "sdpa_bwd_preprocess", "sdpa_bwd_flex", "sdpa_bwd_dq_route",
              "sdpa_bwd_run"):
        assert n in names


def test_library_exports_every_declared_symbol(so):
    for name in _declared_functions():
        assert hasattr(so, name), f"libsdpa_bwd.so does not export {name}"


def test_status_strings(so):
    assert lib.status_string(0) == "ok"
    for s in range(1, 6):
        assert lib.status_string(s) != "ok"
    assert lib.status_string(99) == "unknown status"


def _route(Dqk, Dv, det, B=1, Hq=4, Hkv=4, Sq=256, Skv=256):
    return lib.dq_route(B, Hq, Hkv, Sq, Skv, Dqk, Dv, det)


def test_dq_route_choice(so):
    assert _route(64, 64, 1) == lib.DQ_PARTIALS
    for d in ((128, 128), (192, 128), (256, 256)):
        assert _route(*d, 1) == lib.DQ_DS_PANELS
    for d in ((64, 64), (128, 128), (192, 128), (256, 256)):
        assert _route(*d, 0) == lib.DQ_ATOMIC
        assert _route(*d, 2) == lib.DQ_DS_PANELS
        assert _route(*d, 3) == lib.DQ_PARTIALS
        assert _route(*d, 4) == lib.DQ_RELAY
        assert _route(*d, 5) == -1
    # head dims that are multiples of 8 up to 256 run on the next supported size
    assert _route(96, 96, 1) == _route(128, 128, 1)
    assert _route(40, 40, 1) == _route(64, 64, 1)
    # head dim 32 has its own kernel (256-key tiles): the dQ-partial route is the deterministic
    # choice (32 fp32 per q row < 256 bf16 dS values)
    assert _route(32, 32, 1) == lib.DQ_PARTIALS
    assert _route(24, 24, 1) == _route(16, 8, 1) == lib.DQ_PARTIALS
    for bad in ((100, 100), (264, 264), (128, 192), (4, 4)):
        assert _route(*bad, 0) == -1
    # sizes sdpa_bwd rejects
    assert _route(128, 128, 0, Hkv=3) == -1 and _route(128, 128, 0, Sq=-1) == -1


GIB4 = 1 << 32


def _route_of(d, det=1):
    return lib.dq_route(d["B"], d["Hq"], d["Hkv"], d["Sq"], d["Skv"], d["Dqk"], d["Dv"], det)


def test_deterministic_choice_falls_back_to_the_relay(so):
    # "Determinism": a deterministic call whose quadratic buffer would exceed 4 GiB takes the
    # relay, and its workspace becomes linear in the sequence lengths; route and workspace size
    # switch together
    def det_ws(**kw):
        return _ws(deterministic=True, **kw)

    # dS panels at head dim 128: B*Hq*Skv_pad*Sq_pad*2 bytes; 32 heads at S = 8192 is exactly 4 GiB
    at = dict(B=1, Hq=32, Hkv=32, Sq=8192, Skv=8192, Dqk=128, Dv=128)
    assert _route_of(at) == lib.DQ_DS_PANELS
    assert det_ws(**at) == _al(32 * 8192 * 8) + GIB4
    over = dict(at, Hq=33, Hkv=33)
    assert _route_of(over) == lib.DQ_RELAY
    relay = det_ws(**over)
    assert relay == _ws(deterministic=lib.DQ_RELAY, **over) < GIB4 // 8
    # linear from there on: twice the length, twice the relay workspace (up to alignment)
    long = dict(over, Sq=16384, Skv=16384)
    assert _route_of(long) == lib.DQ_RELAY
    assert abs(det_ws(**long) - 2 * relay) <= 4 * 256
    # the explicit routes keep their buffers whatever the size
    assert _ws(deterministic=lib.DQ_DS_PANELS, **over) == _al(33 * 8192 * 8) + 33 * GIB4 // 32
    # head dim 64 takes the dQ partials, B*Hq*(Skv_pad/256)*Sq_pad*64*4 bytes, until they exceed
    # 4 GiB: 64 heads at S = 8192 are exactly 4 GiB
    d64 = dict(B=2, Hq=32, Hkv=8, Sq=8192, Skv=8192, Dqk=64, Dv=64)
    assert _route_of(d64) == lib.DQ_PARTIALS
    d64o = dict(d64, Sq=8224)
    assert _route_of(d64o) == lib.DQ_RELAY
    assert det_ws(**d64o) == _ws(deterministic=lib.DQ_RELAY, **d64o)
    # sdpa_bwd_run_dq_route agrees without a bias
    torch = pytest.importorskip("torch")
    q = torch.empty(1, 33, 8192, 128, dtype=torch.bfloat16, device="meta")
    k = torch.empty(1, 33, 8192, 128, dtype=torch.bfloat16, device="meta")
    assert lib.run_dq_route(q, k, k, deterministic=1) == lib.DQ_RELAY
    assert lib.run_dq_route(q[:, :32], k[:, :32], k[:, :32], deterministic=1) == lib.DQ_DS_PANELS


def _ws(**kw):
    base = dict(B=1, Hq=4, Hkv=4, Sq=256, Skv=256, Dqk=128, Dv=128, causal=False,
                window_left=-1, deterministic=False, has_seqlens=False)
    base.update(kw)
    return lib.workspace_size(**base)


def _al(n):
    return (n + 255) // 256 * 256


def test_workspace_size_rules(so):
    # non-deterministic MHA: per-row statistics (2 floats per row, rows padded to 32) and the fp32
    # dQ accumulator
    assert _ws() == _al(4 * 256 * 8) + _al(4 * 256 * 128 * 4)
    # GQA adds per-query-head bf16 dK/dV partials
    assert _ws(Hkv=1) == _ws() + 2 * _al(4 * 256 * 128 * 2)
    # deterministic: statistics + bf16 dS (S_kv padded to the 256-key tile, S_q to the 32-row
    # q tile), no fp32 dQ
    assert _ws(deterministic=True, Sq=200, Skv=200) == _al(4 * 224 * 8) + _al(4 * 224 * 256 * 2)
    # explicit dS panels: the same as the deterministic choice at head dim 256
    assert _ws(deterministic=lib.DQ_DS_PANELS, Sq=200, Skv=200) == \
        _al(4 * 224 * 8) + _al(4 * 224 * 256 * 2)
    # dQ partials: one 32 x Dqk fp32 block per (KV tile of 256 keys, q tile)
    parts = _al(4 * 224 * 8) + _al(4 * 1 * 224 * 128 * 4)
    assert _ws(deterministic=lib.DQ_PARTIALS, Sq=200, Skv=200) == parts
    # the deterministic choice at head dim 64 (64 fp32 per q row < 256 bf16 dS values)
    d64 = dict(Dqk=64, Dv=64, Sq=200, Skv=200)
    assert _ws(deterministic=True, **d64) == _ws(deterministic=lib.DQ_PARTIALS, **d64) == \
        _al(4 * 224 * 8) + _al(4 * 1 * 224 * 64 * 4)
    assert _ws(deterministic=lib.DQ_PARTIALS, Sq=200, Skv=300) == \
        _al(4 * 224 * 8) + _al(4 * 2 * 224 * 128 * 4)
    # head dim 256 (128-key tiles): the deterministic choice is the dS panels
    d256 = dict(Dqk=256, Dv=256, Sq=200, Skv=200)
    assert _ws(deterministic=True, **d256) == _ws(deterministic=lib.DQ_DS_PANELS, **d256) == \
        _al(4 * 224 * 8) + _al(4 * 224 * 256 * 2)
    assert _ws(deterministic=lib.DQ_PARTIALS, **d256) == \
        _al(4 * 224 * 8) + _al(4 * 2 * 224 * 256 * 4)
    # head dim 192 (256-key tiles): 192 fp32 per q row > 256 bf16 -> dS panels
    d192 = dict(Dqk=192, Dv=128, Sq=200, Skv=200)
    assert _ws(deterministic=True, **d192) == _ws(deterministic=lib.DQ_DS_PANELS, **d192)
    # the relay: one 32 x Dqk fp32 running sum per q tile, one int32 turn counter per q tile and
    # 16 int32 control words, whatever the key length (linear in the sequence lengths)
    relay = _al(4 * 224 * 8) + _al(4 * 224 * 128 * 4) + _al(4 * 7 * 4) + _al(16 * 4)
    assert _ws(deterministic=lib.DQ_RELAY, Sq=200, Skv=200) == relay
    assert _ws(deterministic=lib.DQ_RELAY, Sq=200, Skv=5000) == relay
    assert _ws(deterministic=lib.DQ_RELAY, Sq=200, Skv=200, Hkv=1) == \
        relay + _al(4 * 200 * 128 * 2) * 2
    # unknown route values are rejected
    assert _ws(deterministic=5) == 0 and _ws(deterministic=-1) == 0
    # monotone in the sequence length
    sizes = [_ws(Sq=s, Skv=s) for s in (64, 128, 300, 1000)]
    assert sizes == sorted(sizes)
    # rejected shapes need nothing
    assert _ws(Hkv=3) == 0
    # head dims that are multiples of 8 up to 256 use the next supported size's workspace
    assert _ws(Dqk=96, Dv=96) == _ws(Dqk=128, Dv=128)
    assert _ws(Dqk=24, Dv=16) == _ws(Dqk=32, Dv=32) < _ws(Dqk=64, Dv=64)
    assert _ws(Dqk=40, Dv=40) == _ws(Dqk=64, Dv=64)
    assert _ws(Dqk=176, Dv=104) == _ws(Dqk=192, Dv=128)
    assert _ws(Dqk=160, Dv=160) == _ws(Dqk=256, Dv=256)
    assert _ws(Dqk=100, Dv=100) == 0 and _ws(Dqk=272, Dv=272) == 0
    assert _ws(Sq=0) == 0


def _call(so, **kw):
    a = dict(B=1, Hq=4, Hkv=4, Sq=64, Skv=64, Dqk=128, Dv=128, scale=0.0, causal=0, wl=-1, det=0,
             lens_q=None, lens_kv=None, br=0, wr=0, ws=None, ws_bytes=0)
    a.update(kw)
    p = ctypes.c_void_p(4096)  # aligned, never dereferenced: validation fails before any launch
    ptrs = [kw.get(n, p) for n in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv")]
    return so.sdpa_bwd_ex(*ptrs, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Skv"], a["Dqk"], a["Dv"],
                          a["scale"], a["causal"], a["wl"], a["det"], a["lens_q"], a["lens_kv"],
                          a["br"], a["wr"], a["ws"], a["ws_bytes"], None)


def test_rejections_before_launch(so):
    assert _call(so, Hkv=3) == lib.INVALID_ARG                    # H_kv does not divide H_q
    assert _call(so, Hq=-1) == lib.INVALID_ARG
    assert _call(so, wl=-2) == lib.INVALID_ARG                    # window_left < -1
    assert _call(so, wr=-1) == lib.INVALID_ARG
    assert _call(so, det=5) == lib.INVALID_ARG                    # unknown dQ route
    assert _call(so, det=4) == lib.INVALID_ARG                    # relay: needs a workspace
    assert _call(so, det=-1) == lib.INVALID_ARG
    assert _call(so, Dqk=100, Dv=100) == lib.UNSUPPORTED          # not a multiple of 8
    assert _call(so, Dqk=264, Dv=264) == lib.UNSUPPORTED          # above 256
    assert _call(so, Dqk=96, Dv=96) == lib.INVALID_ARG            # served as 128: no workspace
    assert _call(so, Dqk=128, Dv=192) == lib.UNSUPPORTED          # D_v > D_qk
    assert _call(so, q=ctypes.c_void_p(4098)) == lib.UNSUPPORTED  # misaligned pointer
    assert _call(so, dk=None) == lib.INVALID_ARG                  # null output
    assert _call(so, ws=None, ws_bytes=0) == lib.INVALID_ARG      # workspace needed but absent
    need = _ws(Sq=64, Skv=64)
    assert _call(so, ws=ctypes.c_void_p(1 << 20), ws_bytes=need - 1) == lib.WORKSPACE_TOO_SMALL
    assert _call(so, ws=ctypes.c_void_p((1 << 20) + 16), ws_bytes=need) == lib.UNSUPPORTED


def _flex(so, layouts=None, dtype=lib.BF16, S=64, D=128, ws=None, ws_bytes=0):
    p = ctypes.c_void_p(4096)  # aligned, never dereferenced: validation fails before any launch
    return so.sdpa_bwd_flex(p, p, p, p, p, p, p, p, p, 1, 4, 4, S, S, D, D, 0.0, 0, -1, 0, None,
                            None, 0, 0, layouts, dtype, ws, ws_bytes, None, None)


def _bhsd(H=4, S=64, D=128):
    return (H * S * D, S * D, D)


def _lay(entries):
    arr = (lib.Layout * 8)()
    for x, e in enumerate(entries):
        arr[x] = lib.Layout(*e)
    return arr


def test_flex_rejections_before_launch(so):
    good = [_bhsd()] * 8
    # contiguous layouts pass every check and stop at the missing workspace
    assert _flex(so, _lay(good)) == lib.INVALID_ARG
    assert _flex(so, None) == lib.INVALID_ARG
    ws = ctypes.c_void_p(1 << 20)
    need = _ws(Sq=64, Skv=64)
    assert _flex(so, _lay(good), ws=ws, ws_bytes=need - 1) == lib.WORKSPACE_TOO_SMALL
    # BSHD storage viewed as BHSD: (S*H*D, D, H*D)
    bshd = [(64 * 4 * 128, 128, 4 * 128)] * 8
    assert _flex(so, _lay(bshd), ws=ws, ws_bytes=need - 1) == lib.WORKSPACE_TOO_SMALL
    assert _flex(so, dtype=lib.FP16) == lib.INVALID_ARG            # fp16 accepted (no workspace)
    assert _flex(so, dtype=7) == lib.UNSUPPORTED                   # unknown io type
    for x in range(8):
        bad = list(good)
        bad[x] = (good[x][0], good[x][1], 120)                     # rows overlap (seq < D)
        assert _flex(so, _lay(bad)) == lib.INVALID_ARG
        bad[x] = (good[x][0], good[x][1], 132)                     # rows not 16-byte aligned
        assert _flex(so, _lay(bad)) == lib.UNSUPPORTED
        bad[x] = (good[x][0] + 4, good[x][1], good[x][2])          # batch stride not a multiple of 8
        assert _flex(so, _lay(bad)) == lib.UNSUPPORTED
        bad[x] = (-good[x][0], good[x][1], good[x][2])             # negative stride
        assert _flex(so, _lay(bad)) == lib.INVALID_ARG
        bad[x] = (good[x][0], good[x][1], 1 << 25)                 # one head spans >= 2^31 bytes
        assert _flex(so, _lay(bad)) == lib.UNSUPPORTED


def test_preprocess_rejections(so):
    p = ctypes.c_void_p(4096)
    assert so.sdpa_bwd_preprocess(p, p, p, p, None, None, 1, 1, 8, 100, 100, None) == lib.UNSUPPORTED
    assert so.sdpa_bwd_preprocess(None, p, p, p, None, None, 1, 1, 8, 128, 128, None) == lib.INVALID_ARG
    assert so.sdpa_bwd_preprocess(p, p, p, None, None, None, 1, 1, 8, 128, 128, None) == lib.INVALID_ARG


def test_args_struct_layout_matches_header(tmp_path):
    # the ctypes mirror of sdpa_bwd_args has the C layout: compile the header with gcc and compare
    # the size and every field offset
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    names = [f[0] for f in lib.Args._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "sdpa_bwd.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(sdpa_bwd_args));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(sdpa_bwd_args, {n}));\n' for n in names) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(lib.Args)
    assert out[1:] == [getattr(lib.Args, n).offset for n in names]


def test_run_rejections_before_launch(so):
    assert so.sdpa_bwd_run(None) == lib.INVALID_ARG
    p = 4096  # aligned, never dereferenced: validation fails before any launch
    a = lib.Args()
    for n in ("q", "k", "v", "o", "dO", "lse", "dq", "dk", "dv"):
        setattr(a, n, p)
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.Dqk, a.Dv = 1, 4, 4, 64, 64, 128, 128
    a.window_left = -1
    need = _ws(Sq=64, Skv=64)
    a.workspace, a.workspace_bytes = 1 << 20, need
    a.dsink = 8192                      # dsink without sink logits
    assert so.sdpa_bwd_run(ctypes.byref(a)) == lib.INVALID_ARG
    a.sink = 8194                       # misaligned sink
    assert so.sdpa_bwd_run(ctypes.byref(a)) == lib.INVALID_ARG
    a.sink = 8196
    a.workspace_bytes = need - 1        # with valid sink arguments the workspace check is reached
    assert so.sdpa_bwd_run(ctypes.byref(a)) == lib.WORKSPACE_TOO_SMALL
    a.deterministic = 5
    assert so.sdpa_bwd_run(ctypes.byref(a)) == lib.INVALID_ARG


def test_io_dtype_dbias_workspace_and_rejections(so):
    # "The kernel chain" dbias_cvt: an io-type dBias summed over the batch (a batch-1 bias with
    # B > 1) adds an fp32 accumulator of Hq * Sq * Skv floats (256-byte aligned) at the end of the
    # carve; a per-batch one is written directly and needs none (host tensors stand in for device
    # ones: the size query reads only their shapes and whether they exist)
    torch = pytest.importorskip("torch")
    for Bb in (1, 2):
        q = torch.empty(2, 4, 200, 128, dtype=torch.bfloat16, device="cpu")
        k = torch.empty(2, 2, 300, 128, dtype=torch.bfloat16, device="cpu")
        bias = torch.empty(Bb, 4, 200, 300, dtype=torch.bfloat16, device="cpu")
        for det in (0, 2, 3):
            base = lib.run_workspace_size(q, k, k, causal=True, deterministic=det, bias=bias)
            f32 = lib.run_workspace_size(q, k, k, causal=True, deterministic=det, bias=bias,
                                         dbias=torch.empty(Bb, 4, 200, 300, device="cpu"))
            io = lib.run_workspace_size(q, k, k, causal=True, deterministic=det, bias=bias,
                                        dbias=torch.empty(Bb, 4, 200, 300, dtype=torch.bfloat16))
            assert f32 == base and io == base + (_al(4 * 200 * 300 * 4) if Bb == 1 else 0)
        # an io-type dBias of another type than the inputs is refused by the binding
        with pytest.raises(ValueError):
            lib.run_workspace_size(q, k, k, bias=bias, dbias=torch.empty(
                Bb, 4, 200, 300, dtype=torch.float16, device="cpu"))
    # alignment: 2 bytes for an io-type dBias, 4 for fp32
    p = 4096
    a = lib.Args()
    for n in ("q", "k", "v", "o", "dO", "lse", "dq", "dk", "dv"):
        setattr(a, n, p)
    a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.Dqk, a.Dv = 1, 4, 4, 64, 64, 128, 128
    a.window_left = -1
    a.bias, a.bias_batch, a.bias_dtype = 8192, 1, lib.BF16
    a.workspace, a.workspace_bytes = 1 << 20, 0
    a.dbias = 8194  # 2-byte aligned: accepted as io type, rejected as fp32
    assert so.sdpa_bwd_run(ctypes.byref(a)) == lib.UNSUPPORTED
    a.dbias_io = 1
    assert so.sdpa_bwd_run(ctypes.byref(a)) == lib.WORKSPACE_TOO_SMALL
    a.dbias = 8193
    assert so.sdpa_bwd_run(ctypes.byref(a)) == lib.UNSUPPORTED


def test_nvfp4_qat_workspace_and_rejections(so):
    # the fake-quantised Q, K, V copies, then the chain's carve in the 8-wave layout (256-key
    # tiles; the relay route keeps 4 waves): statistics and, on the atomic route, the fp32 dQ
    # accumulator
    B, H, Sq, Skv = 1, 2, 200, 300
    hat = _al(B * H * Sq * 128 * 2) + 2 * _al(B * H * Skv * 128 * 2)
    assert lib.nvfp4_qat_workspace_size(B, H, Sq, Skv, 128, False, 0) == \
        hat + _al(B * H * 224 * 8) + _al(B * H * Sq * 128 * 4)
    # dS panels over 256-key tiles (Skv padded to 512)
    assert lib.nvfp4_qat_workspace_size(B, H, Sq, Skv, 128, False, 2) == \
        hat + _al(B * H * 224 * 8) + _al(B * H * 224 * 512 * 2)
    assert lib.nvfp4_qat_workspace_size(B, H, Sq, Skv, 64, False, 0) == 0      # head dim 128 only
    assert lib.nvfp4_qat_workspace_size(B, H, Sq, Skv, 128, True, 0) == 0      # causal: Sq == Skv
    assert lib.nvfp4_qat_workspace_size(B, H, Sq, Skv, 128, False, 5) == 0
    p = ctypes.c_void_p(4096)

    def call(D=128, causal=0, det=0, Sq=64, Skv=64, ws=None, ws_bytes=0):
        return so.sdpa_bwd_nvfp4_qat(p, p, p, p, p, p, p, p, p, 1, 2, Sq, Skv, D, 0.0, causal, det,
                                     ws, ws_bytes, None, None)
    assert call(D=64) == lib.UNSUPPORTED
    assert call(causal=1, Skv=65) == lib.UNSUPPORTED
    assert call(det=5) == lib.INVALID_ARG
    assert call() == lib.INVALID_ARG                                  # no workspace
    assert call(ws=p, ws_bytes=16) == lib.WORKSPACE_TOO_SMALL


def test_bias_layout_choice(so):
    # An io-type bias whose rows split into 16-byte chunks (Skv a multiple of 8, a 16-byte-aligned
    # tensor) runs the 8-wave layout with 256-key tiles, any other bias the 4-wave layout with
    # 128-key tiles. The dQ-partial route's workspace shows the key tile: one 32 x Dqk fp32 block
    # per (head, key tile, q tile).
    def size(Skv, bias, bias_dtype=lib.BF16, det=3):
        a = lib.Args()
        a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.Dqk, a.Dv = 1, 2, 2, 512, Skv, 128, 128
        a.window_left, a.deterministic, a.dtype = -1, det, lib.BF16
        a.bias, a.bias_batch, a.bias_dtype = bias, 1, bias_dtype
        return so.sdpa_bwd_run_workspace_size(ctypes.byref(a))

    blocks = lambda n_kv: 2 * n_kv * 512 * 128 * 4  # heads x key tiles x q rows x Dqk x fp32
    assert size(512, 0) == size(512, 8192)                        # 8 waves, as without a bias
    assert size(512, 8194) == size(512, 8192) + blocks(4) - blocks(2)    # misaligned: 4 waves
    assert size(512, 8192, lib.FP32) == size(512, 8194)            # fp32 bias: 4 waves
    assert size(516, 8192) == size(516, 8194)                      # Skv % 8 != 0: 4 waves
    # the relay keeps the 4-wave layout; its workspace does not depend on the key tile
    assert size(512, 8192, det=4) == size(512, 8194, det=4)
