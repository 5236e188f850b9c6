"""The C-ABI library loads, exports every symbol include/starkv.h declares,
and rejects bad arguments on the host before any HIP call (no GPU needed:
every call here fails validation, so nothing is launched)."""
import ctypes
import os
import re

import pytest

from rank_compressed_paged_amd import starkv as sk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "starkv.h")

FAKE = 0x10000          # aligned, never dereferenced: validation fails first
MISALIGNED = 0x10008


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(starkv_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header():
    decl = declared_symbols()
    assert decl, "no declarations parsed"
    for name in decl:
        assert hasattr(sk.lib(), name), f"{name} declared but not exported"
    assert sorted(sk.EXPORTED) == decl


def test_version_and_status_strings():
    assert sk.abi_version() == 8
    for s in range(0, 8):
        assert sk.lib().starkv_status_string(s)
    assert sk.lib().starkv_status_string(99) == b"unknown status"


def _main_dims(nb=8):
    return sk.make_dims(32, 128, 64, 512, nb)


def test_shape_support():
    assert sk.shape_supported(_main_dims())
    assert sk.shape_supported(sk.make_dims(32, 128, 64, 512, 3, num_kv_heads=8))
    assert sk.shape_supported(sk.make_dims(32, 128, 64, 512, 3, num_kv_heads=32))
    assert sk.shape_supported(sk.make_dims(4, 64, 16, 64, 3, num_kv_heads=2))
    assert sk.shape_supported(sk.make_dims(32, 128, 32, 256, 3))          # low-rank profile
    assert sk.shape_supported(sk.make_dims(4, 64, 16, 64, 3))
    # the generic kernels: any shape with d a multiple of 32 up to 256, r_k a
    # multiple of 8 up to min(d, 256), r_v a multiple of 8 up to
    # min(2048, Hkv d), Hkv dividing H
    for dims in [(32, 128, 32, 512), (32, 128, 64, 256), (28, 96, 48, 640), (32, 128, 128, 1024),
                 (64, 256, 256, 2048), (32, 128, 16, 128), (1, 32, 8, 8)]:
        assert sk.shape_supported(sk.make_dims(*dims, 3)), dims
    for hkv in (4, 16):          # r_v 512 needs Hkv d >= 512
        assert sk.shape_supported(sk.make_dims(32, 128, 64, 512, 3, num_kv_heads=hkv))
    assert not sk.shape_supported(sk.make_dims(32, 100, 64, 512, 3))     # d not a multiple of 32
    assert not sk.shape_supported(sk.make_dims(32, 288, 64, 512, 3))     # d above 256
    assert not sk.shape_supported(sk.make_dims(32, 128, 60, 512, 3))     # r_k not a multiple of 8
    assert not sk.shape_supported(sk.make_dims(32, 128, 64, 4096, 3))    # r_v above 2048
    assert not sk.shape_supported(sk.make_dims(4, 32, 8, 200, 3, num_kv_heads=1))  # r_v > Hkv d
    assert not sk.shape_supported(sk.make_dims(32, 128, 64, 512, 3, num_kv_heads=5))  # not a divisor
    assert not sk.shape_supported(sk.make_dims(32, 128, 64, 512, 3, num_kv_heads=-1))
    assert not sk.shape_supported(sk.make_dims(32, 128, 64, 512, 3, block_size=32))
    assert not sk.shape_supported(sk.make_dims(32, 128, 256, 512, 3))  # r_k > d
    assert not sk.shape_supported(sk.make_dims(32, 128, 64, 512, 0))


def _decode(dims, q=FAKE, kc=FAKE, vc=FAKE, U=FAKE, W=FAKE, bt=FAKE, mb=128, sl=FAKE, B=16,
            msl=2048, scale=0.088, out=FAKE, ws=FAKE, wsb=0):
    return sk.lib().starkv_decode_attn(ctypes.byref(dims), q, kc, vc, U, W, bt, mb, sl, B, msl,
                                       scale, out, ws, wsb, None)


def test_decode_validation():
    d = _main_dims()
    need = sk.decode_workspace_size(d, 16, 2048)
    assert need > 16 * 32 * 512 * 4
    assert _decode(d) == 4                                   # workspace too small
    assert _decode(d, q=None, wsb=need) == 1                 # null pointer
    assert _decode(d, q=MISALIGNED, wsb=need) == 5           # misaligned
    assert _decode(d, mb=100, wsb=need) == 2                 # block table too narrow
    assert _decode(d, B=-1) == 2
    assert _decode(d, scale=0.0) == 7
    assert _decode(d, scale=float("nan")) == 7
    assert _decode(sk.make_dims(32, 100, 64, 256, 8)) == 3   # unsupported shape
    assert sk.lib().starkv_decode_attn(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, FAKE, 1, 1,
                                       0.1, FAKE, FAKE, 0, None) == 1
    assert _decode(d, B=0) == 0                              # empty batch: no-op


def test_append_validation():
    d = _main_dims()
    f = sk.lib().starkv_append
    ws = sk.append_workspace_size(d, 4)
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, FAKE, ws, None) == 2
    assert f(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, ws, None) == 1
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, MISALIGNED, FAKE, 4, FAKE, FAKE, FAKE, ws,
             None) == 5
    assert f(ctypes.byref(d), None, None, None, None, None, 0, None, None, None, 0, None) == 0
    # the few-token path needs its workspace: missing, short or misaligned
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, None, 0, None) == 1
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, ws - 1,
             None) == 4
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, MISALIGNED, ws,
             None) == 5
    # the append only sees key/value heads: the 8-head view of the grouped
    # shape is accepted, an unknown head count is not
    kv8 = sk.make_dims(8, 128, 64, 512, 8)
    assert f(ctypes.byref(kv8), None, None, None, None, None, 0, None, None, None, 0, None) == 0
    assert f(ctypes.byref(kv8), FAKE, None, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, ws, None) == 1
    bad = sk.make_dims(16, 100, 64, 512, 8)       # outside every instance's limits
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, FAKE, ws,
             None) == 3


def test_append_workspace_size():
    """The reserved 256 bytes (arrival counters) and fp32 partials of the value
    projection: up to 64 tokens over S slices of W's Hkv*d rows (S = Hkv*d / R,
    R = max(64, Hkv*d * (r_v/32) / 256)); beyond that, at the main shape,
    over four parts of the contraction up to 1792 tokens, two parts up to
    2816, none above; nothing at the shapes without a tuned instance."""
    d = _main_dims()
    H = 256  # reserved header
    assert sk.append_workspace_size(d, 16) == H + 16 * 16 * 512 * 4      # S 16 (R 256)
    assert sk.append_workspace_size(d, 64) == H + 16 * 64 * 512 * 4
    assert sk.append_workspace_size(d, 65) == H + 4 * 65 * 512 * 4
    assert sk.append_workspace_size(d, 1792) == H + 4 * 1792 * 512 * 4
    assert sk.append_workspace_size(d, 1793) == H + 2 * 1793 * 512 * 4
    assert sk.append_workspace_size(d, 2816) == H + 2 * 2816 * 512 * 4
    assert sk.append_workspace_size(d, 2817) == 0
    assert sk.append_workspace_size(d, 4096) == 0
    assert sk.append_workspace_size(sk.make_dims(32, 128, 32, 256, 8), 1024) == 0
    assert sk.append_workspace_size(sk.make_dims(32, 128, 32, 256, 8), 16) == H + 32 * 16 * 256 * 4
    assert sk.append_workspace_size(sk.make_dims(4, 64, 16, 64, 8), 5) == H + 4 * 5 * 64 * 4
    # shapes without a few-token instance take the tiled kernel: no workspace
    assert sk.append_workspace_size(sk.make_dims(28, 96, 48, 640, 8), 16) == 0
    assert sk.append_workspace_size(sk.make_dims(32, 128, 64, 512, 8, num_kv_heads=16), 16) == 0
    assert sk.append_workspace_size(d, 0) == 0
    # grouped-query caches: only the key/value heads enter (Hkv*d = 1024: R 64, S 16)
    assert sk.append_workspace_size(sk.make_dims(32, 128, 64, 512, 8, num_kv_heads=8), 16) == \
        H + 16 * 16 * 512 * 4
    assert sk.lib().starkv_append_workspace_size(ctypes.byref(d), 4, None) == 1
    assert sk.lib().starkv_append_workspace_size(ctypes.byref(d), -1,
                                                 ctypes.byref(ctypes.c_size_t())) == 2


def test_workspace_header_reserved():
    """Every decode and prefill layout starts after the reserved 256 bytes, so
    a workspace is never smaller than that."""
    d = _main_dims()
    assert sk.decode_workspace_size(d, 0, 2048) >= 256
    assert sk.decode_workspace_size(d, 1, 16) >= 256 + 32 * 64 * 4
    assert sk.prefill_workspace_size(d, 1, 1, 16) >= 256 + 32 * 64 * 4


def test_check_indices_validation():
    """Host checks of the index scan, all before any launch."""
    f = sk.lib().starkv_check_indices
    d = sk.make_dims(1, 32, 8, 8, 100)
    assert f(ctypes.byref(d), FAKE, 8, FAKE, 4, 128, FAKE, 16, None, None) == 1   # no report
    assert f(None, FAKE, 8, FAKE, 4, 128, FAKE, 16, FAKE, None) == 1
    assert f(ctypes.byref(d), None, 8, FAKE, 4, 128, FAKE, 16, FAKE, None) == 1   # no table
    assert f(ctypes.byref(d), FAKE, 8, None, 4, 128, FAKE, 16, FAKE, None) == 1   # no lengths
    assert f(ctypes.byref(d), FAKE, 8, FAKE, 4, 128, None, 16, FAKE, None) == 1   # no slots
    assert f(ctypes.byref(d), FAKE, 8, FAKE, 4, 129, FAKE, 16, FAKE, None) == 2   # table too short
    assert f(ctypes.byref(d), FAKE, 8, FAKE, 4, 128, FAKE, -1, FAKE, None) == 2
    assert f(ctypes.byref(d), FAKE, 8, FAKE, -1, 128, FAKE, 16, FAKE, None) == 2
    d17 = sk.make_dims(1, 32, 8, 8, 100, block_size=17)
    assert f(ctypes.byref(d17), FAKE, 8, FAKE, 4, 128, FAKE, 16, FAKE, None) == 2
    assert f(ctypes.byref(d), FAKE, 8, FAKE, 4, 128, FAKE, 16, FAKE + 4, None) == 5
    assert f(ctypes.byref(d), FAKE + 8, 8, FAKE, 4, 128, FAKE, 16, FAKE, None) == 5


def test_prefill_validation():
    d = _main_dims()
    f = sk.lib().starkv_prefill_attn
    need = sk.prefill_workspace_size(d, 16, 4096, 4352)
    # q~ (fp32, r_k per head) and z (fp16, r_v per head) of every chunk query
    assert need >= 4096 * 32 * (64 * 4 + 512 * 2)
    args = lambda **kw: dict(dict(q=FAKE, qsl=FAKE, T=4096, mq=256, kc=FAKE, vc=FAKE, U=FAKE,
                                  W=FAKE, bt=FAKE, mb=272, sl=FAKE, B=16, msl=4352, scale=0.088,
                                  out=FAKE, ws=FAKE, wsb=0), **kw)

    def call(a):
        return f(ctypes.byref(d), a["q"], a["qsl"], a["T"], a["mq"], a["kc"], a["vc"], a["U"],
                 a["W"], a["bt"], a["mb"], a["sl"], a["B"], a["msl"], a["scale"], a["out"],
                 a["ws"], a["wsb"], None)
    assert call(args()) == 4
    assert call(args(qsl=None, wsb=need)) == 1
    assert call(args(mq=0, wsb=need)) == 2
    assert call(args(mq=5000, wsb=need)) == 2
    assert call(args(mb=10, wsb=need)) == 2
    assert call(args(scale=-1.0, wsb=need)) == 7
    assert call(args(T=0)) == 0


def test_timing_event_validation():
    f = sk.lib().starkv_set_timing_events
    assert f(None, None, 0) == 0
    assert f(None, None, 1) == 1
    assert f(FAKE, FAKE, 9) == 7
    assert f(FAKE, FAKE, 6) == 7
    assert f(None, None, 5) == 1   # the streaming-read selector needs both events
    assert f(None, None, 0) == 0


def test_decode_plan_properties():
    d = _main_dims()
    for B, L in [(16, 2048), (64, 8192), (20, 32768), (1, 1), (2, 256), (1, 40000)]:
        pps, ns = sk.decode_plan(d, B, L)
        pages = -(-L // 16)
        assert ns >= 1 and 1 <= pps <= 256
        assert pps * ns >= pages and pps * (ns - 1) < pages


def test_decode_config_validation():
    """The plan override: fields 0 (the library's choice) or in range; the
    workspace follows the plan."""
    d = _main_dims()
    f = sk.lib().starkv_decode_attn_cfg
    fs = sk.lib().starkv_decode_workspace_size_cfg

    def size(cfg):
        out = ctypes.c_size_t(0)
        st = fs(ctypes.byref(d), 16, 2048, ctypes.byref(cfg) if cfg else None, ctypes.byref(out))
        return st, out.value

    def call(cfg, wsb):
        return f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 16, 2048, 0.088,
                 ctypes.byref(cfg) if cfg else None, FAKE, FAKE, wsb, None)
    st, dflt = size(None)
    assert st == 0 and dflt == sk.decode_workspace_size(d, 16, 2048)
    assert size(sk.DecodeConfig(0, 0)) == (0, dflt)
    st, one = size(sk.DecodeConfig(1, 0))                 # 128 splits per sequence
    assert st == 0 and one > dflt
    assert size(sk.DecodeConfig(257, 0))[0] == 7
    assert size(sk.DecodeConfig(-1, 0))[0] == 7
    assert size(sk.DecodeConfig(0, 3))[0] == 7
    for m in (1, 2, 4, 8):
        assert size(sk.DecodeConfig(0, m))[0] == 0
    assert size(sk.DecodeConfig(0, 0, 1))[0] == 7         # launches: 0, 2 or 3
    assert size(sk.DecodeConfig(0, 0, 3)) == (0, dflt)    # the default: three launches
    st, two = size(sk.DecodeConfig(0, 0, 2))
    assert st == 0 and two > dflt                         # the fused step's counters
    assert call(sk.DecodeConfig(0, 5), one) == 7
    assert call(sk.DecodeConfig(0, 0, 4), one) == 7
    assert call(sk.DecodeConfig(1, 0), one - 1) == 4      # sized for the default plan: too small
    assert call(None, dflt - 1) == 4


def test_decode_noalloc_validation():
    """The entry point without a workspace checks on the host like the others,
    and refuses a plan that needs more than its 32 MiB scratch."""
    d = _main_dims()
    f = sk.lib().starkv_decode_attn_noalloc

    def call(B=16, msl=2048, mb=128, q=FAKE, scale=0.088):
        return f(ctypes.byref(d), q, FAKE, FAKE, FAKE, FAKE, FAKE, mb, FAKE, B, msl, scale, FAKE,
                 None)
    assert sk.decode_workspace_size(d, 256, 4096) > sk.NOALLOC_SCRATCH_BYTES
    assert call(B=256, msl=4096, mb=256) == 4           # beyond the scratch: refused
    assert call(q=None) == 1
    assert call(q=MISALIGNED) == 5
    assert call(mb=100) == 2
    assert call(scale=0.0) == 7
    assert call(B=0) == 0


def test_decode_plan_ignores_environment(monkeypatch):
    """The plan is a function of the call's arguments and the device only:
    the environment variables that tuning builds once read change nothing."""
    d = _main_dims()
    before = [sk.decode_plan(d, B, L) for B, L in [(16, 2048), (1, 8192), (64, 6000)]]
    sizes = [sk.decode_workspace_size(d, B, L) for B, L in [(16, 2048), (1, 8192)]]
    for name, val in [("STARKV_DECODE_TARGET_WGS", "4096"), ("STARKV_DECODE_MIN_PAGES", "64"),
                      ("STARKV_DECODE_SPLIT_COST", "5"), ("STARKV_DECODE_FINISH_TB", "8"),
                      ("STARKV_DECODE_VARIANT", "3")]:
        monkeypatch.setenv(name, val)
    assert [sk.decode_plan(d, B, L) for B, L in [(16, 2048), (1, 8192), (64, 6000)]] == before
    assert [sk.decode_workspace_size(d, B, L) for B, L in [(16, 2048), (1, 8192)]] == sizes
    text = "".join(open(os.path.join(ROOT, "rank_compressed_paged_amd", "csrc", f)).read()
                   for f in os.listdir(os.path.join(ROOT, "rank_compressed_paged_amd", "csrc")))
    assert "getenv" not in text


def test_fit_validation():
    f = sk.lib().starkv_fit_bases
    d = _main_dims()
    need = sk.fit_workspace_size(d)
    # the fp32 value Gram matrix alone is (H*d)^2 * 4 bytes
    assert need >= (32 * 128) ** 2 * 4

    def call(dims=d, N=4096, iters=4, k=FAKE, info=None, wsb=need, res=None):
        return f(ctypes.byref(dims), k, FAKE, N, FAKE, FAKE, iters, FAKE, FAKE, FAKE, wsb, info,
                 res, None)
    assert call(wsb=need - 1) == 4                               # workspace too small
    assert call(k=None) == 1                                     # null pointer
    assert call(k=MISALIGNED) == 5
    assert call(info=FAKE + 2) == 5                              # info must be 4-byte aligned
    assert call(res=FAKE + 2) == 5                               # so must the residual
    assert call(N=511) == 2                                      # fewer samples than r_v
    assert call(iters=0) == 7
    assert call(iters=1001) == 7
    assert call(dims=sk.make_dims(32, 96, 64, 512, 8)) == 3      # d not a multiple of 64
    assert call(dims=sk.make_dims(32, 128, 64, 1024, 8)) == 3    # r_v > 512
    assert call(dims=sk.make_dims(32, 128, 129, 512, 8)) == 2    # r_k > d
    assert f(None, FAKE, FAKE, 1, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, None, None, None) == 1
    # any shape within the limits, block size and page count unused
    odd = sk.make_dims(3, 192, 40, 100, 0, block_size=7)
    assert sk.fit_workspace_size(odd) >= (3 * 192) ** 2 * 4


def test_fp8_validation():
    d = _main_dims()
    fa = sk.lib().starkv_append_fp8
    ws = sk.append_workspace_size(d, 4)
    assert fa(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0.0, 1.0, FAKE, FAKE, FAKE, ws,
              None) == 7
    assert fa(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1.0, float("inf"), FAKE, FAKE,
              FAKE, ws, None) == 7
    assert fa(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1.0, 1.0, None, FAKE, FAKE, ws,
              None) == 1
    assert fa(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1.0, 1.0, FAKE, FAKE, FAKE, ws - 1,
              None) == 4
    assert fa(ctypes.byref(d), None, None, None, None, None, 0, 1.0, 1.0, None, None, None, 0,
              None) == 0
    fd = sk.lib().starkv_decode_attn_fp8
    need = sk.decode_workspace_size(d, 16, 2048)

    def dec(dims=d, ks=0.5, vs=0.5, scale=0.088, wsb=need, q=FAKE):
        return fd(ctypes.byref(dims), q, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 16, 2048, scale,
                  ks, vs, FAKE, FAKE, wsb, None)
    assert dec(wsb=0) == 4
    assert dec(ks=-1.0) == 7
    assert dec(vs=float("nan")) == 7
    assert dec(q=None) == 1
    assert dec(dims=sk.make_dims(32, 100, 32, 256, 8)) == 3   # outside every instance's limits
