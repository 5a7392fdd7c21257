"""The C ABI on the CPU: the library loads, exports every symbol that
include/attn.h declares, and its host-side checks reject bad arguments
before anything is launched (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

from attention_tiled_fmha_amd import attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, E_NULL, E_SHAPE, E_UNSUP, E_WS, E_HIP, E_ARG = range(7)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.LIB_PATH):
        from attention_tiled_fmha_amd import build
        build.build()
    return attn.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), f"{name} declared in attn.h but not exported"
    assert set(names) == set(attn.SIGNATURES), "binding and header disagree"


def test_checked_library(lib):
    """The checked twin exports the same interface, says which build it is,
    and answers its host-side queries (nothing here touches a device)."""
    chk = attn.load(attn.CHECKED_LIB_PATH)
    try:
        for name in declared_functions():
            assert hasattr(chk, name), f"{name} not exported by the checked library"
        assert chk.attn_checked_build() == 1
        assert lib.attn_checked_build() == 0
        flags = ctypes.c_uint(7)
        assert lib.attn_device_errors(ctypes.byref(flags), 1) == E_UNSUP
        assert chk.attn_device_errors(None, 1) == E_NULL
        n = ctypes.c_int(0)
        # no allocation known at NULL: only negative indices would be caught
        assert chk.attn_device_pool_pages(None, 4096, ctypes.byref(n)) == OK
        assert n.value == 2 ** 31 - 1
        assert chk.attn_device_pool_pages(None, 4096, None) == E_NULL
        # the host-side argument checks are the release build's
        assert chk.attn_decode_shared_prefix(None, FAKE, FAKE, FAKE, 64, FAKE, None, 4, 4, 4, 128,
                                             16, 0, 0, 0.1, None, 0, None) == E_NULL
    finally:
        attn.load(attn.LIB_PATH)
    text = open(HEADER).read()
    bits = dict(re.findall(r"#define (ATTN_DEV_ERR_\w+) (\d+)u", text))
    assert bits == {"ATTN_DEV_ERR_KV_LEN": str(attn.DEV_ERR_KV_LEN),
                    "ATTN_DEV_ERR_PAGE": str(attn.DEV_ERR_PAGE)}


def test_status_strings(lib):
    for s in range(7):
        assert attn.status_str(s) and attn.status_str(s) != "unknown status"
    assert attn.status_str(99) == "unknown status"


def prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=1, Hkv=1, Tq=8, Tk=8, D=64,
             dt=0, causal=0, scale=0.125)
    a.update(kw)
    return lib.attn_prefill(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                            a["Tq"], a["Tk"], a["D"], a["dt"], a["causal"], a["scale"], None)


def test_prefill_checks(lib):
    assert prefill(lib, q=None) == E_NULL
    assert prefill(lib, o=None) == E_NULL
    assert prefill(lib, k=None) == E_NULL
    assert prefill(lib, B=-1) == E_SHAPE
    assert prefill(lib, Tq=-3) == E_SHAPE
    assert prefill(lib, Hq=4, Hkv=3) == E_SHAPE
    assert prefill(lib, Hkv=0) == E_SHAPE
    assert prefill(lib, D=96) == E_UNSUP
    assert prefill(lib, dt=7) == E_UNSUP
    assert prefill(lib, scale=0.0) == E_ARG
    assert prefill(lib, scale=-1.0) == E_ARG
    assert prefill(lib, scale=float("nan")) == E_ARG
    assert prefill(lib, scale=float("inf")) == E_ARG
    # nothing to do: no pointers needed, nothing launched
    assert prefill(lib, B=0, q=None, k=None, v=None, o=None) == OK
    assert prefill(lib, Tq=0, q=None, k=None, v=None, o=None) == OK


def decode(lib, ws=None, ws_bytes=0, opts=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, kl=FAKE, o=FAKE, lse=None, B=2, Hq=8, Hkv=2,
             D=128, page=16, maxp=4, maxlen=64, dt=0, odt=0, scale=0.1)
    a.update(kw)
    return lib.attn_decode_paged_ex(a["q"], a["k"], a["v"], a["bt"], a["kl"], a["o"], a["lse"],
                                    a["B"], a["Hq"], a["Hkv"], a["D"], a["page"], a["maxp"],
                                    a["maxlen"], a["dt"], a["odt"], a["scale"], ws, ws_bytes,
                                    None, opts)


def test_decode_checks(lib):
    assert decode(lib, q=None) == E_NULL
    assert decode(lib, bt=None) == E_NULL
    assert decode(lib, kl=None) == E_NULL
    assert decode(lib, Hq=6, Hkv=4) == E_SHAPE
    assert decode(lib, maxp=3) == E_SHAPE            # 3 pages cannot hold 64 tokens
    assert decode(lib, maxlen=-1) == E_SHAPE
    assert decode(lib, page=32) == E_UNSUP
    assert decode(lib, D=80) == E_UNSUP
    assert decode(lib, Hq=34, Hkv=2) == E_UNSUP       # group of 17
    assert decode(lib, Hq=32, Hkv=2, dt=1) == E_UNSUP  # fp32 cache: groups of 1, 2, 4, 8 only
    assert decode(lib, odt=5) == E_UNSUP
    assert decode(lib, scale=0.0) == E_ARG
    opts = attn.DecodeOpts(split_tokens=-5)
    assert decode(lib, opts=ctypes.byref(opts)) == E_ARG
    # a long sequence needs a workspace for its partial states
    need = lib.attn_decode_workspace_bytes(2, 8, 2, 128, 100000, 0)
    assert need > 0
    assert decode(lib, maxlen=100000, maxp=6250) == E_WS
    assert decode(lib, maxlen=100000, maxp=6250, ws=FAKE, ws_bytes=need - 1) == E_WS
    assert decode(lib, B=0, q=None, k=None, v=None, bt=None, kl=None, o=None) == OK


def decode_fp8(lib, ws=None, ws_bytes=0, opts=None, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=0.5, vs=0.25, bt=FAKE, kl=FAKE, o=FAKE, lse=None, B=2,
             Hq=8, Hkv=2, D=128, page=16, maxp=4, maxlen=64, odt=0, scale=0.1)
    a.update(kw)
    return lib.attn_decode_paged_fp8(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["bt"], a["kl"],
                                     a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                     a["page"], a["maxp"], a["maxlen"], a["odt"], a["scale"], ws,
                                     ws_bytes, None, opts)


def test_decode_fp8_checks(lib):
    # every case here is rejected on the host, before anything is launched
    assert decode_fp8(lib, q=None) == E_NULL
    assert decode_fp8(lib, kl=None) == E_NULL
    assert decode_fp8(lib, Hq=6, Hkv=4) == E_SHAPE
    assert decode_fp8(lib, page=32) == E_UNSUP
    assert decode_fp8(lib, D=96) == E_UNSUP
    assert decode_fp8(lib, Hq=34, Hkv=2) == E_UNSUP
    assert decode_fp8(lib, odt=2) == E_UNSUP          # outputs are bf16 or fp32
    assert decode_fp8(lib, ks=0.0) == E_ARG
    assert decode_fp8(lib, vs=float("nan")) == E_ARG
    assert decode_fp8(lib, ks=-1.0) == E_ARG
    assert decode_fp8(lib, scale=float("inf")) == E_ARG
    uni = attn.DecodeOpts(use_unified_max=1, phi=float("nan"))
    assert decode_fp8(lib, opts=ctypes.byref(uni)) == E_ARG   # the unified max must be finite
    neg = attn.DecodeOpts(split_tokens=-1)
    assert decode_fp8(lib, opts=ctypes.byref(neg)) == E_ARG
    need = lib.attn_decode_workspace_bytes(2, 8, 2, 128, 100000, 0)
    assert decode_fp8(lib, maxlen=100000, maxp=6250, ws=FAKE, ws_bytes=need - 1) == E_WS
    assert decode_fp8(lib, B=0, q=None, k=None, v=None, bt=None, kl=None, o=None) == OK
    # the FP8 cache type is not a q / o type of the other calls
    assert decode(lib, dt=2) == E_UNSUP
    assert prefill(lib, dt=2) == E_UNSUP


def test_merge_checks(lib):
    m = lambda **kw: lib.attn_merge_states(kw.get("oa", FAKE), kw.get("la", FAKE),
                                           kw.get("ob", FAKE), kw.get("lb", FAKE),
                                           kw.get("rows", 4), kw.get("D", 128),
                                           kw.get("dt", 0), None)
    assert m(oa=None) == E_NULL
    assert m(lb=None) == E_NULL
    assert m(rows=-1) == E_SHAPE
    assert m(D=48) == E_UNSUP
    assert m(dt=3) == E_UNSUP
    assert m(rows=0, oa=None, la=None, ob=None, lb=None) == OK


def test_shared_prefix_checks(lib):
    f = lambda **kw: lib.attn_decode_shared_prefix(
        kw.get("q", FAKE), FAKE, FAKE, kw.get("pp", FAKE), kw.get("plen", 64), FAKE, None,
        kw.get("B", 4), kw.get("Hq", 4), kw.get("Hkv", 4), 128, kw.get("page", 16), 0, 0,
        kw.get("scale", 0.1), None, 0, None)
    assert f(q=None) == E_NULL
    assert f(pp=None) == E_NULL
    assert f(plen=-1) == E_SHAPE
    assert f(page=8) == E_UNSUP
    assert f(scale=-2.0) == E_ARG
    assert f(B=0) == OK


def test_shared_prefix_fp8_checks(lib):
    # every case here is rejected on the host, before anything is launched
    f = lambda **kw: lib.attn_decode_shared_prefix_fp8(
        kw.get("q", FAKE), FAKE, FAKE, kw.get("ks", 0.5), kw.get("vs", 0.25), kw.get("pp", FAKE),
        kw.get("plen", 64), FAKE, None, kw.get("B", 4), kw.get("Hq", 4), kw.get("Hkv", 4),
        kw.get("D", 128), kw.get("page", 16), kw.get("odt", 0), kw.get("scale", 0.1), None, 0,
        None)
    assert f(q=None) == E_NULL
    assert f(pp=None) == E_NULL
    assert f(plen=-1) == E_SHAPE
    assert f(Hq=6, Hkv=4) == E_SHAPE
    assert f(page=8) == E_UNSUP
    assert f(D=96) == E_UNSUP
    assert f(odt=2) == E_UNSUP
    assert f(ks=0.0) == E_ARG
    assert f(vs=float("inf")) == E_ARG
    assert f(scale=-2.0) == E_ARG
    assert f(plen=100000) == E_WS      # several prefix chunks and no workspace
    assert f(B=0) == OK
    # the plain entry does not take the FP8 cache type
    assert lib.attn_decode_shared_prefix(FAKE, FAKE, FAKE, FAKE, 64, FAKE, None, 4, 4, 4, 128,
                                         16, 2, 0, 0.1, None, 0, None) == E_UNSUP


def test_cascade_checks(lib):
    # every case here is rejected on the host, before anything is launched
    f = lambda **kw: lib.attn_decode_cascade(
        kw.get("q", FAKE), FAKE, FAKE, kw.get("pp", FAKE), kw.get("plen", 64),
        kw.get("st", FAKE), None, FAKE, None, kw.get("B", 4), kw.get("Hq", 4), kw.get("Hkv", 4),
        kw.get("D", 128), kw.get("page", 16), kw.get("mp", 8), kw.get("ml", 100),
        kw.get("dt", 0), kw.get("odt", 0), kw.get("scale", 0.1), kw.get("ks", 1.0),
        kw.get("vs", 1.0), kw.get("ws", None), 0, None)
    assert f(q=None) == E_NULL
    assert f(pp=None) == E_NULL
    assert f(st=None) == E_NULL
    assert f(plen=-1) == E_SHAPE
    assert f(ml=-1) == E_SHAPE
    assert f(Hq=6, Hkv=4) == E_SHAPE
    assert f(mp=6) == E_SHAPE          # 6 pages hold 96 < 100 tokens
    assert f(page=8) == E_UNSUP
    assert f(D=96) == E_UNSUP
    assert f(odt=2) == E_UNSUP
    assert f(dt=1) == E_UNSUP          # fp32 caches are not taken
    assert f(Hq=68, Hkv=4) == E_UNSUP  # 17 query heads per kv head
    assert f(dt=2, ks=0.0) == E_ARG
    assert f(dt=2, vs=float("inf")) == E_ARG
    assert f(ks=0.0) == E_WS           # bf16 ignores the scales; no workspace given
    assert f(scale=-2.0) == E_ARG
    assert f(ws=ctypes.c_void_p(0x1002)) == E_ARG
    assert f() == E_WS                 # prefix and own-chunk states need a workspace
    assert f(B=0) == OK


def test_cascade_workspace(lib):
    # 64 requests, 32 heads, 4096-token prefix: the prefix stage's 4 chunks of
    # 1024 tokens beside the planner's own chunks (1024 tokens: one per request)
    s, n = attn.attn_decode_plan(64, 32, 1024)
    rows = 64 * 32 * (4 + n)
    expect = -(-rows * 128 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    assert attn.attn_cascade_workspace_bytes(64, 32, 32, 128, 4096, 1024) == expect
    # a prefix shorter than one chunk still has one slot
    rows = 3 * 4 * (1 + attn.attn_decode_plan(3, 4, 100)[1])
    expect = -(-rows * 64 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    assert attn.attn_cascade_workspace_bytes(3, 4, 4, 64, 15, 100) == expect
    assert attn.attn_cascade_workspace_bytes(64, 32, 5, 128, 4096, 100) == 0   # bad group
    assert attn.attn_cascade_workspace_bytes(64, 32, 32, 128, 4096, 100, dtype=1) == 0


def test_misaligned_pointers(lib):
    # rejected on the host before any launch: tensors need 16-byte alignment,
    # lse / tables / lengths 4-byte
    odd16 = ctypes.c_void_p(0x1008)
    odd4 = ctypes.c_void_p(0x1002)
    assert prefill(lib, q=odd16) == E_ARG
    assert prefill(lib, o=odd16) == E_ARG
    assert prefill(lib, lse=odd4) == E_ARG
    assert decode(lib, k=odd16) == E_ARG
    assert decode(lib, kl=odd4) == E_ARG
    assert decode(lib, lse=odd4) == E_ARG
    assert decode_fp8(lib, v=odd16) == E_ARG
    assert lib.attn_merge_states(odd16, FAKE, FAKE, FAKE, 4, 128, 0, None) == E_ARG
    assert lib.attn_merge_states(FAKE, odd4, FAKE, FAKE, 4, 128, 0, None) == E_ARG
    assert lib.attn_decode_shared_prefix(FAKE, FAKE, FAKE, odd4, 64, FAKE, None, 4, 4, 4, 128,
                                         16, 0, 0, 0.1, None, 0, None) == E_ARG
    assert lib.attn_decode_shared_prefix(FAKE, FAKE, odd16, FAKE, 64, FAKE, None, 4, 4, 4, 128,
                                         16, 0, 0, 0.1, None, 0, None) == E_ARG


def test_prefill_paged_checks(lib):
    # every case here is rejected on the host, before anything is launched
    f = lambda **kw: lib.attn_prefill_paged(
        kw.get("q", FAKE), kw.get("k", FAKE), FAKE, kw.get("bt", FAKE), kw.get("kl", FAKE),
        kw.get("o", FAKE), kw.get("lse", None), kw.get("B", 2), kw.get("Hq", 8),
        kw.get("Hkv", 2), kw.get("Tq", 64), kw.get("D", 128), kw.get("page", 16),
        kw.get("maxp", 8), kw.get("dt", 0), kw.get("causal", 1), kw.get("scale", 0.1), None)
    assert f(q=None) == E_NULL
    assert f(bt=None) == E_NULL
    assert f(kl=None) == E_NULL
    assert f(Hq=6, Hkv=4) == E_SHAPE
    assert f(Tq=-1) == E_SHAPE
    assert f(maxp=-1) == E_SHAPE
    assert f(dt=1) == E_UNSUP          # bf16 only
    assert f(dt=2) == E_UNSUP
    assert f(page=32) == E_UNSUP
    assert f(D=96) == E_UNSUP
    assert f(scale=0.0) == E_ARG
    assert f(k=ctypes.c_void_p(0x1008)) == E_ARG
    assert f(kl=ctypes.c_void_p(0x1002)) == E_ARG
    assert f(B=0, q=None) == OK
    assert f(Tq=0, q=None) == OK


def test_decode_plan(lib):
    # workload shapes: long contexts over many sequences get 1024-token chunks
    assert attn.attn_decode_plan(32, 32, 8192) == (1024, 8)
    assert attn.attn_decode_plan(128, 8, 32768) == (1024, 32)
    # a small batch gets shorter chunks, about one item per CU: 1 x 8 kv heads
    # x 4096 tokens over 256 CUs -> 128-token chunks, 32 per sequence
    s, n = attn.attn_decode_plan(1, 8, 4096)
    assert s == 128 and n == 32
    assert attn.attn_decode_plan(4, 8, 4096) == (512, 8)
    assert attn.attn_decode_plan(1, 1, 0) == (64, 1)
    # forced chunk lengths round up to a multiple of 64
    assert attn.attn_decode_plan(4, 4, 1000, requested_split=100) == (128, 8)
    for B, H, L in ((1, 1, 1), (3, 5, 777), (64, 32, 1024), (256, 8, 131072)):
        s, n = attn.attn_decode_plan(B, H, L)
        assert s % 64 == 0 and 64 <= s <= 1024
        assert (n - 1) * s < max(L, 1) <= n * s
    with pytest.raises(attn.AttnError):
        attn.attn_decode_plan(1, 0, 10)


def test_workspace_bytes(lib):
    assert attn.attn_decode_workspace_bytes(4, 8, 8, 128, 512, 512) == 0   # one chunk: none
    assert attn.attn_decode_workspace_bytes(4, 8, 8, 128, 512) > 0        # small batch: split
    B, Hq, D = 32, 32, 128
    s, n = attn.attn_decode_plan(B, 32, 8192)
    rows = B * Hq * n
    expect = -(-rows * D * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    assert attn.attn_decode_workspace_bytes(B, Hq, 32, D, 8192) == expect


def test_shared_prefix_workspace(lib):
    # 64 requests x 32 heads over a 4096-token prefix: 4 chunks of 1024 keys
    # (32 kv heads x two blocks of 32 rows x 4 chunks: one item per CU)
    n = attn.attn_shared_prefix_workspace_bytes(64, 32, 32, 128, 4096, 0)
    rows = 64 * 32 * 4
    assert n == -(-rows * 128 * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    assert attn.attn_shared_prefix_workspace_bytes(64, 32, 32, 128, 0, 0) == 0
    assert attn.attn_shared_prefix_workspace_bytes(64, 32, 5, 128, 4096, 0) == 0  # bad group


def flat_gemm(lib, ws=None, ws_bytes=0, splits=0, rows=0, **kw):
    a = dict(a=FAKE, w=FAKE, c=FAKE, m=4, n=64, k=256, dt=0, cdt=0)
    a.update(kw)
    opts = ctypes.byref(attn.FlatGemmOpts(splits, rows))
    return lib.attn_flat_gemm(a["a"], a["w"], a["c"], a["m"], a["n"], a["k"], a["dt"], a["cdt"],
                              ws, ws_bytes, None, opts)


def test_flat_gemm_checks(lib):
    assert flat_gemm(lib, a=None) == E_NULL
    assert flat_gemm(lib, w=None) == E_NULL
    assert flat_gemm(lib, c=None) == E_NULL
    assert flat_gemm(lib, m=-1) == E_SHAPE
    assert flat_gemm(lib, n=-1) == E_SHAPE
    assert flat_gemm(lib, k=-8) == E_SHAPE
    assert flat_gemm(lib, splits=-1) == E_SHAPE
    assert flat_gemm(lib, rows=-16) == E_SHAPE
    assert flat_gemm(lib, rows=48) == E_UNSUP
    opts16 = ctypes.byref(attn.FlatGemmOpts(0, 0, 16))
    assert lib.attn_flat_gemm(FAKE, FAKE, FAKE, 4, 64, 256, 0, 0, None, 0, None, opts16) == E_UNSUP
    assert flat_gemm(lib, m=65) == E_UNSUP          # prefill-size m: a conventional GEMM
    assert flat_gemm(lib, k=100) == E_UNSUP         # k not a multiple of 8
    assert flat_gemm(lib, k=(1 << 22) + 8) == E_UNSUP
    assert flat_gemm(lib, dt=1) == E_UNSUP          # fp32 inputs
    assert flat_gemm(lib, cdt=2) == E_UNSUP
    assert flat_gemm(lib, a=ctypes.c_void_p(0x1008)) == E_ARG
    assert flat_gemm(lib, c=ctypes.c_void_p(0x1002)) == E_ARG
    # k slices need a workspace for their partials
    assert flat_gemm(lib, splits=4) == E_WS
    opts = ctypes.byref(attn.FlatGemmOpts(4, 0))
    need = lib.attn_flat_gemm_workspace_bytes(4, 64, 256, opts)
    assert need == -(-4 * 4 * 64 * 4 // 256) * 256
    assert flat_gemm(lib, splits=4, ws=FAKE, ws_bytes=need - 1) == E_WS
    # empty outputs are a no-op, even with NULL pointers
    assert flat_gemm(lib, a=None, w=None, c=None, m=0) == OK
    assert flat_gemm(lib, a=None, w=None, c=None, n=0) == OK


def test_flat_gemm_plan(lib):
    plan = attn.attn_flat_gemm_plan
    R, L = attn.FG_REGISTER, attn.FG_LDS
    proj = ((12288, 4096), (4096, 4096), (22016, 4096), (4096, 11008))   # qkv, o, gate_up, down
    # m < 8: register-streaming, 16 rows per workgroup.  qkv, o and down
    # have 256..768 row blocks: one round of resident 4-wavefront
    # workgroups, no k slices and no workspace; gate_up's 1376 fill 1.3
    # rounds, so k is sliced 4 ways
    for m in (1, 7):
        assert [plan(m, n, k) for n, k in proj] == [(1, 16, R), (1, 16, R), (4, 16, R), (1, 16, R)]
        assert attn.attn_flat_gemm_workspace_bytes(m, 4096, 4096) == 0
    # LDS-tiled for m > 16, and for m >= 8 on weights above 2^24 elements:
    # 64 rows (128 on gate_up, n >= 16384), k slices doubled until the grid
    # holds two workgroups per CU: qkv 192 tiles x 4, o and down 64 x 8,
    # gate_up 172 x 4.  The 2^24-element o weight at m = 8 / 16 stays on the
    # register-streaming kernel (16 rows)
    for m in (8, 16):
        assert [plan(m, n, k) for n, k in proj] == [(4, 64, L), (1, 16, R), (4, 128, L), (8, 64, L)]
    for m in (17, 32, 48, 64):
        assert [plan(m, n, k) for n, k in proj] == [(4, 64, L), (8, 64, L), (4, 128, L), (8, 64, L)]
    # m = 16 on the register-streaming kernel: 64 rows, except on the o
    # weight; gate_up's 344 blocks of 64 rows are >= 1.25 per CU: 32 rows
    assert [plan(16, n, k, kernel=R) for n, k in proj] == [(1, 64, R), (1, 16, R), (1, 32, R),
                                                           (4, 64, R)]
    assert attn.attn_flat_gemm_workspace_bytes(64, 4096, 4096) == 8 * 64 * 4096 * 4
    # the register-streaming kernel forced at m = 64: 64 rows; 64 blocks of
    # them take 4 slices
    assert plan(64, 4096, 4096, kernel=R) == (4, 64, R)
    # a short, deep weight (16 row blocks of 16, 256 steps): slices double
    # while CUs stay idle and each wavefront keeps an 8-step batch
    assert plan(16, 256, 8192, rows_per_workgroup=16) == (8, 16, R)
    assert plan(16, 256, 8192, num_cus=16, rows_per_workgroup=16) == (1, 16, R)
    # 8 chunks of 64: at most 2 slices of 4 chunks (LDS-tiled); the
    # register-streaming kernel over 16 steps: 2 slices keep two 1-step
    # batches per wavefront
    assert plan(64, 4096, 512) == (2, 64, L)
    assert plan(64, 4096, 512, kernel=R) == (2, 64, R)
    # forced counts are clamped to the number of k steps (chunks)
    assert plan(4, 64, 256, splits=100) == (8, 16, R)
    assert plan(4, 64, 256, splits=3) == (3, 16, R)
    assert plan(40, 300, 2048, splits=64, rows_per_workgroup=64) == (32, 64, L)
    assert plan(1, 1, 0) == (1, 16, R)
    # rows above 64 select the LDS-tiled kernel; options it cannot take
    assert plan(40, 300, 2048, rows_per_workgroup=256)[1:] == (256, L)
    assert plan(1, 300, 2048, kernel=L) == (8, 64, L)     # forced at m = 1: 5 tiles x 8 slices
    for bad in (dict(kernel=L, rows_per_workgroup=32),
                dict(kernel=R, rows_per_workgroup=128), dict(kernel=3)):
        kw = dict(bad)
        m = kw.pop("m", 40)
        with pytest.raises(attn.AttnError):
            plan(m, 300, 2048, **kw)
    with pytest.raises(attn.AttnError):
        plan(40, 300, (1 << 20) + 8, kernel=L)
    with pytest.raises(attn.AttnError):
        plan(65, 64, 256)


def test_probe_checks(lib):
    assert lib.attn_probe_block_bytes() == 4096
    sink = ctypes.c_void_p(0x2000)
    assert lib.attn_probe_hbm_read(FAKE, None, -1, sink, None) == E_SHAPE
    assert lib.attn_probe_hbm_read(None, None, 0, None, None) == OK    # nothing to read
    assert lib.attn_probe_hbm_read(None, None, 4, sink, None) == E_NULL
    assert lib.attn_probe_hbm_read(FAKE, None, 4, None, None) == E_NULL
    assert lib.attn_probe_hbm_read(ctypes.c_void_p(0x1008), None, 4, sink, None) == E_ARG
    assert lib.attn_probe_hbm_read(FAKE, ctypes.c_void_p(0x3002), 4, sink, None) == E_ARG
