"""CPU checks of the C ABI: the library loads, exports every symbol include/mrope.h declares, and
rejects bad arguments on the host with the documented status, before anything reaches the GPU.
No call here passes validation, so nothing is launched."""
import ctypes
import os
import re

import pytest

from canvas_rope_rotary_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mrope.h")
OK, ARG, ALIGN, UNSUP, WS, HIP = range(6)
BF16, F32 = _lib.MROPE_BF16, _lib.MROPE_F32
A = 1 << 20            # a 16-byte (and 256-byte) aligned fake device address, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    decl = set(re.findall(r"^\w[\w \*]*?\b(mrope_\w+)\s*\(", open(HEADER).read(), re.M))
    assert decl == set(_lib.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def test_version_and_strings(lib):
    assert lib.mrope_abi_version() == 5
    for code, text in ((OK, "ok"), (ARG, "invalid argument"), (HIP, "HIP runtime error")):
        assert lib.mrope_status_string(code).decode() == text
    assert lib.mrope_status_string(99).decode() == "unknown status"


def test_workspace_bytes(lib):
    """Header, one status word per 512-token chunk, three words per 32-token part, three words per
    token; every region rounded up to 256 bytes."""
    r = lambda b: (b + 255) // 256 * 256
    for n in (0, 1, 31, 32, 64, 65, 511, 512, 513, 1 << 20, 3_000_001):
        chunks, parts = -(-n // 512), -(-n // 32)
        assert lib.mrope_workspace_bytes(n) == 256 + r(8 * chunks) + r(24 * parts) + r(24 * n), n


def test_test_hooks_round_trip(lib):
    prev = lib.mrope_set_test_hooks(_lib.HOOK_FUSED_SCAN_FIRST)
    try:
        assert lib.mrope_set_test_hooks(_lib.HOOK_SCAN_FALLBACK | 64) == _lib.HOOK_FUSED_SCAN_FIRST
        assert lib.mrope_set_test_hooks(0) == _lib.HOOK_SCAN_FALLBACK  # unknown bits are dropped
    finally:
        lib.mrope_set_test_hooks(prev)


def _apply(lib, **kw):
    a = dict(q=A, qt=2048, qh=256, nq=8, k=A, kt=512, kh=256, nk=2, n=100, hd=256, rot=64, dt=BF16, planes=A,
             ps=100, theta=1e7, qo=None, ko=None)
    a.update(kw)
    return lib.mrope_apply(a["q"], a["qt"], a["qh"], a["nq"], a["k"], a["kt"], a["kh"], a["nk"], a["n"], a["hd"],
                           a["rot"], a["dt"], a["planes"], a["ps"], a["theta"], a["qo"], a["ko"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rot=32), UNSUP), (dict(hd=60), UNSUP), (dict(hd=260), UNSUP), (dict(hd=2048), UNSUP),
    (dict(dt=7), UNSUP), (dict(nq=65), UNSUP), (dict(nk=-1), UNSUP),
    (dict(n=-1), ARG), (dict(q=None), ARG), (dict(k=None), ARG), (dict(planes=None), ARG), (dict(ps=99), ARG),
    (dict(theta=0.0), ARG), (dict(theta=float("nan")), ARG), (dict(theta=float("inf")), ARG),
    (dict(qo=A), ARG), (dict(ko=A), ARG), (dict(qt=-8), ARG),
    (dict(q=A + 8), ALIGN), (dict(k=A + 4), ALIGN), (dict(qt=2044), ALIGN), (dict(kh=252), ALIGN),
    (dict(dt=F32, qt=2050), ALIGN),
])
def test_apply_validation(lib, kw, code):
    assert _apply(lib, **kw) == code
    assert lib.mrope_last_error().decode() != ""


def test_apply_nothing_to_do(lib):
    assert _apply(lib, n=0) == OK
    assert _apply(lib, nq=0, nk=0) == OK


def _planes(lib, **kw):
    a = dict(ids=A, cu=A, ns=4, n=1000, marker=248078, fl=0, planes=A, ps=1000, ws=A, wsb=10 ** 6)
    a.update(kw)
    return lib.mrope_planes(a["ids"], a["cu"], a["ns"], a["n"], a["marker"], a["fl"], None, None, None, a["planes"], a["ps"], None,
                            None, None, None, a["ws"], a["wsb"], 1, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ns=-1), ARG), (dict(n=-1), ARG), (dict(ns=0), ARG), (dict(cu=None), ARG), (dict(ids=None), ARG),
    (dict(planes=None), ARG), (dict(ps=999), ARG), (dict(n=1 << 31), ARG),
    (dict(ws=None), WS), (dict(ws=A + 64), WS), (dict(wsb=256 + 8 * 15), WS), (dict(wsb=24 * 1000), WS),
    (dict(fl=64), ARG), (dict(fl=-1), ARG), (dict(fl=4097), ARG),
])
def test_planes_validation(lib, kw, code):
    assert _planes(lib, **kw) == code


def test_planes_empty_is_ok(lib):
    assert _planes(lib, ns=0, n=0, ws=None) == OK


def test_workspace_init_validation(lib):
    assert lib.mrope_workspace_init(None, 1024, None) == WS
    assert lib.mrope_workspace_init(A + 128, 1024, None) == WS
    assert lib.mrope_workspace_init(A, 100, None) == WS


_CACHE = dict(kc=A, vc=None, slots=A, bs=16, nb=64, cb=8192, ct=512, ch=256)


def _cache_args(a):
    return (a["kc"], a["vc"], a["slots"], a["bs"], a["nb"], a["cb"], a["ct"], a["ch"])


def _decode(lib, **kw):
    a = dict(q=A, qt=2048, qh=256, nq=8, k=A, kt=512, kh=256, nk=2, v=None, vt=512, vh=256, ns=16, pos=A, am=A,
             hd=256, rot=64, dt=BF16, theta=1e7, **_CACHE)
    a.update(kw)
    return lib.mrope_decode(a["q"], a["qt"], a["qh"], a["nq"], a["k"], a["kt"], a["kh"], a["nk"], a["v"], a["vt"],
                            a["vh"], a["ns"], a["pos"], a["am"], *_cache_args(a), a["hd"], a["rot"], a["dt"],
                            a["theta"], None)


_PAGED_CASES = [
    (dict(kc=None), ARG), (dict(slots=None), ARG), (dict(bs=0), ARG), (dict(nb=-1), ARG), (dict(ct=-512), ARG),
    (dict(kc=A + 2), ALIGN), (dict(ch=260), ALIGN), (dict(cb=8190), ALIGN), (dict(ch=128), ARG),
    (dict(v=A), ARG), (dict(vc=A), ARG), (dict(v=A, vc=A + 8), ALIGN), (dict(v=A + 8, vc=A), ALIGN),
    (dict(v=A, vc=A, vh=260), ALIGN), (dict(v=A, vc=A, vh=128), ARG), (dict(v=A, vc=A, vt=-8), ARG),
]


@pytest.mark.parametrize("kw,code", [
    (dict(pos=None), ARG), (dict(am=None), ARG), (dict(rot=128), UNSUP), (dict(theta=-1.0), ARG),
    (dict(ns=-1), ARG),
] + _PAGED_CASES)
def test_decode_validation(lib, kw, code):
    assert _decode(lib, **kw) == code


def test_decode_nothing_to_do(lib):
    assert _decode(lib, ns=0) == OK


def _apply_kv(lib, **kw):
    a = dict(q=A, qt=2048, qh=256, nq=8, k=A, kt=512, kh=256, nk=2, v=A, vt=512, vh=256, n=100, hd=256, rot=64,
             dt=BF16, planes=A, ps=100, theta=1e7, **_CACHE)
    a["vc"] = A
    a.update(kw)
    return lib.mrope_apply_kv(a["q"], a["qt"], a["qh"], a["nq"], a["k"], a["kt"], a["kh"], a["nk"], a["v"], a["vt"],
                              a["vh"], a["n"], a["hd"], a["rot"], a["dt"], a["planes"], a["ps"], a["theta"],
                              *_cache_args(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(planes=None), ARG), (dict(ps=99), ARG), (dict(rot=32), UNSUP), (dict(q=A + 8), ALIGN),
    (dict(v=None), ARG), (dict(vc=None), ARG),
] + [(kw, c) for kw, c in _PAGED_CASES if "v" not in kw and "vc" not in kw])
def test_apply_kv_validation(lib, kw, code):
    assert _apply_kv(lib, **kw) == code


def test_apply_kv_nothing_to_do(lib):
    assert _apply_kv(lib, n=0) == OK
    assert _apply_kv(lib, nq=0, nk=0, kc=None, slots=None) == OK


def _apply_ids_kv(lib, **kw):
    a = dict(q=A, qt=2048, qh=256, nq=8, k=A, kt=512, kh=256, nk=2, v=A, vt=512, vh=256, n=1000, hd=256, rot=64,
             dt=BF16, theta=1e7, ids=A, cu=A, ns=4, marker=248078, fl=0, ws=A, wsb=10 ** 6, **_CACHE)
    a["vc"] = A
    a.update(kw)
    return lib.mrope_apply_ids_kv(a["q"], a["qt"], a["qh"], a["nq"], a["k"], a["kt"], a["kh"], a["nk"], a["v"],
                                  a["vt"], a["vh"], a["n"], a["hd"], a["rot"], a["dt"], a["theta"], a["ids"], a["cu"],
                                  a["ns"], a["marker"], a["fl"], None, None, None, None, 0, None, None, None, None, a["ws"],
                                  a["wsb"], 1, *_cache_args(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(ids=None), ARG), (dict(cu=None), ARG), (dict(ws=None), WS), (dict(wsb=100), WS), (dict(dt=9), UNSUP),
    (dict(fl=30), ARG),
] + [(kw, c) for kw, c in _PAGED_CASES if "v" not in kw and "vc" not in kw])
def test_apply_ids_kv_validation(lib, kw, code):
    assert _apply_ids_kv(lib, **kw) == code


def test_product_path_never_touches_the_oracle():
    """The package (binding, kernels, build) neither imports nor calls the oracle, nor links it."""
    pkg = os.path.join(ROOT, "canvas_rope_rotary_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b|\boracle\.\w+\(|liboracle|mrope_oracle",
                                     src, re.M), f


def _apply_ids_noalloc(lib, **kw):
    a = dict(q=A, qt=2048, qh=256, nq=8, k=A, kt=512, kh=256, nk=2, n=1000, hd=256, rot=64, dt=BF16, theta=1e7,
             ids=A, cu=A, ns=4, marker=248078, fl=0, planes=None, ps=0)
    a.update(kw)
    return lib.mrope_apply_ids_noalloc(a["q"], a["qt"], a["qh"], a["nq"], a["k"], a["kt"], a["kh"], a["nk"], a["n"],
                                       a["hd"], a["rot"], a["dt"], a["theta"], None, None, a["ids"], a["cu"], a["ns"],
                                       a["marker"], a["fl"], None, None, None, a["planes"], a["ps"], None, None, None, None,
                                       None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=(1 << 20) + 1), WS), (dict(ids=None), ARG), (dict(cu=None), ARG), (dict(ns=0), ARG),
    (dict(rot=32), UNSUP), (dict(q=A + 8), ALIGN), (dict(theta=0.0), ARG), (dict(fl=30), ARG),
    (dict(planes=A, ps=999), ARG),
])
def test_apply_ids_noalloc_validation(lib, kw, code):
    """Rejected on the host before the first use of the static scratch (nothing is launched)."""
    assert _apply_ids_noalloc(lib, **kw) == code


def test_check_slots_flags_shared_slots():
    """The cache-writing calls' debug check: slots outside the cache never count; two tokens on one
    slot inside it do (torch operations only, so CPU tensors serve)."""
    import torch

    import canvas_rope_rotary_amd as mr

    mr.check_slots(torch.tensor([0, 5, 3, -1, -1, 64, 64, 2], dtype=torch.int64), 64)
    mr.check_slots(torch.tensor([], dtype=torch.int64), 64)
    with pytest.raises(ValueError, match="slot 3"):
        mr.check_slots(torch.tensor([0, 3, 7, 3], dtype=torch.int64), 64)
    with pytest.raises(ValueError):
        mr.check_slots(torch.tensor([63, 1, 63], dtype=torch.int64), 64)
