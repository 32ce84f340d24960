"""CPU checks of the C ABI: the library loads, exports what include/hs2.h
declares, and rejects invalid arguments before enqueuing anything.

Only calls that fail host-side validation are made here (their contract is to
return before any HIP call), so no GPU is needed.  A pointer value such as
0x1000 below is never dereferenced: the call is rejected first.
"""

import ctypes
import os
import re

import pytest

import kv_cache_reuse_hs2_amd as hs2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hs2.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced
ODD = 0x10004   # misaligned


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"HS2_API\s+[\w\s\*]+?\b(hs2_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hs2.LIB_PATH):
        pytest.fail("libhs2.so is not built; run python -m kv_cache_reuse_hs2_amd.build_lib")
    return hs2.load()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(hs2.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    # nothing beyond the C API is exported
    out = os.popen(f"nm -D --defined-only {hs2.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert {n for n in exported if n.startswith("hs2")} == set(_declared())
    assert not any("launch" in n for n in exported)


def test_status_strings(lib):
    for code in range(6):
        s = hs2.hs2_status_string(code)
        assert s.startswith(["HS2_OK", "HS2_EINVAL", "HS2_EUNSUPPORTED", "HS2_EALIGN",
                             "HS2_EWORKSPACE", "HS2_EHIP"][code])
    assert "unknown" in hs2.hs2_status_string(99)


def _desc(**kw):
    base = dict(batch=4, n_heads=32, n_q=1, tile_q=1, k_top=1024, window=128, dtype=hs2.HS2_BF16)
    base.update(kw)
    return hs2.make_desc(**base)


def test_workspace_size(lib):
    n = hs2.hs2_workspace_size(_desc(), 262144)
    assert n > 0
    # grows with the capacity, is rejected for invalid descriptors
    assert hs2.hs2_workspace_size(_desc(), 1 << 20) > n
    assert hs2.hs2_workspace_size(_desc(head_dim=64), 4096) == 0
    assert hs2.hs2_workspace_size(_desc(), 0) == 0
    assert lib.hs2_workspace_size(None, 4096) == 0


def _scores(desc, *, q=FAKE, k=FAKE, stride=4096 * 128, ctx=FAKE, cap=4096, sc=FAKE, of=None,
            v=None, lse=None, ws=FAKE, nbytes=1 << 30):
    return hs2.load().hs2_full_attn_scores(ctypes.byref(desc) if desc is not None else None, q, k,
                                           v, stride, ctx, cap, sc, of, lse, ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), hs2.HS2_EUNSUPPORTED),
    (dict(n_heads=33), hs2.HS2_EUNSUPPORTED),
    (dict(n_heads=0), hs2.HS2_EINVAL),
    (dict(batch=0), hs2.HS2_EINVAL),
    (dict(k_top=-1), hs2.HS2_EINVAL),
    (dict(window=-1), hs2.HS2_EINVAL),
    (dict(k_top=4096), hs2.HS2_EUNSUPPORTED),
    (dict(n_q=3, tile_q=2), hs2.HS2_EINVAL),
    (dict(causal=0), hs2.HS2_EUNSUPPORTED),
    (dict(sm_scale=0.0), hs2.HS2_EINVAL),
    (dict(sm_scale=float("inf")), hs2.HS2_EINVAL),
    (dict(dtype=7), hs2.HS2_EINVAL),
])
def test_invalid_descriptor(lib, kw, code):
    assert _scores(_desc(**kw)) == code


def test_invalid_pointers_sizes_and_workspace(lib):
    d = _desc()
    assert _scores(None) == hs2.HS2_EINVAL
    assert _scores(d, q=None) == hs2.HS2_EINVAL
    assert _scores(d, k=None) == hs2.HS2_EINVAL
    assert _scores(d, ctx=None) == hs2.HS2_EINVAL
    assert _scores(d, sc=None) == hs2.HS2_EINVAL
    assert _scores(d, of=FAKE) == hs2.HS2_EINVAL          # o_full needs v
    # o_full with every cache type and with prefill: validation still runs
    # first (none of these calls reaches a kernel)
    f32 = _desc(dtype=hs2.HS2_F32)
    assert _scores(f32, of=FAKE, v=FAKE,
                   nbytes=hs2.hs2_workspace_size(f32, 4096) - 1) == hs2.HS2_EWORKSPACE
    pf = _desc(batch=1, n_q=64, tile_q=64)
    assert _scores(pf, of=FAKE, stride=(4096 + 64) * 128) == hs2.HS2_EINVAL
    assert _scores(pf, of=FAKE, v=FAKE, stride=(4096 + 64) * 128,
                   nbytes=hs2.hs2_workspace_size(pf, 4096) - 1) == hs2.HS2_EWORKSPACE
    assert _scores(pf, of=ODD, v=FAKE, stride=(4096 + 64) * 128) == hs2.HS2_EALIGN
    assert _scores(d, of=ODD, v=FAKE) == hs2.HS2_EALIGN
    assert _scores(d, of=FAKE, v=ODD) == hs2.HS2_EALIGN
    assert _scores(d, cap=0) == hs2.HS2_EINVAL
    assert _scores(d, stride=4095 * 128) == hs2.HS2_EINVAL
    assert _scores(d, stride=4096 * 128 + 4) == hs2.HS2_EALIGN
    assert _scores(d, q=ODD) == hs2.HS2_EALIGN
    assert _scores(d, sc=ODD) == hs2.HS2_EALIGN
    assert _scores(d, lse=ODD) == hs2.HS2_EALIGN
    need = hs2.hs2_workspace_size(d, 4096)
    assert _scores(d, nbytes=need - 1) == hs2.HS2_EWORKSPACE
    assert _scores(d, ws=None, nbytes=need) == hs2.HS2_EINVAL
    assert _scores(d, ws=ODD, nbytes=need) == hs2.HS2_EALIGN


def test_select_and_sparse_validation(lib):
    d = _desc()
    L = hs2.load()
    need = hs2.hs2_workspace_size(d, 4096)
    sel = lambda **kw: L.hs2_select_topk_window(  # noqa: E731
        ctypes.byref(d), kw.get("sc", FAKE), kw.get("ctx", FAKE), kw.get("cap", 4096),
        kw.get("ti", FAKE), kw.get("tc", FAKE), kw.get("ws", FAKE), kw.get("nb", need), None)
    assert sel(sc=None) == hs2.HS2_EINVAL
    assert sel(tc=None) == hs2.HS2_EINVAL
    assert sel(ti=None) == hs2.HS2_EINVAL
    assert sel(cap=0) == hs2.HS2_EINVAL
    assert sel(ti=ODD) == hs2.HS2_EALIGN
    assert sel(nb=need - 1) == hs2.HS2_EWORKSPACE
    sp = lambda **kw: L.hs2_sparse_attn_gather(  # noqa: E731
        ctypes.byref(d), kw.get("q", FAKE), FAKE, kw.get("v", FAKE), kw.get("st", 4096 * 128),
        FAKE, 4096, FAKE, FAKE, kw.get("o", FAKE), None, FAKE, kw.get("nb", need), None)
    assert sp(v=None) == hs2.HS2_EINVAL
    assert sp(o=None) == hs2.HS2_EINVAL
    assert sp(q=ODD) == hs2.HS2_EALIGN
    assert sp(st=100) == hs2.HS2_EINVAL
    assert sp(nb=0) == hs2.HS2_EWORKSPACE


def test_decode_step_validation(lib):
    d = _desc()
    L = hs2.load()
    need = hs2.hs2_workspace_size(d, 4096)
    st = lambda **kw: L.hs2_decode_step(  # noqa: E731
        ctypes.byref(d), kw.get("q", FAKE), kw.get("q2", None), FAKE, kw.get("v", FAKE),
        kw.get("st", 4096 * 128), FAKE, kw.get("cap", 4096), kw.get("sc", FAKE), None,
        kw.get("ti", FAKE), FAKE, kw.get("o", FAKE), None, FAKE, kw.get("nb", need), None)
    assert st(v=None) == hs2.HS2_EINVAL
    assert st(sc=None) == hs2.HS2_EINVAL
    assert st(o=None) == hs2.HS2_EINVAL
    assert st(ti=None) == hs2.HS2_EINVAL
    assert st(q2=ODD) == hs2.HS2_EALIGN
    assert st(nb=need - 1) == hs2.HS2_EWORKSPACE
    big = (1 << 22) + 1
    assert st(cap=big, st=big * 128) == hs2.HS2_EUNSUPPORTED
    assert hs2.hs2_workspace_size(d, big) == 0


@pytest.mark.parametrize("packed", [False, True])
def test_bridge_validation(lib, packed):
    L = hs2.load()

    def br(**kw):
        args = (kw.get("h", FAKE), kw.get("ldh", 2048))
        tail = (kw.get("ko", FAKE), kw.get("vo", FAKE), kw.get("ldkv", 128), kw.get("M", 1024),
                kw.get("dm", 2048), kw.get("hd", 128), None)
        if packed:
            return L.hs2_bridge_kv_packed(*args, kw.get("wk", FAKE), *tail)
        return L.hs2_bridge_kv(*args, kw.get("wk", FAKE), kw.get("wv", FAKE), *tail)

    assert br(h=None) == hs2.HS2_EINVAL
    assert br(wk=None) == hs2.HS2_EINVAL
    assert br(vo=None) == hs2.HS2_EINVAL
    assert br(M=0) == hs2.HS2_EINVAL
    assert br(ldh=1024) == hs2.HS2_EINVAL
    assert br(ldkv=64) == hs2.HS2_EINVAL
    assert br(hd=64, ldkv=128) == hs2.HS2_EUNSUPPORTED
    assert br(dm=100, ldh=2048) == hs2.HS2_EUNSUPPORTED
    assert br(ldh=2052) == hs2.HS2_EALIGN
    assert br(h=ODD) == hs2.HS2_EALIGN
    assert br(wk=ODD) == hs2.HS2_EALIGN
    assert br(ko=ODD) == hs2.HS2_EALIGN
    if not packed:
        assert br(wv=None) == hs2.HS2_EINVAL
        assert br(wv=ODD) == hs2.HS2_EALIGN


def test_bridge_pack_validation(lib):
    L = hs2.load()
    pk = lambda **kw: L.hs2_bridge_pack_weights(  # noqa: E731
        kw.get("wk", FAKE), FAKE, kw.get("dm", 2048), kw.get("hd", 128), kw.get("wp", FAKE), None)
    assert pk(wk=None) == hs2.HS2_EINVAL
    assert pk(wp=None) == hs2.HS2_EINVAL
    assert pk(dm=0) == hs2.HS2_EINVAL
    assert pk(dm=96) == hs2.HS2_EUNSUPPORTED
    assert pk(hd=64) == hs2.HS2_EUNSUPPORTED
    assert pk(wp=ODD) == hs2.HS2_EALIGN
    # [W_K | W_V] in bfloat16: d_model x 256 x 2 bytes
    assert hs2.hs2_bridge_packed_bytes(2048) == 2048 * 256 * 2
    assert hs2.hs2_bridge_packed_bytes(64) == 64 * 256 * 2
    assert hs2.hs2_bridge_packed_bytes(96) == 0
    assert hs2.hs2_bridge_packed_bytes(2048, 64) == 0


def test_binding_raises_on_error_status(lib):
    with pytest.raises(hs2.HS2Error) as ei:
        hs2.hs2_bridge_kv(None, 2048, FAKE, FAKE, FAKE, FAKE, 128, 1024, 2048, stream=0)
    assert ei.value.status == hs2.HS2_EINVAL


def test_sparse_layers_validation(lib):
    L = hs2.load()
    d = hs2.make_desc(batch=2, n_heads=32, k_top=1024, window=128)
    need = hs2.hs2_sparse_layers_workspace_size(d, 4)
    assert need > 0
    assert hs2.hs2_sparse_layers_workspace_size(d, 0) == 0
    assert hs2.hs2_sparse_layers_workspace_size(d, 65) == 0

    def call(desc=d, nl=4, q=FAKE, o=FAKE, ws=FAKE, nb=need, cap=4096, st=4096 * 128):
        return L.hs2_sparse_attn_gather_layers(ctypes.byref(desc), nl, q, FAKE, FAKE, st, FAKE,
                                               cap, FAKE, FAKE, o, None, ws, nb, None)

    assert call(q=None) == hs2.HS2_EINVAL
    assert call(o=None) == hs2.HS2_EINVAL
    assert call(nl=0) == hs2.HS2_EINVAL
    assert call(nl=65) == hs2.HS2_EUNSUPPORTED
    assert call(desc=hs2.make_desc(batch=2, n_heads=32, k_top=1024, window=128,
                                   dtype=hs2.HS2_F32)) == hs2.HS2_EUNSUPPORTED
    assert call(desc=hs2.make_desc(batch=1, n_heads=32, n_q=64, tile_q=64, k_top=1024,
                                   window=128)) == hs2.HS2_EUNSUPPORTED
    assert call(q=ODD) == hs2.HS2_EALIGN
    assert call(nb=need - 1) == hs2.HS2_EWORKSPACE
    assert call(ws=None) == hs2.HS2_EINVAL


def test_fp8_descriptor_validation(lib):
    fp8 = dict(dtype=hs2.HS2_FP8_E4M3, k_scale=0.01, v_scale=0.02)
    d = _desc(**fp8)
    assert hs2.hs2_workspace_size(d, 4096) > 0
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _scores(_desc(**dict(fp8, k_scale=bad))) == hs2.HS2_EINVAL
        assert _scores(_desc(**dict(fp8, v_scale=bad))) == hs2.HS2_EINVAL
    # scales are ignored for the other storage types
    assert hs2.hs2_workspace_size(_desc(k_scale=0.0, v_scale=float("nan")), 4096) > 0
    # decode and chunked prefill (tiles of a multiple of 16 queries)
    assert hs2.hs2_workspace_size(_desc(n_q=64, tile_q=64, **fp8), 4096) > 0
    assert _scores(_desc(n_q=2, tile_q=1, **fp8)) == hs2.HS2_EUNSUPPORTED
    assert _scores(_desc(n_q=8, tile_q=8, **fp8)) == hs2.HS2_EUNSUPPORTED
    # rows of 128 bytes stay 16-byte aligned only with a stride multiple of 16
    assert _scores(d, stride=4096 * 128 + 8) == hs2.HS2_EALIGN
    # (bf16 accepts that stride: the call gets as far as the workspace check)
    assert _scores(_desc(), stride=4096 * 128 + 8, nbytes=0) == hs2.HS2_EWORKSPACE


def test_block_selection_validation(lib):
    L = hs2.load()
    d = _desc(k_top=1024)
    need = hs2.hs2_workspace_size(d, 4096)

    def sel(desc=d, block=64, cap=4096, sc=FAKE, ti=FAKE, tc=FAKE, nb=need):
        return L.hs2_select_topk_blocks(ctypes.byref(desc), block, sc, FAKE, cap, ti, tc, FAKE,
                                        nb, None)

    for bad in (0, -64, 3, 48, 128):
        assert sel(block=bad) == hs2.HS2_EINVAL
    assert sel(desc=_desc(k_top=1000)) == hs2.HS2_EINVAL      # not a multiple of 64
    assert sel(sc=None) == hs2.HS2_EINVAL
    assert sel(ti=None) == hs2.HS2_EINVAL
    assert sel(cap=0) == hs2.HS2_EINVAL
    assert sel(tc=ODD) == hs2.HS2_EALIGN
    assert sel(nb=need - 1) == hs2.HS2_EWORKSPACE
    # at most 65,536 blocks per row
    big = 65536 * 4 + 1
    assert sel(block=4, cap=big, nb=1 << 40) == hs2.HS2_EUNSUPPORTED

    def step(block=64, nb=need, v=FAKE, st=4096 * 128):
        return L.hs2_decode_step_blocks(ctypes.byref(d), block, FAKE, None, FAKE, v, st, FAKE,
                                        4096, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, nb, None)

    assert step(block=5) == hs2.HS2_EINVAL
    assert step(v=None) == hs2.HS2_EINVAL
    assert step(st=100) == hs2.HS2_EINVAL
    assert step(nb=need - 1) == hs2.HS2_EWORKSPACE


def test_swa_validation(lib):
    L = hs2.load()

    def call(desc=None, q=FAKE, o=FAKE, lse=None, st=4096 * 128, cap=4096, odt=hs2.HS2_F32):
        d = desc if desc is not None else hs2.make_desc(batch=1, n_heads=32, n_q=64, k_top=0,
                                                         window=128)
        return L.hs2_swa_attention(ctypes.byref(d), q, FAKE, FAKE, st, FAKE, cap, o, odt, lse,
                                   None)

    mk = lambda **kw: hs2.make_desc(**dict(dict(batch=1, n_heads=32, n_q=64, k_top=0,  # noqa: E731
                                                window=128), **kw))
    assert L.hs2_swa_attention(None, FAKE, FAKE, FAKE, 4096 * 128, FAKE, 4096, FAKE, 0, None,
                               None) == hs2.HS2_EINVAL
    assert call(odt=hs2.HS2_FP8_E4M3) == hs2.HS2_EINVAL
    assert call(odt=9) == hs2.HS2_EINVAL
    assert call(desc=mk(window=0)) == hs2.HS2_EINVAL
    assert call(desc=mk(n_q=0)) == hs2.HS2_EINVAL
    assert call(desc=mk(sm_scale=-1.0)) == hs2.HS2_EINVAL
    assert call(desc=mk(dtype=hs2.HS2_F32)) == hs2.HS2_EUNSUPPORTED
    assert call(desc=mk(head_dim=64)) == hs2.HS2_EUNSUPPORTED
    assert call(desc=mk(n_heads=40)) == hs2.HS2_EUNSUPPORTED
    assert call(q=None) == hs2.HS2_EINVAL
    assert call(o=None) == hs2.HS2_EINVAL
    assert call(cap=0) == hs2.HS2_EINVAL
    assert call(st=100) == hs2.HS2_EINVAL
    assert call(st=4096 * 128 + 4) == hs2.HS2_EALIGN
    assert call(lse=ODD) == hs2.HS2_EALIGN


def test_bridge_decode_validation(lib):
    L = hs2.load()

    def call(h=FAKE, ldh=2048, wp=FAKE, rows=4, dm=2048, hd=128, pos=FAKE, kc=FAKE, st=300 * 128,
             cap=300):
        return L.hs2_bridge_kv_decode(h, ldh, wp, rows, dm, hd, pos, kc, FAKE, st, cap, None)

    assert call(h=None) == hs2.HS2_EINVAL
    assert call(wp=None) == hs2.HS2_EINVAL
    assert call(pos=None) == hs2.HS2_EINVAL
    assert call(rows=0) == hs2.HS2_EINVAL
    assert call(ldh=1000) == hs2.HS2_EINVAL
    assert call(cap=0) == hs2.HS2_EINVAL
    assert call(st=100) == hs2.HS2_EINVAL
    assert call(dm=96, ldh=96) == hs2.HS2_EUNSUPPORTED
    assert call(hd=64) == hs2.HS2_EUNSUPPORTED
    assert call(ldh=2052) == hs2.HS2_EALIGN
    assert call(st=300 * 128 + 4) == hs2.HS2_EALIGN
    assert call(kc=ODD) == hs2.HS2_EALIGN


def test_noalloc_step_rejects_before_any_hip_call(lib):
    # A problem whose workspace exceeds the library's 32 MiB array, and invalid
    # arguments, are refused on the host (fake pointers are never touched).
    def call(desc, cap=262144, q=FAKE, k=FAKE):
        return lib.hs2_decode_step_noalloc(ctypes.byref(desc), q, None, k, FAKE, cap * 128, FAKE,
                                           cap, FAKE, None, FAKE, FAKE, FAKE, None, None)

    big = _desc(batch=16)
    assert hs2.hs2_workspace_size(big, 262144) > 32 << 20
    assert call(big) == hs2.HS2_EWORKSPACE
    assert call(_desc(head_dim=64), cap=4096) == hs2.HS2_EUNSUPPORTED
    assert call(_desc(), cap=0) == hs2.HS2_EINVAL
    assert call(_desc(), cap=4096, q=ODD) == hs2.HS2_EALIGN
    assert call(_desc(), cap=4096, k=None) == hs2.HS2_EINVAL
