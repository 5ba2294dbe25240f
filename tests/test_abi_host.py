"""The C-ABI library loads, exports every symbol include/verkv.h declares, and rejects
bad arguments on the host before any GPU work (no compute calls; no GPU needed)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verkv.h")


@pytest.fixture(scope="module")
def vk():
    from long_context_decode_kvfetch_amd import build, verkv
    if not os.path.exists(verkv.LIB_PATH):
        build.build()
    elif not verkv.built_from_current_sources():
        # a library left from older sources: rebuild it here (CPU) before testing it
        verkv._LIB = None
        build.build()
    verkv._LIB = None
    return verkv


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(verkv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("verkv_compress", "verkv_decode_step", "verkv_refine",
              "verkv_compress_workspace_bytes", "verkv_decode_workspace_bytes"):
        assert n in names


def test_every_declared_symbol_is_exported(vk):
    lib = vk.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(vk):
    lib = vk.lib()
    assert lib.verkv_version() == 109
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert lib.verkv_status_str(st).decode() not in ("", "unknown status")
    assert lib.verkv_status_str(7).decode() == "unknown status"


def _shape(vk, lens=(4096,), hkv=1, g=8, dtype="f32", n_sink=4, n_local=64, head_dim=None):
    sh = vk.LayerShape(list(lens), hkv, g, n_sink, n_local, dtype)
    if head_dim is not None:
        sh.c.head_dim = head_dim
    return sh


def test_workspace_sizes(vk):
    a = _shape(vk).decode_workspace_bytes(640)
    b = _shape(vk, lens=(8192,)).decode_workspace_bytes(640)
    assert 0 < a < b and a % 256 == 0
    assert _shape(vk).compress_workspace_bytes() >= 2 * 8 * 4096
    assert _shape(vk, head_dim=64).decode_workspace_bytes(640) == 0
    assert _shape(vk, g=9).compress_workspace_bytes() == 0
    assert _shape(vk).decode_workspace_bytes(0) == 0
    # ragged batch grows with every sequence
    r1 = _shape(vk, lens=(1000, 3000), hkv=8, g=4, dtype="bf16").decode_workspace_bytes(512)
    r2 = _shape(vk, lens=(1000, 3000, 17), hkv=8, g=4, dtype="bf16").decode_workspace_bytes(512)
    assert r2 > r1


FAKE = 4096      # a non-null pointer value the host checks never dereference


def _fake_state(vk, cap=640):
    return vk.State(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, cap, FAKE, 1)


def _fake_out(vk):
    return vk.StepOut(*([FAKE] * 6), FAKE, 16, FAKE, FAKE, *([FAKE] * 5))


def test_decode_step_rejects_bad_arguments_on_host(vk):
    lib = vk.lib()
    sh = _shape(vk)
    st = _fake_state(vk)
    out = _fake_out(vk)
    big = 1 << 40

    def call(shape=sh, beta=1.0, eps=0.05, delta=0.05, state=st, q=FAKE, ws=FAKE, wsb=big):
        return lib.verkv_decode_step(C.byref(shape.c), C.byref(state), q, beta, eps, delta,
                                     C.byref(out), ws, wsb, None)

    assert call(eps=0.0) == vk.EINVAL
    assert call(eps=-1.0) == vk.EINVAL
    assert call(delta=0.0) == vk.EINVAL
    assert call(delta=1.0) == vk.EINVAL
    assert call(beta=-0.5) == vk.EINVAL
    assert call(beta=float("nan")) == vk.EINVAL
    assert call(q=None) == vk.EINVAL
    assert call(wsb=16) == vk.EWORKSPACE
    assert call(shape=_shape(vk, head_dim=64)) == vk.EUNSUPPORTED
    assert call(shape=_shape(vk, g=9)) == vk.EUNSUPPORTED
    assert call(shape=_shape(vk, lens=(0,))) == vk.EINVAL
    assert call(shape=_shape(vk, lens=((1 << 20) + 1,))) == vk.EUNSUPPORTED
    assert call(state=_fake_state(vk, cap=0)) == vk.EINVAL
    nostate = vk.State(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 640, 0, 1)  # no sketch
    assert call(state=nostate) == vk.EINVAL
    assert lib.verkv_decode_step(None, C.byref(st), FAKE, 1.0, 0.05, 0.05, C.byref(out), FAKE,
                                 big, None) == vk.EINVAL


def test_library_carries_the_hash_of_these_sources(vk):
    from long_context_decode_kvfetch_amd import build
    got = vk.lib().verkv_source_hash().decode()
    assert len(got) == 64 and got == build.source_hash()


def test_decode_step_rejects_pageable_value_cache_before_any_launch(vk):
    """A v_host that is neither pinned nor device memory is an argument error, found
    before the first kernel is enqueued (no GPU here, so every HIP call would fail: the
    call must return EINVAL from the pointer check, not EHIP from a launch)."""
    import ctypes
    lib = vk.lib()
    sh = _shape(vk)
    page = ctypes.create_string_buffer(1 << 16)          # ordinary pageable host memory
    st = vk.State(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 640, FAKE, 1,
                  ctypes.cast(page, ctypes.c_void_p).value, 0)
    out = _fake_out(vk)
    rc = lib.verkv_decode_step(C.byref(sh.c), C.byref(st), FAKE, 1.0, 0.05, 0.05, C.byref(out),
                               FAKE, 1 << 40, None)
    assert rc == vk.EINVAL


def test_compress_rejects_bad_arguments_on_host(vk):
    lib = vk.lib()
    st = _fake_state(vk)
    need = C.c_int32(-7)

    def call(shape, eta=0.125, state=st, wsb=1 << 40, tau=FAKE):
        return lib.verkv_compress(C.byref(shape.c), tau, FAKE, FAKE, eta, 0, C.byref(state),
                                  FAKE, wsb, C.byref(need), None)

    sh = _shape(vk)
    assert call(sh, eta=0.0) == vk.EINVAL
    assert call(sh, eta=1.5) == vk.EINVAL
    assert call(sh, eta=float("nan")) == vk.EINVAL
    assert call(sh, tau=None) == vk.EINVAL
    # eta * n below the 68 forced tokens
    assert call(sh, eta=60 / 4096) == vk.EBUDGET
    # budget check is per sequence of a ragged batch
    assert call(_shape(vk, lens=(4096, 100), dtype="bf16"), eta=0.5) == vk.EBUDGET
    assert call(sh, wsb=64) == vk.EWORKSPACE
    assert call(sh, state=_fake_state(vk, cap=0)) == vk.EINVAL


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from long_context_decode_kvfetch_amd import verkv
    monkeypatch.setattr(verkv, "_LIB", None)
    monkeypatch.setattr(verkv, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        verkv.lib()


def test_gather_rows_memcpy_checks_its_list_before_copying(vk):
    """The memcpy form of the host fetch rejects a bad list before it issues any copy
    (the pointers below are never dereferenced: no copy is enqueued)."""
    lib = vk.lib()
    import numpy as np
    runs = C.c_int64(-1)
    bad = np.array([3, 5, 5, 9], dtype=np.int32)
    st = lib.verkv_gather_rows_memcpy(C.c_void_p(16), 256, bad.ctypes.data_as(C.c_void_p), 4,
                                      C.c_void_p(16), C.byref(runs), None)
    assert st == vk.EINVAL and runs.value == 0
    assert "ascending" in lib.verkv_last_error().decode()
    neg = np.array([-1, 2], dtype=np.int32)
    assert lib.verkv_gather_rows_memcpy(C.c_void_p(16), 256, neg.ctypes.data_as(C.c_void_p), 2,
                                        C.c_void_p(16), None, None) == vk.EINVAL
    assert lib.verkv_gather_rows_memcpy(None, 256, None, 0, C.c_void_p(16), None, None) == vk.EINVAL
    assert lib.verkv_gather_rows_memcpy(C.c_void_p(16), 0, None, 0, C.c_void_p(16), None, None) == vk.EINVAL
    runs.value = -1
    assert lib.verkv_gather_rows_memcpy(C.c_void_p(16), 256, None, 0, C.c_void_p(16),
                                        C.byref(runs), None) == vk.OK
    assert runs.value == 0


def test_stage_slots_grow_the_workspace_within_the_packing_limit(vk):
    """A host-row list entry packs the token (the bits of the largest capacity) and its
    staging slot + 1 into 32 bits: 32768-token capacities leave 17 bits (131071 slots),
    2^20 leaves 12 (4095).  Beyond that the shape is refused (workspace size 0, and a
    decode step returns VERKV_EINVAL before any work)."""
    base = vk.LayerShape([32768], 8, 4, 4, 128, "bf16")
    big = vk.LayerShape([32768], 8, 4, 4, 128, "bf16", stage_slots=16384)
    limit = vk.LayerShape([32768], 8, 4, 4, 128, "bf16", stage_slots=131071)
    over = vk.LayerShape([32768], 8, 4, 4, 128, "bf16", stage_slots=131072)
    a, b, c = (x.decode_workspace_bytes(2624) for x in (base, big, limit))
    assert 0 < a < b < c
    # per slot and KV head: one bf16 row, its token, and the two plan entries (the default
    # is 8192 slots per KV head at this shape)
    assert b - a >= 8 * (16384 - 8192) * (256 + 3 * 4) - 4096
    assert over.decode_workspace_bytes(2624) == 0
    longest = vk.LayerShape([1 << 20], 1, 4, 4, 128, "bf16", stage_slots=4095)
    assert longest.decode_workspace_bytes(64) > 0
    assert vk.LayerShape([1 << 20], 1, 4, 4, 128, "bf16", stage_slots=4096).decode_workspace_bytes(64) == 0
    assert vk.LayerShape([1000], 1, 4, 4, 128, "bf16", stage_slots=-1).decode_workspace_bytes(64) == 0
    lib = vk.lib()
    st = _fake_state(vk, 2624)
    step = vk.StepOut()
    for name, _ in vk.StepOut._fields_:
        if name != "fetch_cap":
            setattr(step, name, FAKE)
    step.fetch_cap = 1
    rc = lib.verkv_decode_step(C.byref(over.c), C.byref(st), C.c_void_p(FAKE), 1.0, 0.05, 0.05,
                               C.byref(step), C.c_void_p(FAKE), 1 << 40, None)
    assert rc == vk.EINVAL
    assert "stage_slots" in lib.verkv_last_error().decode()


def test_staged_rows_checks_its_arguments_on_host(vk):
    """verkv_staged_rows refuses a null workspace or result and a workspace smaller than
    the step's layout before it touches the device."""
    lib = vk.lib()
    sh = _shape(vk)
    rows = C.c_int64(-1)
    need = sh.decode_workspace_bytes(640)
    assert lib.verkv_staged_rows(None, need, C.byref(sh.c), 640, None, C.byref(rows)) == vk.EINVAL
    assert lib.verkv_staged_rows(C.c_void_p(FAKE), need, C.byref(sh.c), 640, None, None) == vk.EINVAL
    assert lib.verkv_staged_rows(C.c_void_p(FAKE), need, C.byref(sh.c), 0, None, C.byref(rows)) == vk.EINVAL
    assert lib.verkv_staged_rows(C.c_void_p(FAKE), need - 1, C.byref(sh.c), 640, None,
                                 C.byref(rows)) == vk.EWORKSPACE
    assert rows.value == -1
