"""C-ABI library: loads, exports what include/mla.h declares, validates arguments (CPU only)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from mla_decode_attention_paged_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "mla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = B.lib()
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"libmla.so does not export {n}"
    assert B.abi_version() == 7


def test_status_strings():
    lib = B.lib()
    for s in range(6):
        assert lib.mla_status_string(s)
    assert lib.mla_status_string(99) == b"unknown status"


def _plan(batch=2, q_len=1, heads=16, page=64, lens=(100, 200), num_pages=None, maxp=None, out_fp32=False,
          num_cus=256, force=0, **kw):
    lens = np.asarray(lens, dtype=np.int32)
    if maxp is None:
        maxp = max([1] + [int((l + page - 1) // page) for l in lens])
    if num_pages is None:
        num_pages = int(sum((l + page - 1) // page for l in lens)) or 1
    prob = B.make_problem(batch, q_len, heads, page, num_pages, maxp, out_fp32=out_fp32, **kw)
    if batch == 0:   # the binding checks shapes first; go to the library directly
        h = C.c_void_p()
        st = B.lib().mla_plan(C.byref(prob), (C.c_int32 * 1)(), None, C.byref(h))
        raise B.MlaError(st, "mla_plan", B.last_error())
    return B.Plan(prob, lens, num_cus=num_cus, force_splits=force)


@pytest.mark.parametrize("kw,status", [
    (dict(heads=8), B.MLA_ERR_UNSUPPORTED),                 # R = 8
    (dict(heads=16, q_len=17), B.MLA_ERR_UNSUPPORTED),      # R = 272 > 256
    (dict(page=8), B.MLA_ERR_UNSUPPORTED),
    (dict(page=24), B.MLA_ERR_UNSUPPORTED),
    (dict(head_dim_qk=512), B.MLA_ERR_UNSUPPORTED),
    (dict(head_dim_v=576), B.MLA_ERR_UNSUPPORTED),
    (dict(batch=0, lens=()), B.MLA_ERR_INVALID_ARGUMENT),
    (dict(q_len=0), B.MLA_ERR_INVALID_ARGUMENT),
    (dict(lens=(100, -1)), B.MLA_ERR_INVALID_ARGUMENT),
    (dict(lens=(100, 200), maxp=2), B.MLA_ERR_INVALID_ARGUMENT),  # 200 > 2*64
    (dict(num_cus=-1), B.MLA_ERR_INVALID_ARGUMENT),
    (dict(force=-2), B.MLA_ERR_INVALID_ARGUMENT),
    (dict(causal=2), B.MLA_ERR_INVALID_ARGUMENT),
    (dict(causal=-1), B.MLA_ERR_INVALID_ARGUMENT),
])
def test_plan_rejects_bad_problems(kw, status):
    with pytest.raises(B.MlaError) as ei:
        _plan(**kw)
    assert ei.value.status == status
    assert B.last_error()


def test_plan_null_pointers():
    lib = B.lib()
    h = C.c_void_p()
    assert lib.mla_plan(None, None, None, C.byref(h)) == B.MLA_ERR_INVALID_ARGUMENT
    prob = B.make_problem(1, 1, 16, 64, 1, 1)
    assert lib.mla_plan(C.byref(prob), None, None, C.byref(h)) == B.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_plan(C.byref(prob), None, None, None) == B.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_plan_workspace_bytes(None) == 0
    lib.mla_plan_destroy(None)


def test_reserved_options_must_be_zero():
    lib = B.lib()
    prob = B.make_problem(1, 1, 16, 64, 1, 1)
    sl = (C.c_int32 * 1)(10)
    opt = B.mla_plan_options_t(256, 0)
    opt.reserved[3] = 1
    h = C.c_void_p()
    assert lib.mla_plan(C.byref(prob), sl, C.byref(opt), C.byref(h)) == B.MLA_ERR_INVALID_ARGUMENT


def test_decode_validation_happens_before_any_launch():
    """Bad arguments come back as status codes; nothing touches a device (none here)."""
    lib = B.lib()
    plan = _plan()
    h = plan.handle
    ws_bytes = plan.workspace_bytes
    fake = 1 << 20  # aligned non-null stand-in pointers; validation must reject before use
    call = lambda **o: lib.mla_decode_stages(
        h, o.get("q", fake), o.get("kv", fake), o.get("bt", fake), o.get("sl", fake), o.get("scale", 0.1),
        o.get("out", fake), o.get("lse", fake), o.get("ws", fake), o.get("wsb", ws_bytes), None, o.get("stages", 3))
    assert call(q=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(kv=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(out=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(ws=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(q=fake + 2) == B.MLA_ERR_INVALID_ARGUMENT          # misaligned
    assert call(ws=fake + 16) == B.MLA_ERR_INVALID_ARGUMENT        # workspace alignment
    assert call(wsb=ws_bytes - 1) == B.MLA_ERR_WORKSPACE_TOO_SMALL
    assert call(scale=float("nan")) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(stages=0) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(stages=8) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(stages=B.MLA_STAGE_COMBINED | B.MLA_STAGE_SPLIT) == B.MLA_ERR_INVALID_ARGUMENT
    # the combining launch runs the 16-row kernel only: refused for a 128-row plan before anything else
    wide = B.Plan(B.make_problem(2, 1, 128, 64, 16, 8), [300, 500], num_cus=256)
    assert wide.info()["rows_per_group"] == 128
    assert lib.mla_decode_stages(wide.handle, fake, fake, fake, fake, 0.1, fake, fake, fake, wide.workspace_bytes,
                                 None, B.MLA_STAGE_COMBINED) == B.MLA_ERR_UNSUPPORTED
    assert lib.mla_decode(None, fake, fake, fake, fake, 0.1, fake, fake, fake, ws_bytes, None) == \
        B.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_plan_upload(h, None, ws_bytes, None) == B.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_plan_upload(h, fake, ws_bytes - 1, None) == B.MLA_ERR_WORKSPACE_TOO_SMALL
    assert lib.mla_debug_gather(h, None, fake, fake, None) == B.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_read_status(None, None, None) == B.MLA_ERR_INVALID_ARGUMENT


def test_workspace_layout_scales_with_partials():
    p1 = _plan(lens=(4096,) * 16, batch=16, maxp=64)
    info = p1.info()
    R = 16
    assert info["workspace_bytes"] >= info["metadata_bytes"] + info["num_partials"] * R * (512 + 1) * 4
    assert info["workspace_bytes"] % 256 == 0


def test_devplan_validation():
    lib = B.lib()
    prob = B.make_problem(2, 1, 16, 64, 4, 2)
    assert lib.mla_devplan_workspace_bytes(C.byref(prob), 256) > 0
    assert lib.mla_devplan_workspace_bytes(C.byref(prob), -1) == 0
    bad = B.make_problem(2, 1, 8, 64, 4, 2)                 # R = 8
    assert lib.mla_devplan_workspace_bytes(C.byref(bad), 256) == 0
    n = lib.mla_devplan_workspace_bytes(C.byref(prob), 256)
    fake = 1 << 20
    # nothing launched for bad arguments (no device here)
    assert lib.mla_devplan_prepare(C.byref(prob), 256, None, n, None) == B.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_devplan_prepare(C.byref(prob), 256, fake, n - 1, None) == B.MLA_ERR_WORKSPACE_TOO_SMALL
    call = lambda **o: lib.mla_decode_devplan(
        C.byref(prob), o.get("w", 256), o.get("q", fake), fake, fake, fake, C.c_float(o.get("scale", 0.1)),
        fake, fake, o.get("ws", fake), o.get("n", n), None)
    assert call(q=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(q=fake + 8) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(ws=fake + 64) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(n=n - 256) == B.MLA_ERR_WORKSPACE_TOO_SMALL
    assert call(scale=float("nan")) == B.MLA_ERR_INVALID_ARGUMENT
    assert call(w=-3) == B.MLA_ERR_INVALID_ARGUMENT


def test_layer_step_validation():
    """Query preparation, cache append and output projection reject bad arguments before any launch."""
    lib = B.lib()
    prob = B.make_problem(2, 1, 16, 64, 4, 2)
    fake = 1 << 20
    qa = lambda **o: lib.mla_q_absorb(
        C.byref(o.get("p", prob)), o.get("qn", fake), o.get("qp", fake), o.get("w", fake), o.get("pos", fake),
        C.c_float(o.get("base", 10000.0)), o.get("out", fake), None)
    assert qa(qn=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert qa(pos=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert qa(qn=fake + 8) == B.MLA_ERR_INVALID_ARGUMENT
    assert qa(qp=fake + 2) == B.MLA_ERR_INVALID_ARGUMENT
    assert qa(base=0.0) == B.MLA_ERR_INVALID_ARGUMENT
    assert qa(base=float("inf")) == B.MLA_ERR_INVALID_ARGUMENT
    assert qa(p=B.make_problem(2, 1, 8, 64, 4, 2)) == B.MLA_ERR_UNSUPPORTED       # R = 8
    ap = lambda **o: lib.mla_kv_append(
        C.byref(o.get("p", prob)), o.get("c", fake), o.get("k", fake), o.get("pos", fake), o.get("bt", fake),
        C.c_float(o.get("base", 10000.0)), o.get("kv", fake), o.get("st", None), None)
    assert ap(c=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert ap(bt=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert ap(kv=fake + 4) == B.MLA_ERR_INVALID_ARGUMENT
    assert ap(st=fake + 2) == B.MLA_ERR_INVALID_ARGUMENT
    assert ap(base=-1.0) == B.MLA_ERR_INVALID_ARGUMENT
    assert ap(p=B.make_problem(2, 1, 16, 40, 4, 2)) == B.MLA_ERR_UNSUPPORTED      # page size
    oa = lambda **o: lib.mla_out_absorb(C.byref(o.get("p", prob)), o.get("lat", fake), o.get("w", fake),
                                        o.get("o", fake), None)
    assert oa(lat=None) == B.MLA_ERR_INVALID_ARGUMENT
    assert oa(o=fake + 8) == B.MLA_ERR_INVALID_ARGUMENT
    assert oa(w=fake + 2) == B.MLA_ERR_INVALID_ARGUMENT


def test_last_error_is_per_thread():
    """mla_last_error keeps one message per thread: two threads failing with different
    errors at the same time each read back their own."""
    import threading
    cases = [(B.make_problem(2, 1, 16, 24, 4, 2), "page_size must be a multiple of 16"),
             (B.make_problem(2, 1, 8, 64, 4, 2), "q_len*num_heads must be a multiple of 16")]
    bad = []

    def worker(prob, want):
        for _ in range(300):
            try:
                B.Plan(prob, np.array([10, 10], dtype=np.int32), num_cus=256)
            except B.MlaError:
                msg = B.last_error()
                if want not in msg:
                    bad.append(msg)
            except Exception as e:          # anything else fails the test, not just the thread
                bad.append(repr(e))
            else:
                bad.append("no error")

    threads = [threading.Thread(target=worker, args=c) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:3]


def test_every_declared_status_code_is_returned():
    """Each status code mla.h declares comes back from some call on this (GPU-less) host, before
    anything is launched."""
    import torch
    lib = B.lib()
    prob = B.make_problem(2, 1, 16, 64, 4, 2)
    sl = (C.c_int32 * 2)(100, 50)
    h = C.c_void_p()
    seen = {}
    opt = B.mla_plan_options_t(256, 0)
    seen[B.MLA_OK] = lib.mla_plan(C.byref(prob), sl, C.byref(opt), C.byref(h))
    n = lib.mla_plan_workspace_bytes(h)
    fake = 1 << 20
    bad = B.make_problem(2, 1, 8, 64, 4, 2)
    h2 = C.c_void_p()
    seen[B.MLA_ERR_UNSUPPORTED] = lib.mla_plan(C.byref(bad), sl, C.byref(opt), C.byref(h2))
    seen[B.MLA_ERR_INVALID_ARGUMENT] = lib.mla_plan(None, sl, C.byref(opt), C.byref(h2))
    seen[B.MLA_ERR_WORKSPACE_TOO_SMALL] = lib.mla_plan_upload(h, fake, n - 1, None)
    # a workspace that never received this plan's schedule: refused before any launch
    seen[B.MLA_ERR_PLAN_MISMATCH] = lib.mla_decode(h, fake, fake, fake, fake, C.c_float(0.1), fake, fake, fake, n,
                                                   None)
    assert "mla_plan_upload" in B.last_error()
    for code, got in seen.items():
        assert got == code, (code, got, B.last_error())
    if not torch.cuda.is_available():
        opt0 = B.mla_plan_options_t(0, 0)          # ask the (absent) device for its CU count
        assert lib.mla_plan(C.byref(prob), sl, C.byref(opt0), C.byref(h2)) == B.MLA_ERR_HIP
        assert "hipGetDevice" in B.last_error()
        assert lib.mla_plan_upload(h, fake, n, None) == B.MLA_ERR_HIP
        # a failed upload records nothing: the decode is still refused
        assert lib.mla_decode(h, fake, fake, fake, fake, C.c_float(0.1), fake, fake, fake, n, None) == \
            B.MLA_ERR_PLAN_MISMATCH
    declared = set(int(x) for x in re.findall(r"MLA_(?:OK|ERR_[A-Z_]+) = (\d+)", open(os.path.join(
        ROOT, "include", "mla.h")).read()))
    assert declared == set(range(6))
    lib.mla_plan_destroy(h)
