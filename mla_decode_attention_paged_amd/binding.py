"""ctypes binding of libmla.so (include/mla.h), with the same entry-point names.

Argument marshalling only: every step of the decode runs in the HIP library.
Torch supplies device memory and streams.  If the library is missing or does
not load, every call raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4
MLA_ERR_PLAN_MISMATCH = 5
MLA_DTYPE_BF16 = 0
MLA_DTYPE_FP32 = 1
MLA_KV_BF16 = 0
MLA_KV_FP8_E4M3 = 1
MLA_STAGE_SPLIT = 1
MLA_STAGE_MERGE = 2
MLA_STAGE_ALL = 3
MLA_STAGE_COMBINED = 4


class MlaError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: status {status} ({detail})")
        self.status = status


class mla_problem_t(C.Structure):
    _fields_ = [("batch", C.c_int32), ("q_len", C.c_int32), ("num_heads", C.c_int32),
                ("head_dim_qk", C.c_int32), ("head_dim_v", C.c_int32), ("page_size", C.c_int32),
                ("num_pages", C.c_int32), ("max_pages_per_seq", C.c_int32), ("out_dtype", C.c_int32),
                ("causal", C.c_int32), ("kv_dtype", C.c_int32)]


class mla_plan_options_t(C.Structure):
    _fields_ = [("num_cus", C.c_int32), ("force_splits", C.c_int32), ("rows_per_group", C.c_int32),
                ("reserved", C.c_int32 * 5)]


class mla_plan_info_t(C.Structure):
    _fields_ = [("num_workers", C.c_int32), ("grid_size", C.c_int32), ("num_segments", C.c_int32),
                ("num_partials", C.c_int32), ("num_combine", C.c_int32), ("rows_per_group", C.c_int32),
                ("row_groups", C.c_int32), ("granule", C.c_int32), ("max_worker_cost", C.c_int64),
                ("min_worker_cost", C.c_int64), ("metadata_bytes", C.c_int64), ("workspace_bytes", C.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lib = None

# name -> (restype, argtypes)
_SIGS = {
    "mla_plan": (C.c_int, [C.POINTER(mla_problem_t), C.POINTER(C.c_int32), C.POINTER(mla_plan_options_t),
                           C.POINTER(C.c_void_p)]),
    "mla_plan_get_info": (C.c_int, [C.c_void_p, C.POINTER(mla_plan_info_t)]),
    "mla_plan_get_segments": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int64, C.POINTER(C.c_int32),
                                        C.c_int64]),
    "mla_plan_workspace_bytes": (C.c_size_t, [C.c_void_p]),
    "mla_plan_upload": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "mla_decode": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_float, C.c_void_p,
                             C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "mla_decode_stages": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_float,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p, C.c_uint32]),
    "mla_debug_gather": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "mla_read_status": (C.c_int, [C.c_void_p, C.c_void_p, C.POINTER(C.c_int32)]),
    "mla_stream_probe": (C.c_int, [C.c_void_p, C.c_size_t, C.c_int32, C.c_void_p]),
    "mla_devplan_workspace_bytes": (C.c_size_t, [C.POINTER(mla_problem_t), C.c_int32]),
    "mla_devplan_prepare": (C.c_int, [C.POINTER(mla_problem_t), C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]),
    "mla_decode_devplan": (C.c_int, [C.POINTER(mla_problem_t), C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_float, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                     C.c_void_p]),
    "mla_decode_devplan_combined": (C.c_int, [C.POINTER(mla_problem_t), C.c_int32, C.c_void_p, C.c_void_p,
                                              C.c_void_p, C.c_void_p, C.c_float, C.c_void_p, C.c_void_p,
                                              C.c_void_p, C.c_size_t, C.c_void_p]),
    "mla_decode_devplan_noalloc": (C.c_int, [C.POINTER(mla_problem_t), C.c_int32, C.c_void_p, C.c_void_p,
                                             C.c_void_p, C.c_void_p, C.c_float, C.c_void_p, C.c_void_p,
                                             C.c_void_p]),
    "mla_q_absorb": (C.c_int, [C.POINTER(mla_problem_t), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                               C.c_float, C.c_void_p, C.c_void_p]),
    "mla_kv_append": (C.c_int, [C.POINTER(mla_problem_t), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                C.c_float, C.c_void_p, C.c_void_p, C.c_void_p]),
    "mla_out_absorb": (C.c_int, [C.POINTER(mla_problem_t), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "mla_plan_destroy": (None, [C.c_void_p]),
    "mla_status_string": (C.c_char_p, [C.c_int]),
    "mla_last_error": (C.c_char_p, []),
    "mla_abi_version": (C.c_int32, []),
}


def lib():
    """Load libmla.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mla_decode_attention_paged_amd.build`")
        l = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(status: int, func: str):
    if status != MLA_OK:
        detail = lib().mla_last_error().decode(errors="replace")
        raise MlaError(status, func, detail)


def last_error() -> str:
    return lib().mla_last_error().decode(errors="replace")


def abi_version() -> int:
    return lib().mla_abi_version()


def make_problem(batch, q_len, num_heads, page_size, num_pages, max_pages_per_seq, out_fp32=False,
                 head_dim_qk=576, head_dim_v=512, causal=False, kv_fp8=False) -> mla_problem_t:
    return mla_problem_t(batch, q_len, num_heads, head_dim_qk, head_dim_v, page_size, num_pages,
                         max_pages_per_seq, MLA_DTYPE_FP32 if out_fp32 else MLA_DTYPE_BF16, int(causal),
                         MLA_KV_FP8_E4M3 if kv_fp8 else MLA_KV_BF16)


class Plan:
    """Host-side split-KV schedule (mla_plan)."""

    def __init__(self, problem: mla_problem_t, cache_seqlens_host, num_cus: int = 0, force_splits: int = 0,
                 rows_per_group: int = 0):
        import numpy as np
        self.problem = problem
        sl = np.ascontiguousarray(np.asarray(cache_seqlens_host, dtype=np.int32))
        if sl.shape != (problem.batch,):
            raise ValueError(f"cache_seqlens_host must have shape ({problem.batch},), got {sl.shape}")
        self.seqlens = sl
        opt = mla_plan_options_t(num_cus, force_splits, rows_per_group)
        h = C.c_void_p()
        _check(lib().mla_plan(C.byref(problem), sl.ctypes.data_as(C.POINTER(C.c_int32)), C.byref(opt),
                              C.byref(h)), "mla_plan")
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def info(self) -> dict:
        inf = mla_plan_info_t()
        _check(lib().mla_plan_get_info(self.handle, C.byref(inf)), "mla_plan_get_info")
        return inf.as_dict()

    def segments(self):
        import numpy as np
        inf = self.info()
        seg = np.zeros(4 * max(1, inf["num_segments"]), dtype=np.int32)
        off = np.zeros(inf["num_workers"] + 1, dtype=np.int32)
        _check(lib().mla_plan_get_segments(self.handle, seg.ctypes.data_as(C.POINTER(C.c_int32)), seg.size,
                                           off.ctypes.data_as(C.POINTER(C.c_int32)), off.size),
               "mla_plan_get_segments")
        return seg[:4 * inf["num_segments"]].reshape(-1, 4), off

    @property
    def workspace_bytes(self) -> int:
        return int(lib().mla_plan_workspace_bytes(self.handle))

    def upload(self, workspace, stream=None):
        _check(lib().mla_plan_upload(self.handle, _ptr(workspace), _nbytes(workspace), _stream(stream)),
               "mla_plan_upload")

    def destroy(self):
        if self._h is not None:
            lib().mla_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require(t, name, dtypes, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def mla_decode(plan: Plan, q, kv_cache, block_table, cache_seqlens, softmax_scale, out, lse, workspace,
               stream=None, stages: int = MLA_STAGE_ALL):
    """Launch paged MLA decode (asynchronous on `stream`, default: torch's current stream)."""
    import torch
    p = plan.problem
    _require(q, "q", (torch.bfloat16,), (p.batch, p.q_len, p.num_heads, 576))
    _require(kv_cache, "kv_cache", *_kv_spec(p))
    _require(block_table, "block_table", (torch.int32,), (p.batch, p.max_pages_per_seq))
    _require(cache_seqlens, "cache_seqlens", (torch.int32,), (p.batch,))
    odt = torch.float32 if p.out_dtype == MLA_DTYPE_FP32 else torch.bfloat16
    _require(out, "out", (odt,), (p.batch, p.q_len, p.num_heads, 512))
    if lse is not None:
        _require(lse, "lse", (torch.float32,), (p.batch, p.q_len, p.num_heads))
    _require(workspace, "workspace", (torch.uint8,))
    _check(lib().mla_decode_stages(plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens),
                                   float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream), stages), "mla_decode")


class BoundDecode:
    """mla_decode_stages with every argument but the stream and the stage mask checked and
    marshalled once (the tensors must stay alive and in place while it is used)."""

    def __init__(self, plan: Plan, q, kv_cache, block_table, cache_seqlens, softmax_scale, out, lse, workspace):
        import torch
        p = plan.problem
        _require(q, "q", (torch.bfloat16,), (p.batch, p.q_len, p.num_heads, 576))
        _require(kv_cache, "kv_cache", *_kv_spec(p))
        _require(block_table, "block_table", (torch.int32,), (p.batch, p.max_pages_per_seq))
        _require(cache_seqlens, "cache_seqlens", (torch.int32,), (p.batch,))
        odt = torch.float32 if p.out_dtype == MLA_DTYPE_FP32 else torch.bfloat16
        _require(out, "out", (odt,), (p.batch, p.q_len, p.num_heads, 512))
        if lse is not None:
            _require(lse, "lse", (torch.float32,), (p.batch, p.q_len, p.num_heads))
        _require(workspace, "workspace", (torch.uint8,))
        self._keep = (plan, q, kv_cache, block_table, cache_seqlens, out, lse, workspace)
        self._fn = lib().mla_decode_stages
        self._args = (plan.handle, _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens),
                      C.c_float(float(softmax_scale)), _ptr(out), _ptr(lse), _ptr(workspace),
                      C.c_size_t(_nbytes(workspace)))

    def __call__(self, stream_handle: int, stages: int = MLA_STAGE_ALL):
        st = self._fn(*self._args, stream_handle, stages)
        if st != MLA_OK:
            raise MlaError(st, "mla_decode", last_error())


def _kv_spec(p):
    """(accepted torch dtypes, shape) of the cache for a problem struct."""
    import torch
    if p.kv_dtype == MLA_KV_FP8_E4M3:
        return (torch.uint8,), (p.num_pages, p.page_size, 656)
    return (torch.bfloat16, torch.int16), (p.num_pages, p.page_size, 576)


def mla_debug_gather(plan: Plan, kv_cache, block_table, rows_out, stream=None):
    import torch
    p = plan.problem
    dts, shape = _kv_spec(p)
    _require(kv_cache, "kv_cache", dts, shape)
    _require(block_table, "block_table", (torch.int32,), (p.batch, p.max_pages_per_seq))
    _require(rows_out, "rows_out", dts, (int(plan.seqlens.sum()), shape[-1]))
    _check(lib().mla_debug_gather(plan.handle, _ptr(kv_cache), _ptr(block_table), _ptr(rows_out),
                                  _stream(stream)), "mla_debug_gather")


def devplan_workspace_bytes(problem: mla_problem_t, num_workers: int = 0) -> int:
    n = lib().mla_devplan_workspace_bytes(C.byref(problem), num_workers)
    if n == 0:
        raise MlaError(MLA_ERR_INVALID_ARGUMENT, "mla_devplan_workspace_bytes", last_error())
    return n


def devplan_prepare(problem: mla_problem_t, num_workers: int, workspace, stream=None):
    _check(lib().mla_devplan_prepare(C.byref(problem), num_workers, _ptr(workspace), _nbytes(workspace),
                                     _stream(stream)), "mla_devplan_prepare")


class BoundDevplanDecode:
    """mla_decode_devplan with its arguments checked and marshalled once (the tensors must
    stay alive and in place; the cache_seqlens tensor's contents may change between calls)."""

    def __init__(self, problem: mla_problem_t, num_workers, q, kv_cache, block_table, cache_seqlens,
                 softmax_scale, out, lse, workspace, combined: bool = False):
        """combined: mla_decode_devplan_combined (one launch) instead of mla_decode_devplan."""
        import torch
        p = problem
        _require(q, "q", (torch.bfloat16,), (p.batch, p.q_len, p.num_heads, 576))
        _require(kv_cache, "kv_cache", *_kv_spec(p))
        _require(block_table, "block_table", (torch.int32,), (p.batch, p.max_pages_per_seq))
        _require(cache_seqlens, "cache_seqlens", (torch.int32,), (p.batch,))
        odt = torch.float32 if p.out_dtype == MLA_DTYPE_FP32 else torch.bfloat16
        _require(out, "out", (odt,), (p.batch, p.q_len, p.num_heads, 512))
        if lse is not None:
            _require(lse, "lse", (torch.float32,), (p.batch, p.q_len, p.num_heads))
        _require(workspace, "workspace", (torch.uint8,))
        self._problem = mla_problem_t.from_buffer_copy(p)
        self._keep = (q, kv_cache, block_table, cache_seqlens, out, lse, workspace)
        self._name = "mla_decode_devplan_combined" if combined else "mla_decode_devplan"
        self._fn = getattr(lib(), self._name)
        self._args = (C.byref(self._problem), num_workers, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                      _ptr(cache_seqlens), C.c_float(float(softmax_scale)), _ptr(out), _ptr(lse), _ptr(workspace),
                      C.c_size_t(_nbytes(workspace)))

    def __call__(self, stream_handle: int):
        st = self._fn(*self._args, stream_handle)
        if st != MLA_OK:
            raise MlaError(st, self._name, last_error())


def mla_decode_devplan_noalloc(problem: mla_problem_t, num_workers, q, kv_cache, block_table, cache_seqlens,
                               softmax_scale, out, lse, stream=None):
    """Device-scheduled decode with the library's own device scratch (allocates nothing)."""
    import torch
    p = problem
    _require(q, "q", (torch.bfloat16,), (p.batch, p.q_len, p.num_heads, 576))
    _require(kv_cache, "kv_cache", *_kv_spec(p))
    _require(block_table, "block_table", (torch.int32,), (p.batch, p.max_pages_per_seq))
    _require(cache_seqlens, "cache_seqlens", (torch.int32,), (p.batch,))
    odt = torch.float32 if p.out_dtype == MLA_DTYPE_FP32 else torch.bfloat16
    _require(out, "out", (odt,), (p.batch, p.q_len, p.num_heads, 512))
    if lse is not None:
        _require(lse, "lse", (torch.float32,), (p.batch, p.q_len, p.num_heads))
    _check(lib().mla_decode_devplan_noalloc(C.byref(p), num_workers, _ptr(q), _ptr(kv_cache), _ptr(block_table),
                                            _ptr(cache_seqlens), C.c_float(float(softmax_scale)), _ptr(out),
                                            _ptr(lse), _stream(stream)), "mla_decode_devplan_noalloc")


def mla_stream_probe(buffer, num_workgroups, stream=None):
    """Read `buffer` (a CUDA uint8 tensor) into LDS the way the decode reads its KV rows."""
    _check(lib().mla_stream_probe(_ptr(buffer), _nbytes(buffer), int(num_workgroups), _stream(stream)),
           "mla_stream_probe")


def mla_read_status(workspace, stream=None) -> int:
    v = C.c_int32(0)
    _check(lib().mla_read_status(_ptr(workspace), _stream(stream), C.byref(v)), "mla_read_status")
    return v.value


def mla_q_absorb(problem: mla_problem_t, q_nope, q_pe, w_uk, positions, rope_base, q_out, stream=None):
    """Query preparation: q_out = [W_UK q_nope, rope(q_pe)] per token and head."""
    import torch
    p = problem
    _require(q_nope, "q_nope", (torch.bfloat16,), (p.batch, p.q_len, p.num_heads, 128))
    _require(q_pe, "q_pe", (torch.bfloat16,), (p.batch, p.q_len, p.num_heads, 64))
    _require(w_uk, "w_uk", (torch.bfloat16,), (p.num_heads, 512, 128))
    _require(positions, "positions", (torch.int32,), (p.batch, p.q_len))
    _require(q_out, "q_out", (torch.bfloat16,), (p.batch, p.q_len, p.num_heads, 576))
    _check(lib().mla_q_absorb(C.byref(p), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(positions),
                              float(rope_base), _ptr(q_out), _stream(stream)), "mla_q_absorb")


def mla_kv_append(problem: mla_problem_t, c_kv, k_pe, positions, block_table, rope_base, kv_cache, status=None,
                  stream=None):
    """Write the new tokens' cache rows (bf16 or fp8 layout, as problem.kv_dtype)."""
    import torch
    p = problem
    _require(c_kv, "c_kv", (torch.bfloat16,), (p.batch, p.q_len, 512))
    _require(k_pe, "k_pe", (torch.bfloat16,), (p.batch, p.q_len, 64))
    _require(positions, "positions", (torch.int32,), (p.batch, p.q_len))
    _require(block_table, "block_table", (torch.int32,), (p.batch, p.max_pages_per_seq))
    _require(kv_cache, "kv_cache", *_kv_spec(p))
    if status is not None:
        _require(status, "status", (torch.int32,), (1,))
    _check(lib().mla_kv_append(C.byref(p), _ptr(c_kv), _ptr(k_pe), _ptr(positions), _ptr(block_table),
                               float(rope_base), _ptr(kv_cache), _ptr(status), _stream(stream)), "mla_kv_append")


def mla_out_absorb(problem: mla_problem_t, out_latent, w_uv, o, stream=None):
    """Output projection: o = W_UV out_latent per token and head (dtype: problem.out_dtype)."""
    import torch
    p = problem
    odt = torch.float32 if p.out_dtype == MLA_DTYPE_FP32 else torch.bfloat16
    _require(out_latent, "out_latent", (odt,), (p.batch, p.q_len, p.num_heads, 512))
    _require(w_uv, "w_uv", (torch.bfloat16,), (p.num_heads, 128, 512))
    _require(o, "o", (odt,), (p.batch, p.q_len, p.num_heads, 128))
    _check(lib().mla_out_absorb(C.byref(p), _ptr(out_latent), _ptr(w_uv), _ptr(o), _stream(stream)),
           "mla_out_absorb")


def alloc_workspace(plan: Plan, device="cuda"):
    """Device workspace for `plan` (256-B aligned: torch's allocator aligns to >= 512 B)."""
    import torch
    ws = torch.empty(max(256, plan.workspace_bytes), dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace not 256-B aligned")
    return ws
