"""Move a host problem (see inputs.py) to torch device tensors and run the library on it."""
from __future__ import annotations

import numpy as np

from . import binding as B


def to_device(prob, device="cuda"):
    """Host Problem -> dict of contiguous device tensors (bf16 bit patterns reinterpreted)."""
    import torch
    q = torch.from_numpy(prob.q.view(np.int16)).to(device).view(torch.bfloat16)
    if prob.kv_cache.dtype == np.uint8:           # fp8 rows (656 bytes each)
        kv = torch.from_numpy(prob.kv_cache).to(device)
    else:
        kv = torch.from_numpy(prob.kv_cache.view(np.int16)).to(device).view(torch.bfloat16)
    bt = torch.from_numpy(prob.block_table).to(device)
    sl = torch.from_numpy(prob.cache_seqlens.astype(np.int32)).to(device)
    return {"q": q, "kv_cache": kv, "block_table": bt, "cache_seqlens": sl}


def problem_struct(prob, causal=False):
    return B.make_problem(prob.batch, prob.q_len, prob.num_heads, prob.page_size, prob.num_pages,
                          prob.max_pages_per_seq, out_fp32=prob.out_fp32, causal=causal,
                          kv_fp8=prob.kv_format == "fp8")


class Runner:
    """Plan + workspace + outputs for one problem on one device; call() launches the decode."""

    def __init__(self, prob, dev=None, num_cus=0, force_splits=0, device="cuda", causal=False, rows_per_group=0):
        import torch
        self.prob = prob
        self.dev = dev if dev is not None else to_device(prob, device)
        self.plan = B.Plan(problem_struct(prob, causal), prob.cache_seqlens, num_cus=num_cus,
                           force_splits=force_splits, rows_per_group=rows_per_group)
        self.ws = B.alloc_workspace(self.plan, device)
        self.plan.upload(self.ws)
        odt = torch.float32 if prob.out_fp32 else torch.bfloat16
        self.out = torch.empty((prob.batch, prob.q_len, prob.num_heads, 512), dtype=odt, device=device)
        self.lse = torch.empty((prob.batch, prob.q_len, prob.num_heads), dtype=torch.float32, device=device)

        d = self.dev
        self._bound = B.BoundDecode(self.plan, d["q"], d["kv_cache"], d["block_table"], d["cache_seqlens"],
                                    self.prob.softmax_scale, self.out, self.lse, self.ws)

    def __call__(self, stream=None, stages=B.MLA_STAGE_ALL):
        import torch
        sh = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
        self._bound(sh, stages)
        return self.out, self.lse

    def results(self):
        """(out as float64 numpy, lse as float64 numpy) after synchronising."""
        import torch
        torch.cuda.synchronize()
        return self.out.float().cpu().numpy().astype(np.float64), self.lse.cpu().numpy().astype(np.float64)


class DevplanRunner:
    """Device-scheduled decode (mla_decode_devplan, or mla_decode_devplan_combined with
    combined=True) for one problem: no host plan; the device cache_seqlens may be rewritten
    between calls."""

    def __init__(self, prob, dev=None, num_workers=0, device="cuda", causal=False, combined=False):
        import torch
        self.prob = prob
        self.dev = dev if dev is not None else to_device(prob, device)
        self.problem = problem_struct(prob, causal)
        nbytes = B.devplan_workspace_bytes(self.problem, num_workers)
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)   # torch aligns to >= 512 B
        if self.ws.data_ptr() % 256:
            raise RuntimeError("workspace not 256-B aligned")
        B.devplan_prepare(self.problem, num_workers, self.ws)
        odt = torch.float32 if prob.out_fp32 else torch.bfloat16
        self.out = torch.empty((prob.batch, prob.q_len, prob.num_heads, 512), dtype=odt, device=device)
        self.lse = torch.empty((prob.batch, prob.q_len, prob.num_heads), dtype=torch.float32, device=device)
        d = self.dev
        self._bound = B.BoundDevplanDecode(self.problem, num_workers, d["q"], d["kv_cache"], d["block_table"],
                                           d["cache_seqlens"], prob.softmax_scale, self.out, self.lse, self.ws,
                                           combined=combined)

    def __call__(self, stream=None):
        import torch
        self._bound((stream if stream is not None else torch.cuda.current_stream()).cuda_stream)
        return self.out, self.lse

    def results(self):
        import torch
        torch.cuda.synchronize()
        return self.out.float().cpu().numpy().astype(np.float64), self.lse.cpu().numpy().astype(np.float64)


def layer_to_device(li, device="cuda"):
    """Host LayerInputs (see inputs.py) -> dict of contiguous bf16 device tensors."""
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return {k: bf(getattr(li, k)) for k in ("q_nope", "q_pe", "c_kv", "k_pe", "w_uk", "w_uv")}
