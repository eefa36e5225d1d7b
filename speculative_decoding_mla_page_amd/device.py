"""Torch-side plumbing around the C ABI: device buffers, plan, workspace.

torch provides device memory and the stream; the verify computation itself is
the library's two HIP launches.  Nothing here computes attention.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B


class DeviceInputs:
    """One verify call's buffers on the GPU, built from host arrays.

    ``inst`` is any object with the fields of a verify instance: q (uint16
    [sumT, H, 576]), rows / row_slots (the pool's used rows), num_slots,
    num_heads, qo_indptr, kv_indptr, kv_indices, out_cache_loc, custom_mask,
    mask_indptr, sm_scale.  Unused pool slots hold bf16 NaN when ``poison``.
    With ``fused_save`` the draft tokens' rows are left out of the pool (their
    slots hold the fill value) and handed over as ``kv_new`` [sumT, 576], for
    the call to store at ``out_cache_loc`` itself.
    """

    def __init__(self, inst, device: str = "cuda", kv_indices_dtype: int = B.I32,
                 out_cache_loc_dtype: int = B.I64, row_stride: int = B.D_QK, poison: bool = True,
                 q_pad_heads: int = 0, out_pad_heads: int = 0, fused_save: bool = False):
        self.device = torch.device(device)
        self.num_heads = int(inst.num_heads)
        self.num_slots = int(inst.num_slots)
        self.sm_scale = float(inst.sm_scale)
        self.batch = len(inst.qo_indptr) - 1
        self.kv_indices_dtype = kv_indices_dtype
        self.out_cache_loc_dtype = out_cache_loc_dtype
        d = self.device
        h = self.num_heads
        q = torch.from_numpy(np.ascontiguousarray(inst.q).view(np.int16))
        if q_pad_heads:
            # a strided view: room for extra heads after the used ones
            full = torch.zeros((q.shape[0], h + q_pad_heads, B.D_QK), dtype=torch.int16)
            full[:, :h] = q
            self._q_store = full.to(d)
            self.q = self._q_store[:, :h]
        else:
            self.q = q.to(d)
        fill = -1 if poison else 0          # int16 -1 = bf16 bits 0xFFFF (NaN)
        self.pool = torch.full((self.num_slots, row_stride), fill, dtype=torch.int16, device=d)
        rows = torch.from_numpy(np.ascontiguousarray(inst.rows).view(np.int16)).to(d)
        slots = torch.from_numpy(np.asarray(inst.row_slots, dtype=np.int64)).to(d)
        self.pool[slots, :B.D_QK] = rows
        self.kv_new = None
        total_q = int(inst.qo_indptr[-1])
        if fused_save and total_q > 0:
            ocl = np.asarray(inst.out_cache_loc, np.int64)[:total_q]
            new = np.ascontiguousarray(inst.pool_view()[ocl][:, :B.D_QK]).view(np.int16)
            self.kv_new = torch.from_numpy(new).to(d)
            self.pool[torch.from_numpy(ocl).to(d)] = fill
        idx_t = torch.int64 if kv_indices_dtype == B.I64 else torch.int32
        ocl_t = torch.int64 if out_cache_loc_dtype == B.I64 else torch.int32
        self.qo_indptr = torch.from_numpy(np.asarray(inst.qo_indptr, np.int32)).to(d)
        self.kv_indptr = torch.from_numpy(np.asarray(inst.kv_indptr, np.int32)).to(d)
        self.kv_indices = torch.from_numpy(np.asarray(inst.kv_indices)).to(idx_t).to(d)
        self.out_cache_loc = torch.from_numpy(np.asarray(inst.out_cache_loc)).to(ocl_t).to(d)
        self.custom_mask = torch.from_numpy(np.asarray(inst.custom_mask, np.uint8)).to(d)
        self.mask_indptr = torch.from_numpy(np.asarray(inst.mask_indptr, np.int32)).to(d)
        # keep kernels' index reads in bounds even for empty buffers
        if self.kv_indices.numel() == 0:
            self.kv_indices = torch.zeros(1, dtype=idx_t, device=d)
        if self.out_cache_loc.numel() == 0:
            self.out_cache_loc = torch.zeros(1, dtype=ocl_t, device=d)
        if self.custom_mask.numel() == 0:
            self.custom_mask = torch.zeros(1, dtype=torch.uint8, device=d)
        self.total_q = int(inst.qo_indptr[-1])
        self.total_kv = int(inst.kv_indptr[-1])
        self.out_pad_heads = out_pad_heads

    def alloc_outputs(self, rows: Optional[int] = None):
        n = max(self.total_q if rows is None else rows, 1)
        h = self.num_heads
        if self.out_pad_heads:
            store = torch.full((n, h + self.out_pad_heads, B.D_V), float("nan"),
                               dtype=torch.float32, device=self.device)
            out = store[:, :h]
        else:
            out = torch.full((n, h, B.D_V), float("nan"), dtype=torch.float32, device=self.device)
        lse = torch.full((n, h), float("nan"), dtype=torch.float32, device=self.device)
        return out, lse


class Verifier:
    """A plan plus its workspace; ``__call__`` enqueues one verify call."""

    def __init__(self, num_heads: int, max_batch: int, max_q_tokens: int, max_kv_tokens: int,
                 max_tree_nodes: int = B.MAX_TREE_NODES, target_items: int = 0,
                 kv_indices_dtype: int = B.I32, out_cache_loc_dtype: int = B.I64, flags: int = 0,
                 device: str = "cuda", cu_count: int = 0):
        self.cfg = B.make_config(num_heads, max_batch, max_q_tokens, max_kv_tokens,
                                 max_tree_nodes=max_tree_nodes, target_items=target_items,
                                 cu_count=cu_count, kv_indices_dtype=kv_indices_dtype,
                                 out_cache_loc_dtype=out_cache_loc_dtype, flags=flags)
        self.plan = B.plan(self.cfg)
        self.layout = B.layout(self.plan)
        nbytes = B.workspace_size(self.plan)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)

    @classmethod
    def for_inputs(cls, di: DeviceInputs, **kw):
        return cls(di.num_heads, max(di.batch, 1), max(di.total_q, 1), max(di.total_kv, 0),
                   kv_indices_dtype=di.kv_indices_dtype,
                   out_cache_loc_dtype=di.out_cache_loc_dtype, **kw)

    def args(self, di: DeviceInputs, out, lse, batch_size: Optional[int] = None) -> B.Args:
        return B.make_args(di.batch if batch_size is None else batch_size, di.sm_scale, di.q,
                           di.pool, di.qo_indptr, di.kv_indptr, di.kv_indices, di.out_cache_loc,
                           di.custom_mask, di.mask_indptr, out, lse, num_slots=di.num_slots,
                           kv_new=di.kv_new)

    def __call__(self, di: DeviceInputs, out, lse, stream=None, batch_size: Optional[int] = None):
        B.run(self.plan, self.args(di, out, lse, batch_size), self.workspace, stream)

    # workspace regions (for bit-exact metadata checks)
    def header(self):
        w = self.workspace[self.layout.header_offset:self.layout.header_offset + 32]
        return w.view(torch.int32).cpu().numpy()

    def error_word(self) -> int:
        return int(self.header()[0]) & 0xFFFFFFFF

    def region(self, offset: int, count: int, dtype):
        nbytes = count * torch.empty(0, dtype=dtype).element_size()
        return self.workspace[offset:offset + nbytes].view(dtype)
