"""ctypes binding of libmla_verify.so (argument marshalling only).

Mirrors include/mla_verify.h.  Tensors are torch tensors on the GPU; every step
of the verify computation runs in the library's HIP kernels.  There is no
fallback: if the library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla_verify.so")

D_QK = 576
D_V = 512
MAX_TREE_NODES = 64
I32, I64 = 0, 1
FLAG_TRACE_KEYS = 1
FLAG_MASK_FULL_ROWS = 2
FLAG_CHECK_PREFIX_MASK = 4
FLAG_CONTIGUOUS_PREFIX = 8

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_WORKSPACE_TOO_SMALL = 3
ERR_LAUNCH = 4
ERR_BAD_PLAN = 5

DEVERR_QO_INDPTR = 1 << 0
DEVERR_KV_INDPTR = 1 << 1
DEVERR_TREE_SIZE = 1 << 2
DEVERR_MASK_INDPTR = 1 << 3
DEVERR_SLOT_RANGE = 1 << 4
DEVERR_CAPACITY = 1 << 5
DEVERR_MASK_PREFIX = 1 << 6

PHASE_PARTIAL, PHASE_MERGE = 0, 1
ABI_VERSION = 7


class Config(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("max_q_tokens", ctypes.c_int32),
        ("max_tree_nodes", ctypes.c_int32),
        ("max_kv_tokens", ctypes.c_int64),
        ("target_items", ctypes.c_int32),
        ("cu_count", ctypes.c_int32),
        ("kv_indices_dtype", ctypes.c_int32),
        ("out_cache_loc_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_int32 * 7),
    ]


class Plan(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint64 * 64)]


class Args(ctypes.Structure):
    _fields_ = [
        ("batch_size", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("q_stride_tok", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("kv_pool", ctypes.c_void_p),
        ("kv_row_stride", ctypes.c_int64),
        ("num_slots", ctypes.c_int64),
        ("qo_indptr", ctypes.c_void_p),
        ("kv_indptr", ctypes.c_void_p),
        ("kv_indices", ctypes.c_void_p),
        ("out_cache_loc", ctypes.c_void_p),
        ("custom_mask", ctypes.c_void_p),
        ("mask_indptr", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("out_stride_tok", ctypes.c_int64),
        ("out_stride_head", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
        ("lse_stride_tok", ctypes.c_int64),
        ("kv_new", ctypes.c_void_p),
        ("kv_new_stride_tok", ctypes.c_int64),
    ]


class Layout(ctypes.Structure):
    _fields_ = [
        ("total_bytes", ctypes.c_uint64),
        ("header_offset", ctypes.c_uint64),
        ("request_offset", ctypes.c_uint64),
        ("anc_offset", ctypes.c_uint64),
        ("items_offset", ctypes.c_uint64),
        ("partial_o_offset", ctypes.c_uint64),
        ("partial_ml_offset", ctypes.c_uint64),
        ("trace_offset", ctypes.c_uint64),
        ("stats_offset", ctypes.c_uint64),
        ("tokens_offset", ctypes.c_uint64),
        ("errors_offset", ctypes.c_uint64),
        ("item_capacity", ctypes.c_int32),
        ("rows_per_item", ctypes.c_int32),
        ("keys_per_tile", ctypes.c_int32),
        ("target_items", ctypes.c_int32),
        ("partial_grid", ctypes.c_int32),
        ("merge_grid", ctypes.c_int32),
    ]


class CompareStats(ctypes.Structure):
    _fields_ = [
        ("max_abs_diff_bits", ctypes.c_uint32),
        ("count_over", ctypes.c_uint32),
        ("count_total", ctypes.c_uint32),
        ("max_lse_diff_bits", ctypes.c_uint32),
        ("count_nan_mismatch", ctypes.c_uint32),
        ("count_lse_mismatch", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32 * 2),
    ]


class MlaVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m speculative_decoding_mla_page_amd.build)")
        l = ctypes.CDLL(LIB_PATH)
        l.mla_verify_plan.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Plan)]
        l.mla_verify_plan.restype = ctypes.c_int
        l.mla_verify_workspace_size.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(ctypes.c_size_t)]
        l.mla_verify_workspace_size.restype = ctypes.c_int
        l.mla_verify_workspace_layout.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Layout)]
        l.mla_verify_workspace_layout.restype = ctypes.c_int
        l.mla_verify_run.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_void_p]
        l.mla_verify_run.restype = ctypes.c_int
        l.mla_verify_run_static.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p]
        l.mla_verify_run_static.restype = ctypes.c_int
        l.mla_verify_run_phase.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args),
                                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.c_int32]
        l.mla_verify_run_phase.restype = ctypes.c_int
        l.mla_verify_compare.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        l.mla_verify_compare.restype = ctypes.c_int
        l.mla_verify_compact.argtypes = [ctypes.POINTER(Plan), ctypes.POINTER(Args), ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]
        l.mla_verify_compact.restype = ctypes.c_int
        l.mla_verify_calibrate_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        l.mla_verify_calibrate_mfma.restype = ctypes.c_int
        l.mla_verify_calibrate_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                                ctypes.c_void_p]
        l.mla_verify_calibrate_read.restype = ctypes.c_int
        l.mla_verify_status_string.argtypes = [ctypes.c_int]
        l.mla_verify_status_string.restype = ctypes.c_char_p
        l.mla_verify_abi_version.argtypes = []
        l.mla_verify_abi_version.restype = ctypes.c_int32
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().mla_verify_status_string(int(status)).decode()


def make_config(num_heads: int, max_batch: int, max_q_tokens: int, max_kv_tokens: int,
                max_tree_nodes: int = MAX_TREE_NODES, target_items: int = 0, cu_count: int = 0,
                kv_indices_dtype: int = I32, out_cache_loc_dtype: int = I64,
                flags: int = 0) -> Config:
    c = Config()
    c.num_heads = num_heads
    c.max_batch = max_batch
    c.max_q_tokens = max_q_tokens
    c.max_tree_nodes = max_tree_nodes
    c.max_kv_tokens = max_kv_tokens
    c.target_items = target_items
    c.cu_count = cu_count
    c.kv_indices_dtype = kv_indices_dtype
    c.out_cache_loc_dtype = out_cache_loc_dtype
    c.flags = flags
    return c


def plan(cfg: Config) -> Plan:
    p = Plan()
    st = lib().mla_verify_plan(ctypes.byref(cfg), ctypes.byref(p))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_plan")
    return p


def workspace_size(p: Plan) -> int:
    n = ctypes.c_size_t()
    st = lib().mla_verify_workspace_size(ctypes.byref(p), ctypes.byref(n))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_workspace_size")
    return int(n.value)


def layout(p: Plan) -> Layout:
    out = Layout()
    st = lib().mla_verify_workspace_layout(ctypes.byref(p), ctypes.byref(out))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_workspace_layout")
    return out


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def make_args(batch_size: int, sm_scale: float, q, kv_pool, qo_indptr, kv_indptr, kv_indices,
              out_cache_loc, custom_mask, mask_indptr, out, lse=None, num_slots: Optional[int] = None,
              kv_new=None) -> Args:
    """Build the argument struct from torch tensors (bf16 q/pool may be int16 or
    bfloat16 views; strides are read from the tensors)."""
    a = Args()
    a.batch_size = int(batch_size)
    a.sm_scale = float(sm_scale)
    a.q = _ptr(q)
    a.q_stride_tok = q.stride(0)
    a.q_stride_head = q.stride(1)
    a.kv_pool = _ptr(kv_pool)
    a.kv_row_stride = kv_pool.stride(0)
    a.num_slots = kv_pool.shape[0] if num_slots is None else int(num_slots)
    a.qo_indptr = _ptr(qo_indptr)
    a.kv_indptr = _ptr(kv_indptr)
    a.kv_indices = _ptr(kv_indices)
    a.out_cache_loc = _ptr(out_cache_loc)
    a.custom_mask = _ptr(custom_mask)
    a.mask_indptr = _ptr(mask_indptr)
    a.out = _ptr(out)
    a.out_stride_tok = out.stride(0)
    a.out_stride_head = out.stride(1)
    a.lse = _ptr(lse)
    a.lse_stride_tok = lse.stride(0) if lse is not None else 0
    a.kv_new = _ptr(kv_new)
    a.kv_new_stride_tok = kv_new.stride(0) if kv_new is not None else 0
    return a


def compare(p: Plan, args: Args, ref_out, ref_lse, workspace, stream=None) -> None:
    """Enqueue the shadow comparison of args.out / args.lse against a reference
    (torch tensors in the same layout) into the workspace's stats region."""
    st = lib().mla_verify_compare(ctypes.byref(p), ctypes.byref(args), _ptr(ref_out), ref_out.stride(0),
                                  ref_out.stride(1), _ptr(ref_lse),
                                  ref_lse.stride(0) if ref_lse is not None else 0, _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_compare")


def compact(p: Plan, args: Args, dst_start, error_word, stream=None) -> None:
    """Enqueue the prefix compaction: each request's prefix rows move to the
    contiguous slots starting at dst_start[b] (int64 device tensor) and
    kv_indices is rewritten in place; problems are ORed into error_word
    (int32 device tensor, zeroed by the caller)."""
    st = lib().mla_verify_compact(ctypes.byref(p), ctypes.byref(args), _ptr(dst_start), _ptr(error_word),
                                  _stream(stream))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_compact")


def calibrate_mfma(iters: int, blocks: int, out, stream=None) -> None:
    """Enqueue the bf16 MFMA loop (blocks x 4 waves x iters x 65,536 flops);
    out: float32 device tensor of at least blocks x 256 elements."""
    if out.dtype.itemsize != 4 or out.numel() < blocks * 256:
        raise ValueError("calibrate_mfma: out must hold blocks x 256 float32 values")
    st = lib().mla_verify_calibrate_mfma(int(iters), int(blocks), _ptr(out), _stream(stream))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_calibrate_mfma")


def calibrate_read(buf, blocks: int, out, stream=None) -> None:
    """Enqueue the read stream over every byte of buf (a contiguous device
    tensor); out: float32 device tensor of at least blocks x 256 elements."""
    if not buf.is_contiguous():
        raise ValueError("calibrate_read: buf must be contiguous")
    if out.dtype.itemsize != 4 or out.numel() < blocks * 256:
        raise ValueError("calibrate_read: out must hold blocks x 256 float32 values")
    st = lib().mla_verify_calibrate_read(_ptr(buf), buf.numel() * buf.element_size(), int(blocks), _ptr(out),
                                         _stream(stream))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_calibrate_read")


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def run(p: Plan, args: Args, workspace, stream=None) -> None:
    """Enqueue the two launches on `stream` (default: torch's current stream)."""
    st = lib().mla_verify_run(ctypes.byref(p), ctypes.byref(args), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_run")


def run_static(p: Plan, args: Args, stream=None) -> None:
    """Enqueue the two launches with the library's static device scratch as
    the workspace (no allocation by anyone)."""
    st = lib().mla_verify_run_static(ctypes.byref(p), ctypes.byref(args), _stream(stream))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_run_static")


STATIC_SCRATCH_BYTES = 96 << 20


def run_phase(p: Plan, args: Args, workspace, phase: int, stream=None) -> None:
    st = lib().mla_verify_run_phase(ctypes.byref(p), ctypes.byref(args), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream),
                                    int(phase))
    if st != OK:
        raise MlaVerifyError(st, "mla_verify_run_phase")
