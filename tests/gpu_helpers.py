"""Shared helpers of the GPU tests: the acceptance gate and one-call runners."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import mla_verify_ref as R

MAX_ABS = 1e-2          # max |gpu - oracle| over all output elements
FRAC_2ULP = 0.999       # share of output elements within 2 bf16 ULP of the oracle
LSE_ABS = 1e-3          # max |gpu - oracle| of the log-sum-exp

# every gate evaluated in this process: (label, stats); printed as a table at
# the end of the pytest run so that the margins appear in the summary
GATE_RECORDS: list = []


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg: str):
    """Name the case before each GPU step, flushed, so a failing run shows it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def bf16_ulp(ref: np.ndarray) -> np.ndarray:
    """ULP of bf16 at the oracle's value: 2^(floor(log2|x|) - 7), |x| floored at 2^-126."""
    a = np.maximum(np.abs(ref.astype(np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def gate_stats(out, lse, ref_out, ref_lse, tokens=None):
    if tokens is not None:
        tokens = np.asarray(sorted(tokens))
        out, lse, ref_out, ref_lse = out[tokens], lse[tokens], ref_out[tokens], ref_lse[tokens]
    o = out.astype(np.float64)
    r = ref_out.astype(np.float64)
    diff = np.abs(o - r)
    within = diff <= 2 * bf16_ulp(r)
    fin = np.isfinite(ref_lse)
    lse_err = np.abs(lse.astype(np.float64)[fin] - ref_lse.astype(np.float64)[fin])
    return dict(
        finite=bool(np.isfinite(o).all()),
        max_abs=float(diff.max()) if diff.size else 0.0,
        frac_2ulp=float(within.mean()) if within.size else 1.0,
        lse_max_abs=float(lse_err.max()) if lse_err.size else 0.0,
        empty_rows_ok=bool(np.all(lse[~fin] == -np.inf) and np.all(out[~fin] == 0.0)),
        elements=int(o.size),
    )


def assert_gate(out, lse, ref_out, ref_lse, tokens=None, label=""):
    st = gate_stats(out, lse, ref_out, ref_lse, tokens)
    say(f"{label} gate {st}")
    GATE_RECORDS.append((label, st))
    assert st["finite"], st
    assert st["max_abs"] <= MAX_ABS, st
    assert st["frac_2ulp"] >= FRAC_2ULP, st
    assert st["lse_max_abs"] <= LSE_ABS, st
    assert st["empty_rows_ok"], st
    return st


def assert_rows_finite(out, lse, rows=None, label=""):
    """Every output row (or the given token rows) is finite: no row left unwritten
    (outputs are allocated as NaN) and no NaN produced."""
    o = out if rows is None else out[rows]
    l = lse if rows is None else lse[rows]
    bad = int(np.count_nonzero(~np.isfinite(o)))
    assert bad == 0, f"{label}: {bad} non-finite output elements"
    # lse is -inf only for a row that sees no key (its out is then exactly 0)
    assert not np.isnan(l).any(), f"{label}: NaN lse"


def oracle(inst, tokens=None, pool=None):
    return R.mla_verify_reference(inst.q, inst.pool_view() if pool is None else pool,
                                  inst.qo_indptr, inst.kv_indptr, inst.kv_indices,
                                  inst.out_cache_loc, inst.custom_mask, inst.mask_indptr,
                                  inst.num_heads, inst.sm_scale, tokens=tokens)


def oracle_blocked(inst, block_tokens: int, pool=None):
    """The oracle over every token, computed block_tokens tokens at a time so
    that the score matrices of a wide-head call stay a few hundred MB."""
    total = inst.total_q
    out = np.full((total, inst.num_heads, 512), np.nan, np.float32)
    lse = np.full((total, inst.num_heads), np.nan, np.float32)
    rec = None
    for t0 in range(0, max(total, 1), block_tokens):
        toks = list(range(t0, min(total, t0 + block_tokens)))
        o, l, r = oracle(inst, tokens=toks, pool=pool)
        out[toks] = o[toks]
        lse[toks] = l[toks]
        rec = rec or r
    return out, lse, rec


def run_gpu(inst, flags=0, target_items=0, max_tree_nodes=64, **dev_kw):
    """One call through the C ABI; returns (out, lse, verifier, device_inputs) on the host."""
    import torch
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    di = DeviceInputs(inst, **dev_kw)
    v = Verifier.for_inputs(di, flags=flags, target_items=target_items,
                            max_tree_nodes=max_tree_nodes)
    out, lse = di.alloc_outputs()
    # a known byte pattern, so that a region the call must write and does not
    # shows up in the metadata checks
    v.workspace.fill_(0xA5)
    v(di, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), v, di
