"""CPU checks of the precision emulator used to choose how P enters the PV
product (tests/precision_sim.py): its rounding helpers against torch's own
conversions, and the scheme verdicts on the tiny verify workload."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import mla_verify_ref as R
from tests import precision_sim as P
from workloads import gen


def test_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(4096), rng.standard_normal(4096) * 1e-30,
                        rng.standard_normal(4096) * 1e30]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(P.to_bf16(x), ref)


def test_to_e4m3_matches_torch_in_range_and_saturates():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(-448, 448, 4096), rng.standard_normal(4096) * 1e-2,
                        [2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10, 0.0, 448.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(P.to_e4m3(x), ref)
    assert P.to_e4m3(np.array([500.0, -1e6], np.float32)).tolist() == [448.0, -448.0]


def test_scheme_verdicts_on_tiny():
    """Only the split hi + lo bf16 forms of P (and fp32 itself) clear the gate:
    one bf16 rounding of P, fp16 P and V, and a bf16 + e4m3 split all miss the
    2-ULP share on the tiny 4-node chain workload."""
    inst = gen.config("tiny")
    ref_out, ref_lse, _ = R.mla_verify_reference(inst.q, inst.pool_view(), inst.qo_indptr, inst.kv_indptr,
                                                 inst.kv_indices, inst.out_cache_loc, inst.custom_mask,
                                                 inst.mask_indptr, inst.num_heads, inst.sm_scale)
    verdict = {s: P.passes(P.gate(*P.simulate(inst, s), ref_out, ref_lse)) for s in P.SCHEMES}
    assert verdict == {"fp32": True, "bf16": False, "bf16x2": True, "bf16x2t": True, "fp16": False,
                       "bf16+e4m3": False}
