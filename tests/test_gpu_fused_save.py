"""Fused KV save: the call stores this step's draft rows into the pool at
out_cache_loc (the KV-cache ordering the pages require before the verify
kernel reads the pool) and then attends to them.  The pool bytes are checked
bit for bit, the outputs against the oracle on the pool the rows belong in."""
import numpy as np
import pytest

from tests.gpu_helpers import assert_gate, need_gpu, oracle, say
from workloads import gen

pytestmark = pytest.mark.gpu


def _run_fused(inst, **dev_kw):
    import torch
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    di = DeviceInputs(inst, fused_save=True, **dev_kw)
    total_q = int(inst.qo_indptr[-1])
    ocl = np.asarray(inst.out_cache_loc, np.int64)[:total_q]
    ocl_d = torch.from_numpy(ocl).to(di.pool.device)
    before = di.pool[ocl_d][:, :576].cpu().numpy().view(np.uint16)
    assert np.all(before == 0xFFFF), "draft slots must start out poisoned"
    v = Verifier.for_inputs(di)
    out, lse = di.alloc_outputs()
    v(di, out, lse)
    torch.cuda.synchronize()
    after = di.pool[ocl_d][:, :576].cpu().numpy().view(np.uint16)
    return out.cpu().numpy(), lse.cpu().numpy(), v, after, ocl


@pytest.mark.parametrize("name", ["p5632_t16", "mixed"])
def test_fused_kv_save(name):
    need_gpu()
    if name == "mixed":
        inst = gen.make_instance([0, 37, 5000, 1, 77], [3, 0, 64, 1, 5], 8, num_slots=16384, seed=95)
    else:
        inst = gen.config(name)
    say(f"fused save {name}")
    out, lse, v, stored, ocl = _run_fused(inst)
    assert v.error_word() == 0
    assert np.array_equal(stored, inst.pool_view()[ocl][:, :576]), "pool rows after the save"
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(out, lse, ref_out, ref_lse, label=f"fused save {name}")


def test_fused_kv_save_int32_slots_and_wide_rows():
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.make_instance([700, 129], [16, 7], 8, num_slots=8192, seed=96)
    say("fused save int32 out_cache_loc, row stride 640")
    out, lse, v, stored, ocl = _run_fused(inst, out_cache_loc_dtype=B.I32, row_stride=640)
    assert v.error_word() == 0
    assert np.array_equal(stored, inst.pool_view()[ocl][:, :576])
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(out, lse, ref_out, ref_lse, label="fused save int32")
