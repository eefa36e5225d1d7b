"""Decode workload (T_b = 1 per request, many requests, H = 16 and 128):
the same boundary in its HBM-bound regime, checked against the oracle."""
import numpy as np
import pytest

from tests.gpu_helpers import assert_gate, assert_rows_finite, need_gpu, oracle, oracle_blocked, run_gpu, say
from workloads import gen

pytestmark = pytest.mark.gpu


def test_decode_b32_h16_full():
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.config("decode_b32_h16")
    say("decode_b32_h16")
    out, lse, v, _ = run_gpu(inst, flags=B.FLAG_TRACE_KEYS, max_tree_nodes=1)
    assert v.error_word() == 0
    ref_out, ref_lse, rec = oracle(inst)
    tr = v.region(v.layout.trace_offset, inst.total_kv + inst.total_q, __import__("torch").int64).cpu().numpy()
    for b in range(inst.batch):
        base = int(inst.kv_indptr[b]) + int(inst.qo_indptr[b])
        assert np.array_equal(tr[base:base + len(rec["keys"][b])], rec["keys"][b]), f"request {b}"
    assert_gate(out, lse, ref_out, ref_lse, label="decode_b32_h16")


def test_decode_b64_h128_full():
    """64 requests x 1 node x 128 heads: every row against the oracle."""
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = gen.config("decode_b64_h128")
    say("decode_b64_h128 (all 64 tokens x 128 heads)")
    out, lse, v, _ = run_gpu(inst, flags=B.FLAG_TRACE_KEYS, max_tree_nodes=1)
    assert v.error_word() == 0
    assert_rows_finite(out, lse, label="decode_b64_h128")
    ref_out, ref_lse, rec = oracle_blocked(inst, block_tokens=16)
    tr = v.region(v.layout.trace_offset, inst.total_kv + inst.total_q, __import__("torch").int64).cpu().numpy()
    for b in range(inst.batch):
        base = int(inst.kv_indptr[b]) + int(inst.qo_indptr[b])
        assert np.array_equal(tr[base:base + len(rec["keys"][b])], rec["keys"][b]), f"request {b}"
    assert_gate(out, lse, ref_out, ref_lse, label="decode_b64_h128")
