"""Seeded random instances through the whole call: batch size, prefix and
tree lengths, heads, index dtypes, mask layout, fused save, work-item target
and tree shape drawn per case, every output row against the oracle."""
import numpy as np
import pytest

from tests.gpu_helpers import assert_gate, need_gpu, oracle, say
from workloads import gen

pytestmark = pytest.mark.gpu

N_CASES = 12
MAX_ROW_KEYS = 40_000_000     # bound on sum_b T_b * H * (P_b + T_b), so the oracle takes about a second


def draw_case(seed, head_choices=(1, 2, 8, 16, 32)):
    """One random case: (instance, DeviceInputs keywords, plan keywords, full_rows)."""
    from speculative_decoding_mla_page_amd import binding as B
    rng = np.random.default_rng(seed)
    heads = int(rng.choice(head_choices))
    batch = int(rng.integers(1, 81))
    while True:
        # prefixes: mostly short, some long, some empty
        kind = rng.random(batch)
        prefixes = np.where(kind < 0.1, 0, np.where(kind < 0.7, rng.integers(1, 2000, batch),
                                                    rng.integers(2000, 30000, batch)))
        trees = rng.integers(0 if batch > 1 else 1, 65, batch)
        work = int(np.sum(trees * heads * (prefixes + trees)))
        if work <= MAX_ROW_KEYS and int(np.sum(trees)) > 0:
            break
        batch = max(1, batch // 2)
    total_kv = int(prefixes.sum() + trees.sum())
    num_slots = int(2 ** np.ceil(np.log2(total_kv * 2 + 1024)))
    inst = gen.make_instance(prefixes.tolist(), trees.tolist(), heads, num_slots=num_slots, seed=seed + 1,
                             tree=str(rng.choice(["random", "chain"])),
                             outlier_frac=float(rng.choice([0.0, 0.01])))
    dev_kw = dict(kv_indices_dtype=int(rng.choice([B.I32, B.I64])),
                  out_cache_loc_dtype=int(rng.choice([B.I32, B.I64])),
                  fused_save=bool(rng.random() < 0.3))
    plan_kw = dict(target_items=int(rng.choice([0, 0, 7, 64, 300])),
                   max_tree_nodes=int(max(1, trees.max())))
    full_rows = bool(rng.random() < 0.3)
    return inst, dev_kw, plan_kw, full_rows


def _run_case(case, inst, dev_kw, plan_kw, full_rows):
    torch = need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    from tests.test_gpu_mask_layout import full_row_instance
    dev_inst = full_row_instance(inst) if full_rows else inst
    say(f"random case {case}: B={inst.batch} H={inst.num_heads} T={list(inst.tree_sizes)[:8]}... "
        f"P_max={max(inst.prefix_lens)} {dev_kw} {plan_kw} full_rows={full_rows}")
    di = DeviceInputs(dev_inst, **dev_kw)
    v = Verifier.for_inputs(di, flags=B.FLAG_MASK_FULL_ROWS if full_rows else 0, **plan_kw)
    out, lse = di.alloc_outputs()
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    v(di, out, lse)
    torch.cuda.synchronize()
    assert v.error_word() == 0
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(out.cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, label=f"random case {case}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_instance(case):
    _run_case(case, *draw_case(7000 + case))


@pytest.mark.parametrize("case", range(6))
def test_random_instance_odd_heads(case):
    """Head counts that do not divide the 64-row block: a row block ends in
    the middle of a tree node, and an item's rows span several nodes."""
    _run_case(100 + case, *draw_case(7100 + case, head_choices=(3, 5, 12, 24, 48, 96)))
