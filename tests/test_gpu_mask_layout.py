"""Full-row mask layout (a T_b x (P_b + T_b) block per request, the layout a
serving framework's tree verify passes), the prefix-column check, and the
shadow comparison against a caller's reference ("validate" mode)."""
import copy

import numpy as np
import pytest

from tests.gpu_helpers import assert_gate, need_gpu, oracle, run_gpu, say
from workloads import gen

pytestmark = pytest.mark.gpu


def full_row_instance(inst):
    """The same instance with each request's mask as full rows: prefix columns
    all ones, then its T x T tree block."""
    blocks, ptr = [], [0]
    for b in range(inst.batch):
        t, p = inst.tree_sizes[b], inst.prefix_lens[b]
        tree = np.asarray(inst.custom_mask[inst.mask_indptr[b]:inst.mask_indptr[b + 1]], np.uint8).reshape(t, t)
        blocks.append(np.concatenate([np.ones((t, p), np.uint8), tree], axis=1).reshape(-1))
        ptr.append(ptr[-1] + t * (p + t))
    out = copy.copy(inst)
    out.custom_mask = np.concatenate(blocks) if blocks else np.zeros(0, np.uint8)
    out.mask_indptr = np.asarray(ptr, np.int32)
    return out


def _mixed():
    return gen.make_instance([0, 37, 1500, 1, 77], [3, 0, 16, 1, 5], 8, num_slots=8192, seed=97)


@pytest.mark.parametrize("name", ["p5632_t16", "mixed"])
def test_full_rows_match_square_blocks(name):
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = _mixed() if name == "mixed" else gen.config(name)
    say(f"full-row mask {name}")
    out_sq, lse_sq, _, _ = run_gpu(inst)
    full = full_row_instance(inst)
    for flags in (B.FLAG_MASK_FULL_ROWS, B.FLAG_MASK_FULL_ROWS | B.FLAG_CHECK_PREFIX_MASK):
        out, lse, v, _ = run_gpu(full, flags=flags)
        assert v.error_word() == 0
        # the same computation on the same keys and visibility: bit-identical
        assert np.array_equal(out.view(np.uint32), out_sq.view(np.uint32))
        assert np.array_equal(lse.view(np.uint32), lse_sq.view(np.uint32))
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(out, lse, ref_out, ref_lse, label=f"full rows {name}")


def test_prefix_column_check():
    need_gpu()
    from speculative_decoding_mla_page_amd import binding as B
    inst = _mixed()
    full = full_row_instance(inst)
    b, node, col = 2, 7, 900                      # request 2 (P = 1500, T = 16)
    t, p = inst.tree_sizes[b], inst.prefix_lens[b]
    mask = full.custom_mask.copy()
    mask[full.mask_indptr[b] + node * (p + t) + col] = 0
    full.custom_mask = mask
    say("prefix column check")
    # unchecked: the prefix stays visible, nothing changes
    out, lse, v, _ = run_gpu(full, flags=B.FLAG_MASK_FULL_ROWS)
    assert v.error_word() == 0
    ref_out, ref_lse, _ = oracle(inst)
    assert_gate(out, lse, ref_out, ref_lse, label="unchecked")
    # checked: the hidden key's work items give NaN rows and the error bit
    out, lse, v, _ = run_gpu(full, flags=B.FLAG_MASK_FULL_ROWS | B.FLAG_CHECK_PREFIX_MASK)
    assert v.error_word() == B.DEVERR_MASK_PREFIX
    q0, q1 = int(inst.qo_indptr[b]), int(inst.qo_indptr[b + 1])
    assert np.all(np.isnan(out[q0:q1])) and np.all(np.isnan(lse[q0:q1]))
    others = np.r_[0:q0, q1:inst.total_q]
    assert_gate(out[others], lse[others], ref_out[others], ref_lse[others], label="other requests")


def _host_stats(out, lse, ref, ref_lse):
    o = out.astype(np.float32).reshape(-1)
    r = ref.astype(np.float32).reshape(-1)
    on, rn = np.isnan(o), np.isnan(r)
    both = ~on & ~rn
    d = np.abs(o[both] - r[both])                          # fp32, as on the device
    a = np.maximum(np.abs(r[both].astype(np.float64)), 2.0 ** -126)
    ulp = (2.0 ** (np.floor(np.log2(a)) - 7)).astype(np.float32)
    over = int(np.sum(~(d <= 2 * ulp) & (o[both] != r[both]))) + int(np.sum(on != rn))
    fin = np.isfinite(lse) & np.isfinite(ref_lse)
    return dict(max_abs=float(d[np.isfinite(d)].max()) if d.size else 0.0, over=over,
                nan=int(np.sum(on != rn)), total=o.size,
                lse=float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0)


def test_shadow_compare_stats():
    need_gpu()
    import torch
    from speculative_decoding_mla_page_amd import binding as B
    from speculative_decoding_mla_page_amd.device import DeviceInputs, Verifier
    inst = gen.config("p5632_t16")
    say("shadow compare")
    di = DeviceInputs(inst)
    v = Verifier.for_inputs(di)
    out, lse = di.alloc_outputs()
    args = v.args(di, out, lse)
    ref_out, ref_lse, _ = oracle(inst)
    rng = np.random.default_rng(5)
    for case in ("oracle", "perturbed"):
        r = ref_out.copy()
        rl = ref_lse.copy()
        if case == "perturbed":
            idx = rng.choice(r.size, 200, replace=False)
            r.reshape(-1)[idx] += np.float32(1e-2)
            r.reshape(-1)[idx[:3]] = np.nan
            rl[0, 0] += np.float32(0.5)
        ref_t = torch.from_numpy(r).cuda()
        rl_t = torch.from_numpy(rl).cuda()
        B.run(v.plan, args, v.workspace)
        B.compare(v.plan, args, ref_t, rl_t, v.workspace)
        torch.cuda.synchronize()
        st = B.CompareStats.from_buffer_copy(
            v.workspace[v.layout.stats_offset:v.layout.stats_offset + 32].cpu().numpy().tobytes())
        want = _host_stats(out.cpu().numpy(), lse.cpu().numpy(), r, rl)
        f = lambda bits: float(np.uint32(bits).view(np.float32))
        assert st.count_total == want["total"], case
        assert st.count_over == want["over"], (case, st.count_over, want)
        assert st.count_nan_mismatch == want["nan"], case
        assert f(st.max_abs_diff_bits) == np.float32(want["max_abs"]), (case, f(st.max_abs_diff_bits), want)
        assert abs(f(st.max_lse_diff_bits) - want["lse"]) <= 1e-6, case
