"""Pins of the CPU oracle to things other than itself.

Each test ties the oracle to an independent fact: a pure-Python brute force on
tiny inputs, closed forms, textbook attention (torch SDPA on the CPU in fp64),
invariants of the definition, hand-worked metadata, and planted mistakes that
must be caught.  None of these touch the GPU.
"""
import inspect
import math
import os
import struct
import types

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mla_verify_ref as R
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(inst, **kw):
    return R.mla_verify_reference(inst.q, inst.pool_view(), inst.qo_indptr, inst.kv_indptr,
                                  inst.kv_indices, inst.out_cache_loc, inst.custom_mask,
                                  inst.mask_indptr, inst.num_heads, inst.sm_scale, **kw)


# ---------------------------------------------------------------- brute force
def _bf16_py(bits):
    """bf16 bits -> Python float via struct (independent of numpy views)."""
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _ancestors(parents, i):
    s = set()
    while i >= 0:
        s.add(i)
        i = parents[i]
    return s


def _brute(inst, vis_fn):
    """Pure-Python fp64 loops over an explicit visibility function
    vis_fn(b, node, key_pos) -> bool.  Returns out [sumT][H][512], lse [sumT][H]."""
    h = inst.num_heads
    lut = {int(s): r for r, s in enumerate(inst.row_slots)}
    out, lse = {}, {}
    for b in range(inst.batch):
        p = inst.prefix_lens[b]
        t = inst.tree_sizes[b]
        q0 = int(inst.qo_indptr[b])
        k0 = int(inst.kv_indptr[b])
        slots = [int(inst.kv_indices[k0 + j]) for j in range(p)] + \
                [int(inst.out_cache_loc[q0 + i]) for i in range(t)]
        rows = [[_bf16_py(x) for x in inst.rows[lut[s]]] for s in slots]
        for i in range(t):
            for hh in range(h):
                qv = [_bf16_py(x) for x in inst.q[q0 + i, hh]]
                scores = []
                for j, row in enumerate(rows):
                    if vis_fn(b, i, j):
                        dot = 0.0
                        for d in range(576):
                            dot += qv[d] * row[d]
                        scores.append((j, inst.sm_scale * dot))
                if not scores:
                    out[(q0 + i, hh)] = [0.0] * 512
                    lse[(q0 + i, hh)] = -math.inf
                    continue
                m = max(s for _, s in scores)
                wts = [(j, math.exp(s - m)) for j, s in scores]
                l = sum(w for _, w in wts)
                o = [0.0] * 512
                for j, w in wts:
                    row = rows[j]
                    for d in range(512):
                        o[d] += w * row[d]
                out[(q0 + i, hh)] = [x / l for x in o]
                lse[(q0 + i, hh)] = m + math.log(l)
    return out, lse


def _compare_brute(inst, out, lse, bo, bl):
    for (t, hh), ref in bo.items():
        np.testing.assert_allclose(out[t, hh], np.array(ref), rtol=2e-6, atol=1e-7)
        if math.isinf(bl[(t, hh)]):
            assert lse[t, hh] == -np.inf
        else:
            assert abs(lse[t, hh] - bl[(t, hh)]) <= 1e-5 * max(1.0, abs(bl[(t, hh)]))


@pytest.mark.parametrize("seed,prefix,trees,heads", [
    (11, [7], [3], 2),
    (12, [0], [4], 1),
    (13, [5, 0, 9], [2, 3, 1], 2),
    (14, [16, 3], [6, 0], 1),
])
def test_brute_force_tree_semantics(seed, prefix, trees, heads):
    """Ancestor-or-self trees: brute force derives visibility from the parent lists,
    not from custom_mask, so it pins the mask's orientation and indexing."""
    inst = gen.make_instance(prefix, trees, heads, num_slots=256, seed=seed)
    out, lse, rec = _run(inst)
    vis = lambda b, i, j: j < inst.prefix_lens[b] or \
        (j - inst.prefix_lens[b]) in _ancestors(inst.parents[b], i)
    bo, bl = _brute(inst, vis)
    _compare_brute(inst, out, lse, bo, bl)


def test_brute_force_arbitrary_masks_and_empty_rows():
    """Arbitrary (non-tree, asymmetric) masks, including rows that see nothing."""
    rng = np.random.default_rng(5)
    inst = gen.make_instance([0, 4], [5, 3], 2, num_slots=64, seed=21)
    dense = []
    for t in inst.tree_sizes:
        m = (rng.random((t, t)) < 0.4).astype(np.uint8)
        dense.append(m)
    dense[0][2, :] = 0          # request 0 has no prefix: node 2 sees no key at all
    inst.custom_mask = np.concatenate([m.reshape(-1) for m in dense])
    out, lse, _ = _run(inst)
    vis = lambda b, i, j: j < inst.prefix_lens[b] or bool(dense[b][i][j - inst.prefix_lens[b]])
    bo, bl = _brute(inst, vis)
    _compare_brute(inst, out, lse, bo, bl)
    assert np.all(out[2] == 0.0) and np.all(lse[2] == -np.inf)


def test_duplicate_slots_count_per_position():
    """A slot that appears twice in the key list is two keys."""
    inst = gen.make_instance([6], [2], 1, num_slots=64, seed=31)
    inst.kv_indices[3] = inst.kv_indices[1]
    out, lse, _ = _run(inst)
    vis = lambda b, i, j: j < 6 or (j - 6) in _ancestors(inst.parents[0], i)
    bo, bl = _brute(inst, vis)
    _compare_brute(inst, out, lse, bo, bl)


# ---------------------------------------------------------------- closed forms
def test_zero_query_gives_mean_of_visible_rows():
    inst = gen.make_instance([9], [4], 2, num_slots=128, seed=41)
    inst.q[:] = 0
    out, lse, rec = _run(inst)
    pool = inst.pool_view()
    keys = rec["keys"][0]
    vals = R.bf16_bits_to_f64(pool[keys])[:, :512]
    for i in range(4):
        vis = [j for j in range(9)] + [9 + k for k in _ancestors(inst.parents[0], i)]
        np.testing.assert_allclose(out[i], np.broadcast_to(vals[vis].mean(0), (2, 512)),
                                   rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(lse[i], math.log(len(vis)), rtol=1e-7)


def test_equal_value_rows_give_that_value():
    inst = gen.make_instance([5], [3], 1, num_slots=64, seed=42)
    c = gen.f32_to_bf16_bits(np.linspace(-2, 2, 512, dtype=np.float32))
    inst.rows[:, :512] = c       # every row shares V; rope dims stay random
    out, _, _ = _run(inst)
    np.testing.assert_allclose(out[:, 0], np.broadcast_to(R.bf16_bits_to_f64(c), (3, 512)),
                               rtol=1e-6, atol=1e-7)


def test_single_visible_key():
    """No prefix, each node sees only itself: out = own V row, lse = its score."""
    inst = gen.make_instance([0], [3], 2, num_slots=64, seed=43)
    inst.custom_mask = np.eye(3, dtype=np.uint8).reshape(-1)
    out, lse, _ = _run(inst)
    for i in range(3):
        row = R.bf16_bits_to_f64(inst.rows[i])
        for hh in range(2):
            qv = R.bf16_bits_to_f64(inst.q[i, hh])
            np.testing.assert_allclose(out[i, hh], row[:512], rtol=1e-7)
            assert abs(lse[i, hh] - inst.sm_scale * float(qv @ row)) < 1e-5


def test_hand_worked_three_keys():
    """q = e0, rows 2*e0, e1, e0+e2 (scale 1): scores 2, 0, 1."""
    inst = gen.make_instance([2], [1], 1, num_slots=8, seed=44)
    one = gen.f32_to_bf16_bits(np.float32([1.0]))[0]
    two = gen.f32_to_bf16_bits(np.float32([2.0]))[0]
    inst.q[:] = 0
    inst.q[0, 0, 0] = one
    inst.rows[:] = 0
    inst.rows[0, 0] = two
    inst.rows[1, 1] = one
    inst.rows[2, 0] = one
    inst.rows[2, 2] = one
    inst.sm_scale = 1.0
    out, lse, _ = _run(inst)
    z = math.exp(2) + 1 + math.e
    w0, w1, w2 = math.exp(2) / z, 1 / z, math.e / z
    expect = np.zeros(512)
    expect[0], expect[1], expect[2] = 2 * w0 + w2, w1, w2
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-7, atol=1e-9)
    assert abs(lse[0, 0] - math.log(z)) < 1e-6


def test_empty_key_set():
    inst = gen.make_instance([0], [2], 1, num_slots=8, seed=45)
    inst.custom_mask[:] = 0
    out, lse, _ = _run(inst)
    assert np.all(out == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------- textbook reductions
def _sdpa(q, k, v, mask, scale):
    qt = torch.from_numpy(q)[None]   # [1, H, L, 576]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale)
    return o[0].numpy()


def test_single_node_tree_is_decode_attention():
    inst = gen.make_instance([300], [1], 4, num_slots=1024, seed=51)
    out, lse, rec = _run(inst)
    kv = R.bf16_bits_to_f64(inst.pool_view()[rec["keys"][0]])
    q = R.bf16_bits_to_f64(inst.q[0])[:, None, :]                # [H, 1, 576]
    ref = _sdpa(q, kv[:, :576], kv[:, :512], np.ones((1, 301), bool), inst.sm_scale)
    np.testing.assert_allclose(out[0], ref[:, 0], rtol=1e-6, atol=1e-7)
    s = inst.sm_scale * (R.bf16_bits_to_f64(inst.q[0]) @ kv[:, :576].T)
    from scipy.special import logsumexp
    np.testing.assert_allclose(lse[0], logsumexp(s, axis=1), rtol=1e-6)


def test_chain_tree_is_causal_attention():
    """parent(i) = i-1: node i sits at position P+i and sees the prefix and chain[0..i]."""
    p, t = 40, 6
    inst = gen.make_instance([p], [t], 3, num_slots=128, seed=52, tree="chain")
    out, _, rec = _run(inst)
    kv = R.bf16_bits_to_f64(inst.pool_view()[rec["keys"][0]])
    q = R.bf16_bits_to_f64(inst.q).transpose(1, 0, 2)          # [H, T, 576]
    causal = np.tril(np.ones((t, p + t), bool), k=p)           # bottom-right aligned
    ref = _sdpa(q, kv[:, :576], kv[:, :512], causal, inst.sm_scale)
    np.testing.assert_allclose(out.transpose(1, 0, 2), ref, rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- invariants
def test_slot_permutation_is_bit_identical():
    inst = gen.make_instance([200, 57], [9, 5], 2, num_slots=1024, seed=61)
    out1, lse1, _ = _run(inst)
    perm = np.random.default_rng(3).permutation(inst.num_slots)
    inst.row_slots = perm[inst.row_slots]
    inst.kv_indices = perm[inst.kv_indices].astype(np.int32)
    inst.out_cache_loc = perm[inst.out_cache_loc].astype(np.int64)
    out2, lse2, _ = _run(inst)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


def test_topological_relabel_permutes_outputs():
    """Relabel the tree's nodes by another topological order: outputs follow."""
    inst = gen.make_instance([30], [5], 1, num_slots=128, seed=62)
    inst.parents = [[-1, 0, 0, 1, 2]]
    inst.custom_mask = gen.ancestor_or_self_mask(inst.parents[0]).reshape(-1)
    out1, lse1, _ = _run(inst)
    order = [0, 2, 1, 4, 3]                 # new label n holds old node order[n]
    new_parents = [-1 if inst.parents[0][o] < 0 else order.index(inst.parents[0][o])
                   for o in order]
    inst2 = gen.make_instance([30], [5], 1, num_slots=128, seed=62)
    inst2.q = inst.q[order]
    inst2.out_cache_loc = inst.out_cache_loc[order]
    inst2.custom_mask = gen.ancestor_or_self_mask(new_parents).reshape(-1)
    out2, lse2, _ = _run(inst2)
    np.testing.assert_allclose(out2, out1[order], rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(lse2, lse1[order], rtol=1e-7)


def test_head_independence():
    inst = gen.make_instance([64], [4], 4, num_slots=256, seed=63)
    out, lse, _ = _run(inst)
    for hh in range(4):
        one = gen.make_instance([64], [4], 4, num_slots=256, seed=63)
        one.q = np.ascontiguousarray(inst.q[:, hh:hh + 1])
        one.num_heads = 1
        o1, l1, _ = _run(one)
        assert np.array_equal(o1[:, 0], out[:, hh]) and np.array_equal(l1[:, 0], lse[:, hh])


def test_lse_merge_over_disjoint_key_halves():
    """Full result == merge(first half of prefix, second half + tree)."""
    inst = gen.make_instance([50], [6], 2, num_slots=256, seed=64)
    out, lse, _ = _run(inst)
    a = gen.make_instance([50], [6], 2, num_slots=256, seed=64)
    a.kv_indices = inst.kv_indices[:23].copy()
    a.kv_indptr = np.array([0, 23], np.int32)
    a.custom_mask = np.zeros_like(inst.custom_mask)
    b = gen.make_instance([50], [6], 2, num_slots=256, seed=64)
    b.kv_indices = inst.kv_indices[23:].copy()
    b.kv_indptr = np.array([0, 27], np.int32)
    oa, la, _ = _run(a)
    ob, lb, _ = _run(b)
    mo, ml = R.lse_merge([(oa, la), (ob, lb)])
    np.testing.assert_allclose(mo, out, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(ml, lse, rtol=1e-6)


def test_lse_merge_empty_parts():
    o = np.ones((2, 512))
    mo, ml = R.lse_merge([(o, np.array([-np.inf, 1.0])), (2 * o, np.array([-np.inf, -np.inf]))])
    assert np.all(mo[0] == 0) and ml[0] == -np.inf
    assert np.allclose(mo[1], 1.0) and ml[1] == 1.0


# ---------------------------------------------------------------- metadata literals
def _golden_trees():
    with open(os.path.join(GOLDEN, "tree_ancestor_words.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("|")
            parents = [int(x) for x in lhs.split(",")]
            words = [int(w, 2) for w in rhs.split()]
            yield parents, words


@pytest.mark.parametrize("parents,words", list(_golden_trees()))
def test_ancestor_words_literal(parents, words):
    t = len(parents)
    mask = gen.ancestor_or_self_mask(parents).reshape(-1)
    got = R.ancestor_words(0, np.array([0, t]), mask, np.array([0, t * t]))
    assert [int(x) for x in got] == words


def test_combined_key_order():
    inst = gen.make_instance([3, 2], [2, 1], 1, num_slots=64, seed=71)
    keys0 = R.request_keys(0, inst.qo_indptr, inst.kv_indptr, inst.kv_indices, inst.out_cache_loc)
    keys1 = R.request_keys(1, inst.qo_indptr, inst.kv_indptr, inst.kv_indices, inst.out_cache_loc)
    assert list(keys0) == list(inst.kv_indices[:3]) + list(inst.out_cache_loc[:2])
    assert list(keys1) == list(inst.kv_indices[3:5]) + list(inst.out_cache_loc[2:3])


# ---------------------------------------------------------------- planted mistakes
MUTANTS = {
    "v_slice_offset": ("v_mat = kv[:, :D_V]", "v_mat = kv[:, D_QK - D_V:]"),
    "mask_transposed": ("custom_mask[base + i * t + k]", "custom_mask[base + k * t + i]"),
    "scale_dropped": ("s = scale * (qn @ k_mat.T)", "s = (qn @ k_mat.T)"),
    "tree_keys_reversed": ("tree = np.asarray(out_cache_loc[q0:q1], dtype=np.int64)",
                           "tree = np.asarray(out_cache_loc[q0:q1], dtype=np.int64)[::-1]"),
    "prefix_masked_as_tree": ("vis = np.ones((n, p_b + t_b), dtype=bool)",
                              "vis = np.zeros((n, p_b + t_b), dtype=bool)"),
    "lse_missing_max": ("lrow = m_safe[:, 0] + np.log(", "lrow = 0.0 + np.log("),
    "heads_transposed": ("qn = qn.reshape(n * h, D_QK)",
                         "qn = qn.transpose(1, 0, 2).reshape(n * h, D_QK)"),
    "rope_dropped": ("kv = bf16_bits_to_f64(pool[keys])[:, :D_QK]",
                     "kv = bf16_bits_to_f64(pool[keys])[:, :D_QK].copy(); kv[:, D_V:] = 0"),
}


def _mutant_module(old, new):
    src = inspect.getsource(R)
    assert old in src, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    """Each planted mistake in a copy of the oracle must fail the brute-force pin."""
    mod = _mutant_module(*MUTANTS[name])
    inst = gen.make_instance([6, 3], [4, 3], 2, num_slots=64, seed=81)
    inst.parents = [[-1, 0, 0, 1], [-1, 0, 1]]
    inst.custom_mask = np.concatenate([gen.ancestor_or_self_mask(p).reshape(-1)
                                       for p in inst.parents])
    out, lse, _ = mod.mla_verify_reference(inst.q, inst.pool_view(), inst.qo_indptr,
                                           inst.kv_indptr, inst.kv_indices, inst.out_cache_loc,
                                           inst.custom_mask, inst.mask_indptr,
                                           inst.num_heads, inst.sm_scale)
    vis = lambda b, i, j: j < inst.prefix_lens[b] or \
        (j - inst.prefix_lens[b]) in _ancestors(inst.parents[b], i)
    bo, bl = _brute(inst, vis)
    with pytest.raises(AssertionError):
        _compare_brute(inst, out, lse, bo, bl)
