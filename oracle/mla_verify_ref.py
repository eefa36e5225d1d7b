"""CPU oracle for tree-masked MLA verify attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this module.  The product path (the HIP library and its Python binding) never
calls it, and this module shares no code with that path.

What it computes is the plain definition of the verify step: every draft-tree
query token, per head, attends with an exact softmax over its request's prefix
latent rows (all visible) followed by its own tree nodes (visible where the
request's custom mask says so), and reduces V = the first 512 latent dims.

  * the kernel reads the pool through kv_indices / out_cache_loc directly
    instead of gathering to contiguous memory ("The Integration Chasm",
    The Decision: Adapt the Kernel, Not the System);
  * the combined key order is the prefix indices followed by the draft tokens'
    cache locations ("The Capture-Safe Kernel", The Core Problem);
  * per-request prefix length is kv_indptr[b+1] - kv_indptr[b]
    ("The Capture-Safe Kernel", Decision 2);
  * the tree visibility comes from the raw custom_mask at offset
    mask_indptr[b] ("The Capture-Safe Kernel", Decision 5);
  * the draft rows are already in the pool when attention runs
    ("The Launch Wrapper", The KV Cache Ordering Insight).

Readings where the pages are silent (listed with the rest in the design notes):
the mask block of request b is T_b x T_b uint8, row-major (row = query node,
column = key node), nonzero = visible, with no implicit diagonal; the prefix is
never masked; V is the first 512 of 576 latent dims; the softmax scale is an
input; LSE is the natural log of the sum of exp of the scaled scores; a row with
no visible key gives out = 0 and lse = -inf; a repeated slot counts once per
position.

Arithmetic: bf16 bits -> float64 exactly, float64 matmuls and exp/log, results
rounded once to float32.
"""
from __future__ import annotations

import numpy as np

D_QK = 576
D_V = 512


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 (uint16 bits) -> float64, exactly: the bits are the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def request_keys(b, qo_indptr, kv_indptr, kv_indices, out_cache_loc):
    """Combined key list of request b: its prefix slots, then its tree nodes' slots
    ("The Capture-Safe Kernel", The Core Problem; Decision 2)."""
    k0, k1 = int(kv_indptr[b]), int(kv_indptr[b + 1])
    q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
    prefix = np.asarray(kv_indices[k0:k1], dtype=np.int64)
    tree = np.asarray(out_cache_loc[q0:q1], dtype=np.int64)
    return np.concatenate([prefix, tree])


def ancestor_words(b, qo_indptr, custom_mask, mask_indptr):
    """Packed tree visibility of request b's nodes: bit k of word i is set when
    custom_mask[mask_indptr[b] + i*T + k] != 0 ("The Capture-Safe Kernel", Decision 5)."""
    q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
    t = q1 - q0
    base = int(mask_indptr[b])
    words = np.zeros(t, dtype=np.uint64)
    for i in range(t):
        w = 0
        for k in range(t):
            if custom_mask[base + i * t + k] != 0:
                w |= 1 << k
        words[i] = np.uint64(w)
    return words


def mla_verify_reference(q, pool, qo_indptr, kv_indptr, kv_indices, out_cache_loc,
                         custom_mask, mask_indptr, num_heads, sm_scale, tokens=None):
    """Exact tree-masked verify attention.

    q: uint16 bf16 bits [sumT, H, >=576]; pool: indexable by an int64 slot array,
    returning uint16 bf16 bits [n, >=576].  ``tokens``: optional iterable of
    query-token indices to compute (others stay NaN) for sampled checks.

    Returns (out float32 [sumT, H, 512], lse float32 [sumT, H], record) where
    record = {"keys": [combined slot list per request], "anc": uint64 [sumT]}.
    """
    qo_indptr = np.asarray(qo_indptr)
    batch = len(qo_indptr) - 1
    total_q = int(qo_indptr[-1])
    h = int(num_heads)
    out = np.full((total_q, h, D_V), np.nan, dtype=np.float32)
    lse = np.full((total_q, h), np.nan, dtype=np.float32)
    anc_all = np.zeros(total_q, dtype=np.uint64)
    keys_all = []
    want = None if tokens is None else set(int(t) for t in tokens)
    scale = float(sm_scale)
    for b in range(batch):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        t_b = q1 - q0
        p_b = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        keys = request_keys(b, qo_indptr, kv_indptr, kv_indices, out_cache_loc)
        keys_all.append(keys)
        anc = ancestor_words(b, qo_indptr, custom_mask, mask_indptr)
        anc_all[q0:q1] = anc
        nodes = [i for i in range(t_b) if want is None or (q0 + i) in want]
        if not nodes:
            continue
        kv = bf16_bits_to_f64(pool[keys])[:, :D_QK]          # [N, 576]
        k_mat = kv
        v_mat = kv[:, :D_V]                                  # V = first 512 dims
        n = len(nodes)
        # visibility [n, N]: prefix always visible, tree columns from the mask
        vis = np.ones((n, p_b + t_b), dtype=bool)
        for r, i in enumerate(nodes):
            for k in range(t_b):
                vis[r, p_b + k] = bool((int(anc[i]) >> k) & 1)
        qn = bf16_bits_to_f64(np.asarray(q)[[q0 + i for i in nodes], :, :D_QK])
        qn = qn.reshape(n * h, D_QK)                         # row = node*H + head
        s = scale * (qn @ k_mat.T)                           # [n*H, N]
        vis_rows = np.repeat(vis, h, axis=0)
        s = np.where(vis_rows, s, -np.inf)
        m = s.max(axis=1, keepdims=True) if s.shape[1] else np.full((n * h, 1), -np.inf)
        empty = ~np.isfinite(m[:, 0])
        m_safe = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m_safe)                               # masked -> exp(-inf) = 0
        l = e.sum(axis=1, keepdims=True)
        o = (e @ v_mat) / np.where(l > 0, l, 1.0)
        lrow = m_safe[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0))
        o[empty] = 0.0
        lrow[empty] = -np.inf
        out[[q0 + i for i in nodes]] = o.reshape(n, h, D_V).astype(np.float32)
        lse[[q0 + i for i in nodes]] = lrow.reshape(n, h).astype(np.float32)
    return out, lse, {"keys": keys_all, "anc": anc_all}


def lse_merge(parts):
    """Combine results computed over disjoint key sets of the same query rows.

    parts: list of (out [..., 512] float64, lse [...] float64), each a normalised
    softmax-weighted mean with its log-sum-exp.  The merged row weights part s by
    exp(lse_s - lse*) where lse* = log sum_s exp(lse_s); parts with lse = -inf
    carry no weight, and an all-empty row gives out = 0, lse = -inf.  This is the
    reduction of partial softmax statistics across KV splits
    ("The Capture-Safe Kernel", Decision 4; "The Integration Chasm", Context).
    """
    lses = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])
    outs = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - m_safe), 0.0)
    total = w.sum(axis=0)
    merged = (w[..., None] * outs).sum(axis=0) / np.where(total > 0, total, 1.0)[..., None]
    merged = np.where(finite[..., None], merged, 0.0)
    lse = np.where(finite, m_safe + np.log(np.where(total > 0, total, 1.0)), -np.inf)
    return merged, lse
