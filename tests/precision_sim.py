"""CPU emulation of the split-partial kernel's rounding points, to choose how P
enters the PV product.  TEST INFRASTRUCTURE (not the oracle, and not the
product path).

What is emulated, per query row: scores S = q . k from bf16 inputs with fp32
accumulation; base-2 scaled scores s = fp32(S * scale * log2 e); 32-key tiles
with an online softmax whose reference max moves only when a tile max exceeds
it by more than 8 (so p = 2^(s - m) <= 2^8); the row sum l accumulated from
the fp32 p; O += P . V accumulated in fp32, with P in one of these forms:

  fp32       P as computed (the simulator's own floor)
  bf16       P rounded to bf16 (one bf16 MFMA)
  bf16x2     P = hi + lo, hi = bf16(p), lo = bf16(p - hi) (two bf16 MFMAs)
  bf16x2t    the same with hi = p cut to its top 16 bits (the kernel)
  fp16       P and V rounded to fp16 (one fp16 MFMA; V's bf16 values convert exactly
             unless they fall outside fp16's normal range)
  bf16+e4m3  hi as bf16, lo scaled by 2^9, rounded to OCP fp8 e4m3 (saturating), against V in
             e4m3 (a bf16 MFMA plus an fp8 one at twice the rate)

then out = O / l and lse = (m + log2 l) ln 2.  One key range per row (the
merge of several ranges adds fp32 roundings far below the gate).  Scored with
the parity gate against the fp64 oracle.

Run as a script to print the table for every workload:
    python -m tests.precision_sim
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import mla_verify_ref as R

SCHEMES = ("fp32", "bf16", "bf16x2", "bf16x2t", "fp16", "bf16+e4m3")
LOG2E = 1.4426950408889634


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP fp8 E4M3 (3 mantissa bits, exponent bias 7,
    subnormals down to 2^-9, saturating at 448), nearest-even, as float32."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # the spacing of representable values around a: 2^(e - 3) for normals
    # (e = floor(log2 a) >= -6), 2^-9 for subnormals
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = 2.0 ** (e - 3)
    q = np.round(a / step) * step          # numpy rounds half to even
    q = np.minimum(q, 448.0)
    return (np.sign(x) * q).astype(np.float32)


def trunc_bf16(x: np.ndarray) -> np.ndarray:
    """float32 cut to its top 16 bits (a bf16 value, rounded toward zero)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u & np.uint32(0xFFFF0000)).view(np.float32)


def simulate(inst, scheme: str, tile: int = 32, slack: float = 8.0):
    """Emulated kernel output (out [sumT, H, 512] float32, lse [sumT, H] float32)."""
    h = inst.num_heads
    total_q = inst.total_q
    out = np.zeros((total_q, h, 512), np.float32)
    lse = np.zeros((total_q, h), np.float32)
    pool = inst.pool_view()
    scale2 = np.float32(np.float32(inst.sm_scale) * np.float32(LOG2E))
    for b in range(inst.batch):
        q0, q1 = int(inst.qo_indptr[b]), int(inst.qo_indptr[b + 1])
        t = q1 - q0
        if t == 0:
            continue
        p_len = int(inst.kv_indptr[b + 1]) - int(inst.kv_indptr[b])
        keys = R.request_keys(b, inst.qo_indptr, inst.kv_indptr, inst.kv_indices, inst.out_cache_loc)
        anc = R.ancestor_words(b, inst.qo_indptr, inst.custom_mask, inst.mask_indptr)
        kv = R.bf16_bits_to_f64(pool[keys])[:, :576].astype(np.float32)
        v = kv[:, :512]
        v16 = v.astype(np.float16).astype(np.float32)
        v8 = to_e4m3(v)
        q = R.bf16_bits_to_f64(np.asarray(inst.q)[q0:q1, :, :576]).astype(np.float32).reshape(t * h, 576)
        s = (q.astype(np.float64) @ kv.T.astype(np.float64)).astype(np.float32) * scale2
        n = s.shape[1]
        vis = np.ones((t, n), bool)
        for i in range(t):
            for k in range(t):
                vis[i, p_len + k] = bool((int(anc[i]) >> k) & 1)
        s = np.where(np.repeat(vis, h, axis=0), s, np.float32(-np.inf))
        rows = t * h
        m = np.full(rows, -np.inf, np.float32)
        l = np.zeros(rows, np.float32)
        o = np.zeros((rows, 512), np.float32)
        for k0 in range(0, n, tile):
            st = s[:, k0:k0 + tile]
            mt = st.max(axis=1)
            need = mt > m + np.float32(slack)
            if need.any():
                m_new = np.where(need, mt, m)
                alpha = np.where(m == -np.inf, np.float32(0), np.exp2(m - m_new)).astype(np.float32)
                alpha = np.where(need, alpha, np.float32(1))
                l *= alpha
                o *= alpha[:, None]
                m = m_new
            m_use = np.where(m == -np.inf, np.float32(0), m)
            p = np.exp2(st - m_use[:, None]).astype(np.float32)
            l += p.sum(axis=1, dtype=np.float32)
            vt = v[k0:k0 + tile]
            if scheme == "fp32":
                o += p @ vt
            elif scheme == "bf16":
                o += to_bf16(p) @ vt
            elif scheme == "bf16x2":
                hi = to_bf16(p)
                lo = to_bf16(p - hi)
                o += hi @ vt
                o += lo @ vt
            elif scheme == "bf16x2t":
                hi = trunc_bf16(p)
                lo = to_bf16(p - hi)
                o += hi @ vt
                o += lo @ vt
            elif scheme == "fp16":
                o += p.astype(np.float16).astype(np.float32) @ v16[k0:k0 + tile]
            elif scheme == "bf16+e4m3":
                hi = to_bf16(p)
                lo8 = to_e4m3((p - hi) * np.float32(512.0))
                o += hi @ vt
                o += (lo8 @ v8[k0:k0 + tile]) * np.float32(1.0 / 512.0)
            else:
                raise ValueError(scheme)
        empty = m == -np.inf
        res = np.where(empty[:, None], np.float32(0), o / np.where(l > 0, l, 1)[:, None])
        lrow = np.where(empty, -np.inf, (m + np.log2(np.where(l > 0, l, 1))) * np.float32(np.log(2.0)))
        out[q0:q1] = res.reshape(t, h, 512).astype(np.float32)
        lse[q0:q1] = lrow.reshape(t, h).astype(np.float32)
    return out, lse


def gate(out, lse, ref_out, ref_lse):
    o = out.astype(np.float64)
    r = ref_out.astype(np.float64)
    diff = np.abs(o - r)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126))) - 7)
    fin = np.isfinite(ref_lse)
    return {"max_abs": float(diff.max()), "frac_2ulp": float((diff <= 2 * ulp).mean()),
            "lse_max_abs": float(np.abs(lse[fin].astype(np.float64) - ref_lse[fin]).max()) if fin.any() else 0.0}


def passes(st) -> bool:
    return st["max_abs"] <= 1e-2 and st["frac_2ulp"] >= 0.999 and st["lse_max_abs"] <= 1e-3


def main(names):
    from workloads import gen
    print(f"{'workload':<18} {'scheme':<10} {'max_abs':>10} {'frac_2ulp':>10} {'lse_max':>10}  gate")
    for name in names:
        inst = gen.segmented_replay(0) if name == "segmented_r0" else gen.config(name)
        pool = gen.segmented_pool() if name == "segmented_r0" else None
        if pool is not None:
            class _P:   # the dense pool stands in for the view
                def __init__(self, a):
                    self.a = a

                def pool_view(self):
                    return self.a
            inst.pool_view = _P(pool).pool_view
        ref_out, ref_lse, _ = R.mla_verify_reference(inst.q, inst.pool_view(), inst.qo_indptr, inst.kv_indptr,
                                                     inst.kv_indices, inst.out_cache_loc, inst.custom_mask,
                                                     inst.mask_indptr, inst.num_heads, inst.sm_scale)
        for scheme in SCHEMES:
            st = gate(*simulate(inst, scheme), ref_out, ref_lse)
            print(f"{name:<18} {scheme:<10} {st['max_abs']:>10.3e} {st['frac_2ulp']:>10.6f} "
                  f"{st['lse_max_abs']:>10.3e}  {'pass' if passes(st) else 'FAIL'}", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["tiny", "p5632_t16", "p23040_t32", "p91136_t32", "p91136_t32_h64",
                          "decode_b32_h16", "decode_b64_h128", "segmented_r0"])
