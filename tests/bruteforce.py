"""50-digit decimal brute force for tiny inputs: an independent check on the
fp64 oracle.

Written separately from the oracle: its own bf16 widening (via ``struct``), its
own walk over the block table, and the literal softmax exp(s_t) / sum exp(s)
with no max shift (50 digits leave ample headroom for the small scores used).
"""
from __future__ import annotations

import struct
from decimal import Decimal, getcontext

import numpy as np

getcontext().prec = 50


def _widen(a: np.ndarray):
    """Exact Decimal values of an fp32 array or of bf16 bit patterns (uint16)."""
    flat = a.reshape(-1)
    if a.dtype == np.uint16:
        return [Decimal(struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]) for b in flat]
    return [Decimal(float(x)) for x in flat]


def _attend(qv, keys, vals, scale):
    """softmax(scale * q.k) weighted sum of vals, literal form."""
    if not keys:
        return [Decimal(0)] * len(qv)
    es = [(scale * sum(a * b for a, b in zip(qv, k))).exp() for k in keys]
    tot = sum(es)
    return [sum(e * v[c] for e, v in zip(es, vals)) / tot for c in range(len(qv))]


def decode(q, k_cache, v_cache, block_table, cache_seqlens, k_new=None, v_new=None, scale=None):
    """Returns (out [B, Hq, D] as float, k_cache', v_cache') without touching inputs."""
    B, _, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    G = Hq // Hkv
    scale = Decimal(scale) if scale is not None else Decimal(1) / Decimal(D).sqrt()
    kc = k_cache.copy()
    vc = v_cache.copy()
    if k_new is not None:
        for i in range(B):
            p = int(cache_seqlens[i])
            pb = int(block_table[i][p // bs])
            kc[pb, p % bs] = k_new[i, 0]
            vc[pb, p % bs] = v_new[i, 0]
    Qd = np.array(_widen(q), dtype=object).reshape(q.shape)
    Kd = np.array(_widen(kc), dtype=object).reshape(kc.shape)
    Vd = np.array(_widen(vc), dtype=object).reshape(vc.shape)
    out = np.zeros((B, Hq, D))
    for i in range(B):
        n = int(cache_seqlens[i]) + (1 if k_new is not None else 0)
        for h in range(Hq):
            g = h // G
            keys, vals = [], []
            for t in range(n):
                pb = int(block_table[i][t // bs])
                keys.append(list(Kd[pb, t % bs, g]))
                vals.append(list(Vd[pb, t % bs, g]))
            o = _attend(list(Qd[i, 0, h]), keys, vals, scale)
            out[i, h] = [float(x) for x in o]
    return out, kc, vc


def varlen(q, k, v, cu_q, cu_k, scale=None):
    """q [Tq, Hq, D], k/v [Tk, Hkv, D]; returns out [Tq, Hq, D] as float."""
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = Decimal(scale) if scale is not None else Decimal(1) / Decimal(D).sqrt()
    Qd = np.array(_widen(q), dtype=object).reshape(q.shape)
    Kd = np.array(_widen(k), dtype=object).reshape(k.shape)
    Vd = np.array(_widen(v), dtype=object).reshape(v.shape)
    out = np.zeros((Tq, Hq, D))
    for b in range(len(cu_q) - 1):
        for r in range(cu_q[b], cu_q[b + 1]):
            for h in range(Hq):
                g = h // G
                keys = [list(Kd[c, g]) for c in range(cu_k[b], cu_k[b + 1])]
                vals = [list(Vd[c, g]) for c in range(cu_k[b], cu_k[b + 1])]
                out[r, h] = [float(x) for x in _attend(list(Qd[r, h]), keys, vals, scale)]
    return out
