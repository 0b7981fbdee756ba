"""Scalar brute-force oracle (pure Python loops, float64) for tiny shapes.

TEST INFRASTRUCTURE ONLY (see ``oracle/ref.py`` for who may import it).

Written independently of ``oracle/ref.py``: every quantity is an explicit
loop over indices, one token and one head at a time, with ``math`` scalars, so
that a vectorisation slip in ``ref`` (a transposed operand, a wrong axis, a
broadcasting accident) shows up as a mismatch.  The steps follow the same pages:
LLaMABlock / LLaMAAttention / LLaMAMLP / LLaMARMSNorm / LLaMARoPE (section 二 of
"LLaMA架构深度解析…"), the MLX attention-with-cache fragment and the RoPE
traditional flag of "iOS设备上运行LLaMA2-13B…".
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence


def _mat(w) -> List[List[float]]:
    return [[float(v) for v in row] for row in w]


def matvec(w: List[List[float]], x: Sequence[float]) -> List[float]:
    """y[o] = sum_k W[o][k] x[k] (nn.Linear [out, in])."""
    return [sum(row[k] * x[k] for k in range(len(x))) for row in w]


def rmsnorm_vec(x: Sequence[float], g: Sequence[float], eps: float) -> List[float]:
    ss = 0.0
    for v in x:
        ss += v * v
    r = 1.0 / math.sqrt(ss / len(x) + eps)
    return [g[i] * x[i] * r for i in range(len(x))]


def rope_head(u: Sequence[float], pos: int, theta: float, traditional: bool) -> List[float]:
    d = len(u)
    out = list(u)
    for i in range(d // 2):
        ang = pos * theta ** (-(2.0 * i) / d)
        c, s = math.cos(ang), math.sin(ang)
        ia, ib = (2 * i, 2 * i + 1) if traditional else (i, i + d // 2)
        a, b = u[ia], u[ib]
        out[ia] = a * c - b * s
        out[ib] = a * s + b * c
    return out


def silu(z: float) -> float:
    return z / (1.0 + math.exp(-z))


def attend_one(q: Sequence[float], keys: Sequence[Sequence[float]], vals: Sequence[Sequence[float]]) -> List[float]:
    """softmax over the given (already causally limited) keys, then weight values."""
    d = len(q)
    scores = []
    for kk in keys:
        scores.append(sum(q[t] * kk[t] for t in range(d)) / math.sqrt(d))
    m = max(scores)
    e = [math.exp(s - m) for s in scores]
    z = sum(e)
    out = [0.0] * d
    for j, vv in enumerate(vals):
        for t in range(d):
            out[t] += e[j] / z * vv[t]
    return out


def block(x, w: Dict[str, object], shape, k_cache=None, v_cache=None) -> Dict[str, list]:
    """x: [B][L][D] nested lists/arrays; caches [B][S][G][d]. Returns y, k_new, v_new."""
    D, H, G = shape.dim, shape.n_heads, shape.n_kv_heads
    d = D // H
    rep = H // G
    wq, wk, wv, wo = (_mat(w[k]) for k in ("wq", "wk", "wv", "wo"))
    w1, w2, w3 = (_mat(w[k]) for k in ("w1", "w2", "w3"))
    g1 = [float(v) for v in w["attention_norm"]]
    g2 = [float(v) for v in w["ffn_norm"]]
    ys, kns, vns = [], [], []
    for b in range(len(x)):
        keys = [] if k_cache is None else [[[float(t) for t in kv] for kv in tok] for tok in k_cache[b]]
        vals = [] if v_cache is None else [[[float(t) for t in kv] for kv in tok] for tok in v_cache[b]]
        S = len(keys)
        y_b, kn_b, vn_b = [], [], []
        # every new token's K/V first (a later query may need an earlier new token)
        qs = []
        for l in range(len(x[b])):
            xl = [float(v) for v in x[b][l]]
            xn = rmsnorm_vec(xl, g1, shape.eps)
            qf, kf, vf = matvec(wq, xn), matvec(wk, xn), matvec(wv, xn)
            p = S + l
            qs.append([rope_head(qf[h * d:(h + 1) * d], p, shape.rope_theta, shape.traditional) for h in range(H)])
            kt = [rope_head(kf[g * d:(g + 1) * d], p, shape.rope_theta, shape.traditional) for g in range(G)]
            vt = [vf[g * d:(g + 1) * d] for g in range(G)]
            keys.append(kt)
            vals.append(vt)
            kn_b.append(kt)
            vn_b.append(vt)
        for l in range(len(x[b])):
            p = S + l
            o = []
            for h in range(H):
                g = h // rep
                o.extend(attend_one(qs[l][h], [keys[j][g] for j in range(p + 1)],
                                    [vals[j][g] for j in range(p + 1)]))
            xl = [float(v) for v in x[b][l]]
            att = matvec(wo, o)
            hres = [xl[i] + att[i] for i in range(D)]
            hn = rmsnorm_vec(hres, g2, shape.eps)
            a, c = matvec(w1, hn), matvec(w3, hn)
            gate = [silu(a[i]) * c[i] for i in range(len(a))]
            f = matvec(w2, gate)
            y_b.append([hres[i] + f[i] for i in range(D)])
        ys.append(y_b)
        kns.append(kn_b)
        vns.append(vn_b)
    return {"y": ys, "k_new": kns, "v_new": vns}


def dequant_q4(codes, scales, biases, group: int) -> List[List[float]]:
    out = []
    for o in range(len(codes)):
        row = []
        for k in range(len(codes[o])):
            row.append(float(scales[o][k // group]) * int(codes[o][k]) + float(biases[o][k // group]))
        out.append(row)
    return out
