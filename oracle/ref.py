"""CPU oracle for the LLaMA-style pre-norm decoder block (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``decoder_block_rmsnorm_amd``) never imports, calls or links it, and it imports
nothing from the product path.

Every function is the plain definition of one step, in float64, with no
blocking, fusion or reordering beyond what the definition states.  The pages
cited below are:

* "iOS设备上运行LLaMA2-13B：基于苹果MLX框架的完整技术指南" (geoz.com.cn)
  -- sections "LLaMA 2 的结构分析" (module tree), "模型配置" (config.json),
  "核心模块实现" 2-5 (attention with KV cache, FeedForward, RMSNorm, causal
  mask) and "生成过程" (generation loop, greedy and sampled).
* "LLaMA架构深度解析：从开源大模型设计到高效推理的工程实现全流程"
  (developer.cloud.tencent.com.cn) -- section 二 (LLaMARMSNorm, LLaMARoPE,
  LLaMAAttention, LLaMAMLP, LLaMABlock, LLaMA classes, LLaMA.generate).
* "老码农和你一起学AI系列：关于LLaMA解码器" (jsqmd.com) -- sections
  "解码器块的核心组件" and "数据流动" (pre-norm data flow).
* "《Hands-On Large Language Models》阅读笔记(二)" (yanbin.blog) -- sections
  "第三章" (prefill / decode), "流处理与 KV Cache".

Readings taken where the pages are silent or disagree (each is listed with its
reason in the design notes of the repository):

* norm placement is pre-norm only (two norms per block);
* RoPE "traditional" = adjacent pairs (2i, 2i+1) with the same frequencies and
  rotation sign as the rotate-half form;
* GQA maps query head h to kv head floor(h / n_rep);
* future keys are excluded (weight exactly 0); a sliding window W keeps the
  W most recent positions, the query's own included;
* 4-bit weights dequantize as scale * code + bias per group of 64 inputs;
* a sampled token is chosen by a given uniform u, cumulative mass taken in
  vocabulary order; ties with the last nucleus token are kept.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# RMSNorm -- "4. RMSNorm" (MLX page) and LLaMARMSNorm (page 二):
# divide each row by sqrt(mean of squares + eps), then multiply by the weight.
# ---------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(weight, dtype=F64) * (x / np.sqrt(ms + eps))


# ---------------------------------------------------------------------------
# Linear layers: nn.Linear convention W[out, in], no bias (LLaMAAttention and
# LLaMAMLP on page 二 build every projection with bias=False).
# ---------------------------------------------------------------------------
def dequant_q4(lin: Dict[str, np.ndarray], codes: Optional[np.ndarray] = None) -> np.ndarray:
    """4-bit group-affine weights -> dense float64 [out, in].

    W[o, k] = scale[o, k // g] * code[o, k] + bias[o, k // g]; group g = 64 and
    4 bits per the MLX quantization config ("模型配置" on the MLX page).  The
    products and sums are exact in float64 for bf16 scales/biases and 4-bit codes.
    """
    if codes is None:
        from workloads import unpack_q4_codes
        codes = unpack_q4_codes(lin["packed"])
    g = int(lin["group"])
    n, k = codes.shape
    s = np.asarray(lin["scales"], dtype=F64)[:, :, None]      # one scale and bias per group
    b = np.asarray(lin["biases"], dtype=F64)[:, :, None]
    return (s * codes.reshape(n, k // g, g).astype(F64) + b).reshape(n, k)


def weight_matrix(w) -> np.ndarray:
    if isinstance(w, dict):
        return dequant_q4(w)
    return np.asarray(w, dtype=F64)


def linear(x: np.ndarray, w) -> np.ndarray:
    """y = x W^T."""
    return np.asarray(x, dtype=F64) @ weight_matrix(w).T


# ---------------------------------------------------------------------------
# RoPE -- LLaMARoPE (page 二): inv_freq_i = theta^(-2i/d), angle = pos * inv_freq_i,
# out = u cos + rotate(u) sin with rotate(u) = [-u2, u1] over the two halves.
# The MLX module tree prints RoPE(128, traditional=True): the same rotation on
# adjacent pairs (2i, 2i+1).  Offset = number of cached tokens ("2. 注意力机制",
# KV cache fragment on the MLX page).
# ---------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=F64)
    return theta ** (-2.0 * i / head_dim)


def apply_rope(u: np.ndarray, positions: np.ndarray, theta: float, traditional: bool) -> np.ndarray:
    """u: [..., n_tok, n_heads, d]; positions: [..., n_tok] -> rotated copy."""
    u = np.asarray(u, dtype=F64)
    d = u.shape[-1]
    ang = np.asarray(positions, dtype=F64)[..., None] * rope_inv_freq(d, theta)  # [..., n_tok, d/2]
    c = np.cos(ang)[..., None, :]
    s = np.sin(ang)[..., None, :]
    out = np.empty_like(u)
    if traditional:
        a, b = u[..., 0::2], u[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = b * c + a * s
    else:
        h = d // 2
        a, b = u[..., :h], u[..., h:]
        out[..., :h] = a * c - b * s
        out[..., h:] = b * c + a * s
    return out


# ---------------------------------------------------------------------------
# Attention -- softmax(Q K^T / sqrt(d)) V ("LLaMA 2 的结构分析" and
# "2. 注意力机制" on the MLX page; LLaMAAttention on page 二), causal ("5. 因果掩码":
# a query never sees a later key), grouped-query: kv head shared by n_rep
# consecutive query heads (the expand-then-reshape of LLaMAAttention).
# ---------------------------------------------------------------------------
def kv_head_of(h: int, n_heads: int, n_kv_heads: int) -> int:
    return h // (n_heads // n_kv_heads)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, window: int = 0) -> np.ndarray:
    """One sequence.

    q: [L, H, d] (post-RoPE), k, v: [S, G, d] with key j at position j,
    q_pos: [L] absolute positions; query i attends keys j <= q_pos[i], and
    with a sliding window W > 0 only keys j > q_pos[i] - W (the W most recent
    positions, its own included: the sliding-window attention named in
    "流处理与 KV Cache" of the reading-notes page, whose window rule the pages
    leave open).
    Returns [L, H, d].
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    L, H, d = q.shape
    G = k.shape[1]
    out = np.zeros((L, H, d), dtype=F64)
    scale = 1.0 / np.sqrt(d)
    for h in range(H):
        g = kv_head_of(h, H, G)
        s = (q[:, h, :] @ k[:, g, :].T) * scale             # [L, S]
        j = np.arange(k.shape[0])
        allowed = j[None, :] <= np.asarray(q_pos)[:, None]
        if window > 0:
            allowed &= j[None, :] > np.asarray(q_pos)[:, None] - window
        s = np.where(allowed, s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        p = np.exp(s - m)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def softmax_rows(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=F64)
    m = np.max(s, axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / np.sum(p, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# SwiGLU feed-forward -- "3. 前馈网络" (MLX page) and LLaMAMLP (page 二):
# f = w2( silu(w1 x) * (w3 x) ), silu(z) = z / (1 + exp(-z)).
# ---------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=F64)
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(x: np.ndarray, w1, w2, w3) -> np.ndarray:
    return linear(silu(linear(x, w1)) * linear(x, w3), w2)


# ---------------------------------------------------------------------------
# The block -- LLaMABlock (page 二), "数据流动" (decoder explainer):
#   h = x + attention(attention_norm(x));  y = h + feed_forward(ffn_norm(h)).
# ---------------------------------------------------------------------------
def block_forward(x: np.ndarray, w: Dict[str, object], shape, k_cache: Optional[Sequence] = None,
                  v_cache: Optional[Sequence] = None, query_rows: Optional[Sequence] = None
                  ) -> Dict[str, object]:
    """Forward of one block over new tokens of B sequences.

    x: [B, L, D] new tokens; sequence b's tokens sit at positions S_b .. S_b+L-1
    where S_b = len(k_cache[b]) (0 without a cache).  k_cache[b], v_cache[b]:
    [S_b, G, d] post-RoPE keys and values already cached.
    query_rows: optional list (per sequence) of row indices whose outputs are
    wanted; keys/values are still produced for every new token.

    Returns dict with, per sequence b, arrays indexed like the requested rows:
      y [n, D], h [n, D] (after the attention residual), attn [n, H*d]
      (attention output before wo), ffn [n, D] (feed-forward branch),
      k_new / v_new [L, G, d] (what the cache gains), q [n, H, d] (post-RoPE).
    """
    x = np.asarray(x, dtype=F64)
    B, L, D = x.shape
    H, G, d = shape.n_heads, shape.n_kv_heads, shape.head_dim
    # each weight converted to float64 (or dequantized) once for all sequences
    w = {k: (v if k.endswith("norm") else weight_matrix(v)) for k, v in w.items()}
    res = {k: [] for k in ("y", "h", "attn", "ffn", "k_new", "v_new", "q", "rows")}
    for b in range(B):
        S = 0 if k_cache is None else int(np.asarray(k_cache[b]).shape[0])
        rows = np.arange(L) if query_rows is None else np.asarray(query_rows[b], dtype=np.int64)
        xn = rmsnorm(x[b], w["attention_norm"], shape.eps)                         # [L, D]
        pos = S + np.arange(L)
        k_new = apply_rope(linear(xn, w["wk"]).reshape(L, G, d), pos, shape.rope_theta, shape.traditional)
        v_new = linear(xn, w["wv"]).reshape(L, G, d)
        q = apply_rope(linear(xn[rows], w["wq"]).reshape(len(rows), H, d), pos[rows],
                       shape.rope_theta, shape.traditional)
        if S:
            k_all = np.concatenate([np.asarray(k_cache[b], dtype=F64), k_new], axis=0)
            v_all = np.concatenate([np.asarray(v_cache[b], dtype=F64), v_new], axis=0)
        else:
            k_all, v_all = k_new, v_new
        o = causal_attention(q, k_all, v_all, pos[rows], getattr(shape, "window", 0)).reshape(len(rows), H * d)
        h = x[b, rows] + linear(o, w["wo"])
        f = swiglu_ffn(rmsnorm(h, w["ffn_norm"], shape.eps), w["w1"], w["w2"], w["w3"])
        res["y"].append(h + f)
        res["h"].append(h)
        res["attn"].append(o)
        res["ffn"].append(f)
        res["k_new"].append(k_new)
        res["v_new"].append(v_new)
        res["q"].append(q)
        res["rows"].append(rows)
    return res


def stack_arrays(res: Dict[str, List[np.ndarray]], key: str) -> np.ndarray:
    return np.stack(res[key], axis=0)


# ---------------------------------------------------------------------------
# Stack ends -- embedding lookup ("1. 嵌入层"), final RMSNorm and output head
# (module tree of the MLX page; LLaMA.forward on page 二), logits of the last
# position only (prefill hands only its last token to the LM head, "第三章" of
# the reading notes), greedy choice = argmax ("生成过程": temp 0 is argmax).
# ---------------------------------------------------------------------------
def embed(table: np.ndarray, ids: np.ndarray) -> np.ndarray:
    return np.asarray(table, dtype=F64)[np.asarray(ids)]


def lm_head_logits(x_last: np.ndarray, norm_w: np.ndarray, eps: float, head) -> np.ndarray:
    return linear(rmsnorm(x_last, norm_w, eps), head)


def stack_forward(ids: np.ndarray, layers, head: Dict[str, object], shape, rows: Sequence[int],
                  record=None) -> np.ndarray:
    """The model's forward pass over a whole token sequence, with no cache
    (LLaMA.forward on page 二: embedding, every block causally over all
    positions, final RMSNorm, output head), returning the logits of the
    positions in `rows` [len(rows), vocab].

    ids: [L] token ids.  layers: the blocks' weights in order (an iterable,
    consumed once: each layer's 4-bit weights are dequantized by its own block
    call).  record(i, x_in, res), if given, sees every block: its input
    [L, D] and the block_forward result (k_new / v_new: what it caches).
    By causality the logits of position t equal those of a forward over the
    first t + 1 tokens alone: the no-cache generation of LLaMA.generate, which
    re-runs the model on the sequence so far for every new token.
    """
    x = embed(head["embedding"], np.asarray(ids).reshape(1, -1))          # [1, L, D]
    for i, w in enumerate(layers):
        r = block_forward(x, w, shape)
        if record is not None:
            record(i, x[0], r)
        x = stack_arrays(r, "y")
    out = weight_matrix(head["output"])
    return np.stack([lm_head_logits(x[0, t], head["norm"], shape.eps, out) for t in rows])


def argmax_first(v: np.ndarray) -> int:
    """Index of the largest value; the lowest index wins a tie."""
    v = np.asarray(v)
    return int(np.flatnonzero(v == v.max())[0])


# ---------------------------------------------------------------------------
# Sampling -- "生成过程" (MLX page): at temperature 0 the next id is the argmax,
# above 0 a multinomial draw from softmax(logits / temperature).  LLaMA.generate
# (page 二) limits the draw to the nucleus: tokens in order of decreasing
# probability up to and including the first one at which the cumulative
# probability exceeds top_p.
# Readings: the random draw comes in as u in [0, 1); u selects the first token,
# in vocabulary order, at which the cumulative kept probability exceeds
# u * (kept probability) -- the same distribution as a draw in sorted order;
# tokens tied with the last nucleus token are kept too.
# ---------------------------------------------------------------------------
def sample_probs(logits: np.ndarray, temperature: float, top_p: float) -> np.ndarray:
    """Unnormalised kept probabilities (0 outside the nucleus)."""
    z = np.asarray(logits, dtype=F64) / temperature
    e = np.exp(z - z.max())
    p = e / e.sum()
    if top_p >= 1.0:
        return p
    order = np.argsort(-p, kind="stable")
    cum = np.cumsum(p[order])
    over = np.flatnonzero(cum > top_p)
    if over.size == 0:
        return p
    thr = p[order[over[0]]]
    return np.where(p >= thr, p, 0.0)


def sample(logits: np.ndarray, temperature: float, top_p: float, u: float) -> int:
    if temperature <= 0.0:
        return argmax_first(logits)
    q = sample_probs(logits, temperature, top_p)
    c = np.cumsum(q)
    return int(np.flatnonzero(c > u * c[-1])[0])


def greedy_generate(ids: np.ndarray, layers: Sequence[Dict[str, object]], head: Dict[str, object],
                    shape, steps: int) -> Dict[str, object]:
    """Prompt pass fills every layer's cache, then `steps` single-token passes
    ("生成过程" on the MLX page).  Returns the emitted ids (steps + 1 of them:
    one from the prompt pass, one per step) and the logits behind each."""
    ids = np.asarray(ids).reshape(1, -1)
    # weights as float64 once (4-bit ones dequantized once), not once per step
    layers = [{k: (v if k.endswith("norm") else weight_matrix(v)) for k, v in w.items()} for w in layers]
    head = dict(head, output=weight_matrix(head["output"]))
    kc: List[List[np.ndarray]] = [[np.zeros((0, shape.n_kv_heads, shape.head_dim))] for _ in layers]
    vc: List[List[np.ndarray]] = [[np.zeros((0, shape.n_kv_heads, shape.head_dim))] for _ in layers]
    x = embed(head["embedding"], ids)                     # [1, L, D]
    out_ids, out_logits = [], []
    for t in range(steps + 1):
        for i, w in enumerate(layers):
            r = block_forward(x, w, shape, kc[i], vc[i])
            kc[i][0] = np.concatenate([kc[i][0], r["k_new"][0]], axis=0)
            vc[i][0] = np.concatenate([vc[i][0], r["v_new"][0]], axis=0)
            x = stack_arrays(r, "y")
        logits = lm_head_logits(x[0, -1], head["norm"], shape.eps, head["output"])
        nxt = argmax_first(logits)
        out_ids.append(nxt)
        out_logits.append(logits)
        x = embed(head["embedding"], np.array([[nxt]]))
    return {"ids": np.array(out_ids, dtype=np.int32), "logits": out_logits}
