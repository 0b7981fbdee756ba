"""Seeded synthetic workloads for the LLaMA-style pre-norm decoder block.

This package only *draws* inputs: shapes, random tensors and their rounding to
the storage dtype.  It contains none of the block's arithmetic, so both the CPU
oracle (``oracle/``) and the GPU path (``decoder_block_rmsnorm_amd``) can take
their inputs from it without sharing any computation.

Every tensor comes from one numpy PCG64 stream (seed 0 unless stated) in a fixed
draw order: block inputs, then the pre-filled K and V caches (decode workloads),
then per layer [attention_norm, wq, wk, wv, wo, ffn_norm, w1, w2, w3], then the
token embedding, the final norm and the output head.  Linear weights follow the
``nn.Linear`` ``[out, in]`` convention and are drawn N(0, 0.02) as in the
LLaMA._init_weights of the page "LLaMA架构深度解析" (section 二); RMSNorm weights
are 1 + U(-0.1, 0.1) so that a missing gamma multiply cannot hide.  bf16 tensors
are rounded to nearest-even once, here, and the *same* rounded values are
handed to both sides (as float32 arrays holding bf16-representable numbers).

4-bit weights (group-wise affine, group 64 along the input dim, 4 bits, as the
MLX conversion config of the page "iOS设备上运行LLaMA2-13B" states) are drawn as
uniform random bytes: every byte carries two U{0..15} codes, low nibble first.
Viewed as little-endian uint32 words this is exactly the library's packed
format (code k of a row at bits 4*(k%8) of word k//8).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Dict, Iterator, List, Optional

import numpy as np

__all__ = [
    "BlockShape", "Workload", "WORKLOADS", "get", "round_bf16", "Rng",
    "draw_block_weights", "draw_q4_linear", "unpack_q4_codes",
    "draw_inputs", "draw_decode_caches", "draw_stack",
]


# --------------------------------------------------------------------------
# shapes
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class BlockShape:
    dim: int
    n_heads: int
    n_kv_heads: int
    ffn_dim: int
    eps: float = 1e-5
    rope_theta: float = 10000.0
    traditional: bool = False          # True: interleaved pairs (MLX RoPE traditional=True)
    dtype: str = "bf16"                # "f32" | "bf16"
    weight_format: str = "dense"       # "dense" | "q4"
    group_size: int = 64
    window: int = 0                    # sliding-window attention: W most recent positions (0 = full causal)

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    @property
    def n_rep(self) -> int:
        return self.n_heads // self.n_kv_heads

    @property
    def linear_params(self) -> int:
        d, hd = self.dim, self.head_dim
        qkv = d * (self.n_heads + 2 * self.n_kv_heads) * hd
        return qkv + self.n_heads * hd * d + 3 * d * self.ffn_dim


@dataclass(frozen=True)
class Workload:
    name: str
    shape: BlockShape
    mode: str                  # "prefill" | "decode" | "prefill+decode" | "stack"
    batch: int
    seq_len: int               # new tokens per sequence in the prefill call
    cache_len: int = 0         # pre-filled cache length (decode workloads)
    decode_steps: int = 0
    n_layers: int = 1
    vocab: int = 0
    seed: int = 0
    note: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_L7 = BlockShape(dim=4096, n_heads=32, n_kv_heads=32, ffn_dim=11008, eps=1e-5,
                 traditional=False, dtype="bf16")
_L13 = BlockShape(dim=5120, n_heads=40, n_kv_heads=40, ffn_dim=13824, eps=1e-5,
                  traditional=True, dtype="bf16")
_L70 = BlockShape(dim=8192, n_heads=64, n_kv_heads=8, ffn_dim=28672, eps=1e-5,
                  traditional=False, dtype="bf16")
_TINY = BlockShape(dim=256, n_heads=4, n_kv_heads=4, ffn_dim=688, eps=1e-5,
                   traditional=True, dtype="f32")
_Q13 = dataclasses.replace(_L13, weight_format="q4", group_size=64)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    # tiny fp32 block: causal prefill of 32 tokens, then 8 decode steps through the cache
    Workload("tiny_f32_d256_prefill32_decode8", _TINY, "prefill+decode", batch=1,
             seq_len=32, decode_steps=8),
    # LLaMA-2-7B-shaped block, causal prefill of one 2048-token prompt
    Workload("llama7b_block_prefill_b1_l2048", _L7, "prefill", batch=1, seq_len=2048),
    # LLaMA-2-13B-shaped block, decode of 16 sequences against 4096-token caches
    Workload("llama13b_block_decode_b16_kv4096", _L13, "decode", batch=16, seq_len=1,
             cache_len=4096),
    # 70B-shaped GQA(8) block, causal prefill of 4 x 1024 tokens
    Workload("gqa70b_block_prefill_b4_l1024", _L70, "prefill", batch=4, seq_len=1024),
    # 70B-shaped GQA(8) block, decode of 64 sequences against 4096-token caches
    Workload("gqa70b_block_decode_b64_kv4096", _L70, "decode", batch=64, seq_len=1,
             cache_len=4096),
    # 40-layer 13B-shaped stack, 4-bit weights: 512-token prompt then 128 greedy steps
    Workload("q4_llama13b_stack40_prompt512_greedy128", _Q13, "stack", batch=1,
             seq_len=512, decode_steps=128, n_layers=40, vocab=32000),
]}

# Small shapes used by tests (brute force, several-tile parity with ragged tails).
TEST_SHAPES: Dict[str, BlockShape] = {
    # the tiny GQA config of the test_llama smoke function on the page "LLaMA架构深度解析"
    "tiny_gqa_d128": BlockShape(dim=128, n_heads=4, n_kv_heads=2, ffn_dim=256, eps=1e-6,
                                traditional=False, dtype="f32"),
    "tiny_f32": _TINY,
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# drawing
# --------------------------------------------------------------------------
def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


class Rng:
    """The single seeded stream all draws of one workload come from."""

    def __init__(self, seed: int):
        self.g = np.random.Generator(np.random.PCG64(seed))

    def normal(self, shape, std: float, dtype: str) -> np.ndarray:
        a = self.g.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        return round_bf16(a) if dtype == "bf16" else a

    def uniform(self, shape, lo: float, hi: float) -> np.ndarray:
        return self.g.uniform(lo, hi, size=shape).astype(np.float32)

    def norm_weight(self, n: int, dtype: str) -> np.ndarray:
        a = (1.0 + self.g.uniform(-0.1, 0.1, size=n)).astype(np.float32)
        return round_bf16(a) if dtype == "bf16" else a

    def nibble_bytes(self, rows: int, cols: int) -> np.ndarray:
        """[rows, cols/2] uint8; each byte = two uniform 4-bit codes (low nibble first)."""
        return np.frombuffer(self.g.bytes(rows * cols // 2), dtype=np.uint8).reshape(rows, cols // 2).copy()

    def ids(self, shape, vocab: int) -> np.ndarray:
        return self.g.integers(0, vocab, size=shape, dtype=np.int64).astype(np.int32)


def draw_inputs(w: Workload, rng: Rng) -> np.ndarray:
    """Block input x [batch, seq_len (+decode_steps), dim] ~ N(0, 1)."""
    s = w.shape
    rows = w.seq_len + (w.decode_steps if w.mode == "prefill+decode" else 0)
    return rng.normal((w.batch, rows, s.dim), 1.0, s.dtype)


def draw_decode_caches(w: Workload, rng: Rng):
    """Pre-filled caches K, V [batch, cache_len, n_kv_heads, head_dim] ~ N(0, 1).

    They stand for post-RoPE keys and values of the tokens already seen.
    """
    s = w.shape
    shp = (w.batch, w.cache_len, s.n_kv_heads, s.head_dim)
    k = rng.normal(shp, 1.0, s.dtype)
    v = rng.normal(shp, 1.0, s.dtype)
    return k, v


def draw_q4_linear(rng: Rng, out_f: int, in_f: int, group: int = 64) -> Dict[str, np.ndarray]:
    """4-bit group-affine linear: packed codes, bf16 scales and biases [out, in/group].

    scale = bf16(U(0.5, 1.5) * 0.02 / sqrt(21.25)) gives weights of std ~0.02
    (21.25 is the variance of U{0..15}); bias = bf16(-scale * U(6.5, 8.5)) centres
    them with per-group variety.
    """
    packed = rng.nibble_bytes(out_f, in_f)
    ng = in_f // group
    s = round_bf16(rng.uniform((out_f, ng), 0.5, 1.5) * np.float32(0.02 / math.sqrt(21.25)))
    b = round_bf16(-s * rng.uniform((out_f, ng), 6.5, 8.5))
    return {"packed": packed, "scales": s, "biases": b, "in": in_f, "out": out_f, "group": group}


def unpack_q4_codes(packed: np.ndarray) -> np.ndarray:
    """[rows, cols/2] uint8 -> [rows, cols] uint8 codes (low nibble = even column)."""
    rows, half = packed.shape
    out = np.empty((rows, half * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


LAYER_KEYS = ["attention_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w1", "w2", "w3"]


def draw_block_weights(s: BlockShape, rng: Rng) -> Dict[str, object]:
    """One block's weights in the fixed draw order."""
    d, hd = s.dim, s.head_dim
    shapes = {"wq": (s.n_heads * hd, d), "wk": (s.n_kv_heads * hd, d), "wv": (s.n_kv_heads * hd, d),
              "wo": (d, s.n_heads * hd), "w1": (s.ffn_dim, d), "w2": (d, s.ffn_dim), "w3": (s.ffn_dim, d)}
    out: Dict[str, object] = {}
    for k in LAYER_KEYS:
        if k.endswith("norm"):
            out[k] = rng.norm_weight(d, s.dtype)
        elif s.weight_format == "q4":
            out[k] = draw_q4_linear(rng, *shapes[k], group=s.group_size)
        else:
            out[k] = rng.normal(shapes[k], 0.02, s.dtype)
    return out


def draw_stack(w: Workload, rng: Rng) -> Iterator:
    """Yields ("ids", ids), then ("layer", i, weights) per layer, then ("head", dict).

    Lazy, so a 40-layer 4-bit stack never has to sit in host memory at once.
    """
    s = w.shape
    yield ("ids", rng.ids((w.batch, w.seq_len), w.vocab))
    for i in range(w.n_layers):
        yield ("layer", i, draw_block_weights(s, rng))
    emb = rng.normal((w.vocab, s.dim), 0.02, "bf16")
    fnorm = rng.norm_weight(s.dim, "bf16")
    head = draw_q4_linear(rng, w.vocab, s.dim, s.group_size) if s.weight_format == "q4" \
        else rng.normal((w.vocab, s.dim), 0.02, s.dtype)
    yield ("head", {"embedding": emb, "norm": fnorm, "output": head})


def draw_block_workload(w: Workload, seed: Optional[int] = None) -> Dict[str, object]:
    """All inputs of a single-block workload in draw order."""
    rng = Rng(w.seed if seed is None else seed)
    out: Dict[str, object] = {"x": draw_inputs(w, rng)}
    if w.cache_len:
        out["k_cache"], out["v_cache"] = draw_decode_caches(w, rng)
    out["weights"] = draw_block_weights(w.shape, rng)
    return out


# --------------------------------------------------------------------------
# algorithmic work (measurement bookkeeping)
# --------------------------------------------------------------------------
def prefill_flops(s: BlockShape, batch: int, seq_len: int, cached: int = 0) -> float:
    """2 * tokens * linear params + causal attention: 4 * H * d per (query, key <= query) pair."""
    T = batch * seq_len
    pairs = batch * (seq_len * cached + seq_len * (seq_len + 1) // 2)
    return 2.0 * T * s.linear_params + 4.0 * s.n_heads * s.head_dim * pairs


def linear_flops(s: BlockShape, tokens: int) -> dict:
    d, hd = s.dim, s.head_dim
    return {"qkv": 2.0 * tokens * d * (s.n_heads + 2 * s.n_kv_heads) * hd,
            "wo": 2.0 * tokens * s.n_heads * hd * d,
            "w13": 2.0 * tokens * d * 2 * s.ffn_dim,
            "w2": 2.0 * tokens * s.ffn_dim * d}


def weight_bytes(s: BlockShape) -> float:
    if s.weight_format == "q4":
        return s.linear_params * (0.5 + 2 * 2 / s.group_size)
    return s.linear_params * (4 if s.dtype == "f32" else 2)


def decode_bytes(s: BlockShape, batch: int, cached: int) -> dict:
    """One decode step: every weight byte once, every cached K/V byte once (keys 0..cached, or the
    last `window` of them),
    the new K/V rows written, block input read and output written."""
    e = 4 if s.dtype == "f32" else 2
    keys = min(cached + 1, s.window) if s.window > 0 else cached + 1   # a sliding window reads its W keys
    kv_read = batch * keys * s.n_kv_heads * s.head_dim * 2 * e
    kv_write = batch * s.n_kv_heads * s.head_dim * 2 * e
    act = batch * s.dim * 2 * e
    w = weight_bytes(s)
    return {"weights": w, "kv_read": kv_read, "kv_write": kv_write, "act": act,
            "total": w + kv_read + kv_write + act}
