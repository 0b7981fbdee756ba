"""Helpers shared by the GPU parity tests: move seeded workload arrays to the
device, drive the library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import decoder_block_rmsnorm_amd as L
import workloads as W

DEV = "cuda"


def tdev(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(DEV).contiguous()


def thost(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def act_code(dtype: str) -> int:
    return L.LLAMA_BF16 if dtype == "bf16" else L.LLAMA_F32


def make_config(s: W.BlockShape, max_seq: int):
    return L.block_config(s.dim, s.n_heads, s.n_kv_heads, s.ffn_dim, norm_eps=s.eps, rope_theta=s.rope_theta,
                          rope_traditional=s.traditional, act_dtype=act_code(s.dtype),
                          weight_format=L.LLAMA_W_Q4 if s.weight_format == "q4" else L.LLAMA_W_DENSE,
                          group_size=s.group_size, max_seq=max_seq, sliding_window=s.window)


def q4_dev(lin) -> dict:
    """A drawn 4-bit linear as the library's format: packed bytes viewed as uint32 words."""
    words = torch.from_numpy(np.ascontiguousarray(lin["packed"]).view(np.int32)).to(DEV)
    return {"w": words, "scales": tdev(lin["scales"], "bf16"), "biases": tdev(lin["biases"], "bf16")}


def weights_dev(s: W.BlockShape, w: dict) -> dict:
    out = {}
    for k, v in w.items():
        if isinstance(v, dict):
            out[k] = q4_dev(v)
        elif k.endswith("norm"):
            out[k] = tdev(v, "bf16" if s.weight_format == "q4" else s.dtype)
        else:
            out[k] = tdev(v, s.dtype)
    return out


def make_block(s: W.BlockShape, w: dict, max_seq: int):
    wd = weights_dev(s, w)
    blk = L.Block(make_config(s, max_seq), wd)
    return blk, wd


def make_cache(s: W.BlockShape, n_layers: int, max_batch: int, max_seq: int, page_size: int = 64):
    return L.KVCache(n_layers, max_batch, max_seq, s.n_kv_heads, s.head_dim,
                     dtype=act_code("bf16" if s.weight_format == "q4" else s.dtype), page_size=page_size)


def scratch(blk: L.Block, max_tokens: int, max_batch: int, max_seq: int) -> torch.Tensor:
    n = blk.scratch_bytes(max_tokens, max_batch, max_seq)
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def diag(blk: L.Block, sc: torch.Tensor, which: int, tokens: int, width: int, dtype: str) -> np.ndarray:
    """Copy a diagnostic tensor [tokens, width] out of scratch."""
    ptr = blk.diag(sc, which, tokens)
    base = sc.data_ptr()
    esz = 2 if dtype == "bf16" else 4
    off = ptr - base
    raw = sc[off:off + tokens * width * esz]
    t = raw.view(torch.bfloat16 if dtype == "bf16" else torch.float32).reshape(tokens, width)
    return thost(t)


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rel_inf(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def check(dtype: str, got, ref, what: str, tol_bf16: float = 1e-2, tol_f32: float = 1e-4) -> float:
    """fp32: max relative error (inf-norm); bf16 / 4-bit: relative L2."""
    err = rel_inf(got, ref) if dtype == "f32" else rel_l2(got, ref)
    tol = tol_f32 if dtype == "f32" else tol_bf16
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= tol, f"{what}: error {err:.3e} > {tol:.0e}"
    return err
