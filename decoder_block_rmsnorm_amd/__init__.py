"""MI355X (gfx950) LLaMA-style pre-norm decoder block: thin Python binding.

Every compute step runs in the HIP kernels of ``libllama_block.so``; this
module only marshals arguments.  torch is used for device memory (tensors
allocated on ``cuda``) and streams (``torch.cuda.Stream.cuda_stream``).

The functions named ``llama_*`` mirror the C entry points of
``include/llama_block.h`` one to one (same names, same argument order; device
buffers may be passed as torch tensors or raw addresses; a stream as a
``torch.cuda.Stream``, a raw handle or ``None`` for torch's current stream).
``Block``, ``KVCache`` and ``Stack`` are small owners of the device memory
those calls need.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, Optional, Sequence

from . import _abi
from ._abi import (LLAMA_BF16, LLAMA_DIAG_ATTN, LLAMA_DIAG_FFN, LLAMA_DIAG_H, LLAMA_ERR_CAPACITY, LLAMA_ERR_HIP,  # noqa: F401
                   LLAMA_ERR_INVALID_ARG, LLAMA_ERR_UNSUPPORTED, LLAMA_F32, LLAMA_OK, LLAMA_W_DENSE, LLAMA_W_Q4,
                   STATUS_NAMES, llama_block_config, llama_block_weights, llama_kvcache_config, llama_linear)

__all__ = [n for n in _abi.SIGNATURES] + ["LlamaError", "Block", "KVCache", "Stack", "block_config", "lib"]


class LlamaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


def lib():
    return _abi.load()


def _check(st: int) -> None:
    if st != LLAMA_OK:
        raise LlamaError(st, (lib().llama_last_error() or b"").decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device buffer expected (a cuda tensor)")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(s, int):
        return s or None
    return s.cuda_stream or None


def _i32_array(vals: Sequence[int]):
    return (C.c_int32 * len(vals))(*[int(v) for v in vals])


# ------------------------------------------------------------- 1:1 entry points
def llama_block_weight_bytes(cfg: llama_block_config) -> int:
    return lib().llama_block_weight_bytes(C.byref(cfg))


def llama_block_create(cfg, weights: llama_block_weights, dev_mem, dev_bytes: int, stream=None) -> int:
    out = C.c_void_p()
    _check(lib().llama_block_create(C.byref(cfg), C.byref(weights), _ptr(dev_mem), dev_bytes, _stream(stream),
                                    C.byref(out)))
    return out.value


def llama_block_destroy(blk: int) -> None:
    lib().llama_block_destroy(blk)


def llama_scratch_bytes(cfg, max_tokens: int, max_batch: int, max_seq: int) -> int:
    return lib().llama_scratch_bytes(C.byref(cfg), max_tokens, max_batch, max_seq)


def llama_block_prefill(blk, cache, layer, x, y, batch, seq_len, scratch, scratch_bytes, stream=None) -> None:
    _check(lib().llama_block_prefill(blk, cache, layer, _ptr(x), _ptr(y), batch, seq_len, _ptr(scratch),
                                     scratch_bytes, _stream(stream)))


def llama_block_prefill_ragged(blk, cache, layer, x, y, batch, seq_lens_host: Sequence[int], scratch, scratch_bytes,
                               stream=None) -> None:
    _check(lib().llama_block_prefill_ragged(blk, cache, layer, _ptr(x), _ptr(y), batch, _i32_array(seq_lens_host),
                                            _ptr(scratch), scratch_bytes, _stream(stream)))


def llama_block_decode(blk, cache, layer, x, y, batch, scratch, scratch_bytes, stream=None) -> None:
    _check(lib().llama_block_decode(blk, cache, layer, _ptr(x), _ptr(y), batch, _ptr(scratch), scratch_bytes,
                                    _stream(stream)))


def llama_block_decode_noalloc(blk, cache, layer, x, y, batch, stream=None) -> None:
    _check(lib().llama_block_decode_noalloc(blk, cache, layer, _ptr(x), _ptr(y), batch, _stream(stream)))


def llama_block_diag(blk, scratch, which: int, tokens: int) -> int:
    out = C.c_void_p()
    _check(lib().llama_block_diag(blk, _ptr(scratch), which, tokens, C.byref(out)))
    return out.value


def llama_block_set_diag(blk, enable: int) -> None:
    _check(lib().llama_block_set_diag(blk, int(enable)))


def llama_block_profile_start(blk, max_calls: int, phase_mask: int = 0) -> None:
    _check(lib().llama_block_profile_start(blk, max_calls, phase_mask))


def llama_block_profile_read(blk, max_phases: int = 16):
    ms = (C.c_float * max_phases)()
    n_ph, n_calls = C.c_int32(), C.c_int32()
    _check(lib().llama_block_profile_read(blk, ms, max_phases, C.byref(n_ph), C.byref(n_calls)))
    return list(ms)[:n_ph.value], n_calls.value


def llama_kvcache_bytes(cfg: llama_kvcache_config) -> int:
    return lib().llama_kvcache_bytes(C.byref(cfg))


def llama_kvcache_alloc(cfg, dev_mem, dev_bytes: int, stream=None) -> int:
    out = C.c_void_p()
    _check(lib().llama_kvcache_alloc(C.byref(cfg), _ptr(dev_mem), dev_bytes, _stream(stream), C.byref(out)))
    return out.value


def llama_kvcache_free(cache: int) -> None:
    lib().llama_kvcache_free(cache)


def llama_kvcache_set_block_table(cache, table_host: Sequence[int], stream=None) -> None:
    _check(lib().llama_kvcache_set_block_table(cache, _i32_array(table_host), _stream(stream)))


def llama_kvcache_set_lens(cache, layer: int, lens_host: Sequence[int], batch: int, stream=None) -> None:
    _check(lib().llama_kvcache_set_lens(cache, layer, _i32_array(lens_host), batch, _stream(stream)))


def llama_kvcache_get_lens(cache, layer: int, batch: int):
    arr = (C.c_int32 * batch)()
    _check(lib().llama_kvcache_get_lens(cache, layer, arr, batch))
    return list(arr)


def llama_kvcache_write(cache, layer, seq, pos0, n, k, v, stream=None) -> None:
    _check(lib().llama_kvcache_write(cache, layer, seq, pos0, n, _ptr(k), _ptr(v), _stream(stream)))


def llama_kvcache_read(cache, layer, seq, pos0, n, k, v, stream=None) -> None:
    _check(lib().llama_kvcache_read(cache, layer, seq, pos0, n, _ptr(k), _ptr(v), _stream(stream)))


def llama_embed(table, vocab, dim, dtype, ids, n, out, stream=None) -> None:
    _check(lib().llama_embed(_ptr(table), vocab, dim, dtype, _ptr(ids), n, _ptr(out), _stream(stream)))


def llama_head_scratch_bytes(batch: int, dim: int, vocab: int) -> int:
    return lib().llama_head_scratch_bytes(batch, dim, vocab)


def llama_lm_head_argmax(head: llama_linear, weight_format, group_size, act_dtype, final_norm, eps, x, batch, dim,
                         vocab, logits, ids, scratch, scratch_bytes, stream=None) -> None:
    _check(lib().llama_lm_head_argmax(C.byref(head), weight_format, group_size, act_dtype, _ptr(final_norm), eps,
                                      _ptr(x), batch, dim, vocab, _ptr(logits), _ptr(ids), _ptr(scratch),
                                      scratch_bytes, _stream(stream)))


def llama_stack_create(blocks: Sequence[int], embedding, vocab, final_norm, output: llama_linear) -> int:
    arr = (C.c_void_p * len(blocks))(*blocks)
    out = C.c_void_p()
    _check(lib().llama_stack_create(arr, len(blocks), _ptr(embedding), vocab, _ptr(final_norm), C.byref(output),
                                    C.byref(out)))
    return out.value


def llama_stack_destroy(st: int) -> None:
    lib().llama_stack_destroy(st)


def llama_sample(logits, batch, vocab, temperature, top_p, u, ids, stream=None) -> None:
    _check(lib().llama_sample(_ptr(logits), batch, vocab, temperature, top_p, _ptr(u), _ptr(ids), _stream(stream)))


def llama_stack_set_sampling(st, temperature, top_p, u) -> None:
    _check(lib().llama_stack_set_sampling(st, temperature, top_p, _ptr(u)))


def llama_stack_scratch_bytes(st, max_prompt: int, max_seq: int) -> int:
    return lib().llama_stack_scratch_bytes(st, max_prompt, max_seq)


def llama_stack_generate(st, cache, prompt, prompt_len, n_steps, ids_out, logits_out, scratch, scratch_bytes,
                         use_graph: int, stream=None) -> None:
    _check(lib().llama_stack_generate(st, cache, _ptr(prompt), prompt_len, n_steps, _ptr(ids_out), _ptr(logits_out),
                                      _ptr(scratch), scratch_bytes, use_graph, _stream(stream)))


def llama_stack_generate_recompute(st, cache, prompt, prompt_len, n_steps, ids_out, logits_out, scratch,
                                   scratch_bytes, stream=None) -> None:
    _check(lib().llama_stack_generate_recompute(st, cache, _ptr(prompt), prompt_len, n_steps, _ptr(ids_out),
                                                _ptr(logits_out), _ptr(scratch), scratch_bytes, _stream(stream)))


def llama_probe_mfma_bf16(blocks: int, iters: int, sink, stream=None) -> None:
    _check(lib().llama_probe_mfma_bf16(blocks, iters, _ptr(sink), _stream(stream)))


def llama_last_error() -> str:
    return (lib().llama_last_error() or b"").decode()


# ------------------------------------------------------------- owners
def block_config(dim, n_heads, n_kv_heads, ffn_dim, norm_eps=1e-5, rope_theta=10000.0, rope_traditional=False,
                 act_dtype=LLAMA_BF16, weight_format=LLAMA_W_DENSE, group_size=64, max_seq=4096,
                 sliding_window=0) -> llama_block_config:
    return llama_block_config(dim, n_heads, n_kv_heads, ffn_dim, norm_eps, rope_theta, int(bool(rope_traditional)),
                              act_dtype, weight_format, group_size, max_seq, sliding_window)


def _device_bytes(n: int, device="cuda"):
    import torch
    return torch.empty(max(int(n), 256), dtype=torch.uint8, device=device)


def _linear(w) -> llama_linear:
    if isinstance(w, dict):
        return llama_linear(_ptr(w["w"]), _ptr(w["scales"]), _ptr(w["biases"]))
    return llama_linear(_ptr(w), None, None)


class Block:
    """One decoder block: owns its repacked-weight device memory.

    weights: dict with attention_norm, ffn_norm (tensors [dim]) and wq, wk, wv,
    wo, w1, w2, w3 -- dense tensors [out, in] of the activation dtype, or for
    4-bit weights dicts {w: int32 [out, in/8], scales: bf16, biases: bf16}.
    """

    def __init__(self, cfg: llama_block_config, weights: Dict[str, object], stream=None):
        self.cfg = cfg
        w = llama_block_weights(_ptr(weights["attention_norm"]), _ptr(weights["ffn_norm"]),
                                *[_linear(weights[k]) for k in ("wq", "wk", "wv", "wo", "w1", "w2", "w3")])
        nbytes = llama_block_weight_bytes(cfg)
        if nbytes == 0:
            # reproduce the validation error message
            llama_block_create(cfg, w, 0, 0, stream)
        self.mem = _device_bytes(nbytes)
        self.handle = llama_block_create(cfg, w, self.mem, nbytes, stream)

    def scratch_bytes(self, max_tokens: int, max_batch: int, max_seq: int) -> int:
        return llama_scratch_bytes(self.cfg, max_tokens, max_batch, max_seq)

    def prefill(self, cache: "KVCache", layer: int, x, y, batch: int, seq_len: int, scratch, stream=None) -> None:
        llama_block_prefill(self.handle, cache.handle, layer, x, y, batch, seq_len, scratch, scratch.numel(), stream)

    def prefill_ragged(self, cache: "KVCache", layer: int, x, y, seq_lens: Sequence[int], scratch,
                       stream=None) -> None:
        """x, y: [sum(seq_lens), dim], sequence b's new tokens packed after those of 0 .. b-1."""
        llama_block_prefill_ragged(self.handle, cache.handle, layer, x, y, len(seq_lens), seq_lens, scratch,
                                   scratch.numel(), stream)

    def decode(self, cache: "KVCache", layer: int, x, y, batch: int, scratch, stream=None) -> None:
        llama_block_decode(self.handle, cache.handle, layer, x, y, batch, scratch, scratch.numel(), stream)

    def diag(self, scratch, which: int, tokens: int) -> int:
        return llama_block_diag(self.handle, scratch, which, tokens)

    def set_diag(self, enable: bool) -> None:
        llama_block_set_diag(self.handle, int(enable))

    def profile_start(self, max_calls: int, phases=None) -> None:
        """Time the next max_calls calls; phases: indices of the phases to time
        (None: all)."""
        mask = 0 if phases is None else sum(1 << p for p in phases)
        llama_block_profile_start(self.handle, max_calls, mask)

    def profile_read(self):
        """-> (per-phase summed milliseconds, number of calls)"""
        return llama_block_profile_read(self.handle)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _abi is not None and _abi._lib is not None:
            _abi._lib.llama_block_destroy(h)
        self.handle = None


class KVCache:
    """Paged KV cache in one device buffer (see llama_kvcache_alloc)."""

    def __init__(self, n_layers, max_batch, max_seq, n_kv_heads, head_dim, dtype=LLAMA_BF16, page_size=64,
                 stream=None):
        self.cfg = llama_kvcache_config(n_layers, max_batch, max_seq, n_kv_heads, head_dim, page_size, dtype)
        nbytes = llama_kvcache_bytes(self.cfg)
        if nbytes == 0:
            llama_kvcache_alloc(self.cfg, 0, 0, stream)
        self.mem = _device_bytes(nbytes)
        self.handle = llama_kvcache_alloc(self.cfg, self.mem, nbytes, stream)
        self.pages_per_seq = -(-max_seq // page_size)

    def write(self, layer, seq, pos0, k, v, stream=None):
        llama_kvcache_write(self.handle, layer, seq, pos0, k.shape[0], k, v, stream)

    def read(self, layer, seq, pos0, n, k, v, stream=None):
        llama_kvcache_read(self.handle, layer, seq, pos0, n, k, v, stream)

    def set_lens(self, layer, lens, stream=None):
        llama_kvcache_set_lens(self.handle, layer, lens, len(lens), stream)

    def get_lens(self, layer, batch):
        return llama_kvcache_get_lens(self.handle, layer, batch)

    def set_block_table(self, table, stream=None):
        llama_kvcache_set_block_table(self.handle, table, stream)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _abi is not None and _abi._lib is not None:
            _abi._lib.llama_kvcache_free(h)
        self.handle = None


class Stack:
    """n_layers blocks + embedding + final norm + output head; greedy or sampled generation."""

    def __init__(self, blocks: Sequence[Block], embedding, vocab: int, final_norm, output):
        self.blocks = list(blocks)
        self._refs = (embedding, final_norm, output)
        self.handle = llama_stack_create([b.handle for b in self.blocks], embedding, vocab, final_norm,
                                         _linear(output))
        self.vocab = vocab

    def scratch_bytes(self, max_prompt: int, max_seq: int) -> int:
        return llama_stack_scratch_bytes(self.handle, max_prompt, max_seq)

    def set_sampling(self, temperature: float, top_p: float = 1.0, u=None) -> None:
        """Greedy at temperature <= 0; else u (fp32 [n_steps + 1] on the device,
        kept alive here) gives the draw of each emitted id."""
        llama_stack_set_sampling(self.handle, temperature, top_p, u)
        # (replaced only once the library took it: it keeps reading the old draws until then)
        self._u = u if temperature > 0 else None

    def _check_sizes(self, n_steps: int, ids_out, logits_out) -> None:
        # the device buffers the kernels write or read per emitted id; their sizes
        # cannot be seen through the C ABI
        # (raw addresses pass unchecked)
        n = n_steps + 1
        size = lambda t: t.numel() if hasattr(t, "numel") else None  # noqa: E731
        if n_steps < 0:
            return
        if size(ids_out) is not None and size(ids_out) < n:
            raise ValueError(f"ids_out holds {size(ids_out)} ids, {n} are emitted")
        if size(logits_out) is not None and size(logits_out) < n * self.vocab:
            raise ValueError(f"logits_out holds {size(logits_out)} values, {n} rows of {self.vocab} are written")
        u = getattr(self, "_u", None)
        if size(u) is not None and size(u) < n:
            raise ValueError(f"the sampling draws hold {size(u)} values, {n} ids are drawn")

    def generate(self, cache: KVCache, prompt, n_steps: int, ids_out, logits_out, scratch, use_graph=True,
                 stream=None) -> None:
        self._check_sizes(n_steps, ids_out, logits_out)
        llama_stack_generate(self.handle, cache.handle, prompt, prompt.numel(), n_steps, ids_out, logits_out,
                             scratch, scratch.numel(), int(bool(use_graph)), stream)

    def generate_recompute(self, cache: KVCache, prompt, n_steps: int, ids_out, logits_out, scratch,
                           stream=None) -> None:
        """No cache reuse: every id re-runs the prompt pass over the sequence so
        far (scratch sized by scratch_bytes(prompt + n_steps, max_seq))."""
        self._check_sizes(n_steps, ids_out, logits_out)
        llama_stack_generate_recompute(self.handle, cache.handle, prompt, prompt.numel(), n_steps, ids_out,
                                       logits_out, scratch, scratch.numel(), stream)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _abi is not None and _abi._lib is not None:
            _abi._lib.llama_stack_destroy(h)
        self.handle = None
