"""The decode entry point that allocates nothing (llama_block_decode_noalloc):
its transient values live in the library's fixed per-device array instead of
a caller's scratch.  Checked through the C ABI against llama_block_decode on
twin caches, on two calls in a row (the second with fewer sequences), on a
dense bf16 block and the single-sequence 4-bit path; a request beyond the
array's size is refused with LLAMA_ERR_CAPACITY and leaves the cache as it was.
"""
import numpy as np
import pytest
import torch

import decoder_block_rmsnorm_amd as L
import workloads as W
from oracle import ref
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _flush(*a):
    print(*a, flush=True)


def _twin_caches(s, B, max_seq, lens, rng):
    caches = [G.make_cache(s, 1, B, max_seq) for _ in range(2)]
    kv = []
    for b in range(B):
        k = rng.normal((lens[b], s.n_kv_heads, s.head_dim), 1.0, "bf16")
        v = rng.normal((lens[b], s.n_kv_heads, s.head_dim), 1.0, "bf16")
        kv.append((k, v))
        for c in caches:
            if lens[b]:
                c.write(0, b, 0, G.tdev(k, "bf16"), G.tdev(v, "bf16"))
    for c in caches:
        c.set_lens(0, lens)
    return caches, kv


@pytest.mark.parametrize("fmt", ["bf16", "q4"])
def test_decode_noalloc_matches_decode_two_calls(fmt):
    if fmt == "bf16":
        s = W.BlockShape(dim=1024, n_heads=8, n_kv_heads=2, ffn_dim=2816, dtype="bf16")
        calls = [16, 3]
    else:
        s = W.BlockShape(dim=512, n_heads=4, n_kv_heads=4, ffn_dim=1536, dtype="bf16", weight_format="q4",
                         traditional=True)
        calls = [2, 1]
    rng = W.Rng(61)
    w = W.draw_block_weights(s, rng)
    B = calls[0]
    max_seq = 700
    lens = [int(v) for v in rng.g.integers(0, 600, size=B)]
    _flush(f"case: no-allocation decode {fmt}, calls of {calls} sequences, lens {lens}")
    blk, wd = G.make_block(s, w, max_seq)
    (c_ref, c_na), kv = _twin_caches(s, B, max_seq, lens, rng)
    sc = G.scratch(blk, B, B, max_seq)
    for i, n in enumerate(calls):
        x = G.tdev(rng.normal((n, s.dim), 1.0, "bf16"), "bf16")
        y_ref = torch.empty_like(x)
        y_na = torch.full_like(x, float("nan"))
        L.llama_block_decode(blk.handle, c_ref.handle, 0, x, y_ref, n, sc, sc.numel())
        L.llama_block_decode_noalloc(blk.handle, c_na.handle, 0, x, y_na, n)
        torch.cuda.synchronize()
        a, b = G.thost(y_ref), G.thost(y_na)
        assert np.isfinite(b).all()
        assert np.array_equal(a, b), f"call {i}: outputs differ"
        # and the oracle agrees with both (the first call's sequences)
        if i == 0:
            r = ref.block_forward(G.thost(x)[:, None], w, s, [kv[j][0] for j in range(n)],
                                  [kv[j][1] for j in range(n)])
            G.check("bf16", b, np.concatenate(r["y"]), f"call {i} vs the oracle")
        assert c_na.get_lens(0, B) == c_ref.get_lens(0, B)
    # the appended keys and values are identical too
    for j in range(calls[-1]):
        n = c_ref.get_lens(0, B)[j]
        kr = torch.empty((n, s.n_kv_heads, s.head_dim), device="cuda", dtype=torch.bfloat16)
        vr, kn, vn = torch.empty_like(kr), torch.empty_like(kr), torch.empty_like(kr)
        c_ref.read(0, j, 0, n, kr, vr)
        c_na.read(0, j, 0, n, kn, vn)
        torch.cuda.synchronize()
        assert torch.equal(kr, kn) and torch.equal(vr, vn)


def test_decode_noalloc_refuses_more_than_its_array():
    s = W.BlockShape(dim=8192, n_heads=64, n_kv_heads=1, ffn_dim=512, dtype="bf16")
    rng = W.Rng(62)
    w = W.draw_block_weights(s, rng)
    _flush("case: no-allocation decode beyond its fixed scratch")
    blk, wd = G.make_block(s, w, 16384)
    cache = G.make_cache(s, 1, 64, 16384)
    x = G.tdev(rng.normal((64, s.dim), 1.0, "bf16"), "bf16")
    need = blk.scratch_bytes(0, 64, 16384)
    assert need > 64 << 20
    with pytest.raises(L.LlamaError) as e:
        L.llama_block_decode_noalloc(blk.handle, cache.handle, 0, x, x, 64)
    assert e.value.status == L.LLAMA_ERR_CAPACITY and "fixed" in e.value.message
    assert cache.get_lens(0, 64) == [0] * 64
    # a smaller batch against the same cache fits and runs
    L.llama_block_decode_noalloc(blk.handle, cache.handle, 0, x[:2], x[:2], 2)
    torch.cuda.synchronize()
    assert cache.get_lens(0, 3) == [1, 1, 0]
