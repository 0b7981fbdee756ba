"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times, checked against the oracle on sampled output rows (the oracle computes
every key/value the sampled rows need, then only those rows).

Bars: bf16 relative L2 <= 1e-2 on the sampled block outputs, attention outputs
(before wo), residual h and feed-forward branch; the appended cache rows on a
sample of positions.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _flush(*a):
    print(*a, flush=True)


def _rows_sample(L, rng, n=6):
    fixed = [0, 1, 63, 64, 127, 128, L // 2, L - 1]
    extra = list(rng.choice(L, size=n, replace=False))
    return sorted(set([r for r in fixed if r < L] + extra))


@pytest.mark.parametrize("name", ["llama7b_block_prefill_b1_l2048", "gqa70b_block_prefill_b4_l1024"])
def test_full_prefill_sampled_rows(name):
    wl = W.get(name)
    s, B, Lq = wl.shape, wl.batch, wl.seq_len
    _flush(f"case: {name} full-size prefill")
    inp = W.draw_block_workload(wl)
    x, w = inp["x"], inp["weights"]
    blk, wd = G.make_block(s, w, Lq)
    del wd
    cache = G.make_cache(s, 1, B, Lq)
    sc = G.scratch(blk, B * Lq, B, Lq)
    blk.set_diag(True)
    xd = G.tdev(x.reshape(B * Lq, s.dim), s.dtype)
    y = torch.empty_like(xd)
    blk.prefill(cache, 0, xd, y, B, Lq, sc)
    torch.cuda.synchronize()
    T = B * Lq
    got_y = G.thost(y).reshape(B, Lq, s.dim)
    got_a = G.diag(blk, sc, 0, T, s.n_heads * s.head_dim, s.dtype).reshape(B, Lq, -1)
    got_h = G.diag(blk, sc, 1, T, s.dim, s.dtype).reshape(B, Lq, -1)
    got_f = G.diag(blk, sc, 2, T, s.dim, s.dtype).reshape(B, Lq, -1)
    rng = np.random.default_rng(0)
    rows = [_rows_sample(Lq, rng) for _ in range(B)]
    r = ref.block_forward(x, w, s, query_rows=rows)
    for key, got in (("y", got_y), ("attn", got_a), ("h", got_h), ("ffn", got_f)):
        g = np.concatenate([got[b, rows[b]] for b in range(B)])
        e = np.concatenate(r[key])
        err = G.check("bf16", g, e, f"{name} {key} (sampled rows)")
        _flush(f"  {key}: rel L2 {err:.2e}")
    # cache rows (rotated keys and values) of every sequence, sampled positions
    for b in range(B):
        k = torch.empty((Lq, s.n_kv_heads, s.head_dim), device="cuda", dtype=torch.bfloat16)
        v = torch.empty_like(k)
        cache.read(0, b, 0, Lq, k, v)
        pos = rows[b]
        G.check("bf16", G.thost(k)[pos], r["k_new"][b][pos], f"cache K seq {b}")
        G.check("bf16", G.thost(v)[pos], r["v_new"][b][pos], f"cache V seq {b}")
    assert cache.get_lens(0, B) == [Lq] * B


@pytest.mark.parametrize("name,n_check", [("llama13b_block_decode_b16_kv4096", 16),
                                          ("gqa70b_block_decode_b64_kv4096", 8)])
def test_full_decode(name, n_check):
    wl = W.get(name)
    s, B, S0 = wl.shape, wl.batch, wl.cache_len
    _flush(f"case: {name} full-size decode")
    inp = W.draw_block_workload(wl)
    x, w, kc, vc = inp["x"], inp["weights"], inp["k_cache"], inp["v_cache"]
    max_seq = S0 + 1
    blk, wd = G.make_block(s, w, max_seq)
    del wd
    cache = G.make_cache(s, 1, B, max_seq)
    for b in range(B):
        cache.write(0, b, 0, G.tdev(kc[b], s.dtype), G.tdev(vc[b], s.dtype))
    cache.set_lens(0, [S0] * B)
    sc = G.scratch(blk, B, B, max_seq)
    blk.set_diag(True)
    xd = G.tdev(x.reshape(B, s.dim), s.dtype)
    y = torch.empty_like(xd)
    blk.decode(cache, 0, xd, y, B, sc)
    torch.cuda.synchronize()
    got_y = G.thost(y)
    got_a = G.diag(blk, sc, 0, B, s.n_heads * s.head_dim, s.dtype)
    got_h = G.diag(blk, sc, 1, B, s.dim, s.dtype)
    got_f = G.diag(blk, sc, 2, B, s.dim, s.dtype)
    seqs = list(range(B)) if n_check >= B else sorted(set([0, B - 1] + list(
        np.random.default_rng(1).choice(B, size=n_check - 2, replace=False))))
    r = ref.block_forward(x[seqs], w, s, [kc[b] for b in seqs], [vc[b] for b in seqs])
    for key, got in (("y", got_y), ("attn", got_a), ("h", got_h), ("ffn", got_f)):
        err = G.check("bf16", got[seqs], np.concatenate(r[key]), f"{name} {key}")
        _flush(f"  {key}: rel L2 {err:.2e} over {len(seqs)} sequences")
    assert cache.get_lens(0, B) == [S0 + 1] * B
    # the new token's rotated key and value landed at position S0
    k = torch.empty((1, s.n_kv_heads, s.head_dim), device="cuda", dtype=torch.bfloat16)
    v = torch.empty_like(k)
    for i, b in enumerate(seqs[:4]):
        cache.read(0, b, S0, 1, k, v)
        G.check("bf16", G.thost(k), r["k_new"][i], f"appended K seq {b}")
        G.check("bf16", G.thost(v), r["v_new"][i], f"appended V seq {b}")


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_q4_13b_layer_full_width(mode):
    """One block of the 4-bit 13B stack (dim 5120, ffn 13824, group-64 affine
    weights): a 512-token prompt pass, or a decode step against 512 cached
    positions, on synthetic N(0,1) inputs."""
    base = W.get("q4_llama13b_stack40_prompt512_greedy128")
    s = base.shape
    rng = W.Rng(41)
    _flush(f"case: 13B 4-bit block {mode}")
    w = W.draw_block_weights(s, rng)
    P = base.seq_len
    blk, wd = G.make_block(s, w, P + 8)
    cache = G.make_cache(s, 1, 1, P + 8)
    blk.set_diag(True)
    if mode == "prefill":
        x = rng.normal((1, P, s.dim), 1.0, "bf16")
        sc = G.scratch(blk, P, 1, P + 8)
        xd = G.tdev(x[0], "bf16")
        y = torch.empty_like(xd)
        blk.prefill(cache, 0, xd, y, 1, P, sc)
        rows = [0, 1, 100, 255, 256, P - 1]
        r = ref.block_forward(x, w, s, query_rows=[rows])
        T = P
    else:
        x = rng.normal((1, 1, s.dim), 1.0, "bf16")
        k = rng.normal((P, s.n_kv_heads, s.head_dim), 1.0, "bf16")
        v = rng.normal((P, s.n_kv_heads, s.head_dim), 1.0, "bf16")
        cache.write(0, 0, 0, G.tdev(k, "bf16"), G.tdev(v, "bf16"))
        cache.set_lens(0, [P])
        sc = G.scratch(blk, 1, 1, P + 8)
        xd = G.tdev(x[0], "bf16")
        y = torch.empty_like(xd)
        blk.decode(cache, 0, xd, y, 1, sc)
        rows = [0]
        r = ref.block_forward(x, w, s, [k], [v])
        T = 1
    torch.cuda.synchronize()
    got = {"y": G.thost(y), "attn": G.diag(blk, sc, 0, T, s.dim, "bf16"),
           "h": G.diag(blk, sc, 1, T, s.dim, "bf16"), "ffn": G.diag(blk, sc, 2, T, s.dim, "bf16")}
    for key, g in got.items():
        err = G.check("bf16", g[rows], r[key][0], f"4-bit {mode} {key}")
        _flush(f"  {key}: rel L2 {err:.2e}")
