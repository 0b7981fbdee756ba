"""GPU parity at the workloads' full sizes, in the launch configuration bench.py
times, checked against the oracle on every output row and every sequence.

Bars: bf16 relative L2 <= 1e-2 on the block outputs, attention outputs (before
wo), residual h and feed-forward branch, and on every appended cache row.  The
worst single-row relative L2 is reported beside each global figure.
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


def _compare(got, exp, what):
    """Global relative L2 (the bar) and the worst row's relative L2 (reported)."""
    err = G.check("bf16", got, exp, what)
    g2 = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    e2 = np.asarray(exp, dtype=np.float64).reshape(-1, exp.shape[-1])
    row = float(np.max(np.linalg.norm(g2 - e2, axis=1) / np.maximum(np.linalg.norm(e2, axis=1), 1e-300)))
    return err, row


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama7b_block_prefill_b1_l2048", "gqa70b_block_prefill_b4_l1024"])
def test_full_prefill_every_row(name):
    wl = W.get(name)
    s, B, Lq = wl.shape, wl.batch, wl.seq_len
    _flush(f"case: {name} full-size prefill, every row")
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
    got = {"y": G.thost(y).reshape(B, Lq, s.dim),
           "attn": G.diag(blk, sc, 0, T, s.n_heads * s.head_dim, s.dtype).reshape(B, Lq, -1),
           "h": G.diag(blk, sc, 1, T, s.dim, s.dtype).reshape(B, Lq, -1),
           "ffn": G.diag(blk, sc, 2, T, s.dim, s.dtype).reshape(B, Lq, -1)}
    kg, vg = [], []
    for b in range(B):
        k = torch.empty((Lq, s.n_kv_heads, s.head_dim), device="cuda", dtype=torch.bfloat16)
        v = torch.empty_like(k)
        cache.read(0, b, 0, Lq, k, v)
        kg.append(k)
        vg.append(v)
    torch.cuda.synchronize()
    assert cache.get_lens(0, B) == [Lq] * B
    kg = [G.thost(k) for k in kg]
    vg = [G.thost(v) for v in vg]
    del y, sc, cache, blk
    r = ref.block_forward(x, w, s)
    for key in ("y", "attn", "h", "ffn"):
        err, row = _compare(got[key], np.stack(r[key]), f"{name} {key}")
        _flush(f"  {key}: rel L2 {err:.2e} over {T} rows (worst row {row:.2e})")
    err, row = _compare(np.stack(kg), np.stack(r["k_new"]), f"{name} cached K")
    err2, row2 = _compare(np.stack(vg), np.stack(r["v_new"]), f"{name} cached V")
    _flush(f"  cache: K rel L2 {err:.2e} (worst row {row:.2e}), V {err2:.2e} (worst row {row2:.2e})")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama13b_block_decode_b16_kv4096", "gqa70b_block_decode_b64_kv4096"])
def test_full_decode_every_sequence(name):
    wl = W.get(name)
    s, B, S0 = wl.shape, wl.batch, wl.cache_len
    _flush(f"case: {name} full-size decode, every sequence")
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
    got = {"y": G.thost(y), "attn": G.diag(blk, sc, 0, B, s.n_heads * s.head_dim, s.dtype),
           "h": G.diag(blk, sc, 1, B, s.dim, s.dtype), "ffn": G.diag(blk, sc, 2, B, s.dim, s.dtype)}
    assert cache.get_lens(0, B) == [S0 + 1] * B
    # the new token's rotated key and value landed at position S0 of every sequence
    k = torch.empty((B, s.n_kv_heads, s.head_dim), device="cuda", dtype=torch.bfloat16)
    v = torch.empty_like(k)
    for b in range(B):
        cache.read(0, b, S0, 1, k[b:b + 1], v[b:b + 1])
    torch.cuda.synchronize()
    kn, vn = G.thost(k), G.thost(v)
    del y, sc, cache, blk
    r = ref.block_forward(x, w, s, list(kc), list(vc))
    for key in ("y", "attn", "h", "ffn"):
        err, row = _compare(got[key], np.concatenate(r[key]), f"{name} {key}")
        _flush(f"  {key}: rel L2 {err:.2e} over {B} sequences (worst sequence {row:.2e})")
    err, row = _compare(kn, np.concatenate(r["k_new"]), f"{name} appended K")
    err2, row2 = _compare(vn, np.concatenate(r["v_new"]), f"{name} appended V")
    _flush(f"  appended K rel L2 {err:.2e}, V {err2:.2e}")


@pytest.mark.parametrize("mode", ["prefill", "decode"])
def test_q4_13b_layer_full_width(mode):
    """One block of the 4-bit 13B stack (dim 5120, ffn 13824, group-64 affine
    weights): a 512-token prompt pass (every row), or a decode step against 512
    cached positions, on synthetic N(0,1) inputs."""
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
        rows = list(range(P))
        r = ref.block_forward(x, w, s)
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
