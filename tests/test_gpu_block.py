"""GPU parity of the decoder block against the CPU oracle (small shapes that
still span several tiles, ragged tails and cache offsets).

Bars: fp32 max relative error (inf-norm) <= 1e-4; bf16 and 4-bit relative L2
error <= 1e-2 per output tensor, also on the attention output before wo and on
the feed-forward branch.
"""
import dataclasses

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


def _run_prefill(s, w, x, lens=None, kv=None, max_seq=None, page_size=64):
    """x: [B, L, D] numpy.  lens/kv: optional pre-existing cache per sequence."""
    B, Lq, D = x.shape
    max_seq = max_seq or (max(lens or [0]) + Lq + 8)
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, B, max_seq, page_size)
    if lens is not None:
        for b in range(B):
            if lens[b]:
                cache.write(0, b, 0, G.tdev(kv[0][b], s.dtype), G.tdev(kv[1][b], s.dtype))
        cache.set_lens(0, lens)
    sc = G.scratch(blk, B * Lq, B, max_seq)
    blk.set_diag(True)
    xd = G.tdev(x.reshape(B * Lq, D), s.dtype)
    y = torch.empty_like(xd)
    blk.prefill(cache, 0, xd, y, B, Lq, sc)
    torch.cuda.synchronize()
    return blk, cache, sc, G.thost(y).reshape(B, Lq, D)


def _oracle(s, w, x, lens=None, kv=None):
    kc = vc = None
    if lens is not None:
        kc = [kv[0][b][:lens[b]] for b in range(x.shape[0])]
        vc = [kv[1][b][:lens[b]] for b in range(x.shape[0])]
    return ref.block_forward(x, w, s, kc, vc)


def _check_branches(s, blk, sc, r, y, B, Lq):
    T = B * Lq
    attn = G.diag(blk, sc, 0, T, s.n_heads * s.head_dim, s.dtype)
    h = G.diag(blk, sc, 1, T, s.dim, s.dtype)
    ra = np.concatenate(r["attn"])
    rh = np.concatenate(r["h"])
    rf = np.concatenate(r["ffn"])
    G.check(s.dtype, attn, ra, "attention output (before wo)")
    G.check(s.dtype, h, rh, "h = x + wo o")
    f = G.diag(blk, sc, 2, T, s.dim, s.dtype)
    G.check(s.dtype, f, rf, "feed-forward branch")


# ------------------------------------------------------------------ fp32 --
def test_tiny_fp32_prefill32_then_8_decode_steps():
    wl = W.get("tiny_f32_d256_prefill32_decode8")
    inp = W.draw_block_workload(wl)
    s, w, x = wl.shape, inp["weights"], inp["x"]           # x [1, 40, 256]
    _flush("case: tiny fp32 block, prefill 32 + 8 decode")
    blk, wd = G.make_block(s, w, 64)
    cache = G.make_cache(s, 1, 1, 64)
    sc = G.scratch(blk, 32, 1, 64)
    xd = G.tdev(x[0], "f32")
    y = torch.empty_like(xd)
    blk.prefill(cache, 0, xd[:32], y[:32], 1, 32, sc)
    for t in range(32, 40):
        blk.decode(cache, 0, xd[t:t + 1], y[t:t + 1], 1, sc)
    torch.cuda.synchronize()
    got = G.thost(y)
    pre = ref.block_forward(x[:, :32], w, s)
    G.check("f32", got[:32], pre["y"][0], "prefill y")
    kc, vc = list(pre["k_new"]), list(pre["v_new"])
    for t in range(32, 40):
        r = ref.block_forward(x[:, t:t + 1], w, s, kc, vc)
        G.check("f32", got[t:t + 1], r["y"][0], f"decode step {t - 31} y")
        kc[0] = np.concatenate([kc[0], r["k_new"][0]])
        vc[0] = np.concatenate([vc[0], r["v_new"][0]])
    assert cache.get_lens(0, 1) == [40]
    # the cache holds exactly the rotated keys / values the oracle produced
    k = torch.empty((40, s.n_kv_heads, s.head_dim), device="cuda")
    v = torch.empty_like(k)
    cache.read(0, 0, 0, 40, k, v)
    G.check("f32", G.thost(k), kc[0], "cache K")
    G.check("f32", G.thost(v), vc[0], "cache V")


@pytest.mark.parametrize("traditional", [False, True])
def test_fp32_gqa_chunked_prefill_ragged_cache(traditional):
    s = dataclasses.replace(W.TEST_SHAPES["tiny_gqa_d128"], traditional=traditional)
    rng = W.Rng(5)
    w = W.draw_block_weights(s, rng)
    x = rng.normal((3, 7, s.dim), 1.0, "f32")
    lens = [0, 5, 70]
    kv = (rng.normal((3, 70, s.n_kv_heads, s.head_dim), 1.0, "f32"),
          rng.normal((3, 70, s.n_kv_heads, s.head_dim), 1.0, "f32"))
    _flush(f"case: fp32 GQA chunked prefill traditional={traditional}")
    blk, cache, sc, y = _run_prefill(s, w, x, lens, kv, max_seq=128)
    r = _oracle(s, w, x, lens, kv)
    G.check("f32", y, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, y, 3, 7)
    assert cache.get_lens(0, 3) == [7, 12, 77]


# ------------------------------------------------------------------ bf16 --
SMALL_MHA = W.BlockShape(dim=512, n_heads=4, n_kv_heads=4, ffn_dim=1536, dtype="bf16")
SMALL_GQA = W.BlockShape(dim=1024, n_heads=8, n_kv_heads=2, ffn_dim=2816, dtype="bf16")


@pytest.mark.parametrize("traditional", [False, True])
def test_bf16_prefill_mha_several_tiles_ragged(traditional):
    s = dataclasses.replace(SMALL_MHA, traditional=traditional)
    rng = W.Rng(11)
    x = rng.normal((2, 300, s.dim), 1.0, "bf16")
    w = W.draw_block_weights(s, rng)
    _flush(f"case: bf16 MHA prefill B=2 L=300 traditional={traditional}")
    blk, cache, sc, y = _run_prefill(s, w, x)
    r = _oracle(s, w, x)
    G.check("bf16", y, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, y, 2, 300)
    k = torch.empty((300, s.n_kv_heads, s.head_dim), device="cuda", dtype=torch.bfloat16)
    v = torch.empty_like(k)
    cache.read(0, 1, 0, 300, k, v)
    G.check("bf16", G.thost(k), r["k_new"][1], "cache K (rotated)")
    G.check("bf16", G.thost(v), r["v_new"][1], "cache V")


def test_bf16_prefill_mqa():
    s = MQA
    rng = W.Rng(19)
    x = rng.normal((2, 150, s.dim), 1.0, "bf16")
    w = W.draw_block_weights(s, rng)
    _flush("case: bf16 MQA prefill B=2 L=150")
    blk, cache, sc, y = _run_prefill(s, w, x)
    r = _oracle(s, w, x)
    G.check("bf16", y, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, y, 2, 150)


# sliding-window attention: each query sees its W most recent positions.
# Prefill over a cached prefix (windows that start inside the prefix, inside
# the new tokens, and key tiles wholly before a wave's window), then decode on
# both attention paths (a window shorter than a 64-key step and one that spans
# several splits); fp32 on the tiny shape.
@pytest.mark.parametrize("win", [1, 100, 300])
def test_bf16_prefill_sliding_window(win):
    s = dataclasses.replace(SMALL_GQA, window=win)
    rng = W.Rng(23)
    B, L, S = 2, 200, 150
    x = rng.normal((B, L, s.dim), 1.0, "bf16")
    kv = (rng.normal((B, S, s.n_kv_heads, s.head_dim), 1.0, "bf16"),
          rng.normal((B, S, s.n_kv_heads, s.head_dim), 1.0, "bf16"))
    w = W.draw_block_weights(s, rng)
    lens = [S, 40]
    kvl = ([kv[0][0], kv[0][1][:40]], [kv[1][0], kv[1][1][:40]])
    _flush(f"case: bf16 prefill sliding window W={win} lens={lens} L={L}")
    blk, cache, sc, y = _run_prefill(s, w, x, lens=lens, kv=kvl)
    r = ref.block_forward(x, w, s, kvl[0], kvl[1])
    G.check("bf16", y, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, y, B, L)


@pytest.mark.parametrize("win,lens", [(37, [0, 5, 300, 64]), (700, [2300, 5, 1000, 699])])
def test_bf16_decode_sliding_window(win, lens):
    s = dataclasses.replace(SMALL_GQA, window=win)
    rng = W.Rng(24)
    B, S = len(lens), max(lens)
    x = rng.normal((B, 1, s.dim), 1.0, "bf16")
    kv = (rng.normal((B, S, s.n_kv_heads, s.head_dim), 1.0, "bf16"),
          rng.normal((B, S, s.n_kv_heads, s.head_dim), 1.0, "bf16"))
    w = W.draw_block_weights(s, rng)
    _flush(f"case: bf16 decode sliding window W={win} lens={lens}")
    max_seq = (S + 1 + 63) // 64 * 64
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, B, max_seq)
    for b in range(B):
        if lens[b]:
            cache.write(0, b, 0, G.tdev(kv[0][b, :lens[b]], s.dtype), G.tdev(kv[1][b, :lens[b]], s.dtype))
    cache.set_lens(0, lens)
    sc = G.scratch(blk, B, B, max_seq)
    blk.set_diag(True)
    xd = G.tdev(x.reshape(B, s.dim), s.dtype)
    y = torch.empty_like(xd)
    blk.decode(cache, 0, xd, y, B, sc)
    torch.cuda.synchronize()
    r = _oracle(s, w, x, lens, kv)
    got = G.thost(y).reshape(B, 1, s.dim)
    G.check("bf16", got, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, got, B, 1)


def test_fp32_sliding_window_prefill_then_decode():
    wl = W.get("tiny_f32_d256_prefill32_decode8")
    inp = W.draw_block_workload(wl)
    s, w, x = dataclasses.replace(wl.shape, window=9), inp["weights"], inp["x"]
    _flush("case: fp32 tiny, sliding window 9, prefill 32 then 8 decode steps")
    max_seq = 48
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, 1, max_seq)
    sc = G.scratch(blk, 32, 1, max_seq)
    xd = G.tdev(x[0, :32], "f32")
    y = torch.empty_like(xd)
    blk.prefill(cache, 0, xd, y, 1, 32, sc)
    outs = [G.thost(y)]
    for t in range(32, 40):
        xt = G.tdev(x[0, t:t + 1], "f32")
        yt = torch.empty_like(xt)
        blk.decode(cache, 0, xt, yt, 1, sc)
        outs.append(G.thost(yt))
    torch.cuda.synchronize()
    full = np.stack(ref.block_forward(x[:, :40], w, s)["y"])[0]
    G.check("f32", np.concatenate(outs, 0), full, "prefill + decode with a window vs one windowed prefill")


# "full": the cache and the rotation table hold exactly 130 + 200 positions, so
# the second sequence's prompt ends on the last one
@pytest.mark.parametrize("full", [False, True])
def test_bf16_prefill_gqa_with_cached_prefix(full):
    s = SMALL_GQA
    rng = W.Rng(12)
    x = rng.normal((2, 200, s.dim), 1.0, "bf16")
    lens = [64, 130]
    kv = (rng.normal((2, 130, s.n_kv_heads, s.head_dim), 1.0, "bf16"),
          rng.normal((2, 130, s.n_kv_heads, s.head_dim), 1.0, "bf16"))
    w = W.draw_block_weights(s, rng)
    _flush(f"case: bf16 GQA(4) chunked prefill B=2 L=200 after 64/130 cached full={full}")
    blk, cache, sc, y = _run_prefill(s, w, x, lens, kv, max_seq=330 if full else None)
    r = _oracle(s, w, x, lens, kv)
    G.check("bf16", y, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, y, 2, 200)
    assert cache.get_lens(0, 2) == [264, 330]


# 64 sequences x 4 kv heads of 8 query heads each: the decode attention
# lengthens its key splits past 256 (to about one resident round of
# wavefronts), here to 320-key splits over ragged lengths
WIDE_GQA = W.BlockShape(dim=4096, n_heads=32, n_kv_heads=4, ffn_dim=512, dtype="bf16")


def _long_split_lens():
    r = W.Rng(21)
    return [int(v) for v in r.g.integers(1, 2300, size=59)] + [0, 1, 319, 320, 2301]


# multi-query attention: 32 query heads share one kv head, two wavefronts (or
# in-block groups) of 16 query heads each read it
MQA = W.BlockShape(dim=4096, n_heads=32, n_kv_heads=1, ffn_dim=512, dtype="bf16")


# "empty_cache": sequences at position 0 (the token attends to itself only)
# next to short ones, on the path that merges key ranges inside one block (its
# 63-key sequence decodes into the last slot of a 64-position cache);
# "mqa_short" takes that path too, "mqa_long" (over 2048 keys) the split one;
# "full_split": a 2367-key sequence decodes into the last slot of a
# 2368-position cache on the split path
@pytest.mark.parametrize("shape", ["mha", "gqa", "gqa_long_splits", "empty_cache", "mqa_short", "mqa_long",
                                   "full_split"])
def test_bf16_decode_ragged_lengths(shape):
    if shape == "gqa_long_splits":
        s, lens = WIDE_GQA, _long_split_lens()
    elif shape == "full_split":
        s, lens = WIDE_GQA, [2367, 0, 1000]
    elif shape == "empty_cache":
        s, lens = SMALL_GQA, [0, 5, 0, 63]
    elif shape == "mqa_short":
        s, lens = MQA, [0, 77, 500]
    elif shape == "mqa_long":
        s, lens = dataclasses.replace(MQA, traditional=True), [2300, 5, 1000]
    else:
        s = dataclasses.replace(SMALL_MHA if shape == "mha" else SMALL_GQA, traditional=(shape == "mha"))
        lens = [300, 1, 64, 255, 257]
    rng = W.Rng(13)
    B, S = len(lens), max(lens)
    x = rng.normal((B, 1, s.dim), 1.0, "bf16")
    kv = (rng.normal((B, S, s.n_kv_heads, s.head_dim), 1.0, "bf16"),
          rng.normal((B, S, s.n_kv_heads, s.head_dim), 1.0, "bf16"))
    w = W.draw_block_weights(s, rng)
    _flush(f"case: bf16 {shape} decode B={B} lens={lens}")
    max_seq = (S + 1 + 63) // 64 * 64
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, B, max_seq)
    for b in range(B):
        if lens[b]:
            cache.write(0, b, 0, G.tdev(kv[0][b, :lens[b]], s.dtype), G.tdev(kv[1][b, :lens[b]], s.dtype))
    cache.set_lens(0, lens)
    sc = G.scratch(blk, B, B, max_seq)
    blk.set_diag(True)
    xd = G.tdev(x.reshape(B, s.dim), s.dtype)
    y = torch.empty_like(xd)
    blk.decode(cache, 0, xd, y, B, sc)
    torch.cuda.synchronize()
    r = _oracle(s, w, x, lens, kv)
    got = G.thost(y).reshape(B, 1, s.dim)
    G.check("bf16", got, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, got, B, 1)
    assert cache.get_lens(0, B) == [l + 1 for l in lens]


# A 512-token prompt with a 16640-wide feed-forward: the W1/W3 product is 2 x
# 130 tiles of 256 x 256 (one round of 256 blocks and 4 more), so it runs as
# two launches, 256-row tiles over its first 128 tile columns and 128-row
# tiles over the last 2 (the same product as one tile shape, column for column)
def test_bf16_prefill_gemm_over_two_tile_shapes():
    s = W.BlockShape(dim=512, n_heads=4, n_kv_heads=4, ffn_dim=16640, dtype="bf16")
    rng = W.Rng(15)
    x = rng.normal((1, 512, s.dim), 1.0, "bf16")
    w = W.draw_block_weights(s, rng)
    _flush("case: bf16 prefill 512 tokens, ffn 16640 (W1/W3 over two tile shapes)")
    blk, cache, sc, y = _run_prefill(s, w, x)
    r = _oracle(s, w, x)
    G.check("bf16", y, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, y, 1, 512)


def test_bf16_prefill_then_decode_steps_match_oracle():
    s = SMALL_GQA
    rng = W.Rng(14)
    x = rng.normal((2, 103, s.dim), 1.0, "bf16")
    w = W.draw_block_weights(s, rng)
    _flush("case: bf16 prefill 100 then 3 decode steps")
    max_seq = 128
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, 2, max_seq)
    sc = G.scratch(blk, 200, 2, max_seq)
    xd = G.tdev(x, s.dtype)
    yp_d = torch.empty((2, 100, s.dim), device="cuda", dtype=torch.bfloat16)
    blk.prefill(cache, 0, xd[:, :100].contiguous(), yp_d, 2, 100, sc)
    yp = G.thost(yp_d)
    outs = []
    for t in range(100, 103):
        yt = torch.empty((2, s.dim), device="cuda", dtype=torch.bfloat16)
        blk.decode(cache, 0, xd[:, t].contiguous(), yt, 2, sc)
        outs.append(G.thost(yt))
    torch.cuda.synchronize()
    full = ref.stack_arrays(ref.block_forward(x, w, s), "y")   # one causal pass over all 103
    G.check("bf16", yp, full[:, :100], "prefill rows")
    for i, t in enumerate(range(100, 103)):
        G.check("bf16", outs[i], full[:, t], f"decode step {i + 1}")


# ------------------------------------------------------------------ 4-bit --
SMALL_Q4 = W.BlockShape(dim=512, n_heads=4, n_kv_heads=4, ffn_dim=1536, dtype="bf16", weight_format="q4",
                        traditional=True)


@pytest.mark.parametrize("B", [1, 3])
def test_q4_decode(B):
    _q4_decode_case(SMALL_Q4, B, 15)


# One sequence runs each projection with its epilogue in one kernel; K longer
# than 256 chunks of 32 splits over the block's wavefronts (2 or 4 parts, here
# of unequal lengths), with grouped-query heads and both RoPE layouts.
Q4_SINGLE = {
    "gqa_halves_k2": W.BlockShape(dim=512, n_heads=4, n_kv_heads=2, ffn_dim=9280, dtype="bf16", weight_format="q4",
                                  traditional=False),
    "long_ffn_k4": W.BlockShape(dim=512, n_heads=4, n_kv_heads=4, ffn_dim=17472, dtype="bf16", weight_format="q4",
                                traditional=True),
}


@pytest.mark.parametrize("name", sorted(Q4_SINGLE))
def test_q4_decode_single_row_k_parts(name):
    _q4_decode_case(Q4_SINGLE[name], 1, 17)


def test_q4_decode_single_row_empty_cache():
    _q4_decode_case(SMALL_Q4, 1, 18, lens=[0])


# One sequence with a cache of 1024 positions: each head's keys go to eight
# 128-key ranges merged in one block.  Ranges past the last key are empty (all
# but the first at 0 cached keys); 511 cached keys end one range exactly, 512
# put the new token alone in the next; 900 reach the last range; and six ranges
# with two query heads per kv head.
@pytest.mark.parametrize("case", ["empty", "range_full", "one_key_next", "all_ranges", "gqa_six_ranges"])
def test_q4_decode_single_row_longer_cache(case):
    lens = {"empty": 0, "range_full": 511, "one_key_next": 512, "all_ranges": 900, "gqa_six_ranges": 700}[case]
    s = Q4_SINGLE["gqa_halves_k2"] if case == "gqa_six_ranges" else SMALL_Q4
    _q4_decode_case(s, 1, 19, lens=[lens], max_seq=1024)


def _q4_decode_case(s, B, seed, lens=None, max_seq=256):
    rng = W.Rng(seed)
    lens = lens or [77, 200, 3][:B]
    S = max(200, max(lens))
    x = rng.normal((B, 1, s.dim), 1.0, "bf16")
    kv = (rng.normal((B, S, s.n_kv_heads, s.head_dim), 1.0, "bf16"),
          rng.normal((B, S, s.n_kv_heads, s.head_dim), 1.0, "bf16"))
    w = W.draw_block_weights(s, rng)
    _flush(f"case: 4-bit decode B={B} dim={s.dim} ffn={s.ffn_dim} kv_heads={s.n_kv_heads} lens={lens} "
           f"max_seq={max_seq}")
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, B, max_seq)
    for b in range(B):
        if lens[b]:
            cache.write(0, b, 0, G.tdev(kv[0][b, :lens[b]], "bf16"), G.tdev(kv[1][b, :lens[b]], "bf16"))
    cache.set_lens(0, lens)
    sc = G.scratch(blk, B, B, max_seq)
    blk.set_diag(True)
    xd = G.tdev(x.reshape(B, s.dim), "bf16")
    y = torch.empty_like(xd)
    blk.decode(cache, 0, xd, y, B, sc)
    torch.cuda.synchronize()
    r = _oracle(s, w, x, lens, kv)
    got = G.thost(y).reshape(B, 1, s.dim)
    G.check("bf16", got, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, got, B, 1)


def test_q4_prefill():
    s = SMALL_Q4
    rng = W.Rng(16)
    x = rng.normal((1, 150, s.dim), 1.0, "bf16")
    w = W.draw_block_weights(s, rng)
    _flush("case: 4-bit prefill L=150")
    blk, cache, sc, y = _run_prefill(s, w, x)
    r = _oracle(s, w, x)
    G.check("bf16", y, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, y, 1, 150)


def test_q4_prefill_odd_k_slices():
    """4-bit prompt pass whose Wo and W2 products split K into 3 and 7 slices
    (dim 1536, ffn 3584: the most slices of whole 64-column groups, at least
    512 columns each, that keep slices x 256 x 256 tiles within one round of
    256 blocks), on 150 rows (a ragged tail off every tile); grouped heads."""
    s = W.BlockShape(dim=1536, n_heads=12, n_kv_heads=4, ffn_dim=3584, dtype="bf16", weight_format="q4",
                     traditional=False)
    rng = W.Rng(61)
    x = rng.normal((1, 150, s.dim), 1.0, "bf16")
    w = W.draw_block_weights(s, rng)
    _flush("case: 4-bit prefill L=150, dim 1536, K slices 3 (wo) and 7 (w2)")
    blk, cache, sc, y = _run_prefill(s, w, x)
    r = _oracle(s, w, x)
    G.check("bf16", y, np.stack(r["y"]), "y")
    _check_branches(s, blk, sc, r, y, 1, 150)


@pytest.mark.parametrize("page_size", [128, 256])
def test_prefill_then_decode_pages_larger_than_a_tile(page_size):
    """Pages of 128 and 256 slots (each holds two or four 64-slot blocks, the
    unit the attention kernels copy): a permuted block table, every slot NaN
    before the real rows are written, cached prefixes of 0, 150 and 301
    positions, a 200-token chunked prefill (ragged tails off every tile) and
    then one decode step, both against the oracle."""
    s = SMALL_GQA
    rng = W.Rng(71 + page_size)
    w = W.draw_block_weights(s, rng)
    lens = [0, 150, 301]
    B, Lq = len(lens), 200
    max_seq = 520
    kv = (rng.normal((B, max(lens), s.n_kv_heads, s.head_dim), 1.0, "bf16"),
          rng.normal((B, max(lens), s.n_kv_heads, s.head_dim), 1.0, "bf16"))
    x = rng.normal((B, Lq + 1, s.dim), 1.0, "bf16")
    _flush(f"case: prefill 200 over cached 0/150/301, then decode, page size {page_size}")
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, B, max_seq, page_size)
    perm = np.random.default_rng(page_size).permutation(B * cache.pages_per_seq).tolist()
    cache.set_block_table(perm)
    nan = torch.full((max_seq, s.n_kv_heads, s.head_dim), float("nan"), device="cuda", dtype=torch.bfloat16)
    for b in range(B):
        cache.write(0, b, 0, nan, nan)
        if lens[b]:
            cache.write(0, b, 0, G.tdev(kv[0][b, :lens[b]], "bf16"), G.tdev(kv[1][b, :lens[b]], "bf16"))
    cache.set_lens(0, lens)
    sc = G.scratch(blk, B * Lq, B, max_seq)
    blk.set_diag(True)
    xp = G.tdev(np.ascontiguousarray(x[:, :Lq]).reshape(B * Lq, s.dim), "bf16")
    yp = torch.empty_like(xp)
    blk.prefill(cache, 0, xp, yp, B, Lq, sc)
    torch.cuda.synchronize()
    r = _oracle(s, w, np.ascontiguousarray(x[:, :Lq]), lens, kv)
    got = G.thost(yp).reshape(B, Lq, s.dim)
    G.check("bf16", got, np.stack(r["y"]), "prefill y")
    _check_branches(s, blk, sc, r, got, B, Lq)
    # the decode step attends to the prefix, the prefill's rows and itself
    xd = G.tdev(np.ascontiguousarray(x[:, Lq]), "bf16")
    yd = torch.empty_like(xd)
    blk.decode(cache, 0, xd, yd, B, sc)
    torch.cuda.synchronize()
    rd = ref.block_forward(x, w, s, [kv[0][b][:lens[b]] for b in range(B)], [kv[1][b][:lens[b]] for b in range(B)])
    G.check("bf16", G.thost(yd).reshape(B, s.dim), np.stack([yb[Lq] for yb in rd["y"]]), "decode y")
    assert list(cache.get_lens(0, B)) == [n + Lq + 1 for n in lens]


def _random_attention_case(seed):
    """A seeded random prefill configuration: heads and kv heads, window,
    batch, cached prefix per sequence and new tokens (equal counts)."""
    r = np.random.default_rng(1000 + seed)
    nh, ng = [(8, 2), (4, 4), (8, 1), (16, 2), (4, 2), (8, 8)][seed % 6]
    W_ = int(r.integers(1, 400)) if seed % 3 == 2 else 0
    B = int(r.integers(1, 4))
    L = int(r.choice([int(r.integers(1, 64)), int(r.integers(64, 330))]))
    lens = [int(r.choice([0, int(r.integers(1, 420))])) for _ in range(B)]
    return nh, ng, W_, B, L, lens


@pytest.mark.parametrize("seed", range(10))
def test_prefill_attention_random_configurations(seed):
    """Seeded random configurations of the flash prefill path (grouped, MQA and
    plain heads; windows; cached prefixes of any length; new-token counts below
    and across the 128-query and 64-key tiles), each followed by a decode step;
    y and the attention branch against the oracle."""
    nh, ng, W_, B, L, lens = _random_attention_case(seed)
    s = W.BlockShape(dim=nh * 128, n_heads=nh, n_kv_heads=ng, ffn_dim=768, dtype="bf16", traditional=bool(seed & 1),
                     window=W_)
    rng = W.Rng(2000 + seed)
    w = W.draw_block_weights(s, rng)
    kv = (rng.normal((B, max(max(lens), 1), ng, 128), 1.0, "bf16"),
          rng.normal((B, max(max(lens), 1), ng, 128), 1.0, "bf16"))
    x = rng.normal((B, L + 1, s.dim), 1.0, "bf16")
    _flush(f"case: random seed {seed}: heads {nh} kv heads {ng} window {W_} B {B} L {L} cached {lens}")
    blk, cache, sc, y = _run_prefill(s, w, np.ascontiguousarray(x[:, :L]), lens, kv, max_seq=max(lens) + L + 9)
    r = _oracle(s, w, np.ascontiguousarray(x[:, :L]), lens, kv)
    G.check("bf16", y, np.stack(r["y"]), "prefill y")
    _check_branches(s, blk, sc, r, y, B, L)
    xd = G.tdev(np.ascontiguousarray(x[:, L]), "bf16")
    yd = torch.empty_like(xd)
    blk.decode(cache, 0, xd, yd, B, sc)
    torch.cuda.synchronize()
    rd = ref.block_forward(x, w, s, [kv[0][b][:lens[b]] for b in range(B)], [kv[1][b][:lens[b]] for b in range(B)])
    G.check("bf16", G.thost(yd).reshape(B, s.dim), np.stack([yb[L] for yb in rd["y"]]), "decode y")


@pytest.mark.parametrize("seed", range(6))
def test_q4_prefill_decode_random_configurations(seed):
    """Seeded random 4-bit blocks: model widths that are and are not multiples
    of 256 (the in-GEMM dequantization, or the dequantized-weight fallback),
    grouped heads, windows, cached prefixes and a decode step after the
    prefill; y and the branches against the oracle."""
    r = np.random.default_rng(3000 + seed)
    nh, ng = [(4, 2), (3, 3), (6, 2), (2, 1), (4, 4), (5, 1)][seed]
    ffn = [1536, 1152, 2048, 640, 1024, 1408][seed]
    W_ = int(r.integers(1, 300)) if seed % 2 else 0
    B = int(r.integers(1, 4))
    L = int(r.integers(1, 260))
    lens = [int(r.choice([0, int(r.integers(1, 300))])) for _ in range(B)]
    s = W.BlockShape(dim=nh * 128, n_heads=nh, n_kv_heads=ng, ffn_dim=ffn, dtype="bf16", weight_format="q4",
                     traditional=bool(seed & 2), window=W_)
    rng = W.Rng(4000 + seed)
    w = W.draw_block_weights(s, rng)
    kv = (rng.normal((B, max(max(lens), 1), ng, 128), 1.0, "bf16"),
          rng.normal((B, max(max(lens), 1), ng, 128), 1.0, "bf16"))
    x = rng.normal((B, L + 1, s.dim), 1.0, "bf16")
    _flush(f"case: 4-bit random seed {seed}: dim {s.dim} ffn {ffn} heads {nh}/{ng} window {W_} B {B} L {L} "
           f"cached {lens}")
    blk, cache, sc, y = _run_prefill(s, w, np.ascontiguousarray(x[:, :L]), lens, kv, max_seq=max(lens) + L + 9)
    rp = _oracle(s, w, np.ascontiguousarray(x[:, :L]), lens, kv)
    G.check("bf16", y, np.stack(rp["y"]), "prefill y")
    _check_branches(s, blk, sc, rp, y, B, L)
    xd = G.tdev(np.ascontiguousarray(x[:, L]), "bf16")
    yd = torch.empty_like(xd)
    blk.decode(cache, 0, xd, yd, B, sc)
    torch.cuda.synchronize()
    rd = ref.block_forward(x, w, s, [kv[0][b][:lens[b]] for b in range(B)], [kv[1][b][:lens[b]] for b in range(B)])
    G.check("bf16", G.thost(yd).reshape(B, s.dim), np.stack([yb[L] for yb in rd["y"]]), "decode y")


# ------------------------------------------------ ragged prefill (chunked) --
# Sequences of one call bring different numbers of new tokens: each continues
# from its own cached length (RoPE offset = cache length, "2. 注意力机制" on the
# MLX page).  Two calls: the first from empty caches (one sequence brings no
# token), the second continuing every sequence (one brings 0, one brings 1, the
# others tails off the 128-query and 64-key tiles).
RAGGED = {
    "bf16_gqa": SMALL_GQA,
    "bf16_mha_interleaved": dataclasses.replace(SMALL_MHA, traditional=True),
    "bf16_gqa_window": dataclasses.replace(SMALL_GQA, window=100),
    "q4": SMALL_Q4,
    "f32_gqa": W.BlockShape(dim=256, n_heads=4, n_kv_heads=2, ffn_dim=688, dtype="f32", traditional=True),
}


@pytest.mark.parametrize("name", sorted(RAGGED))
def test_ragged_prefill_two_calls(name):
    s = RAGGED[name]
    rng = W.Rng(51)
    w = W.draw_block_weights(s, rng)
    first, second = [0, 37, 130, 5, 64], [200, 1, 0, 129, 70]
    B = len(first)
    max_seq = max(a + b for a, b in zip(first, second)) + 3
    xs = [[rng.normal((1, n, s.dim), 1.0, s.dtype) for n in call] for call in (first, second)]
    _flush(f"case: ragged prefill {name}: counts {first} then {second}")
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, B, max_seq)
    sc = G.scratch(blk, max(sum(first), sum(second)), B, max_seq)
    blk.set_diag(True)
    dt = "f32" if s.dtype == "f32" else "bf16"
    cdt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    kc = [np.zeros((0, s.n_kv_heads, s.head_dim)) for _ in range(B)]
    vc = [np.zeros((0, s.n_kv_heads, s.head_dim)) for _ in range(B)]
    before = None
    for c, call in enumerate((first, second)):
        x = np.concatenate([a[0] for a in xs[c]])
        T = x.shape[0]
        xd = G.tdev(x, s.dtype)
        y = torch.empty_like(xd)
        blk.prefill_ragged(cache, 0, xd, y, call, sc)
        torch.cuda.synchronize()
        got = {"y": G.thost(y), "attn": G.diag(blk, sc, 0, T, s.n_heads * s.head_dim, s.dtype),
               "h": G.diag(blk, sc, 1, T, s.dim, s.dtype), "ffn": G.diag(blk, sc, 2, T, s.dim, s.dtype)}
        exp = {k: [] for k in got}
        for b in range(B):
            if call[b] == 0:
                continue
            r = ref.block_forward(xs[c][b], w, s, [kc[b]], [vc[b]])
            for k in got:
                exp[k].append(r[k][0])
            kc[b] = np.concatenate([kc[b], r["k_new"][0]])
            vc[b] = np.concatenate([vc[b], r["v_new"][0]])
        for k in got:
            G.check(dt, got[k], np.concatenate(exp[k]), f"call {c} {k}")
        # every sequence on its own too
        off = 0
        for b in range(B):
            if call[b]:
                r_y = exp["y"][sum(1 for j in range(b) if call[j])]
                G.check(dt, got["y"][off:off + call[b]], r_y, f"call {c} sequence {b} y")
            off += call[b]
        assert cache.get_lens(0, B) == [sum(cl[b] for cl in (first, second)[:c + 1]) for b in range(B)]
        # the cache holds every position the oracle produced
        reads = []
        for b in range(B):
            n = kc[b].shape[0]
            if n == 0:
                reads.append(None)
                continue
            kd = torch.empty((n, s.n_kv_heads, s.head_dim), device="cuda", dtype=cdt)
            vd = torch.empty_like(kd)
            cache.read(0, b, 0, n, kd, vd)
            torch.cuda.synchronize()
            G.check(dt, G.thost(kd), kc[b], f"call {c} cache K seq {b}")
            G.check(dt, G.thost(vd), vc[b], f"call {c} cache V seq {b}")
            reads.append((G.thost(kd), G.thost(vd)))
        if c == 0:
            before = reads
        else:
            # the sequence that brought no token kept its cache bit for bit
            assert np.array_equal(reads[2][0], before[2][0]) and np.array_equal(reads[2][1], before[2][1])


def test_ragged_prefill_argument_errors_leave_cache_unchanged():
    s = SMALL_GQA
    rng = W.Rng(52)
    w = W.draw_block_weights(s, rng)
    _flush("case: ragged prefill argument errors")
    blk, wd = G.make_block(s, w, 64)
    cache = G.make_cache(s, 1, 3, 64)
    sc = G.scratch(blk, 128, 3, 64)
    x = G.tdev(rng.normal((100, s.dim), 1.0, "bf16"), "bf16")
    for counts, status in (([5, -1, 2], L.LLAMA_ERR_INVALID_ARG), ([0, 0, 0], L.LLAMA_ERR_INVALID_ARG),
                           ([10, 65, 0], L.LLAMA_ERR_CAPACITY)):
        with pytest.raises(L.LlamaError) as e:
            blk.prefill_ragged(cache, 0, x, x, counts, sc)
        assert e.value.status == status
        assert cache.get_lens(0, 3) == [0, 0, 0]
    blk.prefill_ragged(cache, 0, x, x, [10, 64, 0], sc)      # fills sequence 1 to capacity
    torch.cuda.synchronize()
    assert cache.get_lens(0, 3) == [10, 64, 0]
    with pytest.raises(L.LlamaError) as e:
        blk.prefill_ragged(cache, 0, x, x, [1, 1, 1], sc)
    assert e.value.status == L.LLAMA_ERR_CAPACITY and cache.get_lens(0, 3) == [10, 64, 0]
