"""Paged KV cache indexing (bit-exact), failure handling from the host, and the
greedy head (argmax bit-exact against the CPU argmax of the GPU's own logits)."""
import dataclasses

import numpy as np
import pytest
import torch

import decoder_block_rmsnorm_amd as L
import workloads as W
from oracle import ref
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

S_BF = W.BlockShape(dim=512, n_heads=4, n_kv_heads=2, ffn_dim=1536, dtype="bf16", traditional=True)


def _flush(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_read_roundtrip_bitexact_with_permuted_table(dtype):
    _flush(f"case: cache write/read roundtrip {dtype}")
    G_, d, ps, max_seq, B = 3, 64 if dtype == "f32" else 128, 64, 300, 4
    cache = L.KVCache(2, B, max_seq, G_, d, dtype=G.act_code(dtype), page_size=ps)
    perm = np.random.default_rng(0).permutation(B * cache.pages_per_seq).tolist()
    cache.set_block_table(perm)
    rng = W.Rng(3)
    data = {}
    for layer in range(2):
        for b in range(B):
            n = 37 + 61 * b
            pos0 = 5 * b
            k = G.tdev(rng.normal((n, G_, d), 1.0, dtype), dtype)
            v = G.tdev(rng.normal((n, G_, d), 1.0, dtype), dtype)
            cache.write(layer, b, pos0, k, v)
            data[(layer, b)] = (pos0, k, v)
    for (layer, b), (pos0, k, v) in data.items():
        k2, v2 = torch.empty_like(k), torch.empty_like(v)
        cache.read(layer, b, pos0, k.shape[0], k2, v2)
        assert torch.equal(k2, k) and torch.equal(v2, v)


def _decode_once(s, w, table, fill_nan, lens, kv, max_seq):
    B = len(lens)
    blk, wd = G.make_block(s, w, max_seq)
    cache = G.make_cache(s, 1, B, max_seq)
    if table is not None:
        cache.set_block_table(table)
    if fill_nan:   # every slot of every page holds NaN before the real rows are written
        nan = torch.full((max_seq, s.n_kv_heads, s.head_dim), float("nan"), device="cuda", dtype=torch.bfloat16)
        for b in range(B):
            cache.write(0, b, 0, nan, nan)
    for b in range(B):
        cache.write(0, b, 0, G.tdev(kv[0][b, :lens[b]], "bf16"), G.tdev(kv[1][b, :lens[b]], "bf16"))
    cache.set_lens(0, lens)
    sc = G.scratch(blk, 3 * B, B, max_seq)
    x = torch.from_numpy(np.ascontiguousarray(kv[2])).to(torch.bfloat16).cuda()
    y = torch.empty_like(x)
    blk.decode(cache, 0, x, y, B, sc)
    # then a 3-token chunked prefill on top
    xp = torch.from_numpy(np.ascontiguousarray(kv[3])).to(torch.bfloat16).cuda()
    yp = torch.empty_like(xp)
    blk.prefill(cache, 0, xp, yp, B, 3, sc)
    torch.cuda.synchronize()
    kr = torch.empty((lens[0] + 4, s.n_kv_heads, s.head_dim), device="cuda", dtype=torch.bfloat16)
    vr = torch.empty_like(kr)
    cache.read(0, 0, 0, lens[0] + 4, kr, vr)
    return y, yp, kr, vr


def test_permuted_pages_and_nan_sentinels_give_bitwise_identical_outputs():
    _flush("case: permuted block table + NaN sentinels")
    s = S_BF
    rng = W.Rng(21)
    w = W.draw_block_weights(s, rng)
    lens = [130, 64, 1, 200]
    B = len(lens)
    max_seq = 256
    kv = (rng.normal((B, 200, s.n_kv_heads, s.head_dim), 1.0, "bf16"),
          rng.normal((B, 200, s.n_kv_heads, s.head_dim), 1.0, "bf16"),
          rng.normal((B, s.dim), 1.0, "bf16"), rng.normal((B, 3, s.dim), 1.0, "bf16"))
    base = _decode_once(s, w, None, False, lens, kv, max_seq)
    pps = (max_seq + 63) // 64
    perm = np.random.default_rng(7).permutation(B * pps).tolist()
    for table, nan in ((perm, False), (None, True), (perm, True)):
        out = _decode_once(s, w, table, nan, lens, kv, max_seq)
        for a, b in zip(base, out):
            assert torch.isfinite(b.float()).all()
            assert torch.equal(a, b)
    # and the decode output matches the oracle
    r = ref.block_forward(kv[2][:, None, :], w, s, [kv[0][b, :lens[b]] for b in range(B)],
                          [kv[1][b, :lens[b]] for b in range(B)])
    G.check("bf16", G.thost(base[0]), np.concatenate(r["y"]), "decode y")


def test_capacity_and_shape_errors_leave_cache_unchanged():
    _flush("case: host-side failure handling")
    s = S_BF
    w = W.draw_block_weights(s, W.Rng(22))
    blk, wd = G.make_block(s, w, 128)
    cache = G.make_cache(s, 1, 2, 128)
    cache.set_lens(0, [120, 5])
    sc = G.scratch(blk, 16, 2, 128)
    x = torch.zeros((2 * 9, s.dim), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(L.LlamaError) as e:
        blk.prefill(cache, 0, x, x, 2, 9, sc)      # 120 + 9 > 128
    assert e.value.status == L.LLAMA_ERR_CAPACITY
    assert cache.get_lens(0, 2) == [120, 5]
    with pytest.raises(L.LlamaError) as e:
        blk.prefill(cache, 0, x, x, 3, 1, sc)      # batch above the cache's max_batch
    assert e.value.status == L.LLAMA_ERR_INVALID_ARG
    tiny = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.LlamaError) as e:
        blk.decode(cache, 0, x, x, 2, tiny)          # scratch too small
    assert e.value.status == L.LLAMA_ERR_CAPACITY
    other = G.make_cache(dataclasses.replace(s, n_kv_heads=4), 1, 2, 128)
    with pytest.raises(L.LlamaError) as e:
        blk.decode(other, 0, x, x, 2, sc)            # cache of another block shape
    assert e.value.status == L.LLAMA_ERR_INVALID_ARG
    blk.decode(cache, 0, x[:2], x[:2], 2, sc)      # a valid call still works afterwards
    torch.cuda.synchronize()
    assert cache.get_lens(0, 2) == [121, 6]


@pytest.mark.parametrize("fmt", ["q4", "dense"])
def test_lm_head_argmax(fmt):
    _flush(f"case: lm head + argmax {fmt}")
    rng = W.Rng(23)
    D, V, B = (512, 3000, 2) if fmt == "q4" else (512, 3008, 3)
    x = rng.normal((B, D), 1.0, "bf16")
    fnorm = rng.norm_weight(D, "bf16")
    if fmt == "q4":
        lin = W.draw_q4_linear(rng, V, D, 64)
        head = G.q4_dev(lin)
        lh = L.llama_linear(head["w"].data_ptr(), head["scales"].data_ptr(), head["biases"].data_ptr())
        wf = L.LLAMA_W_Q4
    else:
        lin = rng.normal((V, D), 0.02, "bf16")
        lin[7] = lin[3]                                    # rows 3 and 7 identical: a logit tie
        head = G.tdev(lin, "bf16")
        lh = L.llama_linear(head.data_ptr(), None, None)
        wf = L.LLAMA_W_DENSE
    xd, fd = G.tdev(x, "bf16"), G.tdev(fnorm, "bf16")
    logits = torch.empty((B, V), device="cuda", dtype=torch.float32)
    ids = torch.empty(B, device="cuda", dtype=torch.int32)
    sc = torch.empty(L.llama_head_scratch_bytes(B, D, V), dtype=torch.uint8, device="cuda")
    L.llama_lm_head_argmax(lh, wf, 64, L.LLAMA_BF16, fd, 1e-5, xd, B, D, V, logits, ids, sc, sc.numel())
    torch.cuda.synchronize()
    lg = logits.cpu().numpy()
    got = ids.cpu().numpy()
    for b in range(B):
        assert got[b] == ref.argmax_first(lg[b])           # bit-exact vs CPU argmax of the same logits
    exp = np.stack([ref.lm_head_logits(x[b], fnorm, 1e-5, lin) for b in range(B)])
    G.check("bf16", lg, exp, "logits")
    if fmt == "dense":
        # force a tie at the top: x aligned with row 3 (== row 7) -> index 3 wins
        xt = np.zeros((1, D), dtype=np.float32)
        xt[0] = lin[3] / np.linalg.norm(lin[3]) * 30
        xd1 = G.tdev(W.round_bf16(xt), "bf16")
        L.llama_lm_head_argmax(lh, wf, 64, L.LLAMA_BF16, fd, 1e-5, xd1, 1, D, V, logits, ids, sc, sc.numel())
        torch.cuda.synchronize()
        l0 = logits[0].cpu().numpy()
        assert l0[3] == l0[7] and int(ids[0]) == ref.argmax_first(l0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_embed_bitexact(dtype):
    """llama_embed ("1. 嵌入层", MLX page) equals the oracle's lookup bit for bit
    (a copy of table rows: ids 0 and vocab-1, repeats, a run longer than one
    block); ids outside [0, vocab) give zero rows, as the header states."""
    _flush(f"case: embedding lookup {dtype}")
    rng = W.Rng(29)
    V, D = 3001, 640
    table = rng.normal((V, D), 0.02 if dtype == "bf16" else 1.0, dtype)
    ids = np.concatenate([[0, V - 1, 5, 5, V - 1], rng.ids((700,), V).ravel()]).astype(np.int32)
    td = G.tdev(table, dtype)
    idd = torch.from_numpy(ids).cuda()
    out = torch.empty((ids.size, D), device="cuda", dtype=td.dtype)
    L.llama_embed(td, V, D, G.act_code(dtype), idd, ids.size, out)
    torch.cuda.synchronize()
    assert np.array_equal(G.thost(out), ref.embed(table, ids))
    bad = torch.tensor([-1, V, 7], dtype=torch.int32, device="cuda")
    out2 = torch.full((3, D), 7.0, device="cuda", dtype=td.dtype)
    L.llama_embed(td, V, D, G.act_code(dtype), bad, 3, out2)
    torch.cuda.synchronize()
    got = G.thost(out2)
    assert not got[:2].any() and np.array_equal(got[2], ref.embed(table, [7])[0])
