"""The 4-bit stack: embedding -> n blocks -> final RMSNorm -> output head ->
greedy argmax, prompt pass then single-token steps replayed from a HIP graph.

Token ids: several results can be correct where two logits nearly tie, so ids
are compared with the oracle step by step while the oracle's top-2 margin
exceeds 4x the largest logit error of that step; at the first near-tie the
GPU's choice must be within that bound of the oracle's best, and the
comparison stops there (after it, the two sequences legitimately differ).
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


def _build(wl, max_seq):
    s = wl.shape
    layers_np, blocks, keep = [], [], []
    head = None
    for item in W.draw_stack(wl, W.Rng(wl.seed)):
        if item[0] == "ids":
            ids = item[1]
        elif item[0] == "layer":
            w = item[2]
            layers_np.append(w)
            blk, wd = G.make_block(s, w, max_seq)
            blocks.append(blk)
            del wd
        else:
            head = item[1]
    emb = G.tdev(head["embedding"], "bf16")
    fn = G.tdev(head["norm"], "bf16")
    out = G.q4_dev(head["output"])
    stack = L.Stack(blocks, emb, wl.vocab, fn, out)
    keep += [emb, fn, out]
    return s, ids, layers_np, head, blocks, stack, keep


def _generate(stack, s, wl, ids, steps, use_graph, max_seq):
    cache = G.make_cache(s, wl.n_layers, 1, max_seq)
    sc = torch.empty(stack.scratch_bytes(ids.size, max_seq), dtype=torch.uint8, device="cuda")
    prompt = torch.from_numpy(ids.reshape(-1).astype(np.int32)).cuda()
    out_ids = torch.zeros(steps + 1, dtype=torch.int32, device="cuda")
    logits = torch.zeros((steps + 1, wl.vocab), dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        stack.generate(cache, prompt, steps, out_ids, logits, sc, use_graph=use_graph, stream=st)
    torch.cuda.synchronize()
    return out_ids.cpu().numpy(), logits.cpu().numpy(), cache


def _compare_greedy(gpu_ids, gpu_logits, oracle, tol=1e-2):
    checked = 0
    for t in range(len(gpu_ids)):
        ol = oracle["logits"][t]
        gl = gpu_logits[t].astype(np.float64)
        delta = 4.0 * float(np.max(np.abs(gl - ol)))
        top = np.sort(ol)[-2:]
        margin = float(top[1] - top[0])
        G.check("bf16", gl, ol, f"logits step {t}", tol_bf16=tol)
        if margin > delta:
            assert gpu_ids[t] == oracle["ids"][t], f"step {t}: id {gpu_ids[t]} != {oracle['ids'][t]}"
            checked += 1
            continue
        assert ol[gpu_ids[t]] >= ol.max() - delta, f"step {t}: near tie but GPU id outside the error bound"
        if gpu_ids[t] != oracle["ids"][t]:
            break
        checked += 1
    return checked


# max_seq 52: the prompt and the steps fill the cache and the rotation table
# to their last position
@pytest.mark.parametrize("max_seq", [64, 52])
def test_small_q4_stack_generate_graph_equals_eager_and_oracle(max_seq):
    s = W.BlockShape(dim=512, n_heads=4, n_kv_heads=4, ffn_dim=1536, dtype="bf16", weight_format="q4",
                     traditional=True)
    wl = W.Workload("small_q4_stack", s, "stack", batch=1, seq_len=40, decode_steps=12, n_layers=2, vocab=1000,
                    seed=31)
    _flush(f"case: small 4-bit stack, 2 layers, prompt 40, 12 steps, max_seq {max_seq}")
    s, ids, layers_np, head, blocks, stack, keep = _build(wl, max_seq)
    g_ids, g_log, cache = _generate(stack, s, wl, ids, 12, True, max_seq)
    e_ids, e_log, _ = _generate(stack, s, wl, ids, 12, False, max_seq)
    assert np.array_equal(g_ids, e_ids) and np.array_equal(g_log, e_log), "graph replay differs from eager launches"
    assert cache.get_lens(1, 1) == [40 + 12]
    for t in range(13):
        assert g_ids[t] == ref.argmax_first(g_log[t])      # device argmax == CPU argmax of the same logits
    orc = ref.greedy_generate(ids, layers_np, head, s, steps=12)
    n = _compare_greedy(g_ids, g_log, orc)
    _flush(f"  ids equal to the oracle's for {n} of 13 steps")
    assert n >= 1


def test_small_q4_stack_sampled_generation():
    """Sampled generate loop (temperature 0.8, nucleus 0.9; the draws u are
    seeded inputs): graph replay equals eager launches, every emitted id is
    llama_sample's choice on that step's logits with the same draw, and one the
    oracle's sampler allows on those logits (within a 1e-5 band of the draw)."""
    s = W.BlockShape(dim=512, n_heads=4, n_kv_heads=4, ffn_dim=1536, dtype="bf16", weight_format="q4",
                     traditional=True)
    wl = W.Workload("small_q4_stack", s, "stack", batch=1, seq_len=40, decode_steps=12, n_layers=2, vocab=1000,
                    seed=31)
    _flush("case: small 4-bit stack, sampled generation T=0.8 top_p=0.9")
    max_seq = 64
    s, ids, layers_np, head, blocks, stack, keep = _build(wl, max_seq)
    T, top_p = 0.8, 0.9
    u = torch.from_numpy(W.Rng(41).g.random(13).astype(np.float32)).cuda()
    stack.set_sampling(T, top_p, u)
    g_ids, g_log, _ = _generate(stack, s, wl, ids, 12, True, max_seq)
    e_ids, e_log, _ = _generate(stack, s, wl, ids, 12, False, max_seq)
    assert np.array_equal(g_ids, e_ids) and np.array_equal(g_log, e_log), "graph replay differs from eager launches"
    lg = torch.from_numpy(g_log).cuda()
    one = torch.empty(13, dtype=torch.int32, device="cuda")
    L.llama_sample(lg, 13, wl.vocab, T, top_p, u, one)
    torch.cuda.synchronize()
    assert np.array_equal(one.cpu().numpy(), g_ids)
    uh = u.cpu().numpy()
    greedy_steps = 0
    for t in range(13):
        z = g_log[t].astype(np.float64)
        allowed = {ref.sample(z, T, top_p, min(float(uh[t]) * f, 1 - 1e-12)) for f in (1 - 1e-5, 1.0, 1 + 1e-5)}
        assert int(g_ids[t]) in allowed
        greedy_steps += int(g_ids[t]) == ref.argmax_first(z)
    _flush(f"  {greedy_steps} of 13 sampled ids were also the argmax")
    stack.set_sampling(0.0, 1.0, None)          # back to greedy
    r_ids, r_log, _ = _generate(stack, s, wl, ids, 12, True, max_seq)
    assert all(r_ids[t] == ref.argmax_first(r_log[t]) for t in range(13))


def test_small_q4_stack_recompute_equals_cached_generation():
    """The no-cache loop (each id re-runs the prompt pass over the sequence so
    far) reproduces the cached generation: logits within the bf16 bar at every
    step and ids equal up to the first near-tie (the cached GPU run serves as
    the reference; their agreement in exact arithmetic is pinned on the
    oracle)."""
    s = W.BlockShape(dim=512, n_heads=4, n_kv_heads=4, ffn_dim=1536, dtype="bf16", weight_format="q4",
                     traditional=True)
    wl = W.Workload("small_q4_stack", s, "stack", batch=1, seq_len=40, decode_steps=12, n_layers=2, vocab=1000,
                    seed=31)
    _flush("case: small 4-bit stack, recompute vs cached generation, 12 steps")
    max_seq = 64
    s, ids, layers_np, head, blocks, stack, keep = _build(wl, max_seq)
    c_ids, c_log, _ = _generate(stack, s, wl, ids, 12, True, max_seq)
    cache = G.make_cache(s, wl.n_layers, 1, max_seq)
    sc = torch.empty(stack.scratch_bytes(ids.size + 12, max_seq), dtype=torch.uint8, device="cuda")
    prompt = torch.from_numpy(ids.reshape(-1).astype(np.int32)).cuda()
    r_ids = torch.zeros(13, dtype=torch.int32, device="cuda")
    r_log = torch.zeros((13, wl.vocab), dtype=torch.float32, device="cuda")
    stack.generate_recompute(cache, prompt, 12, r_ids, r_log, sc)
    torch.cuda.synchronize()
    assert cache.get_lens(0, 1) == [40 + 12]
    n = _compare_greedy(r_ids.cpu().numpy(), r_log.cpu().numpy(), {"ids": c_ids, "logits": c_log.astype(np.float64)},
                        tol=2e-2)
    _flush(f"  recompute ids equal to the cached run's for {n} of 13 steps")
    assert n >= 1


def test_q4_13b_width_two_layer_stack_prompt512_vs_oracle():
    """Full-width layers of the 40-layer 13B 4-bit stack (dim 5120, 40 heads, ffn
    13824, vocab 32000, a 512-token prompt) at a depth the oracle can run.

    Per component: each GPU block and the GPU head run on the oracle's own input
    activations (inputs flow from the oracle to the GPU, never back) and must match
    the oracle's outputs to 1e-2.  Chained: the GPU's own generation is compared with
    the oracle's by the margin rule; its logits error is reported, bounded by
    n_layers + 1 times the per-component bar (errors of chained bf16 blocks add up).
    """
    base = W.get("q4_llama13b_stack40_prompt512_greedy128")
    wl = base.replace(n_layers=2, decode_steps=4)
    _flush("case: 13B-width 4-bit stack, 2 layers, prompt 512, 4 steps")
    max_seq = 520
    s, ids, layers_np, head, blocks, stack, keep = _build(wl, max_seq)
    P = ids.size
    # oracle chain over the prompt
    xs = [ref.embed(head["embedding"], ids)]
    for w in layers_np:
        xs.append(ref.stack_arrays(ref.block_forward(xs[-1], w, s), "y"))
    o_logits = ref.lm_head_logits(xs[-1][0, -1], head["norm"], s.eps, head["output"])
    # each GPU block on the oracle's input of that layer
    for l, blk in enumerate(blocks):
        cache = G.make_cache(s, 1, 1, max_seq)
        sc = G.scratch(blk, P, 1, max_seq)
        xd = G.tdev(xs[l][0], "bf16")
        y = torch.empty_like(xd)
        blk.prefill(cache, 0, xd, y, 1, P, sc)
        torch.cuda.synchronize()
        err = G.check("bf16", G.thost(y), xs[l + 1][0], f"layer {l} output on the oracle's input")
        _flush(f"  layer {l}: rel L2 {err:.2e}")
    # the GPU head on the oracle's last hidden row
    hw = keep[2]
    lh = L.llama_linear(hw["w"].data_ptr(), hw["scales"].data_ptr(), hw["biases"].data_ptr())
    lg = torch.empty((1, wl.vocab), device="cuda", dtype=torch.float32)
    gid = torch.empty(1, device="cuda", dtype=torch.int32)
    hsc = torch.empty(L.llama_head_scratch_bytes(1, s.dim, wl.vocab), dtype=torch.uint8, device="cuda")
    xl = G.tdev(xs[-1][0, -1:], "bf16")
    L.llama_lm_head_argmax(lh, L.LLAMA_W_Q4, 64, L.LLAMA_BF16, keep[1], s.eps, xl, 1, s.dim, wl.vocab, lg, gid,
                           hsc, hsc.numel())
    torch.cuda.synchronize()
    err = G.check("bf16", lg.cpu().numpy()[0], o_logits, "head logits on the oracle's input")
    _flush(f"  head: rel L2 {err:.2e}")
    # chained GPU generation vs the oracle's own generation
    g_ids, g_log, _ = _generate(stack, s, wl, ids, 4, True, max_seq)
    orc = ref.greedy_generate(ids, layers_np, head, s, steps=4)
    chained = G.rel_l2(g_log[0], orc["logits"][0])
    _flush(f"  chained prompt-pass logits rel L2 {chained:.2e}")
    assert chained <= (wl.n_layers + 1) * 1e-2
    n = _compare_greedy(g_ids, g_log, orc, tol=(wl.n_layers + 1) * 1e-2)
    _flush(f"  ids equal to the oracle's for {n} of 5 steps")
    assert n >= 1


def test_q4_13b_stack40_full_generation_properties():
    """The full workload (40 layers, 512-token prompt, 128 greedy steps): graph and
    eager launches agree bit for bit, ids are the argmax of the returned logits,
    and every logit is finite."""
    wl = W.get("q4_llama13b_stack40_prompt512_greedy128")
    _flush("case: 40-layer 4-bit stack, prompt 512, 128 steps")
    max_seq = wl.seq_len + wl.decode_steps
    s, ids, layers_np, head, blocks, stack, keep = _build(wl, max_seq)
    del layers_np
    g_ids, g_log, cache = _generate(stack, s, wl, ids, wl.decode_steps, True, max_seq)
    e_ids, e_log, _ = _generate(stack, s, wl, ids, wl.decode_steps, False, max_seq)
    assert np.isfinite(g_log).all()
    assert np.array_equal(g_ids, e_ids) and np.array_equal(g_log, e_log)
    assert ((g_ids >= 0) & (g_ids < wl.vocab)).all()
    for t in range(wl.decode_steps + 1):
        assert g_ids[t] == ref.argmax_first(g_log[t])
    assert cache.get_lens(wl.n_layers - 1, 1) == [max_seq]
