"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes one step of the oracle against a closed form, an invariant the
mathematics guarantees, a library routine (torch on the CPU, float64), or the
independent scalar loops of ``oracle/brute.py``.  The pages print no numeric
worked example of the block, so these are the pins.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import brute, ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _rand(*shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------- RMSNorm --
def test_rmsnorm_rms_of_output_over_weight_is_closed_form():
    # y / gamma = x / sqrt(m + eps)  =>  RMS(y / gamma) = sqrt(m / (m + eps))
    x = _rand(7, 96) * 3.0
    g = 1.0 + rng.uniform(-0.1, 0.1, 96)
    eps = 1e-5
    y = ref.rmsnorm(x, g, eps)
    m = np.mean(x * x, axis=1)
    rms = np.sqrt(np.mean((y / g) ** 2, axis=1))
    np.testing.assert_allclose(rms, np.sqrt(m / (m + eps)), rtol=1e-13)


def test_rmsnorm_constant_weight_gives_rms_equal_to_weight():
    x = _rand(5, 64)
    for c in (0.5, 1.0, 2.0):
        y = ref.rmsnorm(x, np.full(64, c), 0.0)
        np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), c, rtol=1e-13)


def test_rmsnorm_hand_example_and_constant_row():
    # x = [3, 4]: mean square 12.5, eps 0 -> y = gamma * x / sqrt(12.5)
    y = ref.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    np.testing.assert_allclose(y, [[3 / math.sqrt(12.5), 8 / math.sqrt(12.5)]], rtol=1e-15)
    # constant row c*1: y = gamma * c / sqrt(c^2 + eps); eps sits inside the root
    c, eps = 0.01, 1e-4
    y = ref.rmsnorm(np.full((1, 8), c), np.ones(8), eps)
    np.testing.assert_allclose(y, c / math.sqrt(c * c + eps), rtol=1e-14)


def test_rmsnorm_matches_brute_and_torch():
    x = _rand(3, 40)
    g = 1.0 + rng.uniform(-0.1, 0.1, 40)
    y = ref.rmsnorm(x, g, 1e-6)
    for i in range(3):
        np.testing.assert_allclose(y[i], brute.rmsnorm_vec(list(x[i]), list(g), 1e-6), rtol=1e-13)
    yt = torch.nn.functional.rms_norm(torch.from_numpy(x), (40,), torch.from_numpy(g), eps=1e-6)
    np.testing.assert_allclose(y, yt.numpy(), rtol=1e-12)


# -------------------------------------------------------------------- RoPE --
@pytest.mark.parametrize("traditional", [False, True])
def test_rope_preserves_pair_norms_and_identity_at_zero(traditional):
    d = 64
    u = _rand(9, 3, d)
    pos = np.arange(9) * 37
    out = ref.apply_rope(u, pos, 10000.0, traditional)
    if traditional:
        pa, pb, oa, ob = u[..., 0::2], u[..., 1::2], out[..., 0::2], out[..., 1::2]
    else:
        pa, pb, oa, ob = u[..., :d // 2], u[..., d // 2:], out[..., :d // 2], out[..., d // 2:]
    np.testing.assert_allclose(oa ** 2 + ob ** 2, pa ** 2 + pb ** 2, rtol=1e-12)
    np.testing.assert_array_equal(out[0], u[0])           # position 0 is the identity


@pytest.mark.parametrize("traditional", [False, True])
def test_rope_dot_depends_only_on_position_difference(traditional):
    d = 128
    q, k = _rand(1, 1, d), _rand(1, 1, d)

    def dot(m, n):
        a = ref.apply_rope(q, np.array([m]), 10000.0, traditional)
        b = ref.apply_rope(k, np.array([n]), 10000.0, traditional)
        return float(np.sum(a * b))
    base = dot(17, 5)
    for s in (1, 100, 4000):
        assert abs(dot(17 + s, 5 + s) - base) < 1e-10 * max(1.0, abs(base))
    assert abs(dot(18, 5) - base) > 1e-6                  # and it does depend on the difference


def test_rope_closed_form_unit_vectors():
    # frequencies theta^(-2i/d) and rotation sign of LLaMARoPE: u*cos + rotate(u)*sin,
    # rotate(u) = [-u2, u1]
    d, theta, p = 128, 10000.0, 7
    for i in (0, 5, 63):
        w = theta ** (-2.0 * i / d)
        e = np.zeros((1, 1, d)); e[0, 0, i] = 1.0
        out = ref.apply_rope(e, np.array([p]), theta, False)[0, 0]
        assert out[i] == pytest.approx(math.cos(p * w), abs=1e-15)
        assert out[i + d // 2] == pytest.approx(math.sin(p * w), abs=1e-15)
        e2 = np.zeros((1, 1, d)); e2[0, 0, i + d // 2] = 1.0
        out2 = ref.apply_rope(e2, np.array([p]), theta, False)[0, 0]
        assert out2[i] == pytest.approx(-math.sin(p * w), abs=1e-15)
        assert out2[i + d // 2] == pytest.approx(math.cos(p * w), abs=1e-15)
        et = np.zeros((1, 1, d)); et[0, 0, 2 * i] = 1.0  # traditional: pair (2i, 2i+1)
        ot = ref.apply_rope(et, np.array([p]), theta, True)[0, 0]
        assert ot[2 * i] == pytest.approx(math.cos(p * w), abs=1e-15)
        assert ot[2 * i + 1] == pytest.approx(math.sin(p * w), abs=1e-15)


def test_rope_quarter_turn():
    # position chosen so that the first pair turns by exactly pi/2: (a, b) -> (-b, a)
    d = 4
    u = np.array([[[1.5, 0.0, -2.0, 0.0]]])
    theta = 1.0  # all frequencies 1 -> angle = position
    out = ref.apply_rope(u, np.array([math.pi / 2]), theta, False)[0, 0]
    np.testing.assert_allclose(out, [2.0, 0.0, 1.5, 0.0], atol=1e-15)


def test_rope_interleaved_is_permuted_rotate_half():
    d = 16
    u = _rand(4, 2, d)
    pos = np.array([0, 3, 11, 4096])
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])  # de-interleave
    a = ref.apply_rope(u, pos, 10000.0, True)
    b = ref.apply_rope(u[..., perm], pos, 10000.0, False)
    inv = np.argsort(perm)
    np.testing.assert_allclose(a, b[..., inv], rtol=1e-14, atol=1e-15)


def test_rope_matches_brute():
    u = _rand(3, 2, 8)
    pos = np.array([2, 9, 100])
    for trad in (False, True):
        out = ref.apply_rope(u, pos, 500.0, trad)
        for t in range(3):
            for h in range(2):
                np.testing.assert_allclose(out[t, h], brute.rope_head(list(u[t, h]), int(pos[t]), 500.0, trad),
                                           rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------- attention --
def _sdpa_ref(q, k, v):
    """torch SDPA (float64, CPU, causal) on [L, H, d] / [L, H, d]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    return o[0].numpy().transpose(1, 0, 2)


def test_attention_mha_matches_torch_sdpa():
    L, H, d = 13, 3, 16
    q, k, v = _rand(L, H, d), _rand(L, H, d), _rand(L, H, d)
    out = ref.causal_attention(q, k, v, np.arange(L))
    np.testing.assert_allclose(out, _sdpa_ref(q, k, v), rtol=1e-12, atol=1e-13)


def test_attention_gqa_equals_mha_with_expanded_kv():
    L, H, G, d = 11, 8, 2, 8
    q, k, v = _rand(L, H, d), _rand(L, G, d), _rand(L, G, d)
    out = ref.causal_attention(q, k, v, np.arange(L))
    # replicate kv heads the way the page's expand-then-reshape does: kv head g
    # serves query heads g*n_rep ... g*n_rep + n_rep - 1
    kt = torch.from_numpy(k).unsqueeze(2).expand(L, G, H // G, d).reshape(L, H, d).numpy()
    vt = torch.from_numpy(v).unsqueeze(2).expand(L, G, H // G, d).reshape(L, H, d).numpy()
    np.testing.assert_allclose(out, _sdpa_ref(q, kt, vt), rtol=1e-12, atol=1e-13)
    # and it is NOT the h mod G map
    km = k[:, np.arange(H) % G]
    vm = v[:, np.arange(H) % G]
    assert np.max(np.abs(out - _sdpa_ref(q, km, vm))) > 1e-3


def test_attention_invariants():
    L, H, d = 9, 2, 8
    q, k, v = _rand(L, H, d), _rand(L, H, d), _rand(L, H, d)
    out = ref.causal_attention(q, k, v, np.arange(L))
    np.testing.assert_array_equal(out[0], v[0])            # position 0 sees only itself
    # all-equal keys -> uniform weights -> prefix mean of V
    ke = np.repeat(_rand(1, H, d), L, axis=0)
    oe = ref.causal_attention(q, ke, v, np.arange(L))
    pm = np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None, None]
    np.testing.assert_allclose(oe, pm, rtol=1e-12, atol=1e-14)
    # causality: perturbing token j changes no row before j
    j = 5
    k2, v2 = k.copy(), v.copy()
    k2[j] += 3.0
    v2[j] -= 2.0
    o2 = ref.causal_attention(q, k2, v2, np.arange(L))
    np.testing.assert_array_equal(o2[:j], out[:j])
    assert np.max(np.abs(o2[j:] - out[j:])) > 1e-3
    # softmax rows sum to one (also with masked -inf entries)
    s = np.where(np.tril(np.ones((L, L))) > 0, _rand(L, L), -np.inf)
    np.testing.assert_allclose(ref.softmax_rows(s).sum(axis=1), 1.0, rtol=1e-14)


def test_attention_with_cache_offset_matches_brute():
    S, L, H, G, d = 4, 3, 4, 2, 4
    q = _rand(L, H, d)
    k, v = _rand(S + L, G, d), _rand(S + L, G, d)
    out = ref.causal_attention(q, k, v, S + np.arange(L))
    for l in range(L):
        for h in range(H):
            g = h // (H // G)
            exp = brute.attend_one(list(q[l, h]), [list(k[j, g]) for j in range(S + l + 1)],
                                   [list(v[j, g]) for j in range(S + l + 1)])
            np.testing.assert_allclose(out[l, h], exp, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- SwiGLU --
def test_silu_closed_form_and_torch():
    assert ref.silu(np.array(0.0)) == 0.0
    assert float(ref.silu(np.array(1.0))) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    z = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(ref.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-13)


def test_swiglu_gate_is_w1_and_up_is_w3():
    # D = 2, F = 1: w1 picks x0, w3 picks x1, w2 = [1, 2]^T
    a, b = 0.7, -1.3
    x = np.array([[a, b]])
    f = ref.swiglu_ffn(x, np.array([[1.0, 0.0]]), np.array([[1.0], [2.0]]), np.array([[0.0, 1.0]]))
    s = a / (1 + math.exp(-a)) * b
    np.testing.assert_allclose(f, [[s, 2 * s]], rtol=1e-15)
    # W3 = 0 -> no output at all
    f0 = ref.swiglu_ffn(_rand(3, 4), _rand(5, 4), _rand(4, 5), np.zeros((5, 4)))
    np.testing.assert_array_equal(f0, 0.0)


# ------------------------------------------------------------------ block --
def _tiny_weights(shape, seed=7):
    r = W.Rng(seed)
    return W.draw_block_weights(shape, r)


def test_block_zero_projections_is_identity():
    s = W.TEST_SHAPES["tiny_gqa_d128"]
    w = dict(_tiny_weights(s))
    w["wo"] = np.zeros_like(w["wo"])
    w["w2"] = np.zeros_like(w["w2"])
    x = _rand(2, 5, s.dim)
    y = ref.stack_arrays(ref.block_forward(x, w, s), "y")
    np.testing.assert_array_equal(y, x)


@pytest.mark.parametrize("traditional", [False, True])
def test_block_matches_brute_force_tiny_gqa(traditional):
    import dataclasses
    s = dataclasses.replace(W.TEST_SHAPES["tiny_gqa_d128"], traditional=traditional)
    w = _tiny_weights(s)
    x = _rand(2, 6, s.dim)
    kc = [_rand(3, s.n_kv_heads, s.head_dim), _rand(5, s.n_kv_heads, s.head_dim)]
    vc = [_rand(3, s.n_kv_heads, s.head_dim), _rand(5, s.n_kv_heads, s.head_dim)]
    r = ref.block_forward(x, w, s, kc, vc)
    b = brute.block(x.tolist(), w, s, [c.tolist() for c in kc], [c.tolist() for c in vc])
    for i in range(2):
        np.testing.assert_allclose(r["y"][i], b["y"][i], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(r["k_new"][i], b["k_new"][i], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(r["v_new"][i], b["v_new"][i], rtol=1e-11, atol=1e-12)


def test_block_decode_reproduces_last_rows_of_full_prefill():
    # the cached generate of the MLX page and the re-run-everything generate of
    # page 二 must agree: incremental decode == the last rows of one causal pass
    s = W.TEST_SHAPES["tiny_f32"]
    w = _tiny_weights(s)
    x = _rand(2, 12, s.dim)
    full = ref.stack_arrays(ref.block_forward(x, w, s), "y")
    pre = ref.block_forward(x[:, :8], w, s)
    kc, vc = list(pre["k_new"]), list(pre["v_new"])
    for t in range(8, 12):
        r = ref.block_forward(x[:, t:t + 1], w, s, kc, vc)
        for b in range(2):
            np.testing.assert_allclose(r["y"][b][0], full[b, t], rtol=1e-12, atol=1e-12)
            kc[b] = np.concatenate([kc[b], r["k_new"][b]])
            vc[b] = np.concatenate([vc[b], r["v_new"][b]])


def test_block_query_rows_subset_matches_full():
    s = W.TEST_SHAPES["tiny_gqa_d128"]
    w = _tiny_weights(s)
    x = _rand(1, 10, s.dim)
    full = ref.block_forward(x, w, s)
    part = ref.block_forward(x, w, s, query_rows=[[0, 4, 9]])
    np.testing.assert_allclose(part["y"][0], full["y"][0][[0, 4, 9]], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------- q4 --
def test_q4_dequant_closed_form_and_group_identity():
    rr = W.Rng(3)
    lin = W.draw_q4_linear(rr, 4, 256, 64)
    codes = W.unpack_q4_codes(lin["packed"])
    assert codes.min() >= 0 and codes.max() <= 15
    Wd = ref.dequant_q4(lin)
    # element by element: scale[o, k//64] * code + bias[o, k//64]
    o, k = 2, 130
    assert Wd[o, k] == float(lin["scales"][o, 2]) * int(codes[o, k]) + float(lin["biases"][o, 2])
    # W x per group = s (q . x) + b sum(x)
    x = _rand(256)
    y = Wd @ x
    y2 = np.zeros(4)
    for g in range(4):
        sl = slice(64 * g, 64 * g + 64)
        y2 += lin["scales"][:, g].astype(float) * (codes[:, sl].astype(float) @ x[sl]) + \
            lin["biases"][:, g].astype(float) * x[sl].sum()
    np.testing.assert_allclose(y, y2, rtol=1e-12)
    # constant codes -> each group row is constant
    lin_c = dict(lin)
    lin_c["packed"] = np.full_like(lin["packed"], 0x55)
    Wc = ref.dequant_q4(lin_c)
    for g in range(4):
        blk = Wc[:, 64 * g:64 * g + 64]
        np.testing.assert_array_equal(blk, blk[:, :1].repeat(64, axis=1))
    # brute force
    bd = brute.dequant_q4(codes.tolist(), lin["scales"].tolist(), lin["biases"].tolist(), 64)
    np.testing.assert_array_equal(Wd, np.array(bd))


def test_q4_pack_layout_low_nibble_first():
    p = np.array([[0x21, 0x43, 0x65, 0x87]], dtype=np.uint8)   # codes 1,2,3,...,8
    np.testing.assert_array_equal(W.unpack_q4_codes(p)[0], [1, 2, 3, 4, 5, 6, 7, 8])
    # as one little-endian uint32 word: code k at bits 4k
    word = int(p.view("<u4")[0, 0])
    assert [(word >> (4 * k)) & 15 for k in range(8)] == [1, 2, 3, 4, 5, 6, 7, 8]


# ------------------------------------------------------------------ stack --
def _total_params(e):
    d, H, G, F, L, V = e["dim"], e["n_heads"], e["n_kv_heads"], e["ffn_dim"], e["n_layers"], e["vocab"]
    s = W.BlockShape(dim=d, n_heads=H, n_kv_heads=G, ffn_dim=F)
    return V * d + L * (s.linear_params + 2 * d) + d + d * V


def test_page_model_shapes_parameter_counts():
    g = json.load(open(os.path.join(GOLDEN, "page_shapes.json")))
    for key in ("llama2_13b", "llama2_7b", "llama2_70b"):
        assert _total_params(g[key]) == g[key]["total_params"], key
    # the workloads use exactly these block shapes
    for name, key in [("llama7b_block_prefill_b1_l2048", "llama2_7b"),
                      ("llama13b_block_decode_b16_kv4096", "llama2_13b"),
                      ("gqa70b_block_prefill_b4_l1024", "llama2_70b"),
                      ("q4_llama13b_stack40_prompt512_greedy128", "llama2_13b")]:
        s, e = W.get(name).shape, g[key]
        assert (s.dim, s.n_heads, s.n_kv_heads, s.ffn_dim) == (e["dim"], e["n_heads"], e["n_kv_heads"], e["ffn_dim"])
    st = W.get("q4_llama13b_stack40_prompt512_greedy128")
    assert st.n_layers == g["llama2_13b"]["n_layers"] and st.vocab == g["llama2_13b"]["vocab"]
    assert st.shape.group_size == g["llama2_13b"]["q_group_size"] and st.shape.traditional


def test_argmax_lowest_index_wins_ties():
    assert ref.argmax_first(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert ref.argmax_first(np.array([5.0])) == 0
    v = rng.standard_normal(1000)
    assert ref.argmax_first(v) == int(np.argmax(v))


def test_greedy_cached_equals_recompute_without_cache():
    # tiny 2-layer stack: the cached generate must emit what re-running the
    # whole prefix every step emits (the page's generate without cache)
    s = W.BlockShape(dim=64, n_heads=4, n_kv_heads=2, ffn_dim=96, traditional=True, dtype="f32")
    r = W.Rng(11)
    layers = [W.draw_block_weights(s, r) for _ in range(2)]
    head = {"embedding": r.normal((50, 64), 1.0, "f32"), "norm": r.norm_weight(64, "f32"),
            "output": r.normal((50, 64), 0.2, "f32")}
    ids = r.ids((1, 6), 50)
    out = ref.greedy_generate(ids, layers, head, s, steps=5)
    seq = list(ids[0])
    for t in range(6):
        x = ref.embed(head["embedding"], np.array([seq]))
        for w in layers:
            x = ref.stack_arrays(ref.block_forward(x, w, s), "y")
        logits = ref.lm_head_logits(x[0, -1], head["norm"], s.eps, head["output"])
        np.testing.assert_allclose(out["logits"][t], logits, rtol=1e-10, atol=1e-12)
        nxt = ref.argmax_first(logits)
        assert nxt == out["ids"][t]
        seq.append(nxt)


# ---------------------------------------------------------------- sampling --
# "生成过程" (MLX page): temperature 0 is argmax, above 0 a multinomial draw from
# softmax(logits / T); LLaMA.generate (page 二): the draw is limited to the
# nucleus (tokens by decreasing probability up to the first at which the
# cumulative probability exceeds top_p).  Pins: closed forms on a 3-token
# vocabulary, exact stratified frequencies, and the limits T -> 0, top_p -> 0.

def test_sample_closed_form_three_tokens():
    z = np.log([1.0, 2.0, 3.0])           # p = 1/6, 2/6, 3/6; cumulative 1/6, 1/2, 1
    assert ref.sample(z, 1.0, 1.0, 0.1) == 0
    assert ref.sample(z, 1.0, 1.0, 0.17) == 1
    assert ref.sample(z, 1.0, 1.0, 0.49) == 1
    assert ref.sample(z, 1.0, 1.0, 0.5) == 2      # cumulative must exceed u
    assert ref.sample(z, 1.0, 1.0, 0.999) == 2
    # temperature 2: p proportional to sqrt(1, 2, 3)
    r = np.sqrt([1.0, 2.0, 3.0])
    c = np.cumsum(r) / r.sum()
    assert ref.sample(z, 2.0, 1.0, c[0] - 1e-9) == 0
    assert ref.sample(z, 2.0, 1.0, c[0] + 1e-9) == 1
    assert ref.sample(z, 2.0, 1.0, c[1] + 1e-9) == 2


def test_sample_nucleus_closed_form():
    z = np.log([0.2, 0.5, 0.3])           # sorted: 0.5, 0.3, 0.2; cumulative 0.5, 0.8, 1.0
    # top_p 0.6: first cumulative over 0.6 is at 0.3 -> kept {1, 2}, mass 0.8
    q = ref.sample_probs(z, 1.0, 0.6)
    assert np.allclose(q, [0.0, 0.5, 0.3])
    assert ref.sample(z, 1.0, 0.6, 0.6) == 1       # 0.48 < 0.5
    assert ref.sample(z, 1.0, 0.6, 0.7) == 2       # 0.56 > 0.5
    # top_p equal to a cumulative value: strict 'exceeds' keeps one more token
    assert np.allclose(ref.sample_probs(z, 1.0, 0.5 + 1e-12), [0.0, 0.5, 0.3])
    assert np.allclose(ref.sample_probs(z, 1.0, 0.49), [0.0, 0.5, 0.0])
    # ties with the last nucleus token are all kept
    zt = np.log([0.4, 0.3, 0.3])
    assert np.allclose(ref.sample_probs(zt, 1.0, 0.5), [0.4, 0.3, 0.3])


def test_sample_stratified_frequencies_equal_probabilities():
    rng = np.random.default_rng(5)
    z = rng.normal(size=50) * 2.0
    p = np.exp(z - z.max())
    p /= p.sum()
    n = 20000
    counts = np.zeros(50)
    for j in range(n):
        counts[ref.sample(z, 1.0, 1.0, (j + 0.5) / n)] += 1
    # each token owns an interval of length p_i of [0, 1): the grid puts
    # n * p_i +- 1 points in it
    assert np.all(np.abs(counts - n * p) <= 1.0 + 1e-9)


def test_sample_limits_are_argmax():
    rng = np.random.default_rng(6)
    for _ in range(20):
        z = rng.normal(size=300)
        best = ref.argmax_first(z)
        assert ref.sample(z, 0.0, 0.9, 0.7) == best
        assert ref.sample(z, 1e-6, 1.0, float(rng.random())) == best
        assert ref.sample(z, 1.0, 1e-9, float(rng.random())) == best


# ------------------------------------------------------------ sliding window --
# Sliding-window attention ("流处理与 KV Cache", reading-notes page; window rule
# ours: the W most recent positions, the query's own included).  Pins: W = 1
# returns the query's own value row; W at least the sequence length is plain
# causal attention; brute force against an explicit per-query loop.

def test_window_one_returns_own_value():
    rng = np.random.default_rng(11)
    L, H, G, d = 7, 4, 2, 8
    q, k, v = rng.normal(size=(L, H, d)), rng.normal(size=(L, G, d)), rng.normal(size=(L, G, d))
    out = ref.causal_attention(q, k, v, np.arange(L), window=1)
    for h in range(H):
        assert np.allclose(out[:, h], v[:, h // 2], atol=1e-12)


def test_window_covering_everything_is_causal_and_brute_force():
    rng = np.random.default_rng(12)
    L, S, H, G, d = 9, 5, 2, 1, 16
    q = rng.normal(size=(L, H, d))
    k, v = rng.normal(size=(S + L, G, d)), rng.normal(size=(S + L, G, d))
    pos = S + np.arange(L)
    assert np.allclose(ref.causal_attention(q, k, v, pos, window=S + L),
                       ref.causal_attention(q, k, v, pos), atol=1e-12)
    W = 4
    out = ref.causal_attention(q, k, v, pos, window=W)
    for i in range(L):
        keys = [j for j in range(S + L) if pos[i] - W < j <= pos[i]]
        for h in range(H):
            sc = np.array([q[i, h] @ k[j, 0] / np.sqrt(d) for j in keys])
            p = np.exp(sc - sc.max())
            p /= p.sum()
            assert np.allclose(out[i, h], sum(pj * v[j, 0] for pj, j in zip(p, keys)), atol=1e-12)


# ------------------------------------------------------------- stack ends --
def test_embed_is_one_hot_product():
    # "1. 嵌入层" (MLX page): the embedding of id i is row i of the table; as a
    # product, onehot(i) . E, which picks that row exactly (every other term is 0)
    E = _rand(37, 24)
    ids = np.array([[0, 36, 5, 5, 17], [36, 0, 1, 2, 3]])
    got = ref.embed(E, ids)
    onehot = np.zeros(ids.shape + (37,))
    for idx in np.ndindex(ids.shape):
        onehot[idx + (ids[idx],)] = 1.0
    assert got.shape == (2, 5, 24)
    assert np.array_equal(got, onehot @ E)
    assert np.array_equal(got[0, 2], got[0, 3])              # a repeated id gives the same row


def test_stack_forward_is_the_no_cache_generation():
    # LLaMA.forward over the whole sequence: the logits of position t equal the
    # cached generation's logits for the id it emitted at t (the page's generate
    # without a cache re-runs this forward every step); the record hook sees
    # every block's input and cached keys
    s = W.BlockShape(dim=64, n_heads=4, n_kv_heads=2, ffn_dim=96, traditional=False, dtype="f32")
    r = W.Rng(12)
    layers = [W.draw_block_weights(s, r) for _ in range(3)]
    head = {"embedding": r.normal((40, 64), 1.0, "f32"), "norm": r.norm_weight(64, "f32"),
            "output": r.normal((40, 64), 0.2, "f32")}
    ids = r.ids((1, 5), 40)
    gen = ref.greedy_generate(ids, layers, head, s, steps=4)
    seq = np.concatenate([ids[0], gen["ids"][:-1]])
    seen = []
    got = ref.stack_forward(seq, iter(layers), head, s, rows=range(4, 9),
                            record=lambda i, x, res: seen.append((i, x.shape, res["k_new"][0].shape)))
    np.testing.assert_allclose(got, np.stack(gen["logits"]), rtol=1e-10, atol=1e-12)
    assert seen == [(i, (9, 64), (9, 2, 16)) for i in range(3)]
    # a 4-bit stack too: the same weights once dequantized
    q = W.BlockShape(dim=128, n_heads=2, n_kv_heads=2, ffn_dim=128, dtype="bf16", weight_format="q4",
                     traditional=True)
    rq = W.Rng(13)
    ql = [W.draw_block_weights(q, rq) for _ in range(2)]
    qh = {"embedding": rq.normal((64, 128), 0.5, "bf16"), "norm": rq.norm_weight(128, "bf16"),
          "output": W.draw_q4_linear(rq, 64, 128)}
    qids = rq.ids((1, 6), 64)
    gen = ref.greedy_generate(qids, ql, qh, q, steps=3)
    seq = np.concatenate([qids[0], gen["ids"][:-1]])
    got = ref.stack_forward(seq, ql, qh, q, rows=range(5, 9))
    np.testing.assert_allclose(got, np.stack(gen["logits"]), rtol=1e-10, atol=1e-12)
