"""Sampled next id on the GPU against the oracle's sampler ("生成过程", MLX page;
LLaMA.generate, page 二).

A sampled id is a decision taken on floating-point sums, so it is compared
where it is unique: the oracle (fp64) is also run with the draw u and with top_p
moved by a relative 1e-5 either way; where all of those agree the GPU must give
that id, elsewhere (u or top_p within 1e-5 of a boundary) it must give one of
them.  The draws come in as inputs, seeded.
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


def _gpu_sample(logits, temperature, top_p, u):
    B, V = logits.shape
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    ud = torch.from_numpy(np.asarray(u, dtype=np.float32)).cuda()
    ids = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    L.llama_sample(lg, B, V, temperature, top_p, ud, ids)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


def _oracle_choices(z, temperature, top_p, u):
    out = set()
    for du in (1 - 1e-5, 1.0, 1 + 1e-5):
        for dp in ((1 - 1e-5, 1.0, 1 + 1e-5) if top_p < 1 else (1.0,)):
            out.add(ref.sample(z, temperature, min(1.0, top_p * dp), min(u * du, 1 - 1e-12)))
    return out


@pytest.mark.parametrize("V", [32000, 40000, 1000, 97])
@pytest.mark.parametrize("temperature,top_p", [(1.0, 1.0), (0.7, 0.9), (1.5, 0.5), (0.8, 0.05)])
def test_sample_matches_oracle(V, temperature, top_p):
    rng = W.Rng(31)
    B = 16
    logits = rng.g.normal(size=(B, V)).astype(np.float32) * 3.0
    logits[3, 5] = logits[3].max() + 4.0          # one dominant token
    logits[4, :] = 0.25                             # all tied
    u = rng.g.random(B).astype(np.float32)
    _flush(f"case: sample V={V} T={temperature} top_p={top_p}")
    got = _gpu_sample(logits, temperature, top_p, u)
    unique = 0
    for b in range(B):
        z = logits[b].astype(np.float64)
        ch = _oracle_choices(z, temperature, top_p, float(u[b]))
        assert int(got[b]) in ch, f"row {b}: gpu {got[b]} not in {sorted(ch)}"
        unique += len(ch) == 1
    assert unique >= B - 2


def test_sample_stratified_frequencies():
    # one logit row repeated with draws on a regular grid: each token must be
    # chosen for n * q_i of them, to within the grid step and fp32 rounding
    rng = W.Rng(32)
    V, n = 24, 4096
    z = (rng.g.normal(size=V) * 2.0).astype(np.float32)
    for temperature, top_p in [(1.0, 1.0), (0.9, 0.8)]:
        u = ((np.arange(n) + 0.5) / n).astype(np.float32)
        got = _gpu_sample(np.tile(z, (n, 1)), temperature, top_p, u)
        q = ref.sample_probs(z.astype(np.float64), temperature, top_p)
        q = q / q.sum()
        counts = np.bincount(got, minlength=V)
        assert np.all(counts[q == 0] == 0)
        assert np.all(np.abs(counts - n * q) <= 2.0), (counts, n * q)


def test_temperature_zero_is_argmax():
    rng = W.Rng(33)
    logits = rng.g.normal(size=(8, 5000)).astype(np.float32)
    logits[2, [10, 4000]] = logits[2].max() + 1.0    # tie: lowest index
    got = _gpu_sample(logits, 0.0, 1.0, np.zeros(8))
    assert [int(v) for v in got] == [ref.argmax_first(r) for r in logits]
