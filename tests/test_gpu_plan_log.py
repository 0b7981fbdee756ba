"""LLAMA_LOG plan logging (GPU): with LLAMA_LOG=1 every launch plan the library
picks is printed to stderr, and the results are those of an unlogged run.

The variable is read once per process, so each setting runs one small bf16
GQA block (prefill of 96 tokens through the MFMA GEMM and flash attention, one
decode step through the GEMVs and split decode attention) in a child process of
its own, which writes y to a file."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np, torch
sys.path.insert(0, sys.argv[2])
import decoder_block_rmsnorm_amd as L
import workloads as W
s = W.BlockShape(dim=512, n_heads=4, n_kv_heads=2, ffn_dim=1536, dtype="bf16", traditional=False)
rng = W.Rng(3)
x = rng.normal((1, 97, s.dim), 1.0, "bf16")
w = W.draw_block_weights(s, rng)
dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()
wd = {k: dev(v) for k, v in w.items()}
cfg = L.block_config(s.dim, s.n_heads, s.n_kv_heads, s.ffn_dim, norm_eps=s.eps, rope_theta=s.rope_theta,
                     act_dtype=L.LLAMA_BF16, max_seq=128)
blk = L.Block(cfg, wd)
cache = L.KVCache(1, 1, 128, s.n_kv_heads, s.head_dim, dtype=L.LLAMA_BF16)
sc = torch.empty(blk.scratch_bytes(96, 1, 128), dtype=torch.uint8, device="cuda")
xd = dev(x[0]); y = torch.empty_like(xd)
blk.prefill(cache, 0, xd[:96], y[:96], 1, 96, sc)
blk.decode(cache, 0, xd[96:], y[96:], 1, sc)
torch.cuda.synchronize()
np.save(sys.argv[1], y.float().cpu().numpy())
"""


def _run(tmp_path, log: str):
    out = str(tmp_path / f"y_{log}.npy")
    env = dict(os.environ, LLAMA_LOG=log)
    r = subprocess.run([sys.executable, "-c", CHILD, out, ROOT], capture_output=True, text=True, env=env,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    return np.load(out), [l for l in r.stderr.splitlines() if l.startswith("[llama] ")]


@pytest.mark.gpu
def test_plan_log_lines_and_unchanged_results(tmp_path):
    print("case: LLAMA_LOG=1 vs 0, bf16 GQA block dim 512, prefill 96 + decode 1", flush=True)
    y_on, lines = _run(tmp_path, "1")
    y_off, quiet = _run(tmp_path, "0")
    assert quiet == []
    assert np.array_equal(y_on, y_off)
    text = "\n".join(lines)
    for what in ("block prefill", "gemm M 96", "attention prefill", "block decode", "gemv M 1",
                 "attention decode"):
        assert f"[llama] {what}" in text, (what, text)
