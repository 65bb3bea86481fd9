"""Host-side checks of the benchmark's accounting (no GPU).

The effective TFLOP/s the benchmark reports is 4 * head_dim * (causally visible query-key pairs inside the
selected blocks) divided by the time; these tests pin the pair count against a token-level brute force on
small ragged problems, and the one-GPU contract of the command line.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _packed_mask(p, rng, density):
    """Random block mask [hq][NB][W] uint32, LSB first, one row per query block (bits past the row's own
    block count stay zero, as the selection kernels write them)."""
    nb = int(p.cu_blocks[-1])
    w = max(-(-p.nblocks(r) // 32) for r in range(len(p.lens)))
    words = np.zeros((p.hq, nb, w), dtype=np.uint32)
    for r in range(len(p.lens)):
        n = p.nblocks(r)
        for h in range(p.hq):
            for i in range(n):
                bits = rng.random(n) < density
                for j in np.nonzero(bits)[0]:
                    words[h, p.cu_blocks[r] + i, j // 32] |= np.uint32(1 << (j % 32))
    return words


def _brute_force_pairs(p, words):
    """Token by token: query t sees key s <= t of its request when s's block is set in t's block row."""
    total = 0
    for r, L in enumerate(p.lens):
        for h in range(p.hq):
            for t in range(L):
                i = t // p.block
                row = words[h, p.cu_blocks[r] + i]
                for s in range(t + 1):
                    j = s // p.block
                    total += int((row[j // 32] >> np.uint32(j % 32)) & np.uint32(1))
    return total


@pytest.mark.parametrize("lens,hq,block,density", [((200,), 2, 16, 0.4), ((37, 130, 64), 3, 16, 0.25),
                                                    ((96, 1, 50), 1, 32, 0.7)])
def test_visible_pairs_equals_token_level_count(lens, hq, block, density):
    p = synth.make_problem("tiny_f32", lens=lens, hq=hq, hkv=1, block=block)
    rng = np.random.default_rng(len(lens) * 7 + hq)
    words = _packed_mask(p, rng, density)
    assert bench.visible_pairs(p, words, int(p.cu_blocks[-1])) == _brute_force_pairs(p, words)


def test_full_mask_counts_every_causal_pair():
    p = synth.make_problem("tiny_f32", lens=(300, 64, 5), hq=2, hkv=1, block=32)
    words = _packed_mask(p, np.random.default_rng(0), 1.0)
    assert bench.visible_pairs(p, words, int(p.cu_blocks[-1])) == bench.dense_pairs(p)
    assert bench.dense_pairs(p) == 2 * sum(L * (L + 1) // 2 for L in (300, 64, 5))


def test_empty_mask_counts_nothing():
    p = synth.make_problem("tiny_f32", lens=(100, 40), hq=2, hkv=1, block=16)
    words = np.zeros((2, int(p.cu_blocks[-1]), 1), dtype=np.uint32)
    assert bench.visible_pairs(p, words, int(p.cu_blocks[-1])) == 0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
