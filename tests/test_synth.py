"""The seeded generators: determinism, encoding and workload structure."""
import numpy as np
import torch

from synth import CONFIGS, ag_inputs, bf16_bits_to_f32, f32_to_bf16_bits, moe_inputs, zipf_probs
from synth.gen import split_chunks


def test_same_seed_same_bytes():
    a = ag_inputs(64, 32, 16, 4, seed=11)
    b = ag_inputs(64, 32, 16, 4, seed=11)
    c = ag_inputs(64, 32, 16, 4, seed=12)
    assert all(np.array_equal(a[k], b[k]) for k in a)
    assert not np.array_equal(a["a"], c["a"])


def test_bf16_encoding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), want)
    assert np.array_equal(bf16_bits_to_f32(want), torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_split_chunks_ascending_peers():
    a = np.arange(8 * 3, dtype=np.uint16).reshape(8, 3)
    loc, peers = split_chunks(a, 4, 2)
    assert np.array_equal(loc, a[4:6])
    assert np.array_equal(peers, np.stack([a[0:2], a[2:4], a[6:8]]))


def test_configs_shapes():
    assert CONFIGS["llama_ag"]["M"] // CONFIGS["llama_ag"]["R"] == 1024
    assert CONFIGS["gemm_rs"]["K"] == 1792 and CONFIGS["moe"]["E"] == 8


def test_zipf_top2_loads():
    """Top-2 without replacement from Zipf(1.2) over 8 experts: the expected
    number of tokens per expert is T * P(e among the two draws) with
    P = p_e + sum_{f != e} p_f p_e / (1 - p_f)."""
    T, E = 4096, 8
    p = zipf_probs(E, 1.2)
    incl = np.array([p[e] + sum(p[f] * p[e] / (1 - p[f]) for f in range(E) if f != e) for e in range(E)])
    expect = T * incl
    assert np.allclose(expect, [2890, 1656, 1065, 768, 593, 479, 400, 342], atol=2)
    inp = moe_inputs(T=T, H=8, I=8, E=E, k=2, seed=4)
    ids = inp["topk_ids"]
    assert np.all(ids[:, 0] != ids[:, 1])
    counts = np.bincount(ids.ravel(), minlength=E)
    sd = np.sqrt(T * incl * (1 - incl))
    assert np.all(np.abs(counts - expect) < 5 * sd)
    # first-slot frequencies follow p itself
    first = np.bincount(ids[:, 0], minlength=E)
    assert np.all(np.abs(first - T * p) < 5 * np.sqrt(T * p * (1 - p)))
    g = inp["topk_w"]
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-6) and np.all(g > 0)
