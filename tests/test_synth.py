"""The seeded generators: bf16 rounding, determinism, and the pages' shapes."""

import json
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_settings.json")


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10,
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4e38, 1e-40, -1e-40], np.float32),
        # exact ties between two bf16 values, both parities
        (np.array([0x3F808000, 0x3F818000, 0xBF808000], np.uint32)).view(np.float32),
    ])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert synth.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0
    back = synth.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                                  .to(torch.float32).numpy())


def test_generation_is_deterministic_and_head_separable():
    w = synth.WORKLOADS["mid"]
    from dataclasses import replace
    w = replace(w, N=700, H=4)
    a = synth.make_qkv(w)
    b = synth.make_qkv(w, threads=1)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    part = synth.make_qkv(w, heads=[2])
    for x, y in zip(a, part):
        np.testing.assert_array_equal(x[:, :, 2:3], y)


def test_page_workload_matches_pages_settings():
    pages = json.load(open(GOLDEN))
    w = synth.WORKLOADS["page"]
    assert [w.B, w.N, w.H, w.D] == pages["shape_BNHD"]
    assert w.sink == pages["prefix_sink_tokens"]
    assert w.frames == pages["frames"]
    assert synth.BLOCK == pages["block_tokens"]
    assert w.n_padded == 38272 and w.n_padded % pages["block_tokens"] == 0
    calls = synth.varlen_calls()
    assert len(calls) == 16 and all(36000 <= c.N <= 40000 for c in calls)
    assert all(c.H == 14 for c in calls)
