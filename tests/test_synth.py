"""The seeded input generators: determinism, grids and distributions (CPU)."""
import hashlib

import numpy as np
import torch

import synth


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_streams_are_deterministic_and_distinct():
    a = synth.uniform24(synth.generator(0, 5), 100)
    b = synth.uniform24(synth.generator(0, 5), 100)
    c = synth.uniform24(synth.generator(0, 6), 100)
    assert _sha(a) == _sha(b) and _sha(a) != _sha(c)


def test_uniform_grid():
    u = synth.uniform24(synth.generator(1, 2), 100000)
    assert u.dtype == np.float32 and u.min() >= 0 and u.max() < 1
    assert np.all((u.astype(np.float64) * 2 ** 24) % 1 == 0)
    assert abs(u.mean() - 0.5) < 0.01


def test_normal_moments():
    z = synth.normal(synth.generator(1, 3), 200001, 2.0)
    assert abs(z.mean()) < 0.02 and abs(z.std() - 2.0) < 0.02
    assert np.all(np.isfinite(z))


def test_bf16_rounding_matches_torch():
    x = synth.normal(synth.generator(1, 4), 100000).astype(np.float32) * 3
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_q2_random_fields():
    p = synth.q2_random(synth.generator(2, 0, 0, 0), 64, 512, 0.02)
    assert p.qs.size == 64 * 2 * 64 and p.sc.size == 64 * 2 * 16 and p.d.size == 128
    assert p.d.dtype == np.float16 and 0.01 < float(np.std(p.d.astype(np.float64))) < 0.03
    # codes and nibbles cover their full range
    assert set(np.unique(p.qs & 3).tolist()) == {0, 1, 2, 3}
    assert set(np.unique(p.sc & 15).tolist()) == set(range(16))


def test_q8_random_fields():
    p = synth.q8_random(synth.generator(3, 0), 256, 256, 0.01)
    assert p.qs.min() == -127 and p.qs.max() == 127
    assert np.all(p.d >= 0)


def test_tiny_workload_shape():
    t = synth.tiny()
    assert t.x.shape == (4, 256) and t.target_logits.shape == (5, 32)
    assert t.draft_logits.shape == (4, 32) and t.drafts.shape == (1, 4)
    assert np.all((t.drafts >= 0) & (t.drafts < 32))
    assert t.uniforms.shape == (1, 5)


def test_gumbel_drafts_follow_softmax():
    z = np.array([[0.0, 1.0, 2.0, -1.0]] * 40000, np.float32)
    d = synth.gumbel_drafts(z, 0.8, synth.generator(7, 0))
    freq = np.bincount(d, minlength=4) / d.size
    e = np.exp(z[0].astype(np.float64) / np.float64(np.float32(0.8)))
    want = e / e.sum()
    assert np.allclose(freq, want, atol=0.01)


def test_accept_inputs_per_sequence_streams():
    tl = synth.normal_f32(synth.generator(4, 9), (15, 50), 2.0)
    a = synth.accept_inputs(tl, 3, 4, 1.5, 0.8, synth.CFG_COHORT)
    b = synth.accept_inputs(tl, 3, 4, 1.5, 0.8, synth.CFG_COHORT)
    assert a.draft_logits.shape == (12, 50) and a.drafts.shape == (3, 4) and a.uniforms.shape == (3, 5)
    assert _sha(a.draft_logits) == _sha(b.draft_logits) and np.array_equal(a.drafts, b.drafts)
    assert not np.array_equal(a.uniforms[0], a.uniforms[1])
