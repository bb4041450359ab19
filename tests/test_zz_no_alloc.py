"""spec_accept_noalloc (scratch in the library's static device array, no
workspace argument) against spec_accept (the caller's workspace): the same
outputs on calls in a row, each smaller than the one before -- the first at the
largest cohort the scratch array takes at the vocabulary head's size, so the
later calls reuse memory the earlier ones left behind."""
import numpy as np
import pytest

import synth
from tests.gpu_util import dev, empty, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import bit_moe_tiny_amd as m
    m.load()
    return m


def _inputs(seed, S, K, V, T):
    g = synth.generator(seed)
    z = synth.normal(g, S * (K + 1) * V, 2.0).astype(np.float32).reshape(S * (K + 1), V)
    zq = (z.reshape(S, K + 1, V)[:, :K].reshape(S * K, V).astype(np.float64)
          + synth.normal(g, S * K * V, 1.5).reshape(S * K, V)).astype(np.float32)
    drafts = synth.gumbel_drafts(zq, T, g).reshape(S, K) if K else np.zeros((S, 0), np.int32)
    u = synth.uniform24(g, S * (K + 1)).reshape(S, K + 1)
    return z, zq, drafts, u


def test_noalloc_matches_workspace_call(sv):
    T = 0.8
    cases = [(31, 4, 129280, 160), (3, 4, 129280, 161), (2, 2, 5000, 162), (4, 0, 700, 163)]
    assert sv.sv_accept_workspace_bytes(31, 4, 129280) <= sv.ACCEPT_SCRATCH_BYTES
    for S, K, V, seed in cases:
        z, zq, drafts, u = _inputs(seed, S, K, V, T)
        zd, ud = dev(z), dev(u)
        qd, dd = (dev(zq), dev(drafts)) if K else (None, None)
        got = []
        for name in ("spec_accept", "spec_accept_noalloc"):
            say(name, S, K, V)
            toks = empty((S, K + 1), "i32")
            nacc = empty((S,), "i32")
            getattr(sv, name)(S, K, V, zd, sv.SV_LOGITS, T, qd, sv.SV_LOGITS, T, dd, ud, toks, nacc)
            got.append((host(toks), host(nacc)))
        (t0, n0), (t1, n1) = got
        assert np.all(n0 >= 0), f"S={S} K={K} V={V}: invalid sequences {n0}"
        assert np.array_equal(n0, n1), f"S={S} K={K} V={V}: n_accepted {n0} vs {n1}"
        assert np.array_equal(t0, t1), f"S={S} K={K} V={V}: tokens {t0} vs {t1}"


def test_noalloc_refuses_oversized_shape(sv):
    """A cohort beyond the scratch array: SV_ESCRATCH, nothing enqueued."""
    S, K, V = 40, 4, 129280
    assert sv.sv_accept_workspace_bytes(S, K, V) > sv.ACCEPT_SCRATCH_BYTES
    t = empty((S * (K + 1), V), "f32")
    q = empty((S * K, V), "f32")
    with pytest.raises(sv.SvError) as e:
        sv.spec_accept_noalloc(S, K, V, t, sv.SV_LOGITS, 1.0, q, sv.SV_LOGITS, 1.0,
                               empty((S, K), "i32"), empty((S, K + 1), "f32"),
                               empty((S, K + 1), "i32"), empty((S,), "i32"))
    assert e.value.status == sv.SV_ESCRATCH
