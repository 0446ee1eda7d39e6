"""GPU parity of cache position shifting ([sink]: positions inside the
attention are indices in the sink+window cache) against the oracle, which
rotates every key and the query at their cache positions at read time.

Bars: outputs within 2e-3 of the oracle (the GPU keeps K baked at absolute
positions and rounded to bf16, a window key keeping its distance to the
query; only the sinks are scored against the query rotated at its cache
position); bit for bit equal to the unshifted step where shifting changes
nothing (no sinks, or nothing evicted yet); the cache ends in the same state
as after the unshifted step.
"""

import numpy as np
import pytest
import torch

from oracle.decode import ring_shifted_expected, ring_slot_table
from synth import RingWorkload, workload

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _W(**kw):
    base = dict(name="sh", seed=95, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                dtype="bf16", window=96, sinks=4, rope_base=10000.0, scale=0.5,
                decode_steps=5, history="chunks:64:5", positions="cache")
    base.update(kw)
    return RingWorkload(**base)


def _pair(w):
    """A shifted state and an unshifted twin of the same workload."""
    import dataclasses
    from tests.device_data import RingState
    a = RingState(w)
    b = RingState(dataclasses.replace(w, positions=""))
    a.prefill()
    b.prefill()
    return a, b


@pytest.mark.parametrize("kw", [
    dict(),
    dict(num_q_heads=32, num_kv_heads=8, seed=96),
    dict(num_q_heads=24, num_kv_heads=4, seed=97, sinks=20, window=80),
    dict(num_q_heads=16, num_kv_heads=16, seed=98, batch=1, window=1000,
         history="chunks:300:8"),
])
def test_shifted_step_oracle(kw):
    w = _W(**kw)
    a, b = _pair(w)
    try:
        for step in range(w.decode_steps):
            t = int(w.decode_positions(step).min())
            assert t > w.sinks + w.window - 1  # something has been evicted
            a.step(a.step_inputs(step), fused=True)
            b.step(b.step_inputs(step), fused=True)
            torch.cuda.synchronize()
            out = a.out.cpu().numpy()
            for s in range(w.batch):
                want, want_lse = ring_shifted_expected(w, s, step)
                assert float(np.abs(out[s] - want).max()) <= TOL, (step, s)
                assert float(np.abs(a.lse.cpu().numpy()[s] - want_lse).max()) <= 1e-2
            # shifting changes the sink scores: the outputs differ from the unshifted step
            assert not torch.equal(a.out, b.out)
            assert torch.equal(a.cache.k, b.cache.k) and torch.equal(a.cache.v, b.cache.v)
            assert torch.equal(a.cache.slot_pos, b.cache.slot_pos)
        sp = a.cache.slot_pos.cpu().numpy()
        for s in range(w.batch):
            assert np.array_equal(sp[s], ring_slot_table(w, s, w.decode_steps - 1))
    finally:
        a.close()
        b.close()


@pytest.mark.parametrize("kw", [
    dict(sinks=0),                                   # no sinks: nothing moves
    dict(window=600, history="chunks:100:3"),        # nothing evicted yet
])
def test_shifted_equals_unshifted_when_nothing_moves(kw):
    w = _W(**kw)
    a, b = _pair(w)
    try:
        for step in range(w.decode_steps):
            a.step(a.step_inputs(step), fused=True)
            b.step(b.step_inputs(step), fused=True)
            torch.cuda.synchronize()
            assert torch.equal(a.out, b.out) and torch.equal(a.lse, b.lse), step
            out = a.out.cpu().numpy()
            for s in range(w.batch):
                want, _ = ring_shifted_expected(w, s, step)
                assert float(np.abs(out[s] - want).max()) <= TOL, (step, s)
    finally:
        a.close()
        b.close()


def test_shifted_unsupported_on_float32():
    from decode_attention_fixed_amd.binding import SWA_ERR_UNSUPPORTED, SwaError
    from tests.device_data import RingState
    w = _W(dtype="f32", head_dim=64, num_q_heads=4, num_kv_heads=4)
    st = RingState(w)
    try:
        st.prefill()
        with pytest.raises(SwaError) as e:
            st.step(st.step_inputs(0), fused=True)
        assert e.value.code == SWA_ERR_UNSUPPORTED
    finally:
        st.close()


def test_shifted_full_size():
    """mha-ring with shifting: B = 8, W = 4096 + 4 sinks, steps 0 and 1."""
    from tests.device_data import RingState
    w = workload("mha-ring-shift")
    st = RingState(w)
    try:
        st.prefill()
        for step in range(2):
            st.step(st.step_inputs(step), fused=True)
            torch.cuda.synchronize()
            out = st.out.cpu().numpy()
            for s in (0, 7):
                want, _ = ring_shifted_expected(w, s, step)
                assert float(np.abs(out[s] - want).max()) <= TOL, (step, s)
    finally:
        st.close()
