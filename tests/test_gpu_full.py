"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (same entry points: decode_step_ring for the ring caches,
decode_attn_paged for the pools; same split plan), on sampled outputs the
oracle computes one by one: every decode step runs on the GPU, a few steps x
a few sequences (all heads) are checked against the float64 oracle, and the
ring slot tables are checked bit for bit after the history and at every
checked step.  The prefill workloads run their chunks through
prefill_attn_ring with the benchmark's output dtype (bf16) and check sampled
rows of sampled sequences."""

import numpy as np
import pytest
import torch

from oracle.decode import (paged_expected, pool_expected, ring_expected, ring_prefill_expected,
                           ring_slot_table)
from oracle.ring import slot_contents
from synth import WORKLOADS

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _checkpoints(n):
    return sorted({0, 1, n // 2, n - 1})


def _sample(batch, rng, k=3):
    pick = {0, batch - 1}
    while len(pick) < min(batch, k + 2):
        pick.add(int(rng.integers(0, batch)))
    return sorted(pick)


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", ["mha-ring", "gqa-ring"])
def test_ring_workload_full(name):
    from tests.device_data import RingState
    w = WORKLOADS[name]
    rng = np.random.default_rng(123)
    st = RingState(w)
    try:
        contiguous = w.history.startswith("chunks")

        def after(first, n):
            if not contiguous:
                return
            torch.cuda.synchronize()
            sp = st.cache.slot_pos.cpu().numpy()
            t = int(first[0]) + n - 1
            want = np.asarray(slot_contents(t, w.sinks, w.window), dtype=np.int32)
            for b in range(w.batch):
                assert np.array_equal(sp[b], want), (b, t)

        st.prefill(after)
        torch.cuda.synchronize()
        sp = st.cache.slot_pos.cpu().numpy()
        for b in range(w.batch):
            assert np.array_equal(sp[b], ring_slot_table(w, b)), b
        _log(f"{name}: history loaded, slot tables exact")
        checks = _checkpoints(w.decode_steps)
        for step in range(w.decode_steps):
            st.step(st.step_inputs(step), fused=True)  # the step the benchmark times
            if step not in checks:
                continue
            torch.cuda.synchronize()
            out = st.out.cpu().numpy()
            lse = st.lse.cpu().numpy()
            sp = st.cache.slot_pos.cpu().numpy()
            for b in range(w.batch):
                t = int(w.decode_positions(step)[b])
                if contiguous:
                    assert np.array_equal(sp[b], slot_contents(t, w.sinks, w.window))
                else:
                    assert np.array_equal(sp[b], ring_slot_table(w, b, step))
            worst = 0.0
            for b in _sample(w.batch, rng):
                want, want_lse = ring_expected(w, b, step)
                err = float(np.abs(out[b] - want).max())
                worst = max(worst, err)
                assert err <= TOL, (name, step, b, err)
                assert np.abs(lse[b] - want_lse).max() <= 1e-2
            _log(f"{name}: step {step} max-abs error {worst:.2e}")
    finally:
        st.close()


@pytest.mark.parametrize("name", ["mha-prefill", "gqa-prefill"])
def test_prefill_workload_full(name):
    from tests.device_data import RingState
    w = WORKLOADS[name]
    rng = np.random.default_rng(77)
    st = RingState(w)
    try:
        st.prefill()
        n = w.chunk
        out = torch.empty(w.batch, n, w.num_q_heads, w.head_dim, dtype=torch.bfloat16,
                          device="cuda")
        lse = torch.empty(w.batch, n, w.num_q_heads, device="cuda")
        for c in range(2):
            first = c * n
            st.prefill_chunk(st.chunk_inputs(first, n), out, lse)
            torch.cuda.synchronize()
            sp = st.cache.slot_pos.cpu().numpy()
            o = out.float().cpu().numpy()
            l = lse.cpu().numpy()
            rows = [0, 1, n // 2, n - 1]
            worst = 0.0
            for b in _sample(w.batch, rng, k=2):
                assert np.array_equal(sp[b], ring_slot_table(w, b, first + n - 1)), (b, c)
                want, want_lse = ring_prefill_expected(w, b, first, n, rows=rows)
                err = float(np.abs(o[b][rows] - want).max())
                worst = max(worst, err)
                assert err <= TOL, (name, c, b, err)
                assert np.abs(l[b][rows] - want_lse).max() <= 1e-2
            _log(f"{name}: chunk {c} max-abs error {worst:.2e}")
    finally:
        st.close()


@pytest.mark.parametrize("name", ["paged", "long-pool-b1", "long-pool-b16"])
def test_paged_workload_full(name):
    from tests.device_data import PagedState
    w = WORKLOADS[name]
    rng = np.random.default_rng(321)
    st = PagedState(w)
    st.fill()
    expected = paged_expected if w.kind == "paged" else pool_expected
    checks = _checkpoints(w.decode_steps)
    _log(f"{name}: pool loaded ({st.num_phys} blocks)")
    for step in range(w.decode_steps):
        st.step(st.step_query(step))
        if step not in checks:
            continue
        torch.cuda.synchronize()
        out = st.out.cpu().numpy()
        lse = st.lse.cpu().numpy()
        worst = 0.0
        for b in _sample(w.batch, rng, k=2):
            want, want_lse = expected(w, b, step)
            err = float(np.abs(out[b] - want).max())
            worst = max(worst, err)
            assert err <= TOL, (name, step, b, err)
            assert np.abs(lse[b] - want_lse).max() <= 1e-2
        _log(f"{name}: step {step} max-abs error {worst:.2e}")


def test_workspace_reuse_across_lengths():
    """One workspace reused with different sequence lengths (and dirtied in
    between) gives the same bits as a fresh one: no state survives a call."""
    from decode_attention_fixed_amd import binding as B
    g = torch.Generator().manual_seed(3)
    batch, hq, hkv, d, bs, nb = 3, 8, 2, 128, 16, 300
    nphys = batch * nb
    k = (torch.randn(nphys, hkv, bs, d, generator=g) * 0.5).to(torch.bfloat16).cuda()
    v = (torch.randn(nphys, hkv, bs, d, generator=g) * 0.5).to(torch.bfloat16).cuda()
    q = (torch.randn(batch, hq, d, generator=g) * 0.5).to(torch.bfloat16).cuda()
    bt = torch.randperm(nphys, generator=g).reshape(batch, nb).to(torch.int32).cuda()
    desc = B.make_paged_desc(batch, hq, hkv, d, bs, nb, nphys, "bf16")
    shared = B.new_workspace(batch, hq, hkv, d, nb * bs)

    def run(lens, ws):
        out = torch.empty(batch, hq, d, device="cuda")
        B.decode_attn_paged(desc, q, k, v, bt, torch.tensor(lens, dtype=torch.int32,
                                                             device="cuda"),
                            None, out, ws)
        torch.cuda.synchronize()
        return out

    for lens in ([4800, 17, 2000], [1, 4800, 333], [4800, 4800, 4800], [0, 5, 4000]):
        fresh = run(lens, B.new_workspace(batch, hq, hkv, d, nb * bs))
        assert torch.equal(run(lens, shared), fresh)
        shared.fill_(0x7F)  # NaN patterns everywhere
