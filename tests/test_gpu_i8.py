"""GPU parity of int8 caches ([kvc] §5.1: INT8 KV cache) against the oracle.

Every stored row is int8 codes plus one float32 scale (oracle/quant.py).
Bars: V codes and scales bit-exact (V is quantised from its given values);
K codes within one step of the oracle's in a vanishing fraction of elements
and K scales bit-exact in all but a vanishing fraction (K is quantised from a
float64 rotation that the two sides compute with different libm's); slot
tables bit-exact; outputs within 2e-3 max-abs of the float64 oracle's
attention over the dequantised rows.  Pools are poisoned with 0xff bytes
first (codes -1, scales NaN), so a row read outside the resident set would
show.
"""

import numpy as np
import pytest
import torch

from oracle.attention import attend_heads
from oracle.decode import pool_expected, pool_rows, paged_expected, ring_expected, ring_slot_table
from oracle.quant import quantize_rows
from oracle.rope import rope
from synth import TENSOR_K, TENSOR_V, PagedWorkload, PoolWorkload, RingWorkload, workload

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _ring(**kw):
    base = dict(name="r8", seed=81, batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                dtype="bf16", window=300, sinks=4, rope_base=10000.0, scale=0.5,
                decode_steps=6, history="chunks:100:7", cache="i8")
    base.update(kw)
    return RingWorkload(**base)


def _split(buf: torch.Tensor, rows: int, d: int):
    """(codes int8 [rows, d], scales float32 [rows]) of an int8 row buffer."""
    raw = buf.cpu()
    codes_bytes = (rows * d + 255) // 256 * 256
    codes = raw[:rows * d].view(torch.int8).numpy().reshape(rows, d)
    scales = raw[codes_bytes:codes_bytes + 4 * rows].view(torch.float32).numpy()
    return codes, scales


def _check_ring_rows(st, w, style="interleaved"):
    torch.cuda.synchronize()
    sp = st.cache.slot_pos.cpu().numpy()
    slots = w.sinks + w.window
    rows = w.batch * w.num_kv_heads * slots
    kc, ks = _split(st.cache.k, rows, w.head_dim)
    vc, vs = _split(st.cache.v, rows, w.head_dim)
    kc = kc.reshape(w.batch, w.num_kv_heads, slots, w.head_dim)
    vc = vc.reshape(w.batch, w.num_kv_heads, slots, w.head_dim)
    ks = ks.reshape(w.batch, w.num_kv_heads, slots)
    vs = vs.reshape(w.batch, w.num_kv_heads, slots)
    bad_codes = bad_scales = total = 0
    for b in range(w.batch):
        filled = np.nonzero(sp[b] >= 0)[0]
        pos = sp[b][filled].astype(np.int64)
        k_rot = rope(w.rows(TENSOR_K, b, pos), pos[:, None], w.rope_base, style)
        want_kc, want_ks = quantize_rows(k_rot)                   # [n, Hkv, d], [n, Hkv]
        want_vc, want_vs = quantize_rows(w.rows(TENSOR_V, b, pos).astype(np.float64))
        got_kc = kc[b][:, filled].transpose(1, 0, 2)
        got_vc = vc[b][:, filled].transpose(1, 0, 2)
        assert np.array_equal(got_vc, want_vc), b
        assert np.array_equal(vs[b][:, filled].T, want_vs), b
        diff = np.abs(got_kc.astype(np.int32) - want_kc.astype(np.int32))
        assert diff.max() <= 1, b
        bad_codes += int((diff > 0).sum())
        bad_scales += int((ks[b][:, filled].T != want_ks).sum())
        total += diff.size
    assert bad_codes <= max(2, 1e-4 * total), bad_codes
    assert bad_scales <= max(2, 1e-3 * total / w.head_dim), bad_scales
    return sp


@pytest.mark.parametrize("kw", [
    dict(),
    dict(num_q_heads=4, num_kv_heads=4, head_dim=64, seed=82),
    dict(num_q_heads=24, num_kv_heads=4, seed=83, window=200, history="chunks:64:9"),
    dict(num_q_heads=16, num_kv_heads=2, seed=84, sinks=0, window=64, history="chunks:50:5"),
])
@pytest.mark.parametrize("fused", [False, True])
def test_ring_i8(kw, fused):
    from tests.device_data import RingState
    w = _ring(**kw)
    st = RingState(w)
    try:
        st.prefill()
        sp = _check_ring_rows(st, w)
        for b in range(w.batch):
            assert np.array_equal(sp[b], ring_slot_table(w, b))
        for step in range(w.decode_steps):
            st.step(st.step_inputs(step), fused=fused)
            torch.cuda.synchronize()
            out = st.out.cpu().numpy()
            for b in range(w.batch):
                want, want_lse = ring_expected(w, b, step)
                assert float(np.abs(out[b] - want).max()) <= TOL, (step, b)
                assert float(np.abs(st.lse.cpu().numpy()[b] - want_lse).max()) <= 1e-3
        sp = _check_ring_rows(st, w)
        for b in range(w.batch):
            assert np.array_equal(sp[b], ring_slot_table(w, b, w.decode_steps - 1))
    finally:
        st.close()


@pytest.mark.parametrize("fused", [False, True])
def test_ring_i8_half_pairs(fused):
    """RoPE pairs (i, i + d/2) on an int8 ring: the append's and the fused
    step's quantisation of the rotated K (rows checked against the oracle's),
    and the outputs."""
    from tests.device_data import RingState
    w = _ring(seed=89, num_q_heads=16, num_kv_heads=4)
    st = RingState(w, rope_style="half")
    try:
        st.prefill()
        _check_ring_rows(st, w, "half")
        for step in range(w.decode_steps):
            st.step(st.step_inputs(step), fused=fused)
            torch.cuda.synchronize()
            out = st.out.cpu().numpy()
            for b in range(w.batch):
                want, _ = ring_expected(w, b, step, style="half")
                assert float(np.abs(out[b] - want).max()) <= TOL, (step, b)
        _check_ring_rows(st, w, "half")
    finally:
        st.close()


def _pool_state(w):
    from tests.device_data import PagedState
    st = PagedState(w)
    st.k_pool.fill_(255)   # codes -1, scales NaN: never to be read
    st.v_pool.fill_(255)
    st.fill()
    return st


@pytest.mark.parametrize("kw", [
    dict(),
    dict(num_q_heads=8, num_kv_heads=2, seed=86, block_size=16, logical_blocks=96, pool_slots=40),
])
def test_pool_i8(kw):
    base = dict(name="p8", seed=85, batch=2, num_q_heads=6, num_kv_heads=1, head_dim=128,
                dtype="bf16", block_size=64, logical_blocks=64, pool_slots=20,
                rope_base=10000.0, scale=0.5, decode_steps=2, cache="i8")
    base.update(kw)
    w = PoolWorkload(**base)
    st = _pool_state(w)
    for step in range(w.decode_steps):
        st.step(st.step_query(step))
        torch.cuda.synchronize()
        out = st.out.cpu().numpy()
        assert np.isfinite(out).all()
        for b in range(w.batch):
            want, _ = pool_expected(w, b, step)
            assert float(np.abs(out[b] - want).max()) <= TOL, (step, b)


def test_paged_i8_small():
    w = PagedWorkload(name="pg8", seed=87, batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                      dtype="bf16", block_size=16, len_range=(100, 900), shared_prefix=64,
                      scale=0.5, decode_steps=2, cache="i8")
    st = _pool_state(w)
    for step in range(w.decode_steps):
        st.step(st.step_query(step))
        torch.cuda.synchronize()
        out = st.out.cpu().numpy()
        for b in range(w.batch):
            want, _ = paged_expected(w, b, step)
            assert float(np.abs(out[b] - want).max()) <= TOL, (step, b)


@pytest.mark.parametrize("name", ["paged-i8", "long-pool-b16-i8"])
def test_pool_i8_full_size(name):
    """The int8 versions of the paged and long-pool workloads at full size,
    sampled sequences at the first and last step."""
    w = workload(name)
    st = _pool_state(w)
    n = w.decode_steps
    for step in (0, n - 1):
        st.step(st.step_query(step))
        torch.cuda.synchronize()
        out = st.out.cpu().numpy()
        for b in (0, w.batch // 2, w.batch - 1):
            want = (paged_expected if w.kind == "paged" else pool_expected)(w, b, step)[0]
            assert float(np.abs(out[b] - want).max()) <= TOL, (name, step, b)


def test_mha_ring_i8_full_size():
    """The int8 MHA ring workload (B = 8, W = 4096 + 4 sinks, history wrapped
    twice) at full size: decode steps 0 and 1 through decode_step_ring."""
    from tests.device_data import RingState
    w = workload("mha-ring-i8")
    st = RingState(w)
    try:
        st.prefill()
        for step in range(2):
            st.step(st.step_inputs(step), fused=True)
            torch.cuda.synchronize()
            out = st.out.cpu().numpy()
            for b in (0, 7):
                want, _ = ring_expected(w, b, step)
                assert float(np.abs(out[b] - want).max()) <= TOL, (step, b)
        sp = st.cache.slot_pos.cpu().numpy()
        for b in range(w.batch):
            assert np.array_equal(sp[b], ring_slot_table(w, b, 1))
    finally:
        st.close()


@pytest.mark.parametrize("scale", [1e-3, 40.0])
@pytest.mark.parametrize("heads", [(6, 1), (8, 2), (4, 4)])
def test_pool_i8_value_scales(scale, heads):
    """Rows far from unit size (every draw times 1e-3, or times 40: flat and
    one-hot softmax) through every P*V form (g = 6, 4: matrix core with the
    per-tile power-of-two weight scaling; g = 1: VALU), relative to the
    largest output: the bar 2e-3 scaled to the values' size."""
    hq, hkv = heads
    w = PoolWorkload(name="p8s", seed=88, batch=2, num_q_heads=hq, num_kv_heads=hkv,
                     head_dim=128, dtype="bf16", block_size=64, logical_blocks=48, pool_slots=20,
                     rope_base=10000.0, scale=scale, decode_steps=1, cache="i8")
    st = _pool_state(w)
    st.step(st.step_query(0))
    torch.cuda.synchronize()
    out = st.out.cpu().numpy()
    for b in range(w.batch):
        want, _ = pool_expected(w, b, 0)
        bar = TOL * float(np.abs(want).max())
        assert float(np.abs(out[b] - want).max()) <= bar, (b, scale, heads)


@pytest.mark.parametrize("heads", [(8, 2), (4, 4)])
def test_pool_i8_same_sign_queries(heads):
    """The int8 score products take the codes as 1152 + c and start from
    minus 1152 times the query's sum: queries whose dims all share a sign
    make that sum, and so the cancellation, as large as it gets.  Every head
    positive (|N(0, 1)| times 3), then every dim 1 in one head, through the
    matrix-core (g = 4) and the VALU (g = 1) P*V forms."""
    hq, hkv = heads
    w = PoolWorkload(name="p8q", seed=89, batch=2, num_q_heads=hq, num_kv_heads=hkv,
                     head_dim=128, dtype="bf16", block_size=64, logical_blocks=48, pool_slots=20,
                     rope_base=10000.0, scale=0.5, decode_steps=1, cache="i8")
    st = _pool_state(w)
    gen = torch.Generator().manual_seed(90)
    q = (torch.randn(w.batch, hq, w.head_dim, generator=gen).abs() * 3).to(torch.bfloat16)
    q[1, 0] = 1.0
    st.step(q.cuda())
    torch.cuda.synchronize()
    out = st.out.cpu().numpy()
    for b in range(w.batch):
        _, k, v = pool_rows(w, b)
        want, _ = attend_heads(q[b].double().numpy(), k, v, None)
        assert float(np.abs(out[b] - want).max()) <= TOL, b

