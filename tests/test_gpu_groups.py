"""GQA groups of two and three query heads per kv head ([share] §2.2 and §4.1)
on the head_dim 128 matrix-core decode, which builds distinct code for them:
two-query-head tiles (four row subtiles on rings, two on bf16 pools, with the
whole-tile load copy left out), the P*V product on the VALU for g = 2 and on
the matrix core from g = 3 on, and int8 rows for both.

Covered for g = 2 and g = 3, bf16 and int8 caches, against the float64
oracle (out within 2e-3, lse within 1e-3; slot tables bit-exact):
  ring      decode_attn_ring after kv_append_rope, and the fused
            decode_step_ring, on a wrapped ring; a 20000-slot ring at batch 1
            (many splits and the merge launch)
  fused     decode_step_ring leaves the cache bit-identical to
            kv_append_rope + decode_attn_ring
  pools     the eight-wave grid (small pools) and the 512 four-wave grid
            (reached with a wide block table: the grid is chosen from the
            pool's capacity, not from the lengths), pools poisoned first (NaN
            for bf16, 0xff bytes for int8: codes -1 and NaN scales) so that a
            row read outside the resident set shows
"""

import numpy as np
import pytest
import torch

from oracle.decode import paged_expected, pool_expected, ring_expected, ring_slot_table
from synth import PagedWorkload, PoolWorkload, RingWorkload

pytestmark = pytest.mark.gpu

TOL = 2e-3
GROUPS = [(4, 2), (6, 2)]   # (Hq, Hkv): g = 2 and g = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _log(msg):
    print(msg, flush=True)


def _ring(hq, hkv, cache, **kw):
    base = dict(name="g", seed=61 + hq, batch=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                dtype="bf16", window=300, sinks=4, rope_base=10000.0, scale=0.5,
                decode_steps=5, history="chunks:100:7", cache="i8" if cache == "i8" else "")
    base.update(kw)
    return RingWorkload(**base)


@pytest.mark.parametrize("cache", ["bf16", "i8"])
@pytest.mark.parametrize("heads", GROUPS, ids=["g2", "g3"])
@pytest.mark.parametrize("fused", [False, True], ids=["two-calls", "fused"])
@pytest.mark.parametrize("shape", ["wrapped", "splits"])
def test_ring_groups(cache, heads, fused, shape):
    from tests.device_data import RingState
    hq, hkv = heads
    kw = {} if shape == "wrapped" else dict(batch=1, window=20000, history="prefill:25000",
                                           decode_steps=3)
    w = _ring(hq, hkv, cache, **kw)
    st = RingState(w)
    try:
        st.prefill()
        torch.cuda.synchronize()
        for step in range(w.decode_steps):
            st.step(st.step_inputs(step), fused=fused)
            torch.cuda.synchronize()
            out = st.out.cpu().numpy()
            lse = st.lse.cpu().numpy()
            sp = st.cache.slot_pos.cpu().numpy()
            for b in range(w.batch):
                assert np.array_equal(sp[b], ring_slot_table(w, b, step)), (b, step)
                want, want_lse = ring_expected(w, b, step)
                err = float(np.abs(out[b] - want).max())
                assert err <= TOL, (b, step, err)
                assert float(np.abs(lse[b] - want_lse).max()) <= 1e-3, (b, step)
        _log(f"g={hq // hkv} {cache} {shape} {'fused' if fused else 'two calls'}: ok")
    finally:
        st.close()


@pytest.mark.parametrize("cache", ["bf16", "i8"])
@pytest.mark.parametrize("heads", GROUPS, ids=["g2", "g3"])
def test_fused_step_bit_identical_groups(cache, heads):
    """The fused step and the two calls leave identical caches; outputs agree
    to float32 rounding (g = 3 on int8: P*V weights in fp16, the new token
    added in float32 at the merge: 1e-3)."""
    from decode_attention_fixed_amd import binding as B
    from tests.device_data import RingState
    hq, hkv = heads
    w = _ring(hq, hkv, cache, decode_steps=6)
    a, b = RingState(w), RingState(w)
    try:
        for st in (a, b):
            st.cache.k.zero_()
            st.cache.v.zero_()
            st.prefill()
        tol = 1e-3 if (cache == "i8" and hq // hkv >= 3) else 1e-5
        for step in range(w.decode_steps):
            inp = a.step_inputs(step)
            q = inp["q"].clone()
            B.kv_append_rope(a.cache.handle, inp["k"], inp["v"], inp["pos"], q)
            B.decode_attn_ring(a.cache.handle, q[:, 0], a.out, a.workspace, a.lse)
            B.decode_step_ring(b.cache.handle, inp["k"][:, 0], inp["v"][:, 0], inp["pos"],
                               inp["q"][:, 0], b.out, b.workspace, b.lse)
            torch.cuda.synchronize()
            assert torch.equal(a.cache.slot_pos, b.cache.slot_pos), step
            assert torch.equal(a.cache.k, b.cache.k), step
            assert torch.equal(a.cache.v, b.cache.v), step
            assert (a.out - b.out).abs().max().item() <= tol, step
            assert (a.lse - b.lse).abs().max().item() <= 1e-5, step
    finally:
        a.close()
        b.close()


def _poisoned_state(w):
    from tests.device_data import PagedState
    st = PagedState(w)
    if getattr(w, "cache", "") == "i8":
        st.k_pool.fill_(255)   # codes -1, scales NaN
        st.v_pool.fill_(255)
    else:
        st.k_pool.fill_(float("nan"))
        st.v_pool.fill_(float("nan"))
    st.fill()
    return st


def _widen(st, max_blocks):
    """The same pool behind a block table of max_blocks columns (the extra
    entries absent): capacity rows B * Hkv * max_blocks * bs of 2^20 or more
    select the 512-workgroup four-wave grid."""
    from decode_attention_fixed_amd import binding as B
    w = st.w
    n = st.block_table.shape[1]
    bt = torch.full((w.batch, max_blocks), -1, dtype=torch.int32, device="cuda")
    bt[:, :n] = st.block_table
    st.block_table = bt
    if st.block_valid is not None:
        bv = torch.zeros((w.batch, max_blocks), dtype=torch.uint8, device="cuda")
        bv[:, :n] = st.block_valid
        st.block_valid = bv
    assert w.batch * w.num_kv_heads * max_blocks * w.block_size >= 512 * 2048
    st.desc = B.make_paged_desc(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                max_blocks, st.num_phys, w.cache or w.dtype)
    st.workspace = B.new_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                   max_blocks * w.block_size)


def _check(st, expected_fn):
    w = st.w
    for step in range(w.decode_steps):
        st.step(st.step_query(step))
        torch.cuda.synchronize()
        out = st.out.cpu().numpy()
        lse = st.lse.cpu().numpy()
        assert np.isfinite(out).all()
        for b in range(w.batch):
            want, want_lse = expected_fn(w, b, step)
            err = float(np.abs(out[b] - want).max())
            assert err <= TOL, (b, step, err)
            assert float(np.abs(lse[b] - want_lse).max()) <= 1e-3, (b, step)


@pytest.mark.parametrize("cache", ["bf16", "i8"])
@pytest.mark.parametrize("heads", GROUPS, ids=["g2", "g3"])
@pytest.mark.parametrize("grid", ["8-wave", "4-wave"])
def test_pool_groups(cache, heads, grid):
    hq, hkv = heads
    w = PoolWorkload(name="pg", seed=71 + hq, batch=2, num_q_heads=hq, num_kv_heads=hkv,
                     head_dim=128, dtype="bf16", block_size=64, logical_blocks=100, pool_slots=30,
                     rope_base=10000.0, scale=0.5, decode_steps=2,
                     cache="i8" if cache == "i8" else "")
    st = _poisoned_state(w)
    if grid == "4-wave":
        _widen(st, 4096)
    _check(st, pool_expected)


@pytest.mark.parametrize("cache", ["bf16", "i8"])
@pytest.mark.parametrize("heads", GROUPS, ids=["g2", "g3"])
@pytest.mark.parametrize("grid", ["8-wave", "4-wave"])
def test_paged_groups(cache, heads, grid):
    hq, hkv = heads
    w = PagedWorkload(name="pq", seed=75 + hq, batch=4, num_q_heads=hq, num_kv_heads=hkv,
                      head_dim=128, dtype="bf16", block_size=16, len_range=(100, 3000),
                      shared_prefix=64, scale=0.5, decode_steps=2,
                      cache="i8" if cache == "i8" else "")
    st = _poisoned_state(w)
    if grid == "4-wave":
        _widen(st, 8192)
    _check(st, paged_expected)
