"""decode_attn_paged_noalloc (partial results in the library's fixed
per-device array, no workspace argument, nothing allocated) against
decode_attn_paged with a workspace of the caller's, through the C ABI.

Two calls in a row on one device, the second with a smaller input (the
array keeps the first call's contents): each must give out and lse bit for
bit equal to the workspace entry point's on the same inputs, and both agree
with the float64 oracle within 2e-3.  Covered: the paged layout with a shared
prefix on both pool grids (the 512 four-wave grid is chosen from the pool's
capacity), and a pool with a validity mask (NaN in every absent block).
"""

import numpy as np
import pytest
import torch

from oracle.decode import paged_expected, pool_expected
from synth import PagedWorkload, PoolWorkload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _state(w):
    from tests.device_data import PagedState
    st = PagedState(w)
    st.k_pool.fill_(float("nan"))
    st.v_pool.fill_(float("nan"))
    st.fill()
    return st


def _widen(st, max_blocks):
    """The same pool behind a block table of max_blocks columns (extra entries
    absent): B * Hkv * max_blocks * bs >= 2^20 capacity rows select the
    512-workgroup four-wave grid."""
    from decode_attention_fixed_amd import binding as B
    w = st.w
    n = st.block_table.shape[1]
    bt = torch.full((w.batch, max_blocks), -1, dtype=torch.int32, device="cuda")
    bt[:, :n] = st.block_table
    st.block_table = bt
    assert w.batch * w.num_kv_heads * max_blocks * w.block_size >= 512 * 2048
    st.desc = B.make_paged_desc(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                max_blocks, st.num_phys, w.dtype)
    st.workspace = B.new_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                   max_blocks * w.block_size)


def _both(st, step):
    """(noalloc out, lse), (workspace out, lse) for the same query."""
    from decode_attention_fixed_amd import binding as B
    q = st.step_query(step)
    out_n = torch.empty_like(st.out)
    lse_n = torch.empty_like(st.lse)
    B.decode_attn_paged_noalloc(st.desc, q, st.k_pool, st.v_pool, st.block_table, st.seq_lens,
                                st.block_valid, out_n, lse_n)
    B.decode_attn_paged(st.desc, q, st.k_pool, st.v_pool, st.block_table, st.seq_lens,
                        st.block_valid, st.out, st.workspace, st.lse)
    torch.cuda.synchronize()
    return (out_n, lse_n), (st.out, st.lse)


def _check(st, expected_fn, step=0):
    (out_n, lse_n), (out_w, lse_w) = _both(st, step)
    assert torch.equal(out_n, out_w)
    assert torch.equal(lse_n, lse_w)
    out = out_n.cpu().numpy()
    lse = lse_n.cpu().numpy()
    for b in range(st.w.batch):
        want, want_lse = expected_fn(st.w, b, step)
        assert float(np.abs(out[b] - want).max()) <= 2e-3, b
        assert float(np.abs(lse[b] - want_lse).max()) <= 1e-3, b


def test_noalloc_paged_two_calls_second_smaller():
    big = PagedWorkload(name="na1", seed=91, batch=8, num_q_heads=16, num_kv_heads=4,
                        head_dim=128, dtype="bf16", block_size=16, len_range=(2000, 12000),
                        shared_prefix=160, scale=0.5, decode_steps=1)
    small = PagedWorkload(name="na2", seed=92, batch=3, num_q_heads=16, num_kv_heads=4,
                          head_dim=128, dtype="bf16", block_size=16, len_range=(50, 700),
                          shared_prefix=32, scale=0.5, decode_steps=1)
    a, b = _state(big), _state(small)
    _widen(a, 8192)
    _check(a, paged_expected)   # the 512 four-wave grid
    _check(b, paged_expected)   # a small pool: the eight-wave grid, on the same array


def test_noalloc_pool_with_validity_mask():
    w = PoolWorkload(name="na3", seed=93, batch=2, num_q_heads=6, num_kv_heads=1, head_dim=128,
                     dtype="bf16", block_size=64, logical_blocks=80, pool_slots=24,
                     rope_base=10000.0, scale=0.5, decode_steps=2)
    st = _state(w)
    _check(st, pool_expected, 0)
    _check(st, pool_expected, 1)

