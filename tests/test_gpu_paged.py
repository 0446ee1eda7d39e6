"""GPU parity of the paged-pool decode path against the oracle, plus probes
that pin the block mapping exactly.

Mapping probes (block table + validity mask):
  digits      K = 0 makes every weight equal, and V rows carry their logical
              position as base-256 digits (exact in bf16) plus the sequence
              index: the output must be the exact mean over the resident set,
              so a missing, extra or misplaced token shows up.
  one-hot     one token per sequence gets K = c * q with a score 100 above the
              rest: the output must be exactly that token's V.
  permutation the same logical content placed through an identity and through
              a shuffled block table must give bitwise-identical outputs.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import attend_heads
from oracle.decode import paged_expected, pool_expected, pool_rows
from synth import PagedWorkload, PoolWorkload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _paged(**kw):
    base = dict(name="p", seed=31, batch=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                dtype="bf16", block_size=16, len_range=(100, 1000), shared_prefix=64, scale=0.5,
                decode_steps=3)
    base.update(kw)
    return PagedWorkload(**base)


def _pool(**kw):
    base = dict(name="l", seed=32, batch=2, num_q_heads=6, num_kv_heads=1, head_dim=128,
                dtype="bf16", block_size=64, logical_blocks=64, pool_slots=20, rope_base=10000.0,
                scale=0.5, decode_steps=3)
    base.update(kw)
    return PoolWorkload(**base)


def _state(w, poison=True):
    from tests.device_data import PagedState
    st = PagedState(w)
    if poison:  # rows nobody writes hold NaN: they must never reach the arithmetic
        st.k_pool.fill_(float("nan"))
        st.v_pool.fill_(float("nan"))
    st.fill()
    return st


def _check_steps(st, expected_fn, tol=2e-3):
    w = st.w
    for step in range(w.decode_steps):
        q = st.step_query(step)
        st.step(q)
        torch.cuda.synchronize()
        out = st.out.float().cpu().numpy()
        lse = st.lse.cpu().numpy()
        for b in range(w.batch):
            want, want_lse = expected_fn(w, b, step)
            err = np.abs(out[b] - want).max()
            assert err <= tol, (b, step, err)
            assert np.abs(lse[b] - want_lse).max() <= 1e-2


@pytest.mark.parametrize("kw", [
    dict(),
    dict(num_q_heads=2, num_kv_heads=2, len_range=(1, 70), shared_prefix=32),   # g=1, tiny
    dict(num_q_heads=12, num_kv_heads=2, block_size=32, shared_prefix=96),      # g=6, bs=32
    dict(head_dim=64, num_q_heads=8, num_kv_heads=1, len_range=(500, 3000)),    # g=8, d=64
    dict(dtype="f32", num_q_heads=4, num_kv_heads=4, len_range=(10, 400)),
])
def test_paged_variants(kw):
    w = _paged(**kw)
    st = _state(w)
    _check_steps(st, paged_expected, 1e-5 if w.dtype == "f32" else 2e-3)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(batch=3, num_q_heads=8, num_kv_heads=2, logical_blocks=100, pool_slots=30),
    dict(head_dim=64, num_q_heads=4, num_kv_heads=4, block_size=16, logical_blocks=200,
         pool_slots=50),
])
def test_pool_variants(kw):
    """Fixed pool with a validity mask; K rows rotated at their absolute
    position by kv_write_paged, checked row by row against the oracle."""
    w = _pool(**kw)
    st = _state(w)
    torch.cuda.synchronize()
    bs = w.block_size
    for b in range(w.batch):
        pos, k_want, v_want = pool_rows(w, b)
        slots = np.nonzero(w.slot_blocks[b] >= 0)[0]
        phys = w.block_table[b][slots]
        k_got = st.k_pool[torch.from_numpy(phys.astype(np.int64)).cuda()]  # [n, Hkv, bs, d]
        k_got = k_got.permute(0, 2, 1, 3).reshape(-1, w.num_kv_heads, w.head_dim)
        v_got = st.v_pool[torch.from_numpy(phys.astype(np.int64)).cuda()]
        v_got = v_got.permute(0, 2, 1, 3).reshape(-1, w.num_kv_heads, w.head_dim)
        assert np.array_equal(v_got.float().cpu().numpy(), v_want.astype(np.float32))
        kb = (k_got.float().cpu().numpy().view(np.int32) >> 16).astype(np.int64)
        wb = (k_want.astype(np.float32).view(np.int32) >> 16).astype(np.int64)
        assert np.abs(kb - wb).max() <= 1 and (kb != wb).mean() < 1e-4
        assert len(pos) == len(slots) * bs
    _check_steps(st, pool_expected)


# ---------------------------------------------------------------------------
# mapping probes: the pool is built directly with torch (layout
# [Nphys, Hkv, bs, d]), independently of kv_write_paged
# ---------------------------------------------------------------------------

def _digits(pos: np.ndarray, b: int, d: int) -> np.ndarray:
    v = np.zeros((len(pos), d), dtype=np.float32)
    v[:, 0] = pos & 0xFF
    v[:, 1] = (pos >> 8) & 0xFF
    v[:, 2] = pos >> 16
    v[:, 3] = b
    v[:, 4] = 1.0
    return v


def _probe_pool(batch, hkv, d, bs, tables, resident_tokens, nphys, maxb):
    """Pool whose V rows carry (position digits, b); K = 0; returns tensors."""
    k = torch.zeros((nphys, hkv, bs, d), dtype=torch.bfloat16)
    v = torch.full((nphys, hkv, bs, d), float("nan"), dtype=torch.bfloat16)
    for b in range(batch):
        for blk_idx, phys in enumerate(tables[b]):
            if phys < 0 or phys >= nphys:
                continue
            pos = np.arange(blk_idx * bs, (blk_idx + 1) * bs)
            for h in range(hkv):
                v[phys, h] = torch.from_numpy(_digits(pos, b, d)).to(torch.bfloat16)
    bt = np.full((batch, maxb), -1, dtype=np.int32)
    for b in range(batch):
        bt[b, :len(tables[b])] = tables[b]
    return k.cuda(), v.cuda(), torch.from_numpy(bt).cuda()


def _run_paged(batch, hq, hkv, d, bs, maxb, nphys, k, v, bt, lens, valid=None, q=None):
    from decode_attention_fixed_amd import binding as B
    desc = B.make_paged_desc(batch, hq, hkv, d, bs, maxb, nphys, "bf16")
    ws = B.new_workspace(batch, hq, hkv, d, maxb * bs)
    if q is None:
        q = torch.randn(batch, hq, d, device="cuda").to(torch.bfloat16)
    out = torch.empty(batch, hq, d, device="cuda")
    lse = torch.empty(batch, hq, device="cuda")
    B.decode_attn_paged(desc, q, k, v, bt, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                        valid, out, ws, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _mean_digits(resident: np.ndarray, b: int, d: int) -> np.ndarray:
    return _digits(resident, b, d).astype(np.float64).mean(axis=0)


@pytest.mark.parametrize("bs,lens", [(16, [1, 17, 250, 1000]), (64, [64, 65, 3000, 1])])
def test_probe_position_digits_paged(bs, lens):
    rng = np.random.default_rng(7)
    batch, hkv, hq, d = len(lens), 2, 8, 128
    nblocks = [-(-n // bs) for n in lens]
    maxb = max(nblocks) + 3
    nphys = sum(nblocks) + 5
    perm = rng.permutation(nphys)
    tables, o = [], 0
    for nb in nblocks:
        tables.append(perm[o:o + nb].astype(np.int32))
        o += nb
    k, v, bt = _probe_pool(batch, hkv, d, bs, tables, None, nphys, maxb)
    out, lse = _run_paged(batch, hq, hkv, d, bs, maxb, nphys, k, v, bt, lens)
    for b in range(batch):
        want = _mean_digits(np.arange(lens[b]), b, d)
        assert np.allclose(out[b][:, :5], want[:5], rtol=1e-5, atol=1e-5), b
        assert np.allclose(lse[b], math.log(lens[b]), rtol=1e-5)


@pytest.mark.parametrize("lens", [[1, 17, 9000, 16000], [1, 17, 250, 1000]])
def test_probe_position_digits_wide_grid_sparse(lens):
    """A block table of 8192 entries per sequence gives the pool 1M rows of
    capacity, so the call takes the 512 x 4-wave grid, whose shares are
    weighted by workgroup (17/16, 15/16); the sequences are short, so the
    resident granules number between 512 and 1024 (every share holds some,
    uneven ones) or far fewer (most shares empty): the merge then checks
    each share for rows instead of taking them all as present."""
    rng = np.random.default_rng(11)
    batch, hkv, hq, d, bs = len(lens), 2, 8, 128, 16
    maxb = 8192
    assert batch * hkv * maxb * bs >= 512 * 2048  # the 4-wave grid
    nblocks = [-(-n // bs) for n in lens]
    nphys = sum(nblocks) + 5
    perm = rng.permutation(nphys)
    tables, o = [], 0
    for nb in nblocks:
        tables.append(perm[o:o + nb].astype(np.int32))
        o += nb
    k, v, bt = _probe_pool(batch, hkv, d, bs, tables, None, nphys, maxb)
    out, lse = _run_paged(batch, hq, hkv, d, bs, maxb, nphys, k, v, bt, lens)
    for b in range(batch):
        want = _mean_digits(np.arange(lens[b]), b, d)
        assert np.allclose(out[b][:, :5], want[:5], rtol=1e-5, atol=1e-5), b
        assert np.allclose(lse[b], math.log(lens[b]), rtol=1e-5)


def test_probe_position_digits_validity_mask():
    """Pool slots flagged absent (and slots whose id is out of range) drop out
    of the set exactly."""
    rng = np.random.default_rng(8)
    batch, hkv, hq, d, bs, nb = 3, 1, 6, 128, 64, 40
    nphys = batch * nb
    perm = rng.permutation(nphys).astype(np.int32)
    tables = [perm[b * nb:(b + 1) * nb].copy() for b in range(batch)]
    tables[2][5] = nphys + 10       # out of range: absent
    tables[2][6] = -7               # negative: absent
    valid = (rng.random((batch, nb)) < 0.3).astype(np.uint8)
    valid[1, :] = 0                 # nothing resident at all
    k, v, bt = _probe_pool(batch, hkv, d, bs, tables, None, nphys, nb)
    out, lse = _run_paged(batch, hq, hkv, d, bs, nb, nphys, k, v, bt, [nb * bs] * batch,
                          torch.from_numpy(valid).cuda())
    for b in range(batch):
        keep = [j for j in range(nb) if valid[b, j] and 0 <= tables[b][j] < nphys]
        if not keep:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        resident = np.concatenate([np.arange(j * bs, (j + 1) * bs) for j in keep])
        assert np.allclose(out[b][:, :5], _mean_digits(resident, b, d)[:5], rtol=1e-5, atol=1e-5)


def test_probe_one_hot():
    """A token whose score beats all others by >= 100 returns exactly its V."""
    rng = np.random.default_rng(9)
    batch, hkv, hq, d, bs, nb = 2, 2, 8, 128, 16, 30
    g = hq // hkv
    nphys = batch * nb
    tables = [rng.permutation(nphys)[:nb].astype(np.int32) for _ in range(batch)]
    # distinct tables per sequence
    tables[1] = np.setdiff1d(np.arange(nphys), tables[0])[:nb].astype(np.int32)
    k = torch.zeros((nphys, hkv, bs, d), dtype=torch.bfloat16)
    v = (torch.randn((nphys, hkv, bs, d)) * 0.5).to(torch.bfloat16)
    qv = (torch.randn(batch, hkv, d) * 0.5).to(torch.bfloat16)
    q = qv.repeat_interleave(g, dim=1)  # every head of a group asks the same question
    hot = {}
    for b in range(batch):
        for h in range(hkv):
            tok = int(rng.integers(0, nb * bs))
            phys = tables[b][tok // bs]
            qf = qv[b, h].float()
            c = 2 ** math.ceil(math.log2(400.0 * math.sqrt(d) / float(qf @ qf)))
            k[phys, h, tok % bs] = (qf * c).to(torch.bfloat16)
            hot[(b, h)] = v[phys, h, tok % bs].float().numpy()
    bt = torch.from_numpy(np.stack(tables)).cuda()
    out, _ = _run_paged(batch, hq, hkv, d, bs, nb, nphys, k.cuda(), v.cuda(), bt,
                        [nb * bs] * batch, q=q.cuda())
    for b in range(batch):
        for h in range(hq):
            assert np.array_equal(out[b, h], hot[(b, h // g)]), (b, h)


def test_permuted_block_table_is_bitwise_identical():
    rng = np.random.default_rng(10)
    batch, hkv, hq, d, bs, nb = 2, 2, 8, 128, 16, 70
    nphys = batch * nb
    logical_k = (torch.randn(batch, nb, hkv, bs, d) * 0.5).to(torch.bfloat16)
    logical_v = (torch.randn(batch, nb, hkv, bs, d) * 0.5).to(torch.bfloat16)
    q = (torch.randn(batch, hq, d) * 0.5).to(torch.bfloat16).cuda()
    lens = [nb * bs - 5, 333]
    outs = []
    for table in (np.arange(nphys), rng.permutation(nphys)):
        table = table.reshape(batch, nb).astype(np.int32)
        k = torch.empty((nphys, hkv, bs, d), dtype=torch.bfloat16)
        v = torch.empty((nphys, hkv, bs, d), dtype=torch.bfloat16)
        for b in range(batch):
            k[torch.from_numpy(table[b].astype(np.int64))] = logical_k[b]
            v[torch.from_numpy(table[b].astype(np.int64))] = logical_v[b]
        out, lse = _run_paged(batch, hq, hkv, d, bs, nb, nphys, k.cuda(), v.cuda(),
                              torch.from_numpy(table).cuda(), lens, q=q)
        outs.append((out, lse))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    # and both agree with the oracle over the logical rows
    for b in range(batch):
        n = lens[b]
        kk = logical_k[b].permute(0, 2, 1, 3).reshape(nb * bs, hkv, d)[:n].double().numpy()
        vv = logical_v[b].permute(0, 2, 1, 3).reshape(nb * bs, hkv, d)[:n].double().numpy()
        want, _ = attend_heads(q[b].double().cpu().numpy(), kk, vv)
        assert np.abs(outs[0][0][b] - want).max() <= 2e-3


def test_seq_len_zero_and_clamped():
    batch, hkv, hq, d, bs, nb = 3, 1, 4, 64, 16, 8
    nphys = batch * nb
    tables = [np.arange(b * nb, (b + 1) * nb, dtype=np.int32) for b in range(batch)]
    k, v, bt = _probe_pool(batch, hkv, d, bs, tables, None, nphys, nb)
    out, lse = _run_paged(batch, hq, hkv, d, bs, nb, nphys, k, v, bt, [0, 10 ** 9, -4])
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[2] == 0) and np.all(np.isneginf(lse[2]))
    assert np.allclose(out[1][:, :5], _mean_digits(np.arange(nb * bs), 1, d)[:5], rtol=1e-5)


@pytest.mark.parametrize("kw", [
    dict(batch=6, len_range=(2000, 9000), shared_prefix=160),                   # many items per unit
    dict(batch=1, num_q_heads=6, num_kv_heads=1, len_range=(40000, 40000)),     # one unit, all shares
])
def test_streams_and_graph_replay_bitwise(kw):
    """The same decode call issued on the default stream, on a second stream,
    and captured into a graph (replayed several times, with eager calls in
    between) gives the same output and lse bit for bit, and they match the
    oracle.  The second case spreads one (sequence, kv head) over every
    workgroup of the grid."""
    from decode_attention_fixed_amd import binding as B
    w = _paged(**kw)
    st = _state(w, poison=False)
    q = st.step_query(0)

    def call(out, lse):
        B.decode_attn_paged(st.desc, q, st.k_pool, st.v_pool, st.block_table, st.seq_lens,
                            st.block_valid, out, st.workspace, lse)

    out0 = torch.empty_like(st.out)
    lse0 = torch.empty_like(st.lse)
    call(out0, lse0)
    torch.cuda.synchronize()
    for b in range(w.batch):
        want, want_lse = paged_expected(w, b, 0)
        assert np.abs(out0[b].cpu().numpy() - want).max() <= 2e-3
        assert np.abs(lse0[b].cpu().numpy() - want_lse).max() <= 1e-2

    side = torch.cuda.Stream()
    out1 = torch.empty_like(out0)
    lse1 = torch.empty_like(lse0)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            call(out1, lse1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out1, out0) and torch.equal(lse1, lse0)

    out2 = torch.zeros_like(out0)
    lse2 = torch.zeros_like(lse0)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out2, lse2)
    for _ in range(3):
        out2.zero_()
        lse2.zero_()
        call(out1, lse1)  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out2, out0) and torch.equal(lse2, lse0)
        assert torch.equal(out1, out0)
