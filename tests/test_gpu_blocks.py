"""GPU parity of the block manager and the paged append ([share] §3.2 prefix
sharing, §5.1 allocate / share_prefix / append_token with copy-on-write, §6.1
release by reference count) against the oracle's BlockManager.

After every operation the library's block table, lengths and reference
counts equal the oracle's bit for bit (both take the lowest free block).  The
pool is poisoned with NaN first; reading every live sequence's rows back
through the device table gives exactly its own history (isolation: no write
into a shared block reaches another sequence), and the decode over the pool
matches attention over each sequence's history.
"""

import copy
import random

import numpy as np
import pytest
import torch

from oracle.attention import attend_heads
from oracle.blocks import BlockManager, BlocksExhausted
from oracle.decode import paged_append_expected
from oracle.rope import rope
from oracle.rounding import round_store
from synth import TENSOR_K, TENSOR_V, workload
from synth.draws import draw_rows

pytestmark = pytest.mark.gpu

SEED = 71
HKV, HQ, D = 2, 8, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _tag_rows(tensor, tags, dtype="bf16"):
    """Raw rows of tokens tagged (origin stream, position)."""
    out = np.empty((len(tags), HKV, D), dtype=np.float32)
    for i, (origin, pos) in enumerate(tags):
        out[i] = draw_rows(SEED, tensor, origin, [pos], HKV, D, 0.5, dtype)[0]
    return out


def _dev(a, dtype="bf16"):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)


def _state(num_blocks, bs, max_seqs, max_blocks, dtype="bf16"):
    from tests.device_data import BlockPoolState
    st = BlockPoolState(num_blocks, bs, max_seqs, max_blocks, HQ, HKV, D, dtype)
    st.k_pool.fill_(float("nan"))
    st.v_pool.fill_(float("nan"))
    return st


def _compare_state(st, m):
    s = st.state()
    for seq in range(st.max_seqs):
        want = list(m.tables.get(seq, []))
        want += [-1] * (st.max_blocks - len(want))
        assert s["table"][seq] == want, seq
        assert s["lens"][seq] == m.lens.get(seq, 0), seq
    assert s["refs"] == m.ref
    assert s["free"] == m.free_count()
    assert st.seq_lens.cpu().tolist() == s["lens"]
    table = st.block_table.cpu().numpy()
    for seq in range(st.max_seqs):  # live entries of the device table
        n = -(-s["lens"][seq] // st.block_size)
        assert table[seq, :n].tolist() == s["table"][seq][:n], seq


def _readback(st, m, hist, rotate):
    """Every live sequence reads exactly its own history through the device table."""
    kp, vp = st.k_pool.float().cpu().numpy(), st.v_pool.float().cpu().numpy()
    table = st.block_table.cpu().numpy()
    bs = st.block_size
    for seq, tags in hist.items():
        if not tags:
            continue
        idx = np.arange(len(tags))
        blk = table[seq, idx // bs]
        r = idx % bs
        got_k = kp[blk, :, r, :]
        got_v = vp[blk, :, r, :]
        want_v = _tag_rows(TENSOR_V, tags)
        want_k = _tag_rows(TENSOR_K, tags)
        assert np.array_equal(got_v, want_v), seq
        if rotate:
            pos = np.asarray([p for _, p in tags])
            want_k = round_store(rope(want_k, pos[:, None], 10000.0), "bf16")
            ulp = np.abs(want_k) * 2.0 ** -7 + 1e-30
            assert np.all(np.abs(got_k - want_k) <= ulp), seq
        else:
            assert np.array_equal(got_k, want_k), seq


def _decode_check(st, hist, rotate, tol=2e-3):
    q = np.stack([draw_rows(SEED, 0, 900 + s, [0], HQ, D, 0.5, "bf16")[0]
                  for s in range(st.max_seqs)])
    st.decode(_dev(q))
    torch.cuda.synchronize()
    out = st.out.cpu().numpy()
    for seq in range(st.max_seqs):
        tags = hist.get(seq, [])
        if not tags:
            assert np.all(out[seq] == 0), seq  # empty sequence: out = 0
            continue
        k = _tag_rows(TENSOR_K, tags).astype(np.float64)
        if rotate:
            pos = np.asarray([p for _, p in tags])
            k = round_store(rope(k, pos[:, None], 10000.0), "bf16")
        want, _ = attend_heads(q[seq].astype(np.float64), k,
                               _tag_rows(TENSOR_V, tags).astype(np.float64))
        assert float(np.abs(out[seq] - want).max()) <= tol, seq


@pytest.mark.parametrize("bs,rotate,seed", [(16, False, 0), (16, True, 1), (64, False, 2)])
def test_blocks_random_interleaving(bs, rotate, seed):
    """Random allocate / share / append / free with one to several tokens per
    call, checked against the oracle after every operation."""
    from decode_attention_fixed_amd.binding import SwaError
    rng = random.Random(seed)
    max_seqs, max_blocks, num_blocks = 6, 12, 40
    st = _state(num_blocks, bs, max_seqs, max_blocks)
    m = BlockManager(num_blocks, bs)
    hist = {}   # seq -> [(origin stream, position)] of its tokens
    nxt = [100]
    try:
        for it in range(60):
            op = rng.random()
            live = [s for s in range(max_seqs) if hist.get(s)]
            empty = [s for s in range(max_seqs) if not hist.get(s)]
            if op < 0.2 and empty and live:
                src, dst = rng.choice(live), rng.choice(empty)
                n = rng.randrange(1, len(hist[src]) + 1)
                st.share(src, dst, n)
                m.share_prefix(src, dst, n)
                hist[dst] = hist[src][:n]
            elif op < 0.3 and live:
                s = rng.choice(live)
                st.free(s)
                m.free(s)
                hist[s] = []
            else:
                seqs = rng.sample(range(max_seqs), rng.randrange(1, 4))
                t = rng.choice([1, 1, 2, 5, bs + 3])
                need_ok = all(m.lens.get(s, 0) + t <= max_blocks * bs for s in seqs)
                if not need_ok:
                    continue
                tags = []
                for s in seqs:
                    origin = nxt[0]
                    nxt[0] += 1
                    base = m.lens.get(s, 0)
                    tags.append([(origin, base + j) for j in range(t)])
                k = _tag_rows(TENSOR_K, [x for g in tags for x in g]).reshape(len(seqs), t, HKV, D)
                v = _tag_rows(TENSOR_V, [x for g in tags for x in g]).reshape(len(seqs), t, HKV, D)
                saved = copy.deepcopy(m)
                try:
                    for s, g in zip(seqs, tags):
                        for x in g:
                            m.append_token(s, x)
                except BlocksExhausted:
                    # the oracle ran out of blocks: the library must refuse
                    # the whole call and change nothing
                    m = saved
                    before = st.state()
                    with pytest.raises(SwaError):
                        st.append(seqs, _dev(k), _dev(v), rotate)
                    assert st.state() == before
                    continue
                st.append(seqs, _dev(k), _dev(v), rotate)
                for s, g in zip(seqs, tags):
                    hist[s] = hist.get(s, []) + g
            torch.cuda.synchronize()
            _compare_state(st, m)
            if it % 15 == 14:
                _readback(st, m, hist, rotate)
                _decode_check(st, hist, rotate)
        _readback(st, m, hist, rotate)
        _decode_check(st, hist, rotate)
    finally:
        st.close()


def test_copy_on_write_isolation():
    """A shared, partly filled block is copied before a sharer writes into it;
    the other sharer's rows are untouched, bit for bit."""
    st = _state(8, 16, 3, 4)
    m = BlockManager(8, 16)
    try:
        a = [(200, p) for p in range(6)]
        st.append([0], _dev(_tag_rows(TENSOR_K, a))[None], _dev(_tag_rows(TENSOR_V, a))[None])
        for x in a:
            m.append_token(0, x)
        st.share(0, 1, 6)
        m.share_prefix(0, 1, 6)
        b_tok = [(201, 6)]
        st.append([1], _dev(_tag_rows(TENSOR_K, b_tok))[None], _dev(_tag_rows(TENSOR_V, b_tok))[None])
        _, copied = m.append_token(1, b_tok[0])
        assert copied == (0, 1, 6)
        a_tok = [(202, 6)]
        st.append([0], _dev(_tag_rows(TENSOR_K, a_tok))[None], _dev(_tag_rows(TENSOR_V, a_tok))[None])
        _, copied = m.append_token(0, a_tok[0])
        assert copied is None
        torch.cuda.synchronize()
        _compare_state(st, m)
        hist = {0: a + a_tok, 1: a + b_tok}
        _readback(st, m, hist, False)
        _decode_check(st, hist, False)
    finally:
        st.close()


def test_exhaustion_refused_and_unchanged():
    from decode_attention_fixed_amd.binding import SWA_ERR_INVALID_ARG, SwaError
    st = _state(3, 16, 2, 4)
    try:
        tags = [(300, p) for p in range(40)]
        st.append([0], _dev(_tag_rows(TENSOR_K, tags))[None], _dev(_tag_rows(TENSOR_V, tags))[None])
        before = st.state()
        more = [(301, p) for p in range(20)]
        with pytest.raises(SwaError) as e:   # needs 2 blocks, 0 free
            st.append([1], _dev(_tag_rows(TENSOR_K, more))[None],
                      _dev(_tag_rows(TENSOR_V, more))[None])
        assert e.value.code == SWA_ERR_INVALID_ARG
        assert st.state() == before
    finally:
        st.close()


def test_paged_append_full_size():
    """The paged workload (B = 32, lengths 1K-32K, a 2000-token prefix shared
    by reference) built through the manager, then decode steps that each
    append one token per sequence; sampled steps against the oracle."""
    from tests.device_data import build_paged_append, to_device
    w = workload("paged-append")
    steps = 6
    st = build_paged_append(w)
    try:
        s = st.state()
        assert s["lens"][:w.batch] == [int(x) for x in w.lengths] and s["lens"][w.batch] == 0
        assert int(w.lengths[18]) < w.shared_prefix and int(w.lengths[22]) < w.shared_prefix
        # every full sequence references all 125 prefix blocks; the two short
        # ones the blocks their length reaches (the holder was freed)
        want_refs = [sum(1 for n in w.lengths if -(-int(n) // w.block_size) > j)
                     for j in range(w.shared_blocks)]
        assert s["refs"][:w.shared_blocks] == want_refs
        for step in range(steps):
            pos = w.lengths + step
            k = np.stack([w.rows(TENSOR_K, b, [pos[b]]) for b in range(w.batch)])
            v = np.stack([w.rows(TENSOR_V, b, [pos[b]]) for b in range(w.batch)])
            st.append(list(range(w.batch)), to_device(k, w.dtype), to_device(v, w.dtype))
            q = np.stack([w.query(b, step) for b in range(w.batch)] +
                         [np.zeros((w.num_q_heads, w.head_dim), np.float32)])
            st.decode(to_device(q, w.dtype))
            torch.cuda.synchronize()
            if step in (0, steps - 1):
                out = st.out.cpu().numpy()
                # sequences 18 and 22 are shorter than the prefix: their first
                # append copies the shared, partly filled block (copy-on-write)
                for b in (0, 7, 18, 22, 31):
                    want, _ = paged_append_expected(w, b, step)
                    assert float(np.abs(out[b] - want).max()) <= 2e-3, (step, b)
                assert np.all(out[w.batch] == 0)
    finally:
        st.close()
