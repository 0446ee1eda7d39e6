"""The shared-prefix pass of the paged decode ([share] §3.2: sequences whose
block tables start with the same physical blocks), checked exactly.

The pass finds, per call, the leading blocks every sequence shares with the
longest one, attends them once per kv head for all sharers, and leaves each
sequence's other rows to the pool kernel.  A row attended twice, or by
neither, or a shared block used for a sequence that does not name it, would
change the output; the digit probe makes that exact: K = 0 gives every row
the same weight, V rows carry (position digits, tag, kv head, 1), so out is
the mean of the probe rows over the resident set and lse = ln |set|.  Shared
blocks are tagged 100, private ones with their sequence.

Cases: sharing of different depths, a sequence shorter than its shared
blocks, the reference ending inside its last shared block, a validity hole
inside the shared region, an out-of-range id, a second group that shares
among itself but not with the longest sequence (not found: all private),
more than 128 query columns (two column blocks), every GQA group, a shared
region longer than the scanned maximum, batches of 2 .. 32, 33 .. 64 and
above 64 sequences (the table entries loaded ahead differ), and random data
against the float64 oracle.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import attend_heads

pytestmark = pytest.mark.gpu

NDIG = 6
SHARED_TAG = 100


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _digits(pos, tag, head):
    pos = np.asarray(pos, dtype=np.int64)
    v = np.zeros((pos.size, NDIG), dtype=np.float64)
    v[:, 0] = pos & 0xFF
    v[:, 1] = (pos >> 8) & 0xFF
    v[:, 2] = pos >> 16
    v[:, 3] = tag
    v[:, 4] = head
    v[:, 5] = 1.0
    return v


def _layout(lens, shared_depth, bs, seed, extra_phys=3):
    """Block tables: sequence b names shared blocks 0 .. shared_depth[b]-1
    (the same physical ids for everyone), then private blocks.  Returns
    (table [B, maxb], nphys, per physical block (first position, tag))."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    nblocks = [-(-n // bs) for n in lens]
    depth = [min(d, nb) for d, nb in zip(shared_depth, nblocks)]
    n_shared = max(depth) if depth else 0
    n_priv = sum(nb - d for nb, d in zip(nblocks, depth))
    nphys = n_shared + n_priv + extra_phys
    perm = rng.permutation(nphys)
    maxb = max(nblocks) + 2
    table = np.full((B, maxb), -1, dtype=np.int32)
    pos0 = np.full(nphys, -1, dtype=np.int64)
    tag = np.full(nphys, -1, dtype=np.int64)
    nxt = n_shared
    for b in range(B):
        for j in range(nblocks[b]):
            if j < depth[b]:
                phys = perm[j]
                tag[phys] = SHARED_TAG
            else:
                phys = perm[nxt]
                nxt += 1
                tag[phys] = b
            table[b, j] = phys
            pos0[phys] = j * bs
    return table, nphys, pos0, tag


def _run(table, nphys, pos0, tag, lens, bs, hq, hkv, valid=None, q=None, kv=None):
    from decode_attention_fixed_amd import binding as B
    d = 128
    batch, maxb = table.shape
    if kv is None:
        k = torch.zeros((nphys, hkv, bs, d), dtype=torch.bfloat16)
        v = torch.full((nphys, hkv, bs, d), float("nan"), dtype=torch.bfloat16)
        for ph in range(nphys):
            if pos0[ph] < 0:
                continue
            pos = pos0[ph] + np.arange(bs)
            for h in range(hkv):
                v[ph, h] = 0
                v[ph, h, :, :NDIG] = torch.from_numpy(_digits(pos, tag[ph], h)).to(torch.bfloat16)
        k, v = k.cuda(), v.cuda()
    else:
        k, v = kv
    if q is None:
        q = (torch.randn(batch, hq, d) * 0.5).to(torch.bfloat16)
    desc = B.make_paged_desc(batch, hq, hkv, d, bs, maxb, nphys, "bf16")
    ws = B.new_workspace(batch, hq, hkv, d, maxb * bs)
    ws.fill_(0x7F)  # the workspace needs no initialisation
    out = torch.empty(batch, hq, d, device="cuda")
    lse = torch.empty(batch, hq, device="cuda")
    B.decode_attn_paged(desc, q.cuda(), k, v, torch.from_numpy(table).cuda(),
                        torch.tensor(lens, dtype=torch.int32, device="cuda"),
                        torch.from_numpy(valid).cuda() if valid is not None else None,
                        out, ws, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check(out, lse, table, nphys, pos0, tag, lens, bs, hq, hkv, valid=None):
    g = hq // hkv
    for b, n in enumerate(lens):
        keep = []
        for i in range(n):
            j = i // bs
            ph = int(table[b, j])
            if ph < 0 or ph >= nphys or (valid is not None and not valid[b, j]):
                continue
            keep.append(i)
        keep = np.asarray(keep, dtype=np.int64)
        for h in range(hq):
            if keep.size == 0:
                assert np.all(out[b, h] == 0) and np.isneginf(lse[b, h]), (b, h)
                continue
            tags = np.array([tag[table[b, i // bs]] for i in keep])
            want = _digits(keep, tags, h // g).mean(axis=0)
            assert np.allclose(out[b, h, :NDIG], want, rtol=1e-5, atol=1e-5), (b, h, out[b, h, :NDIG], want)
            assert np.all(out[b, h, NDIG:] == 0), (b, h)
            assert abs(float(lse[b, h]) - math.log(keep.size)) <= 1e-5, (b, h, lse[b, h], keep.size)


@pytest.mark.parametrize("case", [
    # lens, shared depth (blocks), bs, hq, hkv
    dict(lens=[3000, 2500, 2200, 900], depth=[100, 100, 60, 100], bs=16, hq=8, hkv=2),
    dict(lens=[1000, 1000, 1000], depth=[63, 63, 63], bs=16, hq=4, hkv=4),         # all identical
    dict(lens=[990, 1500, 1200], depth=[62, 62, 62], bs=16, hq=6, hkv=2),          # short sharer
    dict(lens=[1010, 800, 700], depth=[64, 64, 64], bs=16, hq=16, hkv=2),          # ref ends mid-block
    dict(lens=[4000, 4100, 300, 3000], depth=[0, 40, 0, 40], bs=64, hq=24, hkv=4),  # g = 6, bs 64
    dict(lens=[5000] + [1500] * 39, depth=[70] * 40, bs=16, hq=8, hkv=2),          # 160 columns
    dict(lens=[800, 600], depth=[3, 3], bs=256, hq=2, hkv=1),                      # bs 256, g 2
    dict(lens=[3000, 2000, 2000], depth=[0, 0, 0], bs=16, hq=8, hkv=2),            # nothing shared
    dict(lens=[2000] + [1500] * 47, depth=[90] * 48, bs=16, hq=4, hkv=2),          # 48 sequences
    dict(lens=[900] + [500] * 99, depth=[40] * 100, bs=16, hq=4, hkv=2),           # 100 sequences
    dict(lens=[900] + [600] * 99, depth=[5, 30] * 50, bs=32, hq=4, hkv=4),         # mixed depths
])
def test_digit_probe_sharing(case):
    lens, bs, hq, hkv = case["lens"], case["bs"], case["hq"], case["hkv"]
    table, nphys, pos0, tag = _layout(lens, case["depth"], bs, seed=len(lens) + bs)
    out, lse = _run(table, nphys, pos0, tag, lens, bs, hq, hkv)
    _check(out, lse, table, nphys, pos0, tag, lens, bs, hq, hkv)


def test_second_group_not_sharing_with_the_longest():
    """Sequences 1 and 2 share blocks among themselves, not with the longest
    (sequence 0): nothing is found to share, every row is attended privately."""
    bs = 16
    lens = [3000, 1200, 1100]
    table, nphys, pos0, tag = _layout(lens, [0, 50, 50], bs, seed=5)
    out, lse = _run(table, nphys, pos0, tag, lens, bs, 8, 2)
    _check(out, lse, table, nphys, pos0, tag, lens, bs, 8, 2)


def test_validity_hole_and_bad_id_in_shared_region():
    bs = 16
    lens = [2000, 1900, 1800, 1700]
    table, nphys, pos0, tag = _layout(lens, [80, 80, 80, 80], bs, seed=6)
    valid = np.ones(table.shape, dtype=np.uint8)
    valid[1, 30] = 0          # a shared entry absent for sequence 1 only
    valid[0, 70] = 0          # and one absent for the reference
    table[2, 10] = nphys + 5  # an out-of-range id inside sequence 2's shared run
    out, lse = _run(table, nphys, pos0, tag, lens, bs, 8, 2, valid=valid)
    _check(out, lse, table, nphys, pos0, tag, lens, bs, 8, 2, valid=valid)


def test_shared_region_beyond_the_scanned_maximum():
    """A prefix longer than the 16384 rows the pass scans: the first 16384
    rows are shared, the rest attended privately."""
    bs = 16
    lens = [20000, 19000, 18500]
    table, nphys, pos0, tag = _layout(lens, [1150, 1150, 1150], bs, seed=7)
    out, lse = _run(table, nphys, pos0, tag, lens, bs, 8, 8)
    _check(out, lse, table, nphys, pos0, tag, lens, bs, 8, 8)


@pytest.mark.parametrize("hq,hkv", [(32, 8), (12, 4), (8, 8)])
def test_random_rows_against_the_oracle(hq, hkv):
    """Random K / V / q: the output with the shared pass equals attention over
    each sequence's rows in float64 within the bf16 bar."""
    bs, d = 16, 128
    lens = [2500, 3100, 1900, 2400, 700]
    table, nphys, pos0, tag = _layout(lens, [125] * 5, bs, seed=hq + hkv)
    g = torch.Generator().manual_seed(hq)
    k = (torch.randn(nphys, hkv, bs, d, generator=g) * 0.5).to(torch.bfloat16)
    v = (torch.randn(nphys, hkv, bs, d, generator=g) * 0.5).to(torch.bfloat16)
    q = (torch.randn(len(lens), hq, d, generator=g) * 0.5).to(torch.bfloat16)
    out, lse = _run(table, nphys, pos0, tag, lens, bs, hq, hkv, q=q, kv=(k.cuda(), v.cuda()))
    for b, n in enumerate(lens):
        rows = np.arange(n)
        ph = table[b, rows // bs]
        kk = k[torch.from_numpy(ph.astype(np.int64)), :, torch.from_numpy(rows % bs)].double().numpy()
        vv = v[torch.from_numpy(ph.astype(np.int64)), :, torch.from_numpy(rows % bs)].double().numpy()
        want, want_lse = attend_heads(q[b].double().numpy(), kk, vv)
        assert np.abs(out[b] - want).max() <= 2e-3, b
        assert np.abs(lse[b] - want_lse).max() <= 1e-3, b
