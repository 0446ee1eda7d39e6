"""The block manager and the host-pool pager under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/capi/host_managers.cpp builds blocks_api.cpp and pager_api.cpp with g++
and -fsanitize=address,undefined, their HIP calls and kernel launches done on
the host (the launches apply their kernels' effects to host buffers).  Random
traces then drive the C ABI and every state is compared with the oracles:

  blocks  allocate-on-append / share_prefix / append (several sequences per
          call, copy-on-write of shared partial blocks, refused calls) /
          free / reset, against oracle/blocks.py: tables, lengths, reference counts
          and the free count bit for bit, and every sequence read back
          through the device table (its own history, per head, K and V).
  pager   LRU requests (some refused, copies on the attention stream or a
          second one, or staged and run by the pager's decode), against
          oracle/paging.py: the block in every slot, the device validity
          bytes (= the oracle's visible set), and every valid slot's pool
          block equal to the host store's block.

Any heap misuse, leak (events included), or undefined behaviour aborts the
binary, which fails the test.
"""

import copy
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.blocks import BlockManager, BlocksExhausted
from oracle.paging import LruPool, PoolRefused

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "decode_attention_fixed_amd", "csrc", f)
       for f in ("blocks_api.cpp", "pager_api.cpp")] + [
    os.path.join(ROOT, "tests", "capi", "host_managers.cpp")]


@pytest.fixture(scope="module")
def binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("asan") / "host_managers")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{ROOT}/include",
           f"-I{ROOT}/decode_attention_fixed_amd/csrc", *SRC, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return out


def _run(binary, commands):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([binary], input="\n".join(commands) + "\n", capture_output=True,
                         text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    lines = res.stdout.splitlines()
    assert lines[-1] == "events 0", lines[-1]
    return iter(lines[:-1])


def _ints(line, name):
    head, *rest = line.split()
    assert head == name, (head, name)
    return [int(x) for x in rest]


# ---------------------------------------------------------------------------
# block manager
# ---------------------------------------------------------------------------

def _blocks_trace(seed, nb, bs, seqs, maxb, n_ops):
    """(commands, expectations): the oracle's state after each command."""
    rng = np.random.default_rng(seed)
    om = BlockManager(nb, bs)
    cmds, exp = [f"blocks {nb} {bs} {seqs} {maxb} 2 64"], [("rc", 0)]
    lens = lambda s: om.lens.get(s, 0)  # noqa: E731
    for _ in range(n_ops):
        op = rng.choice(["append", "share", "free", "reset"], p=[0.49, 0.3, 0.18, 0.03])
        if op == "append":
            k = int(rng.integers(1, seqs + 1))
            chosen = [int(s) for s in rng.choice(seqs, size=k, replace=False)]
            if rng.random() < 0.05:
                chosen.append(chosen[0])        # listed twice: refused
            t = int(rng.integers(1, bs + 5)) if rng.random() < 0.9 else int(rng.integers(1, 4 * bs))
            trial = copy.deepcopy(om)
            ok = len(set(chosen)) == len(chosen)
            try:
                for s in chosen if ok else []:
                    if lens(s) + t > maxb * bs:
                        ok = False
                        break
                    for _ in range(t):
                        trial.append_token(s)
            except BlocksExhausted:
                ok = False
            if ok:
                om = trial
            cmds.append(f"append {t} {len(chosen)} " + " ".join(map(str, chosen)))
            exp.append(("rc", 0 if ok else -1))
        elif op == "share":
            full = [s for s in range(seqs) if lens(s) > 0]
            empty = [s for s in range(seqs) if lens(s) == 0]
            if not full or not empty:
                continue
            src, dst = int(rng.choice(full)), int(rng.choice(empty))
            n = int(rng.integers(0, lens(src) + 1))
            om.share_prefix(src, dst, n)
            cmds.append(f"share {src} {dst} {n}")
            exp.append(("rc", 0))
        elif op == "free":
            s = int(rng.integers(seqs))
            om.free(s)
            cmds.append(f"free {s}")
            exp.append(("rc", 0))
        else:  # everything empty again, the device mirrors rewritten
            om = BlockManager(nb, bs)
            cmds += ["reset", "bsync"]
            exp += [("rc", 0), ("rc", 0)]
        cmds.append("bstate")
        exp.append(("bstate", copy.deepcopy(om)))
    return cmds, exp


def _check_bstate(lines, om, seqs, maxb, nb):
    table = _ints(next(lines), "table")
    lens = _ints(next(lines), "lens")
    refs = _ints(next(lines), "refs")
    free = _ints(next(lines), "free")[0]
    dlens = _ints(next(lines), "dlens")
    want_table = []
    for s in range(seqs):
        row = list(om.tables.get(s, []))
        want_table += row + [-1] * (maxb - len(row))
    assert table == want_table
    assert lens == [om.lens.get(s, 0) for s in range(seqs)]
    assert refs == om.ref and free == om.free_count()
    assert dlens == lens
    for s in range(seqs):
        got = next(lines).split()
        assert got[:2] == ["read", str(s)]
        want = [str(a * 100000 + b) for a, b in om.read(s)]
        assert got[2:] == want, s


@pytest.mark.parametrize("seed,nb,bs,seqs,maxb", [
    (1, 40, 16, 4, 12), (2, 24, 16, 6, 6), (3, 100, 32, 8, 20), (4, 12, 16, 3, 10)])
def test_block_manager_sanitized(binary, seed, nb, bs, seqs, maxb):
    cmds, exp = _blocks_trace(seed, nb, bs, seqs, maxb, 120)
    lines = _run(binary, cmds)
    refused = 0
    for kind, want in exp:
        if kind == "rc":
            rc = _ints(next(lines), "rc")[0]
            assert rc == want, (kind, want, rc)
            refused += rc != 0
        else:
            _check_bstate(lines, want, seqs, maxb, nb)
    assert next(lines, None) is None


# ---------------------------------------------------------------------------
# host-pool pager
# ---------------------------------------------------------------------------

def _pager_trace(seed, batch, L, C, n_ops):
    """Advances (copies on the attention stream or a second one), stages
    with their fused decodes, and commits, in random order: the library's
    refusals follow its rules (no stage while an advance's copies or another
    stage are pending; no advance while a stage is pending; no decode while
    an advance's copies are pending).  The state is checked whenever no
    stage is pending (a pending stage's slots still hold their old blocks)."""
    rng = np.random.default_rng(seed)
    pools = [LruPool(C) for _ in range(batch)]
    nphys = batch * C
    cmds, exp = [f"pager {batch} 2 64 16 {L} {C} {nphys}"], [("rc", 0, None)]
    staged = pending = False

    def draw():
        reqs = []
        for _b in range(batch):
            n = int(rng.integers(0, C // 2 + 1)) if rng.random() < 0.85 else \
                int(rng.integers(0, min(L, C + 3)))
            reqs.append([int(x) for x in rng.integers(0, L, size=n)])
        return reqs

    def serve(reqs):
        nonlocal pools
        trial = copy.deepcopy(pools)
        loaded = 0
        try:
            for p, r in zip(trial, reqs):
                loaded += len(p.advance(r))
        except PoolRefused:
            return -1, None
        pools = trial
        return 0, loaded

    def packed(reqs):
        return " ".join(f"{len(r)} " + " ".join(map(str, r)) for r in reqs)

    for _ in range(n_ops):
        x = rng.random()
        if x < 0.12:
            for p in pools:
                p.commit()
            staged = pending = False
            cmds.append("commit")
            exp.append(("rc", 0, None))
        elif x < 0.45:
            reqs = draw()
            if staged:
                rc, loaded = -1, None
            else:
                rc, loaded = serve(reqs)
                if rc == 0:
                    pending = loaded > 0
            cmds.append(f"advance {int(rng.integers(2))} " + packed(reqs))
            exp.append(("advance", rc, loaded))
        elif x < 0.75:
            reqs = draw()
            if staged or pending:
                rc, loaded = -1, None
            else:
                rc, loaded = serve(reqs)
                if rc == 0:
                    staged = loaded > 0
            cmds.append("stage " + packed(reqs))
            exp.append(("advance", rc, loaded))
        else:
            if pending:
                rc = -1
            else:
                rc = 0
                for p in pools:
                    p.commit()
                staged = False
            cmds.append("pdecode")
            exp.append(("rc", rc, None))
        if not staged:
            cmds.append("pstate")
            exp.append(("pstate", copy.deepcopy(pools), None))
    return cmds, exp


@pytest.mark.parametrize("seed,batch,L,C", [(11, 2, 30, 6), (12, 3, 50, 10), (13, 1, 20, 4)])
def test_pager_sanitized(binary, seed, batch, L, C):
    cmds, exp = _pager_trace(seed, batch, L, C, 150)
    lines = _run(binary, cmds)
    refused = 0
    for kind, want, loaded in exp:
        if kind == "rc":
            assert _ints(next(lines), "rc")[0] == want
        elif kind == "advance":
            parts = next(lines).split()
            assert parts[0] == "rc" and int(parts[1]) == want, (parts, want)
            if want == 0:
                assert int(parts[3]) == loaded
            refused += want != 0
        else:
            for p in want:
                slots = _ints(next(lines), "slots")
                valid = _ints(next(lines), "valid")
                assert slots == p.slot_block
                vis = p.visible()
                assert valid == [1 if (b >= 0 and b in vis) else 0 for b in p.slot_block]
            assert _ints(next(lines), "bad")[0] == 0
    assert next(lines, None) is None
    assert refused > 0 or C >= L  # the traces include refused requests
