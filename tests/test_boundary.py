"""The C-ABI boundary on the host: libswa loads, exports every function that
include/swa.h declares, sizes buffers, and rejects bad arguments before any
HIP call (no compute is launched by these tests; they run without a GPU)."""

import ctypes
import os
import re

import pytest

from decode_attention_fixed_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")

FAKE = 0x100000  # never dereferenced: every call below fails validation first


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*([A-Za-z_]\w*)\s*\(", src, re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_functions_are_exported():
    declared = _declared_functions()
    assert len(declared) == 35, declared
    assert sorted(B.EXPORTED) == declared
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def _cfg(**kw):
    base = dict(batch=8, num_kv_heads=32, head_dim=128, window=4096, num_sinks=4, dtype="bf16")
    base.update(kw)
    return B.make_config(**base)


def test_required_bytes():
    kv, sp = B.swa_cache_required_bytes(_cfg())
    assert kv == 8 * 32 * 4100 * 128 * 2
    assert sp == 8 * 4100 * 4
    kv, sp = B.swa_cache_required_bytes(_cfg(batch=1, num_kv_heads=4, head_dim=64, window=16,
                                             dtype="f32"))
    assert kv == 1 * 4 * 20 * 64 * 4 and sp == 20 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), B.SWA_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), B.SWA_ERR_INVALID_ARG),
    (dict(window=0), B.SWA_ERR_INVALID_ARG),
    (dict(num_sinks=-1), B.SWA_ERR_INVALID_ARG),
    (dict(head_dim=96), B.SWA_ERR_UNSUPPORTED),
    (dict(head_dim=256), B.SWA_ERR_UNSUPPORTED),
])
def test_bad_config(kw, code):
    with pytest.raises(B.SwaError) as e:
        B.swa_cache_required_bytes(_cfg(**kw))
    assert e.value.code == code
    assert B.swa_last_error() != ""


def test_bad_rope_base_and_dtype():
    cfg = _cfg()
    cfg.rope_base = 0.0
    with pytest.raises(B.SwaError):
        B.swa_cache_required_bytes(cfg)
    cfg = _cfg()
    cfg.dtype = 7
    with pytest.raises(B.SwaError):
        B.swa_cache_required_bytes(cfg)


def _create(**kw):
    cfg = _cfg(**kw)
    h = ctypes.c_void_p()
    rc = B.LIB.swa_cache_create(ctypes.byref(cfg), FAKE, FAKE, FAKE, ctypes.byref(h))
    assert rc == B.SWA_OK, B.swa_last_error()
    assert B.swa_last_error() == ""
    return h.value


def test_create_and_destroy_touch_no_device_memory():
    h = _create()
    assert h
    B.swa_cache_destroy(h)
    B.swa_cache_destroy(None)


def test_create_rejects_null_and_misaligned():
    cfg = _cfg()
    h = ctypes.c_void_p()
    assert B.LIB.swa_cache_create(ctypes.byref(cfg), None, FAKE, FAKE, ctypes.byref(h)) == \
        B.SWA_ERR_INVALID_ARG
    assert B.LIB.swa_cache_create(ctypes.byref(cfg), FAKE + 2, FAKE, FAKE, ctypes.byref(h)) == \
        B.SWA_ERR_INVALID_ARG
    assert B.LIB.swa_cache_create(ctypes.byref(cfg), FAKE, FAKE, FAKE, None) == \
        B.SWA_ERR_INVALID_ARG
    assert h.value is None


def test_append_validation():
    h = _create(num_kv_heads=4)
    L = B.LIB
    try:
        assert L.kv_append_rope(None, FAKE, FAKE, FAKE, 1, None, 0, None) == B.SWA_ERR_INVALID_ARG
        assert L.kv_append_rope(h, None, FAKE, FAKE, 1, None, 0, None) == B.SWA_ERR_INVALID_ARG
        assert L.kv_append_rope(h, FAKE, FAKE, None, 1, None, 0, None) == B.SWA_ERR_INVALID_ARG
        assert L.kv_append_rope(h, FAKE, FAKE, FAKE, 0, None, 0, None) == B.SWA_ERR_INVALID_ARG
        assert L.kv_append_rope(h, FAKE, FAKE, FAKE, -3, None, 0, None) == B.SWA_ERR_INVALID_ARG
        assert L.kv_append_rope(h, FAKE + 8, FAKE, FAKE, 1, None, 0, None) == B.SWA_ERR_INVALID_ARG
        # query heads: not a multiple of Hkv / unsupported group
        assert L.kv_append_rope(h, FAKE, FAKE, FAKE, 1, FAKE, 6, None) == B.SWA_ERR_INVALID_ARG
        assert L.kv_append_rope(h, FAKE, FAKE, FAKE, 1, FAKE, 20, None) == B.SWA_ERR_UNSUPPORTED
        assert L.kv_append_rope(h, FAKE, FAKE, FAKE, 1, FAKE, 0, None) == B.SWA_ERR_INVALID_ARG
    finally:
        B.swa_cache_destroy(h)


def test_workspace_sizes():
    n = B.decode_attn_workspace_bytes(8, 32, 32, 128, 4100)
    assert n > 8 * 32 * 128 * 4 and n % 256 == 0
    # more tokens never needs less workspace
    sizes = [B.decode_attn_workspace_bytes(64, 32, 8, 128, t) for t in (1, 100, 4100, 40000)]
    assert sizes == sorted(sizes)
    with pytest.raises(B.SwaError):
        B.decode_attn_workspace_bytes(8, 30, 32, 128, 4100)
    with pytest.raises(B.SwaError):
        B.decode_attn_workspace_bytes(8, 32, 32, 80, 4100)


def test_decode_ring_validation():
    h = _create()
    L = B.LIB
    need = B.decode_attn_workspace_bytes(8, 32, 32, 128, 4100)
    try:
        args = dict(q=FAKE, hq=32, scale=0.0, out=FAKE, odt=B.SWA_F32, lse=None, ws=FAKE,
                    wsb=need)

        def call(**kw):
            a = dict(args)
            a.update(kw)
            return L.decode_attn_ring(h, a["q"], a["hq"], a["scale"], a["out"], a["odt"], a["lse"],
                                      a["ws"], a["wsb"], None)

        assert call(wsb=need - 1) == B.SWA_ERR_WORKSPACE
        assert "too small" in B.swa_last_error()
        assert call(ws=None) == B.SWA_ERR_WORKSPACE
        assert call(ws=FAKE + 16) == B.SWA_ERR_WORKSPACE  # not 256-byte aligned
        assert call(q=None) == B.SWA_ERR_INVALID_ARG
        assert call(out=None) == B.SWA_ERR_INVALID_ARG
        assert call(out=FAKE + 4) == B.SWA_ERR_INVALID_ARG
        assert call(odt=5) == B.SWA_ERR_INVALID_ARG
        assert call(hq=48) == B.SWA_ERR_INVALID_ARG
        assert call(hq=32 * 5) == B.SWA_ERR_UNSUPPORTED
        assert L.decode_attn_ring(None, FAKE, 32, 0.0, FAKE, 0, None, FAKE, need, None) == \
            B.SWA_ERR_INVALID_ARG
    finally:
        B.swa_cache_destroy(h)


def test_stream_read_validation():
    L = B.LIB
    sink = B.STREAM_READ_SINK_BYTES
    assert L.swa_stream_read(FAKE, 0, None, 0, None) == B.SWA_OK          # nothing to read
    assert L.swa_stream_read(FAKE, 24, FAKE, sink, None) == B.SWA_ERR_INVALID_ARG  # not 16-byte units
    assert L.swa_stream_read(None, 32, FAKE, sink, None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_stream_read(FAKE, 32, None, sink, None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_stream_read(FAKE + 8, 32, FAKE, sink, None) == B.SWA_ERR_INVALID_ARG  # misaligned
    assert L.swa_stream_read(FAKE, 32, FAKE + 2, sink, None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_stream_read(FAKE, 32, FAKE, sink - 4, None) == B.SWA_ERR_INVALID_ARG


def test_pos_advance_validation():
    L = B.LIB
    assert L.swa_pos_advance(FAKE, -1, 1, None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_pos_advance(None, 4, 1, None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_pos_advance(FAKE + 2, 4, 1, None) == B.SWA_ERR_INVALID_ARG  # misaligned
    assert L.swa_pos_advance(None, 0, 1, None) == B.SWA_OK  # nothing to do, nothing launched


def test_decode_step_ring_validation():
    h = _create()
    L = B.LIB
    need = B.decode_attn_workspace_bytes(8, 32, 32, 128, 4100)
    try:
        args = dict(k=FAKE, v=FAKE, pos=FAKE, q=FAKE, hq=32, out=FAKE, ws=FAKE, wsb=need)

        def call(**kw):
            a = dict(args)
            a.update(kw)
            return L.decode_step_ring(h, a["k"], a["v"], a["pos"], a["q"], a["hq"], 0.0, a["out"],
                                      B.SWA_F32, None, a["ws"], a["wsb"], None)

        assert call(k=None) == B.SWA_ERR_INVALID_ARG
        assert call(v=None) == B.SWA_ERR_INVALID_ARG
        assert call(pos=None) == B.SWA_ERR_INVALID_ARG
        assert call(k=FAKE + 8) == B.SWA_ERR_INVALID_ARG   # not 16-byte aligned
        assert call(pos=FAKE + 2) == B.SWA_ERR_INVALID_ARG
        assert call(q=None) == B.SWA_ERR_INVALID_ARG
        assert call(hq=48) == B.SWA_ERR_INVALID_ARG
        assert call(wsb=need - 1) == B.SWA_ERR_WORKSPACE
        assert L.decode_step_ring(None, FAKE, FAKE, FAKE, FAKE, 32, 0.0, FAKE, 0, None, FAKE, need,
                                  None) == B.SWA_ERR_INVALID_ARG
    finally:
        B.swa_cache_destroy(h)


@pytest.mark.parametrize("kw", [dict(dtype="i8"), dict(dtype="f32"), dict(head_dim=64)])
def test_shifted_step_needs_bf16_d128(kw):
    """Cache position shifting is built for bf16 caches with head_dim 128;
    other caches get SWA_ERR_UNSUPPORTED before anything is launched."""
    h = _create(**kw)
    try:
        d = kw.get("head_dim", 128)
        need = B.decode_attn_workspace_bytes(8, 32, 32, d, 4100)
        rc = B.LIB.decode_step_ring_shifted(h, FAKE, FAKE, FAKE, FAKE, 32, 0.0, FAKE, B.SWA_F32,
                                            None, FAKE, need, None)
        assert rc == B.SWA_ERR_UNSUPPORTED, B.swa_last_error()
        assert "shifting" in B.swa_last_error()
    finally:
        B.swa_cache_destroy(h)


def test_prefill_validation():
    h = _create()
    L = B.LIB
    need = B.prefill_attn_workspace_bytes(8, 32, 32, 128, 64)
    assert need >= 8 * 64 * (32 + 32) * 128 * 2 and need % 256 == 0
    try:
        args = dict(k=FAKE, v=FAKE, pos=FAKE, n=64, q=FAKE, hq=32, out=FAKE, ws=FAKE, wsb=need)

        def call(handle=h, **kw):
            a = dict(args)
            a.update(kw)
            return L.prefill_attn_ring(handle, a["k"], a["v"], a["pos"], a["n"], a["q"], a["hq"],
                                       0.0, a["out"], B.SWA_F32, None, a["ws"], a["wsb"], None)

        assert call(k=None) == B.SWA_ERR_INVALID_ARG
        assert call(q=None) == B.SWA_ERR_INVALID_ARG
        assert call(n=0) == B.SWA_ERR_INVALID_ARG
        assert call(hq=48) == B.SWA_ERR_INVALID_ARG
        assert call(out=FAKE + 4) == B.SWA_ERR_INVALID_ARG
        assert call(wsb=need - 1) == B.SWA_ERR_WORKSPACE
        assert call(ws=FAKE + 16) == B.SWA_ERR_WORKSPACE
        assert call(handle=None) == B.SWA_ERR_INVALID_ARG
    finally:
        B.swa_cache_destroy(h)
    for kw in (dict(dtype="f32"), dict(head_dim=64)):   # only bf16, d = 128
        h = _create(**kw)
        try:
            assert L.prefill_attn_ring(h, FAKE, FAKE, FAKE, 8, FAKE, 32, 0.0, FAKE, B.SWA_F32,
                                       None, FAKE, 1 << 30, None) == B.SWA_ERR_UNSUPPORTED
        finally:
            B.swa_cache_destroy(h)
    with pytest.raises(B.SwaError):
        B.prefill_attn_workspace_bytes(8, 32, 32, 64, 64)


def _desc(**kw):
    base = dict(batch=32, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                max_blocks_per_seq=2048, num_phys_blocks=30000, dtype="bf16")
    base.update(kw)
    return B.make_paged_desc(**base)


def _paged(desc, **kw):
    try:
        need = B.decode_attn_workspace_bytes(desc.batch, desc.num_q_heads, desc.num_kv_heads,
                                             desc.head_dim,
                                             desc.max_blocks_per_seq * desc.block_size)
    except B.SwaError:
        need = 1 << 30  # the descriptor itself is what the call must reject
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, bv=None, out=FAKE, ws=FAKE, wsb=need)
    a.update(kw)
    return B.LIB.decode_attn_paged(ctypes.byref(desc), a["q"], a["k"], a["v"], a["bt"], a["sl"],
                                   a["bv"], 0.0, a["out"], B.SWA_F32, None, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(block_size=8), B.SWA_ERR_UNSUPPORTED),
    (dict(block_size=48), B.SWA_ERR_UNSUPPORTED),
    (dict(block_size=2048), B.SWA_ERR_UNSUPPORTED),
    (dict(num_phys_blocks=0), B.SWA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=0), B.SWA_ERR_INVALID_ARG),
    (dict(num_q_heads=12), B.SWA_ERR_INVALID_ARG),
    (dict(head_dim=32), B.SWA_ERR_UNSUPPORTED),
    (dict(num_phys_blocks=200_000_000), B.SWA_ERR_INVALID_ARG),
])
def test_decode_paged_desc_validation(kw, code):
    assert _paged(_desc(**kw)) == code


def test_decode_paged_pointer_validation():
    d = _desc()
    assert _paged(d, sl=None) == B.SWA_ERR_INVALID_ARG
    assert _paged(d, bt=None) == B.SWA_ERR_INVALID_ARG
    assert _paged(d, k=FAKE + 2) == B.SWA_ERR_INVALID_ARG
    assert _paged(d, wsb=16) == B.SWA_ERR_WORKSPACE


def test_write_paged_validation():
    d = _desc()
    L = B.LIB
    assert L.kv_write_paged(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 1e4, 0,
                            None) == B.SWA_ERR_INVALID_ARG
    assert L.kv_write_paged(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, 5, 1e4, 0,
                            None) == B.SWA_ERR_INVALID_ARG
    assert L.kv_write_paged(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5, -1.0, 0,
                            None) == B.SWA_ERR_INVALID_ARG
    assert L.kv_write_paged(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5, 1e4, 9,
                            None) == B.SWA_ERR_INVALID_ARG


def test_product_path_has_no_fallback():
    """The binding imports nothing from the oracle and has no CPU path."""
    src = open(os.path.join(ROOT, "decode_attention_fixed_amd", "binding.py")).read()
    assert "oracle" not in src and "numpy" not in src
    for f in os.listdir(os.path.join(ROOT, "decode_attention_fixed_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "decode_attention_fixed_amd", "csrc",
                                                 f)).read()


def _pcfg(**kw):
    base = dict(batch=1, num_kv_heads=4, head_dim=128, block_size=64, logical_blocks=4096,
                slots_per_seq=1152, num_phys_blocks=1152, dtype="bf16")
    base.update(kw)
    return B.make_pager_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), B.SWA_ERR_INVALID_ARG),
    (dict(logical_blocks=0), B.SWA_ERR_INVALID_ARG),
    (dict(slots_per_seq=0), B.SWA_ERR_INVALID_ARG),
    (dict(num_phys_blocks=0), B.SWA_ERR_INVALID_ARG),
    (dict(head_dim=96), B.SWA_ERR_UNSUPPORTED),
    (dict(block_size=48), B.SWA_ERR_UNSUPPORTED),
    (dict(block_size=2048), B.SWA_ERR_UNSUPPORTED),
    (dict(batch=1 << 20, logical_blocks=1 << 12), B.SWA_ERR_INVALID_ARG),
])
def test_pager_config_validation(kw, code):
    L = B.LIB
    cfg = _pcfg(**kw)
    out = ctypes.c_void_p()
    slots = (ctypes.c_int32 * 4)(0, 1, 2, 3)
    assert L.swa_pager_create(ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, ctypes.cast(slots,
                              ctypes.c_void_p), FAKE, FAKE, ctypes.byref(out)) == code
    assert out.value is None
    assert B.swa_last_error()


def test_pager_pointer_and_table_validation():
    L = B.LIB
    cfg = _pcfg(slots_per_seq=4, num_phys_blocks=8)
    out = ctypes.c_void_p()
    ok_slots = (ctypes.c_int32 * 4)(7, 0, 3, 5)

    def create(hk=FAKE, hv=FAKE, kp=FAKE, vp=FAKE, slots=ok_slots, bt=FAKE, bv=FAKE, o=out):
        sp = ctypes.cast(slots, ctypes.c_void_p) if slots is not None else None
        return L.swa_pager_create(ctypes.byref(cfg), hk, hv, kp, vp, sp, bt, bv,
                                  ctypes.byref(o) if o is not None else None)

    assert create(hk=None) == B.SWA_ERR_INVALID_ARG
    assert create(slots=None) == B.SWA_ERR_INVALID_ARG
    assert create(bv=None) == B.SWA_ERR_INVALID_ARG
    assert create(o=None) == B.SWA_ERR_INVALID_ARG
    assert create(kp=FAKE + 8) == B.SWA_ERR_INVALID_ARG
    assert create(slots=(ctypes.c_int32 * 4)(0, 1, 2, 8)) == B.SWA_ERR_INVALID_ARG  # out of range
    assert "outside" in B.swa_last_error()
    assert create(slots=(ctypes.c_int32 * 4)(0, 1, 1, 2)) == B.SWA_ERR_INVALID_ARG  # shared
    assert "two slots" in B.swa_last_error()
    # valid arguments, but the host store is not pinned memory the device can read
    assert create() == B.SWA_ERR_INVALID_ARG
    assert out.value is None


def test_pager_null_handle():
    L = B.LIB
    off = (ctypes.c_int32 * 2)(0, 0)
    assert L.swa_pager_reset(None, None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_pager_advance(None, ctypes.cast(off, ctypes.c_void_p), None, None, None,
                               None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_pager_commit(None, None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_pager_slot_blocks(None, 0, FAKE) == B.SWA_ERR_INVALID_ARG
    L.swa_pager_destroy(None)


def test_blocks_null_handle():
    L = B.LIB
    assert L.swa_blocks_reset(None) == B.SWA_ERR_INVALID_ARG
    assert L.swa_blocks_free(None, 0, FAKE, None) == B.SWA_ERR_INVALID_ARG
    L.swa_blocks_destroy(None)


def test_int8_is_not_an_output_dtype():
    """SWA_I8 names a cache element type, never an output type: every entry
    point that writes `out` refuses it before anything is launched (an int8
    out buffer would be a quarter of the float32 rows written into it)."""
    L = B.LIB
    h = _create()
    need = B.decode_attn_workspace_bytes(8, 32, 32, 128, 4100)
    pneed = B.prefill_attn_workspace_bytes(8, 32, 32, 128, 64)
    try:
        rcs = {
            "decode_attn_ring": L.decode_attn_ring(h, FAKE, 32, 0.0, FAKE, B.SWA_I8, None, FAKE,
                                                   need, None),
            "decode_step_ring": L.decode_step_ring(h, FAKE, FAKE, FAKE, FAKE, 32, 0.0, FAKE,
                                                   B.SWA_I8, None, FAKE, need, None),
            "decode_step_ring_shifted": L.decode_step_ring_shifted(h, FAKE, FAKE, FAKE, FAKE, 32,
                                                                   0.0, FAKE, B.SWA_I8, None,
                                                                   FAKE, need, None),
            "prefill_attn_ring": L.prefill_attn_ring(h, FAKE, FAKE, FAKE, 64, FAKE, 32, 0.0, FAKE,
                                                     B.SWA_I8, None, FAKE, pneed, None),
        }
    finally:
        B.swa_cache_destroy(h)
    d = _desc()
    pw = B.decode_attn_workspace_bytes(32, 32, 8, 128, 2048 * 16)
    rcs["decode_attn_paged"] = L.decode_attn_paged(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE,
                                                   None, 0.0, FAKE, B.SWA_I8, None, FAKE, pw,
                                                   None)
    for name, rc in rcs.items():
        assert rc == B.SWA_ERR_INVALID_ARG, name
    assert "out_dtype" in B.swa_last_error()


def test_binding_checks_shapes_before_the_call():
    """The binding compares every tensor with the sizes the call will touch
    and raises ValueError on a mismatch; no pointer reaches the library."""
    import torch
    d = B.make_paged_desc(2, 8, 2, 128, 16, 10, 20, "bf16")
    pool_shape = (20, 2, 16, 128)
    ok = dict(q=torch.zeros(2, 8, 128, dtype=torch.bfloat16),
              k_pool=torch.zeros(pool_shape, dtype=torch.bfloat16),
              v_pool=torch.zeros(pool_shape, dtype=torch.bfloat16),
              block_table=torch.zeros(2, 10, dtype=torch.int32),
              seq_lens=torch.zeros(2, dtype=torch.int32), block_valid=None,
              out=torch.zeros(2, 8, 128), workspace=torch.zeros(16, dtype=torch.uint8))
    bad = [
        ("q", torch.zeros(2, 4, 128, dtype=torch.bfloat16), "shape"),
        ("q", torch.zeros(2, 8, 128), "must be one of"),                    # f32 q on a bf16 pool
        ("k_pool", torch.zeros(19, 2, 16, 128, dtype=torch.bfloat16), "bytes"),
        ("block_table", torch.zeros(2, 9, dtype=torch.int32), "elements"),
        ("block_table", torch.zeros(2, 10, dtype=torch.int64), "int32"),
        ("seq_lens", torch.zeros(1, dtype=torch.int32), "elements"),
        ("block_valid", torch.zeros(2, 9, dtype=torch.uint8), "elements"),
        ("out", torch.zeros(2, 8, 64), "shape"),
        ("out", torch.zeros(2, 8, 128, dtype=torch.float16), "must be one of"),
    ]
    for name, t, what in bad:
        kw = dict(ok)
        kw[name] = t
        with pytest.raises(ValueError, match=what):
            B.decode_attn_paged(d, **kw)
    # the well-shaped CPU tensors get as far as the device check
    with pytest.raises(ValueError, match="device tensor"):
        B.decode_attn_paged(d, **ok)
    with pytest.raises(ValueError, match="shape"):
        B.kv_write_paged(d, ok["k_pool"], ok["v_pool"], torch.zeros(5, 2, 64, dtype=torch.bfloat16),
                         torch.zeros(5, 2, 128, dtype=torch.bfloat16),
                         torch.zeros(5, dtype=torch.int32))


def test_binding_checks_ring_tensors():
    import torch
    cfg = _cfg(batch=2, num_kv_heads=4, window=64)
    kv, sp = B.swa_cache_required_bytes(cfg)
    h = _create(batch=2, num_kv_heads=4, window=64)
    B._RING_CFG[h] = cfg   # what swa_cache_create records for a handle it made
    try:
        q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
        with pytest.raises(ValueError, match="shape"):
            B.decode_attn_ring(h, q, torch.zeros(2, 8, 64), torch.zeros(16, dtype=torch.uint8))
        with pytest.raises(ValueError, match="shape"):
            B.decode_step_ring(h, torch.zeros(2, 2, 128, dtype=torch.bfloat16),
                               torch.zeros(2, 4, 128, dtype=torch.bfloat16),
                               torch.zeros(2, dtype=torch.int32), q, torch.zeros(2, 8, 128),
                               torch.zeros(16, dtype=torch.uint8))
        with pytest.raises(ValueError, match="shape"):
            B.kv_append_rope(h, torch.zeros(2, 3, 4, 128, dtype=torch.bfloat16),
                             torch.zeros(2, 3, 4, 128, dtype=torch.bfloat16),
                             torch.zeros(3, dtype=torch.int32))
        with pytest.raises(ValueError, match="must be one of"):
            B.prefill_attn_ring(h, torch.zeros(2, 3, 4, 128), torch.zeros(2, 3, 4, 128),
                                torch.zeros(2, dtype=torch.int32), torch.zeros(2, 3, 8, 128),
                                torch.zeros(2, 3, 8, 128), torch.zeros(16, dtype=torch.uint8))
    finally:
        B.swa_cache_destroy(h)
    assert h not in B._RING_CFG


def test_noalloc_refuses_beyond_its_maximum():
    """decode_attn_paged_noalloc refuses sizes whose partial results exceed
    its fixed array, on the host and before any HIP call (no GPU here: any HIP
    call would fail with SWA_ERR_HIP instead)."""
    d = B.make_paged_desc(512, 64, 8, 128, 16, 4096, 1 << 16, "bf16")
    assert B.decode_attn_workspace_bytes(512, 64, 8, 128, 4096 * 16) > B.NOALLOC_SCRATCH_BYTES
    rc = B.LIB.decode_attn_paged_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0.0,
                                         FAKE, B.SWA_F32, None, None)
    assert rc == B.SWA_ERR_WORKSPACE
    assert "maximum" in B.swa_last_error()
    # and the argument checks of decode_attn_paged come first
    bad = B.make_paged_desc(4, 12, 8, 128, 16, 64, 256, "bf16")    # 12 heads over 8 kv heads
    assert B.LIB.decode_attn_paged_noalloc(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                           0.0, FAKE, B.SWA_F32, None, None) == \
        B.SWA_ERR_INVALID_ARG
