"""Host-side checks of the two C libraries (no GPU needed, no kernel launched).

- libkda.so exports every function include/kda.h declares, and the Python
  binding offers each under the same name;
- liboracle_kda.so exports every function include/kda_oracle.h declares, and
  libkda_calib.so every function of include/kda_calib.h;
- argument validation of the C ABI: every rejected call returns its status
  before anything touches a device (fake, never-dereferenced pointers are used
  where only alignment or presence is checked);
- the product package fails loudly when libkda.so is missing and never imports
  the oracle.
"""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header: str):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(kda_[a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def K():
    from gated_delta_rule_72_amd import build as B
    if not os.path.exists(B.LIB):
        B.build()
    import gated_delta_rule_72_amd.kda as K
    K.load()
    return K


def test_kda_header_symbols_exported(K):
    names = _declared("kda.h")
    assert set(names) == {"kda_abi_version", "kda_last_error", "kda_snapshot_count",
                          "kda_prefill_workspace_size", "kda_prefill_chunked", "kda_prefill_chunked_noalloc",
                          "kda_decode_step",
                          "kda_decode_tokens", "kda_layer_front", "kda_layer_back",
                          "kda_layer_prefill_workspace_size", "kda_layer_prefill",
                          "kda_prefill_backward_workspace_size", "kda_prefill_backward"}
    lib = ctypes.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
        assert callable(getattr(K, n)), n
    assert set(K.EXPORTED) == set(names)
    assert K.kda_abi_version() == 1


def test_oracle_header_symbols_exported():
    import oracle
    names = _declared("kda_oracle.h")
    assert set(names) == {"kda_oracle_snapshot_count", "kda_oracle_run", "kda_recurrent_ref_check",
                          "kda_oracle_backward"}
    lib = oracle.load()
    for n in names:
        assert hasattr(lib, n), n


def test_calib_header_symbols_exported_and_checked(K):
    from gated_delta_rule_72_amd import build as B
    if not os.path.exists(B.CALIB_LIB):
        B.build()
    names = _declared("kda_calib.h")
    assert set(names) == {"kda_calib_mfma_f16", "kda_calib_copy"}
    lib = ctypes.CDLL(B.CALIB_LIB)
    for n in names:
        assert hasattr(lib, n), n
    lib.kda_calib_mfma_f16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.kda_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                   ctypes.c_void_p]
    # rejected on the host, nothing launched
    assert lib.kda_calib_mfma_f16(0, 10, _fake(0x1000), None) == -1
    assert lib.kda_calib_mfma_f16(4, 10, _fake(0x1004), None) == -1
    assert lib.kda_calib_mfma_f16(4, 10, None, None) == -1
    assert lib.kda_calib_copy(_fake(0x1000), _fake(0x2000), -1, 4, None) == -1
    assert lib.kda_calib_copy(_fake(0x1008), _fake(0x2000), 16, 4, None) == -1
    assert lib.kda_calib_copy(None, None, 0, 4, None) == 0


def test_snapshot_count(K):
    cu = torch.tensor([0, 100, 100, 300, 556], dtype=torch.int64)
    assert K.kda_snapshot_count(cu, 0) == 0
    assert K.kda_snapshot_count(cu, 64) == 1 + 0 + 3 + 4
    assert K.kda_snapshot_count(cu, 128) == 0 + 0 + 1 + 2
    with pytest.raises(K.KdaError) as e:
        K.kda_snapshot_count(torch.tensor([1, 5], dtype=torch.int64), 64)
    assert e.value.code == K.KDA_ERR_SHAPE
    with pytest.raises(K.KdaError) as e:
        K.kda_snapshot_count(torch.tensor([0, 5, 3], dtype=torch.int64), 64)
    assert e.value.code == K.KDA_ERR_SHAPE and "decreases" in K.kda_last_error()


def test_workspace_size_plans(K):
    sh = K.make_shape(2, 64, 64, torch.bfloat16, True)
    cu = torch.tensor([0, 100, 300], dtype=torch.int64)
    plain = K.kda_prefill_workspace_size(sh, cu, 64, 64, 0)
    seg = K.kda_prefill_workspace_size(sh, cu, 64, 64, 128)
    assert 0 < plain <= 1024
    # 128-token segments: 1 + 2 items, each with (M, N) maps and a start state
    items, H, DD = 3, 2, 64 * 64
    assert seg >= plain + items * H * 3 * DD * 4
    # a segment as long as the longest sequence splits nothing
    assert K.kda_prefill_workspace_size(sh, cu, 64, 64, 256) == plain


@pytest.mark.parametrize("field,value,code", [
    ("d_k", 96, "KDA_ERR_SHAPE"), ("d_v", 96, "KDA_ERR_SHAPE"), ("num_heads", 0, "KDA_ERR_SHAPE"),
    ("num_heads", 65536, "KDA_ERR_SHAPE"),
    ("qkv_dtype", 7, "KDA_ERR_ARG"), ("gate", 2, "KDA_ERR_ARG")])
def test_bad_shapes_rejected(K, field, value, code):
    sh = K.make_shape(2, 128, 128, torch.bfloat16, False)
    setattr(sh, field, value)
    with pytest.raises(K.KdaError) as e:
        K.kda_prefill_workspace_size(sh, torch.tensor([0, 64], dtype=torch.int64), 64, 0, 0)
    assert e.value.code == getattr(K, code)


@pytest.mark.parametrize("chunk,interval,seg", [(32, 0, 0), (64, 100, 0), (64, -64, 0), (64, 0, 100),
                                                (64, 0, -2)])
def test_bad_plan_arguments_rejected(K, chunk, interval, seg):
    sh = K.make_shape(1, 64, 64, torch.float32, False)
    with pytest.raises(K.KdaError) as e:
        K.kda_prefill_workspace_size(sh, torch.tensor([0, 64], dtype=torch.int64), chunk, interval, seg)
    assert e.value.code == K.KDA_ERR_SHAPE


def _fake(addr):
    return ctypes.c_void_p(addr)


def _prefill_raw(K, sh, cu, ptrs, ws_bytes, interval=0, seg=0):
    cu = cu.contiguous()
    lib = K.load()
    # fake addresses 16 MiB apart: far enough that no two buffers overlap
    p = dict(cu_dev=0x1000000, q=0x2000000, k=0x3000000, v=0x4000000, alpha=0x5000000, beta=0x6000000, init=None,
             o=0x7000000, fin=0x8000000, snaps=None, ws=0x9000000)
    p.update(ptrs)
    f = lambda n: None if p[n] is None else _fake(p[n])  # noqa: E731
    return lib.kda_prefill_chunked(ctypes.byref(sh), cu.numel() - 1, ctypes.c_void_p(cu.data_ptr()),
                                   f("cu_dev"), 64, interval, seg, f("q"), f("k"), f("v"), f("alpha"),
                                   f("beta"), f("init"), f("o"), f("fin"), f("snaps"), f("ws"),
                                   ws_bytes, None)


def test_prefill_host_rejections(K):
    """Each call below fails a host check, so no pointer is ever dereferenced."""
    sh = K.make_shape(2, 64, 64, torch.bfloat16, True)
    cu = torch.tensor([0, 100, 300], dtype=torch.int64)
    need = K.kda_prefill_workspace_size(sh, cu, 64, 0, 0)
    assert _prefill_raw(K, sh, cu, {"q": 0x2000008}, need) == K.KDA_ERR_ALIGN
    assert "q" in K.kda_last_error()
    assert _prefill_raw(K, sh, cu, {"alpha": 0x5000004}, need) == K.KDA_ERR_ALIGN   # per-key: 16 B
    assert _prefill_raw(K, sh, cu, {"fin": 0x8000004}, need) == K.KDA_ERR_ALIGN
    assert _prefill_raw(K, sh, cu, {"o": 0x7000004}, need) == K.KDA_ERR_ALIGN       # o: 16 B (row stores)
    assert "o" in K.kda_last_error()
    assert _prefill_raw(K, sh, cu, {"q": None}, need) == K.KDA_ERR_ARG
    assert _prefill_raw(K, sh, cu, {"fin": None}, need) == K.KDA_ERR_ARG
    assert _prefill_raw(K, sh, cu, {"cu_dev": None}, need) == K.KDA_ERR_ARG
    assert _prefill_raw(K, sh, cu, {}, need - 1) == K.KDA_ERR_WORKSPACE
    assert _prefill_raw(K, sh, cu, {"ws": None}, need) == K.KDA_ERR_WORKSPACE
    # snapshots due (interval 64 -> 1 + 3 slots) but no buffer
    assert _prefill_raw(K, sh, cu, {}, need, interval=64) == K.KDA_ERR_ARG
    assert "snapshot" in K.kda_last_error()
    # scalar gate needs only 4-byte alpha
    sh_s = K.make_shape(2, 64, 64, torch.bfloat16, False)
    assert _prefill_raw(K, sh_s, cu, {"alpha": 0x5000004, "q": 0x2000008}, need) == K.KDA_ERR_ALIGN
    assert "q" in K.kda_last_error()
    # outputs must not overlap inputs (o over k; final state over q); the final
    # state may be the initial state itself, but not overlap it partially
    assert _prefill_raw(K, sh, cu, {"o": 0x3000000}, need) == K.KDA_ERR_ARG
    assert "overlaps" in K.kda_last_error() and "o" in K.kda_last_error()
    assert _prefill_raw(K, sh, cu, {"fin": 0x2000010}, need) == K.KDA_ERR_ARG
    assert _prefill_raw(K, sh, cu, {"init": 0xA000000, "fin": 0xA000010}, need) == K.KDA_ERR_ARG
    # nothing to do: no sequences
    assert _prefill_raw(K, sh, torch.tensor([0], dtype=torch.int64), {}, 0) == K.KDA_OK


def test_rectangular_heads_plan(K):
    """d_v = 2 d_k runs as twice the value heads of d_k rows (same plan as a
    square problem with 2H heads); d_k = 2 d_v pads the values and states to
    d_k rows in the workspace."""
    cu = torch.tensor([0, 300, 700], dtype=torch.int64)
    wide = K.kda_prefill_workspace_size(K.make_shape(3, 64, 128, torch.bfloat16, True), cu, 64, 64, 0)
    sq = K.kda_prefill_workspace_size(K.make_shape(6, 64, 64, torch.bfloat16, True), cu, 64, 64, 0)
    assert wide == sq
    narrow = K.kda_prefill_workspace_size(K.make_shape(3, 128, 64, torch.bfloat16, True), cu, 64, 64, 0)
    base = K.kda_prefill_workspace_size(K.make_shape(3, 128, 128, torch.bfloat16, True), cu, 64, 64, 0)
    T, H, n_snap = 700, 3, 4 + 6
    padded = T * H * 128 * 2 + T * H * 128 * 4 + (2 * 2 + n_snap) * H * 128 * 128 * 4
    assert base + padded <= narrow <= base + padded + 6 * 256
    # the backward and the layer front end need d_k = d_v
    with pytest.raises(K.KdaError) as e:
        K.kda_prefill_backward_workspace_size(K.make_shape(3, 64, 128, torch.bfloat16, True), cu)
    assert e.value.code == K.KDA_ERR_SHAPE


def test_noalloc_prefill_host_rejections(K):
    """The allocation-free prefill: argument errors and a work table larger than
    its static scratch are rejected on the host (nothing is dereferenced)."""
    lib = K.load()

    def call(sh, cu, interval=0, **kw):
        p = dict(cu_dev=0x10000000, q=0x20000000, k=0x30000000, v=0x40000000, alpha=0x50000000, beta=0x60000000,
                 init=None, o=0x70000000, fin=0x80000000, snaps=None)
        p.update(kw)
        f = lambda n: None if p[n] is None else _fake(p[n])  # noqa: E731
        cu = cu.contiguous()
        return lib.kda_prefill_chunked_noalloc(ctypes.byref(sh), cu.numel() - 1, ctypes.c_void_p(cu.data_ptr()),
                                               f("cu_dev"), 64, interval, f("q"), f("k"), f("v"), f("alpha"),
                                               f("beta"), f("init"), f("o"), f("fin"), f("snaps"), None)

    sh = K.make_shape(2, 64, 64, torch.bfloat16, True)
    cu = torch.tensor([0, 100, 300], dtype=torch.int64)
    assert call(sh, torch.tensor([0], dtype=torch.int64)) == K.KDA_OK          # no sequences
    assert call(sh, cu, q=0x20000008) == K.KDA_ERR_ALIGN
    assert call(sh, cu, fin=None) == K.KDA_ERR_ARG
    assert call(sh, cu, interval=100) == K.KDA_ERR_SHAPE
    assert call(sh, cu, o=0x30000000) == K.KDA_ERR_ARG                         # o overlaps k
    # 40000 short sequences need a work table larger than the 1 MiB scratch
    many = torch.arange(0, 40001, dtype=torch.int64)
    assert call(sh, many) == K.KDA_ERR_WORKSPACE and "scratch" in K.kda_last_error()
    # d_k = 2 d_v pads values and states in the scratch too: 3000 tokens do not fit
    narrow = K.make_shape(2, 128, 64, torch.bfloat16, True)
    assert call(narrow, torch.tensor([0, 100, 3000], dtype=torch.int64)) == K.KDA_ERR_WORKSPACE


def test_decode_host_rejections(K):
    lib = K.load()
    f = _fake

    def call(sh, batch, **kw):
        p = dict(q=0x100000, k=0x200000, v=0x300000, alpha=0x400000, beta=0x500000, state=0x600000, o=0x700000)
        p.update(kw)
        a = [None if p[n] is None else f(p[n]) for n in ("q", "k", "v", "alpha", "beta", "state", "o")]
        return lib.kda_decode_step(ctypes.byref(sh), batch, *a, None)

    bf = K.make_shape(4, 128, 128, torch.bfloat16, True)
    fp = K.make_shape(4, 128, 128, torch.float32, False)
    assert call(bf, 0) == K.KDA_OK                      # empty batch: nothing enqueued
    assert call(bf, -1) == K.KDA_ERR_ARG
    assert call(bf, 2, state=None) == K.KDA_ERR_ARG
    assert call(bf, 2, q=0x100004) == K.KDA_ERR_ALIGN     # bf16 q: 8 B
    assert call(fp, 2, q=0x100008) == K.KDA_ERR_ALIGN     # fp32 q: 16 B
    assert call(bf, 2, state=0x600008) == K.KDA_ERR_ALIGN
    assert call(bf, 2, alpha=0x400004) == K.KDA_ERR_ALIGN  # per-key alpha: 16 B
    bad = K.make_shape(4, 96, 128, torch.bfloat16, True)
    assert call(bad, 2) == K.KDA_ERR_SHAPE
    # o must not overlap the state or an input (B=2, H=4, d=128: state 512 KiB)
    assert call(bf, 2, o=0x600000 + 4096) == K.KDA_ERR_ARG and "overlaps" in K.kda_last_error()
    assert call(bf, 2, state=0x100000) == K.KDA_ERR_ARG


def test_decode_tokens_host_rejections(K):
    lib = K.load()

    def call(sh, batch, n, **kw):
        p = dict(q=0x100000, k=0x200000, v=0x300000, alpha=0x400000, beta=0x500000, state=0x600000, o=0x700000,
                 ts=None, commit=None)
        p.update(kw)
        a = [None if p[x] is None else _fake(p[x]) for x in ("q", "k", "v", "alpha", "beta", "state", "o", "ts",
                                                            "commit")]
        return lib.kda_decode_tokens(ctypes.byref(sh), batch, n, *a, None)

    bf = K.make_shape(4, 128, 128, torch.bfloat16, True)
    assert call(bf, 0, 4) == K.KDA_OK and call(bf, 3, 0) == K.KDA_OK      # nothing to do
    assert call(bf, 2, -1) == K.KDA_ERR_ARG
    assert call(bf, 2, 4, o=None) == K.KDA_ERR_ARG
    assert call(bf, 2, 4, ts=0x800008) == K.KDA_ERR_ALIGN
    assert call(bf, 2, 4, commit=0x900002) == K.KDA_ERR_ALIGN
    assert call(bf, 1 << 20, 1 << 10) == K.KDA_ERR_SHAPE


def test_layer_host_rejections(K):
    lib = K.load()
    cu = torch.tensor([0, 10, 30], dtype=torch.int64)

    def front(sh, cu_h, **kw):
        p = dict(cu_dev=0x100, xq=0x1000, xk=0x2000, xv=0x3000, w=0x4000, st_in=None, al=0x5000, bl=0x6000,
                 q=0x7000, k=0x8000, v=0x9000, a=0xA000, b=0xB000, st_out=None)
        p.update(kw)
        f = lambda n: None if p[n] is None else _fake(p[n])  # noqa: E731
        return lib.kda_layer_front(ctypes.byref(sh), cu_h.numel() - 1,
                                   cu_h.numpy().ctypes.data_as(ctypes.c_void_p), f("cu_dev"), f("xq"), f("xk"),
                                   f("xv"), f("w"), f("st_in"), f("al"), ctypes.c_float(5.0), f("bl"), f("q"),
                                   f("k"), f("v"), f("a"), f("b"), f("st_out"), None)

    pk = K.make_shape(2, 64, 64, torch.bfloat16, True)
    sc = K.make_shape(2, 64, 64, torch.bfloat16, False)
    assert front(pk, torch.tensor([0], dtype=torch.int64)) == K.KDA_OK       # no sequences
    assert front(pk, torch.tensor([1, 5], dtype=torch.int64)) == K.KDA_ERR_SHAPE
    assert front(pk, cu, xq=None) == K.KDA_ERR_ARG
    assert front(pk, cu, cu_dev=None) == K.KDA_ERR_ARG
    assert front(pk, cu, xk=0x2008) == K.KDA_ERR_ALIGN
    assert front(pk, cu, al=0x5004) == K.KDA_ERR_ALIGN                      # per-key logits: 16 B
    assert front(sc, cu, al=0x5004, xk=0x2008) == K.KDA_ERR_ALIGN
    assert "xk" in K.kda_last_error()                                        # scalar logits: 4 B is fine
    assert front(pk, cu, st_out=0xC008) == K.KDA_ERR_ALIGN
    assert front(pk, cu, q=0x1000) == K.KDA_ERR_ARG and "alias" in K.kda_last_error()
    assert front(pk, cu, st_in=0xC000, st_out=0xC000) == K.KDA_ERR_ARG

    def back(sh, n, out_dtype=K.KDA_BF16, eps=1e-6, **kw):
        p = dict(o=0x1000, g=0x2000, w=0x3000, out=0x4000)
        p.update(kw)
        f = lambda n: None if p[n] is None else _fake(p[n])  # noqa: E731
        return lib.kda_layer_back(ctypes.byref(sh), n, f("o"), f("g"), f("w"), ctypes.c_float(eps), out_dtype,
                                  f("out"), None)

    assert back(pk, 0) == K.KDA_OK
    assert back(pk, -1) == K.KDA_ERR_ARG
    assert back(pk, 4, out_dtype=99) == K.KDA_ERR_ARG
    assert back(pk, 4, eps=-1.0) == K.KDA_ERR_ARG
    assert back(pk, 4, eps=float("nan")) == K.KDA_ERR_ARG
    assert back(pk, 4, out=None) == K.KDA_ERR_ARG
    assert back(pk, 4, g=0x2004) == K.KDA_ERR_ALIGN


def test_layer_prefill_plan_and_host_rejections(K):
    lib = K.load()
    sc = K.make_shape(2, 128, 128, torch.bfloat16, False)
    pk = K.make_shape(2, 64, 64, torch.bfloat16, True)
    cu = torch.tensor([0, 1100, 1100, 1741], dtype=torch.int64)     # an empty sequence in the pack
    T, H, d = 1741, 2, 128
    # fused forms (scalar gate at d = 128, per-key gate at d = 64, bf16, every
    # non-empty sequence split): the prefill's plan and a 256-byte sink
    for shape in (sc, pk):
        pre = K.kda_prefill_workspace_size(shape, cu, 64, 0, 256)
        lay = K.kda_layer_prefill_workspace_size(shape, cu, 64, 0, 256)
        assert pre < lay <= (pre + 255) // 256 * 256 + 256
    # composed form (unsegmented, a sequence that stays whole, another form):
    # an fp32 o in the workspace
    pk128 = K.make_shape(2, 128, 128, torch.bfloat16, True)
    for shape, c, seg in ((sc, cu, 0), (sc, torch.tensor([0, 1100, 1200], dtype=torch.int64), 256), (pk, cu, 0),
                          (pk128, cu, 256)):
        pre = K.kda_prefill_workspace_size(shape, c, 64, 0, seg)
        t, dd = int(c[-1]), shape.d_v
        assert K.kda_layer_prefill_workspace_size(shape, c, 64, 0, seg) >= pre + t * H * dd * 4
    with pytest.raises(K.KdaError):
        K.kda_layer_prefill_workspace_size(K.make_shape(2, 64, 128, torch.bfloat16, False), cu)

    def call(sh, cu_h, ws_bytes=1 << 40, out_dtype=K.KDA_BF16, eps=1e-6, seg=256, **kw):
        p = dict(cu_dev=0x100, q=0x100000, k=0x200000, v=0x300000, a=0x400000, b=0x500000, s0=None,
                 g=0x600000, w=0x700000, out=0x800000, fin=0x900000, snaps=None, ws=0x10000000)
        p.update(kw)
        f = lambda n: None if p[n] is None else _fake(p[n])  # noqa: E731
        return lib.kda_layer_prefill(ctypes.byref(sh), cu_h.numel() - 1,
                                     cu_h.numpy().ctypes.data_as(ctypes.c_void_p), f("cu_dev"), 64, 0, seg,
                                     f("q"), f("k"), f("v"), f("a"), f("b"), f("s0"), f("g"), f("w"),
                                     ctypes.c_float(eps), out_dtype, f("out"), f("fin"), f("snaps"), f("ws"),
                                     ctypes.c_size_t(ws_bytes), None)

    assert call(sc, torch.tensor([0], dtype=torch.int64)) == K.KDA_OK        # no sequences
    assert call(K.make_shape(2, 128, 64, torch.bfloat16, False), cu) == K.KDA_ERR_SHAPE
    assert "d_k = d_v" in K.kda_last_error()
    assert call(sc, cu, out_dtype=99) == K.KDA_ERR_ARG
    assert call(sc, cu, eps=-1.0) == K.KDA_ERR_ARG
    assert call(sc, cu, g=None) == K.KDA_ERR_ARG
    assert call(sc, cu, w=None) == K.KDA_ERR_ARG
    assert call(sc, cu, out=None) == K.KDA_ERR_ARG and "out" in K.kda_last_error()
    assert call(sc, cu, g=0x600008) == K.KDA_ERR_ALIGN
    assert call(sc, cu, out=0x800008) == K.KDA_ERR_ALIGN
    assert call(sc, cu, out=0x600000) == K.KDA_ERR_ARG and "g_logit" in K.kda_last_error()
    assert call(sc, cu, fin=0x700000) == K.KDA_ERR_ARG and "norm_w" in K.kda_last_error()
    assert call(sc, cu, out=0x100000) == K.KDA_ERR_ARG and "alias" in K.kda_last_error()   # out over q
    assert call(sc, cu, ws_bytes=16) == K.KDA_ERR_WORKSPACE
    assert call(sc, cu, ws=None) == K.KDA_ERR_WORKSPACE
    # out in bf16 is half the size of o: an out just past q's end is fine for validation
    assert call(sc, cu, out=0x100000 + T * H * d * 2, k=0x2000000, ws_bytes=16) == K.KDA_ERR_WORKSPACE


def test_backward_host_rejections(K):
    """kda_prefill_backward: every call below fails a host check before anything is enqueued."""
    lib = K.load()
    cu = torch.tensor([0, 100, 300], dtype=torch.int64)
    sh = K.make_shape(2, 64, 64, torch.bfloat16, True)
    need = K.kda_prefill_backward_workspace_size(sh, cu)
    assert need > 0

    def call(shape, cu_h, ws_bytes, **kw):
        p = dict(cu_dev=0x100, q=0x1000000, k=0x2000000, v=0x3000000, a=0x4000000, b=0x5000000, init=None,
                 do=0x6000000, df=None, dq=0x7000000, dk=0x8000000, dv=0x9000000, da=0xA000000, db=0xB000000, di=None,
                 ws=0x10000000)
        p.update(kw)
        f = lambda n: None if p[n] is None else _fake(p[n])  # noqa: E731
        return lib.kda_prefill_backward(ctypes.byref(shape), cu_h.numel() - 1,
                                        cu_h.numpy().ctypes.data_as(ctypes.c_void_p), f("cu_dev"), f("q"), f("k"),
                                        f("v"), f("a"), f("b"), f("init"), f("do"), f("df"), f("dq"), f("dk"),
                                        f("dv"), f("da"), f("db"), f("di"), f("ws"), ws_bytes, None)

    assert call(sh, torch.tensor([0], dtype=torch.int64), 0) == K.KDA_OK              # no sequences
    assert call(sh, torch.tensor([2, 5], dtype=torch.int64), need) == K.KDA_ERR_SHAPE
    assert call(sh, cu, need, do=None) == K.KDA_ERR_ARG
    assert call(sh, cu, need, da=None) == K.KDA_ERR_ARG
    assert call(sh, cu, need, cu_dev=None) == K.KDA_ERR_ARG
    assert call(sh, cu, need, q=0x1000008) == K.KDA_ERR_ALIGN                           # 16 B
    assert call(sh, cu, need, a=0x4000004) == K.KDA_ERR_ALIGN                           # per-key alpha: 16 B
    assert call(sh, cu, need, df=0xC000008) == K.KDA_ERR_ALIGN
    assert call(sh, cu, need, di=0xD000004) == K.KDA_ERR_ALIGN
    assert call(sh, cu, need - 1) == K.KDA_ERR_WORKSPACE
    assert call(sh, cu, need, ws=None) == K.KDA_ERR_WORKSPACE
    assert "workspace" in K.kda_last_error()
    bad = K.make_shape(2, 64, 128, torch.bfloat16, True)
    assert call(bad, cu, need) == K.KDA_ERR_SHAPE
    # gradients must not overlap the inputs or each other; d_initial may only be d_final itself
    assert call(sh, cu, need, dq=0x2000000) == K.KDA_ERR_ARG and "overlaps" in K.kda_last_error()
    assert call(sh, cu, need, db=0x9000000 + 64) == K.KDA_ERR_ARG
    assert call(sh, cu, need, df=0xC000000, di=0xC000010) == K.KDA_ERR_ARG
    # the plan grows with the work: more chunks, more workspace
    more = K.kda_prefill_backward_workspace_size(sh, torch.tensor([0, 100, 300, 1000], dtype=torch.int64))
    assert more > need


def test_binding_checks_dtypes_and_shapes(K):
    """The library sees raw pointers, so the binding rejects a tensor of the
    wrong dtype or shape before any call (all checks run on CPU tensors)."""
    sh = K.make_shape(2, 64, 64, torch.bfloat16, False)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)  # noqa: E731
    o, g = f32(5, 2, 64), f32(5, 2, 64)
    out = torch.zeros((5, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="norm_w"):
        K.kda_layer_back(sh, 5, o, g, torch.zeros(64, dtype=torch.float64), 1e-6, K.KDA_BF16, out)
    with pytest.raises(TypeError, match="out"):
        K.kda_layer_back(sh, 5, o, g, f32(64), 1e-6, K.KDA_F32, out)
    with pytest.raises(ValueError, match="contiguous"):
        K.kda_layer_back(sh, 5, o.transpose(0, 1), g, f32(64), 1e-6, K.KDA_BF16, out)
    with pytest.raises(ValueError, match="norm_w"):
        K.layer_back(o, g, f32(32))
    q = torch.zeros((5, 2, 64), dtype=torch.float32)          # shape says bf16
    with pytest.raises(TypeError, match="q"):
        K.kda_decode_step(sh, 5, q, q, q, f32(5, 2), f32(5, 2), f32(5, 2, 64, 64), f32(5, 2, 64))
    qb = q.to(torch.bfloat16)
    with pytest.raises(ValueError, match="beta"):
        K.prefill_chunked(qb, qb, qb, f32(5, 2), f32(5, 3))
    # host tensors would hand host pointers to the kernels
    with pytest.raises(ValueError, match="GPU"):
        K.kda_decode_step(sh, 5, qb, qb, qb, f32(5, 2), f32(5, 2), f32(5, 2, 64, 64), f32(5, 2, 64))
    # the offsets must describe exactly the tokens given
    with pytest.raises(ValueError, match="cu_seqlens"):
        K.prefill_chunked(qb, qb, qb, f32(5, 2), f32(5, 2), cu_seqlens_host=torch.tensor([0, 2, 3]))
    with pytest.raises(ValueError, match="cu_seqlens"):
        K.prefill_chunked(qb, qb, qb, f32(5, 2), f32(5, 2), cu_seqlens=torch.tensor([0, 5]),
                          cu_seqlens_host=torch.tensor([0, 2, 5]))
    # low-level binding: state and offsets are checked against the shape
    shp = K.make_shape(2, 64, 64, torch.bfloat16, False)
    cu = torch.tensor([0, 2, 5])
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="initial_state"):
        K.kda_prefill_chunked(shp, cu, cu, qb, qb, qb, f32(5, 2), f32(5, 2), f32(1, 2, 64, 64), f32(5, 2, 64),
                              f32(2, 2, 64, 64), None, ws)
    with pytest.raises(ValueError, match="state"):
        K.kda_decode_step(shp, 5, qb, qb, qb, f32(5, 2), f32(5, 2), f32(4, 2, 64, 64), f32(5, 2, 64))


def test_input_generators_keep_fp32_under_another_default_dtype():
    from gated_delta_rule_72_amd import workloads as wl
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    try:
        w = wl.Workload("dtype_check", H=2, dk=64, dv=64, seq_lens=(9,), dtype="bf16", gate="per_key")
        li = wl.make_layer_inputs(w, "cpu")
        pi = wl.make_prefill_inputs(w, "cpu")
    finally:
        torch.set_default_dtype(old)
    for name in ("conv_w", "alpha_logit", "beta_logit", "o", "g_logit", "norm_w"):
        assert li[name].dtype == torch.float32, name
    for name in ("alpha", "beta"):
        assert pi[name].dtype == torch.float32, name


def test_binding_fails_loudly_without_library(K, monkeypatch, tmp_path):
    monkeypatch.setattr(K, "_lib", None)
    monkeypatch.setattr(K, "LIB_PATH", str(tmp_path / "missing" / "libkda.so"))
    with pytest.raises(ImportError):
        K.load()


def test_product_package_never_uses_the_oracle():
    pkg = os.path.join(ROOT, "gated_delta_rule_72_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, flags=re.M), fn
                assert "kda_oracle" not in src and "liboracle" not in src, fn


def test_backward_workspace_in_head_groups(K, monkeypatch):
    """Above the workspace budget (KDA_BACKWARD_BUDGET_BYTES, read at every
    call) the backward plans its heads in groups: a smaller workspace that
    still holds one head's plan plus its gathered inputs and gradients."""
    cu = torch.tensor([0, 1100, 1700, 1703, 1703], dtype=torch.int64)
    sh = K.make_shape(5, 64, 64, torch.bfloat16, True)
    full = K.kda_prefill_backward_workspace_size(sh, cu)
    one = K.kda_prefill_backward_workspace_size(K.make_shape(1, 64, 64, torch.bfloat16, True), cu)
    monkeypatch.setenv("KDA_BACKWARD_BUDGET_BYTES", "1")
    per_head = K.kda_prefill_backward_workspace_size(sh, cu)
    T, d = 1703, 64
    gathered = 3 * T * d * 2 + T * d * 4 + T * 4 + 4 * d * d * 4 + T * d * 4 + 4 * d * d * 4
    outs = 3 * T * d * 4 + T * d * 4 + T * 4 + 4 * d * d * 4
    assert one + gathered + outs <= per_head < full
    monkeypatch.setenv("KDA_BACKWARD_BUDGET_BYTES", str(full - 1))
    assert per_head <= K.kda_prefill_backward_workspace_size(sh, cu) < full
    monkeypatch.delenv("KDA_BACKWARD_BUDGET_BYTES")
    assert K.kda_prefill_backward_workspace_size(sh, cu) == full
