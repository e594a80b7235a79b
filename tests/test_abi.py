"""C ABI of libkcr.so on the CPU: the library loads, exports every entry
point include/kcr.h declares, passes its host self-test, and rejects bad
arguments with the documented status before touching any device. No kernel
is launched here (fake, never-dereferenced addresses are used where the
validation only inspects pointer values)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kcr.h")
LIB = os.path.join(ROOT, "kv_cache_rmsnorm_amd", "libkcr.so")

OK, NULL, SHAPE, DTYPE, ALIGN, HEADS, ALIAS, LAUNCH, DEVICE = 0, -1, -2, -3, -4, -5, -6, -7, -8
BF16, F32, F16 = 0, 1, 2
A = 1 << 20  # fake 16-byte-aligned device addresses, never dereferenced


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(kcr_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libkcr.so is not built (python kv_cache_rmsnorm_amd/build.py)")
    L = ctypes.CDLL(LIB)
    P, I64, I, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    L.kcr_rmsnorm.argtypes = [P, I64, P, P, I64, I64, I64, F, I, P]
    L.kcr_add_rmsnorm.argtypes = [P, I64, P, I64, P, P, I64, I64, I64, F, I, P]
    L.kcr_rope_kvstore.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, P, P, P, P, I64, P, P,
                                   I64, I, I, I, I, I64, I, P]
    L.kcr_rope_cos_sin.argtypes = [P, P, I64, I, D, P]
    L.kcr_rope_cos_sin_host.argtypes = [P, P, I64, I, D]
    L.kcr_decode_chain_b1.argtypes = [P, I, P, I, I, I, I, I, P, P, P, P, I64, I, I64, F, I, P]
    L.kcr_decode_chain_batch.argtypes = [P, I, I64, P, I, I, I, I, I, P, P, P, P, I64, I, I64, F, I, P]
    L.kcr_qknorm_rope_kvstore.argtypes = [P, I64, I64, P, I64, I64, P, I64, I64, P, P, F, P, P, P, P,
                                          I64, P, P, I64, I, I, I, I, I64, I, P]
    L.kcr_swiglu.argtypes = [P, I64, P, I64, P, I64, I64, I64, I, P]
    L.kcr_copy.argtypes = [P, P, I64, P]
    L.kcr_reglu.argtypes = [P, I64, P, I64, P, I64, I64, I64, I, P]
    L.kcr_clip_norm.argtypes = [P, I64, I64, P, I64, I64, I64, I, I, P, I, P, I, F, F, I, P]
    L.kcr_paged_kv_gather.argtypes = [P, I64, I, I, I, P, I64, P, I64, I64, P, P, I, P]
    L.kcr_strerror.argtypes = [I]
    L.kcr_strerror.restype = ctypes.c_char_p
    L.kcr_version.restype = ctypes.c_char_p
    return L


def test_exports_every_declared_symbol(lib):
    names = declared()
    assert {"kcr_rmsnorm", "kcr_add_rmsnorm", "kcr_rope_kvstore", "kcr_swiglu"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_host_selftest(lib):
    assert lib.kcr_selftest_host() == 0


def test_strings(lib):
    assert lib.kcr_version().startswith(b"kcr")
    for code in (OK, NULL, SHAPE, DTYPE, ALIGN, HEADS, ALIAS, LAUNCH, DEVICE):
        assert lib.kcr_strerror(code) and lib.kcr_strerror(code) != b"unknown status"


def test_rmsnorm_validation(lib):
    f = lib.kcr_rmsnorm
    assert f(A, 1536, A * 2, A * 3, 1536, 4, 1536, 1e-6, 7, None) == DTYPE
    assert f(A, 1536, A * 2, A * 3, 1536, -1, 1536, 1e-6, BF16, None) == SHAPE
    assert f(A, 1536, A * 2, A * 3, 1536, 4, 0, 1e-6, BF16, None) == SHAPE
    big = (1 << 30) + 1                                   # above KCR_NORM_MAX_D
    assert f(A, big, A * 2, A * 3, big, 4, big, 1e-6, BF16, None) == SHAPE
    # rows wider than the register-resident engine take the two-pass kernel
    assert f(A, 40000, A * 2, A * 3, 40000, 4, 40000, 1e-6, BF16, None) in (DEVICE, OK)
    assert f(A, 200000, A * 64, A * 128, 200000, 4, 200000, 1e-6, F32, None) in (DEVICE, OK)
    # binary16 storage: accepted, 2-byte element alignment
    assert f(A, 1536, A * 2, A * 3, 1536, 4, 1536, 1e-6, F16, None) in (DEVICE, OK)
    assert f(A + 1, 1536, A * 2, A * 3, 1536, 4, 1536, 1e-6, F16, None) == ALIGN
    assert f(None, 1536, None, None, 1536, 0, 1536, 1e-6, BF16, None) == OK  # no work, no launch
    assert f(None, 1536, A * 2, A * 3, 1536, 4, 1536, 1e-6, BF16, None) == NULL
    assert f(A + 1, 1536, A * 2, A * 3, 1536, 4, 1536, 1e-6, BF16, None) == ALIGN
    assert f(A + 2, 1536, A * 2, A * 3, 1536, 4, 1536, 1e-6, F32, None) == ALIGN
    # 2-byte aligned bf16 rows with an odd stride are accepted (element access)
    assert f(A + 2, 1537, A * 2, A * 3, 1536, 4, 1536, 1e-6, BF16, None) in (DEVICE, OK)
    assert f(A, 1000, A * 2, A * 3, 1536, 4, 1536, 1e-6, BF16, None) == SHAPE  # stride < d
    # y overlapping x (not exactly in place) is refused; exactly in place is allowed
    assert f(A, 1536, A * 64, A + 3072, 1536, 4, 1536, 1e-6, BF16, None) == ALIAS
    assert f(A, 1536, A * 64, A, 1536, 4, 1536, 1e-6, BF16, None) in (DEVICE, OK)


def test_add_rmsnorm_validation(lib):
    f = lib.kcr_add_rmsnorm
    assert f(A, 1536, A * 2, 1536, A * 3, A * 4, 1536, 4, 1536, 1e-6, 9, None) == DTYPE
    assert f(None, 1536, A * 2, 1536, A * 3, A * 4, 1536, 4, 1536, 1e-6, BF16, None) == NULL
    assert f(A, 1536, None, 1536, A * 3, A * 4, 1536, 4, 1536, 1e-6, BF16, None) == NULL
    assert f(A, 1536, A * 2 + 1, 1536, A * 3, A * 4, 1536, 4, 1536, 1e-6, BF16, None) == ALIGN
    assert f(A, 1536, A * 2, 1536, A * 3, A, 1536, 4, 1536, 1e-6, BF16, None) == ALIAS  # y == x
    assert f(A, 1536, A, 1536, A * 3, A * 4, 1536, 4, 1536, 1e-6, BF16, None) == ALIAS  # delta == x


def _rope(lib, **kw):
    args = dict(q=A, qts=16 * 128, qhs=128, k=A + 12 * 128 * 2, kts=16 * 128, khs=128,
                v=A + 14 * 128 * 2, vts=16 * 128, vhs=128, qo=A * 8, pos=A * 9, cos=A * 10,
                sin=A * 11, max_pos=4096, cache=A * 16, slots=A * 12, T=4, hq=12, hkv=2, hd=128,
                bs=16, nb=64, dt=BF16)
    args.update(kw)
    a = args
    return lib.kcr_rope_kvstore(a["q"], a["qts"], a["qhs"], a["k"], a["kts"], a["khs"], a["v"],
                                a["vts"], a["vhs"], a["qo"], a["pos"], a["cos"], a["sin"],
                                a["max_pos"], a["cache"], a["slots"], a["T"], a["hq"], a["hkv"],
                                a["hd"], a["bs"], a["nb"], a["dt"], None)


def test_rope_validation(lib):
    assert _rope(lib, dt=5) == DTYPE
    assert _rope(lib, hq=12, hkv=5) == HEADS
    assert _rope(lib, hd=127) == SHAPE
    assert _rope(lib, hd=24) == SHAPE            # half head (12) not a multiple of 8 bf16
    assert _rope(lib, hd=24, dt=F32) in (DEVICE, OK)  # 12 is a multiple of 4 fp32
    assert _rope(lib, hd=1024) == SHAPE
    assert _rope(lib, bs=0) == SHAPE
    assert _rope(lib, max_pos=0) == SHAPE
    assert _rope(lib, T=0, q=None, k=None, v=None) == OK
    assert _rope(lib, slots=None) == NULL
    assert _rope(lib, cos=A * 10 + 4) == ALIGN
    assert _rope(lib, qhs=129) == ALIGN
    assert _rope(lib, pos=A * 9 + 4) == ALIGN
    assert _rope(lib, qo=A + 64) == ALIAS        # q_out inside q's fused buffer
    assert _rope(lib, cache=A) == ALIAS          # cache over the inputs
    assert _rope(lib, pos=A * 8 + 64) == ALIAS   # positions inside q_out
    assert _rope(lib, slots=A * 16 + 1024) == ALIAS  # slot_mapping inside the cache
    # contiguous q may be rotated in place
    assert _rope(lib, qts=12 * 128, k=A * 3, kts=2 * 128, v=A * 4, vts=2 * 128,
                 qo=A) in (DEVICE, OK)


def test_qknorm_rope_validation(lib):
    def q(wq=A * 20, wk=A * 21, **kw):
        a = dict(q=A, qts=16 * 128, qhs=128, k=A + 12 * 128 * 2, kts=16 * 128, khs=128,
                 v=A + 14 * 128 * 2, vts=16 * 128, vhs=128, qo=A * 8, pos=A * 9, cos=A * 10,
                 sin=A * 11, max_pos=4096, cache=A * 16, slots=A * 12, T=4, hq=12, hkv=2, hd=128,
                 bs=16, nb=64, dt=BF16)
        a.update(kw)
        return lib.kcr_qknorm_rope_kvstore(a["q"], a["qts"], a["qhs"], a["k"], a["kts"], a["khs"],
                                           a["v"], a["vts"], a["vhs"], wq, wk, 1e-6, a["qo"], a["pos"],
                                           a["cos"], a["sin"], a["max_pos"], a["cache"], a["slots"],
                                           a["T"], a["hq"], a["hkv"], a["hd"], a["bs"], a["nb"],
                                           a["dt"], None)
    assert q() in (DEVICE, OK)
    assert q(dt=9) == DTYPE
    assert q(hkv=5) == HEADS
    # with no device the shared checks stop at DEVICE before the weight checks;
    # with a device present the weight errors below are reported
    assert q(wq=None) in (DEVICE, NULL)
    assert q(wk=A * 21 + 4) in (DEVICE, ALIGN)
    assert q(T=0, wq=None, wk=None) == OK


def test_swiglu_validation(lib):
    f = lib.kcr_swiglu
    I = 8960
    assert f(A, 2 * I, A + 2 * I, 2 * I, A * 64, I, 4, I, 3, None) == DTYPE
    assert f(A, 2 * I, A + 2 * I, 2 * I, A * 64, I, 4, 0, BF16, None) == SHAPE
    assert f(A, 2 * I, A + 2 * I, 2 * I, A * 64, I, 1 << 30, I, BF16, None) == SHAPE  # > 2^31 vectors
    assert f(A, 2 * I, A + 2 * I, 2 * I, None, I, 4, I, BF16, None) == NULL
    assert f(A, 2 * I, A + 2 * I + 1, 2 * I, A * 64, I, 4, I, BF16, None) == ALIGN
    # output into the gate half of the fused buffer: exact, allowed
    assert f(A, 2 * I, A + 2 * I, 2 * I, A, 2 * I, 4, I, BF16, None) in (DEVICE, OK)
    # output overlapping the up half with a shifted row: refused
    assert f(A, 2 * I, A + 2 * I, 2 * I, A + 16, 2 * I, 4, I, BF16, None) == ALIAS
    # fused halves as inputs, separate output: fine
    assert f(A, 2 * I, A + 2 * I, 2 * I, A * 64, I, 4, I, BF16, None) in (DEVICE, OK)


def test_gather_validation(lib):
    f = lib.kcr_paged_kv_gather
    # cache, blocks, bs, hkv, hd, tables, max blocks/seq, lens, seqs, max_len, k_out, v_out, dtype
    ok = dict(c=A, nb=64, bs=16, hkv=2, hd=128, bt=A * 2, mb=8, ln=A * 3, n=4, ml=128, k=A * 4,
              v=A * 5, dt=BF16)

    def g(**kw):
        a = dict(ok, **kw)
        return f(a["c"], a["nb"], a["bs"], a["hkv"], a["hd"], a["bt"], a["mb"], a["ln"], a["n"],
                 a["ml"], a["k"], a["v"], a["dt"], None)
    assert g() in (DEVICE, OK)
    assert g(dt=7) == DTYPE
    assert g(hkv=1, hd=4) == SHAPE             # 4 bf16 per row: not a 16-byte multiple
    assert g(ml=129) == SHAPE                  # more positions than the table can name
    assert g(n=0, c=None, bt=None) == OK
    assert g(ln=None) == NULL
    assert g(k=A * 4 + 8) == ALIGN
    assert g(bt=A * 2 + 4) == ALIGN
    assert g(v=A * 4) == ALIAS
    assert g(k=A + 64) == ALIAS                # output over the cache


def test_reglu_validation(lib):
    f = lib.kcr_reglu
    I = 8960
    assert f(A, 2 * I, A + 2 * I, 2 * I, A * 64, I, 4, I, 3, None) == DTYPE
    assert f(A, 2 * I, A + 2 * I, 2 * I, None, I, 4, I, BF16, None) == NULL
    assert f(A, 2 * I, A + 2 * I, 2 * I, A + 16, 2 * I, 4, I, BF16, None) == ALIAS
    assert f(A, 2 * I, A + 2 * I, 2 * I, A * 64, I, 4, I, BF16, None) in (DEVICE, OK)


def test_clip_norm_validation(lib):
    f = lib.kcr_clip_norm
    base = dict(x=A, xts=2048, xhs=128, y=A * 8, yts=1536, yhs=128, n=4, h=12, d=128, a=A * 9, apc=1,
                g=A * 10, gpc=0, lo=-1.0, hi=1.0, dt=BF16)

    def c(**kw):
        a = dict(base, **kw)
        return f(a["x"], a["xts"], a["xhs"], a["y"], a["yts"], a["yhs"], a["n"], a["h"], a["d"],
                 a["a"], a["apc"], a["g"], a["gpc"], a["lo"], a["hi"], a["dt"], None)
    assert c() in (DEVICE, OK)
    assert c(dt=7) == DTYPE
    assert c(lo=1.0, hi=-1.0) == SHAPE
    assert c(xhs=100) == SHAPE                     # head stride below the head width
    assert c(a=None) == NULL
    assert c(x=A + 1) == ALIGN
    assert c(y=A + 256) == ALIAS                   # output inside the strided input view
    assert c(y=A, yts=2048, yhs=128) in (DEVICE, OK)   # exactly in place
    assert c(n=0, x=None, y=None) == OK


def test_copy_validation(lib):
    assert lib.kcr_copy(A * 2, A, 17, None) == SHAPE
    assert lib.kcr_copy(A * 2, A + 8, 32, None) == ALIGN
    assert lib.kcr_copy(A + 16, A, 64, None) == ALIAS
    assert lib.kcr_copy(None, None, 0, None) == OK


def test_binding_refuses_missing_library(tmp_path):
    # The binding must fail loudly rather than fall back when the HIP library
    # is absent: load its source against an empty directory.
    import importlib.util
    src = os.path.join(ROOT, "kv_cache_rmsnorm_amd", "__init__.py")
    fake_pkg = tmp_path / "kcr_missing"
    fake_pkg.mkdir()
    (fake_pkg / "__init__.py").write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("kcr_missing", fake_pkg / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError):
        spec.loader.exec_module(mod)


def test_rope_cos_sin_host_values(lib):
    """The host table builder runs on the CPU: every entry is cos/sin of the
    fp64 angle p * theta^(-2i/d) rounded once to fp32. Checked exactly
    against Python's math module (the same fp64 operations) on a sample and
    against numpy over the whole table to within one fp32 ulp."""
    import math
    import numpy as np
    max_pos, hd, theta = 4097, 128, 1e6
    half = hd // 2
    c = np.empty((max_pos, half), dtype=np.float32)
    s_ = np.empty_like(c)
    assert lib.kcr_rope_cos_sin_host(c.ctypes.data, s_.ctypes.data, max_pos, hd, theta) == 0
    assert np.all(c[0] == 1.0) and np.all(s_[0] == 0.0)          # position 0: the identity
    for p in (1, 2, 37, 1000, 4096):
        for i in (0, 1, 31, 63):
            ang = p * math.pow(theta, -2.0 * i / hd)
            assert c[p, i] == np.float32(math.cos(ang)) and s_[p, i] == np.float32(math.sin(ang)), (p, i)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * np.power(theta, -2.0 * np.arange(half) / hd)[None, :]
    for got, ref in ((c, np.cos(ang).astype(np.float32)), (s_, np.sin(ang).astype(np.float32))):
        ulp = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1 and (ulp > 0).mean() < 1e-4
    assert np.allclose(c.astype(np.float64) ** 2 + s_.astype(np.float64) ** 2, 1.0, atol=3e-7)


def test_rope_cos_sin_host_errors(lib):
    import numpy as np
    c = np.empty((8, 4), dtype=np.float32)
    s_ = np.empty_like(c)
    assert lib.kcr_rope_cos_sin_host(c.ctypes.data, s_.ctypes.data, -1, 8, 1e4) == SHAPE
    assert lib.kcr_rope_cos_sin_host(c.ctypes.data, s_.ctypes.data, 8, 7, 1e4) == SHAPE
    assert lib.kcr_rope_cos_sin_host(c.ctypes.data, s_.ctypes.data, 8, 8, 0.0) == SHAPE
    assert lib.kcr_rope_cos_sin_host(c.ctypes.data, s_.ctypes.data, 8, 8, float("nan")) == SHAPE
    assert lib.kcr_rope_cos_sin_host(None, s_.ctypes.data, 8, 8, 1e4) == NULL
    assert lib.kcr_rope_cos_sin_host(c.ctypes.data, c.ctypes.data + 16, 8, 8, 1e4) == ALIAS
    assert lib.kcr_rope_cos_sin_host(None, None, 0, 8, 1e4) == OK
    assert lib.kcr_rope_cos_sin(None, None, 8, 8, -1.0, None) == SHAPE


def test_decode_chain_b1_validation(lib):
    """Host-side checks of the one-launch batch-1 chain: sizes, counts and the
    layer table are refused before anything is launched (no device here, so
    a call that passes every check reports DEVICE)."""
    import ctypes
    A = 1 << 20
    f = lib.kcr_decode_chain_b1

    class Layer(ctypes.Structure):
        _fields_ = [(f"p{i}", ctypes.c_void_p) for i in range(11)]

    def table(n, base=1 << 30, step=1 << 22):
        arr = (Layer * n)()
        for i in range(n):
            arr[i] = Layer(*[base + (i * 11 + j) * step for j in range(11)])
        return arr

    H = 1 << 34  # far from every table pointer

    def call(layers=None, n=2, h=H, hidden=1536, inter=8960, hq=12, hkv=2, hd=128, pos=H + A,
             slot=H + A + 64, cos=H + 2 * A, sin=H + 8 * A, max_pos=4097, bs=16, nb=64, dt=BF16):
        t = table(max(n, 1)) if layers is None else layers
        return f(ctypes.cast(t, ctypes.c_void_p), n, h, hidden, inter, hq, hkv, hd, pos, slot, cos, sin,
                 max_pos, bs, nb, 1e-6, dt, None)

    assert call() == DEVICE
    assert call(n=33) == SHAPE                       # more layers than the argument block holds
    assert call(n=0, h=None) == OK                   # no work
    assert call(hidden=1537) == SHAPE                # not whole 16-byte vectors
    assert call(hidden=8 * 1025) == SHAPE            # more vectors than lanes
    assert call(inter=8 * 4097) == SHAPE
    assert call(hq=12, hkv=5) == HEADS
    assert call(hd=120) == SHAPE                     # half a head not whole vectors
    assert call(dt=7) == DTYPE
    assert call(h=None) == NULL
    assert call(h=H + 2) == ALIGN
    bad = table(2)
    bad[1].p3 = None                                 # layer 1 without qkv
    assert call(layers=bad) == NULL
    bad = table(2)
    bad[0].p0 = (1 << 30) + 8                        # misaligned d_attn
    assert call(layers=bad) == ALIGN
    bad = table(2)
    bad[0].p2 = bad[0].p0                            # y_attn on top of d_attn
    assert call(layers=bad) == ALIAS


def test_decode_chain_batch_validation(lib):
    """Host-side checks of the one-launch chain over a batch: the batch's
    range, and aliasing over the whole batch's rows (a y_attn on row 3 of
    d_attn is refused at batch 4 and accepted at batch 2)."""
    import ctypes
    A = 1 << 20
    f = lib.kcr_decode_chain_batch

    class Layer(ctypes.Structure):
        _fields_ = [(f"p{i}", ctypes.c_void_p) for i in range(11)]

    def table(n, base=1 << 30, step=1 << 22):
        arr = (Layer * n)()
        for i in range(n):
            arr[i] = Layer(*[base + (i * 11 + j) * step for j in range(11)])
        return arr

    H = 1 << 34

    def call(batch, layers=None, n=2, h=H, hidden=1536):
        t = table(max(n, 1)) if layers is None else layers
        return f(ctypes.cast(t, ctypes.c_void_p), n, batch, h, hidden, 8960, 12, 2, 128, H + A, H + A + 64,
                 H + 2 * A, H + 8 * A, 4097, 16, 64, 1e-6, BF16, None)

    assert call(4) == DEVICE
    assert call(1) == DEVICE
    assert call(-1) == SHAPE
    assert call(1 << 20) == SHAPE                     # the grid's lanes would pass 2^32
    assert call(1 << 22) == SHAPE
    assert call(0, h=None) == OK                      # no tokens, no work
    assert call(4, hidden=1537) == SHAPE
    bad = table(2)
    bad[0].p2 = bad[0].p0 + 3 * 1536 * 2              # y_attn = row 3 of d_attn
    assert call(4, layers=bad) == ALIAS
    assert call(2, layers=bad) == DEVICE
    assert call(4, h=H + A - 2 * 1536 * 2) == ALIAS   # h's last rows over positions


def test_decode_chain_cross_layer_alias(lib):
    """A buffer one layer of the one-launch chain writes may not overlap any
    buffer of another layer (the chain reads each layer's inputs ahead of
    the previous layer's ops): refused with ALIAS before any launch. Shared
    inputs (weights, even every input) and one cache named by several layers
    stay allowed."""
    import ctypes
    f = lib.kcr_decode_chain_batch

    class Layer(ctypes.Structure):
        _fields_ = [(f"p{i}", ctypes.c_void_p) for i in range(11)]

    def table(n, base=1 << 30, step=1 << 22):
        arr = (Layer * n)()
        for i in range(n):
            arr[i] = Layer(*[base + (i * 11 + j) * step for j in range(11)])
        return arr

    H = 1 << 34
    # pointer roles in kcr_chain_layer order
    D_ATTN, W_ATTN, Y_ATTN, QKV, Q_OUT, CACHE, D_MLP, W_MLP, Y_MLP, GATE_UP, ACT = range(11)

    def call(layers, n=3, batch=4):
        return f(ctypes.cast(layers, ctypes.c_void_p), n, batch, H, 1536, 8960, 12, 2, 128, H + A,
                 H + A + 64, H + 2 * A, H + 8 * A, 4097, 16, 64, 1e-6, BF16, None)

    def with_(l, role, other_l, other_role, off=0):
        t = table(3)
        setattr(t[l], f"p{role}", getattr(t[other_l], f"p{other_role}") + off)
        return t

    assert call(table(3)) == DEVICE
    # layer 0's act read back as layer 1's d_attn / qkv / gate_up
    assert call(with_(1, D_ATTN, 0, ACT)) == ALIAS
    assert call(with_(2, QKV, 0, Y_MLP)) == ALIAS
    assert call(with_(1, GATE_UP, 0, Q_OUT, off=1024)) == ALIAS
    # layer 1 writing over an input of layer 0 (a later layer's output)
    assert call(with_(0, D_MLP, 1, Y_ATTN)) == ALIAS
    # two layers writing one output buffer, or an output over another layer's cache
    assert call(with_(1, Y_ATTN, 0, Y_ATTN)) == ALIAS
    assert call(with_(2, ACT, 0, CACHE, off=4096)) == ALIAS
    # the same range on a later row only: refused at batch 4, not at batch 1
    row = 1536 * 2
    assert call(with_(1, D_ATTN, 0, Y_MLP, off=3 * row)) == ALIAS
    assert call(with_(1, D_ATTN, 0, Y_MLP, off=3 * row), batch=1) == DEVICE
    # shared inputs: one weight pair for all layers, one gate_up for two layers
    t = table(3)
    for i in range(3):
        t[i].p1, t[i].p7 = t[0].p1, t[0].p1
    t[2].p9 = t[1].p9
    assert call(t) == DEVICE
    # a cache shared by every layer, but not a cache that only partly overlaps
    t = table(3)
    t[1].p5 = t[2].p5 = t[0].p5
    assert call(t) == DEVICE
    assert call(with_(1, CACHE, 0, CACHE, off=4096)) == ALIAS
    # the same checks through the batch-1 entry point
    assert lib.kcr_decode_chain_b1(ctypes.cast(with_(1, D_ATTN, 0, ACT), ctypes.c_void_p), 3, H, 1536, 8960,
                                   12, 2, 128, H + A, H + A + 64, H + 2 * A, H + 8 * A, 4097, 16, 64, 1e-6,
                                   BF16, None) == ALIAS


def test_build_refuses_scratch():
    """The build fails on any kernel that uses scratch memory (a register
    spill, or the argument block copied to private memory). Its check reads
    hipcc's resource-usage remarks; here, two remark excerpts in that form."""
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "kcr_build", os.path.join(os.path.dirname(__file__), "..", "kv_cache_rmsnorm_amd", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    remarks = [
        "a.hip:9:1: remark: Function Name: _Z3fooIiEvv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:9:1: remark:     ScratchSize [bytes/lane]: 2968 [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:20:1: remark: Function Name: _Z3barv [-Rpass-analysis=kernel-resource-usage]",
        "a.hip:20:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
    ]
    assert build.scratch_users(remarks) == ["_Z3fooIiEvv"]
    assert build.scratch_users(remarks[2:]) == []
