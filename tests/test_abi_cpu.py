"""C-ABI library on the CPU: it loads, exports every declared symbol, and rejects
invalid arguments on the host before any HIP call (no compute without a GPU)."""

import ctypes
import os
import re

import pytest

from sparse_long_sequence_longformer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lf_attn.h")

needs_lib = pytest.mark.skipif(not os.path.exists(binding.library_path()),
                               reason="liblfattn.so not built (run __graft_entry__.build())")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(lf_(?:attn|layer)_\w+)\s*\(", text)))


def test_header_declares_binding_exports():
    assert declared_symbols() == sorted(binding.EXPORTS)


def test_stage_names_match_header():
    text = open(HEADER).read()
    n = int(re.search(r"#define LF_N_STAGES (\d+)", text).group(1))
    ids = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define LF_STAGE_(\w+) (\d+)", text)}
    assert n == binding.N_STAGES == len(binding.STAGE_NAMES) == len(ids)
    assert sorted(ids.values()) == list(range(n))
    for name, i in ids.items():
        assert binding.STAGE_NAMES[i] == name.lower(), (name, i)


@needs_lib
def test_library_exports_every_symbol():
    lib = ctypes.CDLL(binding.library_path())
    for name in declared_symbols():
        assert hasattr(lib, name), name


@needs_lib
def test_status_strings():
    lib = binding.load_library()
    for code in range(5):
        assert lib.lf_attn_status_string(code)
    assert lib.lf_attn_status_string(77) == b"unknown status"


@needs_lib
def test_create_destroy_and_bad_dtype():
    lib = binding.load_library()
    h = ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h), 5) == 2  # LF_ERR_UNSUPPORTED
    assert lib.lf_attn_create(None, 1) == 1
    assert lib.lf_attn_create(ctypes.byref(h), 1) == 0 and h.value
    assert lib.lf_attn_last_error(h) == b""
    assert lib.lf_attn_set_stage_timing(h, 1) == 0
    ms = (ctypes.c_double * binding.N_STAGES)()
    n = (ctypes.c_int64 * binding.N_STAGES)()
    assert lib.lf_attn_stage_times(h, ms, n) == 0 and list(n) == [0] * binding.N_STAGES
    assert lib.lf_attn_destroy(h) == 0
    assert lib.lf_attn_destroy(None) == 0


FAKE = 1 << 20  # 16-byte aligned, never dereferenced: validation fails first


def _call(h, **kw):
    lib = binding.load_library()
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, out=FAKE * 4, B=1, H=2, L=64, d_h=64, w=4,
             dil=[1, 2], g=[], ng=None, pad=None)
    a.update(kw)
    dil = a["dil"]
    dil_p = (ctypes.c_int32 * len(dil))(*dil) if dil is not None else None
    g = a["g"]
    g_p = (ctypes.c_int32 * len(g))(*g) if g else None
    ng = len(g) if a["ng"] is None else a["ng"]
    st = lib.lf_attn_forward(h, a["q"], a["k"], a["v"], a["out"], a["B"], a["H"], a["L"], a["d_h"], a["w"],
                             ctypes.cast(dil_p, ctypes.POINTER(ctypes.c_int32)) if dil_p else None,
                             ctypes.cast(g_p, ctypes.POINTER(ctypes.c_int32)) if g_p else None,
                             ng, a["pad"], None)
    return st, lib.lf_attn_last_error(h).decode()


@needs_lib
@pytest.mark.parametrize("kw,code,frag", [
    (dict(q=None), 1, "non-null"),
    (dict(out=None), 1, "non-null"),
    (dict(B=0), 1, "B, H, L"),
    (dict(L=0), 1, "B, H, L"),
    (dict(d_h=32), 2, "d_h"),
    (dict(H=65, dil=[1] * 65), 2, "heads"),
    (dict(w=-1), 1, "w >= 0"),
    (dict(dil=None), 1, "dil_per_head"),
    (dict(dil=[1, 0]), 1, "dil_per_head[1]"),
    (dict(g=[3, 64]), 1, "outside"),
    (dict(g=[-1]), 1, "outside"),
    (dict(g=[], ng=2), 1, "global_idx is NULL"),
    (dict(g=[], ng=-1), 1, "n_global"),
    (dict(g=list(range(64)) * 5), 2, "at most"),
    (dict(q=FAKE + 8), 1, "aligned"),
    (dict(out=FAKE * 3 + 64), 1, "overlap"),
])
def test_invalid_arguments_rejected_on_host(kw, code, frag):
    lib = binding.load_library()
    h = ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h), 1) == 0
    try:
        st, msg = _call(h, **kw)
        assert st == code, (st, msg)
        assert frag in msg, msg
        # the handle stays usable after an error
        st2, _ = _call(h, B=0)
        assert st2 == 1
    finally:
        lib.lf_attn_destroy(h)


def _call_gp(h, qg=FAKE * 5, kg=FAKE * 6, vg=FAKE * 7, out=FAKE * 4):
    lib = binding.load_library()
    dil = (ctypes.c_int32 * 2)(1, 2)
    g = (ctypes.c_int32 * 1)(3)
    st = lib.lf_attn_forward_global_proj(h, FAKE, FAKE * 2, FAKE * 3, qg, kg, vg, out, 1, 2, 64, 64, 4,
                                         ctypes.cast(dil, ctypes.POINTER(ctypes.c_int32)),
                                         ctypes.cast(g, ctypes.POINTER(ctypes.c_int32)), 1, None, None)
    return st, lib.lf_attn_last_error(h).decode()


@needs_lib
@pytest.mark.parametrize("kw,frag", [
    (dict(qg=None), "non-null"),
    (dict(kg=None), "non-null"),
    (dict(vg=None), "non-null"),
    (dict(kg=FAKE * 6 + 4), "aligned"),
    (dict(out=FAKE * 7 + 1024), "overlap q_g, k_g or v_g"),
])
def test_global_proj_invalid_arguments(kw, frag):
    lib = binding.load_library()
    h = ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h), 1) == 0
    try:
        st, msg = _call_gp(h, **kw)
        assert st == 1 and frag in msg, (st, msg)
    finally:
        lib.lf_attn_destroy(h)


@needs_lib
def test_backward_host_validation():
    lib = binding.load_library()
    dil = (ctypes.c_int32 * 1)(1)
    dil_p = ctypes.cast(dil, ctypes.POINTER(ctypes.c_int32))

    def call(h, lse=FAKE * 9, dq=FAKE * 10, dk=FAKE * 11, dv=FAKE * 12, out=FAKE * 4):
        st = lib.lf_attn_backward(h, FAKE, FAKE * 2, FAKE * 3, out, FAKE * 5, lse, dq, dk, dv, 1, 1, 64, 64, 4,
                                  dil_p, None, 0, None, None)
        return st, lib.lf_attn_last_error(h).decode()

    h32, h16 = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h32), 0) == 0 and lib.lf_attn_create(ctypes.byref(h16), 1) == 0
    try:
        for h in (h16, h32):  # both dtypes run the same validation
            for kw, frag in [(dict(lse=None), "non-null"), (dict(dv=None), "non-null"),
                             (dict(lse=FAKE * 9 + 2), "aligned"), (dict(dq=FAKE * 10 + 8), "aligned"),
                             (dict(dk=FAKE * 10 + 4096), "overlap"), (dict(dq=FAKE * 2 + 1024), "overlap"),
                             (dict(dv=FAKE * 9 - 16), "overlap")]:
                st, msg = call(h, **kw)
                assert st == 1 and frag in msg, (kw, st, msg)
        st = lib.lf_attn_forward_lse(h16, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, None, 1, 1, 64, 64, 4, dil_p, None, 0,
                                     None, None)
        assert st == 1
        st = lib.lf_attn_forward_lse(h16, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 3 + 64, 1, 1, 64, 64, 4, dil_p,
                                     None, 0, None, None)
        assert st == 1 and "lse must not overlap" in lib.lf_attn_last_error(h16).decode()
    finally:
        lib.lf_attn_destroy(h32)
        lib.lf_attn_destroy(h16)


@needs_lib
def test_window_mode():
    lib = binding.load_library()
    h = ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h), 1) == 0
    try:
        assert lib.lf_attn_set_window_mode(h, binding.LF_WINDOW_CAUSAL) == 0
        assert lib.lf_attn_set_window_mode(h, binding.LF_WINDOW_SYMMETRIC) == 0
        assert lib.lf_attn_set_window_mode(h, 7) == 1
        assert b"window mode" in lib.lf_attn_last_error(h)
        assert lib.lf_attn_set_window_mode(None, 0) == 1
    finally:
        lib.lf_attn_destroy(h)


@needs_lib
def test_layer_host_validation():
    lib = binding.load_library()
    dil = (ctypes.c_int32 * 12)(*([1] * 12))
    dil_p = ctypes.cast(dil, ctypes.POINTER(ctypes.c_int32))
    ok = binding.LayerWeights(*[FAKE * (20 + i) for i in range(len(binding.LAYER_WEIGHTS))])

    def call(h, wts=ok, hidden=768, ffn=3072, x=FAKE, out=FAKE * 2, eps=1e-5):
        st = lib.lf_layer_forward(h, x, ctypes.byref(wts) if wts is not None else None, out, 1, 64, hidden, ffn,
                                  eps, 4, dil_p, None, 0, None, None)
        return st, lib.lf_attn_last_error(h).decode()

    h32, h16 = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h32), 0) == 0 and lib.lf_attn_create(ctypes.byref(h16), 1) == 0
    try:
        st, msg = call(h32)
        assert st == 2 and "bf16" in msg
        bad = binding.LayerWeights(*[FAKE * (20 + i) for i in range(len(binding.LAYER_WEIGHTS))])
        bad.w_o = None
        for kw, code, frag in [(dict(hidden=100), 2, "hidden"), (dict(hidden=4096), 2, "hidden"),
                               (dict(ffn=12), 2, "ffn"), (dict(wts=None), 1, "non-null"),
                               (dict(wts=bad), 1, "weight"), (dict(x=FAKE + 8), 1, "aligned"),
                               (dict(out=FAKE + 4096), 1, "overlap"), (dict(eps=-1.0), 1, "ln_eps")]:
            st, msg = call(h16, **kw)
            assert st == code and frag in msg, (kw, st, msg)
    finally:
        lib.lf_attn_destroy(h32)
        lib.lf_attn_destroy(h16)


@needs_lib
def test_global_mode_validation():
    lib = binding.load_library()
    h = ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h), 1) == 0
    try:
        assert lib.lf_attn_set_global_mode(h, 5) == 1 and b"global mode" in lib.lf_attn_last_error(h)
        assert lib.lf_attn_set_global_mode(h, binding.LF_GLOBALS_PER_SEQUENCE) == 0
        dil = (ctypes.c_int32 * 2)(1, 2)
        dil_p = ctypes.cast(dil, ctypes.POINTER(ctypes.c_int32))

        def call(B, rows, n):
            flat = [x for r in rows for x in r]
            arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
            st = lib.lf_attn_forward(h, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, B, 2, 64, 64, 4, dil_p,
                                     ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), n, None, None)
            return st, lib.lf_attn_last_error(h).decode()

        st, msg = call(2, [[1, 64], [0, -1]], 2)
        assert st == 1 and "global_idx[0][1]" in msg, msg
        st, msg = call(3, [list(range(100))] * 3, 100)
        assert st == 2 and "per-sequence" in msg, msg
        assert lib.lf_attn_set_global_mode(None, 0) == 1
    finally:
        lib.lf_attn_destroy(h)


@needs_lib
def test_tile_rows_validation():
    lib = binding.load_library()
    h = ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h), 1) == 0
    try:
        for rows in (0, 64, 128, 0):
            assert lib.lf_attn_set_tile_rows(h, rows) == 0, rows
        for rows in (-1, 32, 96, 256):
            assert lib.lf_attn_set_tile_rows(h, rows) == 1 and b"tile rows" in lib.lf_attn_last_error(h), rows
        assert lib.lf_attn_set_tile_rows(None, 64) == 1
    finally:
        lib.lf_attn_destroy(h)


@needs_lib
def test_null_handle():
    lib = binding.load_library()
    assert lib.lf_attn_forward(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 64, 0, None, None, 0, None, None) == 1
    assert lib.lf_attn_last_error(None) == b""
    assert lib.lf_attn_forward_global_proj(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 64, 0,
                                           None, None, 0, None, None) == 1


def test_python_forward_requires_device_tensors():
    import torch

    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises((ValueError, binding.LfAttnError)):
        binding.forward(x, x, x, 2, [1])


@needs_lib
def test_position_bias_validation():
    lib = binding.load_library()
    h = ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h), 1) == 0
    try:
        err = lambda: lib.lf_attn_last_error(h).decode()  # noqa: E731
        assert lib.lf_attn_set_position_bias(None, FAKE, 2, 4) == 1
        assert lib.lf_attn_set_position_bias(h, FAKE, 0, 4) == 1 and "n_heads" in err()
        assert lib.lf_attn_set_position_bias(h, FAKE, 65, 4) == 1 and "n_heads" in err()
        assert lib.lf_attn_set_position_bias(h, FAKE, 2, -1) == 1 and "w >= 0" in err()
        assert lib.lf_attn_set_position_bias(h, FAKE, 2, binding.MAX_BIAS_W + 1) == 2 and "at most" in err()
        assert lib.lf_attn_set_position_bias(h, FAKE + 2, 2, 4) == 1 and "aligned" in err()
        # a table for H = 2, w = 4: calls with another H or w are refused before any launch
        assert lib.lf_attn_set_position_bias(h, FAKE * 5, 2, 4) == 0
        dil = (ctypes.c_int32 * 3)(1, 1, 1)
        dil_p = ctypes.cast(dil, ctypes.POINTER(ctypes.c_int32))

        def call(H, w):
            return lib.lf_attn_forward(h, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1, H, 64, 64, w, dil_p, None, 0,
                                       None, None)

        assert call(3, 4) == 1 and "bias table is for H = 2, w = 4" in err()
        assert call(2, 5) == 1 and "bias table" in err()
        # removing the table lifts the restriction (the call then fails later, on the device)
        assert lib.lf_attn_set_position_bias(h, None, 0, 0) == 0
        assert "bias" not in err()
    finally:
        lib.lf_attn_destroy(h)


@needs_lib
def test_random_blocks_validation():
    lib = binding.load_library()
    h = ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h), 1) == 0
    try:
        err = lambda: lib.lf_attn_last_error(h).decode()  # noqa: E731

        def arr(vals):
            a = (ctypes.c_int32 * max(1, len(vals)))(*vals)
            return ctypes.cast(a, ctypes.POINTER(ctypes.c_int32)), a

        good, keep = arr([1, -1, 0, 0, 1, 1, -5, 0])  # H = 2, 2 query blocks, r = 2
        assert lib.lf_attn_set_random_blocks(None, good, 2, 2, 2) == 1
        assert lib.lf_attn_set_random_blocks(h, good, 0, 2, 2) == 1 and "n_heads" in err()
        assert lib.lf_attn_set_random_blocks(h, good, 2, 0, 2) == 1 and "n_qblocks" in err()
        assert lib.lf_attn_set_random_blocks(h, good, 2, 2, -1) == 1 and "r >= 0" in err()
        assert lib.lf_attn_set_random_blocks(h, good, 2, 2, binding.MAX_RANDOM_DRAWS + 1) == 2
        bad, keep2 = arr([1, 2, 0, 0, 1, 1, 0, 0])
        st = lib.lf_attn_set_random_blocks(h, bad, 2, 2, 2)
        assert st == 1 and "outside [0, 2)" in err(), err()
        assert lib.lf_attn_set_random_blocks(h, good, 2, 2, 2) == 0
        dil = (ctypes.c_int32 * 3)(1, 1, 1)
        dil_p = ctypes.cast(dil, ctypes.POINTER(ctypes.c_int32))

        def call(H, L, d=None):
            dp = dil_p if d is None else ctypes.cast((ctypes.c_int32 * H)(*d), ctypes.POINTER(ctypes.c_int32))
            return lib.lf_attn_forward(h, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, 1, H, L, 64, 8, dp, None, 0, None, None)

        assert call(3, 128) == 1 and "random blocks are for H = 2" in err()
        assert call(2, 129) == 1 and "L = 129 gives 3" in err(), err()
        assert call(2, 128, [1, 2]) == 2 and "undilated" in err()
        st = lib.lf_attn_backward(h, FAKE, FAKE * 2, FAKE * 3, FAKE * 4, FAKE * 5, FAKE * 6, FAKE * 7, FAKE * 8,
                                  FAKE * 9, 1, 3, 128, 64, 8, dil_p, None, 0, None, None)
        assert st == 1 and "random blocks are for H = 2" in err(), err()
        assert lib.lf_attn_set_random_blocks(h, None, 0, 0, 0) == 0
    finally:
        lib.lf_attn_destroy(h)


@needs_lib
def test_global_proj_backward_host_validation():
    lib = binding.load_library()
    dil = (ctypes.c_int32 * 1)(1)
    dil_p = ctypes.cast(dil, ctypes.POINTER(ctypes.c_int32))
    # inputs q, k, v, q_g, k_g, v_g, out, dout at FAKE * 1..8; lse at FAKE * 9;
    # gradients dq, dk, dv, dq_g, dk_g, dv_g at FAKE * 10..15
    names = ("dq", "dk", "dv", "dqg", "dkg", "dvg")

    def call(h, lse=FAKE * 9, **kw):
        grads = [kw.get(n, FAKE * (10 + i)) for i, n in enumerate(names)]
        ins = [kw.get(n, FAKE * (1 + i)) for i, n in enumerate(("q", "k", "v", "qg", "kg", "vg", "out", "dout"))]
        st = lib.lf_attn_backward_global_proj(h, *ins, lse, *grads, 1, 1, 64, 64, 4, dil_p, None, 0, None, None)
        return st, lib.lf_attn_last_error(h).decode()

    h32, h16 = ctypes.c_void_p(), ctypes.c_void_p()
    assert lib.lf_attn_create(ctypes.byref(h32), 0) == 0 and lib.lf_attn_create(ctypes.byref(h16), 1) == 0
    try:
        for h in (h16, h32):  # both dtypes run the same validation
            for kw, frag in [(dict(qg=None), "must all be non-null"), (dict(dvg=None), "must all be non-null"),
                             (dict(lse=None), "non-null"), (dict(kg=FAKE * 5 + 4), "aligned"),
                             (dict(dqg=FAKE * 13 + 8), "aligned"), (dict(dkg=FAKE * 6 + 64), "overlap the inputs"),
                             (dict(dvg=FAKE * 10 + 4096), "must not overlap"), (dict(dqg=FAKE * 9 - 32), "overlap")]:
                st, msg = call(h, **kw)
                assert st == 1 and frag in msg, (kw, st, msg)
        assert lib.lf_attn_backward_global_proj(None, *([FAKE] * 15), 1, 1, 64, 64, 4, dil_p, None, 0, None,
                                                None) == 1
        # the forward that returns the statistics: lse must be given and clear of q_g
        st = lib.lf_attn_forward_global_proj_lse(h16, FAKE, FAKE * 2, FAKE * 3, FAKE * 5, FAKE * 6, FAKE * 7,
                                                 FAKE * 4, None, 1, 1, 64, 64, 4, dil_p, None, 0, None, None)
        assert st == 1 and "non-null" in lib.lf_attn_last_error(h16).decode()
        st = lib.lf_attn_forward_global_proj_lse(h16, FAKE, FAKE * 2, FAKE * 3, FAKE * 5, FAKE * 6, FAKE * 7,
                                                 FAKE * 4, FAKE * 6 + 256, 1, 1, 64, 64, 4, dil_p, None, 0, None,
                                                 None)
        assert st == 1 and "lse must not overlap q_g" in lib.lf_attn_last_error(h16).decode()
    finally:
        lib.lf_attn_destroy(h32)
        lib.lf_attn_destroy(h16)


def test_c_program_builds_and_links():
    """The plain C caller exists after the build and starts without a GPU (usage error)."""
    from sparse_long_sequence_longformer_amd import build as pkg_build

    if not os.path.exists(pkg_build.ABI_CHECK):
        pytest.skip("lf_abi_check not built (run __graft_entry__.build())")
    import subprocess

    res = subprocess.run([pkg_build.ABI_CHECK], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=60)
    assert res.returncode == 2 and "usage" in res.stdout
