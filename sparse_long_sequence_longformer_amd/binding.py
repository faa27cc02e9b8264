"""ctypes binding of liblfattn.so (argument marshalling only).

Every step of the forward runs in the library's HIP kernels; this module only
turns torch tensors into device pointers, Python sequences into int32 host
arrays, and picks torch's current HIP stream.  It raises if the library has not
been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_NAME = "liblfattn.so"

LF_OK = 0
LF_F32 = 0
LF_BF16 = 1
LF_WINDOW_SYMMETRIC = 0
LF_WINDOW_CAUSAL = 1
LF_GLOBALS_SHARED = 0
LF_GLOBALS_PER_SEQUENCE = 1
N_STAGES = 10
STAGE_NAMES = ("band", "merge", "bwd_prep", "bwd_dq", "bwd_dkv", "bwd_merge", "layer_gemm", "layer_pointwise",
               "bwd_dkv_global", "bwd_dbias")
LAYER_WEIGHTS = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b", "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")
MAX_HEADS = 64
MAX_GLOBALS = 256
MAX_BIAS_W = 1024
RANDOM_BLOCK = 64
MAX_RANDOM_DRAWS = 16

# Every symbol declared in include/lf_attn.h.
EXPORTS = (
    "lf_attn_create",
    "lf_attn_forward",
    "lf_attn_forward_static",
    "lf_attn_forward_global_proj",
    "lf_attn_forward_global_proj_lse",
    "lf_attn_forward_lse",
    "lf_attn_backward",
    "lf_attn_backward_bias",
    "lf_attn_backward_global_proj",
    "lf_layer_forward",
    "lf_attn_destroy",
    "lf_attn_status_string",
    "lf_attn_last_error",
    "lf_attn_set_stage_timing",
    "lf_attn_set_window_mode",
    "lf_attn_set_global_mode",
    "lf_attn_set_tile_rows",
    "lf_attn_set_position_bias",
    "lf_attn_set_random_blocks",
    "lf_attn_stage_times",
)

_lib = None


class LayerWeights(ctypes.Structure):
    """lf_layer_weights: device pointers of the layer's parameters."""
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHTS]


class LfAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return os.path.join(PKG, LIBRARY_NAME)


def load_library():
    """Load liblfattn.so from the package directory (built by build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise LfAttnError(-1, f"{path} is not built; run python -m sparse_long_sequence_longformer_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.lf_attn_create.argtypes = [ctypes.POINTER(vp), i32]
    lib.lf_attn_create.restype = i32
    lib.lf_attn_forward.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), i32,
                                    vp, vp]
    lib.lf_attn_forward.restype = i32
    lib.lf_attn_forward_static.argtypes = lib.lf_attn_forward.argtypes
    lib.lf_attn_forward_static.restype = i32
    lib.lf_attn_forward_global_proj.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                                i32, vp, vp]
    lib.lf_attn_forward_global_proj.restype = i32
    lib.lf_attn_forward_global_proj_lse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32),
                                                    i32, vp, vp]
    lib.lf_attn_forward_global_proj_lse.restype = i32
    lib.lf_attn_forward_lse.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), i32,
                                        vp, vp]
    lib.lf_attn_forward_lse.restype = i32
    lib.lf_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                     ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), i32,
                                     vp, vp]
    lib.lf_attn_backward.restype = i32
    lib.lf_attn_backward_bias.argtypes = [vp] * 11 + [i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_int32),
                                                      ctypes.POINTER(ctypes.c_int32), i32, vp, vp]
    lib.lf_attn_backward_bias.restype = i32
    lib.lf_attn_backward_global_proj.argtypes = [vp] * 16 + [i32, i32, i32, i32, i32,
                                                             ctypes.POINTER(ctypes.c_int32),
                                                             ctypes.POINTER(ctypes.c_int32), i32, vp, vp]
    lib.lf_attn_backward_global_proj.restype = i32
    lib.lf_layer_forward.argtypes = [vp, vp, ctypes.POINTER(LayerWeights), vp, i32, i32, i32, i32, ctypes.c_float,
                                     i32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), i32, vp, vp]
    lib.lf_layer_forward.restype = i32
    lib.lf_attn_destroy.argtypes = [vp]
    lib.lf_attn_destroy.restype = i32
    lib.lf_attn_status_string.argtypes = [i32]
    lib.lf_attn_status_string.restype = ctypes.c_char_p
    lib.lf_attn_last_error.argtypes = [vp]
    lib.lf_attn_last_error.restype = ctypes.c_char_p
    lib.lf_attn_set_global_mode.argtypes = [vp, i32]
    lib.lf_attn_set_global_mode.restype = i32
    lib.lf_attn_set_tile_rows.argtypes = [vp, i32]
    lib.lf_attn_set_tile_rows.restype = i32
    lib.lf_attn_set_window_mode.argtypes = [vp, i32]
    lib.lf_attn_set_window_mode.restype = i32
    lib.lf_attn_set_position_bias.argtypes = [vp, vp, i32, i32]
    lib.lf_attn_set_position_bias.restype = i32
    lib.lf_attn_set_random_blocks.argtypes = [vp, ctypes.POINTER(i32), i32, i32, i32]
    lib.lf_attn_set_random_blocks.restype = i32
    lib.lf_attn_set_stage_timing.argtypes = [vp, i32]
    lib.lf_attn_set_stage_timing.restype = i32
    lib.lf_attn_stage_times.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.lf_attn_stage_times.restype = i32
    _lib = lib
    return lib


def _int32_array(values):
    vals = [int(x) for x in values]
    arr = (ctypes.c_int32 * max(1, len(vals)))(*vals) if vals else None
    return arr, len(vals)


class LfAttn:
    """One library handle (fixed element type)."""

    def __init__(self, dtype: str):
        self.lib = load_library()
        self.dtype = dtype
        code = {"f32": LF_F32, "bf16": LF_BF16}.get(dtype, 99)
        h = ctypes.c_void_p()
        st = self.lib.lf_attn_create(ctypes.byref(h), code)
        self._check(st, h)
        self.handle = h
        self.causal = False
        self.per_sequence_globals = False
        self.bias = None  # the table set by set_position_bias (kept alive here)
        self.rand = None  # the draws set by set_random_blocks (int32 [H, n_qblocks, r])

    def _check(self, st, h=None):
        if st != LF_OK:
            msg = self.lib.lf_attn_status_string(st).decode()
            if h is not None and h.value:
                detail = self.lib.lf_attn_last_error(h).decode()
                if detail:
                    msg = f"{msg}: {detail}"
            raise LfAttnError(st, msg)

    _arrays_cache: dict = {}

    @classmethod
    def _host_arrays(cls, dil, global_idx):
        """int32 host arrays of the dilations and globals (cached per distinct value).
        ``global_idx``: a list (one shared set) or (flat row-major list, row length)."""
        n_row = None
        if isinstance(global_idx, tuple):
            global_idx, n_row = global_idx
        key = (tuple(int(x) for x in dil), tuple(int(x) for x in global_idx) if global_idx is not None else (),
               n_row)
        hit = cls._arrays_cache.get(key)
        if hit is not None:
            return hit
        dil_arr, _ = _int32_array(key[0])
        g_arr, ng = _int32_array(key[1])
        if n_row is not None:
            ng = n_row
        null = ctypes.POINTER(ctypes.c_int32)()
        dil_p = null if dil_arr is None else ctypes.cast(dil_arr, ctypes.POINTER(ctypes.c_int32))
        g_p = null if g_arr is None else ctypes.cast(g_arr, ctypes.POINTER(ctypes.c_int32))
        res = ((dil_arr, g_arr), dil_p, g_p, ng)
        if len(cls._arrays_cache) < 64:
            cls._arrays_cache[key] = res
        return res

    def forward_raw(self, q_ptr, k_ptr, v_ptr, out_ptr, B, H, L, d_h, w, dil, global_idx, pad_ptr, stream):
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        st = self.lib.lf_attn_forward(self.handle, q_ptr, k_ptr, v_ptr, out_ptr, B, H, L, d_h, w,
                                      dil_p, g_p, ng, pad_ptr, stream)
        self._check(st, self.handle)

    def forward_static_raw(self, q_ptr, k_ptr, v_ptr, out_ptr, B, H, L, d_h, w, dil, global_idx, pad_ptr, stream):
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        st = self.lib.lf_attn_forward_static(self.handle, q_ptr, k_ptr, v_ptr, out_ptr, B, H, L, d_h, w,
                                             dil_p, g_p, ng, pad_ptr, stream)
        self._check(st, self.handle)

    def forward_global_proj_raw(self, q_ptr, k_ptr, v_ptr, qg_ptr, kg_ptr, vg_ptr, out_ptr, B, H, L, d_h, w,
                                dil, global_idx, pad_ptr, stream):
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        st = self.lib.lf_attn_forward_global_proj(self.handle, q_ptr, k_ptr, v_ptr, qg_ptr, kg_ptr, vg_ptr,
                                                  out_ptr, B, H, L, d_h, w, dil_p, g_p, ng, pad_ptr, stream)
        self._check(st, self.handle)

    def forward_global_proj_lse_raw(self, q_ptr, k_ptr, v_ptr, qg_ptr, kg_ptr, vg_ptr, out_ptr, lse_ptr, B, H, L,
                                    d_h, w, dil, global_idx, pad_ptr, stream):
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        st = self.lib.lf_attn_forward_global_proj_lse(self.handle, q_ptr, k_ptr, v_ptr, qg_ptr, kg_ptr, vg_ptr,
                                                      out_ptr, lse_ptr, B, H, L, d_h, w, dil_p, g_p, ng, pad_ptr,
                                                      stream)
        self._check(st, self.handle)

    def forward_lse_raw(self, q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, H, L, d_h, w, dil, global_idx, pad_ptr,
                        stream):
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        st = self.lib.lf_attn_forward_lse(self.handle, q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, H, L, d_h, w,
                                          dil_p, g_p, ng, pad_ptr, stream)
        self._check(st, self.handle)

    def backward_raw(self, q_ptr, k_ptr, v_ptr, out_ptr, dout_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, B, H, L, d_h,
                     w, dil, global_idx, pad_ptr, stream):
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        st = self.lib.lf_attn_backward(self.handle, q_ptr, k_ptr, v_ptr, out_ptr, dout_ptr, lse_ptr, dq_ptr,
                                       dk_ptr, dv_ptr, B, H, L, d_h, w, dil_p, g_p, ng, pad_ptr, stream)
        self._check(st, self.handle)

    def backward_bias_raw(self, q_ptr, k_ptr, v_ptr, out_ptr, dout_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, db_ptr, B,
                          H, L, d_h, w, dil, global_idx, pad_ptr, stream):
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        st = self.lib.lf_attn_backward_bias(self.handle, q_ptr, k_ptr, v_ptr, out_ptr, dout_ptr, lse_ptr, dq_ptr,
                                            dk_ptr, dv_ptr, db_ptr, B, H, L, d_h, w, dil_p, g_p, ng, pad_ptr, stream)
        self._check(st, self.handle)

    def backward_global_proj_raw(self, ins, grads, lse_ptr, B, H, L, d_h, w, dil, global_idx, pad_ptr, stream):
        """ins: pointers (q, k, v, q_g, k_g, v_g, out, dout); grads: (dq, dk, dv, dq_g, dk_g, dv_g)."""
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        q, k, v, qg, kg, vg, o, do = ins
        dq, dk, dv, dqg, dkg, dvg = grads
        st = self.lib.lf_attn_backward_global_proj(self.handle, q, k, v, qg, kg, vg, o, do, lse_ptr, dq, dk, dv,
                                                   dqg, dkg, dvg, B, H, L, d_h, w, dil_p, g_p, ng, pad_ptr, stream)
        self._check(st, self.handle)

    def set_per_sequence_globals(self, per_seq: bool):
        """Read global_idx as one row per sequence in every later call on this handle."""
        mode = LF_GLOBALS_PER_SEQUENCE if per_seq else LF_GLOBALS_SHARED
        self._check(self.lib.lf_attn_set_global_mode(self.handle, mode), self.handle)
        self.per_sequence_globals = bool(per_seq)

    def set_tile_rows(self, rows: int):
        """Forward work-group rows for every later call on this handle: 0 chooses, 64 or
        128 forces (64: two waves per 32 rows, alternate sub-tiles of every stage)."""
        self._check(self.lib.lf_attn_set_tile_rows(self.handle, int(rows)), self.handle)

    def set_causal(self, causal: bool):
        """One-sided (causal) variant for every later call on this handle."""
        mode = LF_WINDOW_CAUSAL if causal else LF_WINDOW_SYMMETRIC
        self._check(self.lib.lf_attn_set_window_mode(self.handle, mode), self.handle)
        self.causal = bool(causal)

    def set_position_bias(self, table):
        """Relative position bias for every later call: a contiguous float32 device
        tensor [H, 2w + 1] (entry m + w for window offset m), or None to remove it.
        The handle keeps a reference: the library borrows the memory."""
        if table is None:
            self._check(self.lib.lf_attn_set_position_bias(self.handle, None, 0, 0), self.handle)
            self.bias = None
            return
        import torch

        if (table.dtype != torch.float32 or table.dim() != 2 or not table.is_cuda or not table.is_contiguous()
                or table.shape[1] % 2 != 1):
            raise ValueError("the bias table must be a contiguous float32 device tensor [H, 2w + 1]")
        H, n = table.shape
        self._check(self.lib.lf_attn_set_position_bias(self.handle, table.data_ptr(), H, (n - 1) // 2),
                    self.handle)
        self.bias = table

    def set_random_blocks(self, draws):
        """Random key blocks for every later forward: int array [H, ceil(L / 64), r] of
        key-block indices per (head, query block), negative = unused; None removes them.
        The library copies the table (uploaded by the next call)."""
        if draws is None:
            self._check(self.lib.lf_attn_set_random_blocks(self.handle, None, 0, 0, 0), self.handle)
            self.rand = None
            return
        import numpy as np

        a = np.ascontiguousarray(np.asarray(draws.tolist() if hasattr(draws, "tolist") else draws, dtype=np.int32))
        if a.ndim != 3:
            raise ValueError("random blocks must be [H, n_query_blocks, r]")
        H, nq, r = a.shape
        ptr = a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        self._check(self.lib.lf_attn_set_random_blocks(self.handle, ptr, H, nq, r), self.handle)
        self.rand = a

    def layer_raw(self, x_ptr, weights: LayerWeights, out_ptr, B, L, hidden, ffn, eps, w, dil, global_idx, pad_ptr,
                  stream):
        keep, dil_p, g_p, ng = self._host_arrays(dil, global_idx)
        st = self.lib.lf_layer_forward(self.handle, x_ptr, ctypes.byref(weights), out_ptr, B, L, hidden, ffn,
                                       float(eps), w, dil_p, g_p, ng, pad_ptr, stream)
        self._check(st, self.handle)

    def set_stage_timing(self, enable: bool):
        self._check(self.lib.lf_attn_set_stage_timing(self.handle, 1 if enable else 0), self.handle)

    def stage_times(self):
        ms = (ctypes.c_double * N_STAGES)()
        n = (ctypes.c_int64 * N_STAGES)()
        self._check(self.lib.lf_attn_stage_times(self.handle, ms, n), self.handle)
        return {STAGE_NAMES[i]: (ms[i], n[i]) for i in range(N_STAGES)}

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            self.lib.lf_attn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_handles: dict = {}


def _handle_for(dtype: str, causal: bool = False, per_seq: bool = False, rand: bool = False) -> LfAttn:
    key = (dtype, bool(causal), bool(per_seq), bool(rand))
    if key not in _handles:
        h = LfAttn(dtype)
        if causal:
            h.set_causal(True)
        if per_seq:
            h.set_per_sequence_globals(True)
        _handles[key] = h
    return _handles[key]


class _CallBias:
    """Installs a per-call bias table on a handle and restores its previous one."""

    def __init__(self, h: LfAttn, bias):
        self.h, self.bias, self.prev = h, bias, h.bias

    def __enter__(self):
        if self.bias is not None:
            self.h.set_position_bias(self.bias)

    def __exit__(self, *exc):
        if self.bias is not None:
            self.h.set_position_bias(self.prev)
        return False


class _CallRandom:
    """Installs per-call random draws on a handle.  The library's own handles for
    calls with draws keep the last table (re-installed only when it changes); a
    caller's handle gets its previous table back after the call."""

    def __init__(self, h: LfAttn, rand, restore: bool):
        self.h, self.rand, self.restore, self.prev = h, rand, restore, h.rand

    def __enter__(self):
        import numpy as np

        if self.rand is None:
            return
        new = np.asarray(self.rand.tolist() if hasattr(self.rand, "tolist") else self.rand, dtype=np.int32)
        if self.h.rand is None or not np.array_equal(self.h.rand, new):
            self.h.set_random_blocks(new)
        else:
            self.restore = False

    def __exit__(self, *exc):
        if self.rand is not None and self.restore:
            self.h.set_random_blocks(self.prev)
        return False


def _global_arg(global_idx, B: int):
    """Shared set -> (list, False); one set per sequence (2-D, rows may differ in
    length) -> ((flat row-major list padded with -1, row length), True)."""
    if global_idx is None:
        return None, False
    if hasattr(global_idx, "tolist"):
        global_idx = global_idx.tolist()
    rows = list(global_idx)
    if rows and isinstance(rows[0], (list, tuple)):
        if len(rows) != B:
            raise ValueError("per-sequence global sets need one row per sequence")
        n = max((len(r) for r in rows), default=0)
        flat = [int(x) for r in rows for x in (list(r) + [-1] * (n - len(r)))]
        return (flat, n), True
    return [int(x) for x in rows], False


def _marshal(q, others, w, dil, global_idx, key_pad_mask, out, handle, causal=False, rand=False):
    """Checks shared by both entry points; returns (B, H, L, d_h, dilation list,
    global list, pad pointer, out, handle, stream)."""
    import torch

    if q.dtype == torch.bfloat16:
        dt = "bf16"
    elif q.dtype == torch.float32:
        dt = "f32"
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in others:
        if t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError(f"{name} must match q in dtype and shape")
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, L, d_h]")
    for name, t in [("q", q)] + list(others):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    B, H, L, d_h = q.shape
    if isinstance(dil, int):
        dil = [dil] * H
    dil = [int(x) for x in (dil.tolist() if hasattr(dil, "tolist") else dil)]
    if len(dil) != H:
        raise ValueError("need one dilation per head")
    global_idx, per_seq = _global_arg(global_idx, B)
    pad_ptr = None
    if key_pad_mask is not None:
        if key_pad_mask.dtype == torch.bool:
            key_pad_mask = key_pad_mask.view(torch.uint8)
        if key_pad_mask.dtype != torch.uint8 or tuple(key_pad_mask.shape) != (B, L):
            raise ValueError("key_pad_mask must be a [B, L] bool or uint8 tensor")
        if not key_pad_mask.is_cuda or not key_pad_mask.is_contiguous():
            raise ValueError("key_pad_mask must be a contiguous device tensor")
        pad_ptr = key_pad_mask.data_ptr()
    if out is None:
        out = torch.empty_like(q)
    elif out.dtype != q.dtype or out.shape != q.shape or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous device tensor like q")
    h = handle if handle is not None else _handle_for(dt, causal, per_seq, rand)
    if h.dtype != dt:
        raise ValueError("handle dtype does not match the inputs")
    if h.causal != bool(causal):
        raise ValueError("handle window mode does not match causal=")
    if h.per_sequence_globals != per_seq:
        raise ValueError("handle global mode does not match the shape of global_idx")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    return B, H, L, d_h, dil, global_idx, pad_ptr, out, h, stream


def forward(q, k, v, w: int, dil, global_idx=None, key_pad_mask=None, out=None, handle: LfAttn | None = None,
            causal: bool = False, bias=None, rand=None):
    """Longformer window + global attention forward on the GPU.

    q, k, v: contiguous CUDA/HIP tensors [B, H, L, 64], all bfloat16 or all float32.
    w: keys on each side of the window.  dil: one dilation per head (sequence or int).
    global_idx: positions attended by and attending to everything (host sequence).
    key_pad_mask: [B, L] bool/uint8 device tensor, nonzero = padded key, or None.
    causal: the one-sided variant (no key after its query); a given handle must be in
    the same mode.
    bias: relative position bias on window scores, float32 device tensor [H, 2w + 1],
    for this call only; None leaves the handle's own setting (none by default).
    rand: random key blocks [H, ceil(L / 64), r] (int, negative = unused) for this call
    (every head undilated); None leaves the handle's own setting.
    Returns ``out`` (allocated if not given), same shape and dtype as q.
    """
    import torch

    B, H, L, d_h, dil, global_idx, pad_ptr, out, h, stream = _marshal(
        q, [("k", k), ("v", v)], w, dil, global_idx, key_pad_mask, out, handle, causal, rand is not None)
    with torch.cuda.device(q.device), _CallBias(h, bias), _CallRandom(h, rand, handle is not None):
        h.forward_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, d_h, int(w), dil,
                      global_idx, pad_ptr, stream)
    return out


def forward_static(q, k, v, w: int, dil, global_idx=None, key_pad_mask=None, out=None,
                   handle: LfAttn | None = None, causal: bool = False):
    """``forward`` through lf_attn_forward_static: the library allocates no device memory
    in the call (its global-row partials go to a static device array of
    LF_STATIC_SCRATCH_BYTES per GPU; calls that overlap in time on one GPU race).
    Pass ``out`` to keep the call itself free of allocations."""
    import torch

    B, H, L, d_h, dil, global_idx, pad_ptr, out, h, stream = _marshal(
        q, [("k", k), ("v", v)], w, dil, global_idx, key_pad_mask, out, handle, causal)
    with torch.cuda.device(q.device):
        h.forward_static_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, d_h, int(w), dil,
                             global_idx, pad_ptr, stream)
    return out


def forward_global_proj(q, k, v, q_g, k_g, v_g, w: int, dil, global_idx=None, key_pad_mask=None, out=None,
                        handle: LfAttn | None = None, causal: bool = False, bias=None, rand=None):
    """As ``forward``, but the global query rows attend every unpadded key with their
    own projections q_g, k_g, v_g (tensors shaped and typed like q); every other row
    uses q, k, v."""
    import torch

    B, H, L, d_h, dil, global_idx, pad_ptr, out, h, stream = _marshal(
        q, [("k", k), ("v", v), ("q_g", q_g), ("k_g", k_g), ("v_g", v_g)], w, dil, global_idx,
        key_pad_mask, out, handle, causal, rand is not None)
    with torch.cuda.device(q.device), _CallBias(h, bias), _CallRandom(h, rand, handle is not None):
        h.forward_global_proj_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_g.data_ptr(), k_g.data_ptr(),
                                  v_g.data_ptr(), out.data_ptr(), B, H, L, d_h, int(w), dil, global_idx,
                                  pad_ptr, stream)
    return out


def _lse_out(lse, B, H, L, device):
    import torch

    if lse is None:
        return torch.empty((B, H, L), dtype=torch.float32, device=device)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 device tensor [B, H, L]")
    return lse


def forward_global_proj_lse(q, k, v, q_g, k_g, v_g, w: int, dil, global_idx=None, key_pad_mask=None, out=None,
                            lse=None, handle: LfAttn | None = None, causal: bool = False, bias=None, rand=None):
    """``forward_global_proj`` that also returns each row's log-sum-exp: (out, lse), the
    statistics ``backward_global_proj`` needs."""
    import torch

    B, H, L, d_h, dil, global_idx, pad_ptr, out, h, stream = _marshal(
        q, [("k", k), ("v", v), ("q_g", q_g), ("k_g", k_g), ("v_g", v_g)], w, dil, global_idx,
        key_pad_mask, out, handle, causal, rand is not None)
    lse = _lse_out(lse, B, H, L, q.device)
    with torch.cuda.device(q.device), _CallBias(h, bias), _CallRandom(h, rand, handle is not None):
        h.forward_global_proj_lse_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_g.data_ptr(), k_g.data_ptr(),
                                      v_g.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, L, d_h, int(w), dil,
                                      global_idx, pad_ptr, stream)
    return out, lse


def forward_lse(q, k, v, w: int, dil, global_idx=None, key_pad_mask=None, out=None, lse=None,
                handle: LfAttn | None = None, causal: bool = False, bias=None, rand=None):
    """``forward`` that also returns each row's log-sum-exp: (out, lse), lse a float32
    device tensor [B, H, L] (natural log, -inf for rows without keys)."""
    import torch

    B, H, L, d_h, dil, global_idx, pad_ptr, out, h, stream = _marshal(
        q, [("k", k), ("v", v)], w, dil, global_idx, key_pad_mask, out, handle, causal, rand is not None)
    lse = _lse_out(lse, B, H, L, q.device)
    with torch.cuda.device(q.device), _CallBias(h, bias), _CallRandom(h, rand, handle is not None):
        h.forward_lse_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, L, d_h,
                          int(w), dil, global_idx, pad_ptr, stream)
    return out, lse


def backward(q, k, v, out, dout, lse, w: int, dil, global_idx=None, key_pad_mask=None, dq=None, dk=None,
             dv=None, handle: LfAttn | None = None, causal: bool = False, bias=None, rand=None, dbias=None):
    """Gradients (dq, dk, dv) of the forward for the upstream gradient ``dout``.

    q, k, v, out, dout: contiguous device tensors [B, H, L, 64], all bf16 or all
    float32 (the handle's dtype); ``out`` and
    ``lse`` as returned by ``forward_lse`` for the same inputs and pattern (and bias).
    dbias: with a position bias table in use, True (or a float32 device tensor
    [H, 2w + 1] to write into) also returns the gradient of the table, summed over
    the batch, as a fourth result (lf_attn_backward_bias).
    """
    import torch

    B, H, L, d_h, dil, global_idx, pad_ptr, _, h, stream = _marshal(
        q, [("k", k), ("v", v), ("out", out), ("dout", dout)], w, dil, global_idx, key_pad_mask, out, handle,
        causal, rand is not None)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 device tensor [B, H, L]")
    res = []
    for t in (dq, dk, dv):
        if t is None:
            t = torch.empty_like(q)
        elif t.dtype != q.dtype or t.shape != q.shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("dq, dk, dv must be contiguous device tensors like q")
        res.append(t)
    dq, dk, dv = res
    if dbias is not None and dbias is not False:
        if dbias is True:
            dbias = torch.empty((H, 2 * int(w) + 1), dtype=torch.float32, device=q.device)
        elif (dbias.dtype != torch.float32 or tuple(dbias.shape) != (H, 2 * int(w) + 1) or not dbias.is_contiguous()
              or not dbias.is_cuda):
            raise ValueError("dbias must be a contiguous float32 device tensor [H, 2w + 1]")
        with torch.cuda.device(q.device), _CallBias(h, bias), _CallRandom(h, rand, handle is not None):
            h.backward_bias_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dbias.data_ptr(), B, H, L,
                                d_h, int(w), dil, global_idx, pad_ptr, stream)
        return dq, dk, dv, dbias
    with torch.cuda.device(q.device), _CallBias(h, bias), _CallRandom(h, rand, handle is not None):
        h.backward_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, L, d_h, int(w), dil, global_idx, pad_ptr,
                       stream)
    return dq, dk, dv


def backward_global_proj(q, k, v, q_g, k_g, v_g, out, dout, lse, w: int, dil, global_idx=None, key_pad_mask=None,
                         grads=None, handle: LfAttn | None = None, causal: bool = False, bias=None, rand=None):
    """Gradients (dq, dk, dv, dq_g, dk_g, dv_g) of ``forward_global_proj`` for ``dout``.

    All tensors contiguous [B, H, L, 64] on the device, all bf16 or all float32; ``out`` and ``lse`` as
    returned by ``forward_global_proj_lse``.  grads: six preallocated outputs, or None.
    """
    import torch

    B, H, L, d_h, dil, global_idx, pad_ptr, _, h, stream = _marshal(
        q, [("k", k), ("v", v), ("q_g", q_g), ("k_g", k_g), ("v_g", v_g), ("out", out), ("dout", dout)], w, dil,
        global_idx, key_pad_mask, out, handle, causal, rand is not None)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 device tensor [B, H, L]")
    if grads is None:
        grads = tuple(torch.empty_like(q) for _ in range(6))
    grads = tuple(grads)
    if len(grads) != 6:
        raise ValueError("grads must hold six tensors")
    for t in grads:
        if t.dtype != q.dtype or t.shape != q.shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("the gradients must be contiguous device tensors like q")
    ins = tuple(t.data_ptr() for t in (q, k, v, q_g, k_g, v_g, out, dout))
    with torch.cuda.device(q.device), _CallBias(h, bias), _CallRandom(h, rand, handle is not None):
        h.backward_global_proj_raw(ins, tuple(t.data_ptr() for t in grads), lse.data_ptr(), B, H, L, d_h, int(w),
                                   dil, global_idx, pad_ptr, stream)
    return grads


def layer_forward(x, weights: dict, w: int, dil, global_idx=None, key_pad_mask=None, eps: float = 1e-5, out=None,
                  handle: LfAttn | None = None, causal: bool = False, bias=None, rand=None):
    """One Longformer layer (projections, this attention, LayerNorms, GELU feed-forward).

    x: contiguous bf16 device tensor [B, L, hidden]; ``weights`` maps LAYER_WEIGHTS to
    contiguous bf16 device tensors in nn.Linear layout.  Returns ``out`` [B, L, hidden].
    """
    import torch

    if x.dtype != torch.bfloat16 or x.dim() != 3 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 device tensor [B, L, hidden]")
    B, L, E = x.shape
    H = E // 64
    F = int(weights["w_1"].shape[0])
    for n in LAYER_WEIGHTS:
        t = weights[n]
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"weight {n} must be a contiguous bfloat16 device tensor")
    if isinstance(dil, int):
        dil = [dil] * H
    dil = [int(d) for d in dil]
    global_idx, per_seq = _global_arg(global_idx, B)
    pad_ptr = None
    if key_pad_mask is not None:
        if key_pad_mask.dtype == torch.bool:
            key_pad_mask = key_pad_mask.view(torch.uint8)
        if tuple(key_pad_mask.shape) != (B, L) or not key_pad_mask.is_cuda or not key_pad_mask.is_contiguous():
            raise ValueError("key_pad_mask must be a contiguous [B, L] device tensor")
        pad_ptr = key_pad_mask.data_ptr()
    if out is None:
        out = torch.empty_like(x)
    h = handle if handle is not None else _handle_for("bf16", causal, per_seq, rand is not None)
    if h.causal != bool(causal):
        raise ValueError("handle window mode does not match causal=")
    if h.per_sequence_globals != per_seq:
        raise ValueError("handle global mode does not match the shape of global_idx")
    wts = LayerWeights(*[weights[n].data_ptr() for n in LAYER_WEIGHTS])
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device), _CallBias(h, bias), _CallRandom(h, rand, handle is not None):
        h.layer_raw(x.data_ptr(), wts, out.data_ptr(), B, L, E, F, eps, int(w), dil, global_idx, pad_ptr, stream)
    return out
