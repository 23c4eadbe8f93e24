"""ctypes binding of libca2 (include/ca2.h), same names as the C entry points.

Argument marshalling only: tensors become device pointers, torch's current
stream becomes the hipStream_t, shapes and dtypes are checked against the
cache's config so a wrong tensor is rejected before any launch. Every step of
the computation runs in libca2's HIP kernels; if the library is missing this
module raises instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libca2.so")

CA2_OK = 0
CA2_ERR_INVALID_ARG = 1
CA2_ERR_OUT_OF_MEMORY = 2
CA2_ERR_HIP = 3
CA2_ERR_STATE = 4
CA2_ERR_UNSUPPORTED = 5
CA2_F32 = 0
CA2_BF16 = 1
CA2_SPATIAL_PREFIX = 0
CA2_SPATIAL_SELF = 1
CA2_STAGE_RING = 1
CA2_STAGE_SPATIAL = 2
ABI_VERSION = 4      # include/ca2.h CA2_ABI_VERSION this binding is written for

_DTYPES = {"f32": CA2_F32, "bf16": CA2_BF16}


class Ca2Config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("p_max", ctypes.c_int32),
                ("p_spatial", ctypes.c_int32), ("tpe_len", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Ca2CacheInfo(ctypes.Structure):
    _fields_ = [("p_k", ctypes.c_int32), ("head_slot", ctypes.c_int32),
                ("spatial_frames", ctypes.c_int32), ("staged_frames", ctypes.c_int32),
                ("frames_written", ctypes.c_int64), ("bytes_resident", ctypes.c_uint64),
                ("ring_slots", ctypes.c_int32), ("generation", ctypes.c_uint32)]


# name -> (restype, argtypes)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIGS = {
    "ca2_cache_create": (_I32, [ctypes.POINTER(Ca2Config), ctypes.POINTER(_P)]),
    "ca2_cache_create_staged": (_I32, [ctypes.POINTER(Ca2Config), ctypes.POINTER(_P)]),
    "ca2_qkv_proj_stage": (_I32, [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "ca2_cache_commit": (_I32, [_P]),
    "ca2_cache_destroy": (None, [_P]),
    "ca2_cache_write": (_I32, [_P, _P, _P, _P, _P, _I32, _P]),
    "ca2_temporal_attn": (_I32, [_P, _P, _P, _P, _P, _I32, ctypes.c_float, _P]),
    "ca2_spatial_attn": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, ctypes.c_float, _P]),
    "ca2_denoise_attn": (_I32, [_P, _P, _P, _P, _P, _I32, ctypes.c_float, _P, _P, _P, _P, ctypes.c_float, _I32,
                                ctypes.POINTER(_I32), _P]),
    "ca2_tpe_index": (_I32, [_P, _I32, ctypes.POINTER(_I32)]),
    "ca2_tpe_index_raw": (_I32, [_I64, _I32, _I32, ctypes.POINTER(_I32)]),
    "ca2_cache_info_get": (_I32, [_P, ctypes.POINTER(Ca2CacheInfo)]),
    "ca2_cache_slot_map": (_I32, [_P, ctypes.POINTER(_I32)]),
    "ca2_cache_frame_ids": (_I32, [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I32)]),
    "ca2_ring_slot_map_raw": (_I32, [_I64, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "ca2_spatial_slot_map_raw": (_I32, [_I64, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I32)]),
    "ca2_bytes_resident": (ctypes.c_uint64, [ctypes.POINTER(Ca2Config)]),
    "ca2_cache_debug_copy": (_I32, [_P, _P, _P, _P, _P, _P]),
    "ca2_qkv_proj": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _P]),
    "ca2_temporal_attn_frames": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                        ctypes.c_float, _P]),
    "ca2_spatial_attn_frames": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                       ctypes.c_float, _P]),
    "ca2_toy_temb_mod": (_I32, [_P, _I32, _P, _I32, _I32, _P, _P]),
    "ca2_toy_ln_mod": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P]),
    "ca2_toy_linear": (_I32, [_P, _I32, _P, _I32, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "ca2_set_spatial_variant": (_I32, [_I32]),
    "ca2_set_temporal_variant": (_I32, [_I32]),
    "ca2_abi_version": (_I32, []),
    "ca2_status_string": (ctypes.c_char_p, [_I32]),
    "ca2_last_error": (ctypes.c_char_p, []),
}
EXPORTS = tuple(_SIGS)

_lib = None


class Ca2Error(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


def load():
    """Load libca2.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(there is no fallback implementation)")
    # torch ships its own HIP runtime; load it first so that libca2 binds to the
    # same libamdhip64 instance instead of initialising a second runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    if not hasattr(lib, "ca2_abi_version"):
        raise RuntimeError(f"{LIB_PATH} predates the ABI version check: rebuild it")
    lib.ca2_abi_version.restype = _I32
    lib.ca2_abi_version.argtypes = []
    if lib.ca2_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {lib.ca2_abi_version()}, this binding expects "
                           f"{ABI_VERSION}: rebuild it from these sources")
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != CA2_OK:
        lib = load()
        detail = lib.ca2_last_error().decode() or lib.ca2_status_string(status).decode()
        raise Ca2Error(status, where, detail)


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:   # the current stream's handle without building a Stream object (~3 us per call)
        return ctypes.c_void_p(raw(torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_config(B, H, d, S, l, p_max, p_spatial, tpe_len, dtype) -> Ca2Config:
    return Ca2Config(B, H, d, S, l, p_max, p_spatial, tpe_len, _DTYPES.get(dtype, dtype))


# ----------------------------------------------------------------------------
# thin functions with the C names
# ----------------------------------------------------------------------------
def ca2_set_spatial_variant(variant: int):
    """Force the bf16 spatial kernel's launch variant (0 = by grid size)."""
    _check(load().ca2_set_spatial_variant(int(variant)), "ca2_set_spatial_variant")


def ca2_set_temporal_variant(variant: int):
    """Force the bf16 temporal kernel (0, 1 = dimension-split, the default; 2 = matrix-core rows)."""
    _check(load().ca2_set_temporal_variant(int(variant)), "ca2_set_temporal_variant")


def ca2_tpe_index_raw(first_frame: int, n: int, tpe_len: int):
    lib = load()
    out = (_I32 * max(n, 1))()
    _check(lib.ca2_tpe_index_raw(first_frame, n, tpe_len, out), "ca2_tpe_index_raw")
    return list(out)[:n]


def ca2_ring_slot_map_raw(frames_written: int, p_max: int):
    lib = load()
    out = (_I32 * p_max)()
    pk = _I32(0)
    _check(lib.ca2_ring_slot_map_raw(frames_written, p_max, out, ctypes.byref(pk)), "ca2_ring_slot_map_raw")
    return list(out)[:pk.value]


def ca2_spatial_slot_map_raw(frames_written: int, p_spatial: int):
    lib = load()
    fr = (_I64 * max(p_spatial, 1))()
    sl = (_I32 * max(p_spatial, 1))()
    _check(lib.ca2_spatial_slot_map_raw(frames_written, p_spatial, fr, sl), "ca2_spatial_slot_map_raw")
    if frames_written == 0 or p_spatial == 0:
        return [], []
    return list(fr)[:p_spatial], list(sl)[:p_spatial]


def ca2_bytes_resident(cfg: Ca2Config) -> int:
    return int(load().ca2_bytes_resident(ctypes.byref(cfg)))


def ca2_cache_create(cfg: Ca2Config):
    lib = load()
    h = _P()
    _check(lib.ca2_cache_create(ctypes.byref(cfg), ctypes.byref(h)), "ca2_cache_create")
    return h


def ca2_cache_create_staged(cfg: Ca2Config):
    lib = load()
    h = _P()
    _check(lib.ca2_cache_create_staged(ctypes.byref(cfg), ctypes.byref(h)), "ca2_cache_create_staged")
    return h


def ca2_cache_destroy(handle):
    load().ca2_cache_destroy(handle)


def ca2_status_string(status: int) -> str:
    return load().ca2_status_string(status).decode()


def ca2_qkv_proj(x, w, q, k, v, stream=None):
    """x: [m][c_in] bf16, w: [3c][c_in] bf16, q/k/v: [m][c] bf16 (cuda tensors)."""
    import torch
    m, c_in = x.shape
    c3 = w.shape[0]
    c = c3 // 3
    for t, shape in ((x, (m, c_in)), (w, (c3, c_in)), (q, (m, c)), (k, (m, c)), (v, (m, c))):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != shape or not t.is_cuda:
            raise ValueError(f"qkv_proj: expected contiguous cuda bf16 {shape}, got {t.dtype} {tuple(t.shape)}")
    _check(load().ca2_qkv_proj(_ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v), m, c_in, c,
                               _stream(stream)), "ca2_qkv_proj")


def _frames_shape(q, k, v, out, where):
    """[B][T][S][H][d] cuda tensors of one dtype -> (B, T, S, H, d, ca2 dtype)."""
    import torch
    dt = {torch.float32: CA2_F32, torch.bfloat16: CA2_BF16}.get(q.dtype)
    if dt is None:
        raise ValueError(f"{where}: dtype {q.dtype} is not float32 or bfloat16")
    if q.dim() != 5:
        raise ValueError(f"{where}: expected [B][T][S][H][d] tensors, got {tuple(q.shape)}")
    for t in (q, k, v, out):
        if t.dtype != q.dtype or tuple(t.shape) != tuple(q.shape) or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{where}: expected contiguous cuda {q.dtype} {tuple(q.shape)}, "
                             f"got {t.dtype} {tuple(t.shape)}")
    B, T, S, H, d = q.shape
    return B, T, S, H, d, dt


def ca2_temporal_attn_frames(q, k, v, out, causal, scale=None, stream=None):
    """Cache-less temporal attention over the T frames of [B][T][S][H][d]
    tensors: causal (mask over frames) or bidirectional (causal=False)."""
    B, T, S, H, d, dt = _frames_shape(q, k, v, out, "ca2_temporal_attn_frames")
    sc = d ** -0.5 if scale is None else scale
    _check(load().ca2_temporal_attn_frames(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, S, H, d, dt,
                                           1 if causal else 0, sc, _stream(stream)),
           "ca2_temporal_attn_frames")


def ca2_spatial_attn_frames(q, k, v, out, scale=None, stream=None):
    """Cache-less spatial self attention of each of the T frames."""
    B, T, S, H, d, dt = _frames_shape(q, k, v, out, "ca2_spatial_attn_frames")
    sc = d ** -0.5 if scale is None else scale
    _check(load().ca2_spatial_attn_frames(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, T, S, H, d, dt, sc,
                                          _stream(stream)), "ca2_spatial_attn_frames")


def _f32_2d(t, where):
    import torch
    if t.dtype != torch.float32 or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{where}: expected a 2-D cuda float32 tensor with unit column stride, "
                         f"got {t.dtype} {tuple(t.shape)} strides {t.stride()}")
    return t.shape[0], t.shape[1], t.stride(0)


def ca2_toy_temb_mod(t, wmod, out, stream=None):
    """t: [F] float32, wmod: [temb_dim][W], out: [F][W] (cuda)."""
    import torch
    if t.dtype != torch.float32 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError("ca2_toy_temb_mod: t must be a contiguous 1-D float32 tensor")
    td, wd, _ = _f32_2d(wmod, "ca2_toy_temb_mod")
    f, w2, _ = _f32_2d(out, "ca2_toy_temb_mod")
    if not (wmod.is_contiguous() and out.is_contiguous()) or f != t.shape[0] or w2 != wd:
        raise ValueError("ca2_toy_temb_mod: shapes do not match")
    _check(load().ca2_toy_temb_mod(_ptr(t), f, _ptr(wmod), td, wd, _ptr(out), _stream(stream)), "ca2_toy_temb_mod")


def ca2_toy_ln_mod(x, mod, shift_off, scale_off, out, stream=None):
    """x, out: [F][S][C] float32; mod: [F][W] with the shift and scale ranges inside W."""
    import torch
    for u in (x, out, mod):
        if u.dtype != torch.float32 or not u.is_contiguous() or not u.is_cuda:
            raise ValueError("ca2_toy_ln_mod: contiguous cuda float32 tensors expected")
    if x.dim() != 3 or tuple(out.shape) != tuple(x.shape) or mod.dim() != 2 or mod.shape[0] != x.shape[0]:
        raise ValueError("ca2_toy_ln_mod: shapes do not match")
    F, S, C = x.shape
    _check(load().ca2_toy_ln_mod(_ptr(x), _ptr(mod), mod.shape[1], shift_off, scale_off, F, S, C, _ptr(out),
                                 _stream(stream)), "ca2_toy_ln_mod")


def ca2_toy_linear(x, w, y, r=None, act=0, stream=None):
    """y = act(x @ w) (+ r); 2-D cuda float32 views with unit column stride
    (column slices of a wider matrix are fine)."""
    m, k, ldx = _f32_2d(x, "ca2_toy_linear")
    k2, n, ldw = _f32_2d(w, "ca2_toy_linear")
    m2, n2, ldy = _f32_2d(y, "ca2_toy_linear")
    ldr = 0
    if r is not None:
        m3, n3, ldr = _f32_2d(r, "ca2_toy_linear")
        if (m3, n3) != (m, n):
            raise ValueError("ca2_toy_linear: r shape")
    if k2 != k or (m2, n2) != (m, n):
        raise ValueError(f"ca2_toy_linear: shapes {tuple(x.shape)} @ {tuple(w.shape)} -> {tuple(y.shape)}")
    _check(load().ca2_toy_linear(_ptr(x), ldx, _ptr(w), ldw, _ptr(r), ldr, _ptr(y), ldy, m, n, k, act,
                                 _stream(stream)), "ca2_toy_linear")


class Cache:
    """Owner of one ca2_cache handle, with shape/dtype checks on its calls."""

    def __init__(self, B, H, d, S, l, p_max, p_spatial, tpe_len, dtype="bf16", staged=False):
        """staged=True: ca2_cache_create_staged (P_max + l ring slots, for
        ca2_qkv_proj_stage / ca2_cache_commit)."""
        self.shape = dict(B=B, H=H, d=d, S=S, l=l, p_max=p_max, p_spatial=p_spatial,
                          tpe_len=tpe_len, dtype=dtype)
        self.ring_slots = p_max + (l if staged else 0)
        self.cfg = make_config(B, H, d, S, l, p_max, p_spatial, tpe_len, dtype)
        self._lib = load()
        self.handle = (ca2_cache_create_staged if staged else ca2_cache_create)(self.cfg)

    @classmethod
    def from_shape(cls, sh: dict, staged=False):
        return cls(sh["B"], sh["H"], sh["d"], sh["S"], sh["l"], sh["p_max"], sh["p_spatial"],
                   sh["tpe_len"], sh["dtype"], staged=staged)

    def close(self):
        if getattr(self, "handle", None) is not None:
            self._lib.ca2_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- checks -------------------------------------------------------------
    def _torch_dtype(self):
        import torch
        return torch.bfloat16 if self.shape["dtype"] == "bf16" else torch.float32

    def _chk(self, name, t, n):
        sh = self.shape
        want = (sh["B"], n, sh["S"], sh["H"], sh["d"])
        if (t is None or not t.is_cuda or t.dtype != self._torch_dtype() or not t.is_contiguous()
                or tuple(t.shape) != want):
            got = None if t is None else (t.dtype, tuple(t.shape), t.is_contiguous())
            raise ValueError(f"{name}: expected contiguous cuda {self._torch_dtype()} {want}, got {got}")

    # -- entry points -----------------------------------------------------------
    def ca2_cache_write(self, k_t, v_t, k_s, v_s, stream=None):
        n = k_t.shape[1]
        for nm, t in (("k_t", k_t), ("v_t", v_t)):
            self._chk(nm, t, n)
        if self.shape["p_spatial"] > 0 or k_s is not None:
            for nm, t in (("k_s", k_s), ("v_s", v_s)):
                self._chk(nm, t, n)
        _check(self._lib.ca2_cache_write(self.handle, _ptr(k_t), _ptr(v_t), _ptr(k_s), _ptr(v_s),
                                         n, _stream(stream)), "ca2_cache_write")

    def ca2_temporal_attn(self, q, k_new, v_new, out, scale=None, stream=None):
        """k_new = v_new = None: the new frames are the ones staged in the ring."""
        n = q.shape[1]
        staged = k_new is None and v_new is None
        for nm, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("out", out)):
            if not (staged and nm in ("k_new", "v_new")):
                self._chk(nm, t, n)
        scale = self.shape["d"] ** -0.5 if scale is None else scale
        _check(self._lib.ca2_temporal_attn(self.handle, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out),
                                           n, scale, _stream(stream)), "ca2_temporal_attn")

    def ca2_denoise_attn(self, q_s, k_s, v_s, out_s, q_t, k_t, v_t, out_t, mode=CA2_SPATIAL_PREFIX,
                         scale_s=None, scale_t=None, stream=None):
        """Spatial attention (q_s, k_s, v_s -> out_s) and temporal attention
        (q_t, k_t, v_t -> out_t; k_t = v_t = None for staged frames) of one
        denoising call, fused into one launch where the shapes allow it.
        Returns True when the fused launch ran."""
        n = q_s.shape[1]
        for nm, t in (("q_s", q_s), ("k_s", k_s), ("v_s", v_s), ("out_s", out_s), ("q_t", q_t), ("out_t", out_t)):
            self._chk(nm, t, n)
        staged = k_t is None and v_t is None
        if not staged:
            self._chk("k_t", k_t, n)
            self._chk("v_t", v_t, n)
        d = self.shape["d"]
        scale_s = d ** -0.5 if scale_s is None else scale_s
        scale_t = d ** -0.5 if scale_t is None else scale_t
        fused = _I32(0)
        _check(self._lib.ca2_denoise_attn(self.handle, _ptr(q_s), _ptr(k_s), _ptr(v_s), _ptr(out_s), int(mode),
                                          scale_s, _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(out_t), scale_t, n,
                                          ctypes.byref(fused), _stream(stream)), "ca2_denoise_attn")
        return bool(fused.value)

    def ca2_spatial_attn(self, q, k, v, out, mode=CA2_SPATIAL_PREFIX, scale=None, stream=None):
        n = q.shape[1]
        for nm, t in (("q", q), ("k", k), ("v", v), ("out", out)):
            self._chk(nm, t, n)
        scale = self.shape["d"] ** -0.5 if scale is None else scale
        _check(self._lib.ca2_spatial_attn(self.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), n,
                                          int(mode), scale, _stream(stream)), "ca2_spatial_attn")

    def ca2_tpe_index(self, n):
        out = (_I32 * max(n, 1))()
        _check(self._lib.ca2_tpe_index(self.handle, n, out), "ca2_tpe_index")
        return list(out)[:n]

    def ca2_cache_info_get(self) -> dict:
        info = Ca2CacheInfo()
        _check(self._lib.ca2_cache_info_get(self.handle, ctypes.byref(info)), "ca2_cache_info_get")
        return dict(p_k=info.p_k, head_slot=info.head_slot, spatial_frames=info.spatial_frames,
                    staged_frames=info.staged_frames, frames_written=info.frames_written,
                    bytes_resident=info.bytes_resident, ring_slots=info.ring_slots,
                    generation=info.generation)

    def ca2_cache_slot_map(self):
        out = (_I32 * self.shape["p_max"])()
        _check(self._lib.ca2_cache_slot_map(self.handle, out), "ca2_cache_slot_map")
        return list(out)[:self.ca2_cache_info_get()["p_k"]]

    def ca2_cache_frame_ids(self):
        P, Ps = self.shape["p_max"], self.shape["p_spatial"]
        t = (_I64 * P)()
        s = (_I64 * max(Ps, 1))()
        sl = (_I32 * max(Ps, 1))()
        _check(self._lib.ca2_cache_frame_ids(self.handle, t, s, sl), "ca2_cache_frame_ids")
        info = self.ca2_cache_info_get()
        sp = (list(s)[:Ps], list(sl)[:Ps]) if info["frames_written"] and Ps else ([], [])
        return list(t)[:info["p_k"]], sp[0], sp[1]

    def ca2_cache_debug_copy(self, stream=None):
        """Host copies (numpy) of ring K, ring V, spatial K, spatial V in physical slot order."""
        import numpy as np
        sh = self.shape
        npdt = np.uint16 if sh["dtype"] == "bf16" else np.float32
        ring = np.empty((sh["B"], self.ring_slots, sh["S"], sh["H"], sh["d"]), dtype=npdt)
        ringv = np.empty_like(ring)
        sp = np.empty((sh["B"], sh["p_spatial"], sh["S"], sh["H"], sh["d"]), dtype=npdt)
        spv = np.empty_like(sp)
        ptr = lambda a: ctypes.c_void_p(a.ctypes.data) if a.size else None
        _check(self._lib.ca2_cache_debug_copy(self.handle, ptr(ring), ptr(ringv), ptr(sp), ptr(spv),
                                              _stream(stream)), "ca2_cache_debug_copy")
        return ring, ringv, sp, spv

    def ca2_qkv_proj_stage(self, x, w, tpe_rows=None, q=None, k=None, v=None,
                           targets=CA2_STAGE_RING | CA2_STAGE_SPATIAL, stream=None):
        """x: [B][n][S][c_in] bf16; w: [3C][c_in] bf16; tpe_rows: [tpe_len][3C]
        float32 or None; q/k/v: [B][n][S][H][d] bf16 outputs or None."""
        import torch
        sh = self.shape
        if x.dim() != 4 or x.dtype != torch.bfloat16 or not x.is_contiguous() or not x.is_cuda:
            raise ValueError(f"ca2_qkv_proj_stage: x must be contiguous cuda bf16 [B][n][S][c_in], got "
                             f"{x.dtype} {tuple(x.shape)}")
        B, n, S, c_in = x.shape
        C = sh["H"] * sh["d"]
        if (B, S) != (sh["B"], sh["S"]):
            raise ValueError(f"ca2_qkv_proj_stage: x shape {tuple(x.shape)} does not match the cache")
        if w.dtype != torch.bfloat16 or not w.is_contiguous() or tuple(w.shape) != (3 * C, c_in) or not w.is_cuda:
            raise ValueError(f"ca2_qkv_proj_stage: w must be contiguous cuda bf16 {(3 * C, c_in)}")
        if tpe_rows is not None and (tpe_rows.dtype != torch.float32 or not tpe_rows.is_contiguous()
                                     or tuple(tpe_rows.shape) != (sh["tpe_len"], 3 * C) or not tpe_rows.is_cuda):
            raise ValueError(f"ca2_qkv_proj_stage: tpe_rows must be contiguous cuda float32 {(sh['tpe_len'], 3 * C)}")
        for nm, t in (("q", q), ("k", k), ("v", v)):
            if t is not None:
                if t.dtype != torch.bfloat16:
                    raise ValueError(f"ca2_qkv_proj_stage: {nm} must be bf16")
                self._chk(nm, t, n)
        _check(self._lib.ca2_qkv_proj_stage(self.handle, _ptr(x), _ptr(w), _ptr(tpe_rows), _ptr(q), _ptr(k),
                                            _ptr(v), c_in, n, int(targets), _stream(stream)),
               "ca2_qkv_proj_stage")

    def ca2_cache_commit(self):
        _check(self._lib.ca2_cache_commit(self.handle), "ca2_cache_commit")
