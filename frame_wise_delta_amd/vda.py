"""Thin ctypes binding of the libvda C ABI (``include/vda.h``).

Each function has the name of the C entry point and only marshals arguments:
device buffers are passed as torch tensors (or raw integer addresses), the
stream defaults to torch's current stream.  Every step of the computation
runs in the HIP kernels of ``libvda.so``; if the library has not been built
``load()`` raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_size_t, c_uint32, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
# VDA_LIBRARY names another build of the same library (the CPU tests load the
# host-sanitizer build that way); the default is the in-tree libvda.so
LIB_PATH = os.environ.get("VDA_LIBRARY") or os.path.join(_PKG, "libvda.so")

VDA_OK = 0
VDA_ERR_NULL = -1
VDA_ERR_SHAPE = -2
VDA_ERR_DTYPE = -3
VDA_ERR_ALIGN = -4
VDA_ERR_WORKSPACE = -5
VDA_ERR_HIP = -6
VDA_ERR_DEVICE = -7
VDA_ERR_VALUE = -8

VDA_F32, VDA_BF16, VDA_F16 = 0, 1, 2
VDA_NO_BRIDGE = 1
VDA_PREP = 2
VDA_CHUNK_SCAN = 4
VDA_SANA_WM = 8
VDA_NEWTON = 16
VDA_DEV_NONFINITE, VDA_DEV_PIVOT = 1, 2

DTYPES = {"f32": VDA_F32, "bf16": VDA_BF16, "f16": VDA_F16}

EXPORTS = ("vda_workspace_bytes", "vda_state_count", "vda_index_map", "vda_index_map_device", "vda_prepare_frames",
           "vda_compose_chunks", "vda_scan_fwd", "vda_scan_rev", "vda_scan_bidir",
           "vda_readout", "vda_readout_gated", "vda_softmax_branch", "vda_forward", "vda_forward_noalloc",
           "vda_stream_read", "vda_device_status", "vda_status_string", "vda_last_error")


class vda_desc(ctypes.Structure):
    _fields_ = [
        ("heads", c_int32), ("frames", c_int32), ("tokens", c_int32),
        ("d_k", c_int32), ("d_v", c_int32), ("chunk", c_int32),
        ("anchors", c_int32), ("window", c_int32), ("text_tokens", c_int32),
        ("in_dtype", c_int32), ("out_dtype", c_int32),
        ("text_init_scale", c_float), ("flags", c_uint32),
    ]


class VdaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libvda error {code}: {msg}")
        self.code = code


_lib = None


def load(path: str | None = None):
    """Open libvda.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m frame_wise_delta_amd.build`")
    lib = ctypes.CDLL(p)
    D = POINTER(vda_desc)
    sig = {
        "vda_workspace_bytes": [D, POINTER(c_size_t)],
        "vda_state_count": [D, POINTER(c_int32)],
        "vda_index_map": [D, c_void_p, c_void_p],
        "vda_index_map_device": [D, c_void_p, c_void_p, c_void_p],
        "vda_prepare_frames": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_size_t, c_void_p],
        "vda_compose_chunks": [D, c_void_p, c_size_t, c_void_p, c_void_p],
        "vda_scan_fwd": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
        "vda_scan_rev": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
        "vda_scan_bidir": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
        "vda_readout": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
        "vda_readout_gated": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                              c_void_p, c_void_p],
        "vda_softmax_branch": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p,
                               c_void_p],
        "vda_forward": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                        c_void_p, c_void_p, c_size_t, c_void_p, c_void_p, c_void_p, c_void_p],
        "vda_forward_noalloc": [D, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
        "vda_stream_read": [c_void_p, c_size_t, c_void_p, c_int32, c_void_p],
        "vda_device_status": [D, c_void_p, c_void_p, POINTER(c_int32)],
    }
    for name, argt in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = argt
        fn.restype = c_int
    lib.vda_status_string.argtypes = [c_int]
    lib.vda_status_string.restype = c_char_p
    lib.vda_last_error.argtypes = []
    lib.vda_last_error.restype = c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(rc: int):
    if rc != VDA_OK:
        lib = load()
        raise VdaError(rc, lib.vda_last_error().decode())
    return rc


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_desc(heads, frames, tokens, d, chunk=5, anchors=1, window=1, text_tokens=0,
              in_dtype="bf16", out_dtype="bf16", text_init_scale=0.5, bridge=True, prep=False,
              chunk_scan=False, sana_wm=False, newton=False) -> vda_desc:
    return vda_desc(heads, frames, tokens, d, d, chunk, anchors, window, text_tokens,
                    DTYPES[in_dtype], DTYPES[out_dtype], text_init_scale,
                    (0 if bridge else VDA_NO_BRIDGE) | (VDA_PREP if prep else 0) |
                    (VDA_CHUNK_SCAN if chunk_scan else 0) | (VDA_SANA_WM if sana_wm else 0) |
                    (VDA_NEWTON if newton else 0))


def desc_for(cfg, **over) -> vda_desc:
    """Descriptor of an ``inputs.Config`` (fields may be overridden)."""
    kw = dict(heads=cfg.heads, frames=cfg.frames, tokens=cfg.tokens, d=cfg.d, chunk=cfg.chunk,
              anchors=cfg.anchors, window=cfg.window, text_tokens=cfg.text_tokens,
              in_dtype=cfg.in_dtype, out_dtype=cfg.out_dtype)
    kw.update(over)
    return make_desc(**kw)


# ------------------------------------------------------------ entry points --

def vda_workspace_bytes(desc: vda_desc) -> int:
    n = c_size_t(0)
    _check(load().vda_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def vda_state_count(desc: vda_desc) -> int:
    n = c_int32(0)
    _check(load().vda_state_count(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def vda_index_map(desc: vda_desc):
    """Host-side maps -> (chunk_rows int32 [C, 7], frame_chunk int32 [T]) numpy arrays."""
    import numpy as np
    n = desc.frames - 2 * desc.anchors
    C = -(-n // desc.chunk) if n > 0 else 0
    rows = np.zeros((max(C, 0), 7), dtype=np.int32)
    fc = np.zeros((max(desc.frames, 0),), dtype=np.int32)
    _check(load().vda_index_map(ctypes.byref(desc), rows.ctypes.data if rows.size else None,
                                fc.ctypes.data if fc.size else None))
    return rows, fc


def vda_index_map_device(desc: vda_desc, chunk_rows, frame_chunk, stream=None):
    """The maps computed on the device into int32 device tensors
    chunk_rows [C, 7] and frame_chunk [T]."""
    _check(load().vda_index_map_device(ctypes.byref(desc), _ptr(chunk_rows) if chunk_rows.numel() else None,
                                       _ptr(frame_chunk) if frame_chunk.numel() else None, _stream(stream)))


def vda_prepare_frames(desc, k, v, beta, k_text, v_text, beta_text, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().vda_prepare_frames(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(beta), _ptr(k_text),
                                     _ptr(v_text), _ptr(beta_text), _ptr(ws), ws_bytes, _stream(stream)))


def vda_compose_chunks(desc, ws, alpha, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().vda_compose_chunks(ctypes.byref(desc), _ptr(ws), ws_bytes, _ptr(alpha), _stream(stream)))


def vda_scan_fwd(desc, ws, alpha, s_init, states, stream=None):
    _check(load().vda_scan_fwd(ctypes.byref(desc), _ptr(ws), _ptr(alpha), _ptr(s_init), _ptr(states),
                               _stream(stream)))


def vda_scan_rev(desc, ws, alpha, s_init, states, stream=None):
    _check(load().vda_scan_rev(ctypes.byref(desc), _ptr(ws), _ptr(alpha), _ptr(s_init), _ptr(states),
                               _stream(stream)))


def vda_scan_bidir(desc, ws, alpha, s_init, states_fwd, states_rev, stream=None):
    _check(load().vda_scan_bidir(ctypes.byref(desc), _ptr(ws), _ptr(alpha), _ptr(s_init), _ptr(states_fwd),
                                 _ptr(states_rev), _stream(stream)))


def vda_readout(desc, q, alpha, states_fwd, states_rev, out, stream=None):
    _check(load().vda_readout(ctypes.byref(desc), _ptr(q), _ptr(alpha), _ptr(states_fwd),
                              _ptr(states_rev), _ptr(out), _stream(stream)))


def vda_readout_gated(desc, q, alpha, states_fwd, states_rev, gate, norm_weight, eps, out, stream=None):
    _check(load().vda_readout_gated(ctypes.byref(desc), _ptr(q), _ptr(alpha), _ptr(states_fwd),
                                    _ptr(states_rev), _ptr(gate), _ptr(norm_weight), float(eps), _ptr(out),
                                    _stream(stream)))


def vda_softmax_branch(desc, q, k, v, k_text, v_text, scale, out, v_dtype="bf16", stream=None):
    _check(load().vda_softmax_branch(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_text), _ptr(v_text),
                                     DTYPES[v_dtype], float(scale), _ptr(out), _stream(stream)))


def vda_forward(desc, q, k, v, beta, alpha, k_text, v_text, beta_text, ws, states_fwd, states_rev, out,
                ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().vda_forward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
                              _ptr(k_text), _ptr(v_text), _ptr(beta_text), _ptr(ws), ws_bytes,
                              _ptr(states_fwd), _ptr(states_rev), _ptr(out), _stream(stream)))


def vda_forward_noalloc(desc, q, k, v, beta, alpha, k_text, v_text, beta_text, states_fwd, states_rev, out,
                        status=None, stream=None):
    """vda_forward with the library's own device workspace (no allocation);
    status: None or a device int32 tensor receiving the device status word."""
    _check(load().vda_forward_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
                                      _ptr(k_text), _ptr(v_text), _ptr(beta_text), _ptr(states_fwd),
                                      _ptr(states_rev), _ptr(out), _ptr(status), _stream(stream)))


def vda_stream_read(src, sink, blocks, stream=None):
    """Read every byte of the device tensor src (measurement aid)."""
    _check(load().vda_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), blocks, _stream(stream)))


def vda_device_status(desc, ws, stream=None) -> int:
    f = c_int32(0)
    _check(load().vda_device_status(ctypes.byref(desc), _ptr(ws), _stream(stream), ctypes.byref(f)))
    return f.value


def vda_status_string(code: int) -> str:
    return load().vda_status_string(code).decode()


def vda_last_error() -> str:
    return load().vda_last_error().decode()
