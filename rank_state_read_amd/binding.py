"""ctypes binding of libsketchssm.so: the C entry points under the same names.

Argument marshalling only: tensors become device pointers, the stream defaults
to torch's current stream, and a non-OK status raises ``SketchSSMError``.  Every
step of the decode path runs in the HIP library; if the library is not built
this module raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsketchssm.so")

KIND = {"mamba2": 0, "gdn": 1, "kda": 2}
DTYPE = {"bf16": 0, "f32": 1}
STATUS = {0: "SKSSM_OK", 1: "SKSSM_EINVAL", 2: "SKSSM_ESHAPE", 3: "SKSSM_EALIGN",
          4: "SKSSM_ENOMEM", 5: "SKSSM_EDEVICE", 6: "SKSSM_ELAUNCH"}

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p
c_i32p = ctypes.POINTER(ctypes.c_int32)


class SketchSSMError(RuntimeError):
    def __init__(self, where: str, status: int):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


class Shape(ctypes.Structure):
    _fields_ = [("B", c_i32), ("H", c_i32), ("K", c_i32), ("V", c_i32), ("W", c_i32),
                ("G", c_i32), ("basis_rows", c_i32), ("rank_cap", c_i32), ("kind", c_i32),
                ("qkv", c_i32), ("kq_heads", c_i32)]


_lib = None

_PROTOS = {
    "sketchssm_plan_create": (c_i32, [ctypes.POINTER(Shape), c_i32p, c_i32p, ctypes.POINTER(c_vp)]),
    "sketchssm_plan_create_ordered": (c_i32, [ctypes.POINTER(Shape), c_i32p, c_i32p, c_i32p,
                                              ctypes.POINTER(c_vp)]),
    "sketchssm_plan_export": (c_i32, [c_vp] + [c_i32p] * 8),
    "sketchssm_plan_destroy": (None, [c_vp]),
    "sketchssm_z_elems": (ctypes.c_size_t, [c_vp]),
    "sketchssm_frame_elems": (ctypes.c_size_t, [c_vp]),
    "sketchssm_flush": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp]),
    "sketchssm_decode_read": (c_i32, [c_vp] * 13 + [c_i32, c_vp, c_vp]),
    "sketchssm_dense_read": (c_i32, [ctypes.POINTER(Shape)] + [c_vp] * 10 + [c_i32, c_vp, c_vp]),
    "sketchssm_rmw_step": (c_i32, [ctypes.POINTER(Shape)] + [c_vp] * 8),
    "sketchssm_decode_read_seq": (c_i32, [c_vp] * 16),
    "sketchssm_flush_seq": (c_i32, [c_vp] * 10 + [c_i32, c_vp]),
    "sketchssm_decode_read_flush": (c_i32, [c_vp] * 16),
    "sketchssm_status_string": (ctypes.c_char_p, [c_i32]),
    "sketchssm_stream_probe": (c_i32, [c_vp, ctypes.c_size_t, c_vp, ctypes.c_size_t, c_i32, c_i32, c_i32, c_vp]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rank_state_read_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sketchssm_status_string(int(status)).decode()


def _check(where: str, st: int):
    if st != 0:
        raise SketchSSMError(where, st)


def make_shape(B, H, K, V, W, G, basis_rows, rank_cap, kind, qkv, kq_heads=0) -> Shape:
    return Shape(int(B), int(H), int(K), int(V), int(W), int(G), int(basis_rows), int(rank_cap),
                 KIND[kind] if isinstance(kind, str) else int(kind),
                 DTYPE[qkv] if isinstance(qkv, str) else int(qkv), int(kq_heads or 0))


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (None -> NULL).  Integers pass through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("expected a device tensor")
    if not x.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owner of a ``sketchssm_plan`` (host only)."""

    def __init__(self, shape: Shape, rank, group, order=None):
        self.shape = shape
        r = np.ascontiguousarray(rank, dtype=np.int32)
        g = np.ascontiguousarray(group, dtype=np.int32)
        if shape.H >= 1 and (r.shape != (shape.H,) or g.shape != (shape.H,)):
            raise ValueError("rank and group must have H entries")
        h = c_vp()
        if order is None:
            _check("sketchssm_plan_create",
                   lib().sketchssm_plan_create(ctypes.byref(shape), r.ctypes.data_as(c_i32p),
                                               g.ctypes.data_as(c_i32p), ctypes.byref(h)))
        else:
            o = np.ascontiguousarray(order, dtype=np.int32)
            if o.shape != (shape.H,):
                raise ValueError("order must have H entries")
            _check("sketchssm_plan_create_ordered",
                   lib().sketchssm_plan_create_ordered(ctypes.byref(shape), r.ctypes.data_as(c_i32p),
                                                       g.ctypes.data_as(c_i32p), o.ctypes.data_as(c_i32p),
                                                       ctypes.byref(h)))
        self.handle = h.value
        self.rank = r.copy()
        self.group = g.copy()

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.sketchssm_plan_destroy(h)
            self.handle = None

    @property
    def z_elems(self) -> int:
        return int(lib().sketchssm_z_elems(self.handle))

    @property
    def frame_elems(self) -> int:
        return int(lib().sketchssm_frame_elems(self.handle))

    def export(self) -> dict:
        H = self.shape.H
        n = c_i32()
        fi = np.zeros(H, np.int32)
        zo = np.zeros(H + 1, np.int32)
        bk = np.zeros(H, np.int32)
        od = np.zeros(H, np.int32)
        fg = np.zeros(H, np.int32)
        fr = np.zeros(H, np.int32)
        fo = np.zeros(H + 1, np.int32)
        P = lambda a: a.ctypes.data_as(c_i32p)  # noqa: E731
        _check("sketchssm_plan_export",
               lib().sketchssm_plan_export(self.handle, P(fi), P(fo), P(zo), P(bk), P(od), P(fg), P(fr),
                                           ctypes.byref(n)))
        F = n.value
        return {"frame_index": fi, "frame_row_off": fo[:F + 1], "z_row_off": zo, "bucket": bk,
                "order": od, "frames": list(zip(fg[:F].tolist(), fr[:F].tolist())), "n_frames": F}


def sketchssm_flush(plan: Plan, S, Z, basis, kbuf, vbuf, abuf, bbuf, n_tokens: int, stream=None):
    _check("sketchssm_flush",
           lib().sketchssm_flush(plan.handle, _ptr(S), _ptr(Z), _ptr(basis), _ptr(kbuf), _ptr(vbuf),
                                 _ptr(abuf), _ptr(bbuf), int(n_tokens), _stream(stream)))


def sketchssm_decode_read(plan: Plan, S, Z, frames, q, k, v, a, beta, kbuf, vbuf, abuf, bbuf,
                          pos: int, y, stream=None):
    _check("sketchssm_decode_read",
           lib().sketchssm_decode_read(plan.handle, _ptr(S), _ptr(Z), _ptr(frames), _ptr(q), _ptr(k),
                                       _ptr(v), _ptr(a), _ptr(beta), _ptr(kbuf), _ptr(vbuf),
                                       _ptr(abuf), _ptr(bbuf), int(pos), _ptr(y), _stream(stream)))


def sketchssm_dense_read(shape: Shape, S, q, k, v, a, beta, kbuf, vbuf, abuf, bbuf, pos: int, y,
                         stream=None):
    _check("sketchssm_dense_read",
           lib().sketchssm_dense_read(ctypes.byref(shape), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                      _ptr(beta), _ptr(kbuf), _ptr(vbuf), _ptr(abuf), _ptr(bbuf),
                                      int(pos), _ptr(y), _stream(stream)))


def sketchssm_rmw_step(shape: Shape, S, q, k, v, a, beta, y, stream=None):
    _check("sketchssm_rmw_step",
           lib().sketchssm_rmw_step(ctypes.byref(shape), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                    _ptr(beta), _ptr(y), _stream(stream)))


def sketchssm_decode_read_seq(plan: Plan, S, Z, frames, q, k, v, a, beta, kbuf, vbuf, abuf, bbuf, pos,
                              y, stream=None):
    _check("sketchssm_decode_read_seq",
           lib().sketchssm_decode_read_seq(plan.handle, _ptr(S), _ptr(Z), _ptr(frames), _ptr(q), _ptr(k),
                                           _ptr(v), _ptr(a), _ptr(beta), _ptr(kbuf), _ptr(vbuf),
                                           _ptr(abuf), _ptr(bbuf), _ptr(pos), _ptr(y), _stream(stream)))


def sketchssm_flush_seq(plan: Plan, S, Z, basis, kbuf, vbuf, abuf, bbuf, seqs, n_tokens, n_seqs: int,
                        stream=None):
    _check("sketchssm_flush_seq",
           lib().sketchssm_flush_seq(plan.handle, _ptr(S), _ptr(Z), _ptr(basis), _ptr(kbuf), _ptr(vbuf),
                                     _ptr(abuf), _ptr(bbuf), _ptr(seqs), _ptr(n_tokens), int(n_seqs),
                                     _stream(stream)))


def sketchssm_decode_read_flush(plan: Plan, S, Z, frames, basis, q, k, v, a, beta, kbuf, vbuf, abuf, bbuf, y,
                                stream=None):
    _check("sketchssm_decode_read_flush",
           lib().sketchssm_decode_read_flush(plan.handle, _ptr(S), _ptr(Z), _ptr(frames), _ptr(basis), _ptr(q),
                                             _ptr(k), _ptr(v), _ptr(a), _ptr(beta), _ptr(kbuf), _ptr(vbuf),
                                             _ptr(abuf), _ptr(bbuf), _ptr(y), _stream(stream)))


def sketchssm_stream_probe(src, read_bytes: int, dst, write_bytes: int, unroll: int = 8, blocks: int = 0,
                           nontemporal: bool = False, stream=None):
    """Measurement aid (include/sketchssm_measure.h): stream read_bytes of src,
    writing write_bytes of sums to dst."""
    _check("sketchssm_stream_probe",
           lib().sketchssm_stream_probe(_ptr(src), int(read_bytes), _ptr(dst), int(write_bytes), int(unroll),
                                        int(blocks), 1 if nontemporal else 0, _stream(stream)))
