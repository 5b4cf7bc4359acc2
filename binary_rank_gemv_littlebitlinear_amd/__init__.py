"""Python binding of the LittleBit linear-forward C ABI (``include/lb.h``).

Argument marshalling only: every step of the forward runs in the HIP
library ``liblb.so`` built next to this file.  There is no fallback: if
the library is missing, loading fails loudly.  torch is used for device
memory and streams only (tensors are passed as raw pointers).

Functions keep the C names (``lb_create``, ``lb_pack_signs``, ...);
``Layer`` and ``Stack`` are thin owners that call them.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblb.so")

LB_OK, LB_EINVAL, LB_ENOMEM, LB_EHIP, LB_ENOTREADY, LB_EUNSUPPORTED, LB_ETIMEOUT = 0, -1, -2, -3, -4, -5, -6


class LBError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load liblb.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run python -m binary_rank_gemv_littlebitlinear_amd.build)")
    lib = C.CDLL(path)
    vp, i64, i32, u64 = C.c_void_p, C.c_int64, C.c_int, C.c_uint64
    P = C.POINTER
    sig = {
        "lb_create": ([i64, i64, i64, i32, P(vp)], i32),
        "lb_pack_signs": ([vp, i32, vp, vp], i32),
        "lb_set_scales": ([vp, i32, vp, vp, vp], i32),
        "lb_forward": ([vp, vp, vp, i64, vp], i32),
        "lb_forward_noalloc": ([vp, vp, vp, i64, vp], i32),
        "lb_unpack_signs": ([vp, i32, vp, vp], i32),
        "lb_get_scales": ([vp, i32, vp, vp, vp], i32),
        "lb_init_from_factors": ([vp, i32, vp, vp, vp, vp], i32),
        "lb_joint_itq": ([vp, vp, i64, i64, i64, i32, vp, vp, vp], i32),
        "lb_layer_shape": ([vp, P(i64), P(i64), P(i64), P(i32)], i32),
        "lb_prepare": ([vp, i64], i32),
        "lb_layer_device_bytes": ([vp, P(u64), P(u64)], i32),
        "lb_destroy": ([vp], i32),
        "lb_forward_stage1": ([vp, vp, vp, i64, vp], i32),
        "lb_forward_stage2": ([vp, vp, vp, i64, vp], i32),
        "lb_eff_bits": ([i64, i64, i64, i32, P(u64), P(u64)], i32),
        "lb_rank_for_bpw": ([i64, i64, u64, u64, i32, P(i64)], i32),
        "lb_stack_create": ([vp, i32, vp, i32, C.c_float, P(vp)], i32),
        "lb_stack_forward": ([vp, vp, vp, vp, i64, vp], i32),
        "lb_stack_trace_elems": ([vp, i64, P(i64)], i32),
        "lb_stack_reserve": ([vp, i64], i32),
        "lb_stack_set_mode": ([vp, i32], i32),
        "lb_stack_check": ([vp], i32),
        "lb_stack_test_wait_failure": ([vp, i32], i32),
        "lb_stack_test_delay": ([vp, C.c_uint32, C.c_uint32], i32),
        "lb_stack_timeline": ([vp, vp, i64, P(i64)], i32),
        "lb_stack_destroy": ([vp], i32),
        "lb_status_str": ([i32], C.c_char_p),
        "lb_last_error": ([], C.c_char_p),
        "lb_version": ([], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


EXPORTED = ("lb_create", "lb_pack_signs", "lb_set_scales", "lb_forward", "lb_forward_noalloc",
            "lb_unpack_signs",
            "lb_get_scales", "lb_init_from_factors", "lb_joint_itq",
            "lb_layer_shape", "lb_prepare", "lb_layer_device_bytes", "lb_destroy", "lb_forward_stage1", "lb_forward_stage2",
            "lb_eff_bits", "lb_rank_for_bpw", "lb_stack_create", "lb_stack_forward",
            "lb_stack_trace_elems", "lb_stack_reserve", "lb_stack_set_mode", "lb_stack_check",
            "lb_stack_test_wait_failure", "lb_stack_test_delay",
            "lb_stack_timeline", "lb_stack_destroy", "lb_status_str", "lb_last_error", "lb_version")


def _status_name(st: int) -> str:
    names = {0: "LB_OK", -1: "LB_EINVAL", -2: "LB_ENOMEM", -3: "LB_EHIP", -4: "LB_ENOTREADY",
             -5: "LB_EUNSUPPORTED", -6: "LB_ETIMEOUT"}
    return names.get(st, f"status {st}")


def _check(st: int):
    if st != LB_OK:
        msg = load_library().lb_last_error().decode(errors="replace")
        raise LBError(st, msg)


def _ptr(t) -> int | None:
    """Device pointer of a torch tensor / raw int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except Exception:
            pass
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _host(arr, dtype) -> np.ndarray:
    a = np.ascontiguousarray(arr)
    if a.dtype != dtype:
        a = np.ascontiguousarray(a.view(dtype) if a.dtype.itemsize == np.dtype(dtype).itemsize else a.astype(dtype))
    return a


# ------------------------------------------------------------ raw calls
def lb_create(a: int, b: int, s: int, residual: bool) -> int:
    out = C.c_void_p()
    _check(load_library().lb_create(a, b, s, int(bool(residual)), C.byref(out)))
    return out.value


def lb_pack_signs(layer: int, path: int, su_words, sv_words):
    su = _host(su_words, np.uint32)
    sv = _host(sv_words, np.uint32)
    _check(load_library().lb_pack_signs(layer, path, su.ctypes.data, sv.ctypes.data))


def lb_set_scales(layer: int, path: int, h, g, l):
    hh = _host(np.asarray(h, np.float16), np.uint16)
    gg = _host(np.asarray(g, np.float16), np.uint16)
    ll = _host(np.asarray(l, np.float16), np.uint16)
    _check(load_library().lb_set_scales(layer, path, hh.ctypes.data, gg.ctypes.data, ll.ctypes.data))


def lb_forward(layer: int, x, y, M: int, stream=None):
    _check(load_library().lb_forward(layer, _ptr(x), _ptr(y), int(M), _stream(stream)))


def lb_forward_noalloc(layer: int, x, y, M: int, stream=None):
    _check(load_library().lb_forward_noalloc(layer, _ptr(x), _ptr(y), int(M), _stream(stream)))


def lb_forward_stage1(layer: int, x, w, M: int, stream=None):
    _check(load_library().lb_forward_stage1(layer, _ptr(x), _ptr(w), int(M), _stream(stream)))


def lb_forward_stage2(layer: int, w, y, M: int, stream=None):
    _check(load_library().lb_forward_stage2(layer, _ptr(w), _ptr(y), int(M), _stream(stream)))


def lb_unpack_signs(layer: int, path: int):
    a, b, s, _ = lb_layer_shape(layer)
    wk = (s + 31) // 32
    su = np.zeros((b, wk), np.uint32)
    sv = np.zeros((a, wk), np.uint32)
    _check(load_library().lb_unpack_signs(layer, path, su.ctypes.data, sv.ctypes.data))
    return su, sv


def lb_get_scales(layer: int, path: int):
    """(h, g, l) of one path as fp16 arrays."""
    a, b, s, _ = lb_layer_shape(layer)
    h = np.zeros(b, np.uint16)
    g = np.zeros(a, np.uint16)
    l = np.zeros(s, np.uint16)
    _check(load_library().lb_get_scales(layer, path, h.ctypes.data, g.ctypes.data, l.ctypes.data))
    return h.view(np.float16), g.view(np.float16), l.view(np.float16)


def _check_dev(name, t, shape, dtype):
    if isinstance(t, int) or t is None:
        return
    if (t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda"
            or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of shape {shape}")


def lb_init_from_factors(layer: int, path: int, U, V, R=None, stream=None):
    """Signs and scales of one path from device fp32 factors U (b x s), V (a x s),
    rotated first by the device fp64 rotation R (s x s) when given."""
    import torch
    a, b, s, _ = lb_layer_shape(layer)
    _check_dev("U", U, (b, s), torch.float32)
    _check_dev("V", V, (a, s), torch.float32)
    _check_dev("R", R, (s, s), torch.float64)
    _check(load_library().lb_init_from_factors(layer, path, _ptr(U), _ptr(V), _ptr(R),
                                               _stream(stream)))


def lb_joint_itq(U, V, iters: int = 50, R0=None, stream=None):
    """Joint-ITQ rotation (device fp64 s x s tensor) of device fp32 factors U (b x s), V (a x s)."""
    import torch
    b, s = U.shape
    a = V.shape[0]
    _check_dev("U", U, (b, s), torch.float32)
    _check_dev("V", V, (a, s), torch.float32)
    _check_dev("R0", R0, (s, s), torch.float64)
    R = torch.empty((s, s), dtype=torch.float64, device=U.device)
    _check(load_library().lb_joint_itq(_ptr(U), _ptr(V), a, b, s, int(iters), _ptr(R0), _ptr(R),
                                       _stream(stream)))
    return R


def lb_layer_shape(layer: int):
    a, b, s, r = C.c_int64(), C.c_int64(), C.c_int64(), C.c_int()
    _check(load_library().lb_layer_shape(layer, C.byref(a), C.byref(b), C.byref(s), C.byref(r)))
    return a.value, b.value, s.value, bool(r.value)


def lb_prepare(layer: int, M: int):
    _check(load_library().lb_prepare(layer, int(M)))


def lb_layer_device_bytes(layer: int):
    sb, tb = C.c_uint64(), C.c_uint64()
    _check(load_library().lb_layer_device_bytes(layer, C.byref(sb), C.byref(tb)))
    return sb.value, tb.value


def lb_destroy(layer: int):
    _check(load_library().lb_destroy(layer))


def lb_eff_bits(a: int, b: int, s: int, residual: bool):
    n, d = C.c_uint64(), C.c_uint64()
    _check(load_library().lb_eff_bits(a, b, s, int(bool(residual)), C.byref(n), C.byref(d)))
    return n.value, d.value


def lb_rank_for_bpw(a: int, b: int, bpw_num: int, bpw_den: int, residual: bool) -> int:
    s = C.c_int64()
    _check(load_library().lb_rank_for_bpw(a, b, bpw_num, bpw_den, int(bool(residual)), C.byref(s)))
    return s.value


def lb_stack_create(layers, unit_sizes, kappa: float) -> int:
    arr = (C.c_void_p * len(layers))(*layers)
    us = np.ascontiguousarray(unit_sizes, dtype=np.int32)
    out = C.c_void_p()
    _check(load_library().lb_stack_create(C.cast(arr, C.c_void_p), len(layers), us.ctypes.data,
                                          len(us), float(kappa), C.byref(out)))
    return out.value


def lb_stack_forward(stack: int, x0, y, trace, M: int, stream=None):
    _check(load_library().lb_stack_forward(stack, _ptr(x0), _ptr(y), _ptr(trace), int(M),
                                           _stream(stream)))


def lb_stack_trace_elems(stack: int, M: int) -> int:
    n = C.c_int64()
    _check(load_library().lb_stack_trace_elems(stack, int(M), C.byref(n)))
    return n.value


def lb_stack_reserve(stack: int, M: int):
    _check(load_library().lb_stack_reserve(stack, int(M)))


def lb_stack_set_mode(stack: int, mode: int):
    _check(load_library().lb_stack_set_mode(stack, int(mode)))


def lb_stack_test_wait_failure(stack: int, enable: bool):
    _check(load_library().lb_stack_test_wait_failure(stack, int(bool(enable))))


def lb_stack_test_delay(stack: int, seed: int, max_ticks: int):
    _check(load_library().lb_stack_test_delay(stack, int(seed), int(max_ticks)))


def lb_stack_check(stack: int):
    _check(load_library().lb_stack_check(stack))


def lb_stack_timeline(stack: int, buf=None, capacity: int = 0) -> int:
    n = C.c_int64()
    _check(load_library().lb_stack_timeline(stack, _ptr(buf), int(capacity), C.byref(n)))
    return n.value


def lb_stack_destroy(stack: int):
    _check(load_library().lb_stack_destroy(stack))


# --------------------------------------------------------------- owners
class Layer:
    """Owner of one lb_layer handle."""

    def __init__(self, a: int, b: int, s: int, residual: bool):
        self.a, self.b, self.s, self.residual = a, b, s, bool(residual)
        self.handle = lb_create(a, b, s, residual)

    @classmethod
    def from_paths(cls, paths):
        p0 = paths[0]
        L = cls(p0["a"], p0["b"], p0["s"], len(paths) == 2)
        for i, p in enumerate(paths):
            lb_pack_signs(L.handle, i, p["su"], p["sv"])
            lb_set_scales(L.handle, i, p["h"], p["g"], p["l"])
        return L

    def forward(self, x, y, M=None, stream=None):
        lb_forward(self.handle, x, y, x.shape[0] if M is None else M, stream)

    def prepare(self, M: int):
        lb_prepare(self.handle, M)

    def device_bytes(self):
        """(sign bytes, total bytes) the layer holds on the device."""
        return lb_layer_device_bytes(self.handle)

    def close(self):
        if self.handle:
            lb_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Stack:
    """Owner of one lb_stack handle (keeps its layers alive)."""

    def __init__(self, layers, unit_sizes, kappa: float):
        self.layers = list(layers)
        self.unit_sizes = list(unit_sizes)
        self.handle = lb_stack_create([L.handle for L in self.layers], self.unit_sizes, kappa)

    def forward(self, x0, y, trace=None, M=None, stream=None):
        lb_stack_forward(self.handle, x0, y, trace, x0.shape[0] if M is None else M, stream)

    def trace_elems(self, M: int) -> int:
        return lb_stack_trace_elems(self.handle, M)

    def set_mode(self, mode: int):
        lb_stack_set_mode(self.handle, mode)

    def reserve(self, M: int):
        lb_stack_reserve(self.handle, M)

    def check(self):
        lb_stack_check(self.handle)

    def close(self):
        if self.handle:
            lb_stack_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lb_status_str(status: int) -> str:
    return load_library().lb_status_str(int(status)).decode()


def lb_last_error() -> str:
    return load_library().lb_last_error().decode(errors="replace")


def lb_version() -> int:
    return load_library().lb_version()
