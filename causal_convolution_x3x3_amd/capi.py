"""ctypes declarations of the C ABI in include/cc3d.h (argument marshalling only).

Loading fails loudly when libcc3d.so has not been built: there is no fallback
path of any kind.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcc3d.so")

OK, EINVAL, ESHAPE, EDTYPE, ESTATE, ENOMEM, EDEVICE = range(7)
STATUS_NAMES = {0: "OK", 1: "EINVAL", 2: "ESHAPE", 3: "EDTYPE", 4: "ESTATE", 5: "ENOMEM", 6: "EDEVICE"}
F32, BF16 = 0, 1
TPAD_REPLICATE, TPAD_ZERO = 0, 1
EPI_NONE, EPI_RESIDUAL, EPI_ACT, EPI_U8 = 0, 1, 2, 4
GROW_ONCE, GROW_ALIGNED = 0, 1
SLOT_NONE, SLOT_X, SLOT_Y, SLOT_AUX = -1, 0, 1, 2
MAX_SLOTS, MAX_OPS = 64, 256
OP_CONV, OP_NORM_ACT = 0, 1

EXPORTS = (
    "cc3d_plan_create", "cc3d_stack_plan_create", "cc3d_plan_destroy", "cc3d_state_bytes",
    "cc3d_plan_device_bytes", "cc3d_output_elem_bytes", "cc3d_output_shape", "cc3d_reset", "cc3d_forward_chunk",
    "cc3d_to_channels_last", "cc3d_to_channels_first", "cc3d_last_error", "cc3d_version",
    "cc3d_profile_enable", "cc3d_plan_num_ops", "cc3d_profile_read", "cc3d_slot_shape", "cc3d_slot_read",
    "cc3d_conv_forward_noalloc",
)
NOALLOC_SCRATCH_BYTES = 64 << 20


class ConvDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "cin", "cout", "kt", "kh", "kw", "h_in", "w_in", "up_s", "up_t", "max_chunk_t",
        "dtype", "tpad", "epilogue")] + [("eps", ctypes.c_float), ("grow", ctypes.c_int),
                                         ("fold_upsample", ctypes.c_int), ("stride_s", ctypes.c_int),
                                         ("stride_t", ctypes.c_int)]


class State(ctypes.Structure):
    _fields_ = [("arena", ctypes.c_void_p), ("frames_seen", ctypes.c_int64)]


class OpDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "kind", "cout", "kt", "kh", "kw", "up_s", "up_t", "tpad", "src", "res", "out", "act_out")] + [
        ("w", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("out_u8", ctypes.c_int),
        ("stride_s", ctypes.c_int), ("stride_t", ctypes.c_int)]


class StackDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("cin", ctypes.c_int), ("h", ctypes.c_int),
                ("w", ctypes.c_int), ("max_chunk_t", ctypes.c_int), ("eps", ctypes.c_float),
                ("n_ops", ctypes.c_int), ("ops", ctypes.POINTER(OpDesc)), ("grow", ctypes.c_int),
                ("batch_from", ctypes.c_int), ("frame_batch", ctypes.c_int), ("fold_upsample", ctypes.c_int)]


class OpProfile(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char * 64), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


class Cc3dError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__("%s failed with %s: %s" % (where, STATUS_NAMES.get(status, status), message))


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libcc3d.so is not built (%s missing); run `python -m causal_convolution_x3x3_amd.build`"
                % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        pi = ctypes.POINTER(ctypes.c_int)
        sigs = {
            "cc3d_plan_create": (i, [ctypes.POINTER(ConvDesc), vp, vp, vp, vp, ctypes.POINTER(vp)]),
            "cc3d_stack_plan_create": (i, [ctypes.POINTER(StackDesc), vp, ctypes.POINTER(vp)]),
            "cc3d_plan_destroy": (None, [vp]),
            "cc3d_state_bytes": (sz, [vp]),
            "cc3d_plan_device_bytes": (sz, [vp]),
            "cc3d_output_elem_bytes": (i, [vp]),
            "cc3d_output_shape": (i, [vp, i, i, pi, pi, pi, pi]),
            "cc3d_reset": (i, [vp, ctypes.POINTER(State), vp]),
            "cc3d_forward_chunk": (i, [vp, vp, i, ctypes.POINTER(State), ctypes.POINTER(State), vp, vp, vp]),
            "cc3d_to_channels_last": (i, [vp, vp, i, i, i, i, i, vp]),
            "cc3d_to_channels_first": (i, [vp, vp, i, i, i, i, i, vp]),
            "cc3d_profile_enable": (i, [vp, i]),
            "cc3d_plan_num_ops": (i, [vp]),
            "cc3d_profile_read": (i, [vp, i, i, ctypes.POINTER(OpProfile)]),
            "cc3d_slot_shape": (i, [vp, i, i, i, pi, pi, pi, pi]),
            "cc3d_slot_read": (i, [vp, i, i, i, vp, sz, vp]),
            "cc3d_conv_forward_noalloc": (i, [ctypes.POINTER(ConvDesc), vp, vp, vp, vp, i, ctypes.POINTER(State),
                                              ctypes.POINTER(State), vp, vp, vp]),
            "cc3d_last_error": (ctypes.c_char_p, []),
            "cc3d_version": (i, []),
        }
        for name, (res, args) in sigs.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().cc3d_last_error().decode()


def check(status: int, where: str):
    if status != OK:
        raise Cc3dError(status, where, last_error())
