"""Thin torch-facing wrappers over the C ABI: torch supplies device memory and the
stream, the library does every step of the path.

Activations are channels-last: a chunk is a [T, H, W, C] tensor (bf16 or fp32)
on the plan's device.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import List, Optional

import torch

from . import capi as C

_DT = {torch.bfloat16: C.BF16, torch.float32: C.F32}
_TD = {C.BF16: torch.bfloat16, C.F32: torch.float32}


def _numel(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _check_arena(s: "State", nbytes: int, what: str):
    """A state's arena must hold the plan's cc3d_state_bytes: the library writes
    the caches through the bare pointer."""
    a = s.arena
    if a.dtype != torch.uint8 or a.dim() != 1 or a.numel() < nbytes or not a.is_contiguous():
        raise ValueError("%s must be a contiguous byte arena of at least %d bytes, got %s of %s"
                         % (what, nbytes, tuple(a.shape), a.dtype))


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class State:
    """One causal state arena (device bytes) and its frame counter."""

    def __init__(self, nbytes: int, device):
        self.arena = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        self.frames_seen = 0

    def _c(self) -> C.State:
        return C.State(ctypes.c_void_p(self.arena.data_ptr()), self.frames_seen)

    def copy_(self, other: "State") -> "State":
        """Checkpoint/restore: copy another state's arena and counter."""
        self.arena.copy_(other.arena)
        self.frames_seen = other.frames_seen
        return self


@dataclass
class Op:
    """One op of a stack (see cc3d_op_desc).  A CONV op's kernel size ``k`` is
    taken from its weights [Cout][Cin][kt][kh][kw]."""
    kind: int = C.OP_CONV
    cout: int = 0
    k: tuple = (1, 1, 1)
    up_s: int = 1
    up_t: int = 1
    tpad: int = C.TPAD_REPLICATE
    src: int = C.SLOT_X
    res: int = C.SLOT_NONE
    out: int = C.SLOT_NONE
    act_out: int = C.SLOT_NONE
    w: Optional[torch.Tensor] = None
    bias: Optional[torch.Tensor] = None
    gamma: Optional[torch.Tensor] = None
    out_u8: bool = False  # CONV writing the output slot: y as 8-bit codes
    stride_s: int = 1     # CONV: spatial stride (1 or 2; see cc3d_op_desc)
    stride_t: int = 1     # CONV: temporal stride (1 or 2)
    name: str = field(default="")

    def __post_init__(self):
        if self.kind == C.OP_CONV and self.w is not None:
            if self.w.dim() != 5 or self.w.shape[0] != self.cout:
                raise ValueError("op %s: weights %s are not [cout=%d][cin][kt][kh][kw]"
                                 % (self.name, tuple(self.w.shape), self.cout))
            self.k = tuple(int(d) for d in self.w.shape[2:])


class Plan:
    """A created plan (single conv or stack) with its forward/reset calls.
    ``cin``, ``h``, ``w``: the chunk input's channels and frame size; x is
    [T][h][w][cin] of the plan dtype."""

    def __init__(self, handle: ctypes.c_void_p, dtype: int, device, cin: int, h: int, w: int, op_names=None):
        self._h = handle
        self.op_names = list(op_names or [])  # per op of the library's list (profiles name them)
        self.dtype = dtype
        self.device = device
        self.in_shape = (int(h), int(w), int(cin))
        L = C.lib()
        self.state_bytes = int(L.cc3d_state_bytes(self._h))
        self.device_bytes = int(L.cc3d_plan_device_bytes(self._h))
        self.out_dtype = torch.uint8 if L.cc3d_output_elem_bytes(self._h) == 1 else _TD[dtype]
        # whether forward_chunk reads a residual argument (the residual slot is
        # defined; ESHAPE: defined, but a one-frame first chunk is not a whole
        # count for the plan's strided convs)
        self.takes_residual = L.cc3d_slot_shape(self._h, C.SLOT_AUX, 1, 1, None, None, None, None) in (C.OK,
                                                                                                     C.ESHAPE)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                torch.cuda.synchronize(self.device)
            except Exception:
                pass
            C.lib().cc3d_plan_destroy(h)
            self._h = None

    def new_state(self) -> State:
        return State(self.state_bytes, self.device)

    def output_shape(self, t_chunk: int, first: bool):
        c, t, h, w = (ctypes.c_int() for _ in range(4))
        C.check(C.lib().cc3d_output_shape(self._h, t_chunk, int(first), ctypes.byref(c), ctypes.byref(t),
                                          ctypes.byref(h), ctypes.byref(w)), "cc3d_output_shape")
        return (t.value, h.value, w.value, c.value)

    def slot_shape(self, slot: int, t_chunk: int, first: bool):
        c, t, h, w = (ctypes.c_int() for _ in range(4))
        C.check(C.lib().cc3d_slot_shape(self._h, slot, t_chunk, int(first), ctypes.byref(c), ctypes.byref(t),
                                        ctypes.byref(h), ctypes.byref(w)), "cc3d_slot_shape")
        return (t.value, h.value, w.value, c.value)

    def read_slot(self, slot: int, t_chunk: int, first: bool, stream=None) -> torch.Tensor:
        """Copy of an intermediate slot as the last forward_chunk left it ([T][H][W][C])."""
        shape = self.slot_shape(slot, t_chunk, first)
        out = torch.empty(shape, dtype=_TD[self.dtype], device=self.device)
        C.check(C.lib().cc3d_slot_read(self._h, slot, t_chunk, int(first), _ptr(out),
                                       out.numel() * out.element_size(), _stream(stream)), "cc3d_slot_read")
        return out

    def reset(self, state: State, stream=None):
        _check_arena(state, self.state_bytes, "state")
        cs = state._c()
        C.check(C.lib().cc3d_reset(self._h, ctypes.byref(cs), _stream(stream)), "cc3d_reset")
        state.frames_seen = cs.frames_seen

    def forward_chunk(self, x: torch.Tensor, cache_in: State, cache_out: State,
                      residual: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
        """Decode one chunk x [T][h][w][cin] (plan dtype).  The library sees only
        pointers, so every tensor's shape and dtype is checked here, before any
        call: a smaller or wrongly typed buffer would be read past its end.
        Returns y viewed as the chunk's output shape."""
        if x.dim() != 4 or tuple(x.shape[1:]) != self.in_shape or x.dtype != _TD[self.dtype]:
            raise ValueError("x must be [T][%d][%d][%d] of %s, got %s of %s"
                             % (self.in_shape + (_TD[self.dtype], tuple(x.shape), x.dtype)))
        _check_arena(cache_in, self.state_bytes, "cache_in")
        _check_arena(cache_out, self.state_bytes, "cache_out")
        t_chunk = x.shape[0]
        first = cache_in.frames_seen == 0
        shape = self.output_shape(t_chunk, first)
        if residual is not None or self.takes_residual:
            if not self.takes_residual:
                raise ValueError("this plan takes no residual")
            if residual is None:
                raise ValueError("this plan adds a residual; pass one")
            rshape = self.slot_shape(C.SLOT_AUX, t_chunk, first)
            if tuple(residual.shape) != rshape or residual.dtype != _TD[self.dtype]:
                raise ValueError("residual must be %s of %s, got %s of %s"
                                 % (rshape, _TD[self.dtype], tuple(residual.shape), residual.dtype))
        if y is None:
            y = torch.empty(shape, dtype=self.out_dtype, device=self.device)
        elif y.dtype != self.out_dtype or y.numel() < _numel(shape):
            raise ValueError("y must hold %s elements of %s for this chunk, got %s of %s"
                             % (_numel(shape), self.out_dtype, y.numel(), y.dtype))
        ci, co = cache_in._c(), cache_out._c()
        C.check(C.lib().cc3d_forward_chunk(self._h, _ptr(x), t_chunk, ctypes.byref(ci), ctypes.byref(co),
                                           _ptr(residual), _ptr(y), _stream(stream)), "cc3d_forward_chunk")
        cache_out.frames_seen = co.frames_seen
        return y if tuple(y.shape) == shape else y.reshape(-1)[:_numel(shape)].view(shape)


def conv_plan(w: torch.Tensor, h_in: int, w_in: int, *, bias=None, gamma=None, up_s=1, up_t=1,
              max_chunk_t=8, tpad=C.TPAD_REPLICATE, residual=False, act=False, out_u8=False, eps=1e-6,
              aligned=False, fold_upsample=False, stride_s=1, stride_t=1, stream=None) -> Plan:
    """Plan for one causal conv; w is [Cout][Cin][kt][kh][kw] on the GPU (bf16 or fp32).
    ``aligned``: the first chunk doubles every frame at up_t = 2 (CC3D_GROW_ALIGNED),
    and a temporal stride takes every output from two new frames (phase 1).
    ``fold_upsample``: phase-folded kernel for an upsampling 3x3 conv where it applies.
    ``stride_s``, ``stride_t``: a strided conv (1 or 2 each)."""
    cout, cin, kt, kh, kw = w.shape
    if w.dtype not in _DT:
        raise ValueError("weights must be bfloat16 or float32, got %s" % w.dtype)
    for name, v, n in (("bias", bias, cout), ("gamma", gamma, cout)):
        if v is not None and (v.dtype != torch.float32 or v.numel() != n):
            raise ValueError("%s must hold %d float32 values, got %d of %s" % (name, n, v.numel(), v.dtype))
    d = C.ConvDesc(cin=cin, cout=cout, kt=kt, kh=kh, kw=kw, h_in=h_in, w_in=w_in, up_s=up_s, up_t=up_t,
                   max_chunk_t=max_chunk_t, dtype=_DT[w.dtype], tpad=tpad,
                   epilogue=(C.EPI_RESIDUAL if residual else 0) | (C.EPI_ACT if act else 0) |
                   (C.EPI_U8 if out_u8 else 0), eps=eps, grow=C.GROW_ALIGNED if aligned else C.GROW_ONCE,
                   fold_upsample=int(fold_upsample), stride_s=stride_s, stride_t=stride_t)
    h = ctypes.c_void_p()
    with torch.cuda.device(w.device):
        C.check(C.lib().cc3d_plan_create(ctypes.byref(d), _ptr(w), _ptr(bias), _ptr(gamma), _stream(stream),
                                         ctypes.byref(h)), "cc3d_plan_create")
    return Plan(h, d.dtype, w.device, cin, h_in, w_in, ["conv"])


def conv_state_bytes(kt: int, h_in: int, w_in: int, cin: int, elem_bytes: int) -> int:
    """State bytes of one conv: its cache of kt - 1 input frames, in 256-byte
    units (what cc3d_state_bytes reports for a plan of that conv)."""
    return max(256, -(-(kt - 1) * h_in * w_in * cin * elem_bytes // 256) * 256)


def conv_forward_noalloc(w: torch.Tensor, x: torch.Tensor, cache_in: State, cache_out: State, y: torch.Tensor,
                         *, bias=None, gamma=None, residual=None, up_s=1, up_t=1, max_chunk_t=8,
                         tpad=C.TPAD_REPLICATE, act=False, out_u8=False, eps=1e-6, aligned=False,
                         fold_upsample=False, stride_s=1, stride_t=1, stream=None) -> torch.Tensor:
    """One conv chunk through cc3d_conv_forward_noalloc: the result of
    conv_plan(w, ...).forward_chunk(x, ...), with no device allocation (the
    library repacks the weights into its fixed per-device scratch).  The
    caller supplies y and the two state arenas (State objects sized by a plan
    of the same conv); x is [T][h][w][cin] of w's dtype, y the chunk's output
    shape.  Shapes and dtypes are checked here before the call."""
    cout, cin, kt, kh, kw = w.shape
    if w.dtype not in _DT:
        raise ValueError("weights must be bfloat16 or float32, got %s" % w.dtype)
    if x.dim() != 4 or x.shape[3] != cin or x.dtype != w.dtype:
        raise ValueError("x must be [T][h][w][%d] of %s, got %s of %s" % (cin, w.dtype, tuple(x.shape), x.dtype))
    for name, v, n in (("bias", bias, cout), ("gamma", gamma, cout)):
        if v is not None and (v.dtype != torch.float32 or v.numel() != n):
            raise ValueError("%s must hold %d float32 values, got %d of %s" % (name, n, v.numel(), v.dtype))
    d = C.ConvDesc(cin=cin, cout=cout, kt=kt, kh=kh, kw=kw, h_in=x.shape[1], w_in=x.shape[2], up_s=up_s,
                   up_t=up_t, max_chunk_t=max_chunk_t, dtype=_DT[w.dtype], tpad=tpad,
                   epilogue=(C.EPI_RESIDUAL if residual is not None else 0) | (C.EPI_ACT if act else 0) |
                   (C.EPI_U8 if out_u8 else 0), eps=eps, grow=C.GROW_ALIGNED if aligned else C.GROW_ONCE,
                   fold_upsample=int(fold_upsample), stride_s=stride_s, stride_t=stride_t)
    first = cache_in.frames_seen == 0
    t = x.shape[0]
    grow = up_t == 2 and first and not aligned
    t_out = (2 * t - 1 if grow else 2 * t) if up_t == 2 else t
    if stride_t == 2:  # (a length that leaves half a frame is refused by the library)
        t_out = (t + 1) // 2 if (first and not aligned) else t // 2
    hw = (x.shape[1] * up_s, x.shape[2] * up_s) if stride_s == 1 else ((x.shape[1] + 1) // 2, (x.shape[2] + 1) // 2)
    want = (t_out,) + hw + (cout,)
    out_dtype = torch.uint8 if out_u8 else w.dtype
    if tuple(y.shape) != want or y.dtype != out_dtype:
        raise ValueError("y must be %s of %s, got %s of %s" % (want, out_dtype, tuple(y.shape), y.dtype))
    if residual is not None and (tuple(residual.shape) != want or residual.dtype != w.dtype):
        raise ValueError("residual must be %s of %s, got %s of %s" % (want, w.dtype, tuple(residual.shape),
                                                                       residual.dtype))
    need = conv_state_bytes(kt, x.shape[1], x.shape[2], cin, w.element_size())
    _check_arena(cache_in, need, "cache_in")
    _check_arena(cache_out, need, "cache_out")
    ci, co = cache_in._c(), cache_out._c()
    with torch.cuda.device(x.device):
        C.check(C.lib().cc3d_conv_forward_noalloc(ctypes.byref(d), _ptr(w), _ptr(bias), _ptr(gamma), _ptr(x), t,
                                                  ctypes.byref(ci), ctypes.byref(co), _ptr(residual), _ptr(y),
                                                  _stream(stream)), "cc3d_conv_forward_noalloc")
    cache_out.frames_seen = co.frames_seen
    return y


def _check_weights(ops: List[Op], cin: int, dtype):
    """Each CONV op's weights must hold exactly [cout][channels of its src][k]
    of the plan dtype, and every bias and gain its channel count of float32 (the
    library reads that many elements through the pointer)."""
    ch = {C.SLOT_X: cin}

    def vec(i, o, name, v, n):
        if v is not None and n is not None and (v.dtype != torch.float32 or v.numel() != n):
            raise ValueError("op %d (%s): %s must hold %d float32 values, got %d of %s"
                             % (i, o.name, name, n, v.numel(), v.dtype))

    for i, o in enumerate(ops):
        c_src = ch.get(o.src)
        if o.kind == C.OP_CONV:
            if o.w is None:
                raise ValueError("op %d (%s): weights are missing" % (i, o.name))
            want = (o.cout, c_src) + tuple(o.k)
            if c_src is not None and tuple(o.w.shape) != want:
                raise ValueError("op %d (%s): weights %s, expected %s" % (i, o.name, tuple(o.w.shape), want))
            if o.w.dtype != dtype:
                raise ValueError("op %d (%s): weights are %s, the plan is %s" % (i, o.name, o.w.dtype, dtype))
            vec(i, o, "bias", o.bias, o.cout)
            c_out = o.cout
        else:
            c_out = c_src
        vec(i, o, "gamma", o.gamma, c_out)
        for sl in (o.out, o.act_out):
            if sl != C.SLOT_NONE and c_out is not None:
                ch[sl] = c_out


def stack_plan(ops: List[Op], cin: int, h: int, w: int, *, dtype=torch.bfloat16, max_chunk_t=8,
               eps=1e-6, aligned=False, batch_from=0, frame_batch=0, fold_upsample=False, device=None,
               stream=None) -> Plan:
    """Plan for an op list; ``aligned`` as in conv_plan, for every up_t = 2 op.
    ``frame_batch`` > 0: ops[batch_from:] run in batches of that many frames of
    their input (frame batching, see cc3d_stack_desc).  ``fold_upsample``: the
    phase-folded kernel for every upsampling 3x3 conv it applies to."""
    _check_weights(ops, cin, dtype)
    arr = (C.OpDesc * len(ops))()
    for i, o in enumerate(ops):
        kt, kh, kw = o.k
        arr[i] = C.OpDesc(kind=o.kind, cout=o.cout, kt=kt, kh=kh, kw=kw, up_s=o.up_s, up_t=o.up_t,
                          tpad=o.tpad, src=o.src, res=o.res, out=o.out, act_out=o.act_out,
                          w=_ptr(o.w), bias=_ptr(o.bias), gamma=_ptr(o.gamma), out_u8=int(o.out_u8),
                          stride_s=o.stride_s, stride_t=o.stride_t)
    d = C.StackDesc(dtype=_DT[dtype], cin=cin, h=h, w=w, max_chunk_t=max_chunk_t, eps=eps, n_ops=len(ops),
                    ops=arr, grow=C.GROW_ALIGNED if aligned else C.GROW_ONCE, batch_from=batch_from,
                    frame_batch=frame_batch, fold_upsample=int(fold_upsample))
    if device is None:
        device = next((o.w.device for o in ops if o.w is not None), torch.device("cuda", 0))
    hnd = ctypes.c_void_p()
    with torch.cuda.device(device):
        C.check(C.lib().cc3d_stack_plan_create(ctypes.byref(d), _stream(stream), ctypes.byref(hnd)),
                "cc3d_stack_plan_create")
    return Plan(hnd, d.dtype, device, cin, h, w, [o.name or "op%d" % i for i, o in enumerate(ops)])


class Stream:
    """A video being decoded: a plan plus two state arenas used alternately
    (the pages' ping-pong state buffers)."""

    def __init__(self, plan: Plan, stream=None):
        self.plan = plan
        self.states = [plan.new_state(), plan.new_state()]
        self.cur = 0
        self.stream = stream
        self.reset()

    def reset(self):
        for s in self.states:
            self.plan.reset(s, self.stream)
        self.cur = 0

    @property
    def frames_seen(self) -> int:
        return self.states[self.cur].frames_seen

    def step(self, x: torch.Tensor, residual=None, y=None) -> torch.Tensor:
        a, b = self.states[self.cur], self.states[1 - self.cur]
        out = self.plan.forward_chunk(x, a, b, residual=residual, y=y, stream=self.stream)
        self.cur = 1 - self.cur
        return out


def to_channels_last(x_cthw: torch.Tensor, stream=None) -> torch.Tensor:
    c, t, h, w = x_cthw.shape
    out = torch.empty((t, h, w, c), dtype=x_cthw.dtype, device=x_cthw.device)
    C.check(C.lib().cc3d_to_channels_last(_ptr(x_cthw), _ptr(out), c, t, h, w, x_cthw.element_size(),
                                          _stream(stream)), "cc3d_to_channels_last")
    return out


def to_channels_first(x_thwc: torch.Tensor, stream=None) -> torch.Tensor:
    t, h, w, c = x_thwc.shape
    out = torch.empty((c, t, h, w), dtype=x_thwc.dtype, device=x_thwc.device)
    C.check(C.lib().cc3d_to_channels_first(_ptr(x_thwc), _ptr(out), c, t, h, w, x_thwc.element_size(),
                                           _stream(stream)), "cc3d_to_channels_first")
    return out
