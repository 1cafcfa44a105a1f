"""fp64 oracle for the synthetic decoder blocks, run chunk by chunk.

TEST INFRASTRUCTURE ONLY (see oracle.py): imported by tests, the smoke check and
the CPU-baseline leg of the benchmark, never by the GPU library.

The pages name the decoder's pieces (a causal per-layer state, nearest 2x
spatial upsampling before a spatial conv, growth of the frame count) but print
no layer list, channel count or weight.  The blocks below are the synthetic
workloads built from those pieces:

* ``ResBlock``  y = x + conv2(act(conv1(act(x)))), act = SiLU(RMSNorm(.)), each
  conv with its own cache.
* ``UpStage``   conv2(act(conv1(up2x(x)))) -- the 1080p-class and 1440p output
  stages (conv1 reads the nearest-upsampled input).
* ``Decoder``   conv_in, three stages of [nearest up (2x space; 2x time on
  non-first frames for the first two) -> conv -> two ResBlocks], then a head:
  act at low resolution -> nearest 2x -> conv to 3 channels.  Moving the act
  before the upsample is exact because it works per position (the SwiftVR page,
  "TemporalGrow: Compute Before Spatial Upsampling").
* ``TemporalGrow`` (same section): a 1x1 spatial projection followed by a
  causal temporal conv with a 3x1x1 kernel, both per position; it grows the
  frame count (the nearest 2x rule above, applied to the projection's output
  before the temporal conv).  With ``temporal_grow`` the decoder has one per
  stage, growth (2, 2, 1), taking over the stage's temporal growth: "before"
  runs it at the stage's input size, ahead of the upsample conv; "after" runs it
  on the upsampled positions, between the upsample and the spatial conv.

* ``Encoder``   the decoder read backwards (the pages print no encoder layer;
  "ReAE: Causal Halo Exchange" puts the ReAE encoder under the decoder's
  causal-state rule, and "From Pixels to Latents and Back" has it map the
  target-size video to the latents the decoder reads): a stride-2 conv from
  the pixels, three stages of [two ResBlocks -> conv with spatial stride 2 and
  the decoder stage's temporal factor as temporal stride], then act -> conv to
  the latent channels.  Each strided conv mirrors one upsampling conv of the
  decoder; 1 + 4n frames give 1 + n latents (the first frame on its own), or
  4n give n with ``aligned``.

``store`` is the storage rounding: with ``store=round_bf16`` every tensor that
passes between layers is rounded to bfloat16, as a bf16 pipeline stores it
(the conv output after bias and residual; the activation, computed from the
stored conv output).  With ``store=None`` everything stays fp64.

Weights are dicts of numpy arrays: ``w`` [Cout][Cin][kt][kh][kw], ``b`` [Cout]
or None, ``g`` [C] (the RMSNorm gain applied to this conv's input, where it
has one).
"""
from __future__ import annotations

import numpy as np

from . import oracle as O


def _keep(x, store):
    return x if store is None else store(x)


class Conv:
    """One causal conv layer with its cache (see oracle.CausalConvStream)."""

    def __init__(self, p, mode=O.REPLICATE, up_s=1, up_t=1, nthreads=None, aligned=False,
                 stride_s=1, stride_t=1):
        self.s = O.CausalConvStream(p["w"], p.get("b"), mode, up_s, up_t, nthreads, aligned,
                                    stride_s, stride_t)

    def reset(self):
        self.s.reset()

    def step(self, x):
        return self.s.step(x)


class ResBlock:
    def __init__(self, p1, p2, eps=1e-6, mode=O.REPLICATE, store=None, nthreads=None):
        self.c1 = Conv(p1, mode, nthreads=nthreads)
        self.c2 = Conv(p2, mode, nthreads=nthreads)
        self.g1, self.g2 = p1["g"], p2["g"]
        self.eps, self.store = eps, store

    def reset(self):
        self.c1.reset()
        self.c2.reset()

    def step(self, x):
        st = self.store
        a1 = _keep(O.act(x, self.g1, self.eps), st)
        h = _keep(self.c1.step(a1), st)
        a2 = _keep(O.act(h, self.g2, self.eps), st)
        return _keep(x + self.c2.step(a2), st)


class UpStage:
    """conv2(act(conv1(nearest_up(x)))): up_s on conv1's input."""

    def __init__(self, p1, p2, eps=1e-6, mode=O.REPLICATE, up_s=2, store=None, nthreads=None):
        self.c1 = Conv(p1, mode, up_s=up_s, nthreads=nthreads)
        self.c2 = Conv(p2, mode, nthreads=nthreads)
        self.g2 = p2["g"]
        self.eps, self.store = eps, store

    def reset(self):
        self.c1.reset()
        self.c2.reset()

    def step(self, x):
        st = self.store
        h = _keep(self.c1.step(x), st)
        a = _keep(O.act(h, self.g2, self.eps), st)
        return _keep(self.c2.step(a), st)


class TemporalGrow:
    """q = tconv(grow(proj(x))): proj a 1x1x1 conv, grow the nearest temporal
    rule (factor 1 or 2), tconv a causal 3x1x1 conv with its own cache.  With
    up_s = 2 the projection reads the nearest-upsampled input (the "after"
    order: the block then runs on every upsampled position)."""

    def __init__(self, p_proj, p_t, factor, mode=O.REPLICATE, up_s=1, store=None, nthreads=None,
                 aligned=False):
        self.proj = Conv(p_proj, mode, up_s=up_s, nthreads=nthreads)
        self.tconv = Conv(p_t, mode, up_t=factor, nthreads=nthreads, aligned=aligned)
        self.store = store

    def reset(self):
        self.proj.reset()
        self.tconv.reset()

    def step(self, x):
        p = _keep(self.proj.step(x), self.store)
        return _keep(self.tconv.step(p), self.store)


DECODER_STAGES = ((384, 2), (192, 2), (96, 1))  # (channels, temporal factor)
TG_ORDERS = (None, "before", "after")


def decoder_layer_shapes(c_latent=48, stages=DECODER_STAGES, c_out=3, k=3, temporal_grow=None):
    """(name, Cout, Cin, kt, kh, kw, has_gain) for every conv of the decoder,
    in execution order.  ``has_gain``: the conv's input passes an RMSNorm.
    With ``temporal_grow`` each stage starts with a TemporalGrow on its input
    channels: "s<i>.tg.p" (1x1x1) and "s<i>.tg.t" (3x1x1)."""
    if temporal_grow not in TG_ORDERS:
        raise ValueError("temporal_grow must be one of %r" % (TG_ORDERS,))
    shapes = [("conv_in", stages[0][0], c_latent, k, k, k, False)]
    cin = stages[0][0]
    for si, (c, _) in enumerate(stages):
        if temporal_grow:
            shapes.append(("s%d.tg.p" % si, cin, cin, 1, 1, 1, False))
            shapes.append(("s%d.tg.t" % si, cin, cin, 3, 1, 1, False))
        shapes.append(("s%d.up" % si, c, cin, k, k, k, False))
        for r in range(2):
            shapes.append(("s%d.rb%d.c1" % (si, r), c, c, k, k, k, True))
            shapes.append(("s%d.rb%d.c2" % (si, r), c, c, k, k, k, True))
        cin = c
    shapes.append(("head", c_out, cin, k, k, k, True))
    return shapes


class Decoder:
    """``temporal_grow``: None (the stage's up conv grows time), "before" or
    "after" (a TemporalGrow per stage does, see the module docstring).
    ``aligned``: the first chunk is grown like every later one (every frame
    doubled), the reading of the 28-frame first chunk that drops 3 frames."""

    def __init__(self, params, eps=1e-6, mode=O.REPLICATE, stages=DECODER_STAGES,
                 store=None, nthreads=None, temporal_grow=None, aligned=False):
        if temporal_grow not in TG_ORDERS:
            raise ValueError("temporal_grow must be one of %r" % (TG_ORDERS,))
        self.eps, self.store = eps, store
        self.conv_in = Conv(params["conv_in"], mode, nthreads=nthreads)
        self.ups, self.blocks, self.tgs = [], [], []
        for si, (_, up_t) in enumerate(stages):
            if temporal_grow:
                after = temporal_grow == "after"
                self.tgs.append(TemporalGrow(params["s%d.tg.p" % si], params["s%d.tg.t" % si], up_t, mode,
                                             up_s=2 if after else 1, store=store, nthreads=nthreads,
                                             aligned=aligned))
                self.ups.append(Conv(params["s%d.up" % si], mode, up_s=1 if after else 2, nthreads=nthreads))
            else:
                self.tgs.append(None)
                self.ups.append(Conv(params["s%d.up" % si], mode, up_s=2, up_t=up_t,
                                     nthreads=nthreads, aligned=aligned))
            self.blocks.append([
                ResBlock(params["s%d.rb%d.c1" % (si, r)], params["s%d.rb%d.c2" % (si, r)],
                         eps, mode, store, nthreads) for r in range(2)])
        self.head = Conv(params["head"], mode, up_s=2, nthreads=nthreads)
        self.g_head = params["head"]["g"]

    def reset(self):
        self.conv_in.reset()
        self.head.reset()
        for u in self.ups:
            u.reset()
        for g in self.tgs:
            if g is not None:
                g.reset()
        for bl in self.blocks:
            for b in bl:
                b.reset()

    def step(self, x):
        st = self.store
        h = _keep(self.conv_in.step(x), st)
        for tg, up, bl in zip(self.tgs, self.ups, self.blocks):
            if tg is not None:
                h = tg.step(h)
            h = _keep(up.step(h), st)
            for b in bl:
                h = b.step(h)
        a = _keep(O.act(h, self.g_head, self.eps), st)
        return _keep(self.head.step(a), st)


def encoder_layer_shapes(c_in=3, stages=DECODER_STAGES, c_latent=48, k=3):
    """(name, Cout, Cin, kt, kh, kw, has_gain, stride_s, stride_t) for every conv
    of the encoder, in execution order: the decoder's stages taken from the
    last, each strided conv going back to the channels the matching decoder
    stage started from."""
    widths = [stages[0][0]] + [c for c, _ in stages]  # the decoder's conv_in width, then each stage's
    shapes = [("conv_in", stages[-1][0], c_in, k, k, k, False, 2, 1)]
    for ei in range(len(stages)):
        si = len(stages) - 1 - ei  # the decoder stage this one mirrors
        c, f = stages[si]
        for r in range(2):
            shapes.append(("e%d.rb%d.c1" % (ei, r), c, c, k, k, k, True, 1, 1))
            shapes.append(("e%d.rb%d.c2" % (ei, r), c, c, k, k, k, True, 1, 1))
        shapes.append(("e%d.down" % ei, widths[si], c, k, k, k, False, 2, f))
    shapes.append(("conv_out", c_latent, widths[0], k, k, k, True, 1, 1))
    return shapes


class Encoder:
    """The encoder read of the module docstring; ``params`` keyed by the names
    of encoder_layer_shapes.  ``aligned``: every latent takes four new frames
    (the 28-frame first chunk); otherwise the first frame makes the first
    latent on its own."""

    def __init__(self, params, eps=1e-6, mode=O.ZERO, stages=DECODER_STAGES, store=None,
                 nthreads=None, aligned=False):
        self.eps, self.store = eps, store
        self.conv_in = Conv(params["conv_in"], mode, nthreads=nthreads, stride_s=2)
        self.blocks, self.downs = [], []
        for ei in range(len(stages)):
            f = stages[len(stages) - 1 - ei][1]
            self.blocks.append([
                ResBlock(params["e%d.rb%d.c1" % (ei, r)], params["e%d.rb%d.c2" % (ei, r)],
                         eps, mode, store, nthreads) for r in range(2)])
            self.downs.append(Conv(params["e%d.down" % ei], mode, nthreads=nthreads, aligned=aligned,
                                   stride_s=2, stride_t=f))
        self.conv_out = Conv(params["conv_out"], mode, nthreads=nthreads)
        self.g_out = params["conv_out"]["g"]

    def reset(self):
        self.conv_in.reset()
        self.conv_out.reset()
        for d in self.downs:
            d.reset()
        for bl in self.blocks:
            for b in bl:
                b.reset()

    def step(self, x):
        st = self.store
        h = _keep(self.conv_in.step(x), st)
        for bl, down in zip(self.blocks, self.downs):
            for b in bl:
                h = b.step(h)
            h = _keep(down.step(h), st)
        a = _keep(O.act(h, self.g_out, self.eps), st)
        return _keep(self.conv_out.step(a), st)


def output_frames(n_latent: int, temporal_factors=(2, 2), aligned: bool = False) -> int:
    """Frames after temporal growth on non-first frames: n -> 1 + f (n - 1);
    with ``aligned`` (every frame grown): n -> f n."""
    n = n_latent
    for f in temporal_factors:
        if aligned:
            n = f * n
        else:
            n = 1 + f * (n - 1) if n > 0 else 0
    return n


def clip_schedule(n_latent: int, first: int = 7, rest: int = 6):
    """Latent chunk lengths: the first clip of ``first`` latents (25 frames after
    two 2x temporal growths), then clips of ``rest`` (24 frames), the last one
    holding what remains."""
    out, left = [], n_latent
    if left > 0:
        out.append(min(first, left))
        left -= out[-1]
    while left > 0:
        out.append(min(rest, left))
        left -= out[-1]
    return out
