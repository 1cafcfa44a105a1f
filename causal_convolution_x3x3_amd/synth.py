"""Seeded synthetic inputs for the decode workloads.

This module holds input generation only -- random draws and their rounding to
the storage type -- and none of the method's arithmetic.  The tests feed the
same draws to the GPU library and to the fp64 oracle; the benchmark uses it to
make device-resident inputs.

Seeds: ``seed(cfg, tensor_id)`` = 1000*cfg + tensor_id; chunk k of a streamed
input uses tensor_id + 100 + k.  Draws are float32 from a CPU
``torch.Generator``; bf16 tensors are the float32 draw rounded to nearest even
(``Tensor.to(torch.bfloat16)``).

Workloads (sizes from the pages' resolutions and frame counts; the pages' test
videos and trained weights are not available, so these stand in for them):

* c0 -- one fp32 3x3x3 causal conv, 16->16 channels, 9 frames of 32x32, chunks 1+4+4
* c1 -- bf16 residual block, 128 channels, 16 frames of 90x160, 4-frame chunks
* c2 -- bf16 1080p-class stage, 256 channels, 24 frames of 270x480 -> 540x960
* c3 -- bf16 1440p output stage, 128 channels, 361 frames of 720x1280 -> 2560x1440 RGB
* c4 -- bf16 decoder stack, latent 48 x 91 frames of 90x160 -> 3 x 361 x 1440x2560
"""
from __future__ import annotations

import math

import torch

WORKLOADS = {
    0: dict(name="c0_conv_fp32", cin=16, cout=16, t=9, h=32, w=32, splits=(1, 4, 4)),
    1: dict(name="c1_resblock_bf16", c=128, t=16, h=90, w=160, chunk=4),
    2: dict(name="c2_stage1080_bf16", cin=256, cmid=128, cout=128, t=24, h=270, w=480, chunk=4),
    3: dict(name="c3_stage1440_bf16", cin=128, cmid=96, cout=3, t=361, h=720, w=1280,
            first_chunk=1, chunk=4),
    4: dict(name="c4_decoder_bf16", c_latent=48, t=91, h=90, w=160, first_clip=7, clip=6),
}


def seed(cfg: int, tensor_id: int) -> int:
    return 1000 * cfg + tensor_id


def _gen(s: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(s))
    return g


def normal(shape, s: int, std: float = 1.0) -> torch.Tensor:
    """float32 N(0, std^2) draw."""
    t = torch.randn(tuple(shape), generator=_gen(s), dtype=torch.float32)
    return t * std if std != 1.0 else t


def uniform(shape, lo: float, hi: float, s: int) -> torch.Tensor:
    """float32 U(lo, hi) draw."""
    return torch.rand(tuple(shape), generator=_gen(s), dtype=torch.float32) * (hi - lo) + lo


def conv_weight(cout, cin, kt, kh, kw, s: int) -> torch.Tensor:
    """[Cout][Cin][kt][kh][kw] float32 ~ N(0, std = 1/sqrt(Cin*kt*kh*kw))."""
    fan_in = cin * kt * kh * kw
    return normal((cout, cin, kt, kh, kw), s, std=1.0 / math.sqrt(fan_in))


def gain(c, s: int) -> torch.Tensor:
    """RMSNorm gain ~ U(0.5, 1.5), float32."""
    return uniform((c,), 0.5, 1.5, s)


def bias(c, s: int, scale: float = 0.1) -> torch.Tensor:
    """Bias ~ U(-scale, scale), float32 (the parity case that pins the bias path)."""
    return uniform((c,), -scale, scale, s)


def bf16(t: torch.Tensor) -> torch.Tensor:
    """Round a float32 draw to bfloat16 (nearest, ties to even)."""
    return t.to(torch.bfloat16)


def layer_weights(shapes, cfg: int, gain_for, with_bias: bool = False):
    """Seeded weights for a list of layers (name, cout, cin, kt, kh, kw): per
    layer i the bf16 weight draws seed(cfg, 10 + 3i), the float32 RMSNorm gain
    of its input (where ``gain_for(name)``) seed(cfg, 11 + 3i) and the float32
    bias (with ``with_bias``) seed(cfg, 12 + 3i).  CPU tensors; absent ones None."""
    out = {}
    for i, (name, co, ci, kt, kh, kw) in enumerate(shapes):
        out[name] = {
            "w": bf16(conv_weight(co, ci, kt, kh, kw, seed(cfg, 10 + 3 * i))),
            "g": gain(ci, seed(cfg, 11 + 3 * i)) if gain_for(name) else None,
            "b": bias(co, seed(cfg, 12 + 3 * i)) if with_bias else None,
        }
    return out


def video(c, t, h, w, s: int) -> torch.Tensor:
    """A [C][T][H][W] float32 N(0,1) video."""
    return normal((c, t, h, w), s)


def chunk_lengths(total: int, chunk: int, first: int | None = None):
    """Chunk lengths covering ``total`` frames: an optional first chunk, then
    ``chunk``-frame chunks, the last one holding what remains."""
    out, left = [], total
    if first is not None and left > 0:
        out.append(min(first, left))
        left -= out[-1]
    while left > 0:
        out.append(min(chunk, left))
        left -= out[-1]
    return out
