"""Brute-force causal conv for tiny inputs: numpy, one output at a time over an
explicitly built padded array.  TEST INFRASTRUCTURE ONLY: used to pin the C
oracle, never by the GPU library.

It builds the padded tensor the slow, literal way -- the history frames (zeros,
or copies of frame 0) stacked before the video along time, then a zero border
of (k-1)/2 pixels around each frame -- and takes every output as the full
elementwise product of the weight block with the input window, summed.
"""
from __future__ import annotations

import numpy as np


def causal_conv3d_brute(x, w, bias=None, mode="replicate"):
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    cin, t, h, wd = x.shape
    cout, _, kt, kh, kw = w.shape
    hist = []
    for _ in range(kt - 1):
        hist.append(np.zeros_like(x[:, 0]) if mode == "zero" else x[:, 0].copy())
    frames = hist + [x[:, i] for i in range(t)]
    padded = np.zeros((cin, len(frames), h + kh - 1, wd + kw - 1))
    for i, f in enumerate(frames):
        padded[:, i, (kh - 1) // 2:(kh - 1) // 2 + h, (kw - 1) // 2:(kw - 1) // 2 + wd] = f
    y = np.zeros((cout, t, h, wd))
    for o in range(cout):
        for tt in range(t):
            for i in range(h):
                for j in range(wd):
                    win = padded[:, tt:tt + kt, i:i + kh, j:j + kw]
                    y[o, tt, i, j] = np.sum(w[o] * win) + (0.0 if bias is None else bias[o])
    return y


def strided_causal_conv3d_brute(x, w, bias=None, mode="replicate", stride_s=1, stride_t=1, phase=0):
    """The same literal construction with strides: output (j, i, jj) is the
    weight block times the padded window that starts at padded frame
    phase + stride_t*j and at padded pixel (stride_s*i, stride_s*jj), i.e. the
    window centred on input pixel (stride_s*i, stride_s*jj) whose current frame
    is input frame phase + stride_t*j."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    cin, t, h, wd = x.shape
    cout, _, kt, kh, kw = w.shape
    hist = []
    for _ in range(kt - 1):
        hist.append(np.zeros_like(x[:, 0]) if mode == "zero" else x[:, 0].copy())
    frames = hist + [x[:, i] for i in range(t)]
    padded = np.zeros((cin, len(frames), h + kh - 1, wd + kw - 1))
    for i, f in enumerate(frames):
        padded[:, i, (kh - 1) // 2:(kh - 1) // 2 + h, (kw - 1) // 2:(kw - 1) // 2 + wd] = f
    outs_t = [j for j in range(t) if phase + stride_t * j <= t - 1]
    outs_h = [i for i in range(h) if stride_s * i <= h - 1]
    outs_w = [i for i in range(wd) if stride_s * i <= wd - 1]
    y = np.zeros((cout, len(outs_t), len(outs_h), len(outs_w)))
    for o in range(cout):
        for tt in outs_t:
            for i in outs_h:
                for j in outs_w:
                    t0, y0, x0 = phase + stride_t * tt, stride_s * i, stride_s * j
                    win = padded[:, t0:t0 + kt, y0:y0 + kh, x0:x0 + kw]
                    y[o, tt, i, j] = np.sum(w[o] * win) + (0.0 if bias is None else bias[o])
    return y
