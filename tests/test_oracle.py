"""Pins for the fp64 oracle (CPU only).

Each pin is chosen so a plausible slip in the oracle -- a dropped bias, a
reversed temporal or spatial tap, swapped Cin/Cout, a wrong history rule, a
cache that keeps the wrong frames, an upsample that rounds instead of floors, a
norm over the wrong axis -- fails at least one test.
"""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import brute, model as M
from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ brute force --

KSHAPES = [(kt, kh, kw) for kt in (1, 2, 3) for kh in (1, 3) for kw in (1, 3)]


@pytest.mark.parametrize("k", KSHAPES)
@pytest.mark.parametrize("mode", [O.REPLICATE, O.ZERO])
def test_conv_matches_brute_force(k, mode):
    r = _rng(hash((k, mode)) % 2**32)
    cin, cout, t, h, w = 3, 2, 5, 4, 5
    x = r.standard_normal((cin, t, h, w))
    wt = r.standard_normal((cout, cin) + k)
    b = r.standard_normal(cout)
    ref = brute.causal_conv3d_brute(x, wt, b, mode)
    got = O.causal_conv3d(x, wt, b, mode)
    assert got.shape == ref.shape
    assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("mode", [O.REPLICATE, O.ZERO])
def test_conv_matches_torch_conv3d(mode):
    """Library routine: torch CPU float64 conv3d (cross-correlation) on the
    explicitly padded input (history frames + spatial zero border)."""
    r = _rng(7)
    cin, cout, t, h, w = 5, 7, 6, 9, 11
    x = r.standard_normal((cin, t, h, w))
    wt = r.standard_normal((cout, cin, 3, 3, 3))
    b = r.standard_normal(cout)
    xt = torch.from_numpy(x)
    hist = torch.zeros_like(xt[:, :1]) if mode == O.ZERO else xt[:, :1]
    xp = torch.cat([hist, hist, xt], dim=1)
    xp = F.pad(xp, (1, 1, 1, 1))
    ref = F.conv3d(xp[None], torch.from_numpy(wt), torch.from_numpy(b))[0].numpy()
    got = O.causal_conv3d(x, wt, b, mode)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


# ---------------------------------------------------------- delta kernels --

def _delta(c, kt, kh, kw, a, bb, d):
    w = np.zeros((c, c, kt, kh, kw))
    for i in range(c):
        w[i, i, a, bb, d] = 1.0
    return w


def test_delta_identity():
    x = _rng(1).standard_normal((3, 5, 6, 7))
    y = O.causal_conv3d(x, _delta(3, 3, 3, 3, 2, 1, 1), None, O.REPLICATE)
    assert np.array_equal(y, x)


@pytest.mark.parametrize("mode", [O.REPLICATE, O.ZERO])
def test_delta_oldest_tap_shifts_time(mode):
    """k_t=3, delta at a=0: Y_t = X_{t-2} for t>=2; X_0 or 0 before."""
    x = _rng(2).standard_normal((2, 6, 4, 5))
    y = O.causal_conv3d(x, _delta(2, 3, 3, 3, 0, 1, 1), None, mode)
    assert np.array_equal(y[:, 2:], x[:, :-2])
    for t in range(2):
        expect = x[:, 0] if mode == O.REPLICATE else np.zeros_like(x[:, 0])
        assert np.array_equal(y[:, t], expect)


def test_memoryblock_previous_tap_zero_history():
    """k_t=2 previous-frame tap with zero history: Y_0 = 0, Y_t = X_{t-1}."""
    x = _rng(3).standard_normal((2, 4, 3, 3))
    y = O.causal_conv3d(x, _delta(2, 2, 3, 3, 0, 1, 1), None, O.ZERO)
    assert np.array_equal(y[:, 0], np.zeros_like(x[:, 0]))
    assert np.array_equal(y[:, 1:], x[:, :-1])


def test_delta_spatial_shift_zero_border():
    """delta at (b,d)=(0,2): Y[h,w] = X[h-1, w+1], zero outside the image."""
    x = _rng(4).standard_normal((1, 2, 5, 6))
    y = O.causal_conv3d(x, _delta(1, 1, 3, 3, 0, 0, 2), None, O.REPLICATE)
    expect = np.zeros_like(x)
    expect[:, :, 1:, :-1] = x[:, :, :-1, 1:]
    assert np.array_equal(y, expect)


def test_weight_axes_not_transposed():
    """Cin != Cout and a weight that only links input channel 1 to output 0."""
    x = _rng(5).standard_normal((3, 2, 3, 3))
    w = np.zeros((2, 3, 1, 1, 1))
    w[0, 1, 0, 0, 0] = 2.5
    y = O.causal_conv3d(x, w, np.array([0.0, -1.0]), O.REPLICATE)
    assert np.array_equal(y[0], 2.5 * x[1])
    assert np.array_equal(y[1], -np.ones_like(x[0]))


# ------------------------------------------------------------ closed form --

@pytest.mark.parametrize("mode", [O.REPLICATE, O.ZERO])
def test_constant_input_border_counts(mode):
    c, cin, t, h, w = 1.5, 4, 5, 5, 6
    x = np.full((cin, t, h, w), c)
    wt = np.ones((2, cin, 3, 3, 3))
    y = O.causal_conv3d(x, wt, None, mode)
    nh = np.array([2] + [3] * (h - 2) + [2])
    nw = np.array([2] + [3] * (w - 2) + [2])
    for tt in range(t):
        kt_eff = 3 if mode == O.REPLICATE else min(tt + 1, 3)
        expect = c * cin * kt_eff * nh[:, None] * nw[None, :]
        assert np.array_equal(y[0, tt], expect)
        assert np.array_equal(y[1, tt], expect)


def test_rmsnorm_silu_closed_forms():
    g = np.array([0.5, 1.0, 1.5])
    x = np.full((3, 2, 2, 2), 2.0)
    eps = 1e-6
    np.testing.assert_allclose(O.rms_norm(x, g, eps)[:, 0, 0, 0], g * 2.0 / np.sqrt(4.0 + eps),
                               rtol=1e-15)
    # mean over channels, not sum: a 1-hot vector of value v has rms = v / sqrt(C)
    x1 = np.zeros((4, 1, 1, 1))
    x1[2] = 3.0
    np.testing.assert_allclose(O.rms_norm(x1, np.ones(4), 0.0)[2, 0, 0, 0], 2.0, rtol=1e-15)
    z = np.linspace(-8, 8, 33)
    assert O.silu(np.zeros(1))[0] == 0.0
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, atol=1e-14)
    np.testing.assert_allclose(O.silu(np.array([50.0]))[0], 50.0, rtol=1e-15)


def test_round_bf16_matches_torch():
    r = _rng(9)
    x = np.concatenate([r.standard_normal(4096) * 10 ** r.uniform(-6, 6, 4096),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875]])  # ties both ways
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(x), ref)


# -------------------------------------------------------------- chunking --

SPLITS = [[9], [1, 4, 4], [1] * 9, [2, 3, 1, 3], [4, 5]]


@pytest.mark.parametrize("splits", SPLITS)
@pytest.mark.parametrize("mode", [O.REPLICATE, O.ZERO])
@pytest.mark.parametrize("up", [(1, 1), (2, 1), (2, 2)])
def test_chunked_equals_one_shot(splits, mode, up):
    r = _rng(11)
    x = r.standard_normal((3, 9, 4, 5))
    w = r.standard_normal((2, 3, 3, 3, 3))
    b = r.standard_normal(2)
    ref = O.one_shot(x, w, b, mode, up_s=up[0], up_t=up[1])
    got = O.chunked(x, w, b, mode, up_s=up[0], up_t=up[1], splits=splits)
    assert got.shape == ref.shape
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_cache_holds_last_frames_of_window():
    """A first chunk of one frame: the new cache is (history frame, x0); after
    it the next chunk sees x0 twice only in replicate mode."""
    x = _rng(12).standard_normal((2, 3, 2, 2))
    s = O.CausalConvStream(np.zeros((1, 2, 3, 3, 3)), mode=O.ZERO)
    s.step(x[:, :1])
    assert np.array_equal(s.cache[:, 0], np.zeros_like(x[:, 0]))
    assert np.array_equal(s.cache[:, 1], x[:, 0])
    s.step(x[:, 1:3])
    assert np.array_equal(s.cache, x[:, 1:3])


def test_memoryblock_golden_pairs():
    g = _read_golden("memoryblock_pairs.txt")
    assert g["current"].split() == ["A", "B", "C"]
    assert g["previous"].split() == ["P", "A", "B"]
    assert g["first_chunk_history"] == "zero"
    vals = {"P": 1.0, "A": 2.0, "B": 3.0, "C": 4.0}
    # k_t = 2, 1x1 spatial: out = 10*current + 1*previous, so each output
    # spells its (current, previous) pair in base 10.
    w = np.zeros((1, 1, 2, 1, 1))
    w[0, 0, 0] = 1.0   # previous frame
    w[0, 0, 1] = 10.0  # current frame
    s = O.CausalConvStream(w, mode=O.ZERO)
    y0 = s.step(np.full((1, 1, 1, 1), vals["P"]))
    assert y0[0, 0, 0, 0] == 10 * vals["P"] + 0.0  # zero history
    chunk = np.array([vals[k] for k in g["current"].split()]).reshape(1, 3, 1, 1)
    y = s.step(chunk)[0, :, 0, 0]
    for i, (cur, prev) in enumerate(zip(g["current"].split(), g["previous"].split())):
        assert y[i] == 10 * vals[cur] + vals[prev]


# ------------------------------------------------------------- causality --

@pytest.mark.parametrize("up_t", [1, 2])
def test_causality(up_t):
    r = _rng(13)
    x = r.standard_normal((2, 6, 4, 4))
    w = r.standard_normal((2, 2, 3, 3, 3))
    base = O.one_shot(x, w, None, O.REPLICATE, up_s=2, up_t=up_t)
    for tp in range(1, 6):
        x2 = x.copy()
        x2[:, tp] += 1.0
        y2 = O.one_shot(x2, w, None, O.REPLICATE, up_s=2, up_t=up_t)
        first_changed = tp if up_t == 1 else 2 * tp - 1
        assert np.array_equal(base[:, :first_changed], y2[:, :first_changed])
        assert not np.array_equal(base[:, first_changed], y2[:, first_changed])


# ---------------------------------------------------------------- upsample --

def test_upsample_is_repeat_interleave():
    x = _rng(14).standard_normal((2, 3, 4, 5))
    ref = torch.from_numpy(x).repeat_interleave(2, dim=2).repeat_interleave(2, dim=3).numpy()
    assert np.array_equal(O.upsample_spatial(x, 2), ref)
    v = O.upsample_temporal(x, first=True)
    assert v.shape[1] == 1 + 2 * (x.shape[1] - 1)
    assert np.array_equal(v[:, 0], x[:, 0])
    for j in range(1, x.shape[1]):
        assert np.array_equal(v[:, 2 * j - 1], x[:, j]) and np.array_equal(v[:, 2 * j], x[:, j])


def test_act_commutes_with_nearest_upsample_bitwise():
    """Per-position ops before or after nearest 2x give identical bits (the
    reorder the SwiftVR page reports as bitwise identical RGB)."""
    r = _rng(15)
    x = r.standard_normal((8, 2, 5, 6))
    g = r.uniform(0.5, 1.5, 8)
    a = O.upsample_spatial(O.act(x, g, 1e-6), 2)
    b = O.act(O.upsample_spatial(x, 2), g, 1e-6)
    assert np.array_equal(a, b)


def test_conv_points_matches_full():
    r = _rng(16)
    x = r.standard_normal((3, 4, 5, 6)).astype(np.float32)
    w = r.standard_normal((2, 3, 3, 3, 3))
    b = r.standard_normal(2)
    xp = O.temporal_pad(x.astype(np.float64), 3, O.REPLICATE)
    full = O.conv_valid(O.upsample_spatial(xp, 2), w, b)
    z = xp.astype(np.float32).transpose(1, 2, 3, 0).copy().transpose(3, 0, 1, 2)  # strided view
    pts = np.array([[t, y, xx] for t in range(4) for y in (0, 3, 9) for xx in (0, 5, 11)])
    got = O.conv_points(z, w, b, pts, up=2)
    ref = np.stack([full[:, t, y, xx] for t, y, xx in pts])
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


# ---------------------------------------------------------- strided conv --
# The encoder side's strided causal conv: every s-th pixel, every s_t-th frame
# from the phase (0: the first frame on its own; s_t - 1 with ``aligned``).

STRIDES = [(1, 2), (2, 1), (2, 2)]  # (spatial, temporal)


@pytest.mark.parametrize("k", [(1, 1, 1), (2, 3, 3), (3, 1, 1), (3, 3, 3)])
@pytest.mark.parametrize("stride", STRIDES)
@pytest.mark.parametrize("mode", [O.REPLICATE, O.ZERO])
@pytest.mark.parametrize("aligned", [False, True])
def test_strided_conv_matches_brute_force(k, stride, mode, aligned):
    r = _rng(hash((k, stride, mode, aligned)) % 2**32)
    cin, cout, t, h, w = 2, 3, 7, 5, 6  # odd and even frame sizes
    x = r.standard_normal((cin, t, h, w))
    wt = r.standard_normal((cout, cin) + k)
    b = r.standard_normal(cout)
    ss, st = stride
    ref = brute.strided_causal_conv3d_brute(x, wt, b, mode, ss, st, st - 1 if aligned else 0)
    got = O.causal_conv3d(x, wt, b, mode, stride_s=ss, stride_t=st, aligned=aligned)
    assert got.shape == ref.shape
    assert got.shape[2:] == ((h + ss - 1) // ss, (w + ss - 1) // ss)
    assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("stride", STRIDES)
@pytest.mark.parametrize("aligned", [False, True])
def test_strided_conv_matches_torch_conv3d(stride, aligned):
    """Library routine: torch CPU float64 conv3d with stride (s_t, s, s) and
    spatial padding 1 on the history-padded input, started at the phase."""
    r = _rng(31)
    cin, cout, t, h, w = 4, 5, 9, 10, 7
    x = r.standard_normal((cin, t, h, w))
    wt = r.standard_normal((cout, cin, 3, 3, 3))
    b = r.standard_normal(cout)
    ss, st = stride
    xt = torch.from_numpy(x)
    xp = torch.cat([xt[:, :1], xt[:, :1], xt], dim=1)[:, (st - 1 if aligned else 0):]
    ref = F.conv3d(xp[None], torch.from_numpy(wt), torch.from_numpy(b), stride=(st, ss, ss),
                   padding=(0, 1, 1))[0].numpy()
    got = O.causal_conv3d(x, wt, b, O.REPLICATE, stride_s=ss, stride_t=st, aligned=aligned)
    assert got.shape == ref.shape
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("stride", STRIDES)
@pytest.mark.parametrize("aligned", [False, True])
def test_strided_conv_is_the_subsampled_conv(stride, aligned):
    """Striding takes the stride-1 outputs at frames phase + s_t j and pixels
    (s y, s x), bit for bit (the same sum in the same order)."""
    r = _rng(32)
    x = r.standard_normal((3, 8, 7, 6))
    wt = r.standard_normal((2, 3, 3, 3, 3))
    ss, st = stride
    full = O.causal_conv3d(x, wt, None, O.ZERO)
    got = O.causal_conv3d(x, wt, None, O.ZERO, stride_s=ss, stride_t=st, aligned=aligned)
    assert np.array_equal(got, full[:, (st - 1 if aligned else 0)::st, ::ss, ::ss])


def test_strided_delta_picks_frames_and_pixels():
    """A delta at the current frame and the centre pixel: Y[j,y,x] = X[phase +
    s_t j, 2y, 2x]; at the oldest tap, the frame two before (history for j = 0)."""
    x = _rng(33).standard_normal((2, 9, 6, 5))
    for aligned in (False, True):
        ph = 1 if aligned else 0
        y = O.causal_conv3d(x, _delta(2, 3, 3, 3, 2, 1, 1), None, O.ZERO, stride_s=2, stride_t=2,
                            aligned=aligned)
        assert np.array_equal(y, x[:, ph::2, ::2, ::2])
        y = O.causal_conv3d(x, _delta(2, 3, 3, 3, 0, 1, 1), None, O.ZERO, stride_s=2, stride_t=2,
                            aligned=aligned)
        cur = np.arange(ph, 9, 2)
        for j, tau in enumerate(cur):
            ref = x[:, tau - 2, ::2, ::2] if tau >= 2 else np.zeros_like(x[:, 0, ::2, ::2])
            assert np.array_equal(y[:, j], ref)


STRIDED_SPLITS = [[11], [1] * 11, [1, 4, 4, 2], [3, 2, 6], [2, 2, 2, 5], [5, 6]]


@pytest.mark.parametrize("splits", STRIDED_SPLITS)
@pytest.mark.parametrize("mode", [O.REPLICATE, O.ZERO])
@pytest.mark.parametrize("aligned", [False, True])
def test_strided_chunked_equals_one_shot(splits, mode, aligned):
    """Any chunking, even chunks that hold no output frame, gives the one-shot
    frames: the cache is the window's last k_t-1 input frames whatever the
    stride, and each chunk takes the outputs whose current frame it holds."""
    r = _rng(34)
    x = r.standard_normal((3, 11, 5, 6))
    w = r.standard_normal((2, 3, 3, 3, 3))
    b = r.standard_normal(2)
    ref = O.one_shot(x, w, b, mode, stride_s=2, stride_t=2, aligned=aligned)
    s = O.CausalConvStream(w, b, mode, stride_s=2, stride_t=2, aligned=aligned)
    outs, t0 = [], 0
    for n in splits:
        y = s.step(x[:, t0:t0 + n])
        assert y.shape[1] == O.strided_frames(n, 2, aligned, seen=t0)
        outs.append(y)
        t0 += n
    got = np.concatenate(outs, axis=1)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


def test_strided_frame_counts():
    """1 + 4n frames -> 1 + 2n -> 1 + n with the first frame on its own (361 ->
    181 -> 91, the pages' 91 latents of a 361-frame video); with ``aligned``
    4n -> 2n -> n (28 + 14 x 24 = 364 frames, 91 latents; 7 from the first
    28-frame chunk, 6 from each 24-frame chunk)."""
    n = 361
    for _ in range(2):
        n = O.strided_frames(n, 2)
    assert n == 91
    first, seen1, seen2 = [25] + [24] * 14, 0, 0
    lat = []
    for c in first:
        m = O.strided_frames(c, 2, seen=seen1)
        lat.append(O.strided_frames(m, 2, seen=seen2))
        seen1, seen2 = seen1 + c, seen2 + m
    assert lat == [7] + [6] * 14
    seen1, seen2, lat = 0, 0, []
    for c in [28] + [24] * 14:
        m = O.strided_frames(c, 2, True, seen=seen1)
        lat.append(O.strided_frames(m, 2, True, seen=seen2))
        seen1, seen2 = seen1 + c, seen2 + m
    assert lat == [7] + [6] * 14 and sum(lat) == 91


@pytest.mark.parametrize("aligned", [False, True])
def test_strided_causality(aligned):
    r = _rng(35)
    x = r.standard_normal((2, 9, 4, 4))
    w = r.standard_normal((2, 2, 3, 3, 3))
    base = O.one_shot(x, w, None, O.REPLICATE, stride_s=2, stride_t=2, aligned=aligned)
    cur = np.arange(1 if aligned else 0, 9, 2)  # current frame of each output
    for tp in range(1, 9):
        x2 = x.copy()
        x2[:, tp] += 1.0
        y2 = O.one_shot(x2, w, None, O.REPLICATE, stride_s=2, stride_t=2, aligned=aligned)
        before = cur < tp
        assert np.array_equal(base[:, before], y2[:, before])
        if (~before).any():  # the first output whose current frame is tp or later sees it
            assert not np.array_equal(base[:, ~before][:, :1], y2[:, ~before][:, :1])


def test_conv_points_with_spatial_stride():
    r = _rng(36)
    x = r.standard_normal((3, 4, 7, 6)).astype(np.float32)
    w = r.standard_normal((2, 3, 3, 3, 3))
    b = r.standard_normal(2)
    xp = O.temporal_pad(x.astype(np.float64), 3, O.ZERO)
    full = O.conv_strided(xp, w, b, 0, 1, 2)
    pts = np.array([[t, y, xx] for t in range(4) for y in (0, 1, 3) for xx in (0, 2)])
    got = O.conv_points(xp.astype(np.float32), w, b, pts, down=2)
    ref = np.stack([full[:, t, y, xx] for t, y, xx in pts])
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


# ----------------------------------------------------------------- blocks --

def _params(r, cout, cin, gain=True, bias=False):
    p = {"w": r.standard_normal((cout, cin, 3, 3, 3)) / np.sqrt(cin * 27)}
    p["b"] = r.uniform(-0.1, 0.1, cout) if bias else None
    if gain:
        p["g"] = r.uniform(0.5, 1.5, cin)
    return p


def test_resblock_definition_and_chunking():
    r = _rng(17)
    c = 4
    p1, p2 = _params(r, c, c, bias=True), _params(r, c, c, bias=True)
    x = r.standard_normal((c, 6, 3, 4))
    eps = 1e-6
    a1 = O.act(x, p1["g"], eps)
    h = O.causal_conv3d(a1, p1["w"], p1["b"])
    ref = x + O.causal_conv3d(O.act(h, p2["g"], eps), p2["w"], p2["b"])
    blk = M.ResBlock(p1, p2, eps)
    got = np.concatenate([blk.step(x[:, i:i + 2]) for i in range(0, 6, 2)], axis=1)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_upstage_against_torch_primitives():
    """UpStage = conv2(act(conv1(nearest 2x up of x))), the act taking conv2's
    gain, rebuilt from torch primitives -- repeat_interleave for the nearest
    upsample, the first frame repeated twice ahead of the sequence for the causal
    temporal padding, F.conv3d with zero spatial padding, RMSNorm over channels
    and x * sigmoid(x) written out -- and run by the oracle in uneven chunks."""
    r = _rng(21)
    cin, cmid, cout, t = 3, 5, 4, 6
    p1 = _params(r, cmid, cin, gain=False, bias=True)
    p2 = _params(r, cout, cmid, bias=True)
    x = r.standard_normal((cin, t, 2, 3))
    eps = 1e-6

    def conv(v, p):
        v = torch.cat([v[:, :1], v[:, :1], v], dim=1)
        return F.conv3d(v[None], torch.from_numpy(p["w"]), torch.from_numpy(p["b"]), padding=(0, 1, 1))[0]

    xt = torch.from_numpy(x).repeat_interleave(2, dim=2).repeat_interleave(2, dim=3)
    h = conv(xt, p1)
    nh = h / torch.sqrt((h * h).mean(dim=0, keepdim=True) + eps) * torch.from_numpy(p2["g"])[:, None, None, None]
    ref = conv(nh * torch.sigmoid(nh), p2).numpy()
    stage = M.UpStage(p1, p2, eps)
    got = np.concatenate([stage.step(x[:, a:b]) for a, b in ((0, 1), (1, 4), (4, 6))], axis=1)
    assert got.shape == (cout, t, 4, 6)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_decoder_shapes_and_causality():
    r = _rng(18)
    stages = ((6, 2), (5, 2), (4, 1))
    shapes = M.decoder_layer_shapes(c_latent=3, stages=stages, c_out=3)
    params = {}
    for name, co, ci, kt, kh, kw, has_g in shapes:
        params[name] = {"w": r.standard_normal((co, ci, kt, kh, kw)) / np.sqrt(ci * 27), "b": None,
                        "g": r.uniform(0.5, 1.5, ci) if has_g else None}
    x = r.standard_normal((3, 4, 2, 3))
    dec = M.Decoder(params, stages=stages)
    y = dec.step(x)
    assert y.shape == (3, M.output_frames(4), 2 * 16, 3 * 16)
    # chunked with per-layer caches == one shot
    dec.reset()
    yc = np.concatenate([dec.step(x[:, :1]), dec.step(x[:, 1:3]), dec.step(x[:, 3:])], axis=1)
    assert np.max(np.abs(yc - y)) <= 1e-11
    # latent t' leaves output frames < 4t'-3 unchanged
    x2 = x.copy()
    x2[:, 2] += 1.0
    dec.reset()
    y2 = dec.step(x2)
    assert np.array_equal(y[:, :5], y2[:, :5])
    assert not np.array_equal(y[:, 5], y2[:, 5])


def test_chunk_schedule_golden():
    g = _read_golden("chunk_schedule.txt")
    sched = M.clip_schedule(91)
    frames = []
    done = 0
    for n in sched:
        # frames a clip adds: growth of the video prefix it completes
        frames.append(M.output_frames(done + n) - M.output_frames(done))
        done += n
    assert len(sched) == int(g["n_chunks"])
    assert frames[0] == int(g["first_chunk_read"]) - int(g["first_chunk_dropped"])
    assert all(f == int(g["clip_len"]) for f in frames[1:])
    assert sum(frames) == int(g["total_frames"]) == M.output_frames(91)
    assert M.output_frames(2) - M.output_frames(1) == int(g["pixel_frames_per_latent"])


def test_payload_golden():
    g = _read_golden("payload_1440p.txt")
    n = int(g["frames"]) * int(g["channels"]) * int(g["height"]) * int(g["width"])
    assert round(2 * n / 2**30, 3) == float(g["bf16_gib"])
    assert round(n / 2**30, 3) == float(g["uint8_gib"])
    assert int(g["height"]) == 90 * 16 and int(g["width"]) == 160 * 16


def test_stack_rounding_divergence():
    """The oracle against itself: the decoder stack with every stored tensor
    rounded to bf16, vs the same with a one-fp32-ulp perturbation of every value
    before its rounding (what a different summation order does).  The outputs
    drift apart by far more than one bf16 rounding -- so a multi-layer bf16
    stack can only be held to a wider end-to-end bound than a single layer, and
    layer-wise checks carry the tight bound."""
    r = _rng(19)
    stages = ((64, 2), (32, 2), (16, 1))
    shapes = M.decoder_layer_shapes(c_latent=16, stages=stages)
    params = {n: {"w": O.round_bf16(r.standard_normal((co, ci, kt, kh, kw)) / np.sqrt(ci * 27)), "b": None,
                  "g": r.uniform(0.5, 1.5, ci) if g else None} for n, co, ci, kt, kh, kw, g in shapes}
    x = O.round_bf16(r.standard_normal((16, 6, 3, 5)))
    noise = np.random.default_rng(20)

    def run(store):
        d = M.Decoder(params, stages=stages, store=store)
        return np.concatenate([d.step(x[:, :2]), d.step(x[:, 2:5]), d.step(x[:, 5:])], axis=1)

    ref = run(O.round_bf16)
    alt = run(lambda v: O.round_bf16(v * (1 + noise.standard_normal(v.shape) * 6e-8)))
    d = np.abs(alt - ref)
    mx, mn = d.max() / np.abs(ref).max(), d.mean() / np.abs(ref).mean()
    assert mn > 2e-3          # a single-layer mean bound cannot hold end to end
    assert mx < 1e-2 * 3 and mn < 5e-3 * 3  # the stack bound (3x) leaves room for it


def test_rgb8_quantizer_closed_forms():
    """The 8-bit output map at its fixed points: -1 -> 0, +1 -> 255, 0 -> 128
    (127.5 rounds half to even), clamping outside [-1, 1], and the code of every
    integer level k is recovered from y = k / 127.5 - 1."""
    y = np.array([-1.0, 1.0, 0.0, -3.0, 5.0, np.nextafter(-1.0, 0.0), 1.0 / 255.0])
    assert O.quantize_rgb8(y).tolist() == [0, 255, 128, 0, 255, 0, 128]
    k = np.arange(256)
    assert np.array_equal(O.quantize_rgb8(k / 127.5 - 1.0), k.astype(np.uint8))
    # y = 0 is the one exactly half-way input (t = 127.5): it rounds to the even
    # code 128; just below it rounds down
    assert O.quantize_rgb8(np.array([-1e-9, 1e-9])).tolist() == [127, 128]
    # monotone non-decreasing
    ys = np.linspace(-1.2, 1.2, 10001)
    assert np.all(np.diff(O.quantize_rgb8(ys).astype(int)) >= 0)
    amb = O.rgb8_ambiguous(np.array([0.5 / 127.5 - 1.0, 0.0, 0.25, 0.01 / 127.5]))
    assert amb.tolist() == [True, True, False, False]


# ------------------------------------- TemporalGrow and the aligned first chunk --

def _tg_params(r, c, bias=False):
    pp = {"w": r.standard_normal((c, c, 1, 1, 1)) / np.sqrt(c), "b": r.uniform(-0.1, 0.1, c) if bias else None}
    pt = {"w": r.standard_normal((c, c, 3, 1, 1)) / np.sqrt(3 * c), "b": r.uniform(-0.1, 0.1, c) if bias else None}
    return pp, pt


@pytest.mark.parametrize("aligned", [False, True])
@pytest.mark.parametrize("mode", [O.REPLICATE, O.ZERO])
def test_tg_delta_weights_closed_form(mode, aligned):
    """Identity projection; a temporal delta at the current tap gives the grown
    sequence itself, at the oldest tap the grown sequence two frames back (the
    history rule before it) -- across chunk boundaries too."""
    x = _rng(30).standard_normal((3, 5, 2, 3))
    proj = {"w": _delta(3, 1, 1, 1, 0, 0, 0), "b": None}
    for tap in (2, 0):
        tg = M.TemporalGrow(proj, {"w": _delta(3, 3, 1, 1, tap, 0, 0), "b": None}, 2, mode, aligned=aligned)
        y = np.concatenate([tg.step(x[:, :2]), tg.step(x[:, 2:3]), tg.step(x[:, 3:])], axis=1)
        if aligned:
            v = np.repeat(x, 2, axis=1)                                  # V[2j] = V[2j+1] = X[j]
        else:
            v = np.concatenate([x[:, :1], np.repeat(x[:, 1:], 2, axis=1)], axis=1)  # V[0]=X[0]
        assert y.shape == v.shape
        if tap == 2:
            assert np.array_equal(y, v)
        else:
            assert np.array_equal(y[:, 2:], v[:, :-2])
            for u in range(2):
                expect = v[:, 0] if mode == O.REPLICATE else np.zeros_like(v[:, 0])
                assert np.array_equal(y[:, u], expect)


def test_tg_projection_mixes_channels_only():
    """Projection = the channel matrix at every position and frame (a library
    matmul); factor 1 with a delta at the current tap leaves the frame count."""
    r = _rng(31)
    x = r.standard_normal((4, 3, 2, 5))
    pp, _ = _tg_params(r, 4, bias=True)
    tg = M.TemporalGrow(pp, {"w": _delta(4, 3, 1, 1, 2, 0, 0), "b": None}, 1)
    ref = np.einsum("oc,cthw->othw", pp["w"][:, :, 0, 0, 0], x) + pp["b"][:, None, None, None]
    assert np.max(np.abs(tg.step(x) - ref)) <= 1e-14


@pytest.mark.parametrize("store", [None, O.round_bf16])
def test_tg_commutes_with_nearest_upsample_bitwise(store):
    """TemporalGrow at the input size then nearest 2x == nearest 2x then
    TemporalGrow, bit for bit (it never mixes positions) -- the reorder the
    SwiftVR page reports as bitwise identical."""
    r = _rng(32)
    x = r.standard_normal((5, 4, 3, 4))
    pp, pt = _tg_params(r, 5, bias=True)
    before = M.TemporalGrow(pp, pt, 2, store=store)
    after = M.TemporalGrow(pp, pt, 2, up_s=2, store=store)
    for lo, hi in ((0, 2), (2, 4)):
        a = O.upsample_spatial(before.step(x[:, lo:hi]), 2)
        b = after.step(x[:, lo:hi])
        assert np.array_equal(a, b)


def _decoder_params(r, stages, c_latent, temporal_grow):
    shapes = M.decoder_layer_shapes(c_latent=c_latent, stages=stages, temporal_grow=temporal_grow)
    return {n: {"w": r.standard_normal((co, ci, kt, kh, kw)) / np.sqrt(ci * kt * kh * kw),
                "b": r.uniform(-0.1, 0.1, co), "g": r.uniform(0.5, 1.5, ci) if g else None}
            for n, co, ci, kt, kh, kw, g in shapes}


def test_decoder_tg_orders_bitwise_and_chunked():
    r = _rng(33)
    stages = ((6, 2), (5, 2), (4, 1))
    params = _decoder_params(r, stages, 3, "before")
    x = r.standard_normal((3, 4, 2, 3))
    outs = {}
    for order in ("before", "after"):
        d = M.Decoder(params, stages=stages, temporal_grow=order, store=O.round_bf16)
        outs[order] = np.concatenate([d.step(x[:, :1]), d.step(x[:, 1:3]), d.step(x[:, 3:])], axis=1)
    assert outs["before"].shape == (3, M.output_frames(4), 32, 48)
    assert np.array_equal(outs["before"], outs["after"])
    d = M.Decoder(params, stages=stages, temporal_grow="before", store=O.round_bf16)
    assert np.array_equal(d.step(x), outs["before"])
    with pytest.raises(ValueError):
        M.Decoder(params, stages=stages, temporal_grow="sideways")


@pytest.mark.parametrize("temporal_grow", [None, "before"])
def test_aligned_first_chunk_drops_to_the_same_video(temporal_grow):
    """Aligned growth (every frame doubled from the start) with copies of the
    first frame as history: the decoded video is the other rule's video with
    its first frame three extra times in front -- dropping 3 frames of the
    first chunk gives it back exactly.  With zero history it does not."""
    r = _rng(34)
    stages = ((6, 2), (5, 2), (4, 1))
    params = _decoder_params(r, stages, 3, temporal_grow)
    x = r.standard_normal((3, 5, 2, 3))
    g = _read_golden("chunk_schedule.txt")
    drop = int(g["first_chunk_dropped"])

    def run(aligned, mode):
        d = M.Decoder(params, stages=stages, temporal_grow=temporal_grow, aligned=aligned, mode=mode,
                      store=O.round_bf16)
        return [d.step(x[:, :3]), d.step(x[:, 3:])]

    once, al = run(False, O.REPLICATE), run(True, O.REPLICATE)
    assert al[0].shape[1] == M.output_frames(3, aligned=True) == M.output_frames(3) + drop
    assert al[1].shape == once[1].shape
    assert np.array_equal(al[0][:, drop:], once[0]) and np.array_equal(al[1], once[1])
    for u in range(drop):
        assert np.array_equal(al[0][:, u], once[0][:, 0])
    z_once, z_al = run(False, O.ZERO), run(True, O.ZERO)
    assert not np.array_equal(z_al[0][:, drop:], z_once[0])


def test_aligned_schedule_golden():
    """The reader's 28-frame first chunk is 7 latents grown by 4 with no frame
    kept single; dropping 3 leaves the 25 frames of the other rule."""
    g = _read_golden("chunk_schedule.txt")
    assert M.output_frames(7, aligned=True) == int(g["first_chunk_read"])
    assert M.output_frames(7, aligned=True) - int(g["first_chunk_dropped"]) == M.output_frames(7)
    assert M.output_frames(6, aligned=True) == int(g["clip_len"])


# ------------------------- the decoder's composition, rebuilt from primitives --

def _t_causal(v, p, mode):
    """One-shot causal conv of a [C][T][H][W] float64 tensor with torch's conv3d:
    k_t-1 history frames (copies of frame 0, or zeros) ahead of the sequence,
    zero spatial padding of (k-1)/2."""
    w = torch.from_numpy(p["w"])
    kt, kh, kw = w.shape[2:]
    first = v[:, :1] if mode == O.REPLICATE else torch.zeros_like(v[:, :1])
    v = torch.cat([first] * (kt - 1) + [v], dim=1)
    b = None if p.get("b") is None else torch.from_numpy(p["b"])
    return F.conv3d(v[None], w, b, padding=(0, (kh - 1) // 2, (kw - 1) // 2))[0]


def _t_act(v, g, eps=1e-6):
    n = v / torch.sqrt((v * v).mean(dim=0, keepdim=True) + eps) * torch.from_numpy(g)[:, None, None, None]
    return n * torch.sigmoid(n)


def _t_up2(v):
    return v.repeat_interleave(2, dim=2).repeat_interleave(2, dim=3)


def _t_grow(v, factor, aligned):
    """Frame growth of the whole video: factor 1 keeps it; factor 2 doubles every
    frame after the first (the first too under the aligned rule)."""
    if factor == 1:
        return v
    if aligned:
        return v.repeat_interleave(2, dim=1)
    return torch.cat([v[:, :1], v[:, 1:].repeat_interleave(2, dim=1)], dim=1)


def _t_decoder(params, x, stages, temporal_grow, aligned, mode):
    """The decoder of reading B composed one-shot over the whole video from torch
    primitives, written apart from oracle/model.py: conv_in; per stage [nearest
    2x in space (and the stage's growth in time) -> conv -> two residual blocks
    x + conv2(act(conv1(act(x))))], where a TemporalGrow (1x1x1 projection,
    growth, causal 3x1x1 conv) takes over the stage's growth, either at the
    stage's input size ("before") or on the upsampled positions ("after"); head:
    act at the low size -> nearest 2x -> conv to RGB."""
    h = _t_causal(torch.from_numpy(x), params["conv_in"], mode)
    for si, (_, factor) in enumerate(stages):
        if temporal_grow is None:
            h = _t_causal(_t_grow(_t_up2(h), factor, aligned), params["s%d.up" % si], mode)
        else:
            if temporal_grow == "after":
                h = _t_up2(h)
            q = _t_causal(h, params["s%d.tg.p" % si], mode)
            q = _t_causal(_t_grow(q, factor, aligned), params["s%d.tg.t" % si], mode)
            h = _t_causal(q if temporal_grow == "after" else _t_up2(q), params["s%d.up" % si], mode)
        for r in range(2):
            p1, p2 = params["s%d.rb%d.c1" % (si, r)], params["s%d.rb%d.c2" % (si, r)]
            h = h + _t_causal(_t_act(_t_causal(_t_act(h, p1["g"]), p1, mode), p2["g"]), p2, mode)
    return _t_causal(_t_up2(_t_act(h, params["head"]["g"])), params["head"], mode).numpy()


DECODER_PIN_CASES = [
    # stages, temporal_grow, aligned, history, chunks
    (((6, 2), (5, 2), (4, 1)), None, False, O.REPLICATE, (1, 2, 1)),
    (((6, 2), (5, 2), (4, 1)), None, True, O.REPLICATE, (3, 1)),
    (((5, 1), (4, 2)), None, False, O.ZERO, (2, 2)),
    (((6, 2), (5, 2), (4, 1)), "before", False, O.REPLICATE, (2, 2)),
    (((6, 2), (5, 2), (4, 1)), "after", False, O.REPLICATE, (1, 3)),
    (((5, 2), (4, 1)), "before", True, O.ZERO, (1, 1, 2)),
]


@pytest.mark.parametrize("case", DECODER_PIN_CASES, ids=lambda c: "%dst_tg%s_al%d_%s" % (
    len(c[0]), c[1], c[2], c[3]))
def test_decoder_against_torch_primitives(case):
    """oracle/model.py's Decoder, run chunk by chunk with per-layer caches, equals
    the same decoder composed one-shot from torch primitives (F.conv3d on
    explicitly padded input, repeat_interleave for the nearest upsample and the
    frame growth, RMSNorm and x * sigmoid(x) written out) to 1e-12: a dropped or
    misplaced act, residual, gain, stage or growth in the oracle's wiring fails."""
    stages, tg, aligned, mode, chunks = case
    r = _rng(40 + DECODER_PIN_CASES.index(case))
    c_lat = 3
    params = _decoder_params(r, stages, c_lat, tg)
    x = r.standard_normal((c_lat, sum(chunks), 2, 3))
    ref = _t_decoder(params, x, stages, tg, aligned, mode)
    dec = M.Decoder(params, stages=stages, temporal_grow=tg, aligned=aligned, mode=mode)
    got, t0 = [], 0
    for n in chunks:
        got.append(dec.step(x[:, t0:t0 + n]))
        t0 += n
    got = np.concatenate(got, axis=1)
    up = 2 ** (len(stages) + 1)
    assert got.shape == ref.shape == (3, M.output_frames(sum(chunks), [f for _, f in stages], aligned=aligned),
                                      2 * up, 3 * up)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


# ------------------------- the encoder's composition, rebuilt from primitives --

def _encoder_params(r, stages, c_in, c_latent):
    shapes = M.encoder_layer_shapes(c_in=c_in, stages=stages, c_latent=c_latent)
    return {n: {"w": r.standard_normal((co, ci, kt, kh, kw)) / np.sqrt(ci * kt * kh * kw),
                "b": r.uniform(-0.1, 0.1, co), "g": r.uniform(0.5, 1.5, ci) if g else None}
            for n, co, ci, kt, kh, kw, g, _, _ in shapes}


def _t_strided(v, p, mode, ss, st, aligned):
    """One-shot strided causal conv with torch's conv3d: the history frames ahead
    of the sequence, the first window starting at the phase (0, or st - 1 with
    the aligned rule), stride (st, ss, ss), zero spatial padding (k-1)/2."""
    w = torch.from_numpy(p["w"])
    kt, kh, kw = w.shape[2:]
    first = v[:, :1] if mode == O.REPLICATE else torch.zeros_like(v[:, :1])
    v = torch.cat([first] * (kt - 1) + [v], dim=1)[:, (st - 1 if aligned else 0):]
    b = None if p.get("b") is None else torch.from_numpy(p["b"])
    return F.conv3d(v[None], w, b, stride=(st, ss, ss), padding=(0, (kh - 1) // 2, (kw - 1) // 2))[0]


def _t_encoder(params, x, stages, aligned, mode):
    """The encoder read backwards from the decoder, one-shot from torch
    primitives: stride-2 conv from the pixels; per stage, the decoder's stages
    from the last, two residual blocks then a conv with spatial stride 2 and
    the stage's temporal factor as temporal stride; act -> conv to the latent."""
    h = _t_strided(torch.from_numpy(x), params["conv_in"], mode, 2, 1, aligned)
    for ei in range(len(stages)):
        factor = stages[len(stages) - 1 - ei][1]
        for r in range(2):
            p1, p2 = params["e%d.rb%d.c1" % (ei, r)], params["e%d.rb%d.c2" % (ei, r)]
            h = h + _t_causal(_t_act(_t_causal(_t_act(h, p1["g"]), p1, mode), p2["g"]), p2, mode)
        h = _t_strided(h, params["e%d.down" % ei], mode, 2, factor, aligned)
    return _t_causal(_t_act(h, params["conv_out"]["g"]), params["conv_out"], mode).numpy()


ENCODER_PIN_CASES = [
    # stages (as the decoder lists them), aligned, history, chunks
    (((6, 2), (5, 2), (4, 1)), False, O.ZERO, (5, 4)),
    (((6, 2), (5, 2), (4, 1)), True, O.ZERO, (4, 8)),
    (((6, 2), (5, 2), (4, 1)), False, O.REPLICATE, (1, 2, 3, 3)),
    (((5, 1), (4, 2)), True, O.REPLICATE, (2, 3, 1)),
]


@pytest.mark.parametrize("case", ENCODER_PIN_CASES, ids=lambda c: "%dst_al%d_%s" % (len(c[0]), c[1], c[2]))
def test_encoder_against_torch_primitives(case):
    """oracle/model.py's Encoder, chunk by chunk with per-layer caches (chunks that
    do not split evenly into the strides included), equals the same encoder
    composed one-shot from torch primitives to 1e-12."""
    stages, aligned, mode, chunks = case
    r = _rng(60 + ENCODER_PIN_CASES.index(case))
    c_in, c_lat = 3, 4
    params = _encoder_params(r, stages, c_in, c_lat)
    down = 2 ** (len(stages) + 1)
    x = r.standard_normal((c_in, sum(chunks), 2 * down, 3 * down))
    ref = _t_encoder(params, x, stages, aligned, mode)
    enc = M.Encoder(params, stages=stages, aligned=aligned, mode=mode)
    got, t0 = [], 0
    for n in chunks:
        got.append(enc.step(x[:, t0:t0 + n]))
        t0 += n
    got = np.concatenate(got, axis=1)
    n = sum(chunks)
    for _, f in reversed(stages):
        n = O.strided_frames(n, f, aligned)
    assert got.shape == ref.shape == (c_lat, n, 2, 3)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_encoder_causality():
    """Perturbing input frame t' leaves every latent whose last input frame is
    before t' bit for bit unchanged (latent j of the first-frame rule ends at
    frame 4j with two 2x strides)."""
    stages = ((5, 2), (4, 2), (3, 1))
    r = _rng(70)
    params = _encoder_params(r, stages, 3, 2)
    x = r.standard_normal((3, 9, 16, 16))
    base = M.Encoder(params, stages=stages).step(x)
    for tp in (1, 4, 5, 8):
        x2 = x.copy()
        x2[:, tp] += 1.0
        y2 = M.Encoder(params, stages=stages).step(x2)
        keep = (tp + 3) // 4  # latents 0 .. keep-1 end before frame tp
        assert np.array_equal(base[:, :keep], y2[:, :keep])
        assert not np.array_equal(base[:, keep], y2[:, keep])
