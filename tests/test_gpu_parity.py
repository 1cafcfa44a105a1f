"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles and ragged tails."""
import ctypes

import numpy as np
import pytest
import torch

from causal_convolution_x3x3_amd import capi as C
from causal_convolution_x3x3_amd import plan as P
from causal_convolution_x3x3_amd import stacks as S
from causal_convolution_x3x3_amd import synth
from oracle import model as OM
from oracle import oracle as O

import stack_cases as SC
from helpers import (assert_bf16_close, assert_fp32_close, assert_stack_close, from_device_cl, say,
                     to_device_cl, to_oracle)

pytestmark = pytest.mark.gpu

TP = {C.TPAD_REPLICATE: O.REPLICATE, C.TPAD_ZERO: O.ZERO}


def _run_chunks(plan, x_cl, splits, residual_cl=None):
    st = P.Stream(plan)
    outs, t0, r0 = [], 0, 0
    for n in splits:
        res = None
        if residual_cl is not None:
            first = st.frames_seen == 0
            tn = plan.output_shape(n, first)[0]
            res = residual_cl[r0:r0 + tn].clone()  # a fresh (16-byte aligned) buffer
            r0 += tn
        # a fresh buffer: a slice of frames whose byte size is not a multiple
        # of 16 would break the library's 16-byte alignment rule
        outs.append(st.step(x_cl[t0:t0 + n].clone(), residual=res))
        t0 += n
    torch.cuda.synchronize()
    return torch.cat(outs, dim=0)


# -------------------------------------------------------------- fp32 conv --

@pytest.mark.parametrize("tpad", [C.TPAD_REPLICATE, C.TPAD_ZERO])
@pytest.mark.parametrize("splits", [[9], [1, 4, 4], [1] * 9])
def test_c0_fp32_conv_chunked(tpad, splits):
    say("c0 fp32 tpad=%d splits=%s" % (tpad, splits))
    wl = synth.WORKLOADS[0]
    x = synth.video(wl["cin"], wl["t"], wl["h"], wl["w"], synth.seed(0, 1))
    w = synth.conv_weight(wl["cout"], wl["cin"], 3, 3, 3, synth.seed(0, 2))
    ref = O.causal_conv3d(to_oracle(x), to_oracle(w), None, TP[tpad])
    plan = P.conv_plan(w.cuda(), wl["h"], wl["w"], max_chunk_t=9, tpad=tpad)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    assert_fp32_close(got, ref, "c0")


@pytest.mark.parametrize("h,w,k,up_s,up_t,tpad", [
    (1, 1, (3, 3, 3), 1, 1, C.TPAD_REPLICATE),
    (1, 2, (3, 3, 3), 2, 2, C.TPAD_ZERO),
    (2, 1, (2, 1, 3), 2, 1, C.TPAD_REPLICATE),
])
def test_fp32_conv_tiny_frames(h, w, k, up_s, up_t, tpad):
    """fp32 convs on frames of one or two pixels, 1-frame chunks included."""
    say("fp32 tiny frame %dx%d k=%s up=%d/%d" % (h, w, k, up_s, up_t))
    x = synth.video(8, 5, h, w, synth.seed(0, 31))
    wt = synth.conv_weight(4, 8, *k, synth.seed(0, 32))
    b = synth.bias(4, synth.seed(0, 33))
    ref = O.one_shot(to_oracle(x), to_oracle(wt), to_oracle(b), TP[tpad], up_s, up_t)
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), up_s=up_s, up_t=up_t, max_chunk_t=3, tpad=tpad)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), [1, 3, 1]))
    assert_fp32_close(got, ref, "fp32 tiny frame")


def _random_fp32_cases(n, seed):
    """Seeded draws for the fp32 conv: any channel counts (no multiple-of-8
    rule), kernel shapes, nearest 2x in space and time, frame sizes, chunkings,
    history fills, with and without bias."""
    rng = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        k = [(3, 3, 3), (3, 3, 3), (1, 1, 1), (3, 1, 1), (2, 3, 3), (1, 3, 3), (2, 1, 3)][rng.randint(7)]
        cin, cout = int(rng.randint(1, 40)), int(rng.randint(1, 40))
        up_s, up_t = int(rng.randint(1, 3)), int(rng.randint(1, 3))
        h, w = int(rng.randint(1, 12)), int(rng.randint(1, 30))
        splits = [int(v) for v in rng.randint(1, 4, size=rng.randint(1, 4))]
        tpad = [C.TPAD_REPLICATE, C.TPAD_ZERO][rng.randint(2)]
        cases.append((cin, cout, k, up_s, up_t, h, w, splits, tpad, bool(rng.randint(2))))
    return cases


@pytest.mark.parametrize("case", _random_fp32_cases(16, 5), ids=lambda c: "ci%d_co%d_k%d%d%d_up%d%d_%dx%d" % (
    c[0], c[1], c[2][0], c[2][1], c[2][2], c[3], c[4], c[5], c[6]))
def test_fp32_conv_random_shapes(case):
    cin, cout, k, up_s, up_t, h, w, splits, tpad, with_bias = case
    say("fp32 conv, random shape %s" % (case,))
    x = synth.video(cin, sum(splits), h, w, synth.seed(0, 51))
    wt = synth.conv_weight(cout, cin, *k, synth.seed(0, 52))
    b = synth.bias(cout, synth.seed(0, 53)) if with_bias else None
    ref = O.one_shot(to_oracle(x), to_oracle(wt), None if b is None else to_oracle(b), TP[tpad], up_s, up_t)
    plan = P.conv_plan(wt.cuda(), h, w, bias=None if b is None else b.cuda(), up_s=up_s, up_t=up_t,
                       max_chunk_t=max(splits), tpad=tpad)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    assert_fp32_close(got, ref, "random-shape fp32 conv")


def test_fp32_memoryblock_zero_history_with_bias_and_upsample():
    say("fp32 memoryblock kt=2")
    x = synth.video(8, 5, 6, 7, synth.seed(0, 11))
    w = synth.conv_weight(4, 8, 2, 3, 3, synth.seed(0, 12))
    b = synth.bias(4, synth.seed(0, 13))
    ref = O.one_shot(to_oracle(x), to_oracle(w), to_oracle(b), O.ZERO, up_s=2, up_t=2)
    plan = P.conv_plan(w.cuda(), 6, 7, bias=b.cuda(), up_s=2, up_t=2, max_chunk_t=4, tpad=C.TPAD_ZERO)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), [1, 2, 2]))
    assert_fp32_close(got, ref, "memoryblock")


# -------------------------------------------------------------- bf16 conv --

BF16_CASES = [
    # cin, cout, k, up_s, up_t, h, w, splits, tpad, bias
    (32, 16, (3, 3, 3), 1, 1, 20, 36, [1, 3, 2], C.TPAD_REPLICATE, False),
    (48, 96, (3, 3, 3), 1, 1, 18, 33, [2, 2], C.TPAD_REPLICATE, True),
    (64, 128, (3, 3, 3), 2, 1, 9, 21, [1, 2], C.TPAD_REPLICATE, False),
    (64, 192, (3, 3, 3), 1, 2, 10, 17, [1, 2, 1], C.TPAD_ZERO, True),
    (32, 3, (3, 3, 3), 2, 1, 12, 20, [1, 2], C.TPAD_REPLICATE, True),
    (128, 96, (3, 3, 3), 2, 1, 8, 40, [1, 3], C.TPAD_REPLICATE, False),
    (32, 128, (3, 3, 3), 1, 1, 11, 70, [2, 1], C.TPAD_ZERO, True),
    (96, 96, (3, 3, 3), 1, 1, 17, 131, [1, 2], C.TPAD_REPLICATE, False),
    (192, 96, (3, 3, 3), 2, 1, 9, 35, [2, 1], C.TPAD_REPLICATE, True),
    (384, 384, (3, 3, 3), 2, 2, 5, 6, [1, 1], C.TPAD_REPLICATE, False),
    # eight 96-channel blocks: each block's items on its own XCD (the 4- and
    # 8-block dealing), with and without nearest 2x
    (32, 768, (3, 3, 3), 1, 1, 9, 20, [1, 2], C.TPAD_REPLICATE, True),
    (32, 768, (3, 3, 3), 2, 1, 5, 7, [2, 1], C.TPAD_ZERO, True),
    (16, 32, (2, 1, 1), 1, 1, 7, 19, [1, 2, 2], C.TPAD_ZERO, False),
    (16, 64, (1, 3, 3), 2, 1, 7, 9, [2, 1], C.TPAD_REPLICATE, True),
    (24, 16, (3, 1, 1), 1, 2, 5, 17, [2, 1], C.TPAD_ZERO, False),
    # TemporalGrow shapes: 1x1x1 projection (also on upsampled positions), 3x1x1 growing temporal conv
    (384, 384, (1, 1, 1), 1, 1, 5, 9, [1, 2], C.TPAD_REPLICATE, True),
    (192, 192, (1, 1, 1), 2, 1, 5, 7, [2, 1], C.TPAD_REPLICATE, False),
    (384, 384, (3, 1, 1), 1, 2, 4, 9, [1, 2, 1], C.TPAD_REPLICATE, True),
    (192, 192, (3, 1, 1), 1, 1, 7, 5, [2, 2], C.TPAD_ZERO, False),
    # pointwise kernel: ragged last position tile, Cin not a multiple of 64, three
    # 96-channel blocks with nearest 2x and zero history, a growing 3x1x1 conv
    (104, 96, (1, 1, 1), 1, 1, 37, 41, [2, 1], C.TPAD_REPLICATE, True),
    (64, 288, (2, 1, 1), 2, 1, 13, 19, [1, 2], C.TPAD_ZERO, True),
    (192, 384, (3, 1, 1), 1, 2, 11, 23, [1, 3], C.TPAD_REPLICATE, False),
    # output head (taps in the GEMM's N): ragged tiles, runs of frames, cout < 3
    (96, 3, (3, 3, 3), 2, 1, 13, 37, [1, 4, 3], C.TPAD_REPLICATE, True),
    (64, 2, (3, 3, 3), 2, 2, 9, 20, [1, 3, 2], C.TPAD_ZERO, True),
    (96, 1, (3, 3, 3), 2, 1, 8, 16, [2, 5], C.TPAD_REPLICATE, False),
    (32, 3, (3, 3, 3), 2, 1, 128, 1024, [2, 5], C.TPAD_REPLICATE, True),
    # ... at the input's own size (the 1440p stage's last conv)
    (96, 3, (3, 3, 3), 1, 1, 13, 37, [1, 4, 3], C.TPAD_REPLICATE, True),
    (64, 2, (3, 3, 3), 1, 1, 9, 20, [1, 3, 2], C.TPAD_ZERO, True),
    (32, 3, (3, 3, 3), 1, 2, 17, 33, [2, 3], C.TPAD_REPLICATE, False),
    (96, 1, (3, 3, 3), 1, 1, 16, 16, [3], C.TPAD_REPLICATE, False),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "ci%d_co%d_k%s_us%d_ut%d" % (c[0], c[1], "".join(map(str, c[2])), c[3], c[4]))
def test_bf16_conv_vs_oracle(case):
    cin, cout, k, up_s, up_t, h, w, splits, tpad, with_bias = case
    say("bf16 conv %s" % (case,))
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(5, 1)))
    wt = synth.bf16(synth.conv_weight(cout, cin, *k, synth.seed(5, 2)))
    b = synth.bias(cout, synth.seed(5, 3)) if with_bias else None
    ref = O.one_shot(to_oracle(x), to_oracle(wt), None if b is None else to_oracle(b), TP[tpad], up_s, up_t)
    plan = P.conv_plan(wt.cuda(), h, w, bias=None if b is None else b.cuda(), up_s=up_s, up_t=up_t,
                       max_chunk_t=max(splits), tpad=tpad)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    assert_bf16_close(got, ref, "bf16 conv")


TINY_CASES = [
    # cin, cout, k, up_s, up_t, h, w, splits, tpad, fold, kernel that must run:
    # frames of one or two pixels -- a single tile mostly border and padding --
    # through every kernel family, with growth, zero history and 1-frame chunks
    (96, 96, (3, 3, 3), 1, 1, 1, 1, [1, 2], C.TPAD_REPLICATE, False, "conv_bf16_v2_up1_k3_n96"),
    (64, 192, (3, 3, 3), 1, 2, 2, 1, [1, 1, 2], C.TPAD_ZERO, False, "conv_bf16_v2_up1_k3_n96"),
    (96, 96, (3, 3, 3), 2, 1, 1, 2, [2, 1], C.TPAD_REPLICATE, False, "conv_bf16_v2_up2_k3_n96"),
    (96, 96, (3, 3, 3), 2, 2, 1, 1, [1, 2, 1], C.TPAD_REPLICATE, True, "conv_bf16_phase_up2_k3_n96"),
    (128, 96, (3, 3, 3), 2, 1, 2, 1, [1, 2], C.TPAD_ZERO, True, "conv_bf16_phase_up2_k3_n96"),
    (96, 3, (3, 3, 3), 2, 1, 1, 1, [1, 2], C.TPAD_REPLICATE, False, "conv_bf16_head_up2_k3_c3"),
    (64, 2, (3, 3, 3), 1, 1, 2, 1, [2, 1], C.TPAD_ZERO, False, "conv_bf16_head_up1_k3_c2"),
    (96, 96, (1, 1, 1), 1, 1, 1, 1, [1, 1], C.TPAD_REPLICATE, False, "conv_bf16_pw_up1_kt1_n96"),
    (192, 192, (3, 1, 1), 2, 2, 1, 1, [1, 2], C.TPAD_ZERO, False, "conv_bf16_pw_up2_kt3_n192"),
    (16, 32, (3, 3, 3), 1, 1, 1, 1, [1, 2], C.TPAD_REPLICATE, False, "conv_bf16_up1_k3_n"),
]


@pytest.mark.parametrize("case", TINY_CASES, ids=lambda c: "%s_%dx%d" % (c[10], c[5], c[6]))
def test_bf16_conv_tiny_frames(case):
    """Degenerate frame sizes (1x1, 1x2, 2x1 pixels) through each kernel family
    against the definition; the profiled kernel name shows which one ran."""
    cin, cout, k, up_s, up_t, h, w, splits, tpad, fold, kname = case
    say("bf16 conv, tiny frame %s" % (case,))
    x = synth.bf16(synth.video(cin, sum(splits), h, w, synth.seed(5, 41)))
    wt = synth.bf16(synth.conv_weight(cout, cin, *k, synth.seed(5, 42)))
    b = synth.bias(cout, synth.seed(5, 43))
    ref = O.one_shot(to_oracle(x), to_oracle(wt), to_oracle(b), TP[tpad], up_s, up_t)
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), up_s=up_s, up_t=up_t, max_chunk_t=max(splits), tpad=tpad,
                       fold_upsample=fold)
    C.check(C.lib().cc3d_profile_enable(plan._h, 1), "profile_enable")
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    pr = C.OpProfile()
    C.check(C.lib().cc3d_profile_read(plan._h, 0, 0, ctypes.byref(pr)), "profile_read")
    assert pr.kernel.decode().startswith(kname), pr.kernel
    assert_bf16_close(got, ref, "tiny frame conv")


def _random_conv_cases(n, seed):
    """Seeded draws over what a bf16 conv plan accepts: channels (multiples of 8),
    kernel shapes, nearest 2x in space and time, frame sizes, chunkings, history
    fills and the folding request -- so that combinations the listed cases miss
    still meet the definition."""
    rng = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        k = [(3, 3, 3), (3, 3, 3), (1, 1, 1), (3, 1, 1), (2, 3, 3), (1, 3, 3)][rng.randint(6)]
        cin = int(rng.choice([8, 16, 32, 48, 64, 96, 128, 192]))
        cout = int(rng.choice([1, 2, 3, 8, 16, 24, 96, 192]))
        up_s, up_t = int(rng.randint(1, 3)), int(rng.randint(1, 3))
        h, w = int(rng.randint(1, 14)), int(rng.randint(1, 40))
        splits = [int(v) for v in rng.randint(1, 4, size=rng.randint(1, 4))]
        tpad = [C.TPAD_REPLICATE, C.TPAD_ZERO][rng.randint(2)]
        cases.append((cin, cout, k, up_s, up_t, h, w, splits, tpad, bool(rng.randint(2)), bool(rng.randint(2))))
    return cases


@pytest.mark.parametrize("case", _random_conv_cases(24, 2026), ids=lambda c: "ci%d_co%d_k%d%d%d_up%d%d_%dx%d" % (
    c[0], c[1], c[2][0], c[2][1], c[2][2], c[3], c[4], c[5], c[6]))
def test_bf16_conv_random_shapes(case):
    cin, cout, k, up_s, up_t, h, w, splits, tpad, with_bias, fold = case
    say("bf16 conv, random shape %s" % (case,))
    x = synth.bf16(synth.video(cin, sum(splits), h, w, synth.seed(5, 61)))
    wt = synth.bf16(synth.conv_weight(cout, cin, *k, synth.seed(5, 62)))
    b = synth.bias(cout, synth.seed(5, 63)) if with_bias else None
    ref = O.one_shot(to_oracle(x), to_oracle(wt), None if b is None else to_oracle(b), TP[tpad], up_s, up_t)
    plan = P.conv_plan(wt.cuda(), h, w, bias=None if b is None else b.cuda(), up_s=up_s, up_t=up_t,
                       max_chunk_t=max(splits), tpad=tpad, fold_upsample=fold)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    assert_bf16_close(got, ref, "random-shape conv")


def _random_epilogue_cases(n, seed):
    """Seeded draws as above with the epilogue as well: a residual added before
    the store, the pre-activation of the stored sum, or both."""
    rng = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        k = [(3, 3, 3), (3, 3, 3), (1, 1, 1), (3, 1, 1)][rng.randint(4)]
        cin = int(rng.choice([16, 32, 64, 96, 192]))
        cout = int(rng.choice([8, 16, 24, 96, 96, 192, 256, 384]))
        up_s, up_t = int(rng.randint(1, 3)), int(rng.randint(1, 3))
        h, w = int(rng.randint(1, 12)), int(rng.randint(1, 36))
        splits = [int(v) for v in rng.randint(1, 4, size=rng.randint(1, 4))]
        tpad = [C.TPAD_REPLICATE, C.TPAD_ZERO][rng.randint(2)]
        epi = [(True, False), (False, True), (True, True)][rng.randint(3)]
        cases.append((cin, cout, k, up_s, up_t, h, w, splits, tpad, epi[0], epi[1], bool(rng.randint(2))))
    return cases


@pytest.mark.parametrize("case", _random_epilogue_cases(16, 7), ids=lambda c: "ci%d_co%d_k%d%d%d_up%d%d_r%d_a%d" % (
    c[0], c[1], c[2][0], c[2][1], c[2][2], c[3], c[4], c[9], c[10]))
def test_bf16_conv_random_epilogues(case):
    cin, cout, k, up_s, up_t, h, w, splits, tpad, residual, act, fold = case
    say("bf16 conv, random epilogue %s" % (case,))
    x = synth.bf16(synth.video(cin, sum(splits), h, w, synth.seed(5, 71)))
    wt = synth.bf16(synth.conv_weight(cout, cin, *k, synth.seed(5, 72)))
    b = synth.bias(cout, synth.seed(5, 73))
    g = synth.gain(cout, synth.seed(5, 74))
    v = O.one_shot(to_oracle(x), to_oracle(wt), to_oracle(b), TP[tpad], up_s, up_t)
    r = synth.bf16(synth.video(cout, *v.shape[1:], synth.seed(5, 75))) if residual else None
    if residual:
        v = v + to_oracle(r)
    ref = O.act(O.round_bf16(v), to_oracle(g), 1e-6) if act else v
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), gamma=g.cuda() if act else None, up_s=up_s, up_t=up_t,
                       max_chunk_t=max(splits), tpad=tpad, residual=residual, act=act, fold_upsample=fold)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits,
                                     residual_cl=to_device_cl(r) if residual else None))
    assert_bf16_close(got, ref, "random epilogue")


@pytest.mark.parametrize("k,up_s", [((1, 1, 1), 2), ((3, 1, 1), 1)])
def test_bf16_pointwise_conv_residual(k, up_s):
    """The pointwise kernel's epilogue: + bias + residual, stored as bf16."""
    say("bf16 pointwise conv + residual k=%s up_s=%d" % (k, up_s))
    cin, cout, h, w, splits = 96, 192, 9, 30, [1, 2]
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(5, 21)))
    wt = synth.bf16(synth.conv_weight(cout, cin, *k, synth.seed(5, 22)))
    b = synth.bias(cout, synth.seed(5, 23))
    r = synth.bf16(synth.video(cout, t, h * up_s, w * up_s, synth.seed(5, 24)))
    ref = O.one_shot(to_oracle(x), to_oracle(wt), to_oracle(b), O.REPLICATE, up_s) + to_oracle(r)
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), up_s=up_s, residual=True, max_chunk_t=2)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits, residual_cl=to_device_cl(r)))
    assert_bf16_close(got, ref, "pointwise + residual")


PHASE_CASES = [
    # cin, cout, up_t, h, w, splits, tpad, bias, kt, aligned: ragged tiles, two and
    # four 96-channel blocks; with time doubled the temporal taps that read one
    # frame are grouped: zero history (the two history taps read nothing), the
    # replicated first frame (all three taps read X[0]), the two cached frames,
    # pairs of taps in either place, kt = 2 and 1, the aligned growth rule
    (192, 96, 1, 10, 70, [1, 2], C.TPAD_REPLICATE, True, 3, False),
    (128, 96, 2, 9, 40, [1, 2, 1], C.TPAD_ZERO, False, 3, False),
    (96, 192, 1, 7, 130, [2, 1], C.TPAD_REPLICATE, True, 3, False),
    (384, 384, 2, 5, 6, [1, 1], C.TPAD_REPLICATE, False, 3, False),
    (96, 96, 2, 6, 20, [2, 3], C.TPAD_REPLICATE, True, 2, False),
    (64, 96, 2, 5, 9, [1, 2], C.TPAD_ZERO, False, 1, False),
    (160, 96, 2, 8, 17, [3, 1, 2], C.TPAD_ZERO, True, 3, True),
]


@pytest.mark.parametrize("case", PHASE_CASES, ids=lambda c: "ci%d_co%d_ut%d_kt%d%s" % (
    c[:3] + (c[8], "_aligned" if c[9] else "")))
def test_phase_folded_upsample_conv(case):
    """fold_upsample: the nearest-2x 3x3x3 conv computed per output phase from
    folded hi/lo weights (spatial taps, and temporal taps that read one frame,
    summed) matches the definition."""
    cin, cout, up_t, h, w, splits, tpad, with_bias, kt, aligned = case
    say("phase-folded upsample conv %s" % (case,))
    x = synth.bf16(synth.video(cin, sum(splits), h, w, synth.seed(13, 1)))
    wt = synth.bf16(synth.conv_weight(cout, cin, kt, 3, 3, synth.seed(13, 2)))
    b = synth.bias(cout, synth.seed(13, 3)) if with_bias else None
    ref = O.one_shot(to_oracle(x), to_oracle(wt), None if b is None else to_oracle(b), TP[tpad], 2, up_t,
                     aligned=aligned)
    plan = P.conv_plan(wt.cuda(), h, w, bias=None if b is None else b.cuda(), up_s=2, up_t=up_t,
                       max_chunk_t=max(splits), tpad=tpad, aligned=aligned, fold_upsample=True)
    C.check(C.lib().cc3d_profile_enable(plan._h, 1), "profile_enable")
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    pr = C.OpProfile()
    C.check(C.lib().cc3d_profile_read(plan._h, 0, 0, ctypes.byref(pr)), "profile_read")
    assert pr.kernel.decode() == "conv_bf16_phase_up2_k3_n96", pr.kernel
    assert_bf16_close(got, ref, "phase-folded conv")


@pytest.mark.parametrize("residual", [False, True])
def test_phase_folded_conv_fused_act(residual):
    """The phase kernel's epilogue: bias (+ residual) stored as bf16 and the
    fused SiLU(RMSNorm(.)) of the stored value."""
    say("phase-folded conv, fused act, residual=%s" % residual)
    cin, cout, h, w, splits = 64, 96, 9, 30, [1, 2]
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(13, 11)))
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(13, 12)))
    b = synth.bias(cout, synth.seed(13, 13))
    g = synth.gain(cout, synth.seed(13, 14))
    r = synth.bf16(synth.video(cout, t, 2 * h, 2 * w, synth.seed(13, 15))) if residual else None
    v = O.one_shot(to_oracle(x), to_oracle(wt), to_oracle(b), O.REPLICATE, 2)
    if residual:
        v = v + to_oracle(r)
    ref = O.act(O.round_bf16(v), to_oracle(g), 1e-6)
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), gamma=g.cuda(), act=True, residual=residual, up_s=2,
                       max_chunk_t=2, fold_upsample=True)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits,
                                     residual_cl=to_device_cl(r) if residual else None))
    assert_bf16_close(got, ref, "phase-folded epilogue")


def test_fp32_conv_aligned_growth():
    """The fp32 kernel under CC3D_GROW_ALIGNED, against the oracle to the fp32 bound."""
    say("fp32 conv aligned growth")
    cin, cout, h, w, splits = 16, 16, 9, 13, [2, 1, 3]
    x = synth.video(cin, sum(splits), h, w, synth.seed(0, 21))
    wt = synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(0, 22))
    ref = O.one_shot(to_oracle(x), to_oracle(wt), None, O.REPLICATE, 2, 2, aligned=True)
    plan = P.conv_plan(wt.cuda(), h, w, up_s=2, up_t=2, max_chunk_t=3, aligned=True)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    assert_fp32_close(got, ref, "fp32 aligned growth")


@pytest.mark.parametrize("k,up_s", [((3, 1, 1), 1), ((3, 3, 3), 2)])
def test_bf16_conv_aligned_growth(k, up_s):
    """CC3D_GROW_ALIGNED: the first chunk doubles every frame at up_t = 2
    (2T frames out of T), later chunks as usual."""
    say("bf16 conv aligned growth k=%s up_s=%d" % (k, up_s))
    cin, cout, h, w, splits = 32, 32, 6, 13, [3, 1, 2]
    x = synth.bf16(synth.video(cin, sum(splits), h, w, synth.seed(5, 11)))
    wt = synth.bf16(synth.conv_weight(cout, cin, *k, synth.seed(5, 12)))
    ref = O.one_shot(to_oracle(x), to_oracle(wt), None, O.REPLICATE, up_s, 2, aligned=True)
    plan = P.conv_plan(wt.cuda(), h, w, up_s=up_s, up_t=2, max_chunk_t=3, aligned=True)
    assert plan.output_shape(3, True)[0] == 6
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    assert got.shape[1] == 2 * sum(splits)
    assert_bf16_close(got, ref, "aligned growth")


@pytest.mark.parametrize("cout", [96, 192])
@pytest.mark.parametrize("residual", [False, True])
def test_bf16_conv_epilogue_act(cout, residual):
    """v = conv + bias (+ residual), stored as bf16, then SiLU(RMSNorm(v)):
    fused in the conv (96) or by the norm pass (192)."""
    say("bf16 epilogue cout=%d residual=%s" % (cout, residual))
    cin, h, w, splits = 32, 9, 20, [1, 2]
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(6, 1)))
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(6, 2)))
    b = synth.bias(cout, synth.seed(6, 3))
    g = synth.gain(cout, synth.seed(6, 4))
    r = synth.bf16(synth.video(cout, t, h, w, synth.seed(6, 5))) if residual else None
    v = O.causal_conv3d(to_oracle(x), to_oracle(wt), to_oracle(b), O.REPLICATE)
    if residual:
        v = v + to_oracle(r)
    ref = O.act(O.round_bf16(v), to_oracle(g), 1e-6)
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), gamma=g.cuda(), act=True, residual=residual,
                       max_chunk_t=2)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits,
                                     residual_cl=to_device_cl(r) if residual else None))
    assert_bf16_close(got, ref, "epilogue")


WHOLE_TILE_CASES = [
    # cin, cout, up_s, h, w, residual, act, kernel that must run: frames that
    # the register-blocked kernel's tiles cover exactly (9x64 / 8x64 output
    # tiles; 12x16 / 8x16 source tiles when upsampling), so its epilogue runs
    # without bounds tests
    (96, 96, 1, 18, 64, True, True, "conv_bf16_v2_up1_k3_n96"),
    (64, 96, 1, 9, 128, False, True, "conv_bf16_v2_up1_k3_n96"),
    (96, 128, 1, 16, 64, True, False, "conv_bf16_v2_up1_k3_n128"),
    (96, 192, 1, 9, 64, True, True, "conv_bf16_v2_up1_k3_n96"),
    (96, 96, 2, 12, 32, True, True, "conv_bf16_v2_up2_k3_n96"),
    (64, 128, 2, 8, 16, False, False, "conv_bf16_v2_up2_k3_n128"),
]


@pytest.mark.parametrize("case", WHOLE_TILE_CASES, ids=lambda c: "ci%d_co%d_us%d_%dx%d_r%d_a%d" % c[:7])
def test_bf16_conv_whole_tiles(case):
    """The register-blocked conv on frames its tiles cover exactly (the
    epilogue form without per-fragment bounds tests): v = conv + bias
    (+ residual) stored as bf16, and SiLU(RMSNorm(v)) where asked, against the
    oracle; the act is fused in the conv up to 96 channels, else the norm pass."""
    cin, cout, up_s, h, w, residual, act, kname = case
    say("bf16 whole tiles %s" % (case,))
    splits = [1, 2]
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(30, cin + cout)))
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(30, 2)))
    b = synth.bias(cout, synth.seed(30, 3))
    g = synth.gain(cout, synth.seed(30, 4))
    ho, wo = up_s * h, up_s * w
    r = synth.bf16(synth.video(cout, t, ho, wo, synth.seed(30, 5))) if residual else None
    v = O.one_shot(to_oracle(x), to_oracle(wt), to_oracle(b), O.REPLICATE, up_s, 1)
    if residual:
        v = v + to_oracle(r)
    ref = O.act(O.round_bf16(v), to_oracle(g), 1e-6) if act else v
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), gamma=g.cuda() if act else None, act=act,
                       residual=residual, up_s=up_s, max_chunk_t=2)
    C.check(C.lib().cc3d_profile_enable(plan._h, 1), "profile_enable")
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits,
                                     residual_cl=to_device_cl(r) if residual else None))
    pr = C.OpProfile()
    C.check(C.lib().cc3d_profile_read(plan._h, 0, 0, ctypes.byref(pr)), "profile_read")
    assert pr.kernel.decode().startswith(kname), pr.kernel
    assert_bf16_close(got, ref, "whole tiles")


RESIDUAL_ROW_CASES = [
    # cin, cout, h, w, splits, act: the register-blocked conv (no upsampling)
    # with a residual, at odd and even K-step counts (cin 32: 3 steps; 64: 6),
    # on the small-frame 5-row tiles and the 9-/8-row ones, with ragged bottom
    # and right tiles, several and eight channel blocks, and a cout that is not
    # a multiple of 8.
    (32, 96, 130, 400, [3, 1], True),
    (64, 192, 70, 300, [2, 1], False),
    (32, 256, 66, 260, [2, 2], False),
    (64, 128, 13, 70, [1, 2], False),
    (32, 100, 30, 90, [1, 2], False),
    (32, 768, 9, 20, [1, 2], False),
]


@pytest.mark.parametrize("case", RESIDUAL_ROW_CASES, ids=lambda c: "ci%d_co%d_%dx%d" % c[:4])
def test_bf16_conv_residual_rows(case):
    """v = conv + bias + residual (and SiLU(RMSNorm(v)) where asked) from the
    register-blocked kernel, against the oracle."""
    cin, cout, h, w, splits, act = case
    say("bf16 residual rows %s" % (case,))
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(31, cin + cout)))
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(31, 2)))
    b = synth.bias(cout, synth.seed(31, 3))
    g = synth.gain(cout, synth.seed(31, 4))
    r = synth.bf16(synth.video(cout, t, h, w, synth.seed(31, 5)))
    v = O.causal_conv3d(to_oracle(x), to_oracle(wt), to_oracle(b), O.REPLICATE) + to_oracle(r)
    ref = O.act(O.round_bf16(v), to_oracle(g), 1e-6) if act else v
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), gamma=g.cuda() if act else None, act=act,
                       residual=True, max_chunk_t=max(splits))
    C.check(C.lib().cc3d_profile_enable(plan._h, 1), "profile_enable")
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits, residual_cl=to_device_cl(r)))
    pr = C.OpProfile()
    C.check(C.lib().cc3d_profile_read(plan._h, 0, 0, ctypes.byref(pr)), "profile_read")
    assert pr.kernel.decode().startswith("conv_bf16_v2_up1_k3"), pr.kernel
    assert_bf16_close(got, ref, "residual rows")


@pytest.mark.parametrize("c", [16, 24, 32, 64, 96, 128, 192, 256, 320, 384, 512])
def test_norm_act_pass_lane_layouts(c):
    """The standalone norm pass (NORM_ACT ops) in every layout it picks for c
    channels (lanes per pixel x 16-byte chunks per lane; 16 and 24 channels fit
    none and take the element-wise kernel): act = SiLU(RMSNorm(x)),
    then v = act + x stored (bitwise: the sum of two bf16 values rounded once)
    and SiLU(RMSNorm(v))."""
    say("norm pass c=%d" % c)
    t, h, w = 3, 5, 7
    x = synth.bf16(synth.video(c, t, h, w, synth.seed(16, c)))
    g = synth.gain(c, synth.seed(16, c + 1))
    s_a, s_v = C.SLOT_AUX + 1, C.SLOT_AUX + 2  # internal slots
    ops = [P.Op(kind=C.OP_NORM_ACT, src=C.SLOT_X, act_out=s_a, gamma=g.cuda(), name="n1"),
           P.Op(kind=C.OP_NORM_ACT, src=s_a, res=C.SLOT_X, out=s_v, act_out=C.SLOT_Y, gamma=g.cuda(), name="n2")]
    plan = P.stack_plan(ops, c, h, w, max_chunk_t=t)
    st = P.Stream(plan)
    y = st.step(to_device_cl(x))
    torch.cuda.synchronize()
    a1 = from_device_cl(plan.read_slot(s_a, t, True))
    v2 = from_device_cl(plan.read_slot(s_v, t, True))
    assert_bf16_close(a1, O.act(to_oracle(x), to_oracle(g), 1e-6), "act")
    assert np.array_equal(v2, O.round_bf16(a1 + to_oracle(x))), "stored v = bf16(act + x)"
    assert_bf16_close(from_device_cl(y), O.act(v2, to_oracle(g), 1e-6), "act of v")


def test_bf16_head_conv_residual():
    """The output head (3 channels, nearest 2x) with bias and a residual added
    before the bf16 store."""
    say("bf16 head residual")
    cin, cout, h, w, splits = 96, 3, 11, 21, [1, 3]
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(6, 11)))
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(6, 12)))
    b = synth.bias(cout, synth.seed(6, 13))
    r = synth.bf16(synth.video(cout, t, 2 * h, 2 * w, synth.seed(6, 14)))
    ref = O.one_shot(to_oracle(x), to_oracle(wt), to_oracle(b), O.REPLICATE, up_s=2) + to_oracle(r)
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), up_s=2, residual=True, max_chunk_t=3)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits, residual_cl=to_device_cl(r)))
    assert_bf16_close(got, ref, "head + residual")


# ------------------------------------------------------------- boundary --

def _small_plan():
    cin, cout, h, w = 32, 32, 10, 18
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(7, 2))).cuda()
    return P.conv_plan(wt, h, w, max_chunk_t=4), (cin, h, w)


def test_reset_pingpong_checkpoint_and_determinism():
    say("boundary: reset / ping-pong / checkpoint")
    plan, (cin, h, w) = _small_plan()
    x = to_device_cl(synth.bf16(synth.video(cin, 10, h, w, synth.seed(7, 1))))
    splits = [1, 4, 3, 2]
    a = _run_chunks(plan, x, splits)
    b = _run_chunks(plan, x, splits)
    assert torch.equal(a, b), "replay is not bitwise identical"
    # reset mid-stream == fresh stream
    st = P.Stream(plan)
    st.step(x[:3].contiguous())
    st.reset()
    c = torch.cat([st.step(x[i:i + n].contiguous()) for i, n in zip([0, 1, 5, 8], splits)])
    assert torch.equal(a, c)
    # checkpoint after two chunks, resume in a new stream
    st = P.Stream(plan)
    st.step(x[:1].contiguous())
    st.step(x[1:5].contiguous())
    saved = plan.new_state().copy_(st.states[st.cur])
    tail_a = st.step(x[5:8].contiguous())
    st2 = P.Stream(plan)
    st2.states[0].copy_(saved)
    st2.cur = 0
    tail_b = st2.step(x[5:8].contiguous())
    assert torch.equal(tail_a, tail_b)
    torch.cuda.synchronize()


def test_cache_in_untouched_and_aliasing_rejected():
    say("boundary: cache_in untouched, aliasing")
    plan, (cin, h, w) = _small_plan()
    x = to_device_cl(synth.bf16(synth.video(cin, 3, h, w, synth.seed(7, 3))))
    s0, s1 = plan.new_state(), plan.new_state()
    plan.reset(s0)
    plan.reset(s1)
    plan.forward_chunk(x[:1].contiguous(), s0, s1)
    before = s1.arena.clone()
    s2 = plan.new_state()
    plan.forward_chunk(x[1:3].contiguous(), s1, s2)
    torch.cuda.synchronize()
    assert torch.equal(before, s1.arena)
    assert s2.frames_seen == 3
    with pytest.raises(C.Cc3dError) as e:
        plan.forward_chunk(x[:1].contiguous(), s1, s1)
    assert e.value.status == C.ESTATE
    with pytest.raises(C.Cc3dError) as e:
        plan.forward_chunk(torch.empty((5, h, w, cin), dtype=torch.bfloat16, device="cuda"), s1, s2)
    assert e.value.status == C.ESHAPE
    # an empty chunk is refused
    with pytest.raises(C.Cc3dError) as e:
        plan.forward_chunk(x[:0].contiguous(), s1, s2)
    assert e.value.status == C.ESHAPE
    # host memory is refused
    with pytest.raises(ValueError):
        plan.forward_chunk(x[:1].cpu().contiguous(), s1, s2)


def test_misaligned_chunk_rejected_state_unchanged():
    """A chunk pointer off 16-byte alignment (31 fp32 channels: a 3x26 frame is
    9672 bytes, so the slice from frame 1 starts 8 bytes off) is refused with
    EINVAL before anything runs; the stream then continues from the same state
    and matches the definition."""
    say("boundary: misaligned chunk")
    cin, cout, h, w = 31, 5, 3, 26
    x = synth.video(cin, 4, h, w, synth.seed(7, 21))
    wt = synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(7, 22))
    ref = O.causal_conv3d(to_oracle(x), to_oracle(wt), None, O.REPLICATE)
    plan = P.conv_plan(wt.cuda(), h, w, max_chunk_t=3)
    x_cl = to_device_cl(x)
    st = P.Stream(plan)
    y0 = st.step(x_cl[:1].clone())
    bad = x_cl[1:4]
    assert bad.data_ptr() % 16 == 8
    with pytest.raises(C.Cc3dError) as e:
        st.step(bad)
    assert e.value.status == C.EINVAL and "16-byte" in str(e.value)
    assert st.frames_seen == 1
    y1 = st.step(bad.clone())
    torch.cuda.synchronize()
    assert_fp32_close(from_device_cl(torch.cat([y0, y1])), ref, "after a refused chunk")


def test_binding_refuses_mismatched_tensors():
    """x of another frame size, channel count or dtype, and a residual of another
    shape or dtype (or a missing one), are refused by the binding before the
    library is called; the state is unchanged, and a y larger than the chunk's
    output comes back viewed as the output shape."""
    say("boundary: mismatched tensors refused by the binding")
    c, h, w = 16, 5, 7
    wt = synth.bf16(synth.conv_weight(c, c, 3, 3, 3, synth.seed(8, 5)))
    plan = P.conv_plan(wt.cuda(), h, w, residual=True, max_chunk_t=2)
    st = P.Stream(plan)
    x = synth.bf16(synth.video(c, 2, h, w, synth.seed(8, 6)))
    x_cl = to_device_cl(x)
    res = torch.zeros(plan.output_shape(2, True), dtype=torch.bfloat16, device="cuda")
    for bad in (x_cl.float(), x_cl[:, :4].contiguous(), x_cl[..., :8].contiguous()):
        with pytest.raises(ValueError, match="x must be"):
            st.step(bad, residual=res)
    for bad in (None, res[:1].contiguous(), res.float()):
        with pytest.raises(ValueError, match="residual"):
            st.step(x_cl, residual=bad)
    assert st.frames_seen == 0
    y_big = torch.empty(res.numel() + 64, dtype=torch.bfloat16, device="cuda")
    y = st.step(x_cl, residual=res, y=y_big)
    torch.cuda.synchronize()
    assert tuple(y.shape) == plan.output_shape(2, True) and y.data_ptr() == y_big.data_ptr()
    ref = O.chunked(to_oracle(x), to_oracle(wt), None, O.REPLICATE, splits=[2])
    assert_bf16_close(from_device_cl(y), ref, "after refused calls")


def test_transposes_roundtrip():
    say("transposes")
    for dt in (torch.bfloat16, torch.float32):
        x = synth.video(5, 3, 7, 33, synth.seed(8, 1)).to(dt).cuda()
        cl = P.to_channels_last(x)
        assert torch.equal(cl, x.permute(1, 2, 3, 0).contiguous())
        assert torch.equal(P.to_channels_first(cl), x)


# ----------------------------------------------------------------- stacks --

def _params(shapes, cfg, gain_for, with_bias=False):
    """Seeded bf16 weights / fp32 gains and biases for (name, cout, cin, kt, kh, kw),
    as float64 numpy for the oracle and as device tensors for the library."""
    cpu, dev = {}, {}
    for name, p in synth.layer_weights(shapes, cfg, gain_for, with_bias).items():
        cpu[name] = {k: None if v is None else to_oracle(v) for k, v in p.items()}
        dev[name] = {k: None if v is None else v.cuda() for k, v in p.items()}
    return cpu, dev


def test_c1_resblock_small():
    say("c1 resblock small")
    c, t, h, w = 32, 8, 12, 20
    cpu, dev = _params([("c1", c, c, 3, 3, 3), ("c2", c, c, 3, 3, 3)], 1, lambda n: True, with_bias=True)
    x = synth.bf16(synth.video(c, t, h, w, synth.seed(1, 1)))
    ref_blk = OM.ResBlock(cpu["c1"], cpu["c2"], store=O.round_bf16)
    ref = np.concatenate([ref_blk.step(to_oracle(x)[:, i:i + 4]) for i in range(0, t, 4)], axis=1)
    plan = P.stack_plan(S.resblock_ops(c, dev["c1"], dev["c2"]), c, h, w, max_chunk_t=4)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), [4, 4]))
    assert_bf16_close(got, ref, "c1 block")


@pytest.mark.parametrize("cfg,cin,cmid,cout", [(2, 64, 32, 32), (3, 32, 96, 3)])
def test_upstage_small(cfg, cin, cmid, cout):
    say("upstage small cfg=%d" % cfg)
    t, h, w = 6, 7, 19
    cpu, dev = _params([("c1", cmid, cin, 3, 3, 3), ("c2", cout, cmid, 3, 3, 3)], cfg, lambda n: n == "c2")
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(cfg, 1)))
    ref_st = OM.UpStage(cpu["c1"], cpu["c2"], store=O.round_bf16)
    splits = [1, 4, 1] if cfg == 3 else [2, 4]
    ref, t0 = [], 0
    for n in splits:
        ref.append(ref_st.step(to_oracle(x)[:, t0:t0 + n]))
        t0 += n
    ref = np.concatenate(ref, axis=1)
    plan = P.stack_plan(S.upstage_ops(cmid, cout, dev["c1"], dev["c2"]), cin, h, w, max_chunk_t=4)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    assert_bf16_close(got, ref, "upstage")


def _decoder_layerwise(c_latent, stages, t, h, w, splits, cfg=4, temporal_grow=None, aligned=False,
                       keep_slots=False, fold_upsample=False):
    """Run the decoder twice on the GPU -- production slot wiring and the
    unique-slot wiring -- and check (1) both give bitwise identical outputs,
    (2) every layer of the unique-slot run against the oracle fed that layer's
    own GPU input (the per-layer parity bound), (3) the whole stack against the
    storage-rounded oracle run end to end (the stack bound).  ``keep_slots``:
    also return every op's output tensors per chunk (op name -> list)."""
    full = OM.decoder_layer_shapes(c_latent=c_latent, stages=stages, temporal_grow=temporal_grow)
    gains = {s_[0]: s_[6] for s_ in full}
    cpu, dev = _params([s_[:6] for s_ in full], cfg, lambda n: gains[n])
    x = synth.bf16(synth.video(c_latent, t, h, w, synth.seed(cfg, 1)))
    x_cl = to_device_cl(x)
    ops_u = S.decoder_ops(dev, stages=stages, unique_slots=True, temporal_grow=temporal_grow)
    plan_u = P.stack_plan(ops_u, c_latent, h, w, max_chunk_t=max(splits), aligned=aligned,
                          fold_upsample=fold_upsample)
    plan_p = P.stack_plan(S.decoder_ops(dev, stages=stages, temporal_grow=temporal_grow), c_latent, h, w,
                          max_chunk_t=max(splits), aligned=aligned, fold_upsample=fold_upsample)
    su, sp = P.Stream(plan_u), P.Stream(plan_p)
    layer = {i: O.CausalConvStream(cpu[o.name]["w"], cpu[o.name]["b"], O.REPLICATE, o.up_s, o.up_t,
                                   aligned=aligned)
             for i, o in enumerate(ops_u)}
    outs, t0, worst = [], 0, {}
    kept = {}
    for n in splits:
        first = su.frames_seen == 0
        xc = x_cl[t0:t0 + n].contiguous()
        yu, yp = su.step(xc), sp.step(xc)
        torch.cuda.synchronize()
        assert torch.equal(yu, yp), "production wiring differs from the unique-slot wiring"
        outs.append(yu)
        ten = {C.SLOT_X: xc, C.SLOT_Y: yu}
        for o in ops_u:
            for sl in (o.out, o.act_out):
                if sl > C.SLOT_AUX:
                    ten[sl] = plan_u.read_slot(sl, n, first)
        torch.cuda.synchronize()
        if keep_slots:
            for o in ops_u:
                if o.out != C.SLOT_NONE:
                    kept.setdefault(o.name, []).append(ten[o.out])
        for i, o in enumerate(ops_u):
            v = layer[i].step(from_device_cl(ten[o.src]))
            if o.res != C.SLOT_NONE:
                v = v + from_device_cl(ten[o.res])
            if o.out != C.SLOT_NONE:
                mx, mn = assert_bf16_close(from_device_cl(ten[o.out]), v, "%s out (chunk at %d)" % (o.name, t0))
                worst[o.name] = max(worst.get(o.name, 0.0), mn)
            if o.act_out != C.SLOT_NONE:
                ref_act = O.act(O.round_bf16(v), cpu_gain(cpu, ops_u, o), 1e-6)
                assert_bf16_close(from_device_cl(ten[o.act_out]), ref_act, "%s act (chunk at %d)" % (o.name, t0))
        t0 += n
    got = from_device_cl(torch.cat(outs, dim=0))
    dec = OM.Decoder(cpu, stages=stages, store=O.round_bf16, temporal_grow=temporal_grow, aligned=aligned)
    ref, t0 = [], 0
    for n in splits:
        ref.append(dec.step(to_oracle(x)[:, t0:t0 + n]))
        t0 += n
    ref = np.concatenate(ref, axis=1)
    if keep_slots:
        return got, ref, worst, kept
    return got, ref, worst


def _decoder_case(name, **kw):
    """_decoder_layerwise on a named whole-decoder configuration of stack_cases."""
    c = SC.STACK_CASES[name]
    return _decoder_layerwise(c["c_lat"], c["stages"], t=c["t"], h=c["h"], w=c["w"], splits=list(c["splits"]),
                              cfg=c["cfg"], temporal_grow=c["tg"], aligned=c["aligned"], **kw)


def cpu_gain(cpu, ops, o):
    """The oracle-side gain of the act an op stores: the RMSNorm gain of the conv
    that reads it (the next block's conv1, the block's conv2, or the head)."""
    for nxt in ops:
        if nxt.src == o.act_out:
            return cpu[nxt.name]["g"]
    raise AssertionError("no op reads %s's act" % o.name)


def test_decoder_small_channels():
    say("decoder small channels")
    got, ref, _ = _decoder_case("small")
    assert got.shape == (3, OM.output_frames(6), 48, 80)
    assert_stack_close(got, ref, "small", "decoder small")


@pytest.mark.parametrize("aligned,fold", [(False, False), (True, False), (False, True)])
def test_decoder_full_channels_tiny_frame(aligned, fold):
    """Full channel counts (the register-blocked kernels and the head), both
    first-chunk growth rules, and the phase-folded upsample convs."""
    say("decoder full channels tiny frame, aligned=%s fold=%s" % (aligned, fold))
    case = "full_tiny_aligned" if aligned else "full_tiny"
    got, ref, _ = _decoder_case(case, fold_upsample=fold)
    assert got.shape == (3, OM.output_frames(5, aligned=aligned), 32, 48)
    assert_stack_close(got, ref, case, "decoder full channels")


def test_decoder_cache_writes_fused_into_producers():
    """Where a conv's input is a slot an earlier op of the same pass writes (and
    the conv does not grow time), that op stores the conv's cache as it writes
    the slot and no copy kernel runs for it; convs that read x or grow time keep
    the copy.  The full-channel decoder in chunks of two latents (every slot has
    at least the k_t - 1 = 2 frames a cache holds), against the oracle too."""
    say("decoder: cache writes fused into the producers")
    c = SC.STACK_CASES["full_fused_cache"]
    c_lat, h, w, splits = c["c_lat"], c["h"], c["w"], list(c["splits"])
    assert splits == [2, 2] and c["stages"] == OM.DECODER_STAGES
    params = SC.weights(c)
    cpu = {n: {k: None if v is None else v.double().numpy() for k, v in p.items()} for n, p in params.items()}
    gpu = {n: {k: None if v is None else v.cuda() for k, v in p.items()} for n, p in params.items()}
    x = SC.latent(c)
    dec = OM.Decoder(cpu, store=O.round_bf16)
    xo = x.double().numpy()
    ref = np.concatenate([dec.step(xo[:, :2]), dec.step(xo[:, 2:4])], axis=1)
    ops = S.decoder_ops(gpu)
    plan = P.stack_plan(ops, c_lat, h, w, max_chunk_t=2)
    C.check(C.lib().cc3d_profile_enable(plan._h, 1), "profile_enable")
    st = P.Stream(plan)
    x_cl = to_device_cl(x)
    y = torch.cat([st.step(x_cl[:2].contiguous()), st.step(x_cl[2:4].contiguous())])
    torch.cuda.synchronize()
    fused = copied = 0
    for i, o in enumerate(ops):
        if o.kind != C.OP_CONV or o.k[0] < 2:
            continue
        pr = C.OpProfile()
        C.check(C.lib().cc3d_profile_read(plan._h, i, 2, ctypes.byref(pr)), "profile_read")
        if o.src == C.SLOT_X or o.up_t == 2:
            assert pr.launches == 2, "%s: expected the cache copy in both chunks, got %d" % (o.name, pr.launches)
            copied += 1
        else:
            assert pr.launches == 0, "%s: cache copied %d times, expected it stored by the producer" % (
                o.name, pr.launches)
            fused += 1
    assert fused >= 10 and copied >= 1, (fused, copied)
    assert_stack_close(from_device_cl(y), ref, "full_fused_cache", "fused cache writes")


@pytest.mark.parametrize("t_prime,aligned,fold", [(1, False, False), (3, False, False), (4, False, True),
                                                   (3, True, False), (2, True, True)])
def test_decoder_causality_bitwise(t_prime, aligned, fold):
    """Causality of the whole decoder on the GPU: changing latent t' leaves every
    output frame that latents 0 .. t'-1 alone produce (OM.output_frames(t'):
    4t'-3, or 4t' with the aligned rule) bitwise unchanged, in chunks that put
    t' on either side of a chunk boundary, and changes the next frame."""
    say("decoder causality t'=%d aligned=%s fold=%s" % (t_prime, aligned, fold))
    c_latent, t, h, w, splits = 48, 5, 2, 3, [3, 2]
    full = OM.decoder_layer_shapes(c_latent=c_latent)
    gains = {s_[0]: s_[6] for s_ in full}
    _, dev = _params([s_[:6] for s_ in full], 4, lambda n: gains[n])
    x = synth.bf16(synth.video(c_latent, t, h, w, synth.seed(4, 1)))
    x2 = x.clone()
    x2[:, t_prime] = synth.bf16(x2[:, t_prime].float() + 1.0)
    plan = P.stack_plan(S.decoder_ops(dev), c_latent, h, w, max_chunk_t=max(splits), aligned=aligned,
                        fold_upsample=fold)
    ys = []
    for xv in (x, x2):
        st, x_cl, t0, out = P.Stream(plan), to_device_cl(xv), 0, []
        for n in splits:
            out.append(st.step(x_cl[t0:t0 + n].contiguous()).clone())
            t0 += n
        torch.cuda.synchronize()
        ys.append(torch.cat(out))
    cut = OM.output_frames(t_prime, aligned=aligned)
    assert ys[0].shape[0] == OM.output_frames(t, aligned=aligned) > cut
    assert torch.equal(ys[0][:cut], ys[1][:cut]), "an output frame before %d changed" % cut
    assert not torch.equal(ys[0][cut], ys[1][cut]), "output frame %d did not see latent %d" % (cut, t_prime)


SMALL_STAGES = SC.SMALL_STAGES


@pytest.mark.parametrize("order", ["before", "after"])
def test_decoder_temporal_grow_layerwise(order):
    """TemporalGrow (1x1x1 projection, causal 3x1x1 temporal conv on the grown
    sequence) in either order: every layer against the oracle, the stack end to
    end."""
    say("decoder temporal grow %s" % order)
    got, ref, _ = _decoder_case("small_tg_" + order)
    assert got.shape == (3, OM.output_frames(6), 48, 80)
    assert_stack_close(got, ref, "small_tg_" + order, "decoder tg %s" % order)


@pytest.mark.parametrize("fold", [False, True])
def test_decoder_full_channels_one_latent_chunks(fold):
    """Every chunk one latent (the first grows to 1 frame, the rest to 4): each
    layer's window is mostly its cache, and the folded growing convs take their
    history grouping on every chunk."""
    say("decoder full channels, one-latent chunks, fold=%s" % fold)
    got, ref, _ = _decoder_case("full_one_latent", fold_upsample=fold)
    assert got.shape == (3, OM.output_frames(4), 32, 48)
    assert_stack_close(got, ref, "full_one_latent", "decoder one-latent chunks")


@pytest.mark.parametrize("idx", range(len(SC.RANDOM_CASES)), ids=lambda i: "%d_cl%d_%s_t%d_%dx%d_tg%s_al%d_f%d" % (
    (i, SC.RANDOM_CASES[i][0], "-".join("%dx%d" % s_ for s_ in SC.RANDOM_CASES[i][1])) + SC.RANDOM_CASES[i][2:5]
    + SC.RANDOM_CASES[i][6:]))
def test_decoder_random_configs(idx):
    """Every layer of randomly drawn decoder configurations against the oracle,
    the stack end to end, and the production slot wiring bitwise equal to the
    unique-slot one."""
    c_lat, stages, t, h, w, splits, tg, aligned, fold = SC.RANDOM_CASES[idx]
    say("decoder random config %s" % (SC.RANDOM_CASES[idx],))
    got, ref, _ = _decoder_case("random%d" % idx, fold_upsample=fold)
    up = 2 ** (len(stages) + 1)  # each stage and the head double the frame size
    assert got.shape == (3, OM.output_frames(t, [f for _, f in stages], aligned=aligned), h * up, w * up)
    assert_stack_close(got, ref, "random%d" % idx, "decoder random config")


def test_decoder_full_channels_two_clips():
    """The whole decoder end to end at reduced spatial size: latent 48 x 13 x
    4x6 in the benchmark's clips (7 then 6 latents) -> RGB 3 x 49 x 64x96, every
    layer against the oracle, the stack against the storage-rounded oracle."""
    say("decoder full channels, two clips 7+6 at 4x6")
    got, ref, _ = _decoder_case("full_two_clips")
    assert got.shape == (3, 49, 64, 96)
    assert_stack_close(got, ref, "full_two_clips", "decoder two clips")


def test_decoder_temporal_grow_full_channels_tiny_frame():
    say("decoder temporal grow, full channels, tiny frame")
    got, ref, _ = _decoder_case("full_tiny_tg_before")
    assert got.shape == (3, OM.output_frames(5), 32, 48)
    assert_stack_close(got, ref, "full_tiny_tg_before", "decoder tg full channels")


def test_temporal_grow_orders_bitwise():
    """The reorder: TemporalGrow at the stage input size, then nearest 2x, gives
    bit for bit the TemporalGrow output computed on the upsampled positions (the
    SwiftVR page reports bitwise identical results).  The decoders that follow
    read the same values; their spatial convs fold the upsample or not, so the
    RGB is held to the stack bound."""
    say("temporal grow: before vs after, bitwise")
    runs = {}
    for order in ("before", "after"):
        runs[order] = _decoder_layerwise(16, SMALL_STAGES, t=5, h=3, w=5, splits=[3, 2], temporal_grow=order,
                                         keep_slots=True)
        assert_stack_close(runs[order][0], runs[order][1], "small_t5_tg_before", "decoder tg %s" % order)
    kb, ka = runs["before"][3], runs["after"][3]
    for si in range(len(SMALL_STAGES)):
        name = "s%d.tg.t" % si
        for lo, hi in zip(kb[name], ka[name]):
            up = lo.repeat_interleave(2, dim=1).repeat_interleave(2, dim=2)
            assert up.shape == hi.shape
            assert torch.equal(up, hi), "%s: TemporalGrow output differs between the orders" % name
    # two GPU decodes whose fp32 sums differ in order: the drift of one rounded
    # pipeline from another, the quantity the case's bound is measured from
    mx, mn = assert_stack_close(runs["before"][0], runs["after"][0], "small_t5_tg_before", "rgb before vs after")
    say("  rgb before vs after: max-rel %.3g mean-rel %.3g, bitwise %s" % (
        mx, mn, np.array_equal(runs["before"][0], runs["after"][0])))


@pytest.mark.parametrize("temporal_grow", [None, "before"])
def test_decoder_aligned_first_chunk(temporal_grow):
    """Aligned growth (the 28-frame first chunk): layer-wise against the
    oracle's aligned rule, and after dropping the first chunk's first 3 frames
    the same video as the default rule, to the stack bound."""
    say("decoder aligned first chunk, temporal_grow=%s" % temporal_grow)
    case = "small_t5_tg_before" if temporal_grow else "small_t5"
    got, ref, _ = _decoder_case(case + "_aligned")
    assert got.shape[1] == OM.output_frames(5, aligned=True) == OM.output_frames(5) + 3
    assert_stack_close(got, ref, case + "_aligned", "aligned decoder")
    once, ref_once, _ = _decoder_case(case)
    assert_stack_close(once, ref_once, case, "default rule")
    # the oracle's aligned decode minus 3 frames is exactly its default decode;
    # the two GPU decodes differ in rounding order only
    assert np.array_equal(ref[:, 3:], ref_once)
    assert_stack_close(got[:, 3:], once, case, "aligned minus 3 frames vs default rule")


def _op_index(ops, name):
    return next(i for i, o in enumerate(ops) if o.name == name)


@pytest.mark.parametrize("temporal_grow,group,fb,aligned,out_u8", [
    (None, "s2.up", 1, False, False),        # the last stage + head, one frame at a time
    (None, "s2.up", 2, False, True),         # ... writing 8-bit RGB
    (None, "s2.up", 3, False, False),        # batches that do not divide the chunk
    ("before", "s1.tg.p", 2, False, False),  # time grows inside the group
    ("before", "s1.tg.p", 1, True, False),   # ... with the aligned first chunk
    (None, "conv_in", 2, False, False),      # the whole stack (the group reads x)
])
def test_decoder_frame_batching_bitwise(temporal_grow, group, fb, aligned, out_u8):
    """Frame batching: the group of ops from `group` on runs over batches of
    `fb` frames of its input with its caches carried from batch to batch; the
    output equals the whole-chunk run bit for bit, with less plan memory."""
    say("frame batching tg=%s group=%s fb=%d aligned=%s u8=%s" % (temporal_grow, group, fb, aligned, out_u8))
    full = OM.decoder_layer_shapes(c_latent=16, stages=SMALL_STAGES, temporal_grow=temporal_grow)
    gains = {s_[0]: s_[6] for s_ in full}
    _, dev = _params([s_[:6] for s_ in full], 4, lambda n: gains[n])
    ops = S.decoder_ops(dev, stages=SMALL_STAGES, temporal_grow=temporal_grow, out_u8=out_u8)
    h, w, splits = 3, 5, [3, 2]
    x = synth.bf16(synth.video(16, sum(splits), h, w, synth.seed(4, 1)))
    x_cl = to_device_cl(x)
    plan_w = P.stack_plan(ops, 16, h, w, max_chunk_t=3, aligned=aligned)
    plan_b = P.stack_plan(ops, 16, h, w, max_chunk_t=3, aligned=aligned, batch_from=_op_index(ops, group),
                          frame_batch=fb)
    sw, sb = P.Stream(plan_w), P.Stream(plan_b)
    t0 = 0
    for n in splits:
        xc = x_cl[t0:t0 + n].contiguous()
        yw, yb = sw.step(xc), sb.step(xc)
        torch.cuda.synchronize()
        assert yw.shape == yb.shape
        assert torch.equal(yw, yb), "chunk at %d: frame-batched output differs" % t0
        t0 += n
    assert plan_b.device_bytes < plan_w.device_bytes
    say("  plan device bytes %d -> %d" % (plan_w.device_bytes, plan_b.device_bytes))


@pytest.mark.parametrize("group,fb,aligned", [("s0.up", 1, False), ("s0.up", 2, True), ("conv_in", 3, False)])
def test_decoder_frame_batching_folded_bitwise(group, fb, aligned):
    """Frame batching with phase-folded upsample convs, the two that double time
    inside the group: a batch reads from the cache the frames a whole-chunk run
    reads from the input, and groups their temporal taps alike (by source frame),
    so the output still equals the whole-chunk run bit for bit."""
    say("frame batching, folded: group=%s fb=%d aligned=%s" % (group, fb, aligned))
    full = OM.decoder_layer_shapes(c_latent=48)
    gains = {s_[0]: s_[6] for s_ in full}
    _, dev = _params([s_[:6] for s_ in full], 4, lambda n: gains[n])
    ops = S.decoder_ops(dev)
    h, w, splits = 2, 3, [3, 2, 1]
    x_cl = to_device_cl(synth.bf16(synth.video(48, sum(splits), h, w, synth.seed(4, 1))))
    plan_w = P.stack_plan(ops, 48, h, w, max_chunk_t=3, aligned=aligned, fold_upsample=True)
    plan_b = P.stack_plan(ops, 48, h, w, max_chunk_t=3, aligned=aligned, fold_upsample=True,
                          batch_from=_op_index(ops, group), frame_batch=fb)
    sw, sb = P.Stream(plan_w), P.Stream(plan_b)
    t0 = 0
    for n in splits:
        xc = x_cl[t0:t0 + n].contiguous()
        yw, yb = sw.step(xc), sb.step(xc)
        torch.cuda.synchronize()
        assert torch.equal(yw, yb), "chunk at %d: frame-batched folded output differs" % t0
        t0 += n


@pytest.mark.parametrize("tpad", [C.TPAD_ZERO, C.TPAD_REPLICATE])
def test_folded_growing_conv_batched_history(tpad):
    """A phase-folded conv that doubles time, alone in a frame-batched group: a
    one-frame first chunk leaves a history of two different frames under zero
    padding (the zero frame and the first input frame) and two copies of one
    frame under replication; batches of one frame then read every history from
    the cache.  Batched equals whole chunks bit for bit, and both match the
    definition."""
    say("folded growing conv, batched history, tpad=%d" % tpad)
    c, h, w, splits = 96, 5, 9, [1, 1, 3, 2]
    x = synth.bf16(synth.video(c, sum(splits), h, w, synth.seed(13, 31)))
    wt = synth.bf16(synth.conv_weight(c, c, 3, 3, 3, synth.seed(13, 32)))
    ref = O.one_shot(to_oracle(x), to_oracle(wt), None, TP[tpad], 2, 2)
    ops = [P.Op(cout=c, w=wt.cuda(), up_s=2, up_t=2, tpad=tpad, src=C.SLOT_X, out=C.SLOT_Y, name="up")]
    plan_w = P.stack_plan(ops, c, h, w, max_chunk_t=3, fold_upsample=True)
    plan_b = P.stack_plan(ops, c, h, w, max_chunk_t=3, fold_upsample=True, batch_from=0, frame_batch=1)
    sw, sb = P.Stream(plan_w), P.Stream(plan_b)
    x_cl, t0, outs = to_device_cl(x), 0, []
    for n in splits:
        xc = x_cl[t0:t0 + n].contiguous()
        yw, yb = sw.step(xc), sb.step(xc)
        torch.cuda.synchronize()
        assert torch.equal(yw, yb), "chunk at %d: frame-batched output differs" % t0
        outs.append(yw.clone())
        t0 += n
    assert_bf16_close(from_device_cl(torch.cat(outs)), ref, "folded growing conv")


def test_conv_family_override_keeps_v1(monkeypatch):
    """CC3D_CONV_FAMILY=1 at plan creation keeps a conv the register-blocked
    kernel would take on the generic kernel: the profiled kernel name says so
    and its result matches the oracle."""
    say("family override: 96-channel 3x3x3 conv on the generic kernel")
    cin, cout, h, w, splits = 96, 96, 11, 70, [2, 1]
    x = synth.bf16(synth.video(cin, sum(splits), h, w, synth.seed(5, 31)))
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(5, 32)))
    ref = O.one_shot(to_oracle(x), to_oracle(wt), None, O.REPLICATE)
    names = {}
    for fam in (None, "1"):
        if fam:
            monkeypatch.setenv("CC3D_CONV_FAMILY", fam)
        plan = P.conv_plan(wt.cuda(), h, w, max_chunk_t=2)
        monkeypatch.delenv("CC3D_CONV_FAMILY", raising=False)
        C.check(C.lib().cc3d_profile_enable(plan._h, 1), "profile_enable")
        got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
        pr = C.OpProfile()
        C.check(C.lib().cc3d_profile_read(plan._h, 0, 0, ctypes.byref(pr)), "profile_read")
        names[fam] = pr.kernel.decode()
        assert_bf16_close(got, ref, "family %s" % fam)
    assert names[None] == "conv_bf16_v2_up1_k3_n96" and names["1"] == "conv_bf16_up1_k3_n96", names


@pytest.mark.parametrize("kind", ["resblock", "growing_folded", "strided"])
def test_graph_capture_replays_chunks(kind):
    """CDA-VSR page, "CUDA Graph inference": a chunk decode captured into a graph
    (fixed shapes, the two state arenas used alternately, no allocation, no host
    synchronisation) replays the eager decode bit for bit.  The first chunk runs
    eagerly (its first-chunk rule is fixed when a launch is recorded); two graphs
    (state A -> B and B -> A) are then replayed in turn, with eager copies and a
    synchronisation between replays, and every replay is checked.  Stacks: a
    residual block, a phase-folded conv that doubles space and time, and a conv
    that halves them (strides, every output from two new frames)."""
    say("graph capture of forward_chunk: %s" % kind)
    c, h, w, n, nch = 96, 10, 40, 4, 7
    if kind == "resblock":
        cpu, dev = _params([("c1", c, c, 3, 3, 3), ("c2", c, c, 3, 3, 3)], 12, lambda n_: True, with_bias=True)
        plan = P.stack_plan(S.resblock_ops(c, dev["c1"], dev["c2"]), c, h, w, max_chunk_t=n)
    elif kind == "strided":
        wt = synth.bf16(synth.conv_weight(c, c, 3, 3, 3, synth.seed(12, 8))).cuda()
        ops = [P.Op(cout=c, w=wt, stride_s=2, stride_t=2, src=C.SLOT_X, out=C.SLOT_Y, name="down")]
        plan = P.stack_plan(ops, c, h, w, max_chunk_t=n, aligned=True)
    else:
        wt = synth.bf16(synth.conv_weight(c, c, 3, 3, 3, synth.seed(12, 7))).cuda()
        ops = [P.Op(cout=c, w=wt, up_s=2, up_t=2, src=C.SLOT_X, out=C.SLOT_Y, name="up")]
        plan = P.stack_plan(ops, c, h, w, max_chunk_t=n, fold_upsample=True)
    x = to_device_cl(synth.bf16(synth.video(c, n * nch, h, w, synth.seed(12, 1))))
    chunks = [x[i * n:(i + 1) * n].contiguous() for i in range(nch)]
    eager = _run_chunks(plan, x, [n] * nch)
    t1, t_rest = plan.output_shape(n, True)[0], plan.output_shape(n, False)[0]
    st = P.Stream(plan)
    x_s = torch.empty_like(chunks[0])
    y_1 = torch.empty((t1,) + tuple(eager.shape[1:]), dtype=torch.bfloat16, device="cuda")
    y_s = torch.empty((t_rest,) + tuple(eager.shape[1:]), dtype=torch.bfloat16, device="cuda")
    x_s.copy_(chunks[0])
    st.step(x_s, y=y_1)
    torch.cuda.synchronize()
    assert torch.equal(y_1, eager[:t1])
    a, b = st.states[st.cur], st.states[1 - st.cur]
    graphs = []
    for cin_, cout_ in ((a, b), (b, a)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.forward_chunk(x_s, cin_, cout_, y=y_s)
        graphs.append(g)
    for i in range(1, nch):
        x_s.copy_(chunks[i])
        graphs[(i - 1) % 2].replay()
        torch.cuda.synchronize()
        f0 = t1 + (i - 1) * t_rest
        assert torch.equal(y_s, eager[f0:f0 + t_rest]), "replay %d differs from the eager decode" % i


def test_plan_create_failure_releases_everything(monkeypatch):
    """Failing allocation k of plan creation (k = 1, 2, ... until creation needs
    fewer) returns ENOMEM and leaves no plan and no device memory behind."""
    say("boundary: injected allocation failure")
    c, h, w = 32, 24, 40
    ps = {n: {"w": synth.bf16(synth.conv_weight(c, c, 3, 3, 3, synth.seed(7, 20 + i))).cuda(),
              "g": synth.gain(c, synth.seed(7, 30 + i)).cuda(), "b": synth.bias(c, synth.seed(7, 40 + i)).cuda()}
          for i, n in enumerate(("c1", "c2"))}
    ops = S.resblock_ops(c, ps["c1"], ps["c2"])
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    failures = 0
    for k in range(1, 32):
        monkeypatch.setenv("CC3D_TEST_FAIL_ALLOC", str(k))
        try:
            plan = P.stack_plan(ops, c, h, w, max_chunk_t=4)
        except C.Cc3dError as e:
            assert e.status == C.ENOMEM
            failures += 1
            continue
        del plan  # creation needed fewer than k allocations
        break
    assert failures >= 5  # slots, packed weights, biases, gains
    monkeypatch.delenv("CC3D_TEST_FAIL_ALLOC")
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] >= free0 - (2 << 20)
    plan = P.stack_plan(ops, c, h, w, max_chunk_t=4)  # and creation still works
    assert plan.state_bytes > 0


# ------------------------------------------------------------ 8-bit output --

def assert_rgb8_matches(got_u8, y_ref, what):
    """Codes equal the oracle's quantization of its fp64 result, except where that
    result lies within a hair of a rounding boundary (a different summation order
    may flip those by one code); such positions must be rare."""
    ref = O.quantize_rgb8(y_ref)
    amb = O.rgb8_ambiguous(y_ref)
    got = np.asarray(got_u8).astype(np.int64)
    d = np.abs(got - ref.astype(np.int64))
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(d[~amb] == 0), "%s: %d codes differ away from a rounding boundary" % (what, int((d[~amb] > 0).sum()))
    assert np.all(d[amb] <= 1), what
    assert amb.mean() < 0.01, "%s: %.3f of the positions are ambiguous" % (what, amb.mean())
    # the codes span the range (not a degenerate all-0 / all-255 output)
    assert ref.min() < 64 and ref.max() > 192, (what, ref.min(), ref.max())


@pytest.mark.parametrize("case", [
    # cin, cout, up_s, h, w, splits, residual
    (96, 3, 2, 13, 37, [1, 4, 3], False),   # output head kernel
    (64, 3, 2, 9, 20, [2, 3], True),         # output head kernel + residual
    (96, 3, 1, 20, 36, [2, 3], False),       # small-output kernel (1440p stage's last conv)
    (32, 16, 1, 11, 40, [1, 2], True),       # small-output kernel, 16 channels
], ids=lambda c: "ci%d_co%d_us%d_res%d" % (c[0], c[1], c[2], c[6]))
def test_conv_rgb8_output(case):
    cin, cout, up_s, h, w, splits, residual = case
    say("rgb8 conv %s" % (case,))
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(6, 21)))
    # weights scaled so the output spans [-1, 1] and beyond (clamping exercised)
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(6, 22)) * 0.6)
    b = synth.bias(cout, synth.seed(6, 23))
    r = synth.bf16(synth.video(cout, t, h * up_s, w * up_s, synth.seed(6, 24)) * 0.3) if residual else None
    y = O.one_shot(to_oracle(x), to_oracle(wt), to_oracle(b), O.REPLICATE, up_s=up_s)
    if residual:
        y = y + to_oracle(r)
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), up_s=up_s, residual=residual, out_u8=True,
                       max_chunk_t=max(splits))
    assert plan.out_dtype == torch.uint8
    got = _run_chunks(plan, to_device_cl(x), splits, residual_cl=to_device_cl(r) if residual else None)
    assert got.dtype == torch.uint8
    assert_rgb8_matches(got.cpu().permute(3, 0, 1, 2).numpy(), y, "rgb8 conv")


def test_rgb8_rejected_where_unsupported():
    """The 3x3 kernel for 96/128-channel blocks has no 8-bit store: plan creation
    fails with ESHAPE before any device work; an act cannot be 8-bit."""
    wt = synth.bf16(synth.conv_weight(96, 32, 3, 3, 3, synth.seed(6, 30))).cuda()
    with pytest.raises(C.Cc3dError) as e:
        P.conv_plan(wt, 8, 16, out_u8=True)
    assert e.value.status == C.ESHAPE
    w3 = synth.bf16(synth.conv_weight(4, 32, 3, 3, 3, synth.seed(6, 31))).cuda()
    with pytest.raises(C.Cc3dError) as e:
        P.conv_plan(w3, 8, 16, out_u8=True, act=True, gamma=torch.ones(4, device="cuda"))
    assert e.value.status == C.EINVAL


def test_decoder_rgb8_output_matches_bf16_head():
    """The decoder with 8-bit output: the same kernels up to the head, whose codes
    match the oracle's quantization of the head conv fed the GPU's own head input."""
    say("decoder rgb8")
    stages = ((64, 2), (32, 2), (16, 1))
    full = OM.decoder_layer_shapes(c_latent=16, stages=stages)
    gains = {s_[0]: s_[6] for s_ in full}
    cpu, dev = _params([s_[:6] for s_ in full], 4, lambda n: gains[n])
    t, h, w, splits = 5, 3, 5, [2, 3]
    x = synth.bf16(synth.video(16, t, h, w, synth.seed(4, 1)))
    x_cl = to_device_cl(x)
    ops = S.decoder_ops(dev, stages=stages, unique_slots=True, out_u8=True)
    plan = P.stack_plan(ops, 16, h, w, max_chunk_t=max(splits))
    ops_b = S.decoder_ops(dev, stages=stages, unique_slots=True)
    plan_b = P.stack_plan(ops_b, 16, h, w, max_chunk_t=max(splits))
    st, st_b = P.Stream(plan), P.Stream(plan_b)
    head = ops[-1]
    ref_head = O.CausalConvStream(cpu["head"]["w"], cpu["head"]["b"], O.REPLICATE, 2, 1)
    t0 = 0
    for n in splits:
        first = st.frames_seen == 0
        xc = x_cl[t0:t0 + n].contiguous()
        y8, yb = st.step(xc), st_b.step(xc)
        torch.cuda.synchronize()
        hin = plan.read_slot(head.src, n, first)
        assert torch.equal(hin, plan_b.read_slot(ops_b[-1].src, n, first)), "layers before the head differ"
        y_ref = ref_head.step(from_device_cl(hin))
        assert_rgb8_matches(y8.cpu().permute(3, 0, 1, 2).numpy(), y_ref, "decoder head rgb8 (chunk at %d)" % t0)
        # the bf16 output and the codes describe the same values
        assert np.abs(O.quantize_rgb8(from_device_cl(yb)).astype(int) -
                      y8.cpu().permute(3, 0, 1, 2).numpy().astype(int)).max() <= 1
        t0 += n


# ------------------------------------------------------------ strided convs --
# The encoder side: spatial stride 2 (outputs centred on even input pixels) and
# temporal stride 2 (outputs at input frames tau = phase mod 2 over the video),
# against the oracle's strided stream.

STRIDED_CASES = [
    # cin, cout, k, stride_s, stride_t, h, w, splits, tpad, aligned, bias, residual, act
    (32, 96, (3, 3, 3), 2, 1, 17, 35, [2, 3], C.TPAD_REPLICATE, False, True, False, False),
    (32, 128, (3, 3, 3), 2, 2, 16, 34, [1, 2, 4], C.TPAD_ZERO, False, False, False, False),
    (32, 128, (3, 3, 3), 2, 2, 15, 33, [2, 4], C.TPAD_REPLICATE, True, True, False, False),
    (64, 192, (3, 3, 3), 2, 2, 9, 20, [3, 2], C.TPAD_ZERO, False, True, False, False),
    (16, 32, (3, 1, 1), 1, 2, 7, 9, [1, 2, 2], C.TPAD_ZERO, False, False, False, False),
    (32, 64, (1, 1, 1), 2, 1, 10, 33, [2, 1], C.TPAD_REPLICATE, False, True, False, False),
    (8, 96, (3, 3, 3), 2, 1, 36, 70, [1, 2], C.TPAD_ZERO, False, True, True, True),
    (96, 192, (2, 3, 3), 2, 2, 11, 21, [1, 2], C.TPAD_ZERO, False, False, False, True),
    (384, 384, (3, 3, 3), 2, 2, 4, 6, [2, 2], C.TPAD_ZERO, True, False, False, False),
    (16, 16, (3, 3, 3), 2, 2, 1, 1, [1, 2], C.TPAD_REPLICATE, False, True, False, False),
    # the register-blocked strided tile (2 output rows x 64 columns): several
    # column and row tiles with ragged ends, two 128-channel blocks, frames that
    # the tiles cover exactly (with residual and act), one-pixel frames
    (64, 96, (3, 3, 3), 2, 2, 13, 261, [3, 2], C.TPAD_REPLICATE, False, True, False, False),
    (32, 256, (3, 3, 3), 2, 1, 10, 140, [2, 2], C.TPAD_ZERO, False, False, True, False),
    (96, 96, (3, 3, 3), 2, 2, 8, 256, [1, 2], C.TPAD_ZERO, False, True, True, True),
    (64, 128, (3, 3, 3), 2, 2, 1, 2, [2, 2], C.TPAD_REPLICATE, True, True, False, False),
    (192, 384, (3, 3, 3), 2, 2, 6, 9, [1, 4], C.TPAD_ZERO, False, True, False, True),
    # 8 input channels (pixels padded to 8): temporal taps folded into one K step,
    # k_t 3 and 2, both phases, 96 and 128 channels, ragged tiles, one-frame chunks
    (8, 96, (3, 3, 3), 2, 1, 19, 133, [1, 1, 2], C.TPAD_REPLICATE, False, True, True, True),
    (8, 128, (2, 3, 3), 2, 2, 9, 70, [3, 2], C.TPAD_ZERO, False, False, False, False),
    (8, 256, (3, 3, 3), 2, 2, 8, 64, [2, 2], C.TPAD_ZERO, True, True, False, False),
    # output channels a multiple of 192: the strided tile in 192-channel blocks
    # (4 output rows x 32 columns): ragged row and column tiles, tiles covered
    # exactly, two blocks, act fused over one block, k_t 2, one-pixel frames
    (96, 192, (3, 3, 3), 2, 2, 19, 75, [3, 2], C.TPAD_REPLICATE, False, True, True, True),
    (64, 192, (3, 3, 3), 2, 1, 16, 128, [1, 2], C.TPAD_ZERO, True, True, False, True),
    (192, 384, (3, 3, 3), 2, 2, 17, 66, [2, 2], C.TPAD_ZERO, True, True, True, False),
    (32, 192, (2, 3, 3), 2, 2, 9, 33, [1, 2, 2], C.TPAD_REPLICATE, False, False, False, False),
    (128, 384, (3, 3, 3), 2, 1, 1, 1, [2, 1], C.TPAD_REPLICATE, False, True, False, True),
]


def _ntile(cout):
    """Output channels per workgroup of the bf16 conv kernels."""
    if cout <= 16:
        return 16
    if cout <= 32:
        return 32
    if cout <= 64:
        return 64
    if cout <= 96:
        return 96
    if cout <= 128:
        return 128
    return 96 if cout % 96 == 0 else (128 if cout % 128 == 0 else 64)


def _random_strided_cases(n, seed):
    """Seeded strided convs: kernel shapes, channel counts (the register-blocked
    strided tile and the generic kernel), spatial and/or temporal stride, both
    temporal phases, frame sizes from one pixel, chunkings that keep every count
    whole (phase 0: an odd first chunk, even later ones; phase 1: even chunks),
    history fills, bias, residual and act."""
    rng = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        k = [(3, 3, 3), (3, 3, 3), (1, 1, 1), (3, 1, 1), (2, 3, 3)][rng.randint(5)]
        cin = int(rng.choice([8, 16, 32, 64, 96]))
        cout = int(rng.choice([8, 16, 24, 64, 96, 128, 192, 256]))
        ss, st = [(2, 1), (1, 2), (2, 2), (2, 2)][rng.randint(4)]
        aligned = bool(rng.randint(2)) if st == 2 else False
        h, w = int(rng.randint(1, 20)), int(rng.randint(1, 80))
        nch = int(rng.randint(1, 4))
        if st == 2:
            splits = [2 * int(rng.randint(1, 3)) - (0 if aligned else 1)] + [2 * int(rng.randint(1, 3))
                                                                          for _ in range(nch - 1)]
        else:
            splits = [int(v) for v in rng.randint(1, 4, size=nch)]
        tpad = [C.TPAD_REPLICATE, C.TPAD_ZERO][rng.randint(2)]
        epi = [(False, False), (True, False), (False, True), (True, True)][rng.randint(4)]
        cases.append((cin, cout, k, ss, st, h, w, splits, tpad, aligned, bool(rng.randint(2)), epi[0], epi[1]))
    return cases


def _strided_ref(x, wt, b, tpad, splits, ss, st, aligned, r=None, g=None):
    v = O.chunked(to_oracle(x), to_oracle(wt), None if b is None else to_oracle(b), TP[tpad], splits=splits,
                  aligned=aligned, stride_s=ss, stride_t=st)
    if r is not None:
        v = v + to_oracle(r)
    return v if g is None else O.act(O.round_bf16(v), to_oracle(g), 1e-6)


@pytest.mark.parametrize("case", STRIDED_CASES + _random_strided_cases(16, 13),
                         ids=lambda c: "ci%d_co%d_k%s_s%d_t%d_%dx%d_al%d_%s" % (
                             c[0], c[1], "".join(map(str, c[2])), c[3], c[4], c[5], c[6], c[9],
                             "-".join(map(str, c[7]))))
def test_bf16_strided_conv_vs_oracle(case):
    cin, cout, k, ss, st, h, w, splits, tpad, aligned, with_bias, residual, act = case
    say("bf16 strided conv %s" % (case,))
    t = sum(splits)
    x = synth.bf16(synth.video(cin, t, h, w, synth.seed(40, cin + cout)))
    wt = synth.bf16(synth.conv_weight(cout, cin, *k, synth.seed(40, 2)))
    b = synth.bias(cout, synth.seed(40, 3)) if with_bias else None
    g = synth.gain(cout, synth.seed(40, 4)) if act else None
    t_out = sum(O.strided_frames(n, st, aligned, seen=sum(splits[:i])) for i, n in enumerate(splits))
    ho, wo = (h + ss - 1) // ss, (w + ss - 1) // ss
    r = synth.bf16(synth.video(cout, t_out, ho, wo, synth.seed(40, 5))) if residual else None
    ref = _strided_ref(x, wt, b, tpad, splits, ss, st, aligned, r, g)
    plan = P.conv_plan(wt.cuda(), h, w, bias=None if b is None else b.cuda(), gamma=None if g is None else g.cuda(),
                       act=act, residual=residual, max_chunk_t=max(splits), tpad=tpad, aligned=aligned,
                       stride_s=ss, stride_t=st)
    C.check(C.lib().cc3d_profile_enable(plan._h, 1), "profile_enable")
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits,
                                     residual_cl=to_device_cl(r) if residual else None))
    pr = C.OpProfile()
    C.check(C.lib().cc3d_profile_read(plan._h, 0, 0, ctypes.byref(pr)), "profile_read")
    # 3x3 spatial stride 2 in 96/128-channel blocks: the register-blocked kernel
    # (with 8 input channels, its temporal taps folded into one K step; with
    # output channels a multiple of 192, in 192-channel blocks)
    v2 = ss == 2 and k[1:] == (3, 3) and _ntile(cout) in (96, 128)
    fam = ("_v2tf" if cin == 8 else "_v2") if v2 else ""
    nt = 192 if v2 and cin != 8 and cout % 192 == 0 else _ntile(cout)
    assert pr.kernel.decode() == "conv_bf16%s_s%dt%d_k%d_n%d" % (fam, ss, st, k[1], nt), pr.kernel
    assert got.shape == (cout, t_out, ho, wo)
    assert_bf16_close(got, ref, "strided conv")


@pytest.mark.parametrize("case", [
    # cin, cout, k, stride_s, stride_t, h, w, splits, tpad, aligned
    (16, 16, (3, 3, 3), 2, 2, 12, 13, [1, 2, 2], C.TPAD_ZERO, False),
    (8, 24, (2, 3, 3), 2, 1, 9, 10, [3, 1], C.TPAD_REPLICATE, False),
    (12, 8, (3, 1, 1), 1, 2, 5, 6, [4, 2], C.TPAD_REPLICATE, True),
])
def test_fp32_strided_conv_vs_oracle(case):
    cin, cout, k, ss, st, h, w, splits, tpad, aligned = case
    say("fp32 strided conv %s" % (case,))
    x = synth.video(cin, sum(splits), h, w, synth.seed(41, 1))
    wt = synth.conv_weight(cout, cin, *k, synth.seed(41, 2))
    b = synth.bias(cout, synth.seed(41, 3))
    ref = _strided_ref(x, wt, b, tpad, splits, ss, st, aligned)
    plan = P.conv_plan(wt.cuda(), h, w, bias=b.cuda(), max_chunk_t=max(splits), tpad=tpad, aligned=aligned,
                       stride_s=ss, stride_t=st)
    got = from_device_cl(_run_chunks(plan, to_device_cl(x), splits))
    assert_fp32_close(got, ref, "fp32 strided conv")


@pytest.mark.parametrize("aligned", [False, True])
def test_strided_chunk_lengths_checked_before_any_work(aligned):
    """A chunk that would leave a temporal stride a fractional frame count is
    refused (CC3D_ESHAPE) by the shape query and by forward_chunk, before any
    device work: the state keeps its frame count and y is untouched."""
    say("strided chunk rule aligned=%s" % aligned)
    wt = synth.bf16(synth.conv_weight(32, 16, 3, 3, 3, synth.seed(42, 1))).cuda()
    plan = P.conv_plan(wt, 6, 8, max_chunk_t=4, aligned=aligned, stride_s=2, stride_t=2)
    c, t, h, w = (ctypes.c_int() for _ in range(4))
    for tc, first, ok in [(1, 1, not aligned), (2, 1, aligned), (3, 1, not aligned), (2, 0, True), (3, 0, False)]:
        st = C.lib().cc3d_output_shape(plan._h, tc, first, ctypes.byref(c), ctypes.byref(t), ctypes.byref(h),
                                       ctypes.byref(w))
        assert (st == C.OK) == ok, (tc, first, C.last_error())
        if ok:
            assert (t.value, h.value, w.value, c.value) == (
                O.strided_frames(tc, 2, aligned, seen=0 if first else (2 if aligned else 1)), 3, 4, 32)
    stream = P.Stream(plan)
    bad = 1 if aligned else 2
    x = torch.zeros((bad, 6, 8, 16), dtype=torch.bfloat16, device="cuda")
    y = torch.full((4, 3, 4, 32), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(C.Cc3dError):
        plan.forward_chunk(x, stream.states[0], stream.states[1], y=y)
    ci, co = stream.states[0]._c(), stream.states[1]._c()
    co.frames_seen = 5
    st = C.lib().cc3d_forward_chunk(plan._h, ctypes.c_void_p(x.data_ptr()), bad, ctypes.byref(ci),
                                    ctypes.byref(co), None, ctypes.c_void_p(y.data_ptr()), None)
    assert st == C.ESHAPE, C.last_error()
    torch.cuda.synchronize()
    assert co.frames_seen == 5 and stream.states[0].frames_seen == 0
    assert bool((y == 7.0).all())


def _encoder_case(name):
    """Encoder of a stack_cases configuration, twice on the GPU (production and
    unique-slot wiring, bitwise equal), every layer against the oracle fed that
    layer's own GPU input, and the whole stack against the storage-rounded
    oracle (the recorded end-to-end bound).  The pixels go in padded with zero
    channels to 8 (bf16 inputs take multiples of 8), conv_in's weights likewise."""
    c = SC.STACK_CASES[name]
    full = SC.layer_shapes(c)
    gains = {s_[0]: s_[6] for s_ in full}
    cpu, dev = _params([s_[:6] for s_ in full], c["cfg"], lambda n: gains[n])
    w_in = dev["conv_in"]["w"]
    pad = torch.zeros((w_in.shape[0], 8) + tuple(w_in.shape[2:]), dtype=w_in.dtype, device=w_in.device)
    pad[:, :c["c_in"]] = w_in
    dev["conv_in"]["w"] = pad
    x = SC.pixels(c)
    x8 = torch.zeros((8,) + tuple(x.shape[1:]), dtype=x.dtype)
    x8[:c["c_in"]] = x
    x_cl = to_device_cl(x8)
    mode = O.ZERO if c["mode"] == "zero" else O.REPLICATE
    tpad = C.TPAD_ZERO if c["mode"] == "zero" else C.TPAD_REPLICATE
    splits = list(c["splits"])
    ops_u = S.encoder_ops(dev, stages=c["stages"], c_latent=c["c_lat"], unique_slots=True)
    ops_p = S.encoder_ops(dev, stages=c["stages"], c_latent=c["c_lat"])
    for o in ops_u + ops_p:
        o.tpad = tpad
    plan_u = P.stack_plan(ops_u, 8, c["h"], c["w"], max_chunk_t=max(splits), aligned=c["aligned"])
    plan_p = P.stack_plan(ops_p, 8, c["h"], c["w"], max_chunk_t=max(splits), aligned=c["aligned"])
    su, sp = P.Stream(plan_u), P.Stream(plan_p)
    layer = {i: O.CausalConvStream(cpu[o.name]["w"], cpu[o.name]["b"], mode, aligned=c["aligned"],
                                   stride_s=o.stride_s, stride_t=o.stride_t)
             for i, o in enumerate(ops_u)}
    outs, t0 = [], 0
    for n in splits:
        first = su.frames_seen == 0
        xc = x_cl[t0:t0 + n].contiguous()
        yu, yp = su.step(xc), sp.step(xc)
        torch.cuda.synchronize()
        assert torch.equal(yu, yp), "production wiring differs from the unique-slot wiring"
        outs.append(yu)
        ten = {C.SLOT_X: xc, C.SLOT_Y: yu}
        for o in ops_u:
            for sl in (o.out, o.act_out):
                if sl > C.SLOT_AUX:
                    ten[sl] = plan_u.read_slot(sl, n, first)
        torch.cuda.synchronize()
        for i, o in enumerate(ops_u):
            src = from_device_cl(ten[o.src])
            if o.name == "conv_in":
                src = src[:c["c_in"]]
            v = layer[i].step(src)
            if o.res != C.SLOT_NONE:
                v = v + from_device_cl(ten[o.res])
            if o.out != C.SLOT_NONE:
                assert_bf16_close(from_device_cl(ten[o.out]), v, "%s out (chunk at %d)" % (o.name, t0))
            if o.act_out != C.SLOT_NONE:
                ref_act = O.act(O.round_bf16(v), cpu_gain(cpu, ops_u, o), 1e-6)
                assert_bf16_close(from_device_cl(ten[o.act_out]), ref_act, "%s act (chunk at %d)" % (o.name, t0))
        t0 += n
    got = from_device_cl(torch.cat(outs, dim=0))
    enc = OM.Encoder(cpu, stages=c["stages"], store=O.round_bf16, aligned=c["aligned"], mode=mode)
    ref, t0 = [], 0
    for n in splits:
        ref.append(enc.step(to_oracle(x)[:, t0:t0 + n]))
        t0 += n
    return got, np.concatenate(ref, axis=1)


@pytest.mark.parametrize("name", [k for k in SC.STACK_CASES if k.startswith("enc_")])
def test_encoder_layerwise_and_end_to_end(name):
    say("encoder %s" % name)
    c = SC.STACK_CASES[name]
    got, ref = _encoder_case(name)
    n, h, w = c["t"], c["h"], c["w"]
    for _ in range(len(c["stages"]) + 1):  # conv_in and every stage's down conv halve the frame
        h, w = (h + 1) // 2, (w + 1) // 2
    for _, f in reversed(c["stages"]):
        n = O.strided_frames(n, f, c["aligned"])
    assert got.shape == (c["c_lat"], n, h, w)
    assert_stack_close(got, ref, name, "encoder")
