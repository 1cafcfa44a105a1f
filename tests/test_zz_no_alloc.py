"""cc3d_conv_forward_noalloc (no device allocation: the weights are repacked
into the library's fixed per-device scratch on every call) against the plan
path (cc3d_plan_create + cc3d_forward_chunk) on the same inputs: bit for bit,
on calls in a row whose second is smaller than the first, with caches carried
between chunks; and a conv that does not fit the scratch is refused before any
device work."""
import ctypes

import pytest
import torch

from causal_convolution_x3x3_amd import capi as C
from causal_convolution_x3x3_amd import plan as P
from causal_convolution_x3x3_amd import synth

from helpers import say

pytestmark = pytest.mark.gpu


def _inputs(cin, cout, h, w, t_total, act, res, up_s, seed):
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(14, seed))).cuda()
    gamma = synth.gain(cout, synth.seed(14, seed + 1)).cuda() if act else None
    bias = synth.bias(cout, synth.seed(14, seed + 2)).cuda()
    x = synth.bf16(synth.video(cin, t_total, h, w, synth.seed(14, seed + 3))).permute(1, 2, 3, 0).contiguous().cuda()
    r = None
    if res:
        r = synth.bf16(synth.video(cout, t_total, h * up_s, w * up_s, synth.seed(14, seed + 4)))
        r = r.permute(1, 2, 3, 0).contiguous().cuda()
    return wt, gamma, bias, x, r


CASES = [
    # cin, cout, h, w, chunks, act, residual, up_s: the first is larger than the second
    (64, 96, 12, 20, (4, 3), True, False, 2),   # register-blocked kernel, fused act, upsampled
    (32, 16, 5, 7, (2, 1), False, True, 1),     # generic kernel, residual
    (96, 3, 9, 17, (3, 2), False, False, 2),    # output head
]


def test_noalloc_matches_the_plan_path():
    runs = []
    for ci, (cin, cout, h, w, chunks, act, res, up_s) in enumerate(CASES):
        say("no-alloc case %d: %s" % (ci, CASES[ci]))
        wt, gamma, bias, x, r = _inputs(cin, cout, h, w, sum(chunks), act, res, up_s, 10 * ci)
        plan = P.conv_plan(wt, h, w, bias=bias, gamma=gamma, up_s=up_s, max_chunk_t=max(chunks), act=act,
                           residual=res)
        # the binding's size check of the states uses the library's own figure
        assert P.conv_state_bytes(3, h, w, cin, 2) == plan.state_bytes
        runs.append((plan, wt, gamma, bias, x, r, chunks, act, up_s))
    # the plan path: every case's chunks
    refs = []
    for plan, wt, gamma, bias, x, r, chunks, act, up_s in runs:
        st = P.Stream(plan)
        outs, t0 = [], 0
        for n in chunks:
            shape = plan.output_shape(n, st.frames_seen == 0)
            res_c = r[t0:t0 + shape[0]].contiguous() if r is not None else None
            outs.append(st.step(x[t0:t0 + n].contiguous(), residual=res_c).clone())
            t0 += n
        refs.append(outs)
    torch.cuda.synchronize()
    # the no-alloc path: first chunks of every case in a row (each smaller than
    # the one before in scratch use), then the second chunks, caches carried
    states = [[plan.new_state(), plan.new_state()] for plan, *_ in runs]
    got = [[] for _ in runs]
    for k in range(2):
        for ci, (plan, wt, gamma, bias, x, r, chunks, act, up_s) in enumerate(runs):
            t0 = sum(chunks[:k])
            n = chunks[k]
            a, b = states[ci][k % 2], states[ci][1 - k % 2]
            shape = plan.output_shape(n, a.frames_seen == 0)
            y = torch.full(shape, -7.0, dtype=torch.bfloat16, device="cuda")
            res_c = r[t0:t0 + shape[0]].contiguous() if r is not None else None
            P.conv_forward_noalloc(wt, x[t0:t0 + n].contiguous(), a, b, y, bias=bias, gamma=gamma,
                                   residual=res_c, up_s=up_s, max_chunk_t=max(chunks), act=act)
            got[ci].append(y)
    torch.cuda.synchronize()
    for ci in range(len(runs)):
        for k in range(2):
            assert torch.equal(got[ci][k], refs[ci][k]), "case %d chunk %d differs from the plan path" % (ci, k)


def test_noalloc_refuses_a_conv_beyond_the_scratch():
    """384 -> 384 channels with the act in a separate pass: its intermediate
    (8 frames of 128 x 128 x 384 bf16, 100 MB) exceeds the scratch; the call
    fails before any device work and leaves y and the states as they were."""
    say("no-alloc: a conv beyond the scratch")
    cin = cout = 384
    h = w = 128
    t = 8
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(14, 90))).cuda()
    gamma = synth.gain(cout, synth.seed(14, 91)).cuda()
    x = torch.zeros((t, h, w, cin), dtype=torch.bfloat16, device="cuda")
    plan = P.conv_plan(wt, h, w, gamma=gamma, max_chunk_t=t, act=True)
    assert plan.device_bytes > C.NOALLOC_SCRATCH_BYTES
    a, b = plan.new_state(), plan.new_state()
    y = torch.full(plan.output_shape(t, True), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(C.Cc3dError) as e:
        P.conv_forward_noalloc(wt, x, a, b, y, gamma=gamma, max_chunk_t=t, act=True)
    assert e.value.status == C.ENOMEM and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()) and b.frames_seen == 0


@pytest.mark.parametrize("cin,cout", [(64, 96), (96, 192)])
def test_noalloc_strided_matches_the_plan_path(cin, cout):
    """A strided conv (spatial and temporal stride 2, the register-blocked
    kernel's strided tile in 96- and 192-channel blocks, fused act) through the
    no-alloc entry point: a 3-frame first chunk then a 2-frame one (smaller),
    bit for bit the plan path's."""
    say("no-alloc: strided conv %d -> %d" % (cin, cout))
    h, w, chunks = 14, 70, (3, 2)
    wt, gamma, bias, x, _ = _inputs(cin, cout, h, w, sum(chunks), True, False, 1, 70)
    plan = P.conv_plan(wt, h, w, bias=bias, gamma=gamma, max_chunk_t=3, act=True, stride_s=2, stride_t=2)
    assert P.conv_state_bytes(3, h, w, cin, 2) == plan.state_bytes
    st = P.Stream(plan)
    refs, t0 = [], 0
    for n in chunks:
        refs.append(st.step(x[t0:t0 + n].contiguous()).clone())
        t0 += n
    a, b = plan.new_state(), plan.new_state()
    got, t0 = [], 0
    for k, n in enumerate(chunks):
        src, dst = (a, b) if k % 2 == 0 else (b, a)
        y = torch.full(plan.output_shape(n, src.frames_seen == 0), -7.0, dtype=torch.bfloat16, device="cuda")
        P.conv_forward_noalloc(wt, x[t0:t0 + n].contiguous(), src, dst, y, bias=bias, gamma=gamma, max_chunk_t=3,
                               act=True, stride_s=2, stride_t=2)
        got.append(y)
        t0 += n
    torch.cuda.synchronize()
    assert got[0].shape == (2, 7, 35, cout) and got[1].shape == (1, 7, 35, cout)
    for k in range(2):
        assert torch.equal(got[k], refs[k]), "chunk %d differs from the plan path" % k
