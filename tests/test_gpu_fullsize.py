"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, on sampled outputs the fp64 oracle computes one by one.

Each workload runs through the library at its real frame size and chunking
(the first chunks of the stream: the first-chunk rule and at least one carried
cache).  After every chunk, every conv and norm op is checked on sampled
output positions -- the four corners, the first and last rows and columns, the
first and last frame of the chunk (the chunk boundaries), plus seeded random
positions -- against the oracle fed that op's own GPU input (the per-layer
parity bound): ``oracle.conv_points`` evaluates the conv sum of the definition
at each sampled position from the op's causal window.  The window is the op's
input frames behind its history (copies of the first frame on the video's
first chunk, else the last two frames of the previous window) after the
temporal growth; only the rows the sampled positions read are copied to the
host.
"""
import numpy as np
import pytest
import torch

from causal_convolution_x3x3_amd import capi as C
from causal_convolution_x3x3_amd import plan as P
from causal_convolution_x3x3_amd import stacks as S
from causal_convolution_x3x3_amd import synth
from oracle import model as OM
from oracle import oracle as O

from helpers import BF16_MAX_REL, BF16_MEAN_REL, say, to_oracle

pytestmark = pytest.mark.gpu

EPS = 1e-6


class Window:
    """The causal window Z = history || V of one conv op, on the device.  Which
    input frame each window frame holds is the oracle's own stream rule
    (oracle.CausalConvStream.window: history fill, temporal growth, cache of the
    last k_t-1 frames) run on frame numbers (0 = a zero frame); the frames are
    the op's GPU input frames, gathered on the device."""

    def __init__(self, kt, up_t, mode=O.REPLICATE, aligned=False):
        self.rule = O.CausalConvStream(np.zeros((1, 1, kt, 1, 1)), None, mode, 1, up_t, aligned=aligned)
        self.frames, self.seen = {}, 0

    def step(self, x, first):
        if first:
            self.rule.reset()
            self.frames, self.seen = {}, 0
        n = x.shape[0]
        nums = np.arange(self.seen + 1, self.seen + n + 1, dtype=np.float64).reshape(1, n, 1, 1)
        for i in range(n):
            self.frames[self.seen + 1 + i] = x[i]
        self.seen += n
        z_nums = [int(k) for k in self.rule.window(nums)[0, :, 0, 0]]
        zero = torch.zeros_like(x[0])
        z = torch.stack([self.frames[k] if k > 0 else zero for k in z_nums])
        keep = [int(k) for k in self.rule.cache[0, :, 0, 0] if k > 0]
        self.frames = {k: self.frames[k].clone() for k in keep}
        return z


class Tally:
    """Sampled |d| and |ref| sums for the parity bounds over all samples of a check."""

    def __init__(self):
        self.dmax = self.rmax = self.dsum = self.rsum = 0.0

    def add(self, got, ref):
        d = np.abs(got - ref)
        self.dmax = max(self.dmax, float(d.max()))
        self.rmax = max(self.rmax, float(np.abs(ref).max()))
        self.dsum += float(d.mean())
        self.rsum += float(np.abs(ref).mean())

    def check(self, what):
        mx, mn = self.dmax / max(self.rmax, 1e-30), self.dsum / max(self.rsum, 1e-30)
        assert mx <= BF16_MAX_REL and mn <= BF16_MEAN_REL, "%s: sampled max-rel %.3g (<= %g), mean-rel %.3g (<= %g)" % (
            what, mx, BF16_MAX_REL, mn, BF16_MEAN_REL)
        return mx, mn


def _samples(rng, t, h, w, nrows=8, ncols=128, nts=4):
    """Rows (first, last, random), columns (the first two, the last two, random)
    and frames (first, last, random): up to nrows x ncols x nts positions."""
    rows = sorted(set([0, h - 1] + list(rng.randint(0, h, size=nrows - 2))))
    cols = sorted(set([0, 1, w - 2, w - 1] + list(rng.randint(0, w, size=ncols - 4))))
    ts = sorted(set([0, t - 1] + list(rng.randint(0, t, size=nts - 2))))
    return rows, [c for c in cols if 0 <= c < w], ts


def _gather(y, ts, row, cols):
    """y[t, row, c, :] for t in ts, c in cols (device [T][H][W][C]) -> n x C float64."""
    ti = torch.tensor(ts, device=y.device).repeat_interleave(len(cols))
    ci = torch.tensor(cols, device=y.device).repeat(len(ts))
    return y[ti, row][torch.arange(ti.numel(), device=y.device), ci].double().cpu().numpy()


def check_conv(z, w, b, up, ts, rows, cols, out=None, res=None, act=None, gamma=None, tallies=None,
               down=1, t_stride=1, t_first=0):
    """Compare the op's stored result (out = conv + bias (+ res), bf16) and/or
    its act (SiLU(RMSNorm(rounded result))) with the oracle at the sampled
    positions.  z: [Tz][Hin][Win][Cin] device window; w, b: float64 numpy.
    A strided conv (down, t_stride): output frame t's window starts at window
    frame t_stride*t + t_first; output pixel y is centred on input row down*y."""
    hin = z.shape[1]
    for y in rows:
        if down == 1:
            r0 = max(0, (y - 1) // up)
            r1 = min(hin - 1, (y + 1) // up)
            yl = y - up * r0
        else:  # an even first row, so the output row stays on the stride grid
            r0 = max(0, down * y - 2)
            r1 = min(hin - 1, down * y + 1)
            yl = (down * y - r0) // down
        zc = z[:, r0:r1 + 1].float().cpu().numpy().transpose(3, 0, 1, 2)  # [C][T][rows][W], a view
        pts = np.array([(t_stride * t + t_first, yl, c) for t in ts for c in cols], dtype=np.int32)
        v = O.conv_points(zc, w, b, pts, up, down=down)  # n x Cout
        if res is not None:
            v = v + _gather(res, ts, y, cols)
        if out is not None:
            tallies["out"].add(_gather(out, ts, y, cols), v)
        if act is not None:
            ref = O.act(O.round_bf16(v).T, gamma, EPS).T
            tallies["act"].add(_gather(act, ts, y, cols), ref)


def check_norm(src, act, gamma, ts, rows, cols, res=None, out=None, tallies=None):
    for y in rows:
        v = _gather(src, ts, y, cols)
        if res is not None:
            v = O.round_bf16(v + _gather(res, ts, y, cols))
            if out is not None:
                tallies["out"].add(_gather(out, ts, y, cols), v)
        tallies["act"].add(_gather(act, ts, y, cols), O.act(v.T, gamma, EPS).T)


def run_stack_sampled(ops, params_cpu, x_cl, cin, h, w, splits, seed, max_pts_rows=8, fold_upsample=False,
                      chunk_of=None, check_from=0):
    """Run `ops` chunk by chunk and check every op on sampled positions.
    ``chunk_of(k, n)``: the k-th chunk's input (else slices of x_cl);
    ``check_from``: chunks before it run (and move the reference windows on)
    unchecked, and their outputs are not kept."""
    plan = P.stack_plan(ops, cin, h, w, max_chunk_t=max(splits), fold_upsample=fold_upsample)
    st = P.Stream(plan)
    wins = {i: Window(o.k[0], o.up_t, O.ZERO if o.tpad == C.TPAD_ZERO else O.REPLICATE)
            for i, o in enumerate(ops) if o.kind == C.OP_CONV}
    rng = np.random.RandomState(seed)
    worst = {}
    outs, t0 = [], 0
    for ci, n in enumerate(splits):
        first = st.frames_seen == 0
        xc = chunk_of(ci, n) if chunk_of else x_cl[t0:t0 + n].contiguous()
        checking = ci >= check_from
        if checking or ci % 10 == 0:
            say("  chunk %d at %d (%d frames)%s" % (ci, t0, n, "" if checking else ", unchecked"))
        y = st.step(xc)
        torch.cuda.synchronize()
        if checking:
            outs.append(y.cpu())

        def slot(s):
            if s == C.SLOT_X:
                return xc
            if s == C.SLOT_Y:
                return y
            if s == C.SLOT_NONE:
                return None
            return plan.read_slot(s, n, first)

        for i, o in enumerate(ops):
            src = slot(o.src)
            if not checking:  # only the reference windows move on
                if o.kind == C.OP_CONV:
                    wins[i].step(src, first)
                del src
                continue
            res, out, act = slot(o.res), slot(o.out), slot(o.act_out)
            ref_t = out if out is not None else act
            tal = {"out": Tally(), "act": Tally()}
            rows, cols, ts = _samples(rng, ref_t.shape[0], ref_t.shape[1], ref_t.shape[2], nrows=max_pts_rows)
            if o.kind == C.OP_CONV:
                z = wins[i].step(src, first)
                p = params_cpu[o.name]
                g = None
                if act is not None:
                    g = params_cpu["__gain_of_act_%d" % o.act_out]
                # a temporal stride's first output is the window's first frame only on
                # the video's first chunk (the first frame on its own)
                tf = 0 if (o.stride_t == 1 or first) else 1
                if o.name == "conv_in" and p["w"].shape[1] != o.w.shape[1]:
                    z = z[..., :p["w"].shape[1]]  # the pixels' real channels (the rest are zero)
                check_conv(z, p["w"], p["b"], o.up_s, ts, rows, cols, out=out, res=res, act=act, gamma=g,
                           tallies=tal, down=o.stride_s, t_stride=o.stride_t, t_first=tf)
            else:
                check_norm(src, act, to_oracle(o.gamma.cpu()), ts, rows, cols, res=res, out=out, tallies=tal)
            for k in ("out", "act"):
                if tal[k].rsum > 0:
                    mx, mn = tal[k].check("%s %s (chunk at %d)" % (o.name or "op%d" % i, k, t0))
                    key = "%s.%s" % (o.name or "op%d" % i, k)
                    worst[key] = max(worst.get(key, 0.0), mn)
            del src, res, out, act, ref_t
        torch.cuda.synchronize()
        t0 += n
    say("  worst sampled mean-rel per op: " + ", ".join("%s %.2e" % kv for kv in sorted(worst.items())))
    return torch.cat(outs), worst


def _gains_of_acts(ops, params_cpu):
    """For every act slot, the RMSNorm gain of the conv that produces it (the
    gain that belongs to the conv reading it)."""
    for o in ops:
        if o.act_out != C.SLOT_NONE and o.gamma is not None:
            params_cpu["__gain_of_act_%d" % o.act_out] = to_oracle(o.gamma.cpu())


def _param_pair(cout, cin, cfg, i, with_gain, k=(3, 3, 3)):
    w = synth.bf16(synth.conv_weight(cout, cin, *k, synth.seed(cfg, 10 + 3 * i)))
    g = synth.gain(cin, synth.seed(cfg, 11 + 3 * i)) if with_gain else None
    dev = {"w": w.cuda(), "g": None if g is None else g.cuda(), "b": None}
    cpu = {"w": to_oracle(w), "g": None if g is None else to_oracle(g), "b": None}
    return dev, cpu


def test_max_frame_size_sampled():
    """The largest input frame a plan accepts (just under 2^30 elements: 384
    channels x 1440 x 1940, 2.1 GB per frame), two one-frame chunks (the history
    rule, then the carried cache), checked on sampled outputs that include the
    last rows and columns -- where a 32-bit byte offset would wrap."""
    cin, cout, h, w = 384, 96, 1440, 1940
    assert cin * h * w < 2 ** 30 <= cin * h * (w + 2)
    say("max frame size: %d x %d x %d" % (cin, h, w))
    wt = synth.bf16(synth.conv_weight(cout, cin, 3, 3, 3, synth.seed(11, 2)))
    gen = torch.Generator(device="cuda").manual_seed(11001)
    x = torch.randn((2, h, w, cin), device="cuda", generator=gen).to(torch.bfloat16)
    plan = P.stack_plan([P.Op(cout=cout, w=wt.cuda(), out=C.SLOT_Y, name="conv")], cin, h, w, max_chunk_t=1)
    st = P.Stream(plan)
    win = Window(3, 1)
    rng = np.random.RandomState(1101)
    wt64 = to_oracle(wt)
    for t0 in range(2):
        first = t0 == 0
        xc = x[t0:t0 + 1].contiguous()
        y = st.step(xc)
        torch.cuda.synchronize()
        z = win.step(xc, first)
        rows, cols, ts = _samples(rng, 1, h, w, nrows=8, ncols=128, nts=2)
        tal = {"out": Tally(), "act": Tally()}
        check_conv(z, wt64, None, 1, ts, sorted(set(rows + [h - 2])), cols, out=y, tallies=tal)
        mx, mn = tal["out"].check("max frame, chunk %d" % t0)
        say("  chunk %d: sampled max-rel %.2e mean-rel %.2e" % (t0, mx, mn))
        del y, z
    torch.cuda.empty_cache()


def test_c1_resblock_fullsize_sampled():
    """128-channel residual block at 90x160, 16 frames in 4-frame chunks."""
    wl = synth.WORKLOADS[1]
    say("full size c1: %s" % wl)
    c = wl["c"]
    d1, c1 = _param_pair(c, c, 1, 0, True)
    d2, c2 = _param_pair(c, c, 1, 1, True)
    ops = S.resblock_ops(c, d1, d2)
    ops[0].name, ops[1].name, ops[2].name = "act1", "conv1", "conv2"
    cpu = {"conv1": c1, "conv2": c2}
    _gains_of_acts(ops, cpu)
    x = synth.bf16(synth.video(c, wl["t"], wl["h"], wl["w"], synth.seed(1, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().cuda()
    run_stack_sampled(ops, cpu, x_cl, c, wl["h"], wl["w"], [wl["chunk"]] * (wl["t"] // wl["chunk"]), seed=101)


def test_c2_stage1080_fullsize_sampled():
    """256 channels at 270x480 -> nearest 2x -> conv 256->128 -> act -> conv 128->128,
    24 frames in 4-frame chunks."""
    wl = synth.WORKLOADS[2]
    say("full size c2: %s" % wl)
    d1, c1 = _param_pair(wl["cmid"], wl["cin"], 2, 0, False)
    d2, c2 = _param_pair(wl["cout"], wl["cmid"], 2, 1, True)
    ops = S.upstage_ops(wl["cmid"], wl["cout"], d1, d2)
    ops[0].name, ops[1].name = "conv1", "conv2"
    cpu = {"conv1": c1, "conv2": c2}
    _gains_of_acts(ops, cpu)
    x = synth.bf16(synth.video(wl["cin"], wl["t"], wl["h"], wl["w"], synth.seed(2, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().cuda()
    del x
    run_stack_sampled(ops, cpu, x_cl, wl["cin"], wl["h"], wl["w"], [wl["chunk"]] * (wl["t"] // wl["chunk"]),
                      seed=202)


@pytest.mark.parametrize("fold", [False, True])
def test_c3_stage1440_fullsize_sampled(fold):
    """128 channels at 720x1280 -> nearest 2x -> conv 128->96 -> act -> conv 96->3
    at 2560x1440: the stream's first chunk (1 frame) and the two after it; with
    `fold`, the upsampling conv phase-folded."""
    wl = synth.WORKLOADS[3]
    say("full size c3 (fold=%s): %s" % (fold, wl))
    d1, c1 = _param_pair(wl["cmid"], wl["cin"], 3, 0, False)
    d2, c2 = _param_pair(wl["cout"], wl["cmid"], 3, 1, True)
    ops = S.upstage_ops(wl["cmid"], wl["cout"], d1, d2)
    ops[0].name, ops[1].name = "conv1", "conv2"
    cpu = {"conv1": c1, "conv2": c2}
    _gains_of_acts(ops, cpu)
    splits = [wl["first_chunk"], wl["chunk"], wl["chunk"]]
    x = synth.bf16(synth.video(wl["cin"], sum(splits), wl["h"], wl["w"], synth.seed(3, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().cuda()
    del x
    run_stack_sampled(ops, cpu, x_cl, wl["cin"], wl["h"], wl["w"], splits, seed=303, fold_upsample=fold)


@pytest.mark.parametrize("fold", [False, True])
def test_c3_stage1440_whole_stream_sampled(fold):
    """The whole 361-frame stream of the 1440p stage (1 + 90 chunks of 4, the
    caches carried through all 91), its inputs cycled from 8 distinct chunks as
    in the benchmark; the last three chunks checked on sampled positions against
    the oracle fed each op's own GPU input, its causal windows carried along."""
    wl = synth.WORKLOADS[3]
    say("full size c3, whole stream (fold=%s)" % fold)
    d1, c1 = _param_pair(wl["cmid"], wl["cin"], 3, 0, False)
    d2, c2 = _param_pair(wl["cout"], wl["cmid"], 3, 1, True)
    ops = S.upstage_ops(wl["cmid"], wl["cout"], d1, d2)
    ops[0].name, ops[1].name = "conv1", "conv2"
    cpu = {"conv1": c1, "conv2": c2}
    _gains_of_acts(ops, cpu)
    splits = [wl["first_chunk"]] + [wl["chunk"]] * ((wl["t"] - wl["first_chunk"]) // wl["chunk"])
    assert sum(splits) == wl["t"] == 361 and len(splits) == 91
    pool = [synth.bf16(synth.video(wl["cin"], wl["chunk"], wl["h"], wl["w"], synth.seed(3, 100 + k)))
            .permute(1, 2, 3, 0).contiguous().cuda() for k in range(8)]
    got, worst = run_stack_sampled(ops, cpu, None, wl["cin"], wl["h"], wl["w"], splits, seed=313,
                                   fold_upsample=fold, chunk_of=lambda k, n: pool[k % 8][:n].contiguous(),
                                   check_from=len(splits) - 3)
    assert got.shape == (3 * wl["chunk"], 1440, 2560, 3)
    assert set(worst) == {"conv1.act", "conv2.out"}


def test_c4tg_decoder_fullsize_sampled():
    """The decoder with a TemporalGrow (1x1x1 projection + causal 3x1x1 temporal
    conv) ahead of each stage's upsample conv, at full size: the first two
    clips, every op checked on sampled positions."""
    wl = synth.WORKLOADS[4]
    say("full size c4tg: %s" % wl)
    shapes = OM.decoder_layer_shapes(temporal_grow="before")
    dev, cpu = {}, {}
    for i, (name, co, ci, kt, kh, kw, has_g) in enumerate(shapes):
        d, c = _param_pair(co, ci, 4, i, has_g, k=(kt, kh, kw))
        dev[name], cpu[name] = d, c
    ops = S.decoder_ops(dev, unique_slots=True, temporal_grow="before")
    _gains_of_acts(ops, cpu)
    splits = [wl["first_clip"], wl["clip"]]
    x = synth.bf16(synth.video(wl["c_latent"], sum(splits), wl["h"], wl["w"], synth.seed(4, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().cuda()
    got, worst = run_stack_sampled(ops, cpu, x_cl, wl["c_latent"], wl["h"], wl["w"], splits, seed=414,
                                   max_pts_rows=8)
    assert got.shape == (OM.output_frames(sum(splits)), 1440, 2560, 3)
    assert any(k.startswith("s2.tg.t") for k in worst)


def test_c4_decoder_fullsize_frame_batching():
    """The benchmark's decoder wiring with the last stage and the head run one
    frame at a time (frame batching): bitwise the same RGB as whole clips, on
    the first two clips at full size, in less plan memory."""
    wl = synth.WORKLOADS[4]
    say("full size c4: frame batching of the last stage + head")
    shapes = OM.decoder_layer_shapes()
    dev = {}
    for i, (name, co, ci, kt, kh, kw, has_g) in enumerate(shapes):
        dev[name], _ = _param_pair(co, ci, 4, i, has_g)
    ops = S.decoder_ops(dev)
    g0 = next(i for i, o in enumerate(ops) if o.name == "s2.up")
    splits = [wl["first_clip"], wl["clip"]]
    x = synth.bf16(synth.video(wl["c_latent"], sum(splits), wl["h"], wl["w"], synth.seed(4, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().cuda()
    outs = {}
    mem = {}
    for fb in (0, 1):
        plan = P.stack_plan(ops, wl["c_latent"], wl["h"], wl["w"], max_chunk_t=max(splits), batch_from=g0,
                            frame_batch=fb)
        mem[fb] = plan.device_bytes
        st = P.Stream(plan)
        t0, ys = 0, []
        for n in splits:
            ys.append(st.step(x_cl[t0:t0 + n].contiguous()).cpu())
            t0 += n
        torch.cuda.synchronize()
        outs[fb] = torch.cat(ys)
        del plan, st
        torch.cuda.empty_cache()
    assert torch.equal(outs[0], outs[1]), "frame-batched RGB differs from whole clips"
    say("  plan device memory %.2f GB -> %.2f GB" % (mem[0] / 1e9, mem[1] / 1e9))
    assert mem[1] < mem[0]


def test_c4_decoder_fullsize_sampled():
    """The whole decoder at the full latent size 48 x 90x160 -> 3 x 1440x2560:
    the first two clips (7 then 6 latents -> 25 then 24 frames), every op
    checked; then the benchmark's own slot wiring must give bitwise the same
    RGB output."""
    wl = synth.WORKLOADS[4]
    say("full size c4: %s" % wl)
    shapes = OM.decoder_layer_shapes()
    dev, cpu = {}, {}
    for i, (name, co, ci, kt, kh, kw, has_g) in enumerate(shapes):
        d, c = _param_pair(co, ci, 4, i, has_g)
        dev[name], cpu[name] = d, c
    ops = S.decoder_ops(dev, unique_slots=True)
    _gains_of_acts(ops, cpu)
    splits = [wl["first_clip"], wl["clip"]]
    x = synth.bf16(synth.video(wl["c_latent"], sum(splits), wl["h"], wl["w"], synth.seed(4, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().cuda()
    got, worst = run_stack_sampled(ops, cpu, x_cl, wl["c_latent"], wl["h"], wl["w"], splits, seed=404,
                                   max_pts_rows=8)
    assert got.shape == (OM.output_frames(sum(splits)), 1440, 2560, 3)
    torch.cuda.empty_cache()
    say("  production wiring")
    plan = P.stack_plan(S.decoder_ops(dev), wl["c_latent"], wl["h"], wl["w"], max_chunk_t=max(splits))
    st = P.Stream(plan)
    t0, outs = 0, []
    for n in splits:
        outs.append(st.step(x_cl[t0:t0 + n].contiguous()).cpu())
        t0 += n
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs), got), "production slot wiring differs from the unique-slot wiring"


@pytest.mark.parametrize("fold", [False, True])
def test_c4_decoder_whole_video_sampled(fold):
    """The whole 91-latent video through the decoder at full size in the
    benchmark's 15 clips (7, then 14 of 6 latents -> 361 frames at 1440x2560),
    every cache carried through; every op of the last clip checked on sampled
    positions against the oracle fed its own GPU input, the causal windows
    carried along; with `fold`, the upsampling convs phase-folded."""
    wl = synth.WORKLOADS[4]
    say("full size c4, whole video (fold=%s)" % fold)
    shapes = OM.decoder_layer_shapes()
    dev, cpu = {}, {}
    for i, (name, co, ci, kt, kh, kw, has_g) in enumerate(shapes):
        d, c = _param_pair(co, ci, 4, i, has_g)
        dev[name], cpu[name] = d, c
    ops = S.decoder_ops(dev, unique_slots=True)
    _gains_of_acts(ops, cpu)
    splits = OM.clip_schedule(wl["t"], wl["first_clip"], wl["clip"])
    assert len(splits) == 15 and OM.output_frames(sum(splits)) == 361
    x = synth.bf16(synth.video(wl["c_latent"], sum(splits), wl["h"], wl["w"], synth.seed(4, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().cuda()
    got, worst = run_stack_sampled(ops, cpu, x_cl, wl["c_latent"], wl["h"], wl["w"], splits, seed=434,
                                   max_pts_rows=8, fold_upsample=fold, check_from=len(splits) - 1)
    assert got.shape == (24, 1440, 2560, 3)
    assert all("%s.out" % k in worst for k in ("s0.up", "s1.up", "s2.up", "head"))


def test_c4_decoder_fullsize_folded_sampled():
    """The whole decoder at full size with phase-folded upsample convs (the two
    that double time group their temporal taps): the first two clips, every op
    checked on sampled positions to the same bound as the exact path."""
    wl = synth.WORKLOADS[4]
    say("full size c4, folded upsample convs: %s" % wl)
    shapes = OM.decoder_layer_shapes()
    dev, cpu = {}, {}
    for i, (name, co, ci, kt, kh, kw, has_g) in enumerate(shapes):
        d, c = _param_pair(co, ci, 4, i, has_g)
        dev[name], cpu[name] = d, c
    ops = S.decoder_ops(dev, unique_slots=True)
    _gains_of_acts(ops, cpu)
    splits = [wl["first_clip"], wl["clip"]]
    x = synth.bf16(synth.video(wl["c_latent"], sum(splits), wl["h"], wl["w"], synth.seed(4, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().cuda()
    got, worst = run_stack_sampled(ops, cpu, x_cl, wl["c_latent"], wl["h"], wl["w"], splits, seed=424,
                                   max_pts_rows=8, fold_upsample=True)
    assert got.shape == (OM.output_frames(sum(splits)), 1440, 2560, 3)
    assert all("%s.out" % k in worst for k in ("s0.up", "s1.up", "s2.up"))


def test_e4_encoder_fullsize_sampled():
    """The encoder at its full size, pixels 3 (+5 zero channels) x 1440x2560 ->
    48 x 90x160 latents, zero history: the first two chunks (25 then 24 frames:
    the first frame on its own, then pairs at each temporal stride), every op
    checked on sampled outputs (the strided tile included); then the production
    slot wiring must give bitwise the same latents."""
    say("full size e4")
    h, w, c_pix, c_in = 1440, 2560, 3, 8
    dev, cpu = {}, {}
    for i, (name, co, ci, kt, kh, kw, has_g, _, _) in enumerate(OM.encoder_layer_shapes(c_in=c_pix)):
        d, c = _param_pair(co, ci, 6, i, has_g)
        if name == "conv_in":
            wp = torch.zeros((co, c_in, kt, kh, kw), dtype=d["w"].dtype, device=d["w"].device)
            wp[:, :c_pix] = d["w"]
            d["w"] = wp
        dev[name], cpu[name] = d, c
    ops = S.encoder_ops(dev, unique_slots=True)
    for o in ops:
        o.tpad = C.TPAD_ZERO
    _gains_of_acts(ops, cpu)
    splits = [25, 24]
    x = synth.bf16(synth.video(c_pix, sum(splits), h, w, synth.seed(6, 1)))
    x_cl = torch.zeros((sum(splits), h, w, c_in), dtype=torch.bfloat16, device="cuda")
    x_cl[..., :c_pix] = x.permute(1, 2, 3, 0).cuda()
    del x
    got, worst = run_stack_sampled(ops, cpu, x_cl, c_in, h, w, splits, seed=606, max_pts_rows=6)
    assert got.shape == (13, 90, 160, 48)  # 7 + 6 latents
    torch.cuda.empty_cache()
    say("  production wiring")
    prod = S.encoder_ops(dev)
    for o in prod:
        o.tpad = C.TPAD_ZERO
    plan = P.stack_plan(prod, c_in, h, w, max_chunk_t=max(splits))
    st = P.Stream(plan)
    t0, outs = 0, []
    for n in splits:
        outs.append(st.step(x_cl[t0:t0 + n].contiguous()).cpu())
        t0 += n
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs), got), "production slot wiring differs from the unique-slot wiring"


def test_e4_encoder_whole_video_sampled():
    """The whole 361-frame video through the encoder at full size in the
    benchmark's chunks (25, then 14 of 24 frames -> 91 latents), every cache
    and temporal-stride phase carried through 15 chunks; every op of the last
    chunk checked on sampled outputs against the oracle fed its own GPU input."""
    say("full size e4, whole video")
    h, w, c_pix, c_in = 1440, 2560, 3, 8
    dev, cpu = {}, {}
    for i, (name, co, ci, kt, kh, kw, has_g, _, _) in enumerate(OM.encoder_layer_shapes(c_in=c_pix)):
        d, c = _param_pair(co, ci, 6, i, has_g)
        if name == "conv_in":
            wp = torch.zeros((co, c_in, kt, kh, kw), dtype=d["w"].dtype, device=d["w"].device)
            wp[:, :c_pix] = d["w"]
            d["w"] = wp
        dev[name], cpu[name] = d, c
    ops = S.encoder_ops(dev, unique_slots=True)
    for o in ops:
        o.tpad = C.TPAD_ZERO
    _gains_of_acts(ops, cpu)
    splits = [25] + [24] * 14
    assert sum(splits) == 361

    def chunk_of(k, n):  # chunk k of the pixels, padded with zero channels to 8
        x = synth.bf16(synth.video(c_pix, n, h, w, synth.seed(6, 100 + k)))
        xc = torch.zeros((n, h, w, c_in), dtype=torch.bfloat16, device="cuda")
        xc[..., :c_pix] = x.permute(1, 2, 3, 0).cuda()
        return xc

    got, worst = run_stack_sampled(ops, cpu, None, c_in, h, w, splits, seed=616, max_pts_rows=6,
                                   chunk_of=chunk_of, check_from=len(splits) - 1)
    assert got.shape == (6, 90, 160, 48)  # the last chunk's 6 latents (91 = 7 + 14 x 6)
    # every strided conv was checked (the last down conv stores only its act)
    assert all(k in worst for k in ("conv_in.out", "e0.down.out", "e1.down.out", "e2.down.act", "conv_out.out"))
