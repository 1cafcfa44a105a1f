"""Benchmark of the chunked causal Conv3d decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4|c4tg|c3|c2|c1|e4]
                    [--tg-order before|after] [--frame-batch B] [--fold-upsample] [--videos N]
                    [--no-cpu-baseline] [--no-delivery] [--per-op FILE] [--band N]

Workloads (synthetic, seeded; the pages' test videos and trained weights are not
available):
  c4 (default): the decoder stack, latent 48 x 91 frames x 90x160 -> RGB
      3 x 361 x 1440x2560, decoded in clips of 7 then 6 latents (25, then 24
      output frames).  One step = one clip through every layer.
  c4tg: the same decoder with each stage's time growth done by a TemporalGrow
      (1x1x1 projection + causal 3x1x1 temporal conv) on the stage input, run
      before the upsample conv (--tg-order before, the reordered decoder) or on
      the upsampled positions (--tg-order after, the original order).
  --frame-batch B (c4, c4tg): the last stage and the head run over batches of B
      frames of their input (frame batching); reports the plan's device memory.
  --fold-upsample: the upsampling 3x3x3 convs run phase-folded (7/9 of their MFMA
      work; about 16/27 where the conv also doubles time); value stays the
      definition's FLOP rate, executed_tflops and mfma_frac count the MFMA work
      actually done.
  c3: the 1440p output stage, 128 ch x 720x1280 -> nearest 2x -> conv 128->96 ->
      RMSNorm+SiLU -> conv 96->3, 361 frames streamed as 1 + 90 chunks of 4.
      One step = one chunk.
  c2: the 1080p-class stage, 256 ch x 270x480 -> nearest 2x -> conv 256->128 ->
      RMSNorm+SiLU -> conv 128->128 at 540x960, 24 frames in chunks of 4.
  c1: the residual block, 128 ch at 90x160, x + conv(act(conv(act(x)))), 16
      frames in chunks of 4.
  e4: the encoder side, the decoder read backwards: pixels 3 x 361 x 1440x2560
      (padded with zero channels to 8) -> conv_in 3->96 with spatial stride 2 ->
      3 stages (96/192/384 ch; 2 residual blocks, then a conv with spatial
      stride 2 and temporal stride 1/2/2) -> act -> conv 384->48: latents
      48 x 91 x 90x160, in chunks of 25 then 24 frames (7, then 6 latents; zero
      history).  One step = one chunk; value counts conv_in with its 3 real
      input channels.
Inputs are resident in HBM before timing; outputs go to a device ring.
--videos N: whole videos (c4: the 15 clips of 361 frames; c3: 91 chunks; c2, c1:
      their 24 or 16 frames) decoded 1 + N times, the first untimed; the seconds
      per video (min / mean / p99 over the N timed ones) go in `video`, the
      protocol of the Synthesia digest ("Summary": 1 warmup + 10 runs).

--band N (c3): one GPU's share when the frame is split into N bands of rows (the
      design's multi-GPU split): 720/N low-resolution rows plus a halo row on each
      side, timed alone.
--per-op FILE: one JSON line per launch kind of every op over the timed steps
      (op name; part: main = the op's own kernel, norm = a conv's separate norm
      pass, cache = its cache copy; kernel, launches, ms per launch, algorithmic
      TFLOP/s and GB/s) from the library's event profile.

Prints one JSON line: value = algorithmic conv TFLOP/s (2*Cin*Cout*27 FLOP per
output voxel of every conv) over the timed steps; plus output frames/s, the
dominant kernel's roofline (live HIP-event timing on the plan's stream), every
kernel's algorithmic rates and fraction of the roof that bounds it, the
host-delivery rate (c4: every clip's output copied to pinned host memory on a
second stream, bf16 and 8-bit; never the headline value), the phase-folded
decode's frames/s and executed MFMA rate (c4: fold_upsample) and the CPU
oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
HBM_PEAK_GBS = 8000.0
METRIC = "causal Conv3d decode TFLOP/s + output frames/s at 1440p, % of bf16 MFMA peak"


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def conv_flops_per_voxel(cin, cout, k=27):
    return 2.0 * cin * cout * k


def make_decoder(dev, synth, S, OMshapes):
    params = {}
    for i, (name, co, ci, kt, kh, kw, has_g) in enumerate(OMshapes):
        w = synth.bf16(synth.conv_weight(co, ci, kt, kh, kw, synth.seed(4, 10 + 3 * i))).to(dev)
        g = synth.gain(ci, synth.seed(4, 11 + 3 * i)).to(dev) if has_g else None
        params[name] = {"w": w, "g": g, "b": None}
    return params


def decoder_layer_list(c_latent=48, stages=((384, 2), (192, 2), (96, 1)), c_out=3, temporal_grow=None):
    """(name, cout, cin, kt, kh, kw, has_gain) -- the decoder's conv list
    (with a TemporalGrow's projection and temporal conv ahead of each stage)."""
    out = [("conv_in", stages[0][0], c_latent, 3, 3, 3, False)]
    cin = stages[0][0]
    for si, (c, _) in enumerate(stages):
        if temporal_grow:
            out.append(("s%d.tg.p" % si, cin, cin, 1, 1, 1, False))
            out.append(("s%d.tg.t" % si, cin, cin, 3, 1, 1, False))
        out.append(("s%d.up" % si, c, cin, 3, 3, 3, False))
        for r in range(2):
            out.append(("s%d.rb%d.c1" % (si, r), c, c, 3, 3, 3, True))
            out.append(("s%d.rb%d.c2" % (si, r), c, c, 3, 3, 3, True))
        cin = c
    out.append(("head", c_out, cin, 3, 3, 3, True))
    return out


def grown(n, first):
    return 2 * n - 1 if first else 2 * n


def c4_step_flops(t_lat, first, h=90, w=160, temporal_grow=None):
    """Algorithmic conv FLOP of one clip of t_lat latents."""
    f = 0.0
    t = t_lat
    f += conv_flops_per_voxel(48, 384) * t * h * w
    cin = 384
    for si, (c, up_t) in enumerate(((384, 2), (192, 2), (96, 1))):
        if temporal_grow:
            pos = h * w * (4 if temporal_grow == "after" else 1)
            t_g = grown(t, first) if up_t == 2 else t
            f += conv_flops_per_voxel(cin, cin, 1) * t * pos + conv_flops_per_voxel(cin, cin, 3) * t_g * pos
        h, w = 2 * h, 2 * w
        if up_t == 2:
            t = grown(t, first)
        f += conv_flops_per_voxel(cin, c) * t * h * w
        f += 4 * conv_flops_per_voxel(c, c) * t * h * w
        cin = c
    f += conv_flops_per_voxel(96, 3) * t * (2 * h) * (2 * w)
    return f, t


def folded_up_units(t_in, first, up_t):
    """MFMA work of one phase-folded upsampling 3x3x3 conv (replicate history, the
    default growth rule) for t_in input frames, in units of one spatial tap per
    output pixel (27 per frame unfolded).  Per output frame and temporal tap: 7
    (four folded offsets, a hi each, a lo for the three that sum several taps).
    A conv that doubles time groups the taps that read one source frame: 8 per
    group (every lo applied); on a later chunk its two history frames are one
    source frame (the previous window's last grown pair)."""
    if up_t == 1:
        return 21 * t_in
    ts = 1 if first else 0  # V[u] = X[(u + ts) // 2]
    t_v = 2 * t_in - ts

    def frame(zi):  # the source frame window frame zi holds
        if zi < 2:
            return ("x", 0) if first else ("previous",)
        return ("x", (zi - 2 + ts) >> 1)
    units = 0
    for t in range(t_v):
        z = [frame(t + k) for k in range(3)]
        units += 8 * (1 + (z[1] != z[0]) + (z[2] != z[1]))
    return units


def c4_up_flops(t_lat, first, h=90, w=160, grown_in_conv=True):
    """(algorithmic, executed-when-phase-folded) FLOP of the three upsampling convs
    (up_s = 2) of one clip; grown_in_conv False: the time growth happened before
    them (a TemporalGrow), so they see the grown frame count with up_t = 1."""
    f, ex, t, cin = 0.0, 0.0, t_lat, 384
    for c, up_t in ((384, 2), (192, 2), (96, 1)):
        h, w = 2 * h, 2 * w
        t_in = t
        if up_t == 2:
            t = grown(t, first)
        per_frame = conv_flops_per_voxel(cin, c) * h * w
        f += per_frame * t
        units = folded_up_units(t_in, first, up_t) if grown_in_conv else 21 * t
        ex += per_frame / 27.0 * units
        cin = c
    return f, ex


def setup_c4(dev, torch, synth, P, S, out_u8=False, temporal_grow=None, frame_batch=0, fold=False):
    lat_c, lat_t, lh, lw = 48, 91, 90, 160
    layers = decoder_layer_list(temporal_grow=temporal_grow)
    params = make_decoder(dev, synth, S, layers)
    ops = S.decoder_ops(params, out_u8=out_u8, temporal_grow=temporal_grow)
    g0 = next(i for i, o in enumerate(ops) if o.name == ("s2.tg.p" if temporal_grow else "s2.up"))
    plan = P.stack_plan(ops, lat_c, lh, lw, max_chunk_t=7, device=dev, batch_from=g0, frame_batch=frame_batch,
                        fold_upsample=fold)
    del params
    log("c4 plan: %d ops, state %.2f GB, plan device memory %.2f GB" % (
        len(ops), plan.state_bytes / 1e9, plan.device_bytes / 1e9))
    x = synth.bf16(synth.video(lat_c, lat_t, lh, lw, synth.seed(4, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().to(dev)
    del x
    sched = [7] + [6] * 14
    starts = [0]
    for n in sched[:-1]:
        starts.append(starts[-1] + n)
    clips = [(x_cl[s:s + n].contiguous(), s == 0) for s, n in zip(starts, sched)]
    ring = [torch.empty((25, 1440, 2560, 3), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    work = []
    for (xc, first), n in zip(clips, sched):
        fl, tout = c4_step_flops(n, first, temporal_grow=temporal_grow)
        ex = fl
        if fold and temporal_grow != "after":  # executed MFMA FLOP of the folded upsample convs
            up, up_ex = c4_up_flops(n, first, grown_in_conv=not temporal_grow)
            ex = fl - up + up_ex
        work.append((xc, first, fl, tout, ex))
    if temporal_grow:
        name = ("c4tg_decoder_bf16: latent 48x91x90x160 -> conv_in 48->384 -> 3 stages (384/192/96 ch; "
                "TemporalGrow [1x1x1 projection + causal 3x1x1 temporal conv, 2x time on non-first frames "
                "for stages 1-2] %s the nearest 2x spatial upsample, then conv; 2 residual blocks each) -> "
                "head 96->3 at 1440x2560; clips of 7+14x6 latents" % (
                    "before" if temporal_grow == "before" else "after"))
    else:
        name = ("c4_decoder_bf16: latent 48x91x90x160 -> conv_in 48->384 -> 3 stages "
                "(384/192/96 ch; nearest 2x space, 2x time on non-first frames for stages 1-2; "
                "2 residual blocks each) -> head 96->3 at 1440x2560; clips of 7+14x6 latents")
    desc = {"workload": name, "output": "3x361x1440x2560 bf16",
            "step": "one clip (24 output frames; 25 for the first)"}
    if fold:
        desc["fold_upsample"] = ("upsampling 3x3x3 convs phase-folded (hi/lo bf16 weights; 7/9 of their MFMA work, "
                                 "about 16/27 where time doubles)")
    if frame_batch:
        desc["frame_batch"] = "%d frames of the last stage's input through the last stage and the head" % frame_batch
    if temporal_grow or frame_batch:
        desc["plan_device_gb"] = round(plan.device_bytes / 1e9, 3)
    return plan, work, ring, desc


def setup_c3(dev, torch, synth, P, S, fold=False, band=1):
    """band > 1: one GPU's share when the frame is split into `band` bands of
    rows: 720/band low-resolution rows plus one halo row on each side, so that
    both convs' outputs over the band's own 2*720/band rows are exact."""
    cin, cmid, cout, h, w = 128, 96, 3, 720, 1280
    if band > 1:
        h = 720 // band + 2
    w1 = synth.bf16(synth.conv_weight(cmid, cin, 3, 3, 3, synth.seed(3, 10))).to(dev)
    w2 = synth.bf16(synth.conv_weight(cout, cmid, 3, 3, 3, synth.seed(3, 13))).to(dev)
    g2 = synth.gain(cmid, synth.seed(3, 14)).to(dev)
    plan = P.stack_plan(S.upstage_ops(cmid, cout, {"w": w1}, {"w": w2, "g": g2}), cin, h, w, max_chunk_t=4,
                        device=dev, fold_upsample=fold)
    pool = []
    for k in range(8):  # distinct input chunks, cycled (content does not change the time)
        x = synth.bf16(synth.video(cin, 4, h, w, synth.seed(3, 100 + k)))
        pool.append(x.permute(1, 2, 3, 0).contiguous().to(dev))
    sched = [1] + [4] * 90
    fl_up = conv_flops_per_voxel(cin, cmid) * (2 * h) * 2560
    fl_frame = fl_up + conv_flops_per_voxel(cmid, cout) * (2 * h) * 2560
    ex_frame = fl_frame - (2.0 / 9.0) * fl_up if fold else fl_frame
    work = []
    for i, n in enumerate(sched):
        work.append((pool[i % 8][:n], i == 0, fl_frame * n, n, ex_frame * n))
    ring = [torch.empty((4, 2 * h, 2 * w, 3), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    desc = {"workload": "c3_stage1440_bf16: 128x720x1280 -> nearest 2x -> conv 128->96 -> RMSNorm+SiLU -> "
                        "conv 96->3 at 1440x2560; 361 frames as 1+90x4 chunks with caches",
            "output": "3x361x1440x2560 bf16", "step": "one 4-frame chunk"}
    if band > 1:
        desc["band"] = {"of": band, "input_rows": h, "computed_rows": 2 * h, "own_rows": 2 * (h - 2),
                        "note": "one GPU's share of a frame split by rows (frames_per_s counts band frames; "
                                "the algorithmic FLOP are those of the computed rows)"}
    if fold:
        desc["fold_upsample"] = "the upsampling conv phase-folded (hi/lo bf16 weights, 7/9 of its MFMA work)"
    return plan, work, ring, desc


def setup_c2(dev, torch, synth, P, S):
    cin, cmid, cout, h, w, t_all = 256, 128, 128, 270, 480, 24
    w1 = synth.bf16(synth.conv_weight(cmid, cin, 3, 3, 3, synth.seed(2, 10))).to(dev)
    w2 = synth.bf16(synth.conv_weight(cout, cmid, 3, 3, 3, synth.seed(2, 13))).to(dev)
    g2 = synth.gain(cmid, synth.seed(2, 14)).to(dev)
    plan = P.stack_plan(S.upstage_ops(cmid, cout, {"w": w1}, {"w": w2, "g": g2}), cin, h, w, max_chunk_t=4,
                        device=dev)
    x = synth.bf16(synth.video(cin, t_all, h, w, synth.seed(2, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().to(dev)
    del x
    fl_frame = (conv_flops_per_voxel(cin, cmid) + conv_flops_per_voxel(cmid, cout)) * (2 * h) * (2 * w)
    work = [(x_cl[t:t + 4].contiguous(), t == 0, fl_frame * 4, 4, fl_frame * 4) for t in range(0, t_all, 4)]
    ring = [torch.empty((4, 2 * h, 2 * w, cout), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    desc = {"workload": "c2_stage1080_bf16: 256x24x270x480 -> nearest 2x -> conv 256->128 -> RMSNorm+SiLU -> "
                        "conv 128->128 at 540x960; 4-frame chunks with caches",
            "output": "128x24x540x960 bf16", "step": "one 4-frame chunk"}
    return plan, work, ring, desc


def setup_c1(dev, torch, synth, P, S):
    c, h, w, t_all = 128, 90, 160, 16
    p = [{"w": synth.bf16(synth.conv_weight(c, c, 3, 3, 3, synth.seed(1, 10 + 3 * i))).to(dev),
          "g": synth.gain(c, synth.seed(1, 11 + 3 * i)).to(dev)} for i in range(2)]
    plan = P.stack_plan(S.resblock_ops(c, p[0], p[1]), c, h, w, max_chunk_t=4, device=dev)
    x = synth.bf16(synth.video(c, t_all, h, w, synth.seed(1, 1)))
    x_cl = x.permute(1, 2, 3, 0).contiguous().to(dev)
    del x
    fl_frame = 2 * conv_flops_per_voxel(c, c) * h * w
    work = [(x_cl[t:t + 4].contiguous(), t == 0, fl_frame * 4, 4, fl_frame * 4) for t in range(0, t_all, 4)]
    ring = [torch.empty((4, h, w, c), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    desc = {"workload": "c1_resblock_bf16: x 128x16x90x160 -> x + conv 128->128(act(conv 128->128(act(x)))), "
                        "act = RMSNorm+SiLU; 4-frame chunks with caches",
            "output": "128x16x90x160 bf16", "step": "one 4-frame chunk"}
    return plan, work, ring, desc


def encoder_layer_list(c_in=8, stages=((384, 2), (192, 2), (96, 1)), c_latent=48):
    """(name, cout, cin, kt, kh, kw, has_gain, stride_s, stride_t) -- the
    encoder's conv list: the decoder's stages from the last, each [two residual
    blocks, a conv with spatial stride 2 and the stage's temporal factor as
    temporal stride] between a stride-2 conv_in and conv_out."""
    widths = [stages[0][0]] + [c for c, _ in stages]
    out = [("conv_in", stages[-1][0], c_in, 3, 3, 3, False, 2, 1)]
    n = len(stages)
    for ei in range(n):
        c, f = stages[n - 1 - ei]
        for r in range(2):
            out.append(("e%d.rb%d.c1" % (ei, r), c, c, 3, 3, 3, True, 1, 1))
            out.append(("e%d.rb%d.c2" % (ei, r), c, c, 3, 3, 3, True, 1, 1))
        out.append(("e%d.down" % ei, widths[n - 1 - ei], c, 3, 3, 3, False, 2, f))
    out.append(("conv_out", c_latent, widths[0], 3, 3, 3, True, 1, 1))
    return out


def halved(n, first):
    """Outputs of a temporal stride of 2 with the first frame on its own."""
    return (n + 1) // 2 if first else n // 2


def e4_step_flops(t_in, first, h=1440, w=2560, c_pix=3):
    """Algorithmic conv FLOP of one encoder chunk of t_in frames (conv_in with
    its c_pix real channels) and the latents it yields."""
    f, t = 0.0, t_in
    h, w = (h + 1) // 2, (w + 1) // 2
    f += conv_flops_per_voxel(c_pix, 96) * t * h * w
    for c, c_next, st in ((96, 192, 1), (192, 384, 2), (384, 384, 2)):
        f += 4 * conv_flops_per_voxel(c, c) * t * h * w
        h, w = (h + 1) // 2, (w + 1) // 2
        if st == 2:
            t = halved(t, first)
        f += conv_flops_per_voxel(c, c_next) * t * h * w
    f += conv_flops_per_voxel(384, 48) * t * h * w
    return f, t


def setup_e4(dev, torch, synth, P, S):
    h, w, c_pix, c_in = 1440, 2560, 3, 8
    params = {}
    for i, (name, co, ci, kt, kh, kw, has_g, _, _) in enumerate(encoder_layer_list(c_in=c_pix)):
        wt = synth.bf16(synth.conv_weight(co, ci, kt, kh, kw, synth.seed(6, 10 + 3 * i)))
        if name == "conv_in":  # the pixels' zero channels get zero weights
            wp = torch.zeros((co, c_in, kt, kh, kw), dtype=wt.dtype)
            wp[:, :c_pix] = wt
            wt = wp
        params[name] = {"w": wt.to(dev), "b": None,
                        "g": synth.gain(ci, synth.seed(6, 11 + 3 * i)).to(dev) if has_g else None}
    ops = S.encoder_ops(params)
    for o in ops:
        o.tpad = S.C.TPAD_ZERO  # zero history: the ReAE rule
    plan = P.stack_plan(ops, c_in, h, w, max_chunk_t=25, device=dev)
    del params
    log("e4 plan: %d ops, state %.2f GB, plan device memory %.2f GB" % (
        len(ops), plan.state_bytes / 1e9, plan.device_bytes / 1e9))
    pool = []
    for k, n in enumerate((25, 24, 24)):  # distinct chunks, cycled (content does not change the time)
        x = synth.bf16(synth.video(c_pix, n, h, w, synth.seed(6, 100 + k)))
        xc = torch.zeros((n, h, w, c_in), dtype=torch.bfloat16, device=dev)
        xc[..., :c_pix] = x.permute(1, 2, 3, 0).to(dev)
        del x
        pool.append(xc)
    sched = [25] + [24] * 14
    work = []
    for i, n in enumerate(sched):
        fl, lat = e4_step_flops(n, i == 0)
        xc = pool[0] if i == 0 else pool[1 + i % 2]
        work.append((xc, i == 0, fl, lat, fl))
    ring = [torch.empty((7, 90, 160, 48), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    desc = {"workload": "e4_encoder_bf16: pixels 3x361x1440x2560 (zero-padded to 8 channels) -> conv_in 3->96 "
                        "stride 2 -> 3 stages (96/192/384 ch; 2 residual blocks, then conv with spatial stride 2, "
                        "temporal stride 1/2/2) -> act -> conv 384->48 at 90x160; chunks of 25+14x24 frames, "
                        "zero history",
            "output": "48x91x90x160 bf16", "step": "one chunk (24 input frames; 25 for the first)",
            "frames": "frames_per_s counts input frames"}
    return plan, work, ring, desc


VIDEO_STEPS = {"c4": 15, "c4tg": 15, "c3": 91, "c2": 6, "c1": 4, "e4": 15}


def video_times(torch, plan, work, ring, runs, warmup=1):
    """Whole videos decoded back to back (work holds one video's steps in
    order, its first step with the first-chunk rule): `warmup` untimed, then
    `runs` timed by events around each video; seconds per video, sorted."""
    states = [plan.new_state(), plan.new_state()]
    cur = [0]

    def video():
        for i, (xc, first, fl, tout, ex) in enumerate(work):
            if first:
                plan.reset(states[cur[0]])
            plan.forward_chunk(xc, states[cur[0]], states[1 - cur[0]], y=ring[i % 2][:tout])
            cur[0] = 1 - cur[0]

    for _ in range(warmup):
        video()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(runs + 1)]
    marks[0].record()
    for r in range(runs):
        video()
        marks[r + 1].record()
    torch.cuda.synchronize()
    return sorted(marks[r].elapsed_time(marks[r + 1]) * 1e-3 for r in range(runs))


def _counter_record(kernel_name, workload=None):
    """The fields of `kernel_name`'s record in a committed PMC summary in
    profiles/ (a "traffic_record:" line; one that names a workload counts for
    that workload only), or None when no record exists or a source it names
    (comma-separated: the kernel, the op list that sets its launches, the build
    script that holds its compiler flags) changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith("traffic_record:"):
                continue
            kv = dict(item.split("=", 1) for item in line.split()[1:])
            if kv.get("kernel") != kernel_name:
                continue
            if "workload" in kv and workload is not None and kv["workload"] != workload:
                continue
            srcs = [os.path.join(ROOT, f) for f in kv["source"].split(",")]
            if not all(os.path.exists(f) for f in srcs):
                continue
            h = hashlib.sha256()
            for f in srcs:
                h.update(open(f, "rb").read())
            if h.hexdigest()[:16] == kv.get("source_sha256_16"):
                return kv
    return None


def recorded_traffic(kernel_name, workload=None):
    """HBM bytes per launch of `kernel_name` in `workload` (FETCH_SIZE +
    WRITE_SIZE runs, copy-calibrated), or None (see _counter_record)."""
    kv = _counter_record(kernel_name, workload)
    return float(kv["bytes_per_launch"]) if kv else None


def recorded_clock(kernel_name, workload=None):
    """Mean shader clock in GHz over `kernel_name`'s dispatches in the counter
    run (GRBM_GUI_ACTIVE per XCD / dispatch time), or None."""
    kv = _counter_record(kernel_name, workload)
    return float(kv["clock_ghz"]) if kv and "clock_ghz" in kv else None


def timed_decode(torch, plan, work, ring, steps, warmup, before_timed=None):
    """Decode `warmup` clips untimed, then time `steps` clips (inputs resident,
    outputs to the device ring).  Returns (seconds, algorithmic FLOP, frames,
    executed MFMA FLOP, sorted per-step GPU ms)."""
    states = [plan.new_state(), plan.new_state()]
    cur = [0]

    def step(i):
        xc, first, fl, tout, ex = work[i % len(work)]
        if first:
            plan.reset(states[cur[0]])
        a, b = states[cur[0]], states[1 - cur[0]]
        plan.forward_chunk(xc, a, b, y=ring[i % 2][:tout])
        cur[0] = 1 - cur[0]
        return fl, tout, ex

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    if before_timed:
        before_timed()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    flops, frames, executed = 0.0, 0, 0.0
    marks[0].record()
    for i in range(warmup, warmup + steps):
        fl, tout, ex = step(i)
        marks[i - warmup + 1].record()
        flops += fl
        executed += ex
        frames += tout
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    step_ms = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(steps))
    return dt, flops, frames, executed, step_ms


def delivery_rate(torch, plan, work, steps, warmup, dev):
    """Frames/s of the decode with every clip's output copied to pinned host
    memory on a second stream (the SwiftVR page's overlap of output transfer with
    compute, "Other Engineering Optimizations"): device output ring of two,
    pinned host ring of two, the copy of clip i overlapping the decode of clip
    i+1; timed to the end of the last copy.  Returns (frames/s, host GB/s of
    the copies alone, bytes per clip)."""
    copy_stream = torch.cuda.Stream(device=dev)
    comp = torch.cuda.current_stream(dev)
    shape = (25, 1440, 2560, 3)
    ring = [torch.empty(shape, dtype=plan.out_dtype, device=dev) for _ in range(2)]
    host = [torch.empty(shape, dtype=plan.out_dtype, pin_memory=True) for _ in range(2)]
    produced = [torch.cuda.Event() for _ in range(2)]
    copied = [torch.cuda.Event() for _ in range(2)]
    timing = []  # (start, end) events of every timed copy, read after the run
    states = [plan.new_state(), plan.new_state()]
    cur = [0]
    nbytes = [0]

    def clip(i, timed):
        xc, first, fl, tout, _ = work[i % len(work)]
        k = i % 2
        if i >= 2:
            comp.wait_event(copied[k])  # the copy out of this ring slot is done
        if first:
            plan.reset(states[cur[0]])
        plan.forward_chunk(xc, states[cur[0]], states[1 - cur[0]], y=ring[k][:tout])
        cur[0] = 1 - cur[0]
        produced[k].record(comp)
        copy_stream.wait_event(produced[k])
        with torch.cuda.stream(copy_stream):
            if timed:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ev[0].record(copy_stream)
            host[k][:tout].copy_(ring[k][:tout], non_blocking=True)
            copied[k].record(copy_stream)
            if timed:
                ev[1].record(copy_stream)
                timing.append(ev)
                nbytes[0] += ring[k][:tout].numel() * ring[k].element_size()
        return tout

    for i in range(warmup):
        clip(i, False)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    frames = 0
    for i in range(warmup, warmup + steps):
        frames += clip(i, True)
    torch.cuda.synchronize(dev)
    dt = time.perf_counter() - t0
    copy_ms = sum(a.elapsed_time(b) for a, b in timing)
    return frames / dt, nbytes[0] / (copy_ms * 1e-3) / 1e9, nbytes[0] / steps


def cpu_baseline(workload, temporal_grow=None):
    """The fp64 oracle, as it stands, on a bounded crop of the same workload."""
    import numpy as np

    from causal_convolution_x3x3_amd import synth
    from oracle import model as OM
    from oracle import oracle as O

    O.build()
    threads = O.default_threads()
    if workload in ("c4", "c4tg"):
        lt, lh, lw = 3, 6, 20  # about 15 s on 16 host threads
        shapes = OM.decoder_layer_shapes(temporal_grow=temporal_grow)
        params = {}
        for i, (name, co, ci, kt, kh, kw, has_g) in enumerate(shapes):
            params[name] = {"w": synth.conv_weight(co, ci, kt, kh, kw, synth.seed(4, 10 + 3 * i)).double().numpy(),
                            "g": synth.gain(ci, synth.seed(4, 11 + 3 * i)).double().numpy() if has_g else None,
                            "b": None}
        x = synth.video(48, lt, lh, lw, synth.seed(4, 1)).double().numpy()
        dec = OM.Decoder(params, nthreads=threads, temporal_grow=temporal_grow)
        t0 = time.perf_counter()
        y = dec.step(x)
        dt = time.perf_counter() - t0
        fl, tout = c4_step_flops(lt, True, lh, lw, temporal_grow=temporal_grow)
        sample = ("whole decoder, one first clip of %d latents on a %dx%d latent crop "
                  "(-> %d frames of %dx%d), fp64, %d threads" % (lt, lh, lw, y.shape[1], y.shape[2], y.shape[3],
                                                                threads))
        frames_per_s = y.shape[1] / dt * (y.shape[2] * y.shape[3]) / (1440 * 2560)
    elif workload == "c2":
        cin, cmid, rows, cols, lt = 256, 128, 16, 480, 4  # about 15 s on 16 host threads
        w1 = synth.conv_weight(cmid, cin, 3, 3, 3, synth.seed(2, 10)).double().numpy()
        w2 = synth.conv_weight(cmid, cmid, 3, 3, 3, synth.seed(2, 13)).double().numpy()
        g2 = synth.gain(cmid, synth.seed(2, 14)).double().numpy()
        st = OM.UpStage({"w": w1, "b": None}, {"w": w2, "b": None, "g": g2}, nthreads=threads)
        x = synth.video(cin, lt, rows, cols, synth.seed(2, 1)).double().numpy()
        t0 = time.perf_counter()
        y = st.step(x)
        dt = time.perf_counter() - t0
        fl = (conv_flops_per_voxel(cin, cmid) + conv_flops_per_voxel(cmid, cmid)) * y.shape[1] * y.shape[2] * y.shape[3]
        sample = "1080p-class stage on one %d-frame chunk of a %dx%d crop (-> %dx%d), fp64, %d threads" % (
            lt, rows, cols, y.shape[2], y.shape[3], threads)
        frames_per_s = lt / dt * (y.shape[2] * y.shape[3]) / (540 * 960)
    elif workload == "e4":
        lt, rows, cols = 5, 96, 480  # about 11 s on 16 host threads
        shapes = OM.encoder_layer_shapes()
        params = {}
        for i, (name, co, ci, kt, kh, kw, has_g, _, _) in enumerate(shapes):
            params[name] = {"w": synth.conv_weight(co, ci, kt, kh, kw, synth.seed(6, 10 + 3 * i)).double().numpy(),
                            "g": synth.gain(ci, synth.seed(6, 11 + 3 * i)).double().numpy() if has_g else None,
                            "b": None}
        x = synth.video(3, lt, rows, cols, synth.seed(6, 100)).double().numpy()
        enc = OM.Encoder(params, nthreads=threads)
        t0 = time.perf_counter()
        y = enc.step(x)
        dt = time.perf_counter() - t0
        fl, _ = e4_step_flops(lt, True, rows, cols)
        sample = ("whole encoder, one first chunk of %d frames on a %dx%d pixel crop (-> %d latents of %dx%d), "
                  "fp64, %d threads" % (lt, rows, cols, y.shape[1], y.shape[2], y.shape[3], threads))
        frames_per_s = lt / dt * (rows * cols) / (1440 * 2560)
    elif workload == "c1":
        c, rows, cols, lt = 128, 90, 160, 4  # one whole 4-frame chunk, about 10 s on 16 host threads
        p = [{"w": synth.conv_weight(c, c, 3, 3, 3, synth.seed(1, 10 + 3 * i)).double().numpy(), "b": None,
              "g": synth.gain(c, synth.seed(1, 11 + 3 * i)).double().numpy()} for i in range(2)]
        blk = OM.ResBlock(p[0], p[1], nthreads=threads)
        x = synth.video(c, lt, rows, cols, synth.seed(1, 1)).double().numpy()
        t0 = time.perf_counter()
        y = blk.step(x)
        dt = time.perf_counter() - t0
        fl = 2 * conv_flops_per_voxel(c, c) * lt * rows * cols
        sample = "residual block on its first 4-frame chunk at the full 90x160, fp64, %d threads" % threads
        frames_per_s = lt / dt
    else:
        cin, cmid, rows, cols, lt = 128, 96, 32, 320, 4  # about 15 s on 16 host threads
        w1 = synth.conv_weight(cmid, cin, 3, 3, 3, synth.seed(3, 10)).double().numpy()
        w2 = synth.conv_weight(3, cmid, 3, 3, 3, synth.seed(3, 13)).double().numpy()
        g2 = synth.gain(cmid, synth.seed(3, 14)).double().numpy()
        st = OM.UpStage({"w": w1, "b": None}, {"w": w2, "b": None, "g": g2}, nthreads=threads)
        x = synth.video(cin, lt, rows, cols, synth.seed(3, 100)).double().numpy()
        t0 = time.perf_counter()
        y = st.step(x)
        dt = time.perf_counter() - t0
        fl = (conv_flops_per_voxel(cin, cmid) + conv_flops_per_voxel(cmid, 3)) * y.shape[1] * y.shape[2] * y.shape[3]
        sample = "1440p stage on one %d-frame chunk of a %dx%d crop (-> %dx%d), fp64, %d threads" % (
            lt, rows, cols, y.shape[2], y.shape[3], threads)
        frames_per_s = lt / dt * (y.shape[2] * y.shape[3]) / (1440 * 2560)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "sample": sample, "seconds": round(dt, 3),
            "frames_per_s_equiv": frames_per_s}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=45)  # c4: three passes over the 15-clip video
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", choices=["c4", "c4tg", "c3", "c2", "c1", "e4"], default="c4")
    ap.add_argument("--tg-order", choices=["before", "after"], default="before",
                    help="c4tg: TemporalGrow before (reordered) or after (original) the spatial upsample")
    ap.add_argument("--frame-batch", type=int, default=0,
                    help="c4/c4tg: run the last stage and the head over batches of this many frames (0: whole clips)")
    ap.add_argument("--fold-upsample", action="store_true",
                    help="phase-folded upsampling convs (value stays algorithmic; executed FLOP reported)")
    ap.add_argument("--videos", type=int, default=10,
                    help="whole videos timed one by one after one untimed (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-delivery", action="store_true",
                    help="skip the host-delivery measurement (c4: output copied to pinned host memory)")
    ap.add_argument("--band", type=int, default=1,
                    help="c3: one GPU's share of the frame split into this many bands of rows (halo included)")
    ap.add_argument("--per-op", metavar="FILE", default=None,
                    help="write the timed steps' per-op event profile to FILE (one JSON line per op and part)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this decode path has no multi-GPU mode; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.band != 1 and (args.workload != "c3" or args.band < 1 or 720 % args.band):
        print("--band applies to --workload c3 and must divide 720", file=sys.stderr)
        sys.exit(2)

    import torch

    from causal_convolution_x3x3_amd import capi as C
    from causal_convolution_x3x3_amd import plan as P
    from causal_convolution_x3x3_amd import stacks as S
    from causal_convolution_x3x3_amd import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    C.lib()
    tg = args.tg_order if args.workload == "c4tg" else None
    if args.workload == "c3":
        plan, work, ring, desc = setup_c3(dev, torch, synth, P, S, fold=args.fold_upsample, band=args.band)
    elif args.workload == "c2":
        plan, work, ring, desc = setup_c2(dev, torch, synth, P, S)
    elif args.workload == "c1":
        plan, work, ring, desc = setup_c1(dev, torch, synth, P, S)
    elif args.workload == "e4":
        plan, work, ring, desc = setup_e4(dev, torch, synth, P, S)
    else:
        plan, work, ring, desc = setup_c4(dev, torch, synth, P, S, temporal_grow=tg, frame_batch=args.frame_batch,
                                          fold=args.fold_upsample)
    log("warmup %d steps, timing %d steps" % (args.warmup, args.steps))
    dt, flops, frames, executed, step_ms = timed_decode(
        torch, plan, work, ring, args.steps, args.warmup,
        before_timed=lambda: C.check(C.lib().cc3d_profile_enable(plan._h, 1), "profile_enable"))
    log("timed %.3f s" % dt)
    in_frames = None
    if args.workload == "e4":  # an encoder's rate is in input frames; tout counts latents
        in_frames = sum(work[i % len(work)][0].shape[0] for i in range(args.warmup, args.warmup + args.steps))

    # per-kernel event totals over the timed region
    import ctypes
    kern = {}
    per_op = []
    for op in range(C.lib().cc3d_plan_num_ops(plan._h)):
        for part in range(3):
            pr = C.OpProfile()
            C.check(C.lib().cc3d_profile_read(plan._h, op, part, ctypes.byref(pr)), "profile_read")
            if pr.launches == 0:
                continue
            ms = pr.total_ms / pr.launches
            per_op.append({"op": op, "name": plan.op_names[op] if op < len(plan.op_names) else "op%d" % op,
                           "part": ("main", "norm", "cache")[part], "kernel": pr.kernel.decode(),
                           "launches": pr.launches, "ms_per_launch": round(ms, 4),
                           "tflops": round(pr.flops / pr.launches / (ms * 1e-3) / 1e12, 1),
                           "gbs": round(pr.bytes / pr.launches / (ms * 1e-3) / 1e9, 1)})
            k = kern.setdefault(pr.kernel.decode(), {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
            k["launches"] += pr.launches
            k["ms"] += pr.total_ms
            k["flops"] += pr.flops
            k["bytes"] += pr.bytes
    C.check(C.lib().cc3d_profile_enable(plan._h, 0), "profile_enable")
    if args.per_op:
        with open(args.per_op, "w") as f:
            for row in per_op:
                f.write(json.dumps(row) + "\n")
    # MFMA work a kernel executes: the definition's count, except for the
    # phase-folded upsample convs, which execute fewer MFMAs -- all of the
    # timed steps' difference between algorithmic and executed FLOP is theirs
    saved = flops - executed
    for name, k in kern.items():
        k["exec_flops"] = k["flops"] - saved if (saved > 0 and "phase" in name) else k["flops"]
    total_kernel_ms = sum(k["ms"] for k in kern.values())
    dom_name, dom = max(kern.items(), key=lambda kv: kv[1]["ms"])
    avg_ms = dom["ms"] / dom["launches"]
    if dom["flops"] > 0:
        # executed FLOP: a folded kernel is never priced at its 27-tap equivalent
        achieved = dom["exec_flops"] / dom["launches"] / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = dom["bytes"] / dom["launches"] / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    # counter records are per workload shape (none for a band)
    wl_key = args.workload + ("_" + tg if tg else "") + ("_band%d" % args.band if args.band > 1 else "")
    clock = recorded_clock(dom_name, wl_key)
    if clock and roof["bound"] == "mfma":
        # the part runs below its 2.4 GHz peak clock under this load (power): the
        # same rate against the dense peak at the clock the counters saw
        roof["clock_ghz"] = clock
        roof["peak_at_clock"] = round(MFMA_BF16_PEAK_TFLOPS * clock / 2.4, 1)
        roof["frac_at_clock"] = round(achieved / roof["peak_at_clock"], 4)
    if dom["exec_flops"] != dom["flops"]:
        roof["flop_basis"] = "the folded kernel's own MFMA work (27-tap equivalent: %.1f TFLOP/s)" % (
            dom["flops"] / dom["launches"] / (avg_ms * 1e-3) / 1e12)
    roof.update({"traffic": recorded_traffic(dom_name, wl_key), "kernel": dom_name, "launches": dom["launches"],
                 "avg_launch_ms": round(avg_ms, 4), "share_of_kernel_time": round(dom["ms"] / total_kernel_ms, 3)})
    # per kernel: algorithmic rates and the fraction of the roof that bounds it
    # (MFMA where its FLOP per algorithmic byte reach the ridge point, else HBM)
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    per_kernel = {}
    for name, k in sorted(kern.items(), key=lambda kv: -kv[1]["ms"]):
        e = {"ms": round(k["ms"], 3), "launches": k["launches"]}
        tf = k["flops"] / (k["ms"] * 1e-3) / 1e12
        tf_ex = k["exec_flops"] / (k["ms"] * 1e-3) / 1e12
        gbs = k["bytes"] / (k["ms"] * 1e-3) / 1e9
        if k["flops"] > 0:
            e["tflops"] = round(tf, 1)
            if k["exec_flops"] != k["flops"]:
                e["executed_tflops"] = round(tf_ex, 1)
        e["gbs"] = round(gbs, 1)
        if k["flops"] > 0 and k["flops"] >= ridge * k["bytes"]:
            e["bound"], e["frac"] = "mfma", round(tf_ex / MFMA_BF16_PEAK_TFLOPS, 4)
        else:
            e["bound"], e["frac"] = "hbm", round(gbs / HBM_PEAK_GBS, 4)
        per_kernel[name] = e

    value = flops / dt / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dt / args.steps * 1e3, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": desc, "frames_per_s": round((in_frames if in_frames is not None else frames) / dt, 2),
        "mfma_frac": round(executed / dt / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": roof, "kernels": per_kernel,
        # per-step GPU time between events on the stream (the first clip is the
        # 25-frame one only when it falls in the timed steps)
        "step_ms": {"min": round(step_ms[0], 3), "mean": round(sum(step_ms) / len(step_ms), 3),
                    "p99": round(step_ms[min(len(step_ms) - 1, int(0.99 * len(step_ms)))], 3)},
    }
    if in_frames is not None:
        out["latents_per_s"] = round(frames / dt, 2)
    if args.fold_upsample:
        out["executed_tflops"] = round(executed / dt / 1e12, 2)
    if args.videos > 0:
        # seconds per whole video (the work list holds one video's steps in order)
        n_video = VIDEO_STEPS[args.workload]
        assert len(work) == n_video
        log("%d whole videos (%d steps each) after one untimed" % (args.videos, n_video))
        vt = video_times(torch, plan, work, ring, args.videos)
        v_frames = sum((wk[0].shape[0] if in_frames is not None else wk[3]) for wk in work)
        v_flops = sum(wk[2] for wk in work)
        mean = sum(vt) / len(vt)
        out["video"] = {"frames": v_frames, "steps": n_video, "warmup": 1, "runs": len(vt),
                        "s_min": round(vt[0], 4), "s_mean": round(mean, 4),
                        "s_p99": round(vt[min(len(vt) - 1, int(0.99 * len(vt)))], 4),
                        "frames_per_s": round(v_frames / mean, 2), "tflops": round(v_flops / mean / 1e12, 2)}
    if args.workload == "c4" and not args.no_delivery and not args.frame_batch and not args.fold_upsample:
        # Host delivery: the same decode with every clip's RGB copied to pinned host
        # memory, overlapped with the next clip; bf16 output, then 8-bit codes.
        # PCIe-inclusive, so never the headline value.
        deliv = {}
        out_dtype_names = {False: "bf16", True: "uint8"}
        for u8 in (False, True):
            if u8:
                del plan
                torch.cuda.empty_cache()
                plan, work, ring, _ = setup_c4(dev, torch, synth, P, S, out_u8=True)
            log("delivery to pinned host memory, %s output" % out_dtype_names[u8])
            fps, gbs, per_clip = delivery_rate(torch, plan, work, args.steps, args.warmup, dev)
            deliv[out_dtype_names[u8]] = {"frames_per_s": round(fps, 2), "copy_gbs": round(gbs, 1),
                                          "bytes_per_clip": per_clip}
        out["delivery"] = deliv
        # The same decode with the upsampling convs phase-folded (7/9 of their MFMA
        # work, results equal to the definition up to fp32 rounding): frames/s and
        # the MFMA work actually done; the headline value stays the exact path's.
        del plan
        torch.cuda.empty_cache()
        plan, work, ring, _ = setup_c4(dev, torch, synth, P, S, fold=True)
        log("phase-folded upsample convs")
        fdt, _, fframes, fexec, fstep = timed_decode(torch, plan, work, ring, args.steps, args.warmup)
        out["fold_upsample"] = {"frames_per_s": round(fframes / fdt, 2), "ms_per_step": round(fdt / args.steps * 1e3, 3),
                                "executed_tflops": round(fexec / fdt / 1e12, 2),
                                "mfma_frac": round(fexec / fdt / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        out["cpu_baseline"] = cpu_baseline(args.workload, tg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
