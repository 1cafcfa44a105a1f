"""Op lists for the decoder blocks run by the stack runner.

The pages name the decoder's pieces -- per-layer causal state, nearest 2x
upsampling followed by a spatial conv, growth of the frame count (LightX2V blog,
"SwiftVR Inference Optimization ...", sections "From Pixels to Latents and Back",
"TemporalGrow: Compute Before Spatial Upsampling") -- but no layer list; these
are the synthetic blocks built from them.  act = SiLU(RMSNorm(.)) is always
produced by the op that writes its input (fused into the conv when one
workgroup holds all output channels), and is computed once at the lower
resolution when an upsample follows: it works per position, so it commutes with
nearest upsampling.

Parameter dicts hold device tensors: ``w`` [Cout][Cin][kt][kh][kw], ``b``
[Cout] float32 or None, ``g`` [Cin] float32 (the RMSNorm gain of the conv's
input) or None.
"""
from __future__ import annotations

from typing import Dict, List

from . import capi as C
from .plan import Op

X, Y = C.SLOT_X, C.SLOT_Y
NONE = C.SLOT_NONE


def resblock_ops(c: int, p1: Dict, p2: Dict, src: int = X, out: int = Y, first_tmp: int = 3,
                 next_gain=None, act_out: int = NONE) -> List[Op]:
    """y = x + conv2(act2(conv1(act1(x)))); x in ``src``.  Uses slots
    first_tmp (act1 x) and first_tmp+1 (act2 of conv1).  With ``next_gain`` the
    last conv also stores act(y) for what follows into ``act_out``."""
    a1, a2 = first_tmp, first_tmp + 1
    return [
        Op(kind=C.OP_NORM_ACT, src=src, act_out=a1, gamma=p1["g"], name="rb.act1"),
        Op(cout=c, w=p1["w"], bias=p1.get("b"), src=a1, act_out=a2, gamma=p2["g"], name="rb.conv1"),
        Op(cout=c, w=p2["w"], bias=p2.get("b"), src=a2, res=src, out=out,
           act_out=act_out if next_gain is not None else NONE, gamma=next_gain, name="rb.conv2"),
    ]


def upstage_ops(c_mid: int, c_out: int, p1: Dict, p2: Dict) -> List[Op]:
    """conv2(act(conv1(nearest_up2(x)))) -- conv1 reads the upsampled input
    through its operand load; its epilogue stores act for conv2."""
    return [
        Op(cout=c_mid, w=p1["w"], bias=p1.get("b"), up_s=2, src=X, act_out=3, gamma=p2["g"], name="up.conv1"),
        Op(cout=c_out, w=p2["w"], bias=p2.get("b"), src=3, out=Y, name="up.conv2"),
    ]


DECODER_STAGES = ((384, 2), (192, 2), (96, 1))


TG_ORDERS = (None, "before", "after")


def temporal_grow_ops(c: int, p_proj: Dict, p_t: Dict, factor: int, src: int, p_slot: int, out: int,
                      up_s: int = 1, name: str = "tg") -> List[Op]:
    """TemporalGrow (SwiftVR page, "TemporalGrow: Compute Before Spatial
    Upsampling"): a 1x1x1 projection, then a causal 3x1x1 temporal conv that
    reads the projection grown in time (nearest 2x when ``factor`` is 2).  Both
    work per position.  ``up_s`` = 2 makes the projection read the nearest-
    upsampled input, so the block runs on the upsampled positions."""
    return [
        Op(cout=c, w=p_proj["w"], bias=p_proj.get("b"), up_s=up_s, src=src, out=p_slot, name=name + ".p"),
        Op(cout=c, w=p_t["w"], bias=p_t.get("b"), up_t=factor, src=p_slot, out=out, name=name + ".t"),
    ]


def decoder_ops(params: Dict[str, Dict], stages=DECODER_STAGES, c_out: int = 3,
                unique_slots: bool = False, out_u8: bool = False, temporal_grow=None) -> List[Op]:
    """conv_in -> per stage [nearest up (2x space, 2x time on non-first frames
    when the stage's factor is 2) + conv, two residual blocks] -> head (act at low
    resolution, nearest 2x, conv to c_out).

    ``temporal_grow`` = "before" or "after": each stage's time growth moves into
    a TemporalGrow (params "s<i>.tg.p" [C][C][1][1][1], "s<i>.tg.t"
    [C][C][3][1][1]) on the stage input, run at the input size ahead of the
    upsample conv ("before", the reordered decoder) or on the upsampled
    positions between the upsample and the spatial conv ("after", the original
    order).  The two give bitwise the same TemporalGrow output.

    Slots per stage s (base = 3 + 5 s): raw A, raw B (the residual stream
    alternates between them), act A, act B, inner act.  Slot 3 + 5*len(stages)
    holds conv_in's output; slots 4 + 5*len(stages) + 2 s and the next hold a
    stage's TemporalGrow projection and output.  ``unique_slots`` gives every
    tensor a slot of its own instead (same ops and kernels; every layer's input
    and output stay readable after a chunk, for layer-wise checks).  ``out_u8``:
    the head stores 8-bit RGB codes instead of bf16."""
    if temporal_grow not in TG_ORDERS:
        raise ValueError("temporal_grow must be one of %r" % (TG_ORDERS,))
    nxt = [3]

    def slot(fixed):
        if not unique_slots:
            return fixed
        nxt[0] += 1
        return nxt[0] - 1

    ops: List[Op] = []
    h0 = slot(3 + 5 * len(stages))
    ops.append(Op(cout=stages[0][0], w=params["conv_in"]["w"], bias=params["conv_in"].get("b"), src=X,
                  out=h0, name="conv_in"))
    prev_raw, last_act = h0, NONE
    c_in = stages[0][0]
    for si, (c, up_t) in enumerate(stages):
        base = 3 + 5 * si
        raw_fixed = [base, base + 1]
        act_fixed = [base + 2, base + 3]
        rb = [(params["s%d.rb%d.c1" % (si, r)], params["s%d.rb%d.c2" % (si, r)]) for r in range(2)]
        up = params["s%d.up" % si]
        up_s_conv, up_t_conv = 2, up_t
        if temporal_grow:
            tg_base = 4 + 5 * len(stages) + 2 * si
            tg_p, tg_q = slot(tg_base), slot(tg_base + 1)
            tg_up = 2 if temporal_grow == "after" else 1
            ops += temporal_grow_ops(c_in, params["s%d.tg.p" % si], params["s%d.tg.t" % si], up_t, prev_raw,
                                     tg_p, tg_q, up_s=tg_up, name="s%d.tg" % si)
            prev_raw = tg_q
            up_s_conv, up_t_conv = 2 // tg_up, 1
        raw_cur, act_cur = slot(raw_fixed[0]), slot(act_fixed[0])
        # up conv: stores the raw result (residual of block 0) and act for block 0's conv1
        ops.append(Op(cout=c, w=up["w"], bias=up.get("b"), up_s=up_s_conv, up_t=up_t_conv, src=prev_raw,
                      out=raw_cur, act_out=act_cur, gamma=rb[0][0]["g"], name="s%d.up" % si))
        cur = 0
        for r in range(2):
            p1, p2 = rb[r]
            inner = slot(base + 4)
            ops.append(Op(cout=c, w=p1["w"], bias=p1.get("b"), src=act_cur, act_out=inner, gamma=p2["g"],
                          name="s%d.rb%d.c1" % (si, r)))
            # block 0 hands act(y) to block 1; the last block of the last stage hands
            # it to the head; otherwise the next stage's up conv reads the raw stream
            need_act = r == 0 or si == len(stages) - 1
            nxt_g = (rb[1][0]["g"] if r == 0 else params["head"]["g"]) if need_act else None
            # the last block's raw sum is read by nothing (the head reads its act)
            last = r == 1 and si == len(stages) - 1
            new_raw = NONE if last else slot(raw_fixed[1 - cur])
            new_act = slot(act_fixed[1 - cur]) if need_act else NONE
            ops.append(Op(cout=c, w=p2["w"], bias=p2.get("b"), src=inner, res=raw_cur, out=new_raw,
                          act_out=new_act, gamma=nxt_g, name="s%d.rb%d.c2" % (si, r)))
            raw_cur, act_cur, cur = new_raw, new_act, 1 - cur
        prev_raw, last_act = raw_cur, act_cur
        c_in = c
    head = params["head"]
    ops.append(Op(cout=c_out, w=head["w"], bias=head.get("b"), up_s=2, src=last_act, out=Y, out_u8=out_u8,
                  name="head"))
    return ops


def encoder_ops(params: Dict[str, Dict], stages=DECODER_STAGES, c_latent: int = 48,
                unique_slots: bool = False) -> List[Op]:
    """The encoder side (SwiftVR page, "ReAE: Causal Halo Exchange": the encoder
    keeps the decoder's per-layer causal state; the page prints no encoder
    layer): the decoder read backwards.  conv_in with spatial stride 2 from the
    pixels -> per stage, the decoder's stages from the last, [two residual
    blocks, then a conv with spatial stride 2 and the stage's temporal factor as
    temporal stride, back to the channels the decoder stage started from] ->
    act -> conv_out to the latent channels.  Params are keyed as
    oracle/model.py's encoder_layer_shapes ("conv_in", "e<i>.rb<r>.c1|c2",
    "e<i>.down", "conv_out"); conv_in's weights take the plan's input channels
    (pixels padded with zero channels to a multiple of 8).

    Slots per stage e (base = 3 + 5 e): raw A, raw B, act A, act B, inner act;
    slot 3 + 5*len(stages) holds the act conv_out reads.  ``unique_slots`` as in
    decoder_ops."""
    nxt = [3]

    def slot(fixed):
        if not unique_slots:
            return fixed
        nxt[0] += 1
        return nxt[0] - 1

    n = len(stages)
    widths = [stages[0][0]] + [c for c, _ in stages]  # the decoder's conv_in width, then each stage's
    ops: List[Op] = []
    raw_cur, act_cur = slot(3), slot(5)
    ops.append(Op(cout=stages[-1][0], w=params["conv_in"]["w"], bias=params["conv_in"].get("b"), stride_s=2,
                  src=X, out=raw_cur, act_out=act_cur, gamma=params["e0.rb0.c1"]["g"], name="conv_in"))
    for ei in range(n):
        si = n - 1 - ei  # the decoder stage this one mirrors
        c, factor = stages[si]
        base = 3 + 5 * ei
        raw_fixed, act_fixed = [base, base + 1], [base + 2, base + 3]
        cur = 0
        for r in range(2):
            p1, p2 = params["e%d.rb%d.c1" % (ei, r)], params["e%d.rb%d.c2" % (ei, r)]
            inner = slot(base + 4)
            ops.append(Op(cout=c, w=p1["w"], bias=p1.get("b"), src=act_cur, act_out=inner, gamma=p2["g"],
                          name="e%d.rb%d.c1" % (ei, r)))
            # block 0 hands act(y) to block 1; the down conv reads the raw stream
            need_act = r == 0
            new_raw = slot(raw_fixed[1 - cur])
            new_act = slot(act_fixed[1 - cur]) if need_act else NONE
            ops.append(Op(cout=c, w=p2["w"], bias=p2.get("b"), src=inner, res=raw_cur, out=new_raw,
                          act_out=new_act, gamma=params["e%d.rb1.c1" % ei]["g"] if need_act else None,
                          name="e%d.rb%d.c2" % (ei, r)))
            raw_cur, act_cur, cur = new_raw, new_act, 1 - cur
        down = params["e%d.down" % ei]
        if ei == n - 1:  # only conv_out's act is read after the last stage
            d_raw, d_act, g = NONE, slot(3 + 5 * n), params["conv_out"]["g"]
        else:
            d_raw, d_act, g = slot(base + 5), slot(base + 7), params["e%d.rb0.c1" % (ei + 1)]["g"]
        ops.append(Op(cout=widths[si], w=down["w"], bias=down.get("b"), stride_s=2, stride_t=factor, src=raw_cur,
                      out=d_raw, act_out=d_act, gamma=g, name="e%d.down" % ei))
        raw_cur, act_cur = d_raw, d_act
    out = params["conv_out"]
    ops.append(Op(cout=c_latent, w=out["w"], bias=out.get("b"), src=act_cur, out=Y, name="conv_out"))
    return ops
