"""The whole-decoder (and whole-encoder) configurations the GPU tests compare
end to end, and their seeded inputs.  Shared by the GPU tests and by ``golden/make_stack_bounds.py``,
which measures, per configuration, how far the storage-rounded oracle drifts
from itself under rounding-level perturbations (the end-to-end bound).

A case: latent channels, stages ((channels, temporal factor), ...), latent
frames t, frame size h x w, chunk lengths, weight seed cfg, TemporalGrow order
(None, "before", "after") and the aligned first-chunk rule.  An encoder case
(kind "encoder") has the pixel channels c_in, frames t of the video, its frame
size h x w, the stages as the decoder lists them, and history mode (zeros: the
ReAE rule of the SwiftVR page, "ReAE: Causal Halo Exchange").
"""
from __future__ import annotations

import numpy as np

from causal_convolution_x3x3_amd import synth
from oracle import model as OM

SMALL_STAGES = ((64, 2), (32, 2), (16, 1))
FULL_STAGES = OM.DECODER_STAGES


def case(c_lat, stages, t, h, w, splits, cfg=4, tg=None, aligned=False):
    return dict(kind="decoder", c_lat=c_lat, stages=tuple(tuple(s) for s in stages), t=t, h=h, w=w,
                splits=tuple(splits), cfg=cfg, tg=tg, aligned=aligned)


def enc_case(c_in, c_lat, stages, t, h, w, splits, cfg=5, aligned=False):
    return dict(kind="encoder", c_in=c_in, c_lat=c_lat, stages=tuple(tuple(s) for s in stages), t=t, h=h, w=w,
                splits=tuple(splits), cfg=cfg, tg=None, aligned=aligned, mode="zero")


def random_decoder_cases(n, seed):
    """Seeded decoder configurations: two or three stages of random widths and
    temporal factors, latent width, frame size, chunking, TemporalGrow order,
    first-chunk growth rule and the folding request (the last item)."""
    rng = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        nst = int(rng.randint(2, 4))
        stages = tuple((int(rng.choice([16, 32, 64, 96, 128, 192])), int(rng.randint(1, 3))) for _ in range(nst))
        c_lat = int(rng.choice([8, 16, 32, 48]))
        t, h, w = int(rng.randint(2, 6)), int(rng.randint(1, 5)), int(rng.randint(1, 7))
        splits, left = [], t
        while left:
            k = int(rng.randint(1, left + 1))
            splits.append(k)
            left -= k
        tg = [None, "before", "after"][rng.randint(3)]
        cases.append((c_lat, stages, t, h, w, splits, tg, bool(rng.randint(2)), bool(rng.randint(2))))
    return cases


RANDOM_CASES = random_decoder_cases(8, 11)

STACK_CASES = {
    "small": case(16, SMALL_STAGES, 6, 3, 5, (2, 3, 1)),
    "small_t5": case(16, SMALL_STAGES, 5, 3, 5, (3, 2)),
    "small_t5_aligned": case(16, SMALL_STAGES, 5, 3, 5, (3, 2), aligned=True),
    "small_tg_before": case(16, SMALL_STAGES, 6, 3, 5, (2, 3, 1), tg="before"),
    "small_tg_after": case(16, SMALL_STAGES, 6, 3, 5, (2, 3, 1), tg="after"),
    "small_t5_tg_before": case(16, SMALL_STAGES, 5, 3, 5, (3, 2), tg="before"),
    "small_t5_tg_before_aligned": case(16, SMALL_STAGES, 5, 3, 5, (3, 2), tg="before", aligned=True),
    "full_tiny": case(48, FULL_STAGES, 5, 2, 3, (3, 2)),
    "full_tiny_aligned": case(48, FULL_STAGES, 5, 2, 3, (3, 2), aligned=True),
    "full_tiny_tg_before": case(48, FULL_STAGES, 5, 2, 3, (3, 2), tg="before"),
    "full_one_latent": case(48, FULL_STAGES, 4, 2, 3, (1, 1, 1, 1)),
    "full_two_clips": case(48, FULL_STAGES, 13, 4, 6, (7, 6)),
    "smoke": case(48, FULL_STAGES, 3, 2, 3, (2, 1), cfg=9),
    "full_fused_cache": case(48, FULL_STAGES, 4, 2, 3, (2, 2), cfg=9),
}
for _i, (_cl, _st, _t, _h, _w, _sp, _tg, _al, _fold) in enumerate(RANDOM_CASES):
    STACK_CASES["random%d" % _i] = case(_cl, _st, _t, _h, _w, _sp, cfg=9, tg=_tg, aligned=_al)
def random_encoder_cases(n, seed):
    """Seeded encoder configurations: two or three stages of random widths and
    temporal factors, latent width, frame size, history fill, phase, and chunks
    that keep every strided layer's count whole (with m = 2^(temporal strides):
    a first chunk of 1 mod m frames then multiples of m; all multiples of m with
    the aligned rule)."""
    rng = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        nst = int(rng.randint(2, 4))
        stages = tuple((int(rng.choice([16, 32, 64, 96, 128, 192])), int(rng.randint(1, 3))) for _ in range(nst))
        m = 2 ** sum(1 for _, f in stages if f == 2)
        aligned = bool(rng.randint(2))
        first = m * int(rng.randint(1, 3)) if aligned else 1 + m * int(rng.randint(0, 2))
        splits = [first] + [m * int(rng.randint(1, 3)) for _ in range(int(rng.randint(0, 3)))]
        c_lat = int(rng.choice([8, 16, 48]))
        h, w = int(rng.randint(1, 40)), int(rng.randint(1, 60))
        mode = ["zero", "replicate"][rng.randint(2)]
        c = enc_case(3, c_lat, stages, sum(splits), h, w, splits, cfg=7, aligned=aligned)
        c["mode"] = mode
        cases.append(c)
    return cases


STACK_CASES.update({
    # 1 + 4n frames with the first frame on its own (an odd first chunk, even later
    # ones at every temporal stride), or 4n with the aligned rule
    "enc_small": enc_case(3, 16, SMALL_STAGES, 9, 16, 24, (5, 4)),
    "enc_small_aligned": enc_case(3, 16, SMALL_STAGES, 8, 16, 24, (4, 4), aligned=True),
    "enc_full_tiny": enc_case(3, 48, FULL_STAGES, 5, 16, 16, (1, 4), cfg=9),
    "enc_full_aligned": enc_case(3, 48, FULL_STAGES, 8, 16, 24, (4, 4), cfg=9, aligned=True),
})
for _i, _c in enumerate(random_encoder_cases(6, 17)):
    STACK_CASES["enc_random%d" % _i] = _c


def layer_shapes(c):
    """(name, Cout, Cin, kt, kh, kw, has_gain, ...) of every conv of the case."""
    if c["kind"] == "encoder":
        return OM.encoder_layer_shapes(c_in=c["c_in"], stages=c["stages"], c_latent=c["c_lat"])
    return OM.decoder_layer_shapes(c_latent=c["c_lat"], stages=c["stages"], temporal_grow=c["tg"])


def weights(c):
    """The case's seeded layer weights (CPU tensors, see synth.layer_weights)."""
    full = layer_shapes(c)
    gains = {s[0]: s[6] for s in full}
    return synth.layer_weights([s[:6] for s in full], c["cfg"], lambda n: gains[n])


def latent(c):
    """The case's seeded bf16 latent video [C][T][H][W] (CPU)."""
    return synth.bf16(synth.video(c["c_lat"], c["t"], c["h"], c["w"], synth.seed(c["cfg"], 1)))


def pixels(c):
    """An encoder case's seeded bf16 input video [c_in][T][H][W] (CPU)."""
    return synth.bf16(synth.video(c["c_in"], c["t"], c["h"], c["w"], synth.seed(c["cfg"], 2)))
