"""CPU checks of the benchmark's own accounting: the FLOP and frame counts its
headline value divides by, its layer list, the traffic record lookup, and the
one-GPU contract."""
import hashlib
import os
import subprocess
import sys

import pytest

import bench
from oracle import model as OM

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STAGES = OM.DECODER_STAGES


def _layer_sizes(t_lat, first, temporal_grow, h=90, w=160):
    """(name, frames, height, width) of every conv's output for one clip, walked
    stage by stage; frame growth from the oracle's rule (first chunk) or 2x."""
    def frames_after(factors):
        if first:
            return OM.output_frames(t_lat, factors)
        n = t_lat
        for f in factors:
            n *= f
        return n

    out = [("conv_in", t_lat, h, w)]
    factors = []
    for si, (c, f) in enumerate(STAGES):
        t_in = frames_after(factors)
        factors.append(f)
        t_out = frames_after(factors)
        if temporal_grow:
            sh, sw = (2 * h, 2 * w) if temporal_grow == "after" else (h, w)
            out.append(("s%d.tg.p" % si, t_in, sh, sw))
            out.append(("s%d.tg.t" % si, t_out, sh, sw))
        h, w = 2 * h, 2 * w
        out.append(("s%d.up" % si, t_out, h, w))
        for r in range(2):
            out.append(("s%d.rb%d.c1" % (si, r), t_out, h, w))
            out.append(("s%d.rb%d.c2" % (si, r), t_out, h, w))
    out.append(("head", frames_after(factors), 2 * h, 2 * w))
    return out


@pytest.mark.parametrize("temporal_grow", [None, "before", "after"])
@pytest.mark.parametrize("t_lat,first", [(7, True), (6, False), (1, True), (3, False)])
def test_step_flops_match_a_per_layer_count(temporal_grow, t_lat, first):
    shapes = {n: (co, ci, kt, kh, kw) for n, co, ci, kt, kh, kw, _ in
              OM.decoder_layer_shapes(temporal_grow=temporal_grow)}
    sizes = _layer_sizes(t_lat, first, temporal_grow)
    assert [s[0] for s in sizes] == list(shapes)
    want = 0
    for name, t, h, w in sizes:
        co, ci, kt, kh, kw = shapes[name]
        want += 2 * ci * co * kt * kh * kw * t * h * w
    got, t_out = bench.c4_step_flops(t_lat, first, temporal_grow=temporal_grow)
    assert got == want
    assert t_out == sizes[-1][1]


@pytest.mark.parametrize("temporal_grow", [None, "before"])
def test_bench_layer_list_is_the_decoder(temporal_grow):
    assert bench.decoder_layer_list(temporal_grow=temporal_grow) == OM.decoder_layer_shapes(
        temporal_grow=temporal_grow)


@pytest.mark.parametrize("t_in,first,want", [
    # first chunk, 7 frames grown to 13: frame 0's taps all read X[0] (replicated
    # history, then X[0]): one group; every later frame has one pair: two groups
    (7, True, 8 * (1 + 2 * 12)),
    # later chunk, 6 frames grown to 12: frame 0 reads the two history frames (one
    # source frame, the previous chunk's last) and X[0]: two groups, as every frame
    (6, False, 8 * 2 * 12),
    (1, True, 8 * 1),
    (1, False, 8 * 2 * 2),
])
def test_folded_upsample_units_count_temporal_groups(t_in, first, want):
    assert bench.folded_up_units(t_in, first, 2) == want
    assert bench.folded_up_units(t_in, first, 1) == 21 * t_in


def test_folded_upsample_flops_are_below_the_algorithmic_count():
    for n, first in ((7, True), (6, False)):
        alg, ex = bench.c4_up_flops(n, first)
        assert 16.0 / 27.0 * alg < ex < 7.0 / 9.0 * alg
        alg2, ex2 = bench.c4_up_flops(n, first, grown_in_conv=False)
        assert alg2 == alg and ex2 == pytest.approx(7.0 / 9.0 * alg)


def test_clip_schedule_covers_the_video():
    sched = [7] + [6] * 14
    assert sched == OM.clip_schedule(91)
    frames = [bench.c4_step_flops(n, i == 0)[1] for i, n in enumerate(sched)]
    assert frames[0] == 25 and set(frames[1:]) == {24} and sum(frames) == OM.output_frames(91) == 361


def test_traffic_record_follows_the_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "x.md").write_text("traffic_record: kernel=kk source=k.hip source_sha256_16=%s bytes_per_launch=123.5\n" % sha)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("kk") == 123.5
    assert bench.recorded_traffic("other") is None
    src.write_text("kernel source, changed\n")
    assert bench.recorded_traffic("kk") is None
    # two sources: the hash covers both, in order
    other = tmp_path / "ops.py"
    other.write_text("op list\n")
    sha2 = hashlib.sha256(src.read_bytes() + other.read_bytes()).hexdigest()[:16]
    (prof / "x.md").write_text("traffic_record: kernel=kk source=k.hip,ops.py source_sha256_16=%s "
                               "bytes_per_launch=7\n" % sha2)
    assert bench.recorded_traffic("kk") == 7.0
    assert bench.recorded_clock("kk") is None
    other.write_text("op list, changed\n")
    assert bench.recorded_traffic("kk") is None
    # the counter run's clock rides on the same record
    sha3 = hashlib.sha256(src.read_bytes() + other.read_bytes()).hexdigest()[:16]
    (prof / "x.md").write_text("traffic_record: kernel=kk source=k.hip,ops.py source_sha256_16=%s "
                               "bytes_per_launch=7 clock_ghz=1.994\n" % sha3)
    assert bench.recorded_clock("kk") == 1.994 and bench.recorded_traffic("kk") == 7.0
    # a record that names its workload counts for that workload only (one kernel
    # can dominate two workloads with different bytes per launch)
    (prof / "x.md").write_text("traffic_record: kernel=kk workload=c4 source=k.hip,ops.py source_sha256_16=%s "
                               "bytes_per_launch=7\n"
                               "traffic_record: kernel=kk workload=e4 source=k.hip,ops.py source_sha256_16=%s "
                               "bytes_per_launch=9\n" % (sha3, sha3))
    assert bench.recorded_traffic("kk", "c4") == 7.0 and bench.recorded_traffic("kk", "e4") == 9.0
    assert bench.recorded_traffic("kk", "c3") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("args", [["--band", "8"], ["--workload", "c3", "--band", "7"],
                                  ["--workload", "c3", "--band", "0"]])
def test_band_is_refused_off_the_1440p_stage_or_off_its_rows(args):
    """--band splits the 1440p stage's 720 low-resolution rows: other workloads
    and counts that do not divide 720 are refused before any GPU work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "--band" in r.stderr and r.stdout == ""


def test_video_steps_cover_each_workload():
    """A whole video is the steps each workload's schedule gives: c4 the 15 clips,
    c3 its 1 + 90 chunks, c2 and c1 their 24 and 16 frames in 4-frame chunks."""
    from causal_convolution_x3x3_amd import synth
    assert bench.VIDEO_STEPS["c4"] == bench.VIDEO_STEPS["c4tg"] == len(OM.clip_schedule(91))
    wl = synth.WORKLOADS
    assert bench.VIDEO_STEPS["c3"] == len(synth.chunk_lengths(wl[3]["t"], wl[3]["chunk"], wl[3]["first_chunk"]))
    assert bench.VIDEO_STEPS["c2"] == len(synth.chunk_lengths(wl[2]["t"], wl[2]["chunk"]))
    assert bench.VIDEO_STEPS["c1"] == len(synth.chunk_lengths(wl[1]["t"], wl[1]["chunk"]))


def test_cpu_model_is_read():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


def test_encoder_layer_list_is_the_oracles():
    assert bench.encoder_layer_list(c_in=3) == OM.encoder_layer_shapes(c_in=3)


@pytest.mark.parametrize("t_in,first", [(25, True), (24, False), (1, True), (4, False)])
def test_encoder_step_flops_match_a_per_layer_count(t_in, first):
    """The e4 step's FLOP, summed here layer by layer over the oracle's layer list
    with the oracle's strided frame counts and ceil(H/2) frame sizes."""
    from oracle import oracle as O
    h, w, t = 1440, 2560, t_in
    seen = 0 if first else 25 + 24 * 3  # a later chunk starts at an odd frame
    want = 0.0
    for name, co, ci, kt, kh, kw, _, ss, st in OM.encoder_layer_shapes(c_in=3):
        if ss == 2:
            h, w = (h + 1) // 2, (w + 1) // 2
        if st == 2:
            t_new = O.strided_frames(t, 2, seen=seen)
            seen = O.strided_frames(seen, 2)  # frames this layer's output held before the chunk
            t = t_new
        want += 2.0 * ci * co * kt * kh * kw * t * h * w
    got, lat = bench.e4_step_flops(t_in, first)
    assert got == want and lat == t


def test_encoder_schedule_covers_the_video():
    lats = [bench.e4_step_flops(n, i == 0)[1] for i, n in enumerate([25] + [24] * 14)]
    assert lats == [7] + [6] * 14 and sum(lats) == 91 and bench.VIDEO_STEPS["e4"] == 15
