"""Writes stack_bounds.txt: the end-to-end bound of every whole-decoder (and
whole-encoder) configuration the GPU tests compare with the storage-rounded
oracle.

Calls only the oracle (and the seeded input generators).  For each case of
``tests/stack_cases.py`` the decoder runs chunk by chunk in the oracle with every
stored tensor rounded to bfloat16 (the reference the GPU tests use), and again
with every value multiplied by (1 + sigma * n), n ~ N(0, 1), before its rounding
-- what a different fp32 summation order does to a value before it is stored.
sigma = 2^-19 (32 fp32 ulps) is above the accumulation error of the longest sum
on the path (384 channels x 27 taps in 324 MFMA accumulations: sqrt(324) = 18
ulps as a random walk).  The drift of each perturbed run from the reference
(max|d| / max|ref|, mean|d| / mean|ref|) is taken over SEEDS seeds; the bound is
FACTOR times the largest drift seen.  Also recorded, for information: the
reference against the unrounded fp64 decoder.

    python tests/golden/make_stack_bounds.py [case ...]
"""
from __future__ import annotations

import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
for p in (ROOT, os.path.dirname(HERE)):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402

import stack_cases as SC  # noqa: E402
from oracle import model as OM  # noqa: E402
from oracle import oracle as O  # noqa: E402

SIGMA = 2.0 ** -19
SEEDS = 3
FACTOR = 1.5
OUT = os.path.join(HERE, "stack_bounds.txt")


def run_oracle(c, store):
    cpu = {n: {k: None if v is None else v.double().numpy() for k, v in p.items()}
           for n, p in SC.weights(c).items()}
    if c["kind"] == "encoder":
        x = SC.pixels(c).double().numpy()
        dec = OM.Encoder(cpu, stages=c["stages"], store=store, aligned=c["aligned"], mode=c["mode"])
    else:
        x = SC.latent(c).double().numpy()
        dec = OM.Decoder(cpu, stages=c["stages"], store=store, temporal_grow=c["tg"], aligned=c["aligned"])
    out, t0 = [], 0
    for n in c["splits"]:
        out.append(dec.step(x[:, t0:t0 + n]))
        t0 += n
    return np.concatenate(out, axis=1)


def rel(a, ref):
    d = np.abs(a - ref)
    return float(d.max() / np.abs(ref).max()), float(d.mean() / np.abs(ref).mean())


def measure(c, seeds=SEEDS, sigma=SIGMA):
    """(drifts per seed, reference vs unrounded fp64)."""
    ref = run_oracle(c, O.round_bf16)
    drifts = []
    for s in range(seeds):
        noise = np.random.default_rng(1000 + s)
        alt = run_oracle(c, lambda v: O.round_bf16(v * (1.0 + sigma * noise.standard_normal(v.shape))))
        drifts.append(rel(alt, ref))
    return drifts, rel(ref, run_oracle(c, None))


def bound(drifts, factor=FACTOR):
    return factor * max(d[0] for d in drifts), factor * max(d[1] for d in drifts)


def fmt(name, drifts, vs64):
    bm, bn = bound(drifts)
    per = " ".join("%.4e/%.4e" % d for d in drifts)
    return "%s: %.4e %.4e | drift %s | fp64 %.4e/%.4e" % (name, bm, bn, per, vs64[0], vs64[1])


def read(path=OUT):
    """name -> (max bound, mean bound)."""
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, rest = line.split(":", 1)
            vals = rest.split("|")[0].split()
            out[name.strip()] = (float(vals[0]), float(vals[1]))
    return out


def main(names):
    lines = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            for line in f:
                if line.strip() and not line.startswith("#"):
                    lines[line.split(":", 1)[0].strip()] = line.rstrip("\n")
    for name in names or list(SC.STACK_CASES):
        t = time.time()
        drifts, vs64 = measure(SC.STACK_CASES[name])
        lines[name] = fmt(name, drifts, vs64)
        print(lines[name], "(%.0f s)" % (time.time() - t), flush=True)
    with open(OUT, "w") as f:
        f.write("# End-to-end bound per decoder configuration (tests/stack_cases.py), written by\n"
                "# make_stack_bounds.py from the oracle alone: name: max-rel bound, mean-rel bound |\n"
                "# the storage-rounded oracle's drift under %d seeds of relative perturbation %.3g\n"
                "# before every bf16 store (max/mean per seed); bound = %.1f x the largest |\n"
                "# the reference against the unrounded fp64 decoder (information).\n"
                % (SEEDS, SIGMA, FACTOR))
        for name in SC.STACK_CASES:
            if name in lines:
                f.write(lines[name] + "\n")


if __name__ == "__main__":
    main(sys.argv[1:])
