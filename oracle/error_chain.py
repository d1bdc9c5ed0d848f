"""Error chain of the rotation choices on a synthetic calibrated layer.

TEST INFRASTRUCTURE (analysis with the oracle only; CPU, fp64).  The OSCAR write-up's figure 1
(section OSCAR 的动机) compares naive INT2, Hadamard-only, clip-only and OSCAR by the errors their
quantisation noise causes downstream -- the attention-score KL divergence and the attention-output
MSE -- and argues that K/V reconstruction error alone does not predict them.  This module
computes those metrics for one KV head of a synthetic workload: keys and values of the history
segment (positions 64 .. L - 257; the BF16 sink and recent window stay exact) are quantised in
each variant's frame and compared, for held-out decode queries, with attention over the exact
cache.

  naive          R = I,              no clip
  hadamard_only  R = H P / sqrt(d),  no clip          (U = I)
  clip_only      R = I,              clip = 99.9th percentile of |x|
  oscar          R = U H P / sqrt(d) with the calibrated U_k / U_v, clip = 99.9th percentile
                 of |x R|
  oscar_lloyd_max  the OSCAR frame and clip with a Lloyd-Max codebook in place of the uniform
                 grid (the oracle's reading R19), its levels fitted on the keys / values of
                 another sequence of the same layer (calibration data, not the evaluated history)
  oscar_lm_uniform  the same with the codebook held to equally spaced levels (reading R20: the
                 form the GPU encoder takes; fitted on the same calibration data)

Calibration follows the oracle's calibration functions (U_k from the calibration queries' Q^T Q,
U_v from the score-weighted values (S V)^T (S V)); evaluation queries are drawn from a seed
stream of their own.

Usage:  python -m oracle.error_chain [--context N] [--calib N] [--eval N] [--kv-heads 0,1]
                                    [--group 64]
"""
from __future__ import annotations

import argparse
import math
import os
import sys

import numpy as np

if __package__ in (None, ""):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import workloads  # noqa: E402
from oracle import oscar_oracle as O  # noqa: E402

VARIANTS = ("naive", "hadamard_only", "clip_only", "oscar", "oscar_lloyd_max", "oscar_lm_uniform")


def _f64(t) -> np.ndarray:
    return t.double().cpu().numpy()


def layer_errors(wl, kv: int, n_calib: int, n_eval: int, layer: int = 0, percentile=99.9,
                 variants=VARIANTS):
    """{variant: (score KL, output MSE, key MSE, value MSE)} for KV head ``kv`` of sequence 0."""
    d = wl.head_dim
    gq = wl.gqa
    length = wl.context
    sm = 1.0 / math.sqrt(d)
    k_all, v_all = workloads.kv_tokens(wl, layer, 0, 0, length)
    k, v = _f64(k_all[:, kv]), _f64(v_all[:, kv])
    q_cal = _f64(workloads.calibration_queries(wl, layer, n=n_calib)[:, kv * gq:(kv + 1) * gq])
    q_cal = q_cal.reshape(-1, d)
    q_eval = np.concatenate([
        _f64(workloads.queries(wl, layer, step=1000 + i, batch=1)[0, kv * gq:(kv + 1) * gq])
        for i in range(n_eval)])
    frames = variant_frames(q_cal, k, v, sm, percentile)
    hist = slice(64, max(64, length - 256))
    levels = codebooks(wl, kv, frames["oscar"], layer) if "oscar_lloyd_max" in variants else None
    spaced = (codebooks(wl, kv, frames["oscar"], layer, uniform=True)
              if "oscar_lm_uniform" in variants else None)
    out = {}
    for name in variants:
        rk, ck, rv, cv = frames[name]
        k_hat, v_hat = k.copy(), v.copy()
        if name == "oscar_lloyd_max":
            k_hat[hist] = O.quantize_roundtrip_codebook(k[hist], rk, ck, wl.group_size, levels[0])
            v_hat[hist] = O.quantize_roundtrip_codebook(v[hist], rv, cv, wl.group_size, levels[1])
        elif name == "oscar_lm_uniform":
            k_hat[hist] = O.quantize_roundtrip(k[hist], rk, ck, wl.group_size, spaced[0])
            v_hat[hist] = O.quantize_roundtrip(v[hist], rv, cv, wl.group_size, spaced[1])
        else:
            k_hat[hist] = O.quantize_roundtrip(k[hist], rk, ck, wl.group_size)
            v_hat[hist] = O.quantize_roundtrip(v[hist], rv, cv, wl.group_size)
        out[name] = O.attention_error_metrics(q_eval, k, v, k_hat, v_hat, sm)
    return out


def variant_frames(q_cal, k, v, sm_scale: float, percentile=99.9):
    """{variant: (R_k, clip_k, R_v, clip_v)}: each variant's orthogonal frame (fp64) and clip
    threshold (inf = no clip) for one KV head, from its calibration queries q_cal (n, d) and the
    keys / values k, v (L, d) of the evaluated context."""
    d = k.shape[1]
    u_k = O.key_rotation(q_cal).astype(np.float32)
    u_v = O.value_rotation(q_cal, k, v, sm_scale).astype(np.float32)
    frames = {
        "naive": (O.frame_matrix(None, d), np.inf, O.frame_matrix(None, d), np.inf),
        "hadamard_only": (O.frame_matrix(np.eye(d), d), np.inf, O.frame_matrix(np.eye(d), d),
                          np.inf),
        "clip_only": (O.frame_matrix(None, d), float(np.percentile(np.abs(k), percentile)),
                      O.frame_matrix(None, d), float(np.percentile(np.abs(v), percentile))),
        "oscar": (O.frame_matrix(u_k, d), O.clip_threshold(k, u_k, percentile),
                  O.frame_matrix(u_v, d), O.clip_threshold(v, u_v, percentile)),
    }
    frames["oscar_lloyd_max"] = frames["oscar_lm_uniform"] = frames["oscar"]
    return frames


def codebooks(wl, kv: int, frame, layer: int = 0, n_tokens: int = 4096, iters: int = 100,
              uniform: bool = False):
    """Lloyd-Max levels (keys, values) for KV head ``kv``, fitted on the coordinates t of the
    first ``n_tokens`` keys / values of sequence 1 in the given (R_k, clip_k, R_v, clip_v) frame;
    with ``uniform`` the equally spaced optimum instead, as (lo, step) in fp32."""
    rk, ck, rv, cv = frame
    k_cal, v_cal = workloads.kv_tokens(wl, layer, 1, 0, n_tokens)
    out = []
    for x, r, c in ((_f64(k_cal[:, kv]), rk, ck), (_f64(v_cal[:, kv]), rv, cv)):
        t = O.codebook_coordinates((x @ r).astype(np.float32), c, wl.group_size)
        if uniform:
            lo, step, _ = O.lloyd_max_uniform(t, iters=iters)
            out.append((np.float32(lo), np.float32(step)))
        else:
            out.append(O.lloyd_max(t, iters=iters)[0])
    return out


def table(results) -> str:
    lines = ["| variant | attention-score KL | attention-output MSE | key MSE | value MSE |",
             "|---|---|---|---|---|"]
    for name in (v for v in VARIANTS if v in results):
        kl, mse, ke, ve = results[name]
        lines.append(f"| {name} | {kl:.4e} | {mse:.4e} | {ke:.4e} | {ve:.4e} |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="qwen3_4b_32k")
    ap.add_argument("--context", type=int, default=None)
    ap.add_argument("--calib", type=int, default=None, help="calibration query positions")
    ap.add_argument("--eval", type=int, default=64, help="held-out decode query positions")
    ap.add_argument("--kv-heads", default="0")
    ap.add_argument("--group", type=int, default=None, help="channels per scale / zero group")
    args = ap.parse_args(argv)
    wl = workloads.get(args.workload)
    if args.context:
        wl = workloads.scaled(wl, context=args.context)
    if args.group:
        wl = workloads.scaled(wl, group_size=args.group)
    n_calib = args.calib or wl.calib_queries or 4096
    for kv in (int(x) for x in args.kv_heads.split(",")):
        res = layer_errors(wl, kv, n_calib, args.eval)
        print(f"{wl.name}: context {wl.context}, KV head {kv}, group {wl.group_size}, "
              f"{n_calib} calibration positions, {args.eval} evaluation positions x {wl.gqa} "
              f"query heads")
        print(table(res))


if __name__ == "__main__":
    main()
