"""The four rotation choices of the OSCAR write-up's figure 1 run through the HIP kernels.

"超越TurboQuant！OSCAR：面向真实服务的2-bit KV Cache量化", section OSCAR 的动机, figure 1, compares
naive INT2, Hadamard-only, clip-only and OSCAR by the attention-output error their quantisation
noise causes.  Every variant is a frame R and a clip threshold, and the kernels take any frame:
they store x U H P / sqrt(d), so U = R (H P / sqrt(d))^T gives frame R -- U = P H / sqrt(d) is the
identity frame of naive INT2 and clip-only, U = I the Hadamard-only frame; "no clip" is the
largest finite fp16 threshold.

For two KV heads of the Qwen3-4B-shaped calibrated layer (context 32,768, frames and clips from
oracle.error_chain's calibration), the GPU demotes the history in each variant's frame, then
decodes 16 held-out queries.  Checked: pool bytes against the oracle under the acceptance rule,
attention against the oracle's attention over its own pool (2e-3), and the attention-output MSE
against exact attention next to oracle.error_chain's MSE for the same variant and queries.
"""
import math

import numpy as np
import pytest
import torch

import bit_rotated_kv_decode_amd as ok
import oracle
import workloads
from oracle import error_chain as EC
from oracle import oscar_oracle as O
from oscar_cases import ATTN_TOL, Case, attention_error, compare_pool_blocks

pytestmark = pytest.mark.gpu

HEADS = (0, 3)
N_CALIB = 256
N_EVAL = 16
NO_CLIP = 65504.0
VARIANTS = ("naive", "hadamard_only", "clip_only", "oscar")


def _f64(t):
    return t.double().cpu().numpy()


@pytest.fixture(scope="module")
def chain():
    wl = workloads.get("qwen3_4b_32k")
    d, G = wl.head_dim, wl.gqa
    sm = 1.0 / math.sqrt(d)
    k_all, v_all = workloads.kv_tokens(wl, 0, 0, 0, wl.context)
    q_cal = workloads.calibration_queries(wl, 0, n=N_CALIB)
    q_eval = torch.cat([workloads.queries(wl, 0, step=1000 + i, batch=1) for i in range(N_EVAL)])
    frames, metrics = {}, {}
    for kv in HEADS:
        qc = _f64(q_cal[:, kv * G:(kv + 1) * G]).reshape(-1, d)
        frames[kv] = EC.variant_frames(qc, _f64(k_all[:, kv]), _f64(v_all[:, kv]), sm)
        metrics[kv] = EC.layer_errors(wl, kv, N_CALIB, N_EVAL, variants=VARIANTS)
    print(f"error chain: {wl.name}, context {wl.context}, heads {HEADS}", flush=True)
    return dict(wl=wl, k=k_all, v=v_all, q=q_eval, frames=frames, metrics=metrics)


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_through_kernels(chain, variant):
    wl = chain["wl"]
    d, G, hkv, L = wl.head_dim, wl.gqa, wl.num_kv_heads, wl.context
    hp = O.frame_matrix(np.eye(d), d)                   # H P / sqrt(d)
    u = [np.tile(np.eye(d), (hkv, 1, 1)) for _ in range(2)]
    clip = [np.full(hkv, NO_CLIP, np.float32) for _ in range(2)]
    for kv in HEADS:
        rk, ck, rv, cv = chain["frames"][kv][variant]
        for i, (r, c) in enumerate(((rk, ck), (rv, cv))):
            u[i][kv] = r @ hp.T
            clip[i][kv] = min(c, NO_CLIP)
    u = tuple(torch.from_numpy(x.astype(np.float32)) for x in u)
    case = Case(wl, [L], u=u, clip=tuple(clip))
    print(f"variant {variant}: clips k {[float(clip[0][h]) for h in HEADS]} "
          f"v {[float(clip[1][h]) for h in HEADS]}", flush=True)
    g = case.gpu_inputs()
    cache = case.gpu_cache(g)                           # the GPU's own demotion
    torch.cuda.synchronize()
    ref_pool = case.oracle_pool(heads=HEADS)
    compare_pool_blocks(cache.pool.cpu().numpy(), ref_pool, case, heads=list(HEADS))

    # the held-out queries decode as a batch of sequences that alias one cache
    table = g["table"].expand(N_EVAL, -1).contiguous()
    slots = torch.zeros(N_EVAL, dtype=torch.int32, device="cuda")
    lens = torch.full((N_EVAL,), L, dtype=torch.int32, device="cuda")
    q = chain["q"].to("cuda").contiguous()
    out = torch.empty((N_EVAL, wl.num_q_heads, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(ok.decode_workspace_bytes(case.layout, N_EVAL, L), dtype=torch.uint8,
                     device="cuda")
    ok.decode_attn(case.layout, cache.pool, table, cache.sink_k, cache.sink_v, cache.recent_k,
                   cache.recent_v, slots, lens, q, g["u_k"], g["u_v"], out, ws, L)
    torch.cuda.synchronize()
    o_gpu = out.double().cpu().numpy()

    rows = [(i, kv * G + j) for i in range(N_EVAL) for kv in HEADS for j in range(G)]
    sk, sv, rk_, rv_ = case.oracle_segments()
    ref, _ = oracle.decode_attention(ref_pool, case.table.repeat(N_EVAL, 0), sk, sv, rk_, rv_,
                                     np.zeros(N_EVAL, np.int64), [L] * N_EVAL,
                                     _f64(chain["q"]), case.u_k.numpy(), case.u_v.numpy(),
                                     case.geom, heads=rows)
    err = attention_error(o_gpu, ref, rows)
    assert err <= ATTN_TOL, err

    qn = _f64(chain["q"])
    for kv in HEADS:
        k, v = _f64(chain["k"][:, kv]), _f64(chain["v"][:, kv])
        qs = qn[:, kv * G:(kv + 1) * G].reshape(-1, d)
        s = qs @ k.T / math.sqrt(d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        exact = (p / p.sum(axis=1, keepdims=True)) @ v
        mse_gpu = float(np.mean((o_gpu[:, kv * G:(kv + 1) * G].reshape(-1, d) - exact) ** 2))
        mse_oracle = chain["metrics"][kv][variant][1]
        print(f"| {kv} | {variant} | oracle {mse_oracle:.4e} | GPU {mse_gpu:.4e} |", flush=True)
        assert abs(mse_gpu - mse_oracle) <= 0.03 * mse_oracle + 1e-12, (mse_gpu, mse_oracle)


def test_variant_ordering(chain):
    # on these inputs (x16 outlier channels), the two unrotated variants are far worse than the
    # two rotated ones (the figure's point that rotation is what makes INT2 usable)
    for kv in HEADS:
        m = {name: chain["metrics"][kv][name][1] for name in VARIANTS}
        assert min(m["naive"], m["clip_only"]) > 4 * max(m["hadamard_only"], m["oscar"]), m
