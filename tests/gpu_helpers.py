"""Shared helpers for the GPU tests: move seeded 16-bit inputs to the device,
call the HIP library through its binding, and compare with the oracle."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from synth import inputs as si

# Tolerances: forward max-abs on O and LSE; backward relative Frobenius norm
# per gradient tensor (2e-2), and a bound on every row: a row's error is at
# most 16 unit roundoffs of the input format (u = 2^-11 fp16, 2^-8 bf16: the
# relative rounding of P and dS before their 16-bit products) times the
# larger of its own norm and the tensor's RMS row norm.  The floor is needed
# because a row's exact gradient can be far smaller than the terms it sums
# (dQ_i sums dS_ij k_j with sum_j dS_ij = 0; a nearly one-hot softmax row has
# dS close to 0 while D carries the rounding of the stored O), and those
# rows keep the absolute error of the typical row.  Measured worst rows:
# 11u (fp16, scale 1) and 7u (bf16); a wrong row of typical size reads ~1.
TOL_O = {si.FMT_F16: 2e-3, si.FMT_BF16: 8e-3}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
UNIT_ROUNDOFF = {si.FMT_F16: 2.0 ** -11, si.FMT_BF16: 2.0 ** -8}
TOL_GRAD_ROW = {f: 16 * u for f, u in UNIT_ROUNDOFF.items()}
ROW_FLOOR = 1.0

# Where O is stored in bf16 and the exact O reaches 2 in magnitude, rounding
# the exact value to bf16 alone costs up to half an ulp, 7.8e-3 for |O| in
# [2, 4): there the bf16 bound applies to the error beyond that rounding.
BF16_FLOOR_FROM = 2.0

_POOL = ThreadPoolExecutor(max_workers=8)


def to_dev(bits, fmt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if fmt == si.FMT_F16 else torch.bfloat16)
    return t.to("cuda")


def dev_inputs(w):
    out = [to_dev(w.q, w.fmt), to_dev(w.k, w.fmt), to_dev(w.v, w.fmt)]
    if w.do is not None:
        out.append(to_dev(w.do, w.fmt))
    return out


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_fwd(w, out_f32=False):
    import torch
    import io_aware_exact_08_amd as fa
    q, k, v = dev_inputs(w)[:3]
    o, lse = fa.flash_attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out_f32=out_f32)
    torch.cuda.synchronize()
    return o, lse


def oracle_forward(w, heads=None):
    """The oracle's forward of every (or the listed) (b, h) of a workload, heads
    in parallel threads.  Returns {(b, h): (O, LSE)}."""
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    res = _POOL.map(lambda bh: oracle.forward_head(q[bh], k[bh], v[bh], w.scale, w.causal), heads)
    return dict(zip(heads, res))


def oracle_backward(w, heads=None):
    """The oracle's gradients for every (or the listed) (b, h), heads in
    parallel threads.  Returns {(b, h): (dQ, dK, dV)}."""
    q, k, v, do = w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do")
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    res = _POOL.map(lambda bh: oracle.backward_head(q[bh], k[bh], v[bh], do[bh], w.scale, w.causal),
                    heads)
    return dict(zip(heads, res))


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def grad_errors(g, gr):
    """(relative Frobenius error, worst row relative error) of a gradient
    against its reference; the last axis is d.  A row's error is measured
    against the larger of its own norm and ROW_FLOOR times the RMS row norm."""
    g2 = g.reshape(-1, g.shape[-1])
    r2 = gr.reshape(-1, gr.shape[-1])
    fro = rel_fro(g2, r2)
    rn = np.linalg.norm(r2, axis=1)
    en = np.linalg.norm(g2 - r2, axis=1)
    floor = ROW_FLOOR * float(np.sqrt(np.mean(rn * rn)))
    if floor == 0.0:
        return fro, float(en.max())
    return fro, float((en / np.maximum(rn, floor)).max())


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (the largest RNE storage error for that value)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return 0.5 * np.exp2(e - 7)


def o_error(o_gpu, o_ref, stored_bf16, plain=False):
    """(error checked against the O bound, description).  The plain max|dO|,
    except where O is stored in bf16 and max|O_ref| >= 2 (unless `plain`):
    there it is each element's error beyond half a bf16 ulp of the exact
    value."""
    err = np.abs(o_gpu - o_ref)
    if stored_bf16 and not plain and np.abs(o_ref).max() >= BF16_FLOOR_FROM:
        return float((err - bf16_half_ulp(o_ref)).max()), "beyond bf16 storage rounding"
    return float(err.max()), "plain"
