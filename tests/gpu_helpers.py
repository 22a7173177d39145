"""Shared helpers for the GPU tests: move seeded 16-bit inputs to the device,
call the HIP library through its binding, and compare with the oracle."""
import numpy as np

from synth import inputs as si

# tolerances (forward max-abs on O and LSE; backward relative Frobenius norm)
TOL_O = {si.FMT_F16: 2e-3, si.FMT_BF16: 8e-3}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2


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


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (the largest RNE storage error for that value)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return 0.5 * np.exp2(e - 7)


def gated_o_error(o_gpu, o_ref, stored_bf16):
    """Max error of O measured against the bound: where O is stored in bf16 the
    bound applies to the error beyond each element's bf16 storage rounding
    (half an ulp of the exact value); otherwise to the plain error."""
    err = np.abs(o_gpu - o_ref)
    return float((err - bf16_half_ulp(o_ref)).max() if stored_bf16 else err.max())
