"""Backward parity: dQ, dK, dV from the HIP kernels (recomputing P from the
forward's LSE) against the fp64 oracle's gradients of <dO, O>, relative
Frobenius error <= 2e-2 per gradient tensor."""
import numpy as np
import pytest

import oracle
from synth import inputs as si
from gpu_helpers import (TOL_GRAD, TOL_GRAD_ROW, TOL_LSE, TOL_O, dev_inputs, f64, grad_errors,
                         o_error, oracle_backward, oracle_forward)

pytestmark = pytest.mark.gpu


def run_fwd_bwd(w, out_f32=False):
    import torch
    import io_aware_exact_08_amd as fa
    q, k, v, do = dev_inputs(w)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=w.causal, scale=w.scale, out_f32=out_f32)
    dq, dk, dv = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def check_grad(name, g, gr, fmt, tag=""):
    """Relative Frobenius error of one gradient tensor (<= 2e-2) and its worst
    row (<= 16 unit roundoffs of the format, against the larger of the row's
    norm and the RMS row norm); an exactly-zero reference (e.g. N = 1:
    dQ = dK = 0) must come out as zeros up to 1e-4."""
    assert np.isfinite(g).all(), (tag, name)
    if np.linalg.norm(gr) < 1e-6:
        e = float(np.abs(g).max())
        assert e <= 1e-4, (tag, name, e)
        return e, e
    fro, row = grad_errors(g, gr)
    assert fro <= TOL_GRAD, (tag, name, fro)
    assert row <= TOL_GRAD_ROW[fmt], (tag, name, "row", row)
    return fro, row


def check_heads(w, res, heads=None):
    """Every element of the listed heads (default: all) against the oracle:
    O and LSE within the forward bounds, each gradient within the relative
    bounds per tensor and per row."""
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    stored_bf16 = str(res[0].dtype) == "torch.bfloat16"
    o, lse, dq, dk, dv = (f64(t) for t in res)
    fwd_ref = oracle_forward(w, heads)
    bwd_ref = oracle_backward(w, heads)
    worst = {"o": 0.0, "lse": 0.0, "dq": (0.0, 0.0), "dk": (0.0, 0.0), "dv": (0.0, 0.0)}
    for b, h in heads:
        o_ref, l_ref = fwd_ref[(b, h)]
        eo, _ = o_error(o[b, h], o_ref, stored_bf16)
        el = float(np.abs(lse[b, h] - l_ref).max())
        assert eo <= TOL_O[w.fmt] and el <= TOL_LSE, (w.name, b, h, eo, el)
        worst["o"], worst["lse"] = max(worst["o"], eo), max(worst["lse"], el)
        for name, g, gr in zip(("dq", "dk", "dv"), (dq[b, h], dk[b, h], dv[b, h]), bwd_ref[(b, h)]):
            fro, row = check_grad(name, g, gr, w.fmt, tag=f"{w.name} b={b} h={h}")
            worst[name] = (max(worst[name][0], fro), max(worst[name][1], row))
    print(f"{w.name} ({len(heads)} heads): |dO|={worst['o']:.2e} |dLSE|={worst['lse']:.2e} "
          + " ".join(f"{n} rel={worst[n][0]:.2e} row={worst[n][1]:.2e}" for n in ("dq", "dk", "dv")),
          flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_bwd_workload(causal):
    """B=2 H=12 N=4096 d=64 fp16, forward then backward in the benchmark's
    launch configuration; every element of all 24 heads."""
    w = si.fwd_bwd(causal)
    res = run_fwd_bwd(w)
    check_heads(w, res)


@pytest.mark.parametrize("fmt,out_f32", [(si.FMT_F16, False), (si.FMT_BF16, False),
                                         (si.FMT_BF16, True)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 17, 64, 100, 129, 300])
def test_small_shapes(N, d, causal, fmt, out_f32):
    w = si.random_case(1, 2, N, d, fmt, causal, seed=7 * N + d, with_do=True)
    res = run_fwd_bwd(w, out_f32=out_f32)
    check_heads(w, res, [(0, 0), (0, 1)])


@pytest.mark.parametrize("fmt", [si.FMT_F16, si.FMT_BF16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [1.0, 0.3, 0.01])
def test_non_default_scales(scale, causal, fmt):
    """Softmax scales other than 1/sqrt(d), forward and backward: a sharp
    softmax (scale 1: scores with std 8), a moderate one and a nearly flat
    one (scale 0.01)."""
    w = si.random_case(1, 2, 200, 64, fmt, causal, seed=int(scale * 1000) + 3, with_do=True,
                       scale=scale)
    res = run_fwd_bwd(w)
    check_heads(w, res, [(0, 0), (0, 1)])


def test_long_causal_bwd_sampled():
    """Backward at the long-sequence causal shape (B=1 H=8 N=32768 d=64 bf16,
    N(0, 0.5^2), dO likewise): dQ on the sampled query rows of every head, dK
    and dV on the sampled key rows of the first and last head; relative error
    over the sampled rows <= 2e-2 for each gradient, and on every sampled row."""
    w = si.long_causal(with_do=True)
    res = run_fwd_bwd(w)
    _, _, dq, dk, dv = (f64(t) for t in res)
    q, k, v, do = w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do")
    pairs = si.long_causal_sample_rows(w.H, w.N)
    rows = [(0, int(h), int(i)) for h, i in pairs]
    dq_ref = oracle.backward_dq_rows(q, k, v, do, rows, w.scale, True)
    dq_gpu = np.stack([dq[b, h, i] for b, h, i in rows])
    cols = [r for r in rows if r[1] in (0, w.H - 1)]
    dk_ref, dv_ref = oracle.backward_kv_cols(q, k, v, do, cols, w.scale, True)
    dk_gpu = np.stack([dk[b, h, j] for b, h, j in cols])
    dv_gpu = np.stack([dv[b, h, j] for b, h, j in cols])
    errs = {name: check_grad(name, g, gr, w.fmt, tag=w.name)
            for name, g, gr in (("dq", dq_gpu, dq_ref), ("dk", dk_gpu, dk_ref), ("dv", dv_gpu, dv_ref))}
    print(f"{w.name} bwd: {len(rows)} dQ rows, {len(cols)} dK/dV rows, "
          + " ".join(f"{n} rel={e[0]:.2e} row={e[1]:.2e}" for n, e in errs.items()), flush=True)


def test_bench_shape_bwd_full():
    """Forward and backward in the benchmark's own launch (B=2 H=12 N=8192 d=64
    fp16 non-causal, the step bench.py times): every element of all 24 heads."""
    w = si.a100_sweep(8192, with_do=True)
    res = run_fwd_bwd(w)
    check_heads(w, res)


@pytest.mark.parametrize("fmt", [si.FMT_F16, si.FMT_BF16])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_256_bwd(causal, fmt):
    """d=256 forward and backward (32-row query tiles in dK/dV, 32-key tiles in
    dQ, accumulators in the accumulation registers) at B=1 H=4 N=1000: 32
    query tiles of dK/dV, a ragged tail, every element of every head."""
    w = si.random_case(1, 4, 1000, 256, fmt, causal, seed=2560 + causal, with_do=True)
    res = run_fwd_bwd(w)
    check_heads(w, res)


@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_256_bwd_bench_shape(causal):
    """d=256 at B=2 H=8 N=4096 fp16, the benchmarked shape, every element of
    all 16 heads."""
    w = si.random_case(2, 8, 4096, 256, si.FMT_F16, causal, seed=2570 + causal, with_do=True)
    res = run_fwd_bwd(w)
    check_heads(w, res)


def test_long_causal_bwd_full_2048():
    """The same distribution at N=2048, every gradient row of two heads."""
    w = si.long_causal(N=2048, with_do=True)
    res = run_fwd_bwd(w)
    check_heads(w, res, [(0, 0), (0, 7)])


def test_bwd_deterministic_and_in_bounds():
    import torch
    import io_aware_exact_08_amd as fa
    w = si.random_case(1, 3, 450, 64, si.FMT_F16, True, seed=3, with_do=True)
    q, k, v, do = dev_inputs(w)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=True, scale=w.scale)
    n, pad = 3 * 450 * 64, 2048
    bufs = [torch.full((n + 2 * pad,), 3.0, dtype=torch.float16, device="cuda") for _ in range(3)]
    views = [b[pad:pad + n].view(1, 3, 450, 64) for b in bufs]
    fa.flash_attn_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale,
                      dq=views[0], dk=views[1], dv=views[2])
    again = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for vw, a, b in zip(views, again, bufs):
        assert torch.equal(vw, a)
        assert (b[:pad] == 3.0).all() and (b[pad + n:] == 3.0).all()
    check_heads(w, (o, lse, *views), [(0, 0), (0, 2)])


def test_stages_compose_to_bwd_bitwise():
    """preprocess -> dK/dV -> dQ equals flash_attn_bwd bit for bit, also with
    dK/dV and dQ on two streams after the preprocess."""
    import torch
    import io_aware_exact_08_amd as fa
    w = si.random_case(2, 2, 333, 64, si.FMT_F16, True, seed=21, with_do=True)
    q, k, v, do = dev_inputs(w)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=True, scale=w.scale)
    ref = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    ws = torch.empty(fa.workspace_bytes(2, 2, 333, 64) // 4, dtype=torch.float32, device="cuda")
    fa.flash_attn_bwd_preprocess(o, lse, do, ws)
    dk, dv = fa.flash_attn_bwd_dkdv(q, k, v, do, ws, causal=True, scale=w.scale)
    dq = fa.flash_attn_bwd_dq(q, k, v, do, ws, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a_, b_ in zip((dq, dk, dv), ref):
        assert torch.equal(a_, b_)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    fa.flash_attn_bwd_preprocess(o, lse, do, ws)
    done = torch.cuda.Event()
    done.record()
    s1.wait_event(done)
    s2.wait_event(done)
    with torch.cuda.stream(s1):
        dk2, dv2 = fa.flash_attn_bwd_dkdv(q, k, v, do, ws, causal=True, scale=w.scale)
    with torch.cuda.stream(s2):
        dq2 = fa.flash_attn_bwd_dq(q, k, v, do, ws, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a_, b_ in zip((dq2, dk2, dv2), ref):
        assert torch.equal(a_, b_)


# ----------------------------------------------------------------------------
# backward with an additive attention bias
# ----------------------------------------------------------------------------
def run_bias_fwd_bwd(w, bias_bits, out_f32=False):
    import torch
    import io_aware_exact_08_amd as fa
    from gpu_helpers import to_dev
    q, k, v, do = dev_inputs(w)
    bias = to_dev(bias_bits, w.fmt)
    o, lse = fa.flash_attn_fwd_bias(q, k, v, bias, causal=w.causal, scale=w.scale, out_f32=out_f32)
    dq, dk, dv = fa.flash_attn_bwd_bias(q, k, v, bias, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_bias_grads(w, bias_bits, res, tag=""):
    q, k, v, do = w.f64("q"), w.f64("k"), w.f64("v"), w.f64("do")
    bias = si.bits_to_f64(bias_bits, w.fmt)
    g_ref = oracle.backward(q, k, v, do, w.scale, w.causal, bias)
    errs = [check_grad(name, g, gr, w.fmt, tag=w.name + tag)
            for name, g, gr in zip(("dq", "dk", "dv"), (f64(t) for t in res), g_ref)]
    print(f"{w.name}{tag}: " + " ".join(f"{n} rel={e[0]:.2e} row={e[1]:.2e}"
                                        for n, e in zip(("dq", "dk", "dv"), errs)), flush=True)
    return g_ref


@pytest.mark.parametrize("fmt,out_f32", [(si.FMT_F16, False), (si.FMT_BF16, True)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [8, 64, 136, 264])
@pytest.mark.parametrize("layout", ["shared", "per_batch_head"])
def test_bias_bwd_random(N, d, causal, fmt, out_f32, layout):
    """Random N(0, 2^2) bias with -inf holes and one fully hidden row (whose
    dQ must be exactly zero), broadcast or per (b, h)."""
    w = si.random_case(2, 2, N, d, fmt, causal, seed=9 * N + d, with_do=True)
    shape = (N, N) if layout == "shared" else (2, 2, N, N)
    bb = si.attn_bias(shape, fmt, [N, d, 5], "random")
    res = run_bias_fwd_bwd(w, bb, out_f32=out_f32)
    check_bias_grads(w, bb, res, tag=f" {layout}")
    if N > 3:
        assert np.all(f64(res[0])[:, :, 3] == 0.0), "hidden row must have dQ = 0"


def test_bias_bwd_keypad():
    """Per-batch key padding at B=2 H=2 N=1024 d=64 fp16: batch 0 sees keys
    < 300, batch 1 all of them; every gradient element."""
    w = si.random_case(2, 2, 1024, 64, si.FMT_F16, False, seed=41, with_do=True)
    bb = si.attn_bias((2, 1, 1024, 1024), w.fmt, [41], "keypad", lengths=[300, 1024])
    res = run_bias_fwd_bwd(w, bb)
    check_bias_grads(w, bb, res, tag=" keypad")
    # hidden keys receive no gradient
    assert np.all(f64(res[1])[0, :, 300:] == 0.0) and np.all(f64(res[2])[0, :, 300:] == 0.0)


def test_bias_bwd_zero_equals_plain():
    import torch
    import io_aware_exact_08_amd as fa
    w = si.random_case(1, 3, 512, 64, si.FMT_F16, True, seed=43, with_do=True)
    res_b = run_bias_fwd_bwd(w, np.zeros((512, 512), dtype=np.uint16))
    q, k, v, do = dev_inputs(w)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=True, scale=w.scale)
    res = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a_, b_ in zip(res_b, res):
        assert torch.equal(a_, b_)
