"""Forward parity: the HIP kernel through the C ABI against the fp64 oracle on
the same seeded 16-bit inputs.

Bounds: max|dO| <= 2e-3 (fp16) or 8e-3 (bf16) and max|dLSE| <= 1e-3.  Where O
is stored in bf16 and the exact O reaches 2 in magnitude, rounding the exact
O to bf16 alone costs up to half a bf16 ulp (7.8e-3 for |O| in [2, 4)), so
there the 8e-3 bound applies to each element's error beyond half an ulp of
the exact value; everywhere else (fp16, float32 O, bf16 O below 2, and the
long causal bf16 workload, whose O is small) it applies to the plain error.
The spiked bf16 causal workload is gated on its float32-output variant, and
its bf16-output run must equal the float32 run rounded to bf16, bit for bit.
"""
import numpy as np
import pytest

import oracle
from synth import inputs as si
from gpu_helpers import TOL_LSE, TOL_O, dev_inputs, f64, o_error, oracle_forward, run_fwd

pytestmark = pytest.mark.gpu


def check(w, o, lse, rows=None, tol_o=None, tag="", plain=False):
    """Every element (or the listed (b, h, i) rows) against the oracle."""
    tol_o = TOL_O[w.fmt] if tol_o is None else tol_o
    og, lg = f64(o), f64(lse)
    if rows is None:
        ref = oracle_forward(w)
        o_ref = np.stack([np.stack([ref[(b, h)][0] for h in range(w.H)]) for b in range(w.B)])
        l_ref = np.stack([np.stack([ref[(b, h)][1] for h in range(w.H)]) for b in range(w.B)])
    else:
        q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
        o_ref, l_ref = oracle.forward_rows(q, k, v, rows, w.scale, w.causal)
        idx = tuple(np.array(rows).T)
        og, lg = og[idx], lg[idx]
    eo, el = np.abs(og - o_ref).max(), np.abs(lg - l_ref).max()
    bf16_store = str(o.dtype) == "torch.bfloat16"
    gated, how = o_error(og, o_ref, bf16_store, plain=plain)
    print(f"{w.name}{tag}: max|dO|={eo:.3e} (checked: {how} {gated:.3e})"
          f" max|dLSE|={el:.3e} elements={og.size}", flush=True)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    assert gated <= tol_o, (w.name, eo, gated, how)
    assert el <= TOL_LSE, (w.name, el)


def test_tiny_fwd_workload():
    """B=1 H=4 N=128 d=64 fp16, non-causal, full comparison."""
    w = si.tiny_fwd()
    o, lse = run_fwd(w)
    check(w, o, lse)


@pytest.mark.parametrize("fmt,out_f32", [(si.FMT_F16, False), (si.FMT_BF16, False),
                                         (si.FMT_F16, True), (si.FMT_BF16, True)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 2, 17, 64, 100, 129, 256, 300, 520])
def test_small_shapes(N, d, causal, fmt, out_f32):
    """Tails, single tiles, several tiles, every head dim, masks and dtypes."""
    w = si.random_case(1, 2, N, d, fmt, causal, seed=N + d)
    o, lse = run_fwd(w, out_f32=out_f32)
    check(w, o, lse)


@pytest.mark.parametrize("fmt,d", [(si.FMT_F16, 64), (si.FMT_BF16, 64), (si.FMT_F16, 128), (si.FMT_BF16, 128)])
@pytest.mark.parametrize("N", [700, 1000, 1536])
def test_causal_fully_visible_rounds(N, d, fmt):
    """Causal forwards run whole rounds (four key tiles) of tiles that every
    row of the 128-row workgroup sees through a loop body without masks, then
    the rest (a partial round, the diagonal, a ragged end) through the masked
    one.  Query tile qt has 2 qt such tiles at d = 64 (a partial round left
    over when qt is odd) and 4 qt at d = 128; the last tiles of N = 700 and
    1000 are ragged, N = 1536 is not.  Every element against the oracle."""
    w = si.random_case(1, 2, N, d, fmt, True, seed=N + 3 * d + (fmt == si.FMT_BF16))
    o, lse = run_fwd(w)
    check(w, o, lse)


@pytest.mark.parametrize("N", [1024, 2048, 4096, 8192])
def test_a100_shape_full(N):
    """B=2 H=12 d=64 fp16 non-causal at the A100 table's shape, in the
    benchmark's launch configuration, every element of every head."""
    w = si.a100_sweep(N)
    o, lse = run_fwd(w)
    check(w, o, lse)


def test_spiked_causal_bf16():
    """B=2 H=16 N=4096 d=128 bf16 causal, every 64th key x8: the float32-O run
    on every element of all 32 heads, and the bf16-O run equal to it rounded."""
    w = si.spiked_causal()
    o32, lse = run_fwd(w, out_f32=True)
    check(w, o32, lse, tag=" fp32 O")
    o16, lse16 = run_fwd(w, out_f32=False)
    import torch
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 O differs from rounded fp32 O"
    assert torch.equal(lse16, lse)


def test_long_causal_sampled_rows():
    """B=1 H=8 N=32768 d=64 bf16 N(0, 0.5^2) causal on the sampled rows, O
    stored in bf16 and held to the plain 8e-3 bound."""
    w = si.long_causal()
    o, lse = run_fwd(w)
    rows = [(0, int(h), int(i)) for h, i in si.long_causal_sample_rows(w.H, w.N)]
    check(w, o, lse, rows=rows, plain=True)


def test_long_causal_full_2048():
    """The same distribution at N=2048, every element, plain 8e-3 bound on the
    bf16-stored O."""
    w = si.long_causal(N=2048)
    o, lse = run_fwd(w)
    check(w, o, lse, plain=True)


# ----------------------------------------------------------------------------
# metamorphic and robustness checks on the GPU
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_constant_output(causal):
    import torch
    import io_aware_exact_08_amd as fa
    w = si.random_case(2, 3, 333, 64, si.FMT_F16, causal, seed=5)
    q, k, _ = dev_inputs(w)
    c = torch.linspace(-3, 3, 64, dtype=torch.float32).to(torch.float16)
    v = c.to("cuda").expand(2, 3, 333, 64).contiguous()
    o, _ = fa.flash_attn_fwd(q, k, v, causal=causal, scale=w.scale, out_f32=True)
    torch.cuda.synchronize()
    err = (o - c.float().cuda()).abs().max().item()
    assert err <= 2e-3, err


def test_causal_future_poison_is_bit_identical():
    """Large finite garbage in keys/values after row i0 leaves rows <= i0
    bit-identical (masked probabilities are exactly zero)."""
    import torch
    import io_aware_exact_08_amd as fa
    w = si.random_case(1, 4, 700, 64, si.FMT_F16, True, seed=9)
    q, k, v = dev_inputs(w)
    o1, l1 = fa.flash_attn_fwd(q, k, v, causal=True, scale=w.scale)
    i0 = 301
    k2, v2 = k.clone(), v.clone()
    k2[:, :, i0 + 1:] = 30.0
    v2[:, :, i0 + 1:] = 6.0e4
    o2, l2 = fa.flash_attn_fwd(q, k2, v2, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, : i0 + 1], o2[:, :, : i0 + 1])
    assert torch.equal(l1[:, :, : i0 + 1], l2[:, :, : i0 + 1])
    assert not torch.equal(o1[:, :, i0 + 1:], o2[:, :, i0 + 1:])


def test_deterministic_and_in_bounds():
    """Repeated runs are bitwise equal and nothing is written outside O and LSE."""
    import torch
    import io_aware_exact_08_amd as fa
    w = si.random_case(2, 3, 777, 128, si.FMT_BF16, False, seed=11)
    q, k, v = dev_inputs(w)
    n, pad = 2 * 3 * 777 * 128, 4096
    o_big = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    l_big = torch.full((2 * 3 * 777 + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    o = o_big[pad:pad + n].view(2, 3, 777, 128)
    lse = l_big[pad:pad + 2 * 3 * 777].view(2, 3, 777)
    fa.flash_attn_fwd(q, k, v, scale=w.scale, o=o, lse=lse)
    o_again, l_again = fa.flash_attn_fwd(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_again) and torch.equal(lse, l_again)
    assert (o_big[:pad] == 7.0).all() and (o_big[pad + n:] == 7.0).all()
    assert (l_big[:pad] == 7.0).all() and (l_big[pad + 2 * 3 * 777:] == 7.0).all()
    check(w, o, lse)


@pytest.mark.parametrize("fmt,out_f32,causal", [(si.FMT_F16, False, False), (si.FMT_BF16, True, True)])
def test_head_dim_256_full(fmt, out_f32, causal):
    """d=256 (LDS-resident Q, three K/V stages) at B=1 H=4 N=1000: 32 key
    tiles and a ragged tail, every element."""
    w = si.random_case(1, 4, 1000, 256, fmt, causal, seed=256)
    o, lse = run_fwd(w, out_f32=out_f32)
    check(w, o, lse)


@pytest.mark.parametrize("causal", [False, True])
def test_head_dim_256_bench_shape(causal):
    """d=256 at B=2 H=8 N=4096 bf16 (float32 O), the benchmarked shape, every
    element."""
    w = si.random_case(2, 8, 4096, 256, si.FMT_BF16, causal, seed=257)
    o, lse = run_fwd(w, out_f32=True)
    check(w, o, lse)


def test_errors_through_binding():
    import torch
    import io_aware_exact_08_amd as fa
    x = torch.zeros(1, 1, 16, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        fa.flash_attn_fwd(x.float(), x.float(), x.float())
    big = torch.zeros(1 * 1 * 16 * 64 + 1, dtype=torch.float16, device="cuda")
    mis = big[1:].view(1, 1, 16, 64)  # 2-byte offset: not 16-byte aligned
    with pytest.raises(fa.FlashAttnError) as ei:
        fa.flash_attn_fwd(mis, x, x)
    assert ei.value.status == 5
    y = torch.zeros(1, 1, 16, 96, dtype=torch.float16, device="cuda")
    with pytest.raises(fa.FlashAttnError) as ei:
        fa.flash_attn_fwd(y, y, y)
    assert ei.value.status == 3


# ----------------------------------------------------------------------------
# split-KV forward (key range cut over several workgroups, merged by LSE)
# ----------------------------------------------------------------------------
def run_splitkv(w, num_splits, out_f32=False):
    import torch
    import io_aware_exact_08_amd as fa
    q, k, v = dev_inputs(w)[:3]
    o, lse = fa.flash_attn_fwd_splitkv(q, k, v, causal=w.causal, scale=w.scale, out_f32=out_f32,
                                       num_splits=num_splits)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("fmt,out_f32", [(si.FMT_F16, False), (si.FMT_BF16, True)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N,splits", [(1, 1), (1, 3), (37, 2), (64, 5), (200, 2), (200, 3),
                                      (520, 4), (520, 64), (1000, 7)])
def test_splitkv_small_shapes(N, splits, d, causal, fmt, out_f32):
    """Every split count from one to more splits than key tiles (empty ranges),
    ragged N, both head dims, causal ranges that end before some rows begin."""
    w = si.random_case(1, 2, N, d, fmt, causal, seed=3 * N + d + splits)
    o, lse = run_splitkv(w, splits, out_f32=out_f32)
    check(w, o, lse, tag=f" splits={splits}")


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_a100_shape(causal):
    """B=2 H=12 N=1024 d=64 fp16 (the A100 table's smallest N) in three splits,
    every element; also within the bound of the unsplit forward's output."""
    w = si.a100_sweep(1024)
    w.causal = causal
    o, lse = run_splitkv(w, 3)
    check(w, o, lse, tag=" splits=3")
    o1, l1 = run_fwd(w)
    assert (o.float() - o1.float()).abs().max().item() <= 2e-3
    assert (lse - l1).abs().max().item() <= 1e-3


def test_splitkv_default_splits_few_heads():
    """B=1 H=4 N=8192 d=128 bf16 (fp32 O), where the default splits the key
    range (256 unsplit workgroups), every element."""
    import io_aware_exact_08_amd as fa
    w = si.random_case(1, 4, 8192, 128, si.FMT_BF16, False, seed=11)
    assert fa._lib.flash_attn_fwd_splitkv_default_splits(1, 4, 8192, 128, 0) == 2
    o, lse = run_splitkv(w, 0, out_f32=True)
    check(w, o, lse, tag=" default splits")


def test_splitkv_long_causal_sampled():
    """B=1 H=8 N=32768 d=64 bf16 causal, 16 splits, on the sampled rows."""
    w = si.long_causal()
    o, lse = run_splitkv(w, 16)
    rows = [(0, int(h), int(i)) for h, i in si.long_causal_sample_rows(w.H, w.N)]
    check(w, o, lse, rows=rows, tag=" splits=16", plain=True)


# ----------------------------------------------------------------------------
# additive attention bias
# ----------------------------------------------------------------------------
def run_bias(w, bias_bits, out_f32=False):
    import torch
    import io_aware_exact_08_amd as fa
    from gpu_helpers import to_dev
    q, k, v = dev_inputs(w)[:3]
    bias = to_dev(bias_bits, w.fmt)
    o, lse = fa.flash_attn_fwd_bias(q, k, v, bias, causal=w.causal, scale=w.scale,
                                    out_f32=out_f32)
    torch.cuda.synchronize()
    return o, lse


def check_bias(w, bias_bits, o, lse, tag=""):
    q, k, v = w.f64("q"), w.f64("k"), w.f64("v")
    bias = si.bits_to_f64(bias_bits, w.fmt)
    o_ref, l_ref = oracle.forward(q, k, v, w.scale, w.causal, bias)
    og, lg = f64(o), f64(lse)
    dead = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lg), dead), "rows with every key hidden must give LSE = -inf"
    assert np.all(og[dead] == 0.0), "rows with every key hidden must give O = 0"
    live = ~dead
    eo = np.abs(og[live] - o_ref[live]).max() if live.any() else 0.0
    el = np.abs(lg[live] - l_ref[live]).max() if live.any() else 0.0
    gated = o_error(og[live], o_ref[live], str(o.dtype) == "torch.bfloat16")[0] if live.any() else 0.0
    print(f"{w.name}{tag}: max|dO|={eo:.3e} max|dLSE|={el:.3e} hidden rows={int(dead.sum())}",
          flush=True)
    assert np.isfinite(og).all()
    assert gated <= TOL_O[w.fmt] and el <= TOL_LSE, (eo, gated, el)


@pytest.mark.parametrize("fmt,out_f32", [(si.FMT_F16, False), (si.FMT_BF16, True)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [8, 64, 200, 520])
@pytest.mark.parametrize("layout", ["shared", "per_head", "per_batch_head"])
def test_bias_random(N, d, causal, fmt, out_f32, layout):
    """Random N(0, 2^2) bias with 20% of entries -inf and one row fully hidden,
    broadcast as [N, N], [H, N, N] or stored as [B, H, N, N]."""
    w = si.random_case(2, 2, N, d, fmt, causal, seed=5 * N + d)
    shape = {"shared": (N, N), "per_head": (2, N, N), "per_batch_head": (2, 2, N, N)}[layout]
    bb = si.attn_bias(shape, fmt, [N, d, len(shape)], "random")
    o, lse = run_bias(w, bb, out_f32=out_f32)
    check_bias(w, bb, o, lse, tag=f" {layout}")


def test_bias_zero_equals_plain_forward():
    import torch
    w = si.random_case(1, 3, 256, 64, si.FMT_F16, False, seed=21)
    zero = np.zeros((256, 256), dtype=np.uint16)
    o, lse = run_bias(w, zero)
    o0, l0 = run_fwd(w)
    assert torch.equal(o, o0) and torch.equal(lse, l0)


@pytest.mark.parametrize("kind,kw", [("window", dict(width=100)), ("keypad", dict(lengths=[300, 2048]))])
def test_bias_masks_long(kind, kw):
    """Sliding-window band and per-batch key padding at N=2048 (B=2 H=2 d=64
    fp16), every element; the window keeps each row 201 keys, the padding
    hides keys past 300 in batch 0."""
    w = si.random_case(2, 2, 2048, 64, si.FMT_F16, False, seed=33)
    bb = si.attn_bias((2, 1, 2048, 2048) if kind == "keypad" else (2048, 2048), w.fmt, [33], kind,
                      **kw)
    o, lse = run_bias(w, bb)
    check_bias(w, bb, o, lse, tag=f" {kind}")


@pytest.mark.parametrize("kind", ["window", "leftpad"])
def test_bias_hidden_first_tiles_low_logits_f16(kind):
    """fp16, B=1 H=2 N=1024 d=64, non-causal.  The bias hides whole leading key
    tiles of many rows (a band |i - j| <= 100, or every key j < 300), and each
    visible entry carries -20, so against a reference of 0 every exponent of
    those rows would underflow fp16.  Checked against the oracle, and against
    the run without the -20: the same O and an LSE lower by 20 (softmax shift
    invariance)."""
    import torch
    w = si.random_case(1, 2, 1024, 64, si.FMT_F16, False, seed=77)
    i = np.arange(w.N)[:, None]
    j = np.arange(w.N)[None, :]
    vis = (np.abs(i - j) <= 100) if kind == "window" else (j >= 300) & (i >= 0)
    b0 = si.f32_to_bits(np.where(vis, 0.0, -np.inf).astype(np.float32), w.fmt)
    b20 = si.f32_to_bits(np.where(vis, -20.0, -np.inf).astype(np.float32), w.fmt)
    o20, l20 = run_bias(w, b20)
    check_bias(w, b20, o20, l20, tag=f" {kind} -20")
    o0, l0 = run_bias(w, b0)
    assert (o20.float() - o0.float()).abs().max().item() <= 2e-3
    assert ((l20 - l0) + 20.0).abs().max().item() <= 1e-3
    assert torch.isfinite(l20).all()


@pytest.mark.parametrize("B,H,N,d,fmt,causal,out_f32", [
    (2, 12, 4096, 64, si.FMT_F16, False, False),   # 1.5 rounds: half a round, no split
    (2, 12, 8200, 64, si.FMT_F16, False, False),   # ragged N: 1536 tiles whole, the last 24 in 16
    (1, 4, 8192, 128, si.FMT_BF16, False, True),   # half a round: every tile split in two
    (2, 12, 1024, 64, si.FMT_F16, False, False),   # short key range: no split
    (2, 12, 4096, 64, si.FMT_F16, True, False),    # causal: the uniform default
    (1, 3, 3000, 256, si.FMT_BF16, False, True),   # d=256 (one workgroup per compute unit)
])
def test_splitkv_automatic_plan(B, H, N, d, fmt, causal, out_f32):
    """num_splits = 0 (the library's plan) on every element, and within the
    bound of the plain forward's output."""
    w = si.random_case(B, H, N, d, fmt, causal, seed=N + d + 7)
    o, lse = run_splitkv(w, 0, out_f32=out_f32)
    check(w, o, lse, tag=" automatic splits")
    o1, l1 = run_fwd(w, out_f32=out_f32)
    assert (o.float() - o1.float()).abs().max().item() <= TOL_O[fmt]
    assert (lse - l1).abs().max().item() <= TOL_LSE
