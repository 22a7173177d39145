"""The allocation-free backward (workspace in the library's static device
scratch) through the C ABI, against flash_attn_bwd with a caller workspace on
the same inputs: bit-identical dQ, dK, dV on two calls in a row, the second
with a smaller input than the first."""
import pytest

from synth import inputs as si
from gpu_helpers import dev_inputs

pytestmark = pytest.mark.gpu


def _pair(w):
    import torch
    import io_aware_exact_08_amd as fa
    q, k, v, do = dev_inputs(w)
    o, lse = fa.flash_attn_fwd(q, k, v, causal=w.causal, scale=w.scale)
    ref = fa.flash_attn_bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    got = fa.flash_attn_bwd_noalloc(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_bwd_on_two_calls_second_smaller():
    import torch
    big = si.random_case(2, 6, 3000, 64, si.FMT_F16, True, seed=61, with_do=True)
    small = si.random_case(1, 2, 333, 128, si.FMT_BF16, False, seed=62, with_do=True)
    for w in (big, small):
        ref, got = _pair(w)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), (w.name, name)
        print(f"{w.name}: noalloc == bwd", flush=True)


def test_noalloc_at_its_row_limit():
    """B*H*N = 2^21 rows (all 16 MiB of the scratch): equal to flash_attn_bwd."""
    import torch
    w = si.random_case(1, 256, 8192, 64, si.FMT_F16, False, seed=63, with_do=True)
    ref, got = _pair(w)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
