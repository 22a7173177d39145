"""Pins for the fp64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: closed forms
derived by hand from the definition softmax(sigma Q K^T) V (page 1, examples
1-3; page 2, "Kernel Fusion"), invariants of that definition, the pages' claim
that blockwise online softmax equals the full computation (page 2, "Tiling"),
the query-chunked loop of page 1 example 2, brute force on tiny inputs, and
finite-difference gradients (the small-scale gradient check that page 1
recommends in its precision practice and FAQ).  The cases are chosen so that a
dropped term, a wrong sign or index, a transposed operand, a missing scale or
an off-by-one causal mask fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------
def test_hand_closed_forms():
    """Three cases computed by hand from the definition."""
    e = math.e
    Z = e + 1.0 + 1.0 / e
    ln3 = math.log(3.0)
    cases = [
        # s = (0, ln 3) -> weights (1/4, 3/4) -> O = 1 + 6; equal scores -> mean.
        dict(scale=1.0, causal=False, q=[[1.0], [0.0]], k=[[0.0], [ln3]], v=[[4.0], [8.0]],
             o=[[7.0], [6.0]], lse=[math.log(4.0), math.log(2.0)]),
        # causal: row 0 sees key 0 only.
        dict(scale=1.0, causal=True, q=[[1.0], [0.0]], k=[[0.0], [ln3]], v=[[4.0], [8.0]],
             o=[[4.0], [6.0]], lse=[0.0, math.log(2.0)]),
        # s = 0.5 * (2, 0, -2) = (1, 0, -1) -> weights (e, 1, 1/e) / Z.
        dict(scale=0.5, causal=False, q=[[2.0, 0.0]], k=[[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0]],
             v=[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]],
             o=[[(e + 1 / e) / Z, (1 + 1 / e) / Z]], lse=[math.log(Z)]),
    ]
    for c in cases:
        q, k, v = (np.array(c[n], dtype=np.float64) for n in "qkv")
        o, lse = oracle.forward_head(q, k, v, c["scale"], c["causal"])
        np.testing.assert_allclose(o, np.array(c["o"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_single_key(causal):
    """N = 1: O = V, LSE = sigma q.k."""
    q, k, v = rand((1, 5), 1), rand((1, 5), 2), rand((1, 3), 3)
    o, lse = oracle.forward_head(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, v, atol=1e-15)
    np.testing.assert_allclose(lse, [0.3 * float(q[0] @ k[0])], atol=1e-14)


def test_two_keys_sigmoid():
    """N = 2: O_i = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1; LSE = logaddexp(s0, s1)."""
    q, k, v = rand((2, 4), 4), rand((2, 4), 5), rand((2, 3), 6)
    sc = 0.7
    o, lse = oracle.forward_head(q, k, v, sc, False)
    for i in range(2):
        s0, s1 = sc * float(q[i] @ k[0]), sc * float(q[i] @ k[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        np.testing.assert_allclose(o[i], w0 * v[0] + w1 * v[1], atol=1e-14)
        np.testing.assert_allclose(lse[i], np.logaddexp(s0, s1), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_is_mean(causal):
    """Q = 0: every visible key has score 0, so O_i = mean of visible V rows and
    LSE_i = ln(#visible)."""
    N = 9
    q = np.zeros((N, 4))
    k, v = rand((N, 4), 7), rand((N, 5), 8)
    o, lse = oracle.forward_head(q, k, v, 0.5, causal)
    for i in range(N):
        nvis = i + 1 if causal else N
        np.testing.assert_allclose(o[i], v[:nvis].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[i], math.log(nvis), atol=1e-14)


# ----------------------------------------------------------------------------
# Invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    """With V = identity (d_v = N) the output row is the probability row itself:
    non-negative, summing to 1, zero on masked keys (page 2, "Tiling", final
    normalisation)."""
    N = 12
    q, k = rand((N, 6), 9, 2.0), rand((N, 6), 10, 2.0)
    p, _ = oracle.forward_head(q, k, np.eye(N), 0.4, causal)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(axis=1), np.ones(N), atol=1e-14)
    if causal:
        assert np.all(p[np.triu_indices(N, 1)] == 0.0)
    # and P itself matches exp(s - LSE) using the LSE the oracle returns
    _, lse = oracle.forward_head(q, k, rand((N, 2), 1), 0.4, causal)
    s = 0.4 * q @ k.T
    ref = np.exp(s - lse[:, None])
    if causal:
        ref = np.tril(ref)
    np.testing.assert_allclose(p, ref, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_value_rows(causal):
    """Every V row equal to c gives O_i = c regardless of Q and K."""
    N = 33
    q, k = rand((N, 8), 11, 3.0), rand((N, 8), 12, 3.0)
    c = rand((8,), 13)
    o, _ = oracle.forward_head(q, k, np.tile(c, (N, 1)), 0.35, causal)
    np.testing.assert_allclose(o, np.tile(c, (N, 1)), atol=1e-13)


def test_affine_in_values():
    """V -> a V + 1 b^T gives O -> a O + 1 b^T (O is a convex combination)."""
    N = 20
    q, k, v = rand((N, 6), 14), rand((N, 6), 15), rand((N, 4), 16)
    a, b = -2.5, rand((4,), 17)
    o1, l1 = oracle.forward_head(q, k, v, 0.41, True)
    o2, l2 = oracle.forward_head(q, k, a * v + b, 0.41, True)
    np.testing.assert_allclose(o2, a * o1 + b, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=0)


def test_joint_key_value_permutation():
    """Non-causal: permuting K and V rows together leaves O and LSE unchanged;
    permuting only V changes O (catches a transposed P)."""
    N = 31
    q, k, v = rand((N, 8), 18), rand((N, 8), 19), rand((N, 8), 20)
    perm = np.random.default_rng(21).permutation(N)
    o1, l1 = oracle.forward_head(q, k, v, 0.3, False)
    o2, l2 = oracle.forward_head(q, k[perm], v[perm], 0.3, False)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)
    o3, _ = oracle.forward_head(q, k, v[perm], 0.3, False)
    assert np.abs(o3 - o1).max() > 1e-3


def test_query_permutation_equivariance():
    """Non-causal: permuting Q rows permutes O rows and LSE."""
    N = 17
    q, k, v = rand((N, 8), 22), rand((N, 8), 23), rand((N, 8), 24)
    perm = np.random.default_rng(25).permutation(N)
    o1, l1 = oracle.forward_head(q, k, v, 0.3, False)
    o2, l2 = oracle.forward_head(q[perm], k, v, 0.3, False)
    np.testing.assert_allclose(o2, o1[perm], atol=1e-13)
    np.testing.assert_allclose(l2, l1[perm], atol=1e-13)


def test_causal_future_poison():
    """Causal: overwriting K and V rows j > i with large finite garbage leaves
    rows <= i unchanged; row 0 is V_0 with LSE sigma q_0.k_0."""
    N = 24
    q, k, v = rand((N, 8), 26), rand((N, 8), 27), rand((N, 8), 28)
    o, lse = oracle.forward_head(q, k, v, 0.25, True)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.25 * float(q[0] @ k[0]), atol=1e-14)
    for i in (0, 5, 13, N - 2):
        k2, v2 = k.copy(), v.copy()
        k2[i + 1:] = 1e4 * rand((N - i - 1, 8), 100 + i)
        v2[i + 1:] = 1e6
        o2, l2 = oracle.forward_head(q, k2, v2, 0.25, True)
        np.testing.assert_allclose(o2[: i + 1], o[: i + 1], atol=1e-13)
        np.testing.assert_allclose(l2[: i + 1], lse[: i + 1], atol=1e-13)
        # and the non-causal result does see the poison
        o3, _ = oracle.forward_head(q, k2, v2, 0.25, False)
        assert np.abs(o3[: i + 1] - o[: i + 1]).max() > 1.0


def test_key_shift_invariance():
    """K -> K + 1 u^T leaves O unchanged and adds sigma q_i.u to LSE_i (softmax
    is invariant to a per-row constant)."""
    N = 19
    q, k, v = rand((N, 8), 29), rand((N, 8), 30), rand((N, 8), 31)
    u = rand((8,), 32)
    for causal in (False, True):
        o1, l1 = oracle.forward_head(q, k, v, 0.3, causal)
        o2, l2 = oracle.forward_head(q, k + u, v, 0.3, causal)
        np.testing.assert_allclose(o2, o1, atol=1e-13)
        np.testing.assert_allclose(l2, l1 + 0.3 * (q @ u), atol=1e-12)


def test_scale_enters_scores():
    """Doubling sigma equals doubling Q (catches a dropped or misplaced scale)."""
    N = 14
    q, k, v = rand((N, 8), 33), rand((N, 8), 34), rand((N, 8), 35)
    o1, l1 = oracle.forward_head(q, k, v, 0.6, False)
    o2, l2 = oracle.forward_head(2 * q, k, v, 0.3, False)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    o3, _ = oracle.forward_head(q, k, v, 0.3, False)
    assert np.abs(o3 - o1).max() > 1e-3


# ----------------------------------------------------------------------------
# Blockwise / chunked equal full (page 2 "Tiling"; page 1 example 2)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 3, 64, 200])
def test_online_softmax_blocks_equal_full(causal, block):
    N = 200
    q, k, v = rand((N, 16), 36, 2.0), rand((N, 16), 37, 2.0), rand((N, 16), 38)
    o_ref, l_ref = oracle.forward_head(q, k, v, 0.25, causal)
    o, l = oracle.forward_key_blocked(q, k, v, 0.25, causal, block)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("chunk", [1, 7, 128])
def test_query_chunks_equal_full(causal, chunk):
    N = 150
    q, k, v = rand((N, 16), 39), rand((N, 16), 40), rand((N, 16), 41)
    o_ref, l_ref = oracle.forward_head(q, k, v, 0.25, causal)
    o, l = oracle.forward_query_chunked(q, k, v, 0.25, causal, chunk)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(l, l_ref, atol=1e-13)


def test_page1_example2_shape():
    """Page 1 example 2 runs chunked attention on (2, 4, 1024, 64) with chunk 128
    and prints an output of the query's shape."""
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))["chunked_attention_shape"]
    B, H, N, d = facts["input_shape"]
    # seed convention of that example: PRNG keys 0, 1, 2 for q, k, v
    q = rand((N, d), 0)
    k = rand((N, d), 1)
    v = rand((N, d), 2)
    o, _ = oracle.forward_query_chunked(q, k, v, 1 / math.sqrt(d), False, facts["chunk_size"])
    assert [B, H] + list(o.shape) == facts["output_shape"]
    o_ref, _ = oracle.forward_head(q, k, v, 1 / math.sqrt(d), False)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)


# ----------------------------------------------------------------------------
# Brute force on tiny inputs
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 1), (2, 3), (5, 4), (8, 2)])
def test_bruteforce_tiny(causal, n, d):
    q, k, v = rand((n, d), 42 + n), rand((n, d), 43 + n), rand((n, d + 1), 44 + n)
    o_ref, l_ref = oracle.forward_scalar(q.tolist(), k.tolist(), v.tolist(), 0.6, causal)
    o, l = oracle.forward_head(q, k, v, 0.6, causal)
    np.testing.assert_allclose(o, o_ref, atol=1e-14)
    np.testing.assert_allclose(l, l_ref, atol=1e-14)


def test_batched_forward_matches_heads_and_rows():
    B, H, N, d = 2, 3, 40, 8
    q, k, v = rand((B, H, N, d), 45), rand((B, H, N, d), 46), rand((B, H, N, d), 47)
    for causal in (False, True):
        o, l = oracle.forward(q, k, v, 0.3, causal)
        rows = [(1, 2, 0), (0, 1, 17), (1, 0, N - 1)]
        orow, lrow = oracle.forward_rows(q, k, v, rows, 0.3, causal)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(orow[n], o[b, h, i], atol=1e-13)
            np.testing.assert_allclose(lrow[n], l[b, h, i], atol=1e-13)
            o1, l1 = oracle.forward_scalar(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(),
                                           0.3, causal)
            np.testing.assert_allclose(orow[n], o1[i], atol=1e-13)
            np.testing.assert_allclose(lrow[n], l1[i], atol=1e-13)


# ----------------------------------------------------------------------------
# Gradients: central finite differences of L = <dO, O>
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 2), (3, 4), (7, 2), (7, 4)])
def test_gradients_finite_difference(causal, n, d):
    B, H = 1, 2
    q, k, v = rand((B, H, n, d), 50 + n), rand((B, H, n, d), 51 + n), rand((B, H, n, d), 52 + n)
    do = rand((B, H, n, d), 53 + n)
    sc = 0.45
    dq, dk, dv = oracle.backward(q, k, v, do, sc, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.forward(q_, k_, v_, sc, causal)
        return float((o * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.linalg.norm(fd - g) / max(np.linalg.norm(fd), 1e-30)
        if n == 1 and name != "v":
            # one key: O = V regardless of q and k, so dq = dk = 0 exactly
            assert np.abs(g).max() < 1e-12 and np.abs(fd).max() < 1e-6
        else:
            assert err < 1e-6, (name, err)


def test_backward_D_identity_and_dv_structure():
    """sum_c dO_ic O_ic equals sum_j P_ij dP_ij, and dV = P^T dO: checked through
    the V = identity trick (O = P) and the public functions."""
    N, d = 11, 5
    q, k = rand((N, d), 60), rand((N, d), 61)
    v, do = rand((N, d), 62), rand((N, d), 63)
    for causal in (False, True):
        p, _ = oracle.forward_head(q, k, np.eye(N), 0.5, causal)
        o, _ = oracle.forward_head(q, k, v, 0.5, causal)
        _, _, dv = oracle.backward_head(q, k, v, do, 0.5, causal)
        np.testing.assert_allclose(dv, p.T @ do, atol=1e-13)
        lhs = (do * o).sum(axis=1)
        rhs = (p * (do @ v.T)).sum(axis=1)
        np.testing.assert_allclose(lhs, rhs, atol=1e-13)


def test_gradient_sums():
    """Softmax rows are shift invariant, so sum_j dS_ij = 0 for each query; hence
    dK summed over keys is zero (dK = sigma dS^T Q), and dQ is unchanged by a
    common shift of all keys."""
    N, d = 16, 6
    q, k, v, do = (rand((1, 1, N, d), s) for s in (64, 65, 66, 67))
    for causal in (False, True):
        dq, dk, dv = oracle.backward(q, k, v, do, 0.3, causal)
        np.testing.assert_allclose(dk[0, 0].sum(axis=0), np.zeros(d), atol=1e-12)
        dq2, dk2, dv2 = oracle.backward(q, k + rand((d,), 68), v, do, 0.3, causal)
        np.testing.assert_allclose(dq2, dq, atol=1e-12)
        np.testing.assert_allclose(dv2, dv, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_gradients_equal_full_backward(causal):
    """The per-row dQ and per-key dK/dV routines (used where the N x N matrices
    are too large) reproduce the full backward, which the finite differences
    above pin; the key routine's forward chunking does not change the result."""
    B, H, N, d = 2, 2, 37, 8
    q, k, v, do = (rand((B, H, N, d), s) for s in (70, 71, 72, 73))
    dq, dk, dv = oracle.backward(q, k, v, do, 0.31, causal)
    sel = [(b, h, i) for b in range(B) for h in range(H) for i in range(N)]
    np.testing.assert_allclose(oracle.backward_dq_rows(q, k, v, do, sel, 0.31, causal),
                               dq.reshape(-1, d), atol=1e-12)
    for chunk in (1, 5, N, 1000):
        dks, dvs = oracle.backward_kv_cols(q, k, v, do, sel, 0.31, causal, chunk=chunk)
        np.testing.assert_allclose(dks, dk.reshape(-1, d), atol=1e-12)
        np.testing.assert_allclose(dvs, dv.reshape(-1, d), atol=1e-12)
    # a sparse, unordered selection over several heads gives the same rows
    few = [(1, 0, 36), (0, 1, 0), (0, 1, 17), (1, 1, 5), (0, 0, 20)]
    dks, dvs = oracle.backward_kv_cols(q, k, v, do, few, 0.31, causal, chunk=4)
    for n, (b, h, j) in enumerate(few):
        np.testing.assert_allclose(dks[n], dk[b, h, j], atol=1e-12)
        np.testing.assert_allclose(dvs[n], dv[b, h, j], atol=1e-12)
    dqs = oracle.backward_dq_rows(q, k, v, do, few, 0.31, causal)
    for n, (b, h, i) in enumerate(few):
        np.testing.assert_allclose(dqs[n], dq[b, h, i], atol=1e-12)


def test_sampled_gradients_finite_difference():
    """Direct pin of the per-row routines: central differences of <dO, O> in one
    query row and in one key row."""
    N, d, sc, h = 6, 3, 0.4, 1e-6
    q, k, v, do = (rand((1, 1, N, d), s) for s in (80, 81, 82, 83))
    for causal in (False, True):
        def loss(q_, k_, v_):
            o, _ = oracle.forward(q_, k_, v_, sc, causal)
            return float((o * do).sum())
        i, j = 4, 2
        g_q = oracle.backward_dq_rows(q, k, v, do, [(0, 0, i)], sc, causal)[0]
        g_k, g_v = oracle.backward_kv_cols(q, k, v, do, [(0, 0, j)], sc, causal, chunk=2)
        for name, x, row, g in (("q", q, i, g_q), ("k", k, j, g_k[0]), ("v", v, j, g_v[0])):
            fd = np.zeros(d)
            for c in range(d):
                xp, xm = x.copy(), x.copy()
                xp[0, 0, row, c] += h
                xm[0, 0, row, c] -= h
                args_p, args_m = [q, k, v], [q, k, v]
                pos = "qkv".index(name)
                args_p[pos], args_m[pos] = xp, xm
                fd[c] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert np.linalg.norm(fd - g) <= 1e-6 * max(np.linalg.norm(fd), 1e-12), (name, causal)


# ----------------------------------------------------------------------------
# Additive attention bias
# ----------------------------------------------------------------------------
def test_bias_special_cases():
    """Zero bias is no bias; a bias constant along each row leaves O unchanged
    and adds that constant to LSE; -inf above the diagonal is the causal mask;
    a bias of log(w_j) reweights the softmax by w_j (checked against a direct
    weighted average); a row of -inf gives O = 0, LSE = -inf."""
    N, d, sc = 9, 4, 0.6
    q, k, v = rand((N, d), 90), rand((N, d), 91), rand((N, d), 92)
    o0, l0 = oracle.forward_head(q, k, v, sc, False)
    o, l = oracle.forward_head(q, k, v, sc, False, np.zeros((N, N)))
    np.testing.assert_allclose(o, o0, atol=1e-14)
    np.testing.assert_allclose(l, l0, atol=1e-14)
    rowc = rand((N, 1), 93)
    o, l = oracle.forward_head(q, k, v, sc, False, np.repeat(rowc, N, axis=1))
    np.testing.assert_allclose(o, o0, atol=1e-13)
    np.testing.assert_allclose(l, l0 + rowc[:, 0], atol=1e-13)
    tri = np.where(np.tri(N) > 0, 0.0, -np.inf)
    oc, lc = oracle.forward_head(q, k, v, sc, True)
    o, l = oracle.forward_head(q, k, v, sc, False, tri)
    np.testing.assert_allclose(o, oc, atol=1e-14)
    np.testing.assert_allclose(l, lc, atol=1e-14)
    w = np.abs(rand((N,), 94)) + 0.1
    o, l = oracle.forward_head(q, k, v, sc, False, np.log(np.broadcast_to(w, (N, N))))
    e = np.exp(sc * (q @ k.T)) * w
    np.testing.assert_allclose(o, (e @ v) / e.sum(axis=1, keepdims=True), atol=1e-12)
    np.testing.assert_allclose(l, np.log(e.sum(axis=1)), atol=1e-12)
    hole = np.zeros((N, N))
    hole[3] = -np.inf
    o, l = oracle.forward_head(q, k, v, sc, True, hole)
    assert np.all(o[3] == 0) and l[3] == -np.inf
    np.testing.assert_allclose(np.delete(o, 3, 0), np.delete(oc, 3, 0), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_bias_gradients_finite_difference(causal):
    """Gradients with a bias (including -inf entries and one fully hidden row):
    central differences of <dO, O> in Q, K and V."""
    B, H, N, d, sc, h = 1, 1, 6, 3, 0.5, 1e-6
    q, k, v, do = (rand((B, H, N, d), s) for s in (95, 96, 97, 98))
    bias = rand((N, N), 99)
    bias[1, 4] = -np.inf
    bias[2] = -np.inf
    dq, dk, dv = oracle.backward(q, k, v, do, sc, causal, bias)
    def loss(q_, k_, v_):
        o, _ = oracle.forward(q_, k_, v_, sc, causal, bias)
        return float((o * do).sum())
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p, args_m = [q, k, v], [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.linalg.norm(fd - g) <= 1e-6 * max(np.linalg.norm(fd), 1e-12), name
    assert np.all(dq[0, 0, 2] == 0)


# ----------------------------------------------------------------------------
# Input generator and tolerance feasibility
# ----------------------------------------------------------------------------
def test_rounding_formats():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e-3, 65504.0],
                    dtype=np.float32)
    bf = si.f32_to_bits(vals, si.FMT_BF16)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1+3*2^-8 ties -> 1+2^-6... even
    np.testing.assert_array_equal(si.bits_to_f32(bf, si.FMT_BF16)[:4],
                                  np.array([1.0, 1.0, 1.0 + 2**-6, 1.0], dtype=np.float32))
    assert si.bits_to_f32(bf, si.FMT_BF16)[4] == -2.5
    f16 = si.f32_to_bits(vals, si.FMT_F16)
    np.testing.assert_array_equal(si.bits_to_f32(f16, si.FMT_F16), vals.astype(np.float16).astype(np.float32))


def test_generator_is_seeded_and_structured():
    a = si.random_case(1, 2, 70, 64, si.FMT_BF16, seed=3)
    b = si.random_case(1, 2, 70, 64, si.FMT_BF16, seed=3)
    np.testing.assert_array_equal(a.q, b.q)
    assert not np.array_equal(a.q, a.k)
    w = si.spiked_causal(N=256, H=2)
    k = si.bits_to_f64(w.k, w.fmt)
    # spiked rows are exactly 8x the unspiked draw
    base = si.normal_bits([3, 1], w.shape, 1.0, si.FMT_BF16)
    kb = si.bits_to_f64(base, w.fmt)
    np.testing.assert_array_equal(k[:, :, ::64], 8 * kb[:, :, ::64])
    mask = np.ones(256, bool)
    mask[::64] = False
    np.testing.assert_array_equal(k[:, :, mask], kb[:, :, mask])
    rows = si.long_causal_sample_rows(8, 32768)
    assert len(rows) >= 256 and (rows[:, 1] < 32768).all()


@pytest.mark.slow
def test_bf16_storage_floor_reaches_tolerance():
    """Rounding the exact O of the spiked bf16 causal workload to bf16 already
    costs about 7.8e-3 (half a bf16 ulp for |O| in [2, 4)) on its first two
    heads, leaving no room under the 8e-3 bound for the kernel's own rounding.
    That workload's gate is therefore applied to the fp32-output variant."""
    w = si.spiked_causal()
    q, k, v = (si.bits_to_f64(getattr(w, n)[0, :2], w.fmt) for n in "qkv")
    floor = 0.0
    for h in range(2):
        o, _ = oracle.forward_head(q[h], k[h], v[h], w.scale, True)
        ob = si.bits_to_f64(si.f32_to_bits(o.astype(np.float32), si.FMT_BF16), si.FMT_BF16)
        floor = max(floor, np.abs(ob - o).max())
    assert floor > 0.95 * 8e-3
