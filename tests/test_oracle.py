"""Pins of the fp64 oracle against what the pages and mathematics fix.

No GPU.  Every check compares the oracle with something other than itself:
values printed on the pages (tests/golden), closed forms, invariants, special
cases that reduce to library routines (scipy's softmax/logsumexp, torch's fp64
autograd), brute-force finite differences, and the tiled formulation.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
from io_aware_tiled_fwd_amd import inputs



def _worked(golden):
    g = golden("worked_example.txt")
    q = np.array(g["q"][0])
    K = np.array([g[f"K{i}"][0] for i in range(4)])
    V = np.array([g[f"V{i}"][0] for i in range(4)])
    return g, q, K, V


def _close(got, want_tol, what):
    want, tol = want_tol
    got = np.atleast_1d(np.asarray(got, dtype=np.float64))
    assert got.shape == (len(want),), what
    err = np.max(np.abs(got - np.array(want)))
    assert err <= tol, f"{what}: got {got}, page prints {want} (tol {tol}, err {err})"


# --- the worked example (page 5) ------------------------------------------------

def test_worked_example_direct(golden):
    """Plain oracle: the query row of the worked example gives the printed output."""
    g, q, K, V = _worked(golden)
    Q = np.zeros((4, 2))
    Q[0] = q
    Q[1:] = [[0.5, -1.0], [2.0, 0.25], [-0.75, 1.5]]  # other rows are independent
    O, L = oracle.attn_fwd(Q, K, V, scale=g["scale"][0][0])
    _close(O[0, 0], g["final_o_printed"], "O (printed program output)")
    _close(O[0, 0], g["final_o_hand"], "O (hand trace)")
    # L = m + ln l, m = 3 is the row max and l the softmax denominator (1.20344)
    _close(np.exp(L[0, 0] - 3.0), g["tile2_l"], "exp(L - m)")
    _close(np.exp(L[0, 0] - 3.0), g["block4_l"], "exp(L - m), one block")


def test_worked_example_probabilities(golden):
    """With V = identity the output row is the probability row."""
    g, q, K, _ = _worked(golden)
    Q = np.zeros((4, 4))
    Q[0, :2] = q
    K4 = np.zeros((4, 4))
    K4[:, :2] = K
    O, _ = oracle.attn_fwd(Q, K4, np.eye(4), scale=1.0)
    _close(O[0, 0], g["probs"], "softmax probabilities")


def test_worked_example_tile_trace(golden):
    """Tiled oracle with key blocks of 2 reproduces the page's per-tile trace."""
    g, q, K, V = _worked(golden)
    Q = np.zeros((4, 2))
    Q[0] = q
    O, L, tr = oracle.attn_fwd_tiled(Q, K, V, scale=1.0, br=4, bc=2, trace_row=0)
    assert tr.shape == (2, 4)
    _close(tr[0, 0], g["tile1_m"], "m after tile 1")
    _close(tr[0, 1], g["tile1_l"], "l after tile 1")
    _close(tr[0, 2:], g["tile1_acc"], "acc after tile 1")
    _close(tr[1, 0], g["tile2_m"], "m after tile 2")
    _close(tr[1, 1], g["tile2_l"], "l after tile 2")
    _close(tr[1, 2:], g["tile2_acc"], "acc after tile 2")
    _close(np.exp(tr[0, 0] - tr[1, 0]), g["tile2_correction"], "rescale factor exp(m_old - m_new)")
    _close(O[0, 0], g["final_o_printed"], "tiled O")
    # one block of four keys: same l and O
    O4, _, tr4 = oracle.attn_fwd_tiled(Q, K, V, scale=1.0, br=4, bc=4, trace_row=0)
    assert tr4.shape == (1, 4)
    _close(tr4[0, 1], g["block4_l"], "l with one block")
    _close(O4[0, 0], g["final_o_printed"], "O with one block")


def test_worked_example_unnormalised_p(golden):
    """The page's per-tile p = exp(s - m_new) values follow from the scores it
    prints and the trace's running max."""
    g, q, K, V = _worked(golden)
    s = K @ q
    _close(s, g["scores"], "scores")
    _, _, tr = oracle.attn_fwd_tiled(np.vstack([q, np.zeros((3, 2))]), K, V, 1.0, br=4, bc=2,
                                     trace_row=0)
    _close(np.exp(s[:2] - tr[0, 0]), g["tile1_p"], "tile 1 p")
    _close(np.exp(s[2:] - tr[1, 0]), g["tile2_p"], "tile 2 p")
    _close(np.exp(s - 3.0), g["block4_p"], "block-4 p")


# --- the deep-dive page's self-test recipe (page 4) -----------------------------

def test_page_recipe_tiled_vs_naive():
    """n=300, d=64, the page's generator with seeds 1/2/3, 64x64 tiles (ragged):
    tiled output within 1e-4 of naive attention, as the page asserts."""
    n, d = 300, 64
    q, k, v = (inputs.page_generator(n, d, s).astype(np.float64) for s in (1, 2, 3))
    scale = 1.0 / math.sqrt(d)
    O_t, L_t = oracle.attn_fwd_tiled(q, k, v, scale, br=64, bc=64)
    O_n, L_n = oracle.attn_fwd(q, k, v, scale)
    assert np.max(np.abs(O_t - O_n)) < 1e-4
    assert np.max(np.abs(O_t - O_n)) < 1e-12  # both fp64
    assert np.max(np.abs(L_t - L_n)) < 1e-12


# --- library routines -------------------------------------------------------

def _masked_scores(q, k, scale, causal):
    S = scale * np.einsum("bid,bjd->bij", q, k)
    if causal:
        N = q.shape[1]
        S = np.where(np.tril(np.ones((N, N), dtype=bool))[None], S, -np.inf)
    return S


@pytest.mark.parametrize("causal", [False, True])
def test_against_scipy_softmax(causal):
    rng = np.random.default_rng(7)
    BH, N, d = 3, 37, 16
    q, k, v = (rng.standard_normal((BH, N, d)) * 1.7 for _ in range(3))
    scale = 0.3
    O, L = oracle.attn_fwd(q, k, v, scale, causal)
    S = _masked_scores(q, k, scale, causal)
    P = scipy.special.softmax(S, axis=-1)
    np.testing.assert_allclose(O, P @ v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, scipy.special.logsumexp(S, axis=-1), rtol=1e-13, atol=1e-13)


def test_against_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    BH, N, d = 2, 29, 8
    q, k, v = (rng.standard_normal((BH, N, d)) for _ in range(3))
    for causal in (False, True):
        O, _ = oracle.attn_fwd(q, k, v, 0.4, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=0.4).numpy()
        np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)


# --- closed forms and invariants -------------------------------------------

def test_rows_of_p_sum_to_one():
    rng = np.random.default_rng(3)
    N = d = 24
    q, k = rng.standard_normal((N, d)) * 2, rng.standard_normal((N, d)) * 2
    for causal in (False, True):
        P, _ = oracle.attn_fwd(q, k, np.eye(N), 1.0, causal)
        assert np.all(P >= 0)
        assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-14 * N
        if causal:
            assert np.all(np.triu(P[0], 1) == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(causal):
    rng = np.random.default_rng(5)
    BH, N, d = 2, 50, 8
    q, k = rng.standard_normal((BH, N, d)), rng.standard_normal((BH, N, d))
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (BH, N, d)).copy()
    O, _ = oracle.attn_fwd(q, k, v, 0.5, causal)
    np.testing.assert_allclose(O, v, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero(causal):
    rng = np.random.default_rng(6)
    BH, N, d = 2, 40, 8
    k, v = rng.standard_normal((BH, N, d)), rng.standard_normal((BH, N, d))
    O, L = oracle.attn_fwd(np.zeros((BH, N, d)), k, v, 0.7, causal)
    if causal:
        counts = np.arange(1, N + 1)[None, :, None]
        np.testing.assert_allclose(O, np.cumsum(v, axis=1) / counts, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(L, np.log(np.arange(1, N + 1))[None].repeat(BH, 0), atol=1e-14)
    else:
        np.testing.assert_allclose(O, v.mean(axis=1, keepdims=True).repeat(N, 1), atol=1e-14)
        np.testing.assert_allclose(L, np.full((BH, N), math.log(N)), atol=1e-14)


def test_causal_row0():
    rng = np.random.default_rng(8)
    BH, N, d = 3, 20, 8
    q, k, v = (rng.standard_normal((BH, N, d)) for _ in range(3))
    O, L = oracle.attn_fwd(q, k, v, 0.35, True)
    np.testing.assert_array_equal(O[:, 0], v[:, 0])
    np.testing.assert_allclose(L[:, 0], 0.35 * np.sum(q[:, 0] * k[:, 0], -1), rtol=1e-15, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    """K' = K + 1 u^T leaves O unchanged and adds scale * q_i . u to L_i."""
    rng = np.random.default_rng(9)
    BH, N, d = 2, 31, 8
    q, k, v = (rng.standard_normal((BH, N, d)) for _ in range(3))
    u = rng.standard_normal(d)
    O, L = oracle.attn_fwd(q, k, v, 0.6, causal)
    O2, L2 = oracle.attn_fwd(q, k + u, v, 0.6, causal)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L + 0.6 * (q @ u), atol=1e-12)


def test_permutations():
    rng = np.random.default_rng(10)
    N, d = 33, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = oracle.attn_fwd(q, k, v, 0.5)
    pk = rng.permutation(N)
    O2, L2 = oracle.attn_fwd(q, k[pk], v[pk], 0.5)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L, atol=1e-13)
    pq = rng.permutation(N)
    O3, L3 = oracle.attn_fwd(q[pq], k, v, 0.5)
    np.testing.assert_allclose(O3[0], O[0][pq], atol=1e-13)
    np.testing.assert_allclose(L3[0], L[0][pq], atol=1e-13)


def test_scale_enters_as_product_with_q():
    rng = np.random.default_rng(12)
    N, d = 21, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = oracle.attn_fwd(q, k, v, 0.25)
    O2, L2 = oracle.attn_fwd(q * 4.0, k, v, 0.0625)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2, L, atol=1e-13)
    # and scale does matter: a different scale changes the result
    O3, _ = oracle.attn_fwd(q, k, v, 0.5)
    assert np.max(np.abs(O3 - O)) > 1e-3


@pytest.mark.parametrize("N", [1, 5, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_untiled(N, causal):
    rng = np.random.default_rng(N)
    d = 16
    q, k, v = (rng.standard_normal((2, N, d)) * 2 for _ in range(3))
    O, L = oracle.attn_fwd(q, k, v, 0.25, causal)
    for blk in (1, 2, 7, 64, N):
        for br in (blk, 3):
            Ot, Lt = oracle.attn_fwd_tiled(q, k, v, 0.25, causal, br=br, bc=blk)
            assert np.max(np.abs(Ot - O)) <= 1e-12, (blk, br)
            assert np.max(np.abs(Lt - L)) <= 1e-12, (blk, br)


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(13)
    q, k, v, g = (rng.standard_normal((2, 45, 8)) for _ in range(4))
    a = oracle.attn_fwd(q, k, v, 0.3, True, threads=1)
    b = oracle.attn_fwd(q, k, v, 0.3, True, threads=7)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    a = oracle.attn_bwd(q, k, v, g, 0.3, True, threads=1)
    b = oracle.attn_bwd(q, k, v, g, 0.3, True, threads=5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# --- backward -----------------------------------------------------------------

def _fd_grads(q, k, v, g, scale, causal, h=1e-6):
    """Central finite differences of f = sum(O * G) through the pinned forward."""
    def f(q_, k_, v_):
        return float(np.sum(oracle.attn_fwd(q_, k_, v_, scale, causal, threads=1)[0] * g))
    out = []
    for which in range(3):
        base = [q, k, v]
        grad = np.zeros_like(base[which])
        for idx in np.ndindex(grad.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            grad[idx] = (f(*plus) - f(*minus)) / (2 * h)
        out.append(grad)
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 3), (4, 2), (6, 4)])
def test_backward_finite_differences(causal, N, d):
    rng = np.random.default_rng(100 + N)
    q, k, v, g = (rng.standard_normal((1, N, d)) for _ in range(4))
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, g, 0.7, causal)
    for name, got, want in zip("qkv", (dq, dk, dv), _fd_grads(q, k, v, g, 0.7, causal)):
        scale_ = max(1.0, np.max(np.abs(want)))
        assert np.max(np.abs(got - want)) <= 1e-7 * scale_, name


def test_backward_against_torch_autograd_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    BH, N, d = 2, 17, 8
    arrs = [rng.standard_normal((BH, N, d)) for _ in range(4)]
    for causal in (False, True):
        dq, dk, dv, _ = oracle.attn_bwd(*arrs, 0.45, causal)
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in arrs[:3])
        S = 0.45 * tq @ tk.transpose(-1, -2)
        if causal:
            S = S.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(), float("-inf"))
        O = torch.softmax(S, -1) @ tv
        O.backward(torch.tensor(arrs[3]))
        for got, t in zip((dq, dk, dv), (tq, tk, tv)):
            np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    """sum_j dS_ij = 0 gives sum_j dK_j = 0; sum_i P_ij summed over j gives
    sum_j dV_j = sum_i dO_i; D equals rowsum(dO * O) of the forward."""
    rng = np.random.default_rng(22)
    BH, N, d = 2, 64, 16
    q, k, v, g = (rng.standard_normal((BH, N, d)) for _ in range(4))
    dq, dk, dv, D = oracle.attn_bwd(q, k, v, g, 0.25, causal)
    np.testing.assert_allclose(dk.sum(1), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(1), g.sum(1), atol=1e-12)
    O, _ = oracle.attn_fwd(q, k, v, 0.25, causal)
    np.testing.assert_allclose(D, np.sum(g * O, -1), atol=1e-13)


def test_causal_backward_last_key_row0():
    """Under a causal mask, query 0 sees only key 0, and the last key is seen
    only by the last query: dV_{N-1} = P_{N-1,N-1} dO_{N-1}."""
    rng = np.random.default_rng(23)
    N, d = 9, 4
    q, k, v, g = (rng.standard_normal((1, N, d)) for _ in range(4))
    _, dk, dv, _ = oracle.attn_bwd(q, k, v, g, 0.5, True)
    S = 0.5 * q[0] @ k[0].T
    p_last = math.exp(S[N - 1, N - 1] - scipy.special.logsumexp(S[N - 1]))
    np.testing.assert_allclose(dv[0, N - 1], p_last * g[0, N - 1], atol=1e-14)


# --- grouped heads (GQA / MQA) ------------------------------------------------

def _gqa_inputs(seed, B, Hq, Hkv, N, d, with_dout=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, N, d))
    k, v = (rng.standard_normal((B, Hkv, N, d)) for _ in range(2))
    g = rng.standard_normal((B, Hq, N, d)) if with_dout else None
    return q, k, v, g


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1), (3, 3)])
def test_gqa_forward_against_torch_sdpa(Hq, Hkv):
    """Grouped heads reduce to torch's fp64 scaled_dot_product_attention with
    enable_gqa (query head h uses key/value head h // (Hq // Hkv)); L against
    scipy's logsumexp of each head's scaled scores."""
    torch = pytest.importorskip("torch")
    B, N, d = 2, 23, 8
    q, k, v, _ = _gqa_inputs(31, B, Hq, Hkv, N, d)
    for causal in (False, True):
        O, L = oracle.attn_fwd_gqa(q, k, v, 0.35, causal)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=0.35, enable_gqa=True).numpy()
        np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)
        mask = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
        for b in range(B):
            for h in range(Hq):
                S = np.where(mask, 0.35 * q[b, h] @ k[b, h // (Hq // Hkv)].T, -np.inf)
                np.testing.assert_allclose(L[b, h], scipy.special.logsumexp(S, axis=-1), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (5, 1)])
def test_gqa_backward_against_torch_autograd_fp64(Hq, Hkv):
    """Gradients of shared K and V are the sums over the query heads that use
    them: torch's fp64 autograd through scaled_dot_product_attention."""
    torch = pytest.importorskip("torch")
    B, N, d = 2, 13, 8
    q, k, v, g = _gqa_inputs(32, B, Hq, Hkv, N, d, with_dout=True)
    for causal in (False, True):
        dq, dk, dv, _ = oracle.attn_bwd_gqa(q, k, v, g, 0.5, causal)
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        O = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.5,
                                                             enable_gqa=True)
        O.backward(torch.tensor(g))
        for got, t in zip((dq, dk, dv), (tq, tk, tv)):
            np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_gqa_group_of_one_is_plain_attention():
    """Hkv = Hq: the grouped entry points give the per-head oracle's results."""
    B, H, N, d = 2, 3, 11, 4
    q, k, v, g = _gqa_inputs(33, B, H, H, N, d, with_dout=True)
    O, L = oracle.attn_fwd_gqa(q, k, v, 0.6, True)
    O1, L1 = oracle.attn_fwd(q.reshape(B * H, N, d), k.reshape(B * H, N, d), v.reshape(B * H, N, d), 0.6, True)
    np.testing.assert_array_equal(O.reshape(B * H, N, d), O1)
    np.testing.assert_array_equal(L.reshape(B * H, N), L1)
    grads = oracle.attn_bwd_gqa(q, k, v, g, 0.6, True)
    grads1 = oracle.attn_bwd(*(x.reshape(B * H, N, d) for x in (q, k, v, g)), 0.6, True)
    for a, b_ in zip(grads, grads1):
        np.testing.assert_array_equal(a.reshape(b_.shape), b_)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_invariants(causal):
    """Per key/value head: sum_j dK_j = 0, and sum_j dV_j equals the sum of dO
    over every row of the query heads in its group."""
    B, Hq, Hkv, N, d = 2, 6, 2, 40, 8
    q, k, v, g = _gqa_inputs(34, B, Hq, Hkv, N, d, with_dout=True)
    dq, dk, dv, _ = oracle.attn_bwd_gqa(q, k, v, g, 0.3, causal)
    G = Hq // Hkv
    np.testing.assert_allclose(dk.sum(2), 0.0, atol=1e-12)
    want = g.reshape(B, Hkv, G, N, d).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(2), want, atol=1e-11)


# --- decode: one query row against a key/value cache -----------------------------

def _dec_inputs(seed, B, Hq, Hkv, Nk, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, d))
    k, v = (rng.standard_normal((B, Hkv, Nk, d)) for _ in range(2))
    return q, k, v


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (6, 1)])
def test_decode_against_torch_sdpa(Hq, Hkv):
    """Each batch's row against its first kv_len[b] keys is torch's fp64
    scaled_dot_product_attention of a length-1 query (enable_gqa); L is
    scipy's logsumexp of the scaled scores."""
    torch = pytest.importorskip("torch")
    B, Nk, d = 3, 37, 8
    q, k, v = _dec_inputs(41, B, Hq, Hkv, Nk, d)
    lens = [37, 1, 20]
    O, L = oracle.attn_decode(q, k, v, 0.4, kv_len=lens)
    for b, n in enumerate(lens):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b:b + 1, :, None, :]), torch.from_numpy(k[b:b + 1, :, :n]),
            torch.from_numpy(v[b:b + 1, :, :n]), scale=0.4, enable_gqa=True).numpy()[0, :, 0]
        np.testing.assert_allclose(O[b], ref, rtol=1e-12, atol=1e-12)
        for h in range(Hq):
            s = 0.4 * k[b, h // (Hq // Hkv), :n] @ q[b, h]
            np.testing.assert_allclose(L[b, h], scipy.special.logsumexp(s), rtol=1e-13, atol=1e-13)


def test_decode_is_the_last_row_of_causal_attention():
    """A decode step over n cached keys is the last query row of causal
    attention over a sequence of length n (that row sees every key)."""
    B, Hq, Hkv, n, d = 2, 4, 2, 29, 8
    rng = np.random.default_rng(42)
    qs = rng.standard_normal((B, Hq, n, d))
    k, v = (rng.standard_normal((B, Hkv, n, d)) for _ in range(2))
    Of, Lf = oracle.attn_fwd_gqa(qs, k, v, 0.3, causal=True)
    O, L = oracle.attn_decode(np.ascontiguousarray(qs[:, :, -1]), k, v, 0.3)
    np.testing.assert_allclose(O, Of[:, :, -1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L, Lf[:, :, -1], rtol=1e-13, atol=1e-14)


def test_decode_short_caches():
    """kv_len 0: no visible key, O = 0 and L = -inf (fully masked rows output
    zero, deep-dive page, "Pitfalls").  kv_len 1: O = v_0 and L = scale q.k_0."""
    q, k, v = _dec_inputs(43, 2, 3, 3, 5, 4)
    O, L = oracle.attn_decode(q, k, v, 0.7, kv_len=[0, 1])
    assert np.all(O[0] == 0.0) and np.all(np.isneginf(L[0]))
    np.testing.assert_array_equal(O[1], v[1, :, 0])
    np.testing.assert_allclose(L[1], 0.7 * np.einsum("hd,hd->h", q[1], k[1, :, 0]), rtol=1e-15)


def test_decode_groups_read_their_own_kv_head():
    """Grouped decode equals per-head decode with K, V repeated per query head."""
    B, Hq, Hkv, Nk, d = 2, 6, 3, 19, 4
    q, k, v = _dec_inputs(44, B, Hq, Hkv, Nk, d)
    O, L = oracle.attn_decode(q, k, v, 0.5)
    O1, L1 = oracle.attn_decode(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), 0.5)
    np.testing.assert_array_equal(O, O1)
    np.testing.assert_array_equal(L, L1)


def test_decode_rejects_bad_lengths():
    q, k, v = _dec_inputs(45, 2, 2, 2, 5, 4)
    for lens in ([6, 1], [-1, 2]):
        with pytest.raises(RuntimeError):
            oracle.attn_decode(q, k, v, 1.0, kv_len=lens)


# --- dropout (Philox mask regenerated from seed and offset) ---------------------

def test_dropout_p0_is_plain_attention():
    """p = 0 keeps every element with factor 1: forward and backward equal the
    grouped oracle bitwise."""
    q, k, v, g = _gqa_inputs(51, 2, 4, 2, 37, 8, with_dout=True)
    for causal in (False, True):
        O, L = oracle.attn_fwd_dropout(q, k, v, 0.3, causal, 0.0, seed=7)
        O1, L1 = oracle.attn_fwd_gqa(q, k, v, 0.3, causal)
        np.testing.assert_array_equal(O, O1)
        np.testing.assert_array_equal(L, L1)
        for a, b in zip(oracle.attn_bwd_dropout(q, k, v, g, 0.3, causal, 0.0, seed=7),
                        oracle.attn_bwd_gqa(q, k, v, g, 0.3, causal)):
            np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_against_torch_with_the_mask(p):
    """Given its keep mask Z, the dropout forward is softmax(S) * Z * s @ V
    (s = 256 / (256 - thr)) and L the logsumexp of the undropped scores; the
    backward is torch's fp64 autograd through that expression (Z constant)."""
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, N, d = 2, 4, 2, 29, 8
    G = Hq // Hkv
    q, k, v, g = _gqa_inputs(52, B, Hq, Hkv, N, d, with_dout=True)
    seed, offset = 0x1234_5678_9ABC_DEF0, 11
    thr, ks = oracle.dropout_threshold(p)
    Z = oracle.dropout_mask(B * Hq, N, p, seed, offset).reshape(B, Hq, N, N).astype(np.float64)
    for causal in (False, True):
        O, L = oracle.attn_fwd_dropout(q, k, v, 0.4, causal, p, seed, offset)
        tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
        S = 0.4 * tq @ tk.repeat_interleave(G, dim=1).transpose(-1, -2)
        if causal:
            S = S.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        P = torch.softmax(S, dim=-1)
        Ot = (P * torch.tensor(Z) * ks) @ tv.repeat_interleave(G, dim=1)
        np.testing.assert_allclose(O, Ot.detach().numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(L, torch.logsumexp(S, dim=-1).detach().numpy(), rtol=1e-13, atol=1e-13)
        Ot.backward(torch.tensor(g))
        dq, dk, dv, _ = oracle.attn_bwd_dropout(q, k, v, g, 0.4, causal, p, seed, offset)
        for got, t in zip((dq, dk, dv), (tq, tk, tv)):
            np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_dropout_bytes_are_uniform_and_independent():
    """The generator's bytes: chi-square of the byte histogram within 6 sigma
    of its expectation, keep fractions within 6 binomial sigma for several p,
    and no correlation between neighbouring rows, keys, heads, seeds and
    offsets (the mapping gives every element its own byte)."""
    BH, N = 8, 512
    b = oracle.dropout_bytes(BH, N, seed=99, offset=3).astype(np.float64)
    n = b.size
    hist = np.bincount(b.astype(np.int64).ravel(), minlength=256)
    chi2 = float(((hist - n / 256) ** 2 / (n / 256)).sum())
    assert abs(chi2 - 255) < 6 * np.sqrt(2 * 255), chi2
    for p in (1 / 256, 0.25, 0.5, 0.9):
        thr, _ = oracle.dropout_threshold(p)
        keep = float(oracle.dropout_mask(BH, N, p, 99, 3).mean())
        want = 1 - thr / 256
        assert abs(keep - want) < 6 * np.sqrt(want * (1 - want) / n), (p, keep)
    z = (b - b.mean()) / b.std()

    def corr(a, c):
        return float((a * c).mean())

    lim = 6 / np.sqrt(n / 2)
    for shift in (1, 4, 8, 16, 32):
        assert abs(corr(z[:, :, :-shift], z[:, :, shift:])) < lim, ("key shift", shift)
    assert abs(corr(z[:, :-1], z[:, 1:])) < lim
    assert abs(corr(z[:-1], z[1:])) < lim
    for other in (oracle.dropout_bytes(BH, N, seed=100, offset=3), oracle.dropout_bytes(BH, N, seed=99, offset=4)):
        o = other.astype(np.float64)
        assert abs(corr(z, (o - o.mean()) / o.std())) < lim


def test_dropout_rejects_bad_arguments():
    q, k, v, g = _gqa_inputs(53, 1, 2, 2, 5, 4, with_dout=True)
    for p in (-0.1, 1.0, float("nan")):
        with pytest.raises(RuntimeError):
            oracle.attn_fwd_dropout(q, k, v, 1.0, False, p, seed=1)
    with pytest.raises(RuntimeError):
        oracle.attn_fwd_dropout(q, k, v, 1.0, False, 0.1, seed=1, offset=2 ** 32)


def _kat_vectors():
    path = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    out = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append([[int(x, 16) for x in part.split()] for part in line.split("|")])
    return out


def test_philox_known_answer_vectors():
    """The dropout generator reproduces the published Philox4x32-10 known-answer
    vectors (tests/golden/philox4x32_10_kat.txt), so its exact bits are pinned;
    the GPU mask is then pinned through the dropout parity tests."""
    vecs = _kat_vectors()
    assert len(vecs) == 3
    for ctr, key, want in vecs:
        assert oracle.philox4x32_10(ctr, key) == want, (ctr, key)


def test_dropout_bytes_follow_the_philox_words():
    """Element (bh, i, j) reads byte j % 4 of word (j / 8) % 4 of the Philox
    output for counter (2 (j / 32) + (j / 4) % 2, i, bh, offset) and key = seed."""
    seed, offset, BH, N = 0x0123_4567_89AB_CDEF, 5, 3, 70
    b = oracle.dropout_bytes(BH, N, seed, offset)
    rng = np.random.default_rng(3)
    for _ in range(200):
        bh, i, j = (int(rng.integers(0, n)) for n in (BH, N, N))
        w = oracle.philox4x32_10([2 * (j // 32) + (j // 4) % 2, i, bh, offset], [seed & 0xFFFFFFFF, seed >> 32])
        assert b[bh, i, j] == (w[(j // 8) % 4] >> (8 * (j % 4))) & 0xFF, (bh, i, j)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rows_equals_the_full_forward(causal):
    """oracle.attn_fwd_rows on an unsorted list of rows (several heads,
    repeats, first and last rows) returns exactly the full forward's rows."""
    rng = np.random.default_rng(21)
    BH, N, d = 5, 83, 16
    q, k, v = (rng.standard_normal((BH, N, d)) for _ in range(3))
    O, L = oracle.attn_fwd(q, k, v, 0.37, causal)
    rows = np.concatenate([rng.integers(0, BH * N, 60), [0, N - 1, BH * N - 1, 2 * N + 7, 2 * N + 7]])
    rng.shuffle(rows)
    Or, Lr = oracle.attn_fwd_rows(q, k, v, rows, 0.37, causal)
    np.testing.assert_array_equal(Or, O.reshape(BH * N, d)[rows])
    np.testing.assert_array_equal(Lr, L.reshape(BH * N)[rows])


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rows_dropout_equals_the_full_dropout_forward(causal):
    """oracle.attn_fwd_rows_dropout returns exactly the rows of the full
    dropout forward (same seed, offset and p) at the listed flat rows."""
    rng = np.random.default_rng(22)
    BH, N, d = 4, 71, 8
    q, k, v = (rng.standard_normal((BH, N, d)) for _ in range(3))
    seed, offset, p = 0xFEED_0000_1234, 9, 0.25
    O, L = oracle.attn_fwd_dropout(q[None], k[None], v[None], 0.5, causal, p, seed, offset)
    rows = np.concatenate([rng.integers(0, BH * N, 50), [0, BH * N - 1, N, N]])
    rng.shuffle(rows)
    Or, Lr = oracle.attn_fwd_rows_dropout(q, k, v, rows, 0.5, causal, p, seed, offset)
    np.testing.assert_array_equal(Or, O.reshape(BH * N, d)[rows])
    np.testing.assert_array_equal(Lr, L.reshape(BH * N)[rows])
