"""Pins for the fp64 oracle: values the pages print, closed forms, invariants,
independent library routines and finite differences.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign, an off-by-one mask, a transposed operand) fails at least one of
them; the ``test_planted_*`` tests plant such mistakes in a copy of the oracle
on the CPU and check that they are caught.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention as oa
from golden_io import worked_example

RNG = np.random.default_rng(12345)


def rand(*shape, rng=None):
    return (rng or RNG).standard_normal(shape)


# --------------------------------------------------------------------------
# Worked example (FlashAttention Algorithm > Worked Example): printed values
# --------------------------------------------------------------------------

def _close(got, want, tol, what):
    err = np.max(np.abs(np.asarray(got) - np.asarray(want)))
    assert err <= tol, f"{what}: max err {err} > {tol}"


def test_worked_example_trace_matches_printed_console():
    Q, K, V, exp = worked_example()
    O, L, tr = oracle.attention_tiled_ref(Q, K, V, 1.0 / math.sqrt(4), 4, 4, trace=True)
    t0, t1 = tr[0]
    _close(t0["S"], exp["S_block0"][0], exp["S_block0"][1], "S block 0")
    _close(t0["m"], exp["m_block0"][0], exp["m_block0"][1], "running max after block 0")
    _close(t0["l"], exp["l_block0"][0], exp["l_block0"][1], "running sum after block 0")
    _close(t1["S"], exp["S_block1"][0], exp["S_block1"][1], "S block 1")
    _close(t1["alpha"], exp["alpha_block1"][0], exp["alpha_block1"][1], "rescale factor")
    _close(t1["m"], exp["m_block1"][0], exp["m_block1"][1], "final running max")
    _close(t1["l"], exp["l_block1"][0], exp["l_block1"][1], "final running sum")
    _close(O[:4], exp["O_rows0to3"][0], exp["O_rows0to3"][1], "O rows 0-3 (tiled)")


def test_worked_example_one_pass_and_L():
    Q, K, V, exp = worked_example()
    O, L = oracle.attention_ref(Q[None], K[None], V[None], 0.5)
    _close(O[0, :4], exp["O_rows0to3"][0], exp["O_rows0to3"][1], "O rows 0-3 (one pass)")
    # L = m + ln(l) from the printed final max and sum (sum printed to 3-4 digits).
    L_printed = exp["m_block1"][0] + np.log(exp["l_block1"][0])
    _close(L[0, :4], L_printed, 1e-3, "L rows 0-3")


def test_worked_example_causal_closed_forms():
    """Causal mask on the worked example's inputs: rows 0-3 in closed form."""
    Q, K, V, _ = worked_example()
    O, L = oracle.attention_ref(Q[None], K[None], V[None], 0.5, causal=True)
    O, L = O[0], L[0]
    e = math.exp(0.5)
    np.testing.assert_allclose(O[0], [1, 0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(L[0], 0.5, atol=1e-15)
    np.testing.assert_allclose(O[1], [1 / (1 + e), e / (1 + e), 0, 0], atol=1e-15)
    np.testing.assert_allclose(L[1], math.log(1 + e), atol=1e-15)
    np.testing.assert_allclose(O[2], [1 / 3, 1 / 3, 1 / 3, 0], atol=1e-15)
    np.testing.assert_allclose(L[2], math.log(3), atol=1e-15)
    np.testing.assert_allclose(O[3], [0.25] * 4, atol=1e-15)
    np.testing.assert_allclose(L[3], math.log(4), atol=1e-15)
    On, Ln = oracle.attention_ref(Q[None], K[None], V[None], 0.5)
    np.testing.assert_allclose(O[7], On[0, 7], atol=1e-15)  # last row sees every key
    np.testing.assert_allclose(L[7], Ln[0, 7], atol=1e-15)


# --------------------------------------------------------------------------
# Independent library routines
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 5), (False, 3)])
def test_softmax_and_logsumexp_match_scipy(causal, window):
    N, d = 23, 7
    Q, K, V = rand(N, d), rand(N, d), rand(N, d)
    scale = 0.37
    O, L = oracle.attention_ref(Q[None], K[None], V[None], scale, causal, window)
    P = oracle.attention_probs_ref(Q, K, scale, causal, window)
    S = scale * (Q @ K.T)
    for i in range(N):
        vis = [j for j in range(N) if (not causal or j <= i) and (window < 0 or j >= i - window)]
        p = scipy.special.softmax(S[i, vis])
        np.testing.assert_allclose(P[i, vis], p, rtol=0, atol=1e-15)
        np.testing.assert_allclose(L[0, i], scipy.special.logsumexp(S[i, vis]), atol=1e-13)
        np.testing.assert_allclose(O[0, i], p @ V[vis], atol=1e-13)


def _torch_mask(N, causal, window):
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    ok = torch.ones(N, N, dtype=torch.bool)
    if causal:
        ok &= j <= i
    if window >= 0:
        ok &= j >= i - window
    return ok


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 9)])
def test_forward_matches_torch_sdpa_fp64(causal, window):
    """torch's math SDPA on the CPU in float64 is an independent implementation."""
    g = torch.Generator().manual_seed(0)
    B, H, N, d = 2, 3, 50, 16
    q, k, v = (torch.randn(B, H, N, d, generator=g, dtype=torch.float64) for _ in range(3))
    scale = 1 / math.sqrt(d)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=_torch_mask(N, causal, window), scale=scale)
    O, _ = oracle.attention_ref(q.numpy(), k.numpy(), v.numpy(), scale, causal, window)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd_fp64(causal):
    """The NumPy page's gradient-test shape (4, 8, 64, 32), autograd in float64."""
    g = torch.Generator().manual_seed(0)
    B, H, N, d = 4, 8, 64, 32
    q, k, v = (torch.randn(B, H, N, d, generator=g, dtype=torch.float64, requires_grad=True)
               for _ in range(3))
    dO = torch.randn(B, H, N, d, generator=g, dtype=torch.float64)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    out.backward(dO)
    dq, dk, dv = oracle.attention_bwd_ref(q.detach().numpy(), k.detach().numpy(),
                                          v.detach().numpy(), dO.numpy(), 1 / math.sqrt(d), causal)
    np.testing.assert_allclose(dq, q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, v.grad.numpy(), atol=1e-12)


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 4), (False, 2)])
def test_I1_rows_sum_to_one(causal, window):
    N, d = 31, 5
    P = oracle.attention_probs_ref(rand(N, d), rand(N, d), 0.9, causal, window)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-14)
    ok = oracle.allowed_mask(np.arange(N), N, causal, window)
    assert np.all(P[~ok] == 0.0)


# The NumPy page's test matrix: (N, d) x (block_q, block_k).
P1_SHAPES = [(64, 32), (128, 64), (256, 64), (512, 128)]
P1_BLOCKS = [(32, 32), (64, 64), (128, 64)]


@pytest.mark.parametrize("N,d", P1_SHAPES)
@pytest.mark.parametrize("bq,bk", P1_BLOCKS)
def test_I2_block_size_invariance_page_grid(N, d, bq, bk):
    rng = np.random.default_rng(0)
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    s = 1 / math.sqrt(d)
    O1, L1 = oracle.attention_ref(Q[None], K[None], V[None], s)
    O4, L4, _ = oracle.attention_tiled_ref(Q, K, V, s, bq, bk)
    assert np.abs(O4 - O1[0]).max() <= 1e-12
    assert np.abs(L4 - L1[0]).max() <= 1e-12


@pytest.mark.parametrize("bq,bk", [(1, 1), (3, 5), (4, 4), (5, 3), (100, 7), (37, 37), (64, 64)])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 6), (False, 4)])
def test_I2_block_size_invariance_odd_blocks_and_masks(bq, bk, causal, window):
    N, d = 37, 6  # ragged against every block size above; 64 > N
    Q, K, V = rand(N, d), rand(N, d), rand(N, d)
    O1, L1 = oracle.attention_ref(Q[None], K[None], V[None], 0.41, causal, window)
    O4, L4, _ = oracle.attention_tiled_ref(Q, K, V, 0.41, bq, bk, causal, window)
    assert np.abs(O4 - O1[0]).max() <= 1e-12
    assert np.abs(L4 - L1[0]).max() <= 1e-12


def _per_tile_softmax(Q, K, V, scale, tile):
    """Negative control: normalise each tile on its own, sum tiles, no rescale
    (the per-tile loop of the tiled self-attention block page)."""
    O = np.zeros((Q.shape[0], V.shape[1]))
    for ks in range(0, K.shape[0], tile):
        S = Q @ K[ks:ks + tile].T * scale
        E = np.exp(S - S.max(axis=1, keepdims=True))
        O += (E / E.sum(axis=1, keepdims=True)) @ V[ks:ks + tile]
    return O


def _normalised_probs_update(Q, K, V, scale, tile):
    """Negative control: the online update fed with per-tile probabilities
    instead of raw scores (the FlashAttention-2 inference page's Step 3)."""
    N = Q.shape[0]
    o = np.zeros((N, V.shape[1]))
    ell = np.zeros(N)
    m = np.full(N, -np.inf)
    for ks in range(0, N, tile):
        S = Q @ K[ks:ks + tile].T * scale
        E = np.exp(S - S.max(axis=1, keepdims=True))
        p = E / E.sum(axis=1, keepdims=True)
        new_m = np.maximum(m, p.max(axis=1))
        a = np.exp(m - new_m)
        m = new_m
        o = a[:, None] * o + (p * a[:, None]) @ V[ks:ks + tile]
        ell = a * ell + (p * a[:, None]).sum(axis=1)
    return o / ell[:, None]


def test_negative_controls_fail_block_invariance():
    rng = np.random.default_rng(0)
    N, d = 8, 4
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    O1, _ = oracle.attention_ref(Q[None], K[None], V[None], 0.5)
    assert np.abs(_per_tile_softmax(Q, K, V, 0.5, 4) - O1[0]).max() > 0.1
    np.testing.assert_allclose(_per_tile_softmax(Q, K, V, 0.5, 8), O1[0], atol=1e-14)
    assert np.abs(_normalised_probs_update(Q, K, V, 0.5, 4) - O1[0]).max() > 1e-3


@pytest.mark.parametrize("causal,window", [(True, -1), (True, 5), (False, 5)])
def test_I3_masked_positions_contribute_exactly_zero(causal, window):
    N, d = 40, 8
    rng = np.random.default_rng(7)
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = oracle.attention_ref(Q[None], K[None], V[None], 0.3, causal, window)
    r = 20  # rows 0..r-1 (causal) / rows >= r+? (window) are checked
    K2, V2 = K.copy(), V.copy()
    if causal:
        K2[r:] = 1e3 * rng.standard_normal((N - r, d))  # future keys of rows < r
        V2[r:] = -1e3
        rows = np.arange(r)
        if window >= 0:  # also perturb keys too old for rows near r
            K2[: r - 1 - window] += 77.0
            rows = np.arange(r - 1, r)
    else:  # window only: keys older than i-window are hidden
        K2[:3] = 1e3
        V2[:3] = 5e2
        rows = np.arange(3 + window, N)
    O2, L2 = oracle.attention_ref(Q[None], K2[None], V2[None], 0.3, causal, window)
    assert np.array_equal(O2[0, rows], O[0, rows])
    assert np.array_equal(L2[0, rows], L[0, rows])


@pytest.mark.parametrize("n", [1, 2, 8, 33])
def test_I4_decode_equals_last_row_of_causal_attention(n):
    """The KV-cache page's harness: d=64, uniform [0,1) inputs, the decode of
    the newest token equals the last row of causal attention."""
    rng = np.random.default_rng(0)
    d, H, Lmax = 64, 3, 40
    q = rng.random((1, H, d))
    kc = rng.random((1, H, Lmax, d))
    vc = rng.random((1, H, Lmax, d))
    kc[:, :, n:] = np.nan  # rows past the length are never read
    vc[:, :, n:] = np.nan
    o, lse = oracle.decode_ref(q, kc, vc, [n], 1 / 8)
    for h in range(H):
        Q = np.concatenate([rng.random((n - 1, d)), q[0, h][None]], axis=0)
        O, L = oracle.attention_ref(Q[None], kc[0, h, :n][None], vc[0, h, :n][None], 1 / 8, causal=True)
        np.testing.assert_allclose(o[0, h], O[0, -1], atol=1e-14)
        np.testing.assert_allclose(lse[0, h], L[0, -1], atol=1e-14)
    # decode with a window equals the last row of windowed causal attention
    if n > 3:
        o2, l2 = oracle.decode_ref(q, kc, vc, [n], 1 / 8, window=2)
        O, L = oracle.attention_ref(q[0, :, None].repeat(n, 1), kc[0, :, :n], vc[0, :, :n], 1 / 8,
                                    causal=True, window=2)
        np.testing.assert_allclose(o2[0], O[:, -1], atol=1e-14)
        np.testing.assert_allclose(l2[0], L[:, -1], atol=1e-14)


def _fd_check(bwd, N, d, causal, window, eps=1e-6):
    rng = np.random.default_rng(N * 31 + d)
    Q, K, V, G = (rng.standard_normal((N, d)) for _ in range(4))
    s = 0.7

    def f(Q_, K_, V_):
        O, _ = oracle.attention_ref(Q_[None], K_[None], V_[None], s, causal, window)
        return float((O[0] * G).sum())

    dQ, dK, dV = bwd(Q[None], K[None], V[None], G[None], s, causal, window)
    worst = 0.0
    for X, dX, which in ((Q, dQ[0], 0), (K, dK[0], 1), (V, dV[0], 2)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            args = [Q.copy(), K.copy(), V.copy()]
            args[which][idx] += eps
            fp = f(*args)
            args[which][idx] -= 2 * eps
            fm = f(*args)
            num[idx] = (fp - fm) / (2 * eps)
        rel = np.abs(num - dX).max() / max(np.abs(num).max(), 1e-30)
        worst = max(worst, rel)
    return worst


@pytest.mark.parametrize("N,d", [(8, 4), (16, 8)])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 3), (False, 3)])
def test_I5_finite_differences(N, d, causal, window):
    assert _fd_check(oracle.attention_bwd_ref, N, d, causal, window) <= 1e-6


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 7)])
def test_I6_gradient_identities(causal, window):
    rng = np.random.default_rng(3)
    B, H, N, d = 1, 2, 29, 6
    q, k, v, g = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd_ref(q, k, v, g, 0.45, causal, window)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), g.sum(axis=2), atol=1e-12)


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 10)])
def test_I7_convex_hull_with_corrupted_keys(causal, window):
    """Corrupt 5% of K's entries (the NumPy page's fault-injection idea): each
    output component must stay within the range of the visible V values."""
    rng = np.random.default_rng(11)
    N, d = 60, 8
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    bad = rng.random(K.shape) < 0.05
    K[bad] = rng.uniform(-50, 50, size=bad.sum())
    O, _ = oracle.attention_ref(Q[None], K[None], V[None], 1.0, causal, window)
    ok = oracle.allowed_mask(np.arange(N), N, causal, window)
    for i in range(N):
        vis = V[ok[i]]
        assert np.all(O[0, i] >= vis.min(axis=0) - 1e-12)
        assert np.all(O[0, i] <= vis.max(axis=0) + 1e-12)


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 4), (False, 4)])
def test_I8_scale_zero_gives_uniform_weights(causal, window):
    rng = np.random.default_rng(5)
    N, d = 19, 3
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    O, L = oracle.attention_ref(Q[None], K[None], V[None], 0.0, causal, window)
    for i in range(N):
        lo = max(0, i - window) if window >= 0 else 0
        hi = i if causal else N - 1
        np.testing.assert_allclose(L[0, i], math.log(hi - lo + 1), atol=1e-14)
        np.testing.assert_allclose(O[0, i], V[lo:hi + 1].mean(axis=0), atol=1e-14)


def test_I9_constant_v():
    rng = np.random.default_rng(9)
    q, k = rng.standard_normal((2, 2, 17, 5)), rng.standard_normal((2, 2, 17, 5))
    v = np.full((2, 2, 17, 5), -2.75)
    for causal, window in ((False, -1), (True, -1), (True, 3)):
        O, _ = oracle.attention_ref(q, k, v, 0.8, causal, window)
        np.testing.assert_allclose(O, -2.75, atol=1e-14)


SHIFTS = np.array([-800.0, -45.0, -17.0, 0.0, 10.0, 750.0, -300.0, 60.0, -1.5, 400.0, -600.0])


def _shifted(Q, K, offsets, scale):
    """Q, K with one extra column: 1 in every key, offsets / scale in the
    queries, so that row i's scaled scores move by offsets[i] exactly."""
    col_k = np.ones(K.shape[:-1] + (1,))
    col_q = (offsets / scale)[:, None] * np.ones(Q.shape[:-1] + (1,))
    return np.concatenate([Q, col_q], axis=-1), np.concatenate([K, col_k], axis=-1)


@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 4)])
def test_shift_invariance_far_offsets(causal, window):
    """A per-row constant added to the scores leaves O unchanged and moves L by
    exactly that constant (NumPy page, Step 1: the stable softmax subtracts
    the row max) -- also at offsets where exp of the raw scores overflows or
    underflows in float64."""
    rng = np.random.default_rng(31)
    N, d = len(SHIFTS), 6
    Q, K, V = (rng.standard_normal((2, N, d)) for _ in range(3))
    scale = 0.4
    O0, L0 = oracle.attention_ref(Q, K, V, scale, causal, window)
    Qs, Ks = _shifted(Q, K, SHIFTS, scale)
    O1, L1 = oracle.attention_ref(Qs, Ks, V, scale, causal, window)
    assert np.isfinite(O1).all() and np.isfinite(L1).all()
    np.testing.assert_allclose(O1, O0, atol=1e-12)
    np.testing.assert_allclose(L1 - SHIFTS, L0, atol=1e-9)
    # The exact gradients move only in the extra columns: dQ, dV and the
    # original columns of dK are unchanged.
    G = rng.standard_normal((2, N, d))
    g0 = oracle.attention_bwd_ref(Q, K, V, G, scale, causal, window)
    g1 = oracle.attention_bwd_ref(Qs, Ks, V, G, scale, causal, window)
    np.testing.assert_allclose(g1[0][..., :d], g0[0], atol=1e-9)
    np.testing.assert_allclose(g1[0][..., d], 0.0, atol=1e-9)
    np.testing.assert_allclose(g1[1][..., :d], g0[1], atol=1e-9)
    np.testing.assert_allclose(g1[2], g0[2], atol=1e-9)


def test_empty_rows_give_zero_output_and_neg_inf_lse():
    """Non-causal window with more keys hidden than exist cannot empty a row,
    but a query row with no visible key (reading R4) is O=0, L=-inf."""
    ok = np.zeros((2, 3), dtype=bool)
    P, L = oa._softmax_rows(np.ones((2, 3)), ok)
    assert np.all(P == 0) and np.all(np.isneginf(L))


def test_rows_ref_equals_full():
    rng = np.random.default_rng(2)
    N, d = 70, 9
    Q, K, V = (rng.standard_normal((N, d)) for _ in range(3))
    rows = [0, 5, 33, 69]
    for causal, window in ((False, -1), (True, -1), (True, 8)):
        O, L = oracle.attention_ref(Q[None], K[None], V[None], 0.3, causal, window)
        Or, Lr = oracle.attention_rows_ref(Q, K, V, 0.3, rows, causal, window)
        np.testing.assert_allclose(Or, O[0, rows], atol=1e-14)
        np.testing.assert_allclose(Lr, L[0, rows], atol=1e-14)


def test_single_key_and_single_row_special_cases():
    rng = np.random.default_rng(4)
    Q, K, V = (rng.standard_normal((1, 6)) for _ in range(3))
    O, L = oracle.attention_ref(Q[None], K[None], V[None], 0.5)
    np.testing.assert_allclose(O[0, 0], V[0], atol=1e-15)
    np.testing.assert_allclose(L[0, 0], 0.5 * float(Q[0] @ K[0]), atol=1e-15)


# --------------------------------------------------------------------------
# Planted mistakes: the pins above must catch each of them.
# --------------------------------------------------------------------------

def _mask_strict_causal(rows, n_keys, causal, window):
    i = np.asarray(rows)[:, None]
    j = np.arange(n_keys)[None, :]
    ok = np.ones((i.shape[0], n_keys), bool)
    if causal:
        ok &= j < i  # planted: the diagonal is hidden
    if window >= 0:
        ok &= j >= i - window
    return ok


def _mask_window_off_by_one(rows, n_keys, causal, window):
    i = np.asarray(rows)[:, None]
    j = np.arange(n_keys)[None, :]
    ok = np.ones((i.shape[0], n_keys), bool)
    if causal:
        ok &= j <= i
    if window >= 0:
        ok &= j > i - window  # planted: W keys instead of W+1
    return ok


def test_planted_strict_causal_mask_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "allowed_mask", _mask_strict_causal)
    with pytest.raises(AssertionError):
        test_worked_example_causal_closed_forms()


def _softmax_without_max(S, ok):
    S = np.where(ok, S, -np.inf)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        E = np.exp(S)  # planted: the row max is not subtracted
        ell = E.sum(axis=1)
        return E / ell[:, None], np.log(ell)


def test_planted_unstable_softmax_fails_shift_pin(monkeypatch):
    monkeypatch.setattr(oa, "_softmax_rows", _softmax_without_max)
    with pytest.raises(AssertionError):
        test_shift_invariance_far_offsets(False, -1)


def test_planted_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "allowed_mask", _mask_window_off_by_one)
    with pytest.raises(AssertionError):
        test_I8_scale_zero_gives_uniform_weights(True, 4)


def _bwd_variant(mistake):
    def bwd(q, k, v, dO, scale, causal=False, window=-1):
        Q, K, V, G = q[0], k[0], v[0], dO[0]
        O, _, P = oa._head(Q, K, V, scale, np.arange(Q.shape[0]), causal, window)
        D = (G * O).sum(axis=1)
        dP = G @ V.T
        dS = P * (dP - (0.0 if mistake == "drop_D" else D[:, None]))
        dV = P.T @ G if mistake != "transpose_dV" else P @ G
        dQ = scale * (dS @ K)
        dK = scale * (dS.T @ Q) if mistake != "transpose_dK" else scale * (dS @ Q)
        if mistake == "sign_dQ":
            dQ = -dQ
        return dQ[None], dK[None], dV[None]
    return bwd


@pytest.mark.parametrize("mistake", ["drop_D", "transpose_dV", "transpose_dK", "sign_dQ"])
def test_planted_backward_mistakes_fail_finite_differences(mistake):
    assert _fd_check(_bwd_variant(mistake), 8, 4, False, -1) > 1e-3


def test_planted_backward_variant_harness_is_faithful():
    assert _fd_check(_bwd_variant("none"), 8, 4, True, -1) <= 1e-6


def test_planted_missing_rescale_fails_trace_pin(monkeypatch):
    """An online update that forgets exp(m_old - m_new) misses the printed sums."""
    real_exp = np.exp
    Q, K, V, exp = worked_example()

    def run():
        N = Q.shape[0]
        m = np.full(4, -np.inf)
        ell = np.zeros(4)
        for ks in (0, 4):
            S = Q[:4] @ K[ks:ks + 4].T * 0.5
            m_new = np.maximum(m, S.max(axis=1))
            P = real_exp(S - m_new[:, None])
            ell = ell + P.sum(axis=1)  # planted: no rescale
            m = m_new
        return ell

    with pytest.raises(AssertionError):
        _close(run(), exp["l_block1"][0], exp["l_block1"][1], "final running sum")


# --------------------------------------------------------------------------
# Paged KV cache (FlashAttention-2 inference page, Extending It): the pages
# hold the KV-cache page's logical cache, token t at row t % P of page
# table[t // P]
# --------------------------------------------------------------------------

def _paged_pool(lens, H, d, P, rng, hide=()):
    """A pool whose row for token t of sequence s, head h holds
    V = [t, t^2 / 100, s, h, 0, ...] (and random K); stale rows are NaN; the table
    maps each sequence's page slots to a random permutation of the pool.
    Slots listed in ``hide`` as (s, slot) get table entries outside the pool."""
    slots = [-(-n // P) for n in lens]
    num_pages = sum(slots) + 3  # 3 pages belong to nobody
    perm = rng.permutation(num_pages)
    max_pages = max(slots) + 1
    table = np.full((len(lens), max_pages), -7, dtype=np.int64)
    kp = np.full((num_pages, H, P, d), np.nan)
    vp = np.full((num_pages, H, P, d), np.nan)
    nxt = 0
    for s, n in enumerate(lens):
        for j in range(slots[s]):
            p = perm[nxt]
            nxt += 1
            table[s, j] = p if (s, j) not in hide else (num_pages if j % 2 else -1)
            for r in range(P):
                t = j * P + r
                if t < n:
                    kp[p, :, r] = rng.standard_normal((H, d))
                    for h in range(H):
                        vp[p, h, r] = 0.0
                        vp[p, h, r, :4] = [t, t * t / 100.0, s, h]
    return kp, vp, table


def _visible_mean(positions, s, h):
    t = np.asarray(positions, dtype=np.float64)
    return np.array([t.mean(), (t * t / 100.0).mean(), s, h])


@pytest.mark.parametrize("window", [-1, 0, 5])
def test_paged_decode_scale_zero_closed_form(window):
    """scale = 0: the output is the mean of V over the visible positions, which
    identifies those positions; L = ln(count)."""
    rng = np.random.default_rng(21)
    lens, H, d, P = [1, 4, 5, 11, 16], 2, 4, 4
    kp, vp, table = _paged_pool(lens, H, d, P, rng)
    q = rng.standard_normal((len(lens), H, d))
    o, lse = oracle.decode_paged_ref(q, kp, vp, table, lens, 0.0, window)
    for s, n in enumerate(lens):
        lo = 0 if window < 0 else max(0, n - 1 - window)
        for h in range(H):
            _close(o[s, h], _visible_mean(range(lo, n), s, h), 1e-12, f"o[{s},{h}]")
            _close(lse[s, h], math.log(n - lo), 1e-14, f"lse[{s},{h}]")


def test_paged_decode_hidden_pages_drop_their_tokens():
    rng = np.random.default_rng(22)
    lens, H, d, P = [9, 12], 1, 4, 4
    kp, vp, table = _paged_pool(lens, H, d, P, rng, hide={(0, 0), (1, 1)})
    q = rng.standard_normal((2, H, d))
    o, lse = oracle.decode_paged_ref(q, kp, vp, table, lens, 0.0)
    _close(o[0, 0], _visible_mean(range(4, 9), 0, 0), 1e-12, "seq 0 without its first page")
    _close(o[1, 0], _visible_mean(list(range(0, 4)) + list(range(8, 12)), 1, 0), 1e-12,
           "seq 1 without its second page")
    _close(lse[:, 0], np.log([5, 8]), 1e-14, "lse")


@pytest.mark.parametrize("window", [-1, 3])
def test_paged_decode_equals_dense_decode_on_the_logical_cache(window):
    rng = np.random.default_rng(23)
    lens, H, d, P = [1, 7, 8, 13], 3, 8, 4
    kp, vp, table = _paged_pool(lens, H, d, P, rng)
    vp = np.where(np.isnan(vp), np.nan, rng.standard_normal(vp.shape))  # V random as well
    q = rng.standard_normal((len(lens), H, d))
    Lmax = max(lens)
    kc = np.full((len(lens), H, Lmax, d), np.nan)
    vc = np.full((len(lens), H, Lmax, d), np.nan)
    for s, n in enumerate(lens):  # unpage token by token, slot by slot
        for j in range(-(-n // P)):
            rows = min(P, n - j * P)
            kc[s, :, j * P:j * P + rows] = kp[table[s, j], :, :rows]
            vc[s, :, j * P:j * P + rows] = vp[table[s, j], :, :rows]
    o1, l1 = oracle.decode_paged_ref(q, kp, vp, table, lens, 0.4, window)
    o2, l2 = oracle.decode_ref(q, kc, vc, lens, 0.4, window)
    _close(o1, o2, 1e-14, "o")
    _close(l1, l2, 1e-14, "lse")


@pytest.mark.parametrize("mistake", ["row_from_slot", "page_from_row"])
def test_planted_page_mapping_mistakes_are_caught(monkeypatch, mistake):
    def wrong(table_row, n, P, num_pages):
        t = np.arange(n)
        tr = np.asarray(table_row, dtype=np.int64)
        if mistake == "row_from_slot":
            page, row = tr[t // P], (t // P) % P
        else:
            page, row = tr[np.minimum(t % P, len(tr) - 1)], t % P
        return page, row, (page >= 0) & (page < num_pages)

    monkeypatch.setattr(oa, "_page_rows", wrong)
    with pytest.raises(AssertionError):
        test_paged_decode_scale_zero_closed_form(-1)
