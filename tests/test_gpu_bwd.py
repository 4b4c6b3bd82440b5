"""GPU parity of fa_bwd (recompute from L) against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_04_amd as fa
from parity import check_bf16, need_gpu, to64
from tiled_attention_04_amd.inputs import WORKLOADS, attention_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run(q, k, v, dO, causal, window=-1, scale=None):
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, dO))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, window=window, scale=scale)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, gd, lse, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 64, 200, 257])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 45), (False, 30)])
def test_small_shapes(d, N, causal, window):
    q, k, v, dO = attention_inputs(1, 2, N, d, "bf16", seed=N + d, with_grad=True)
    dq, dk, dv = run(q, k, v, dO, causal, window)
    s = 1 / math.sqrt(d)
    rq, rk, rv = oracle.attention_bwd_ref(q, k, v, dO, s, causal, window)
    check_bf16(dq, rq, "dQ")
    check_bf16(dk, rk, "dK")
    check_bf16(dv, rv, "dV")


def test_gradient_test_shape_of_numpy_page():
    """(B, H, N, d) = (4, 8, 64, 32) in the page; d=32 is not a bf16 kernel size,
    so the same batch/head/length with d=64."""
    q, k, v, dO = attention_inputs(4, 8, 64, 64, "bf16", seed=0, with_grad=True)
    for causal in (False, True):
        dq, dk, dv = run(q, k, v, dO, causal)
        rq, rk, rv = oracle.attention_bwd_ref(q, k, v, dO, 1 / 8, causal)
        check_bf16(dq, rq, "dQ")
        check_bf16(dk, rk, "dK")
        check_bf16(dv, rv, "dV")


def test_gradient_identities_on_gpu():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per (b, h)."""
    q, k, v, dO = attention_inputs(2, 3, 300, 128, "bf16", seed=8, with_grad=True)
    dq, dk, dv = run(q, k, v, dO, True)
    sdk = to64(dk).sum(axis=2)
    sdv = to64(dv).sum(axis=2)
    sdo = to64(dO).sum(axis=2)
    assert np.abs(sdk).max() <= 0.05 * np.abs(to64(dk)).max() * math.sqrt(300)
    assert np.abs(sdv - sdo).max() <= 0.05


@pytest.mark.slow
def test_full_size_sampled_heads():
    """B=2, H=16, N=4096, d=128, causal: two whole heads against the oracle."""
    w = WORKLOADS["bwd_b2_h16_n4096_d128_bf16"]
    q, k, v, dO = attention_inputs(w["B"], w["H"], w["N"], w["d"], "bf16", seed=0, with_grad=True)
    dq, dk, dv = run(q, k, v, dO, True)
    s = 1 / math.sqrt(128)
    for b, h in ((0, 0), (1, 9)):
        rq, rk, rv = oracle.attention_bwd_ref(q[b, h][None], k[b, h][None], v[b, h][None],
                                              dO[b, h][None], s, True)
        check_bf16(dq[b, h], rq[0], f"dQ[{b},{h}]")
        check_bf16(dk[b, h], rk[0], f"dK[{b},{h}]")
        check_bf16(dv[b, h], rv[0], f"dV[{b},{h}]")


@pytest.mark.slow
def test_full_size_window_sampled_heads():
    """The windowed backward stage the bench times: B=2, H=16, N=4096, d=128,
    causal with a 1024-token window; two whole heads against the oracle."""
    w = WORKLOADS["bwd_b2_h16_n4096_d128_bf16"]
    q, k, v, dO = attention_inputs(w["B"], w["H"], w["N"], w["d"], "bf16", seed=0, with_grad=True)
    dq, dk, dv = run(q, k, v, dO, True, 1024)
    s = 1 / math.sqrt(128)
    for b, h in ((0, 3), (1, 15)):
        rq, rk, rv = oracle.attention_bwd_ref(q[b, h][None], k[b, h][None], v[b, h][None],
                                              dO[b, h][None], s, True, 1024)
        check_bf16(dq[b, h], rq[0], f"dQ[{b},{h}]")
        check_bf16(dk[b, h], rk[0], f"dK[{b},{h}]")
        check_bf16(dv[b, h], rv[0], f"dV[{b},{h}]")


@pytest.mark.parametrize("B,H,N,d", [(1, 3, 700, 128), (1, 2, 1100, 64)])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 100), (False, 50)])
def test_several_tiles_ragged(B, H, N, d, causal, window):
    """Several 128-key and 128-query tiles of both kernels, a ragged tail."""
    q, k, v, dO = attention_inputs(B, H, N, d, "bf16", seed=N + 7 * d, with_grad=True)
    dq, dk, dv = run(q, k, v, dO, causal, window)
    rq, rk, rv = oracle.attention_bwd_ref(q, k, v, dO, 1 / math.sqrt(d), causal, window)
    check_bf16(dq, rq, "dQ")
    check_bf16(dk, rk, "dK")
    check_bf16(dv, rv, "dV")


def test_backward_is_deterministic():
    """No atomics: two calls on the same inputs give identical bits."""
    q, k, v, dO = attention_inputs(2, 4, 515, 128, "bf16", seed=3, with_grad=True)
    a = run(q, k, v, dO, True)
    b = run(q, k, v, dO, True)
    for x, y, name in zip(a, b, ("dQ", "dK", "dV")):
        assert torch.equal(x, y), name


@pytest.mark.parametrize("B,H,N,d", [(1, 64, 1100, 128), (1, 128, 600, 64)])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 300), (False, 200)])
def test_many_heads_256_row_dq_tiles(B, H, N, d, causal, window):
    """Enough (head, 256-row tile) pairs to fill the chip, which selects the
    256-row dQ kernel; ragged tails; sampled heads against the oracle."""
    q, k, v, dO = attention_inputs(B, H, N, d, "bf16", seed=N + d + H, with_grad=True)
    dq, dk, dv = run(q, k, v, dO, causal, window)
    s = 1 / math.sqrt(d)
    for h in (0, H // 2 + 5, H - 1):
        rq, rk, rv = oracle.attention_bwd_ref(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1],
                                              dO[:, h:h + 1], s, causal, window)
        check_bf16(dq[:, h:h + 1], rq, f"dQ[h={h}]")
        check_bf16(dk[:, h:h + 1], rk, f"dK[h={h}]")
        check_bf16(dv[:, h:h + 1], rv, f"dV[h={h}]")
