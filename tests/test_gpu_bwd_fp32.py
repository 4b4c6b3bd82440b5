"""GPU parity of the float32 backward (fa_bwd with float32 inputs) against the
fp64 oracle, at the float32 bar (max |err| <= 1e-5)."""

import math

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_04_amd as fa
from golden_io import worked_example
from parity import check_fp32, need_gpu, to64
from tiled_attention_04_amd.inputs import attention_inputs

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


def check_all(got, ref, tag="", smax=None):
    """The float32 bar.  With smax (the largest |scaled score|) given, the bar
    widens to 8 u smax |output|max (u = 2^-24) where that is larger: a float32
    score s is itself only held to u |s|, which moves P, and every gradient
    with it, by that relative amount (8 covers the product, the subtraction of
    L, L's own rounding and exp)."""
    for g, r, name in zip(got, ref, ("dQ", "dK", "dV")):
        atol = 1e-5
        if smax is not None:
            atol = max(atol, 8 * 2.0 ** -24 * smax * float(np.abs(to64(r)).max()))
        check_fp32(g, r, name + tag, atol=atol)


@pytest.mark.parametrize("causal", [False, True])
def test_worked_example_shape(causal):
    """n = 8, d = 4 ("FlashAttention Algorithm > Worked Example"), with an
    upstream gradient drawn from the same seed family."""
    Q, K, V, _ = worked_example()
    t = lambda a: torch.tensor(a, dtype=torch.float32).reshape(1, 1, 8, 4)
    dO = attention_inputs(1, 1, 8, 4, "fp32", seed=5)[0]
    got = run(t(Q), t(K), t(V), dO, causal)
    ref = oracle.attention_bwd_ref(t(Q), t(K), t(V), dO, 0.5, causal)
    check_all(got, ref)


@pytest.mark.parametrize("causal", [False, True])
def test_random_n8_d4(causal):
    q, k, v, dO = attention_inputs(1, 1, 8, 4, "fp32", seed=0, with_grad=True)
    check_all(run(q, k, v, dO, causal), oracle.attention_bwd_ref(q, k, v, dO, 0.5, causal))


@pytest.mark.parametrize("N", [1, 7, 64, 65, 200])
@pytest.mark.parametrize("d", [1, 4, 30, 64, 128, 129, 200, 256])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 45), (False, 30)])
def test_shape_matrix(N, d, causal, window):
    """Both tile shapes (64-row tiles up to d = 128, 32-row beyond), head
    sizes that are not multiples of 4, ragged tails and every mask."""
    q, k, v, dO = attention_inputs(1, 2, N, d, "fp32", seed=N + d, with_grad=True)
    got = run(q, k, v, dO, causal, window)
    check_all(got, oracle.attention_bwd_ref(q, k, v, dO, 1 / math.sqrt(d), causal, window))


@pytest.mark.parametrize("B,H,N,d", [(2, 3, 700, 128), (1, 2, 333, 256), (4, 8, 64, 32)])
@pytest.mark.parametrize("causal,window", [(True, -1), (False, -1), (True, 100)])
def test_multi_tile(B, H, N, d, causal, window):
    """Several key and query tiles per head; (4, 8, 64, 32) is the gradient
    test shape of "Building Flash Attention from Scratch in Pure NumPy"."""
    q, k, v, dO = attention_inputs(B, H, N, d, "fp32", seed=B * N + d, with_grad=True)
    got = run(q, k, v, dO, causal, window)
    check_all(got, oracle.attention_bwd_ref(q, k, v, dO, 1 / math.sqrt(d), causal, window))


@pytest.mark.parametrize("factor", [0.0, -1.0, 2.0])
def test_scale_values(factor):
    d = 64
    scale = factor / math.sqrt(d)
    q, k, v, dO = attention_inputs(1, 2, 150, d, "fp32", seed=3, with_grad=True)
    got = run(q, k, v, dO, True, 40, scale)
    check_all(got, oracle.attention_bwd_ref(q, k, v, dO, scale, True, 40))


@pytest.mark.parametrize("offset", [-40.0, 25.0])
def test_row_offsets(offset):
    """Scores shifted far from zero per row (q_i gets a multiple of a
    direction every key shares): the softmax is shift-invariant, so the
    gradients are those of the unshifted problem, taken by the oracle."""
    N, d = 180, 64
    q, k, v, dO = attention_inputs(1, 2, N, d, "fp32", seed=11, with_grad=True)
    k = k.clone()
    k[..., 0] = 1.0
    q = q.clone()
    q[..., 0] = offset * math.sqrt(d)
    got = run(q, k, v, dO, True)
    smax = float(np.abs(to64(q)[0] @ to64(k)[0].transpose(0, 2, 1)).max()) / math.sqrt(d)
    check_all(got, oracle.attention_bwd_ref(q, k, v, dO, 1 / math.sqrt(d), True), smax=smax)


def test_backward_is_deterministic():
    q, k, v, dO = attention_inputs(2, 2, 300, 100, "fp32", seed=4, with_grad=True)
    a = run(q, k, v, dO, True)
    b = run(q, k, v, dO, True)
    for x, y, name in zip(a, b, ("dQ", "dK", "dV")):
        assert torch.equal(x, y), name


@pytest.mark.parametrize("N,d", [(65, 128), (100, 200)])
def test_outputs_written_only_in_bounds(N, d):
    """Guard bands after dq, dk, dv and the workspace stay untouched."""
    B, H = 1, 2
    q, k, v, dO = (t.cuda() for t in attention_inputs(B, H, N, d, "fp32", seed=N, with_grad=True))
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    n = B * H * N * d
    bufs = [torch.full((n + 4096,), 7.0, dtype=torch.float32, device="cuda") for _ in range(3)]
    need = fa.fa_bwd_workspace_size(B, H, N, d)
    wbuf = torch.full((need // 4 + 4096,), 7.0, dtype=torch.float32, device="cuda")
    dq, dk, dv = (b[:n].view(B, H, N, d) for b in bufs)
    fa.fa_bwd(q, k, v, o, dO, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=wbuf[:need // 4])
    torch.cuda.synchronize()
    for b, name in zip(bufs, ("dq", "dk", "dv")):
        assert torch.all(b[n:] == 7.0), name
    assert torch.all(wbuf[need // 4:] == 7.0)
    ref = oracle.attention_bwd_ref(q.cpu(), k.cpu(), v.cpu(), dO.cpu(), 1 / math.sqrt(d), True)
    check_all((dq.cpu(), dk.cpu(), dv.cpu()), ref)


def test_gradient_identities():
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per (b, h): the rows of P
    sum to one and dS's rows to zero."""
    q, k, v, dO = attention_inputs(1, 3, 400, 64, "fp32", seed=9, with_grad=True)
    dq, dk, dv = run(q, k, v, dO, True)
    assert np.abs(to64(dk).sum(axis=2)).max() <= 1e-4
    assert np.abs(to64(dv).sum(axis=2) - to64(dO).sum(axis=2)).max() <= 1e-4


def test_tuning_calls_refuse_float32():
    q, k, v, dO = (t.cuda() for t in attention_inputs(1, 1, 64, 64, "fp32", seed=1, with_grad=True))
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    with pytest.raises(fa.FaError):
        fa.fa_bwd_tune(q, k, v, o, dO, lse, causal=True)
