"""GPU parity of the fp16 instantiations (forward, backward, decode, paged
decode) against the fp64 oracle.  fp16 inputs run the same matrix-core and
decode kernels as bf16 (v_mfma_f32_32x32x16_f16, fp32 accumulation) and are
held to the same bar."""

import math

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_04_amd as fa
from parity import check_bf16, check_lse, need_gpu
from tiled_attention_04_amd.inputs import attention_inputs, decode_inputs, dense_cache, paged_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


MASKS = [(False, -1), (True, -1), (True, 37), (False, 20)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 333])
@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("bq", [32, 64, 128, 256])
def test_fp16_forward(d, N, causal, window, bq):
    q, k, v = attention_inputs(2, 2, N, d, "fp16", seed=5 * N + d)
    o, lse = fa.fa_fwd_ex(q.cuda(), k.cuda(), v.cuda(), bq, 0, causal=causal, window=window)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(d), causal, window)
    check_bf16(o.cpu(), O, "O")
    check_lse(lse.cpu(), L, "L")


@pytest.mark.parametrize("scale", [0.0, -0.4])
def test_fp16_forward_scale_values(scale):
    q, k, v = attention_inputs(1, 3, 150, 128, "fp16", seed=3)
    o, lse = fa.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_ref(q, k, v, scale, True)
    check_bf16(o.cpu(), O, "O")
    check_lse(lse.cpu(), L, "L")


def test_fp16_forward_full_size_sampled_heads():
    """4 x 32 x 4096 x 128 causal in fp16 (256-row kernel): three whole heads."""
    q, k, v = attention_inputs(4, 32, 4096, 128, "fp16", seed=0)
    o, lse = fa.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    for b, h in [(0, 0), (2, 9), (3, 31)]:
        O, L = oracle.attention_ref(q[b, h][None], k[b, h][None], v[b, h][None], 1 / math.sqrt(128), True)
        check_bf16(o[b, h], O[0], f"O[{b},{h}]")
        check_lse(lse[b, h], L[0], f"L[{b},{h}]")


def test_fp16_masked_positions_contribute_exactly_zero():
    N, r = 300, 150
    q, k, v = attention_inputs(1, 2, N, 128, "fp16", seed=11)
    o1, l1 = fa.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, r:] = 1e4
    v2[:, :, r:] = -3e3
    o2, l2 = fa.fa_fwd(q.cuda(), k2.cuda(), v2.cuda(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :r], o2[:, :, :r]) and torch.equal(l1[:, :, :r], l2[:, :, :r])


@pytest.mark.parametrize("stored_ds", [True, False], ids=["stored_ds", "recompute"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [64, 257])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 45)])
def test_fp16_backward(d, N, causal, window, stored_ds):
    q, k, v, dO = attention_inputs(1, 2, N, d, "fp16", seed=N + d, with_grad=True)
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, dO))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, window=window)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, gd, lse, causal=causal, window=window, stored_ds=stored_ds)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_ref(q, k, v, dO, 1 / math.sqrt(d), causal, window)
    check_bf16(dq.cpu(), rq, "dQ")
    check_bf16(dk.cpu(), rk, "dK")
    check_bf16(dv.cpu(), rv, "dV")


@pytest.mark.parametrize("stored_ds", [True, False], ids=["stored_ds", "recompute"])
def test_fp16_backward_many_tiles(stored_ds):
    """Enough heads that the 256-row recompute dQ kernel is chosen (grid fills
    the chip) when dS is not stored."""
    q, k, v, dO = attention_inputs(2, 64, 600, 128, "fp16", seed=2, with_grad=True)
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, dO))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, gd, lse, causal=True, stored_ds=stored_ds)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (1, 63)]:
        rq, rk, rv = oracle.attention_bwd_ref(q[b, h][None], k[b, h][None], v[b, h][None],
                                              dO[b, h][None], 1 / math.sqrt(128), True)
        check_bf16(dq[b, h].cpu(), rq[0], "dQ")
        check_bf16(dk[b, h].cpu(), rk[0], "dK")
        check_bf16(dv[b, h].cpu(), rv[0], "dV")


def _decode_oracle(inp, window):
    S, H, d = inp.q.shape
    o = np.empty((S, H, d))
    lse = np.empty((S, H))
    for i in range(S):
        oi, li = oracle.decode_ref(inp.q[i:i + 1], inp.k_rows[i][None], inp.v_rows[i][None],
                                   [int(inp.seqlens[i])], 1 / math.sqrt(d), window)
        o[i], lse[i] = oi[0], li[0]
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [-1, 70])
@pytest.mark.parametrize("paged", [False, True])
def test_fp16_decode(d, window, paged):
    lens = [1, 63, 64, 65, 300, 129]
    inp = decode_inputs(len(lens), 3, d, 1, 300, dtype="fp16", seed=d, seqlens=lens)
    sl = torch.from_numpy(inp.seqlens).cuda()
    if paged:
        kp, vp, table = paged_cache(inp, 64, device="cuda", seed=1, spare_pages=2)
        o, lse = fa.fa_decode_paged(inp.q.cuda(), kp, vp, table, sl, window=window)
    else:
        kc, vc = dense_cache(inp, 300, device="cuda")
        o, lse = fa.fa_decode(inp.q.cuda(), kc, vc, sl, window=window)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    O, L = _decode_oracle(inp, window)
    check_bf16(o.cpu(), O, "o")
    check_lse(lse.cpu(), L, "lse")


# ------------------------------------------- full size: the timed fp16 stages

@pytest.mark.slow
def test_fp16_full_size_ragged_decode():
    """The fp16 decode stage the bench times: 64 sequences x 32 heads, d=128,
    lengths U[512, 8192], automatic splits (1024 tokens); every (s, h)."""
    from tiled_attention_04_amd.inputs import WORKLOADS
    w = WORKLOADS["decode_s64_h32_d128_len512to8192_bf16"]
    inp = decode_inputs(w["S"], w["H"], w["d"], w["len_lo"], w["len_hi"], dtype="fp16", seed=0)
    kc, vc = dense_cache(inp, w["Lmax"], device="cuda")
    sl = torch.from_numpy(inp.seqlens).cuda()
    o, lse = fa.fa_decode(inp.q.cuda(), kc, vc, sl)
    torch.cuda.synchronize()
    del kc, vc
    O, L = _decode_oracle(inp, -1)
    check_bf16(o.cpu(), O, "o")
    check_lse(lse.cpu(), L, "lse")


@pytest.mark.slow
def test_fp16_full_size_backward_sampled_heads():
    """The fp16 backward stage the bench times: B=2, H=16, N=4096, d=128,
    causal (the 256-row dQ kernel); two whole heads against the oracle."""
    q, k, v, dO = attention_inputs(2, 16, 4096, 128, "fp16", seed=0, with_grad=True)
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, dO))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, o, gd, lse, causal=True)
    torch.cuda.synchronize()
    for b, h in ((0, 4), (1, 13)):
        rq, rk, rv = oracle.attention_bwd_ref(q[b, h][None], k[b, h][None], v[b, h][None],
                                              dO[b, h][None], 1 / math.sqrt(128), True)
        check_bf16(dq[b, h].cpu(), rq[0], f"dQ[{b},{h}]")
        check_bf16(dk[b, h].cpu(), rk[0], f"dK[{b},{h}]")
        check_bf16(dv[b, h].cpu(), rv[0], f"dV[{b},{h}]")
