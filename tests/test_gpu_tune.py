"""GPU checks of the tuning calls (fa_fwd_tune, fa_decode_tune, fa_bwd_tune):
each measures its candidates, remembers the fastest, and automatic calls then
run that choice."""

import math

import pytest
import torch

import oracle
import tiled_attention_04_amd as fa
from parity import check_bf16, check_lse, need_gpu
from tiled_attention_04_amd.inputs import attention_inputs, decode_inputs, dense_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    fa.fa_tune_reset()
    yield
    fa.fa_tune_reset()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal,window", [(True, -1), (True, 100), (False, -1)])
def test_tune_remembers_the_fastest_tile(dtype, causal, window):
    B, H, N, d = 2, 8, 700, 128
    q, k, v = attention_inputs(B, H, N, d, dtype, seed=4)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    best, times, o, lse = fa.fa_fwd_tune(qd, kd, vd, causal=causal, window=window, reps=3)
    assert best in fa.TUNE_CANDIDATES
    ran = {t: ms for t, ms in times.items() if ms >= 0}
    # every tile ran except the 128-key ones at d = 128
    assert set(times) - set(ran) == {t for t in fa.TUNE_CANDIDATES if t[1] == 128 and d != 64}
    assert all(ms > 0 for ms in ran.values())
    assert times[best] == min(ran.values())
    assert fa.fa_fwd_auto_tile(B, H, N, d, causal=causal, window=window, dtype=qd.dtype) == (best, True)
    assert fa.fa_fwd_auto_block_q(B, H, N, d, causal=causal, window=window, dtype=qd.dtype) == (best[0], True)
    # the tuned outputs, an explicit call with that tile and the automatic call agree bit for bit
    o_ex, l_ex = fa.fa_fwd_ex(qd, kd, vd, best[0], best[1], causal=causal, window=window)
    o_auto, l_auto = fa.fa_fwd(qd, kd, vd, causal=causal, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ex) and torch.equal(lse, l_ex)
    assert torch.equal(o_auto, o_ex) and torch.equal(l_auto, l_ex)
    # and they are right
    O, L = oracle.attention_ref(q[1, 5][None], k[1, 5][None], v[1, 5][None], 1 / math.sqrt(d), causal,
                                window)
    check_bf16(o[1, 5].cpu(), O[0], "O")
    check_lse(lse[1, 5].cpu(), L[0], "L")


def test_tuned_choice_is_per_problem():
    q, k, v = (t.cuda() for t in attention_inputs(1, 4, 300, 64, "bf16", seed=1))
    best, times, _, _ = fa.fa_fwd_tune(q, k, v, causal=True, reps=2)
    assert min(times.values()) > 0  # at d = 64 every tile runs
    assert fa.fa_fwd_auto_tile(1, 4, 300, 64, causal=True) == (best, True)
    assert not fa.fa_fwd_auto_block_q(1, 4, 301, 64, causal=True)[1]
    assert not fa.fa_fwd_auto_block_q(1, 4, 300, 64, causal=False)[1]
    assert not fa.fa_fwd_auto_block_q(1, 4, 300, 64, causal=True, dtype=torch.float16)[1]
    fa.fa_tune_reset()
    assert not fa.fa_fwd_auto_block_q(1, 4, 300, 64, causal=True)[1]


def _oracle_decode_seq(inp, i, window):
    d = inp.q.shape[2]
    n = int(inp.seqlens[i])
    return oracle.decode_ref(inp.q[i:i + 1], inp.k_rows[i][None], inp.v_rows[i][None], [n], 1 / math.sqrt(d),
                             window)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("window", [-1, 300])
def test_decode_tune_remembers_the_fastest_split(dtype, window):
    """fa_decode_tune times the split lengths that keep within an automatic
    call's workspace, remembers the fastest, and automatic calls (dense and
    no-allocation) then use it: same bits as an explicit call with that split."""
    lens = [1, 700, 2100, 4100, 64, 3000]
    Lmax = 4100
    inp = decode_inputs(len(lens), 4, 128, 1, Lmax, dtype=dtype, seed=11, seqlens=lens)
    kc, vc = dense_cache(inp, Lmax, device="cuda")
    q, sl = inp.q.cuda(), torch.from_numpy(inp.seqlens).cuda()
    S, H, d = q.shape
    best, times, o, lse = fa.fa_decode_tune(q, kc, vc, sl, window=window, reps=3)
    ran = {c: t for c, t in times.items() if t >= 0}
    assert best in ran and ran[best] == min(ran.values())
    # skipped: splits shorter than the shortest automatic one, and those past one split
    min_auto = fa.fa_decode_auto_chunk(S, H, Lmax, d, window=0, dtype=q.dtype)[0]
    cands = fa.DECODE_TUNE_CANDIDATES
    for i, c in enumerate(cands):
        assert (times[c] >= 0) == (c >= min_auto and (i == 0 or cands[i - 1] < Lmax)), (c, times)
    assert fa.fa_decode_auto_chunk(S, H, Lmax, d, window=window, dtype=q.dtype) == (best, True)
    o_ex, l_ex = fa.fa_decode(q, kc, vc, sl, window=window, chunk=best)
    o_auto, l_auto = fa.fa_decode(q, kc, vc, sl, window=window)
    o_na, l_na = fa.fa_decode_noalloc(q, kc, vc, sl, window=window)
    torch.cuda.synchronize()
    for a, b in ((o, o_ex), (lse, l_ex), (o_auto, o_ex), (l_auto, l_ex), (o_na, o_ex), (l_na, l_ex)):
        assert torch.equal(a, b)
    for i in (1, 3):
        O, L = _oracle_decode_seq(inp, i, window)
        check_bf16(o[i].cpu(), O[0], "o")
        check_lse(lse[i].cpu(), L[0], "lse")
    # a different problem is not tuned
    assert not fa.fa_decode_auto_chunk(S, H, Lmax + 64, d, window=window, dtype=q.dtype)[1]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d,causal,window", [(128, True, -1), (64, False, -1), (128, True, 200)])
def test_bwd_tune_remembers_the_faster_dq_kernel(dtype, d, causal, window):
    """fa_bwd_tune times the backward with each way of forming dQ, remembers
    the fastest, and fa_bwd then uses it; dV does not depend on the choice."""
    B, H, N = 1, 4, 700
    q, k, v, dO = attention_inputs(B, H, N, d, dtype, seed=21, with_grad=True)
    qd, kd, vd, gd = (t.cuda() for t in (q, k, v, dO))
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, window=window)
    # every candidate is tried: the workspace holds the stored dS (at this size the binding's
    # default would not provide it)
    ws_bytes = fa.fa_bwd_workspace_size_ds(B, H, N, d, causal, window)
    best, times, (dq, dk, dv) = fa.fa_bwd_tune(qd, kd, vd, o, gd, lse, causal=causal, window=window, reps=3,
                                               stored_ds=True)
    assert set(times) == set(fa.BWD_TUNE_CANDIDATES) and min(times.values()) > 0
    assert best in fa.BWD_TUNE_CANDIDATES and times[best] == min(times.values())
    assert fa.fa_bwd_auto_dq_rows(B, H, N, d, causal=causal, window=window, dtype=qd.dtype,
                                  workspace_bytes=ws_bytes) == (best, True)
    dq2, dk2, dv2 = fa.fa_bwd(qd, kd, vd, o, gd, lse, causal=causal, window=window, stored_ds=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    rq, rk, rv = oracle.attention_bwd_ref(q[:, 2:3], k[:, 2:3], v[:, 2:3], dO[:, 2:3], 1 / math.sqrt(d), causal,
                                          window)
    # every other choice: identical dV; between the two recompute kernels identical dK and dQ
    # to rounding order; the stored-dS path sums D in another kernel, so its dS can round to a
    # neighbouring 16-bit value: dK and dQ then agree at the parity bar (checked on one head)
    for other in fa.BWD_TUNE_CANDIDATES:
        if other == best:
            continue
        fa.fa_tune_import([dict(kind=fa.TUNE_KINDS["bwd_dq_rows"],
                                dtype=fa.FA_FP16 if dtype == "fp16" else fa.FA_BF16, d=d, causal=int(causal),
                                window=window, rows=B * H, n=N, value=other)])
        assert fa.fa_bwd_auto_dq_rows(B, H, N, d, causal=causal, window=window, dtype=qd.dtype,
                                      workspace_bytes=ws_bytes) == (other, True)
        dq3, dk3, dv3 = fa.fa_bwd(qd, kd, vd, o, gd, lse, causal=causal, window=window, stored_ds=True)
        torch.cuda.synchronize()
        assert torch.equal(dv, dv3)
        if (other == fa.FA_BWD_DQ_STORED) == (best == fa.FA_BWD_DQ_STORED):
            assert torch.equal(dk, dk3)
            assert torch.allclose(dq, dq3, rtol=1e-5, atol=1e-5)
        else:
            check_bf16(dq3[:, 2:3].cpu(), rq, f"dQ ({other})")
            check_bf16(dk3[:, 2:3].cpu(), rk, f"dK ({other})")
    check_bf16(dq[:, 2:3].cpu(), rq, "dQ")
    check_bf16(dk[:, 2:3].cpu(), rk, "dK")
    check_bf16(dv[:, 2:3].cpu(), rv, "dV")
