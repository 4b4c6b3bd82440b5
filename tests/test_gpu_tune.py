"""GPU checks of the forward's tile tuning (fa_fwd_tune): it measures every
candidate, remembers the fastest, and automatic calls then run that tile."""

import math

import pytest
import torch

import oracle
import tiled_attention_04_amd as fa
from parity import check_bf16, check_lse, need_gpu
from tiled_attention_04_amd.inputs import attention_inputs

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
    assert all(t > 0 for t in times.values())
    assert times[best] == min(times.values())
    assert fa.fa_fwd_auto_block_q(B, H, N, d, causal=causal, window=window, dtype=qd.dtype) == (best, True)
    # the tuned outputs, an explicit call with that tile and the automatic call agree bit for bit
    o_ex, l_ex = fa.fa_fwd_ex(qd, kd, vd, best, 64, causal=causal, window=window)
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
    best, _, _, _ = fa.fa_fwd_tune(q, k, v, causal=True, reps=2)
    assert fa.fa_fwd_auto_block_q(1, 4, 300, 64, causal=True) == (best, True)
    assert not fa.fa_fwd_auto_block_q(1, 4, 301, 64, causal=True)[1]
    assert not fa.fa_fwd_auto_block_q(1, 4, 300, 64, causal=False)[1]
    assert not fa.fa_fwd_auto_block_q(1, 4, 300, 64, causal=True, dtype=torch.float16)[1]
    fa.fa_tune_reset()
    assert not fa.fa_fwd_auto_block_q(1, 4, 300, 64, causal=True)[1]
