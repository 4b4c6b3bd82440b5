"""GPU parity of fa_decode (split-K + logsumexp merge) against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_04_amd as fa
from parity import check_bf16, check_fp32, check_lse, need_gpu
from tiled_attention_04_amd.inputs import (WORKLOADS, attention_inputs, decode_inputs, dense_cache,
                                          paged_cache)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run(inp, Lmax, window=-1, chunk=0, scale=None):
    kc, vc = dense_cache(inp, Lmax, device="cuda")  # rows past the length are NaN
    sl = torch.from_numpy(inp.seqlens).cuda()
    o, lse = fa.fa_decode(inp.q.cuda(), kc, vc, sl, window=window, chunk=chunk, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def oracle_decode(inp, window=-1, scale=None):
    d = inp.q.shape[2]
    s = 1 / math.sqrt(d) if scale is None else scale
    S, H = inp.q.shape[:2]
    o = np.empty((S, H, d))
    lse = np.empty((S, H))
    for i in range(S):
        n = int(inp.seqlens[i])
        # a cache holding exactly the valid rows; the oracle reads rows < n only
        oi, li = oracle.decode_ref(inp.q[i:i + 1], inp.k_rows[i][None], inp.v_rows[i][None], [n], s, window)
        o[i], lse[i] = oi[0], li[0]
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("chunk", [0, 64, 128, 320])
@pytest.mark.parametrize("window", [-1, 0, 70])
def test_small_ragged_batch(d, dtype, chunk, window):
    lens = [1, 2, 63, 64, 65, 300, 129]
    inp = decode_inputs(len(lens), 3, d, 1, 300, dtype=dtype, seed=d + chunk, seqlens=lens)
    o, lse = run(inp, 300, window, chunk)
    O, L = oracle_decode(inp, window)
    if dtype == "fp32":
        check_fp32(o, O, "o")
        check_fp32(lse, L, "lse")
    else:
        check_bf16(o, O, "o")
        check_lse(lse, L, "lse")


def test_split_count_independence():
    """The merge is associative: every split length gives the same result."""
    lens = [700, 1, 1024, 513]
    inp = decode_inputs(4, 4, 128, 1, 1024, seed=2, seqlens=lens)
    outs = [run(inp, 1024, -1, c) for c in (64, 128, 192, 512, 1024)]
    for o, l in outs[1:]:
        check_bf16(o, outs[0][0], "o vs chunk 64")
        check_lse(l, outs[0][1], "lse vs chunk 64")


def test_decode_equals_last_row_of_causal_forward():
    """Decode of the newest token = last row of the causal forward (both GPU)."""
    B, H, N, d = 1, 4, 777, 128
    q, k, v = attention_inputs(B, H, N, d, "bf16", seed=9)
    o_f, l_f = fa.fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    sl = torch.tensor([N], dtype=torch.int32, device="cuda")
    o_d, l_d = fa.fa_decode(q[0, :, N - 1][None].cuda().contiguous(), k.cuda(), v.cuda(), sl)
    torch.cuda.synchronize()
    check_bf16(o_d[0].cpu(), o_f[0, :, N - 1].cpu(), "decode vs forward")
    check_lse(l_d[0].cpu(), l_f[0, :, N - 1].cpu(), "lse decode vs forward")


def test_seqlens_out_of_range_are_clamped():
    lens = np.array([0, 5, 999], dtype=np.int32)  # 0 -> 1 row, 999 -> Lmax rows
    inp = decode_inputs(3, 2, 64, 1, 100, seed=4, seqlens=[1, 5, 100])
    kc, vc = dense_cache(inp, 100, device="cuda")
    o, lse = fa.fa_decode(inp.q.cuda(), kc, vc, torch.from_numpy(lens).cuda())
    O, L = oracle_decode(inp)
    check_bf16(o.cpu(), O, "o")
    check_lse(lse.cpu(), L, "lse")


@pytest.mark.slow
def test_full_size_ragged_decode():
    """64 sequences x 32 heads, d=128, lengths U[512, 8192]: every (s, h)."""
    w = WORKLOADS["decode_s64_h32_d128_len512to8192_bf16"]
    inp = decode_inputs(w["S"], w["H"], w["d"], w["len_lo"], w["len_hi"], seed=0)
    o, lse = run(inp, w["Lmax"])
    O, L = oracle_decode(inp)
    check_bf16(o, O, "o")
    check_lse(lse, L, "lse")


@pytest.mark.slow
def test_full_size_ragged_decode_window():
    """The windowed decode stage the bench times: the ragged batch with a
    1024-token window, every (sequence, head) against the oracle."""
    w = WORKLOADS["decode_s64_h32_d128_len512to8192_bf16"]
    inp = decode_inputs(w["S"], w["H"], w["d"], w["len_lo"], w["len_hi"], seed=0)
    o, lse = run(inp, w["Lmax"], window=1024)
    O, L = oracle_decode(inp, window=1024)
    check_bf16(o, O, "o")
    check_lse(lse, L, "lse")


# ------------------------------------------------------------ paged cache --

def run_paged(inp, page_size, window=-1, chunk=0, scale=None, spare=2, seed=0, hide=()):
    kp, vp, table = paged_cache(inp, page_size, device="cuda", seed=seed, spare_pages=spare)
    for s, j, val in hide:  # table entries outside the pool hide their tokens
        table[s, j] = val
    sl = torch.from_numpy(inp.seqlens).cuda()
    o, lse = fa.fa_decode_paged(inp.q.cuda(), kp, vp, table, sl, window=window, chunk=chunk,
                                scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), (kp.cpu(), vp.cpu(), table.cpu().numpy())


def oracle_paged(inp, pool, window=-1, scale=None):
    kp, vp, table = pool
    d = inp.q.shape[2]
    s = 1 / math.sqrt(d) if scale is None else scale
    return oracle.decode_paged_ref(inp.q, kp, vp, table, inp.seqlens, s, window)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("page_size,chunk", [(64, 0), (64, 192), (128, 64), (192, 320)])
@pytest.mark.parametrize("window", [-1, 0, 70])
def test_paged_small_ragged_batch(d, dtype, page_size, chunk, window):
    lens = [1, 2, 63, 64, 65, 300, 129, 500]
    inp = decode_inputs(len(lens), 3, d, 1, 500, dtype=dtype, seed=d + page_size, seqlens=lens)
    o, lse, pool = run_paged(inp, page_size, window, chunk, seed=chunk)
    O, L = oracle_paged(inp, pool, window)
    if dtype == "fp32":
        check_fp32(o, O, "o")
        check_fp32(lse, L, "lse")
    else:
        check_bf16(o, O, "o")
        check_lse(lse, L, "lse")


def test_paged_equals_dense_decode():
    lens = [700, 1, 1024, 513, 64, 65]
    inp = decode_inputs(len(lens), 4, 128, 1, 1024, seed=5, seqlens=lens)
    o_p, l_p, _ = run_paged(inp, 64, chunk=256)
    o_d, l_d = run(inp, 1024, -1, 256)
    check_bf16(o_p, o_d, "paged vs dense o")
    check_lse(l_p, l_d, "paged vs dense lse")


def test_paged_hidden_table_entries_drop_their_tokens():
    """Entries -1 and >= num_pages hide whole pages (never read)."""
    lens = [300, 260, 129]
    inp = decode_inputs(len(lens), 2, 128, 1, 300, seed=6, seqlens=lens)
    hide = [(0, 0, -1), (0, 2, 1 << 30), (1, 1, -5)]
    o, lse, pool = run_paged(inp, 64, hide=hide)
    O, L = oracle_paged(inp, pool)
    check_bf16(o, O, "o")
    check_lse(lse, L, "lse")


def test_paged_sequence_with_every_page_hidden():
    lens = [100, 150]
    inp = decode_inputs(len(lens), 2, 64, 1, 150, seed=7, seqlens=lens)
    o, lse, pool = run_paged(inp, 64, hide=[(0, 0, -1), (0, 1, -1)])
    O, L = oracle_paged(inp, pool)
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    check_bf16(o[1], O[1], "o")
    check_lse(lse[1], L[1], "lse")


@pytest.mark.slow
def test_full_size_ragged_paged_decode():
    """The ragged decode batch (64 x 32, d=128, lengths U[512, 8192]) in
    64-token pages: sampled (sequence, head) pairs against the oracle."""
    w = WORKLOADS["decode_s64_h32_d128_len512to8192_bf16"]
    inp = decode_inputs(w["S"], w["H"], w["d"], w["len_lo"], w["len_hi"], seed=0)
    o, lse, pool = run_paged(inp, 64)
    kp, vp, table = pool
    rng = np.random.default_rng(1)
    for s in rng.choice(w["S"], 8, replace=False):
        O, L = oracle.decode_paged_ref(inp.q[s:s + 1], kp, vp, table[s:s + 1], inp.seqlens[s:s + 1],
                                       1 / math.sqrt(w["d"]))
        check_bf16(o[s], O[0], f"o[{s}]")
        check_lse(lse[s], L[0], f"lse[{s}]")


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("window", [-1, 50])
def test_outputs_written_only_in_bounds(paged, window):
    """Guard bands after o, lse and the workspace stay untouched."""
    lens = [1, 130, 257, 64]
    S, H, d = len(lens), 3, 128
    inp = decode_inputs(S, H, d, 1, 257, seed=9, seqlens=lens)
    sl = torch.from_numpy(inp.seqlens).cuda()
    n = S * H * d
    obuf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((S * H + 1024,), 7.0, dtype=torch.float32, device="cuda")
    o, lse = obuf[:n].view(S, H, d), lbuf[:S * H].view(S, H)
    if paged:
        kp, vp, table = paged_cache(inp, 64, device="cuda", seed=3, spare_pages=1)
        need = fa.fa_decode_workspace_size(S, H, table.shape[1] * 64, d)
        wbuf = torch.full((need // 4 + 4096,), 7.0, dtype=torch.float32, device="cuda")
        fa.fa_decode_paged(inp.q.cuda(), kp, vp, table, sl, window=window, o=o, lse=lse,
                           workspace=wbuf[:need // 4])
    else:
        kc, vc = dense_cache(inp, 257, device="cuda")
        need = fa.fa_decode_workspace_size(S, H, 257, d)
        wbuf = torch.full((need // 4 + 4096,), 7.0, dtype=torch.float32, device="cuda")
        fa.fa_decode(inp.q.cuda(), kc, vc, sl, window=window, o=o, lse=lse, workspace=wbuf[:need // 4])
    torch.cuda.synchronize()
    assert torch.all(obuf[n:] == 7.0) and torch.all(lbuf[S * H:] == 7.0)
    assert torch.all(wbuf[need // 4:] == 7.0)
    O, L = oracle_decode(inp, window)
    check_bf16(o.cpu(), O, "o")
    check_lse(lse.cpu(), L, "lse")


def test_decode_check_flags_what_the_decode_repairs():
    """fa_decode_check reports the lengths the decode clamps and the absent
    pages it leaves out -- only among the pages the call reads."""
    Lmax = 100
    lens = torch.tensor([0, 5, 100, 101, -3], dtype=torch.int32, device="cuda")
    f = fa.fa_decode_check(lens, Lmax=Lmax)
    assert f.cpu().tolist() == [fa.FA_CHECK_LENGTH, 0, 0, fa.FA_CHECK_LENGTH, fa.FA_CHECK_LENGTH]
    # Paged: 64-token pages, 4 table columns, a pool of 10 pages.
    lens = torch.tensor([130, 300, 64, 200, 1], dtype=torch.int32, device="cuda")
    table = torch.tensor([[1, 2, -1, 99],     # token 128-129 on an absent page
                          [0, 1, 2, 3],       # 300 > 4 * 64: clamped to 256, every page present
                          [3, 99, 99, 99],    # only page 0 is read
                          [99, 99, 4, 5],     # pages 0 and 1 absent
                          [10, 0, 0, 0]],     # entry == num_pages: absent
                         dtype=torch.int32, device="cuda")
    f = fa.fa_decode_check(lens, table, page_size=64, num_pages=10).cpu().tolist()
    assert f == [fa.FA_CHECK_PAGE, fa.FA_CHECK_LENGTH, 0, fa.FA_CHECK_PAGE, fa.FA_CHECK_PAGE]
    # With a 50-token window sequence 3 reads tokens 149..199 (pages 2 and 3):
    # the absent pages 0 and 1 are never read.
    f = fa.fa_decode_check(lens, table, page_size=64, num_pages=10, window=50).cpu().tolist()
    assert f == [fa.FA_CHECK_PAGE, fa.FA_CHECK_LENGTH, 0, 0, fa.FA_CHECK_PAGE]
    # A batch the decode tests use is clean.
    inp = decode_inputs(3, 2, 128, 1, 300, seed=6, seqlens=[300, 260, 129])
    sl = torch.from_numpy(inp.seqlens).cuda()
    assert not fa.fa_decode_check(sl, Lmax=300).any()
