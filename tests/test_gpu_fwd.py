"""GPU parity of fa_fwd against the fp64 oracle (through the C ABI)."""

import math

import numpy as np
import pytest
import torch

import oracle
import tiled_attention_04_amd as fa
from golden_io import worked_example
from parity import check_bf16, check_fp32, check_lse, need_gpu, to64
from tiled_attention_04_amd.inputs import WORKLOADS, attention_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def run(q, k, v, causal=False, window=-1, scale=None, bq=0, bk=0):
    o, lse = fa.fa_fwd_ex(q.cuda(), k.cuda(), v.cuda(), bq, bk, causal=causal, window=window,
                          scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


# ------------------------------------------------------------------ fp32 ---
# The worked example's setting: n=8, d=4, block size 4 (2 query x 2 K/V tiles).

@pytest.mark.parametrize("causal", [False, True])
def test_tiny_random_fp32_block4(causal):
    w = WORKLOADS["tiny_n8_d4_fp32"]
    q, k, v = attention_inputs(w["B"], w["H"], w["N"], w["d"], "fp32", seed=0)
    o, lse = run(q, k, v, causal, bq=4, bk=4)
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(4), causal)
    check_fp32(o, O, "O")
    check_fp32(lse, L, "L")


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_worked_example_fp32_block4(causal):
    Q, K, V, exp = worked_example()
    t = lambda a: torch.tensor(a, dtype=torch.float32).reshape(1, 1, 8, 4)
    o, lse = run(t(Q), t(K), t(V), causal, bq=4, bk=4)
    O, L = oracle.attention_ref(Q[None, None], K[None, None], V[None, None], 0.5, causal)
    check_fp32(o, O, "O")
    check_fp32(lse, L, "L")
    if not causal:  # the page's printed rows 0-3
        got = to64(o)[0, 0, :4]
        assert np.abs(got - exp["O_rows0to3"][0]).max() <= exp["O_rows0to3"][1]


@pytest.mark.parametrize("N,d", [(64, 32), (128, 64), (256, 64), (512, 128), (37, 5), (1, 1)])
@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 64), (64, 32), (3, 5)])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 9)])
def test_fp32_shape_and_block_matrix(N, d, bq, bk, causal, window):
    """The NumPy page's (N, d) x (block_q, block_k) test matrix, plus odd sizes."""
    q, k, v = attention_inputs(1, 2, N, d, "fp32", seed=N + d)
    o, lse = run(q, k, v, causal, window, bq=bq, bk=bk)
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(d), causal, window)
    check_fp32(o, O, "O")
    check_fp32(lse, L, "L")


@pytest.mark.parametrize("d,bq,bk", [(256, 0, 0), (256, 32, 31), (200, 40, 17), (129, 63, 63)])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 50)])
def test_fp32_large_head_dims(d, bq, bk, causal, window):
    """Head sizes above 128 on the float32 kernel (tiles sized to its LDS)."""
    q, k, v = attention_inputs(1, 2, 150, d, "fp32", seed=d)
    o, lse = run(q, k, v, causal, window, bq=bq, bk=bk)
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(d), causal, window)
    check_fp32(o, O, "O")
    check_fp32(lse, L, "L")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 31, 33, 128, 129, 300, 1000])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 45), (False, 30), (True, 0)])
def test_fp32_matrix_core_tile(N, d, causal, window):
    """The automatic float32 tile at d = 64 and 128: 128 query rows x 32 keys
    on float32 MFMA, ragged tails and every mask."""
    assert fa.fa_fwd_auto_tile(1, 2, N, d, dtype=torch.float32)[0] == (128, 32)
    q, k, v = attention_inputs(1, 2, N, d, "fp32", seed=N + d + 1)
    o, lse = run(q, k, v, causal, window)
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(d), causal, window)
    check_fp32(o, O, "O")
    check_fp32(lse, L, "L")


@pytest.mark.parametrize("causal,window", [(True, -1), (False, -1), (True, 1024)])
def test_fp32_matrix_core_many_heads(causal, window):
    """2 x 16 x 2048 x 128 float32 (a grid over every XCD), sampled heads
    against the oracle; the explicit 128 x 32 tile gives the same bits."""
    q, k, v = attention_inputs(2, 16, 2048, 128, "fp32", seed=5)
    o, lse = run(q, k, v, causal, window)
    o2, lse2 = run(q, k, v, causal, window, bq=128, bk=32)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    s = 1 / math.sqrt(128)
    for b, h in ((0, 0), (1, 11)):
        O, L = oracle.attention_ref(q[b, h], k[b, h], v[b, h], s, causal, window)
        check_fp32(o[b, h], O, f"O[{b},{h}]")
        check_fp32(lse[b, h], L, f"L[{b},{h}]")


@pytest.mark.parametrize("offset", [-40.0, 25.0])
def test_fp32_matrix_core_row_offsets(offset):
    """Every score of a row shifted far from zero: the softmax is
    shift-invariant.  A float32 score s is itself held only to 2^-24 |s|, so
    the bar widens to max(1e-5, 8 * 2^-24 * max|s| * max|O|)."""
    N, d = 180, 64
    q, k, v = attention_inputs(1, 2, N, d, "fp32", seed=11)
    k = k.clone()
    k[..., 0] = 1.0
    q = q.clone()
    q[..., 0] = offset * math.sqrt(d)
    o, lse = run(q, k, v, True)
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(d), True)
    smax = float(np.abs(to64(q)[0] @ to64(k)[0].transpose(0, 2, 1)).max()) / math.sqrt(d)
    check_fp32(o, O, "O", atol=max(1e-5, 8 * 2.0 ** -24 * smax * float(np.abs(O).max())))
    check_fp32(lse, L, "L", atol=max(1e-5, 8 * 2.0 ** -24 * smax))


# ------------------------------------------------------------------ bf16 ---

@pytest.mark.parametrize("causal", [False, True])
def test_bf16_n1024_d64_tile64(causal):
    w = WORKLOADS["fwd_b1_h8_n1024_d64_bf16"]
    q, k, v = attention_inputs(w["B"], w["H"], w["N"], w["d"], "bf16", seed=0)
    o, lse = run(q, k, v, causal, bq=64, bk=64)
    O, L = oracle.attention_ref(q, k, v, 1 / 8, causal)
    check_bf16(o, O, "O")
    check_lse(lse, L, "L")


MASKS = [(False, -1), (True, -1), (True, 37), (False, 20), (True, 0)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 37, 64, 65, 200, 333])
@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("bq", [32, 64, 128, 256])
def test_bf16_ragged_masks_tiles(d, N, causal, window, bq):
    q, k, v = attention_inputs(2, 2, N, d, "bf16", seed=7 * N + d)
    o, lse = run(q, k, v, causal, window, bq=bq)
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(d), causal, window)
    check_bf16(o, O, "O")
    check_lse(lse, L, "L")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 33, 200, 333])
@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 32), (128, 32), (32, 128), (64, 128), (128, 128)])
def test_bf16_key_tiles_32_and_128(d, N, causal, window, bq, bk):
    """The 32- and 128-key tiles of the 1-4 wave kernels (128 at d = 64 only)
    over ragged lengths and every mask."""
    if bk == 128 and d != 64:
        pytest.skip("128-key tiles are built for d = 64 only")
    q, k, v = attention_inputs(2, 2, N, d, "bf16", seed=11 * N + d + bk)
    o, lse = run(q, k, v, causal, window, bq=bq, bk=bk)
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(d), causal, window)
    check_bf16(o, O, "O")
    check_lse(lse, L, "L")


@pytest.mark.parametrize("bq,bk", [(128, 32), (64, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_key_tiles_many_heads_and_fp16(bq, bk, dtype):
    """A grid of several workgroups per CU in both 16-bit types, the key
    tiles other than 64, sampled heads against the oracle."""
    d = 64
    q, k, v = attention_inputs(2, 48, 900, d, dtype, seed=bq + bk)
    o, lse = run(q, k, v, True, -1, bq=bq, bk=bk)
    for b, h in ((0, 3), (1, 47)):
        O, L = oracle.attention_ref(q[b, h][None], k[b, h][None], v[b, h][None], 1 / math.sqrt(d), True)
        check_bf16(o[b, h], O[0], "O")
        check_lse(lse[b, h], L[0], "L")


@pytest.mark.parametrize("B,H,N,d", [(1, 160, 700, 128), (2, 96, 1100, 64)])
@pytest.mark.parametrize("causal,window", [(True, -1), (False, -1), (True, 200), (False, 300)])
def test_bf16_many_query_tiles_per_workgroup(B, H, N, d, causal, window):
    """More 256-row query tiles than compute units, so each workgroup of the
    256-row kernel runs several of them back to back (ragged N, all masks)."""
    q, k, v = attention_inputs(B, H, N, d, "bf16", seed=N + H)
    o, lse = run(q, k, v, causal, window, bq=256)
    O, L = oracle.attention_ref(q, k, v, 1 / math.sqrt(d), causal, window)
    check_bf16(o, O, "O")
    check_lse(lse, L, "L")


@pytest.mark.parametrize("scale", [0.0, -0.3, 0.9])
def test_bf16_scale_values(scale):
    q, k, v = attention_inputs(1, 3, 150, 128, "bf16", seed=3)
    o, lse = run(q, k, v, True, -1, scale=scale)
    O, L = oracle.attention_ref(q, k, v, scale, True)
    check_bf16(o, O, "O")
    check_lse(lse, L, "L")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 32), ("fp32", 128)])
@pytest.mark.parametrize("causal,window", [(True, -1), (True, 23), (False, 23)])
def test_masked_positions_contribute_exactly_zero(dtype, d, causal, window):
    """Perturbing K and V where the mask hides them leaves O and L bitwise equal."""
    N, r = 300, 150
    q, k, v = attention_inputs(1, 2, N, d, dtype, seed=11)
    o1, l1 = run(q, k, v, causal, window)
    k2, v2 = k.clone(), v.clone()
    if causal:
        k2[:, :, r:] = 1e4 * torch.randn(k2[:, :, r:].shape).to(k2.dtype)
        v2[:, :, r:] = -3e3
        rows = slice(0, r)
        if window >= 0:
            k2[:, :, : r - 1 - window] = 50.0
            rows = slice(r - 1, r)
    else:
        k2[:, :, :5] = 1e4
        v2[:, :, :5] = 2e3
        rows = slice(5 + window, N)
    o2, l2 = run(q, k2, v2, causal, window)
    assert torch.equal(o1[:, :, rows], o2[:, :, rows])
    assert torch.equal(l1[:, :, rows], l2[:, :, rows])


def test_forward_is_deterministic():
    q, k, v = attention_inputs(2, 4, 777, 128, "bf16", seed=5)
    a = run(q, k, v, True)
    b = run(q, k, v, True)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 128), ("fp32", 64), ("fp32", 40)])
def test_output_written_only_in_bounds(dtype, d):
    """Guard band after o and lse stays untouched (16-bit, float32 matrix-core
    and float32 vector-ALU kernels)."""
    B, H, N = 1, 2, 65
    q, k, v = (t.cuda() for t in attention_inputs(B, H, N, d, dtype, seed=1))
    n = B * H * N * d
    obuf = torch.full((n + 4096,), 7.0, dtype=q.dtype, device="cuda")
    lbuf = torch.full((B * H * N + 1024,), 7.0, dtype=torch.float32, device="cuda")
    fa.fa_fwd(q, k, v, causal=True, o=obuf[:n].view(B, H, N, d), lse=lbuf[: B * H * N].view(B, H, N))
    torch.cuda.synchronize()
    assert torch.all(obuf[n:] == 7.0) and torch.all(lbuf[B * H * N:] == 7.0)
    O, L = oracle.attention_ref(q.cpu(), k.cpu(), v.cpu(), 1 / math.sqrt(d), True)
    check = check_fp32 if dtype == "fp32" else check_bf16
    check(obuf[:n].view(B, H, N, d).cpu(), O, "O")
    check_lse(lbuf[: B * H * N].view(B, H, N).cpu(), L, "L")


# -------------------------------------------- full size: 4 x 32 x 4096 x 128

@pytest.fixture(scope="module")
def llama_layer():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    w = WORKLOADS["fwd_b4_h32_n4096_d128_bf16"]
    q, k, v = attention_inputs(w["B"], w["H"], w["N"], w["d"], "bf16", seed=0)
    return q, k, v, (q.cuda(), k.cuda(), v.cuda())


SAMPLED_HEADS = [(0, 0), (1, 17), (3, 31)]


@pytest.mark.parametrize("causal,window", [(True, -1), (True, 1024)])
def test_full_size_sampled_heads(llama_layer, causal, window):
    q, k, v, (qd, kd, vd) = llama_layer
    o, lse = fa.fa_fwd(qd, kd, vd, causal=causal, window=window)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    s = 1 / math.sqrt(128)
    for b, h in SAMPLED_HEADS:
        O, L = oracle.attention_ref(q[b, h][None], k[b, h][None], v[b, h][None], s, causal, window)
        check_bf16(o[b, h], O[0], f"O[{b},{h}]")
        check_lse(lse[b, h], L[0], f"L[{b},{h}]")


@pytest.mark.parametrize("window", [-1, 1024])
def test_full_size_scale_zero_property(llama_layer, window):
    """scale = 0: every row averages its visible V rows and L = ln(#visible),
    checked on every row of every head (the mask at full size)."""
    _, _, _, (qd, kd, vd) = llama_layer
    o, lse = fa.fa_fwd(qd, kd, vd, causal=True, window=window, scale=0.0)
    N = qd.shape[2]
    i = torch.arange(N, device="cuda", dtype=torch.float64)
    cnt = i + 1 if window < 0 else torch.clamp(i + 1, max=window + 1)
    assert torch.max(torch.abs(lse.double() - torch.log(cnt))) <= 1e-3
    c = torch.cumsum(vd.double(), dim=2)
    if window >= 0:
        c = c - torch.nn.functional.pad(c, (0, 0, window + 1, 0))[:, :, :N]
    mean = c / cnt[None, None, :, None]
    diff = o.double() - mean
    assert diff.abs().max().item() <= 2e-2
    assert (diff.norm() / mean.norm()).item() <= 1e-2


# ------------------------------------------------ long sequences, one head

@pytest.mark.parametrize("causal,window", [(True, -1), (True, 3000), (False, -1)])
def test_long_sequence_sampled_rows(causal, window):
    """N = 65536 in one (batch, head): the 256-row kernel's key loop runs 1024
    tiles and the offsets inside the slice reach 16 MiB.  Sampled rows, each
    computed on its own by the oracle."""
    N, d = 65536, 128
    q, k, v = attention_inputs(1, 1, N, d, "bf16", seed=12)
    o, lse = run(q, k, v, causal, window, bq=256)
    rows = [0, 1, 255, 256, 4095, 30001, 65534, 65535]
    O, L = oracle.attention_rows_ref(q[0, 0], k[0, 0], v[0, 0], 1 / math.sqrt(d), rows, causal, window)
    check_bf16(o[0, 0, rows], O, "O rows")
    check_lse(lse[0, 0, rows], L, "L rows")


def test_heads_not_multiple_of_eight_use_plain_order():
    """B*H = 13: the XCD-aware tile order falls back to the plain one."""
    q, k, v = attention_inputs(1, 13, 600, 64, "bf16", seed=13)
    for bq in (128, 256):
        o, lse = run(q, k, v, True, -1, bq=bq)
        O, L = oracle.attention_ref(q, k, v, 1 / 8, True)
        check_bf16(o, O, "O")
        check_lse(lse, L, "L")


@pytest.mark.parametrize("bk", [32, 64])
def test_automatic_tile_with_explicit_key_tile(bk):
    """fa_fwd_ex(block_q = 0, block_k) where the built-in choice is the 256-row
    kernel (64-key tiles only): a 32-key request runs 128 query rows instead,
    and the result is the explicit tile's, bit for bit."""
    B, H, N, d = 1, 64, 1024, 128
    fa.fa_tune_reset()
    assert fa.fa_fwd_auto_tile(B, H, N, d, causal=True) == ((256, 64), False)
    q, k, v = (t.cuda() for t in attention_inputs(B, H, N, d, "bf16", seed=12))
    o, lse = fa.fa_fwd_ex(q, k, v, 0, bk, causal=True)
    o_ref, lse_ref = fa.fa_fwd_ex(q, k, v, 256 if bk == 64 else 128, bk, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    O, L = oracle.attention_ref(q[0, 5][None].cpu(), k[0, 5][None].cpu(), v[0, 5][None].cpu(), 1 / math.sqrt(d), True)
    check_bf16(o[0, 5].cpu(), O[0], "O")
    check_lse(lse[0, 5].cpu(), L[0], "L")
