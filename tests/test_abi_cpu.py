"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest
import torch

from tiled_attention_04_amd import build as fa_build
from tiled_attention_04_amd import fa355

HEADER = os.path.join(fa_build.ROOT, "include", "fa355.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails before any HIP call


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa355.LIB_PATH):
        fa_build.build()
    return fa355.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_calls():
    names = declared_functions()
    for must in ("fa_fwd", "fa_fwd_ex", "fa_fwd_tune", "fa_tune_export", "fa_tune_import", "fa_decode_tune",
                 "fa_decode_auto_chunk", "fa_bwd_tune", "fa_bwd_auto_dq_rows", "fa_decode", "fa_decode_paged",
                 "fa_bwd", "fa_decode_workspace_size", "fa_bwd_workspace_size", "fa_status_str", "fa_last_error",
                 "fa_version", "fa_decode_check"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in fa355.SIGNATURES, f"binding lacks a signature for {name}"


def test_header_has_no_torch_or_hip_types():
    code = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    assert "hipStream_t" not in code and "hip/" not in code
    assert "at::" not in code and "Tensor" not in code and "torch" not in code


def test_status_strings(lib):
    assert lib.fa_version() >= 100
    assert fa355.status_str(0) == "FA_OK"
    assert fa355.status_str(1) == "FA_ERR_INVALID_ARG"
    assert fa355.status_str(2) == "FA_ERR_UNSUPPORTED"
    assert fa355.status_str(3) == "FA_ERR_WORKSPACE"
    assert fa355.status_str(4) == "FA_ERR_HIP"


def fwd(lib, q=FAKE, B=1, H=1, N=8, d=64, scale=0.125, causal=0, window=-1, dtype=1, bq=0, bk=0):
    return lib.fa_fwd_ex(q, FAKE, FAKE, FAKE, None, B, H, N, d, scale, causal, window, dtype, None, bq, bk)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(B=0), 1), (dict(N=-3), 1), (dict(d=0), 1),
    (dict(causal=2), 1), (dict(window=-2), 1), (dict(scale=float("inf")), 1),
    (dict(scale=float("nan")), 1), (dict(dtype=7), 1),
    (dict(d=96), 2), (dict(d=257, dtype=0), 2), (dict(d=256, dtype=0, bq=64, bk=65), 1),
    (dict(d=200, dtype=0, bq=0, bk=64), 1), (dict(d=96, dtype=0, bq=128, bk=32), 1),
    (dict(d=128, dtype=0, bq=128, bk=64), 1), (dict(d=96, dtype=2), 2), (dict(dtype=3), 1),
    (dict(dtype=2, bq=48), 1),
    (dict(bq=48), 1), (dict(bq=512), 1), (dict(bq=256, bk=32), 1), (dict(bq=64, bk=96), 1),
    (dict(d=128, bq=64, bk=128), 1), (dict(bq=256, bk=128), 1),
    (dict(dtype=0, bq=65, bk=4), 1), (dict(dtype=0, bq=0, bk=5), 1),
    (dict(B=1 << 16, H=1 << 16), 1),
    (dict(N=1 << 23, d=128), 2),          # one slice of N*d bf16 above 2 GiB
    (dict(N=1 << 22, d=128, dtype=0), 2),  # the same in float32
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert fa355.last_error() != ""


def test_decode_check_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(sl=FAKE, table=None, S=4, L=128, ps=64, mp=4, npg=10, window=-1, flags=FAKE)
        a.update(kw)
        return lib.fa_decode_check(a["sl"], a["table"], a["S"], a["L"], a["ps"], a["mp"], a["npg"], a["window"],
                                   a["flags"], None)
    assert call(sl=None) == 1
    assert call(flags=None) == 1
    assert call(S=-1) == 1
    assert call(window=-2) == 1
    assert call(L=0) == 1                       # dense cache needs a length
    assert call(table=FAKE, L=0, ps=0) == 1     # paged: sizes must be positive
    assert call(table=FAKE, mp=0) == 1
    assert call(table=FAKE, npg=0) == 1
    assert call(table=FAKE, ps=1 << 20, mp=1 << 12) == 1
    assert "2^31" in fa355.last_error()
    assert call(S=0) == 0                       # nothing to check: no launch
    assert call(S=0, table=FAKE, L=0) == 0


def test_decode_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, sl=FAKE, o=FAKE, S=2, H=2, L=128, d=128, scale=0.1,
                 window=-1, chunk=0, ws=FAKE, wsb=1 << 30, dtype=1)
        a.update(kw)
        return lib.fa_decode(a["q"], a["kc"], a["vc"], a["sl"], a["o"], None, a["S"], a["H"], a["L"],
                             a["d"], a["scale"], a["window"], a["chunk"], a["ws"], a["wsb"], a["dtype"], None)
    assert call(sl=None) == 1
    assert call(S=0) == 1
    assert call(chunk=100) == 1
    assert call(chunk=-64) == 1
    assert call(window=-5) == 1
    assert call(d=96) == 2
    assert call(ws=None) == 3
    assert call(wsb=16) == 3
    assert "workspace" in fa355.last_error()


def test_decode_noalloc_rejects_bad_arguments_and_oversized_requests(lib):
    def call(**kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, sl=FAKE, o=FAKE, S=2, H=2, L=128, d=128, scale=0.1,
                 window=-1, chunk=0, dtype=1)
        a.update(kw)
        return lib.fa_decode_noalloc(a["q"], a["kc"], a["vc"], a["sl"], a["o"], None, a["S"], a["H"],
                                     a["L"], a["d"], a["scale"], a["window"], a["chunk"], a["dtype"], None)
    assert call(q=None) == 1
    assert call(S=0) == 1
    assert call(chunk=100) == 1
    assert call(window=-5) == 1
    assert call(scale=float("inf")) == 1
    assert call(d=96) == 2
    # 64 x 32 caches of 8192 rows in 64-token splits: 136 MB of partials, above
    # the 32 MiB static scratch -- refused before any HIP call
    assert call(S=64, H=32, L=8192, chunk=64) == 3
    assert "static scratch" in fa355.last_error()
    # the largest request that fits (d = 128, 1024-token splits): 64,527 partials
    assert fa355.fa_decode_workspace_size(64527, 1, 1024, 128, 1024) <= 32 << 20
    assert fa355.fa_decode_workspace_size(64528, 1, 1024, 128, 1024) > 32 << 20
    assert call(S=64528, H=1, L=1024, chunk=1024) == 3


def test_tune_rejects_bad_arguments_and_starts_empty(lib):
    def call(**kw):
        a = dict(q=FAKE, B=1, H=2, N=64, d=128, scale=0.1, causal=1, window=-1, dtype=1, reps=5)
        a.update(kw)
        return lib.fa_fwd_tune(a["q"], FAKE, FAKE, FAKE, None, a["B"], a["H"], a["N"], a["d"], a["scale"],
                               a["causal"], a["window"], a["dtype"], None, a["reps"], None, None, None)
    assert call(q=None) == 1
    assert call(N=0) == 1
    assert call(reps=0) == 1
    assert call(reps=1001) == 1
    assert call(window=-3) == 1
    assert call(dtype=0) == 2
    assert call(d=96) == 2
    lib.fa_tune_reset()
    # nothing tuned: the heuristic (256 rows only when the grid fills 256 CUs)
    assert fa355.fa_fwd_auto_block_q(1, 2, 64, 128, causal=True) == (128, False)
    assert fa355.fa_fwd_auto_block_q(4, 32, 4096, 128, causal=True) == (256, False)
    assert fa355.fa_fwd_auto_block_q(4, 32, 4096, 128, causal=True, window=1024) == (128, False)
    assert fa355.fa_fwd_auto_block_q(1, 1, 8, 4, dtype=torch.float32) == (64, False)
    assert fa355.fa_fwd_auto_tile(4, 32, 4096, 128, causal=True) == ((256, 64), False)
    assert fa355.fa_fwd_auto_tile(4, 32, 4096, 128, causal=True, window=1024) == ((128, 32), False)
    assert fa355.fa_fwd_auto_tile(1, 2, 64, 128, causal=True) == ((128, 32), False)
    assert fa355.fa_fwd_auto_tile(1, 2, 64, 64, causal=True) == ((128, 64), False)
    assert fa355.fa_fwd_auto_tile(4, 32, 4096, 64, causal=True) == ((128, 64), False)
    assert fa355.fa_fwd_auto_tile(4, 32, 4096, 128, causal=True, window=128) == ((32, 32), False)
    assert fa355.fa_fwd_auto_tile(4, 32, 4096, 128, causal=True, window=129) == ((128, 32), False)
    assert fa355.fa_fwd_auto_tile(1, 8, 1024, 128) == ((128, 32), False)
    assert fa355.fa_fwd_auto_tile(1, 1, 8, 4, dtype=torch.float32) == ((64, 64), False)
    # float32 at d = 64 and 128: the matrix-core kernel's 128 x 32
    assert fa355.fa_fwd_auto_tile(2, 16, 4096, 128, dtype=torch.float32) == ((128, 32), False)
    assert fa355.fa_fwd_auto_tile(1, 1, 8, 64, dtype=torch.float32) == ((128, 32), False)
    assert fa355.fa_fwd_auto_tile(1, 1, 8, 96, dtype=torch.float32) == ((64, 64), False)
    assert fa355.fa_fwd_auto_block_q(0, 1, 8, 4)[0] == 0


def test_tune_table_export_import_round_trip(tmp_path, lib):
    """The remembered tuning table is host state: it round-trips through
    export/import and a JSON file, every kind's rows steer the matching
    automatic choice, and a bad row changes nothing."""
    lib.fa_tune_reset()
    K = fa355.TUNE_KINDS
    rows = [dict(kind=K["fwd_tile"], dtype=1, d=128, causal=1, window=-1, rows=128, n=4096, value=256064),
            dict(kind=K["fwd_tile"], dtype=2, d=64, causal=0, window=100, rows=8, n=1024, value=128128),
            dict(kind=K["decode_chunk"], dtype=1, d=128, causal=0, window=-1, rows=2048, n=8192, value=2048),
            dict(kind=K["bwd_dq_rows"], dtype=1, d=128, causal=1, window=-1, rows=32, n=4096, value=128)]
    fa355.fa_tune_import(rows)
    assert sorted(fa355.fa_tune_export(), key=str) == sorted(rows, key=str)
    assert fa355.fa_fwd_auto_block_q(1, 8, 1024, 64, window=100, dtype=torch.float16) == (128, True)
    assert fa355.fa_fwd_auto_tile(1, 8, 1024, 64, window=100, dtype=torch.float16) == ((128, 128), True)
    assert fa355.fa_fwd_auto_tile(4, 32, 4096, 128, causal=True) == ((256, 64), True)
    assert fa355.fa_decode_auto_chunk(64, 32, 8192, 128) == (2048, True)
    assert fa355.fa_decode_auto_chunk(64, 32, 8192, 128, window=1024) == (512, False)
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=True) == (128, True)
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=False) == (1, False)
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=False, workspace_bytes=8) == (256, False)
    path = str(tmp_path / "tune.json")
    fa355.save_tuning(path)
    lib.fa_tune_reset()
    assert fa355.fa_tune_export() == []
    assert fa355.fa_decode_auto_chunk(64, 32, 8192, 128) == (1024, False)
    fa355.load_tuning(path)
    assert sorted(fa355.fa_tune_export(), key=str) == sorted(rows, key=str)
    for bad in (dict(rows[0], value=96), dict(rows[0], value=256), dict(rows[0], value=256128),
                dict(rows[0], value=128128), dict(rows[0], value=64096), dict(rows[0], dtype=0), dict(rows[0], d=80),
                dict(rows[0], causal=2), dict(rows[0], window=-2), dict(rows[0], n=0), dict(rows[0], kind=3),
                dict(rows[2], value=300), dict(rows[2], value=8192), dict(rows[2], causal=1),
                dict(rows[3], value=64), dict(rows[3], value=256 + 128)):
        with pytest.raises(fa355.FaError):
            fa355.fa_tune_import([rows[1] | {"n": 7}, bad])
        assert len(fa355.fa_tune_export()) == 4  # unchanged
    lib.fa_tune_reset()


def test_decode_and_bwd_tune_reject_bad_arguments(lib):
    """Argument checks of the decode and backward tuning calls happen before
    any HIP call (so they run here, without a GPU), and the automatic choices
    with nothing tuned are the built-in ones."""
    lib.fa_tune_reset()

    def dec(**kw):
        a = dict(q=FAKE, S=2, H=2, L=256, d=128, scale=0.1, window=-1, ws=FAKE, wsb=1 << 30, dtype=1, reps=3)
        a.update(kw)
        return lib.fa_decode_tune(a["q"], FAKE, FAKE, FAKE, FAKE, None, a["S"], a["H"], a["L"], a["d"],
                                  a["scale"], a["window"], a["ws"], a["wsb"], a["dtype"], None, a["reps"],
                                  None, None)
    assert dec(q=None) == 1
    assert dec(S=0) == 1
    assert dec(reps=0) == 1
    assert dec(reps=1001) == 1
    assert dec(window=-2) == 1
    assert dec(d=96) == 2
    assert dec(ws=None) == 3
    assert dec(wsb=16) == 3

    def bwd(**kw):
        a = dict(q=FAKE, B=1, H=2, N=64, d=128, scale=0.1, causal=1, window=-1, ws=FAKE, wsb=1 << 30,
                 dtype=1, reps=3)
        a.update(kw)
        return lib.fa_bwd_tune(a["q"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["H"], a["N"],
                               a["d"], a["scale"], a["causal"], a["window"], a["ws"], a["wsb"], a["dtype"],
                               None, a["reps"], None, None)
    assert bwd(q=None) == 1
    assert bwd(N=0) == 1
    assert bwd(reps=0) == 1
    assert bwd(dtype=0) == 2
    assert bwd(d=96) == 2
    assert bwd(ws=None) == 3
    # built-in choices: 1024-token splits without a window on the 64 x 32 batch, 512 under one;
    # the 256-row dQ kernel while its grid fills 256 CUs
    assert fa355.fa_decode_auto_chunk(64, 32, 8192, 128) == (1024, False)
    assert fa355.fa_decode_auto_chunk(64, 32, 8192, 128, window=1024) == (512, False)
    assert fa355.fa_decode_auto_chunk(0, 32, 8192, 128)[0] == 0
    # the backward: dQ from the stored dS when the workspace holds it (as the binding's default
    # does), else the recompute kernel whose grid fills the chip
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=True) == (1, False)
    small = fa355.fa_bwd_workspace_size(2, 16, 4096, 128)
    big = fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, True, -1)
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=True, workspace_bytes=small) == (256, False)
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=True, workspace_bytes=big - 1) == (256, False)
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=True, workspace_bytes=big) == (1, False)
    assert fa355.fa_bwd_auto_dq_rows(1, 8, 1024, 64, workspace_bytes=0) == (128, False)
    # the binding's default workspace stores dS only once the product grid fills the chip
    assert fa355.fa_bwd_auto_dq_rows(1, 8, 1024, 64) == (128, False)
    big64 = fa355.fa_bwd_workspace_size_ds(1, 8, 1024, 64, False, -1)
    assert fa355.fa_bwd_auto_dq_rows(1, 8, 1024, 64, workspace_bytes=big64) == (1, False)
    assert fa355.fa_bwd_auto_dq_rows(1, 8, 1024, 64, dtype=torch.float32)[0] == 0
    # a tuned stored-dS choice needs the workspace for it
    fa355.fa_tune_import([dict(kind=fa355.TUNE_KINDS["bwd_dq_rows"], dtype=1, d=128, causal=1, window=-1,
                               rows=32, n=4096, value=1)])
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=True) == (1, True)
    assert fa355.fa_bwd_auto_dq_rows(2, 16, 4096, 128, causal=True, workspace_bytes=small) == (256, False)
    lib.fa_tune_reset()


def test_decode_paged_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(q=FAKE, kp=FAKE, vp=FAKE, tb=FAKE, sl=FAKE, o=FAKE, S=2, H=2, d=128, num_pages=8,
                 page=64, max_pages=4, scale=0.1, window=-1, chunk=0, ws=FAKE, wsb=1 << 30, dtype=1)
        a.update(kw)
        return lib.fa_decode_paged(a["q"], a["kp"], a["vp"], a["tb"], a["sl"], a["o"], None, a["S"],
                                   a["H"], a["d"], a["num_pages"], a["page"], a["max_pages"],
                                   a["scale"], a["window"], a["chunk"], a["ws"], a["wsb"], a["dtype"],
                                   None)
    assert call(tb=None) == 1
    assert call(kp=None) == 1
    assert call(num_pages=0) == 1
    assert call(max_pages=0) == 1
    assert call(page=0) == 1
    assert call(page=32) == 1
    assert call(page=100) == 1
    assert call(page=1 << 20, max_pages=1 << 12) == 1
    assert call(chunk=96) == 1
    assert call(window=-2) == 1
    assert call(scale=float("nan")) == 1
    assert call(dtype=5) == 1
    assert call(d=80) == 2
    assert call(page=1 << 24, max_pages=1, dtype=0) == 2  # one page of one head above 2 GiB
    assert call(ws=None) == 3
    need = fa355.fa_decode_workspace_size(2, 2, 4 * 64, 128, 0)
    assert call(wsb=need - 1) == 3
    assert "workspace" in fa355.last_error()


def test_bwd_rejects_bad_arguments(lib):
    def call(**kw):
        a = dict(ptr=FAKE, B=1, H=1, N=64, d=128, dtype=1, ws=FAKE, wsb=1 << 20, window=-1)
        a.update(kw)
        p = a["ptr"]
        return lib.fa_bwd(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["H"], a["N"],
                          a["d"], 0.1, 1, a["window"], a["ws"], a["wsb"], a["dtype"], None)
    assert call(ptr=None) == 1
    assert call(N=0) == 1
    assert call(dtype=3) == 1
    assert call(d=32) == 2
    assert call(d=32, dtype=2) == 2
    assert call(wsb=8) == 3
    # float32: any d <= 256 passes the checks up to the workspace
    assert call(dtype=0, d=257) == 2
    assert call(dtype=0, d=32, wsb=8) == 3
    assert call(dtype=0, d=256, ws=None) == 3


def test_workspace_sizes(lib):
    # decode: S*H*ceil(Lmax/chunk) partials of (d + 2) floats
    assert fa355.fa_decode_workspace_size(64, 32, 8192, 128, 512) == 64 * 32 * 16 * 130 * 4
    assert fa355.fa_decode_workspace_size(2, 2, 100, 64, 64) == 2 * 2 * 2 * 66 * 4
    assert fa355.fa_decode_workspace_size(2, 2, 100, 64, 65) == 0
    assert fa355.fa_decode_workspace_size(0, 2, 100, 64, 64) == 0
    # auto chunk for the ragged decode batch is 512 tokens
    assert fa355.fa_decode_workspace_size(64, 32, 8192, 128, 0) == 64 * 32 * 16 * 130 * 4
    # backward: D and L (log2 units) per row
    assert fa355.fa_bwd_workspace_size(2, 16, 4096, 128) == 2 * 16 * 4096 * 2 * 4
    assert fa355.fa_bwd_workspace_size(0, 16, 4096, 128) == 0
    # stored dS: that (256-byte aligned), then a 2 KB block per visible (32-query, 32-key) block pair
    rows = 2 * 16 * 4096
    nb = 4096 // 32
    tri = nb * (nb + 1) // 2
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, True, -1) == rows * 8 + 32 * tri * 2048
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 64, False, -1) == rows * 8 + 32 * nb * nb * 2048
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, False, 100) == rows * 8 + 32 * nb * nb * 2048
    # a causal window of W keys: ceil(W / 32) + 1 blocks per query block (33 for W = 1024)
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, True, 1024) == rows * 8 + 32 * nb * 33 * 2048
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, True, 1000) == rows * 8 + 32 * nb * 33 * 2048
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, True, 0) == rows * 8 + 32 * nb * 1 * 2048
    # a window over the whole slice: the triangle
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, True, 5000) == rows * 8 + 32 * tri * 2048
    # ragged: D and L of 3 * 100 rows take 2400 bytes, padded to 2560
    assert fa355.fa_bwd_workspace_size_ds(1, 3, 100, 64, True, -1) == 2560 + 3 * 10 * 2048
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 96, True, -1) == 0
    assert fa355.fa_bwd_workspace_size_ds(0, 16, 4096, 128, True, -1) == 0
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, 2, -1) == 0
    assert fa355.fa_bwd_workspace_size_ds(2, 16, 4096, 128, True, -2) == 0
    # the binding allocates the stored-dS workspace up to its cap, else the minimum
    assert fa355.fa_bwd_default_workspace_size(2, 16, 4096, 128, True) == rows * 8 + 32 * tri * 2048
    assert fa355.fa_bwd_default_workspace_size(2, 16, 4096, 128, True, stored_ds=False) == rows * 8
    assert fa355.fa_bwd_default_workspace_size(2, 16, 4096, 128, True, dtype=torch.float32) == rows * 8
    assert fa355.fa_bwd_default_workspace_size(1, 32, 65536, 128, True) == 32 * 65536 * 8
    # below two product workgroups per CU (B * H * ceil(N / 128) < 512) the minimum, unless asked
    assert fa355.fa_bwd_default_workspace_size(1, 8, 1024, 64, True) == 8 * 1024 * 8
    assert fa355.fa_bwd_default_workspace_size(1, 8, 1024, 64, True, stored_ds=True) == \
        fa355.fa_bwd_workspace_size_ds(1, 8, 1024, 64, True, -1)
    assert fa355.fa_bwd_default_workspace_size(1, 16, 4096, 128, True) == 16 * 4096 * 8 + 16 * tri * 2048
