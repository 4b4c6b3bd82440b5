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
    for must in ("fa_fwd", "fa_fwd_ex", "fa_fwd_tune", "fa_tune_export", "fa_tune_import", "fa_decode", "fa_decode_paged", "fa_bwd", "fa_decode_workspace_size",
                 "fa_bwd_workspace_size", "fa_status_str", "fa_last_error", "fa_version"):
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
    (dict(d=96), 2), (dict(d=257, dtype=0), 2), (dict(d=256, dtype=0, bq=64, bk=32), 1),
    (dict(d=256, dtype=0, bq=32, bk=64), 1), (dict(d=171, dtype=0, bq=32, bk=48), 1), (dict(d=96, dtype=2), 2), (dict(dtype=3), 1),
    (dict(dtype=2, bq=48), 1),
    (dict(bq=48), 1), (dict(bq=512), 1), (dict(bk=32), 1), (dict(dtype=0, bq=65, bk=4), 1), (dict(dtype=0, bq=0, bk=5), 1),
    (dict(B=1 << 16, H=1 << 16), 1),
    (dict(N=1 << 23, d=128), 2),          # one slice of N*d bf16 above 2 GiB
    (dict(N=1 << 22, d=128, dtype=0), 2),  # the same in float32
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    assert fwd(lib, **kw) == status
    assert fa355.last_error() != ""


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


def test_tune_rejects_bad_arguments_and_starts_empty(lib):
    def call(**kw):
        a = dict(q=FAKE, B=1, H=2, N=64, d=128, scale=0.1, causal=1, window=-1, dtype=1, reps=5)
        a.update(kw)
        return lib.fa_fwd_tune(a["q"], FAKE, FAKE, FAKE, None, a["B"], a["H"], a["N"], a["d"], a["scale"],
                               a["causal"], a["window"], a["dtype"], None, a["reps"], None, None)
    assert call(q=None) == 1
    assert call(N=0) == 1
    assert call(reps=0) == 1
    assert call(reps=1001) == 1
    assert call(window=-3) == 1
    assert call(dtype=0) == 2
    assert call(d=96) == 2
    lib.fa_tune_reset()
    # nothing tuned: the heuristic (256 rows only when the grid fills 256 CUs)
    assert fa355.fa_fwd_auto_block_q(1, 2, 64, 128, causal=True) == (32, False)
    assert fa355.fa_fwd_auto_block_q(4, 32, 4096, 128, causal=True) == (256, False)
    assert fa355.fa_fwd_auto_block_q(4, 32, 4096, 128, causal=True, window=1024) == (128, False)
    assert fa355.fa_fwd_auto_block_q(1, 1, 8, 4, dtype=torch.float32) == (64, False)
    assert fa355.fa_fwd_auto_block_q(0, 1, 8, 4)[0] == 0


def test_tune_table_export_import_round_trip(tmp_path, lib):
    """The remembered tile table is host state: it round-trips through
    export/import and a JSON file, and a bad row changes nothing."""
    lib.fa_tune_reset()
    rows = [dict(dtype=1, d=128, causal=1, window=-1, BH=128, N=4096, block_q=256),
            dict(dtype=2, d=64, causal=0, window=100, BH=8, N=1024, block_q=128)]
    fa355.fa_tune_import(rows)
    assert sorted(fa355.fa_tune_export(), key=str) == sorted(rows, key=str)
    assert fa355.fa_fwd_auto_block_q(1, 8, 1024, 64, window=100, dtype=torch.float16) == (128, True)
    assert fa355.fa_fwd_auto_block_q(4, 32, 4096, 128, causal=True) == (256, True)
    path = str(tmp_path / "tune.json")
    fa355.save_tuning(path)
    lib.fa_tune_reset()
    assert fa355.fa_tune_export() == []
    fa355.load_tuning(path)
    assert sorted(fa355.fa_tune_export(), key=str) == sorted(rows, key=str)
    for bad in (dict(rows[0], block_q=96), dict(rows[0], dtype=0), dict(rows[0], d=80),
                dict(rows[0], causal=2), dict(rows[0], window=-2), dict(rows[0], N=0)):
        with pytest.raises(fa355.FaError):
            fa355.fa_tune_import([rows[1] | {"N": 7}, bad])
        assert len(fa355.fa_tune_export()) == 2  # unchanged
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
    assert call(dtype=0) == 2
    assert call(dtype=3) == 1
    assert call(d=32) == 2
    assert call(d=32, dtype=2) == 2
    assert call(wsb=8) == 3


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
