"""The library's calls under HIP graph capture (torch.cuda.graph).

Every compute entry point launches on the caller's stream and makes no
allocation, memset or synchronising call, so a whole step can be captured
once and replayed.  The graph here holds the causal forward and backward
(bf16 and float32), the dense, paged and allocation-free decodes; it is
replayed three times with new inputs copied into its buffers eagerly in
between (and the program's own eager calls and synchronisations between the
replays), and every replay must equal eager calls on the same inputs bit for
bit (the kernels are deterministic).
"""

import pytest
import torch

import tiled_attention_04_amd as fa
from parity import need_gpu
from tiled_attention_04_amd.inputs import attention_inputs, decode_inputs, dense_cache, paged_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def test_captured_step_replays_match_eager_calls():
    B, H, N, d = 2, 4, 700, 128
    dev = "cuda"
    # Static buffers of the captured step.
    q, k, v, g = (t.to(dev) for t in attention_inputs(B, H, N, d, "bf16", seed=1, with_grad=True))
    q32, k32, v32, g32 = (t.to(dev) for t in attention_inputs(1, 2, 300, 64, "fp32", seed=2, with_grad=True))
    inp = decode_inputs(4, 4, 128, 64, 600, seed=3)
    Lmax = 600
    kc, vc = dense_cache(inp, Lmax, device=dev)
    kp, vp, table = paged_cache(inp, 64, device=dev, seed=3)
    qd = inp.q.to(dev)
    lens0 = torch.from_numpy(inp.seqlens).to(dev)
    sl = lens0.clone()

    o, lse = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
    # the stored-dS backward, as the eager call below
    ws = torch.empty(fa.fa_bwd_workspace_size_ds(B, H, N, d, True, -1), dtype=torch.uint8, device=dev)
    o32, lse32 = torch.empty_like(q32), torch.empty((1, 2, 300), dtype=torch.float32, device=dev)
    dq32, dk32, dv32 = (torch.empty_like(q32) for _ in range(3))
    ws32 = torch.empty(fa.fa_bwd_workspace_size(1, 2, 300, 64), dtype=torch.uint8, device=dev)
    od, ld = torch.empty_like(qd), torch.empty(qd.shape[:2], dtype=torch.float32, device=dev)
    op, lp = torch.empty_like(qd), torch.empty_like(ld)
    on, ln = torch.empty_like(qd), torch.empty_like(ld)
    wsd = torch.empty(fa.fa_decode_workspace_size(4, 4, Lmax, 128), dtype=torch.uint8, device=dev)
    wsp = torch.empty(fa.fa_decode_workspace_size(4, 4, table.shape[1] * 64, 128), dtype=torch.uint8, device=dev)

    def step():
        fa.fa_fwd(q, k, v, causal=True, o=o, lse=lse)
        fa.fa_bwd(q, k, v, o, g, lse, causal=True, dq=dq, dk=dk, dv=dv, workspace=ws)
        fa.fa_fwd(q32, k32, v32, causal=True, window=50, o=o32, lse=lse32)
        fa.fa_bwd(q32, k32, v32, o32, g32, lse32, causal=True, window=50, dq=dq32, dk=dk32, dv=dv32,
                  workspace=ws32)
        fa.fa_decode(qd, kc, vc, sl, o=od, lse=ld, workspace=wsd)
        fa.fa_decode_paged(qd, kp, vp, table, sl, o=op, lse=lp, workspace=wsp)
        fa.fa_decode_noalloc(qd, kc, vc, sl, o=on, lse=ln)

    # Warm up on a side stream (default priority), then capture.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        # New inputs, copied eagerly into the graph's buffers; decode lengths
        # stay within the rows the caches hold.
        nq, nk, nv, ng = attention_inputs(B, H, N, d, "bf16", seed=10 + rep, with_grad=True)
        for dst, src in ((q, nq), (k, nk), (v, nv), (g, ng)):
            dst.copy_(src.to(dev))
        for dst, src in zip((q32, k32, v32, g32), attention_inputs(1, 2, 300, 64, "fp32", seed=20 + rep,
                                                                   with_grad=True)):
            dst.copy_(src.to(dev))
        qd.copy_(decode_inputs(4, 4, 128, 64, 600, seed=30 + rep).q.to(dev))
        sl.copy_(torch.clamp(lens0 - 37 * rep, min=1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv, o32, lse32, dq32, dk32, dv32, od, ld, op, lp, on, ln)]

        eo, el = fa.fa_fwd(q, k, v, causal=True)
        edq, edk, edv = fa.fa_bwd(q, k, v, eo, g, el, causal=True, stored_ds=True)
        eo32, el32 = fa.fa_fwd(q32, k32, v32, causal=True, window=50)
        edq32, edk32, edv32 = fa.fa_bwd(q32, k32, v32, eo32, g32, el32, causal=True, window=50)
        eod, eld = fa.fa_decode(qd, kc, vc, sl)
        eop, elp = fa.fa_decode_paged(qd, kp, vp, table, sl)
        eon, eln = fa.fa_decode_noalloc(qd, kc, vc, sl)
        torch.cuda.synchronize()
        want = [eo, el, edq, edk, edv, eo32, el32, edq32, edk32, edv32, eod, eld, eop, elp, eon, eln]
        names = ["o", "lse", "dq", "dk", "dv", "o32", "lse32", "dq32", "dk32", "dv32", "decode o", "decode lse",
                 "paged o", "paged lse", "noalloc o", "noalloc lse"]
        for a, b, name in zip(got, want, names):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
