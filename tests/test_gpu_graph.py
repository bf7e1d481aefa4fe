"""The fused launch inside a captured HIP graph: every replay equals the eager launch.

Replays are interleaved with eager launches of the same op on other buffers, output wipes
(torch fill kernels, not memsets) and device synchronizations."""
import pytest
import torch

from rmsnorm_quantization_amd import binding as B
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    GH.require_gpu()


@pytest.mark.parametrize("mode,G", [(B.RMSQ_FP8_STATIC, 0), (B.RMSQ_FP8_TOKEN, 0),
                                    (B.RMSQ_FP8_GROUP, 128), (B.RMSQ_FP4_BLOCK16, 16)])
def test_graph_replays_match_eager(mode, G):
    T, H = 96, 4096
    g = torch.Generator().manual_seed(77)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda()
    r = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda()
    w = (torch.rand((H,), generator=g) + 0.5).to(torch.bfloat16).cuda()
    sc = torch.tensor([0.02 if mode == B.RMSQ_FP8_STATIC else 300.0], device="cuda") \
        if mode in (B.RMSQ_FP8_STATIC, B.RMSQ_FP4_BLOCK16) else None
    qcols = H // 2 if mode == B.RMSQ_FP4_BLOCK16 else H
    sshape = {B.RMSQ_FP8_STATIC: None, B.RMSQ_FP8_TOKEN: (T,), B.RMSQ_FP8_GROUP: (T, H // max(G, 1)),
              B.RMSQ_FP4_BLOCK16: (T, H // 16)}[mode]
    sdt = torch.uint8 if mode == B.RMSQ_FP4_BLOCK16 else torch.float32

    def outputs():
        return (torch.empty((T, qcols), dtype=torch.uint8, device="cuda"),
                None if sshape is None else torch.empty(sshape, dtype=sdt, device="cuda"),
                torch.empty_like(r))

    def launch(q, s, ro, stream=None):
        B.rmsq_fused(x, r, w, 1e-6, mode, sc, q, s, ro, group_size=G, stream=stream)

    ref = outputs()
    launch(*ref)
    torch.cuda.synchronize()

    gq = outputs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        launch(*gq, stream=torch.cuda.current_stream())
    other = outputs()
    for rep in range(4):
        print(f"[graph] mode={mode} replay={rep}", flush=True)
        for t in gq:
            if t is not None:
                t.fill_(0x5A if t.dtype == torch.uint8 else 7)
        launch(*other)            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(gq, ref):
            if a is not None:
                assert torch.equal(a, b), f"replay {rep} differs from the eager launch"
        for a, b in zip(other, ref):
            if a is not None:
                assert torch.equal(a, b)
