"""Every entry point inside a captured HIP graph: every replay equals the eager launch.

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


def _replay_check(launch_into, make_outputs, what, inplace_source=None):
    """Capture launch_into(outputs) once; replay it 4 times with eager launches of the same op,
    output wipes and synchronizations in between; every replay must equal the eager result.
    inplace_source: for an in-place op, the input to restore before each launch."""
    ref = make_outputs()
    launch_into(ref)
    torch.cuda.synchronize()
    gq = make_outputs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        launch_into(gq, stream=torch.cuda.current_stream())
    other = make_outputs()
    for rep in range(4):
        print(f"[graph] {what} replay={rep}", flush=True)
        for t in gq:
            t.fill_(0x5A if t.dtype == torch.uint8 else 7)
        if inplace_source is not None:
            gq[0].copy_(inplace_source)
            other[0].copy_(inplace_source)
        launch_into(other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(gq, ref):
            assert torch.equal(a, b), f"{what}: replay {rep} differs from the eager launch"
        for a, b in zip(other, ref):
            assert torch.equal(a, b)


@pytest.mark.parametrize("mode,G", [(B.RMSQ_FP8_STATIC, 0), (B.RMSQ_FP8_GROUP, 64),
                                    (B.RMSQ_FP4_BLOCK16, 16)])
def test_graph_silu_mul_quant(mode, G):
    T, I = 40, 2048
    g = torch.Generator().manual_seed(78)
    x = torch.randn((T, 2 * I), generator=g).to(torch.bfloat16).cuda()
    sc = torch.tensor([0.02 if mode == B.RMSQ_FP8_STATIC else 300.0], device="cuda") \
        if mode in (B.RMSQ_FP8_STATIC, B.RMSQ_FP4_BLOCK16) else None
    qcols = I // 2 if mode == B.RMSQ_FP4_BLOCK16 else I
    sshape = {B.RMSQ_FP8_STATIC: None, B.RMSQ_FP8_GROUP: (T, I // max(G, 1)),
              B.RMSQ_FP4_BLOCK16: (T, I // 16)}[mode]
    sdt = torch.uint8 if mode == B.RMSQ_FP4_BLOCK16 else torch.float32

    def outs():
        o = [torch.empty((T, qcols), dtype=torch.uint8, device="cuda")]
        if sshape is not None:
            o.append(torch.empty(sshape, dtype=sdt, device="cuda"))
        return o

    def launch(o, stream=None):
        B.rmsq_silu_mul_quant(x, mode, sc, o[0], o[1] if len(o) > 1 else None, group_size=G,
                              stream=stream)

    _replay_check(launch, outs, f"silu_mul mode={mode}")


def test_graph_rms_norm_pad():
    T, H, ld = 33, 2880, 3072
    g = torch.Generator().manual_seed(79)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda()
    r = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda()
    w = (torch.rand((H,), generator=g) + 0.5).to(torch.bfloat16).cuda()

    def outs():
        return [torch.empty((T, ld), dtype=torch.bfloat16, device="cuda"), torch.empty_like(r)]

    def launch(o, stream=None):
        B.rmsq_rms_norm_pad(x, r, w, 1e-5, o[0], o[1], stream=stream)

    _replay_check(launch, outs, "rms_norm_pad")


def test_graph_qk_norm_rope():
    """In place: each replay first gets the original qkv back (a copy kernel in the eager
    stream), then the captured launch rewrites it."""
    T, hq, hkv, D = 24, 32, 8, 128
    g = torch.Generator().manual_seed(80)
    qkv0 = torch.randn((T, (hq + 2 * hkv) * D), generator=g).to(torch.bfloat16).cuda()
    qw = (torch.rand((D,), generator=g) + 0.5).to(torch.bfloat16).cuda()
    kw = (torch.rand((D,), generator=g) + 0.5).to(torch.bfloat16).cuda()
    th = torch.arange(64, dtype=torch.float64)[:, None] * \
        (1e6 ** (-2.0 * torch.arange(D // 2, dtype=torch.float64) / D))[None, :]
    cache = torch.cat([th.cos(), th.sin()], dim=1).float().cuda()
    pos = torch.randint(0, 64, (T,), generator=g).cuda()

    def outs():
        return [qkv0.clone()]

    def launch(o, stream=None):
        B.rmsq_qk_norm_rope(o[0], qw, kw, cache, pos, 1e-6, hq, hkv, D, True, stream=stream)

    _replay_check(launch, outs, "qk_norm_rope", inplace_source=qkv0)


@pytest.mark.parametrize("T,H,launch", [(40, 2048, None), (4096, 2048, None),
                                         (8200, 64, (64, 1, 1))])
def test_graph_fp4_dynamic(T, H, launch):
    """Batch-scale FP4 in one graph: two launches (row pass; block quantization, whose first
    workgroup derives the global scale and hands it to the others through global_scale), or with
    a caller's one-row workgroups over 8200 rows three (the reduction between them).  Each replay
    starts from a wiped, non-zero global_scale, which the row pass must clear."""
    lb = None if launch is None else B.rmsq_launch(*launch, 0)
    g = torch.Generator().manual_seed(81)
    x = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda()
    r = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda()
    w = (torch.rand((H,), generator=g) + 0.5).to(torch.bfloat16).cuda()

    def outs():
        return [torch.empty((T, H // 2), dtype=torch.uint8, device="cuda"),
                torch.empty((T, H // 16), dtype=torch.uint8, device="cuda"),
                torch.empty_like(r), torch.empty((1,), dtype=torch.float32, device="cuda")]

    def run(o, stream=None):
        B.rmsq_fused_fp4_dynamic(x, r, w, 1e-6, o[0], o[1], o[2], o[3], stream=stream, launch=lb)

    _replay_check(run, outs, f"fp4_dynamic T={T} H={H} launch={launch}")
