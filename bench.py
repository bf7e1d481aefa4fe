"""Benchmark of the fused add + RMSNorm + quantization kernel family on one MI355X.

Default workload: fused residual add + RMSNorm -> FP8 static per-tensor quant, 4096 tokens x
hidden 4096, bf16 inputs ~N(0,1), weight ~U(0.5,1.5), eps 1e-5, static scale from a fixed
512x4096 warm-up batch.  One step = one launch of the fused kernel over the whole batch
(residual add, sum of squares, normalize, scale, quantize, stores).

Inputs are resident in HBM before timing starts.  Launches rotate over several buffer sets
whose total footprint is well above the 256 MB last-level cache, so each launch reads cold
data.  Prints ONE JSON line:
  value          algorithmic GB/s over the timed region (bytes each launch must move)
  roofline       HBM roofline of the fused kernel: algorithmic bytes / the kernel's average
                 duration (HIP events stamped by each dispatch itself on the launch stream),
                 against 8 TB/s; traffic = HBM
                 bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE (scaled by a plain
                 copy's counters) when the committed counters match the current kernel source
  cpu_baseline   the CPU oracle on a bounded sample of the same workload, one core

Other workloads (--workload w0..w8; w5 is SiLU+Mul -> quant with --quant
static|token|group|fp4, w6 add+RMSNorm -> padded bf16, w7 QK-norm + RoPE, w8 add+RMSNorm -> FP4
with the global scale taken from the batch, two launches timed as one step) and forced launch
shapes (--launch tpr,vpt,rpb[,options]; for w7 --launch heads_per_block,heads_per_lane) are
for exploration;
only one GPU is supported (--gpus above 1 exits with a message).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FOOTPRINT_BYTES = 1536 << 20   # rotating buffer sets: at least 6x the 256 MB MALL
MODE_NAMES = {0: "fp8_static", 1: "fp8_per_token", 2: "fp8_per_group", 3: "fp4_block16",
              4: "bf16_padded", 5: "bf16_qk_norm_rope", 6: "fp4_block16_batch_scale"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash():
    """Identity of what the HBM counters were taken on: every source unit and kernel header of
    librmsq (kernels, instantiation tables, launch heuristics) and its hipcc flags."""
    from rmsnorm_quantization_amd import build as hb

    h = hashlib.sha256()
    for p in sorted(hb.SRC + hb.KERNEL_SOURCES):
        h.update(open(p, "rb").read())
    h.update(" ".join(a for a in hb.command("lib.so")[1:] if not a.startswith("/")).encode())
    return h.hexdigest()[:16]


def workload_spec(args):
    from rmsnorm_quantization_amd import binding as B
    from rmsnorm_quantization_amd import synth

    wl = synth.WORKLOADS[int(args.workload[1:])]
    T = args.tokens or max(wl.tokens)
    H = args.hidden or (7168 if wl.index == 3 else wl.hidden[0])
    if wl.kind == "rope":
        mode = 5  # not a quantization scheme: normalized and rotated heads, bf16 in place
    elif wl.kind == "pad":
        mode = 4  # not a quantization scheme: the normalized row as padded bf16
    elif wl.kind == "fp4dyn":
        mode = 6  # FP4 block-16 whose global scale the library derives from the batch
    elif wl.kind == "act":
        mode = {"static": B.RMSQ_FP8_STATIC, "token": B.RMSQ_FP8_TOKEN,
                "group": B.RMSQ_FP8_GROUP, "fp4": B.RMSQ_FP4_BLOCK16}[args.quant]
    else:
        mode = {0: B.RMSQ_FP8_STATIC, 1: B.RMSQ_FP8_STATIC, 2: B.RMSQ_FP8_TOKEN,
                3: B.RMSQ_FP8_GROUP, 4: B.RMSQ_FP4_BLOCK16}[wl.index]
    G = {2: args.group, 3: 16}.get(mode, 0)
    flags = 0
    if mode == B.RMSQ_FP8_GROUP:
        for f in (args.flags or "").split(","):
            flags |= {"": 0, "col": B.RMSQ_SCALE_COLMAJOR, "e8m0": B.RMSQ_SCALE_E8M0,
                      "e8m0u8": B.RMSQ_SCALE_E8M0_U8}[f]
    return wl, T, H, mode, G, flags


def algorithmic_bytes(mode, T, H, G, flags, residual, kind="norm"):
    """Bytes one launch must move: every input read once, every output written once, the
    weight once per launch.  For SiLU+Mul (kind "act") H is I and the input is [T, 2I] bf16."""
    if kind == "pad":  # H here is the padded row length of the bf16 output; see gpu_leg
        raise ValueError("use pad_bytes")
    if kind == "act":
        rd = 4 * T * H + (4 if mode in (0, 3) else 0)
    else:
        rd = 2 * T * H + (2 * T * H if residual else 0) + 2 * H + (4 if mode in (0, 3) else 0)
    wr = (2 * T * H if residual else 0) + (T * H // 2 if mode == 3 else T * H)
    if mode == 1:
        wr += 4 * T
    elif mode == 2:
        wr += T * (H // G) * (1 if flags & 4 else 4)
    elif mode == 3:
        wr += T * (H // 16)
    return rd, wr


def pad_bytes(T, H, ld, residual=True):
    """Residual add + RMSNorm -> padded bf16: read x (and the residual) and the weight once,
    write the new residual and the padded output rows."""
    rd = 2 * T * H + (2 * T * H if residual else 0) + 2 * H
    wr = (2 * T * H if residual else 0) + 2 * T * ld
    return rd, wr


def rope_bytes(T, hq, hkv, D):
    """QK-norm + RoPE: read and rewrite the q and k heads once, read both weights once per
    launch, each token's position and its cos/sin cache row (D f32) once."""
    qk = 2 * T * (hq + hkv) * D
    return qk + 2 * 2 * D + 8 * T + 4 * D * T, qk


def fp4dyn_bytes(T, H, residual=True):
    """FP4 with the global scale from the batch: the row pass reads x (and the residual) and the
    weight and writes the new residual and the row maxima (one per workgroup of rows, counted
    here as T, an upper bound worth 0.05% of the total); their reduction reads them and writes
    gs; the block pass reads the normalized input again (the new residual, or x) and the weight
    and writes codes and block scales.  The second read of the input (2H per token) is
    inherent: gs depends on every row."""
    rd = 2 * T * H + (2 * T * H if residual else 0) + 2 * H + 4 * T + 2 * T * H + 2 * H + 4
    wr = (2 * T * H if residual else 0) + 4 * T + 4 + T * H // 2 + T * (H // 16)
    return rd, wr


def fp4dyn_leg(args, wl, T, H):
    """GPU timing of rmsq_fused_fp4_dynamic (two launches per step), structured like gpu_leg;
    the per-step duration runs from the first launch's dispatch to the last one's end."""
    import torch

    from rmsnorm_quantization_amd import binding as B
    from rmsnorm_quantization_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x, r, w = synth.make_inputs(wl.index, T, H)
    rd, wr = fp4dyn_bytes(T, H, True)
    nsets = max(2, math.ceil(FOOTPRINT_BYTES / (rd + wr)))
    xd, rdv, wd = x.to(dev), r.to(dev), w.to(dev).contiguous()
    sets = []
    for _ in range(nsets):
        s = {"x": xd.clone(), "r": rdv.clone(), "ro": torch.empty_like(xd),
             "q": torch.empty((T, H // 2), dtype=torch.uint8, device=dev),
             "s": torch.empty((T, H // 16), dtype=torch.uint8, device=dev),
             "g": torch.empty((1,), dtype=torch.float32, device=dev)}
        if args.inplace:
            s["ro"] = s["r"]
        sets.append(s)
    launch = None  # the library's own default shapes for both launches
    if args.launch:
        vals = [int(v) for v in args.launch.split(",")]
        launch = B.rmsq_launch(*(vals + [0] * (4 - len(vals))))
    import ctypes

    lib = B.lib()
    lref = None if launch is None else ctypes.byref(launch)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    status = []
    argsets = [(s_["x"].data_ptr(), s_["r"].data_ptr(), wd.data_ptr(), float(wl.eps),
                s_["q"].data_ptr(), s_["s"].data_ptr(), s_["ro"].data_ptr(), s_["g"].data_ptr(),
                T, H, 0) for s_ in sets]

    def launch_on(a, e0, e1, hs):
        st = lib.rmsq_fused_fp4_dynamic_ex(*a, lref, e0, e1, hs)
        if st:
            status.append(st)

    for i in range(args.warmup):
        launch_on(argsets[i % nsets], None, None, sh)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        launch_on(argsets[i % nsets], None, None, sh)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    ms_per_step_graph = None
    if args.graph:
        g_ = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_, stream=torch.cuda.Stream()):
            hs = torch.cuda.current_stream().cuda_stream
            for i in range(args.steps):
                launch_on(argsets[i % nsets], None, None, hs)
        g_.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        g_.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms_per_step_graph = t0.elapsed_time(t1) / args.steps
        del g_
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a_, b_ in evs:
        a_.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()
    for i in range(args.warmup):  # lead-in: the timed dispatches do not start from an idle GPU
        launch_on(argsets[i % nsets], None, None, sh)
    for i in range(args.steps):
        launch_on(argsets[i % nsets], evs[i][0].cuda_event, evs[i][1].cuda_event, sh)
    torch.cuda.synchronize()
    if status:
        raise RuntimeError(f"rmsq_fused_fp4_dynamic failed: {B.rmsq_status_string(status[0])}")
    per = sorted(a.elapsed_time(b) for a, b in evs)
    copy_gbs = copy_ceiling(dev, stream)
    return {"ms_per_step": ms_per_step, "ms_per_step_graph": ms_per_step_graph,
            "avg_launch_ms": sum(per) / len(per), "median_launch_ms": per[len(per) // 2],
            "p10_launch_ms": per[len(per) // 10], "p90_launch_ms": per[(9 * len(per)) // 10],
            "bytes": rd + wr, "read": rd, "write": wr, "sets": nsets,
            "launch": None if launch is None else launch.as_tuple(), "copy_gbs": copy_gbs,
            "device": torch.cuda.get_device_name(dev)}


def rope_cache(max_pos, D, base):
    """The caller-built [max_pos, D] f32 cos | sin table (binary64, rounded once)."""
    import torch

    inv = base ** (-2.0 * torch.arange(D // 2, dtype=torch.float64) / D)
    th = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cat([th.cos(), th.sin()], dim=1).float()


def rope_leg(args, wl, T, D):
    """GPU timing of QK-norm + RoPE, structured like gpu_leg."""
    import ctypes

    import torch

    from rmsnorm_quantization_amd import binding as B
    from rmsnorm_quantization_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hq, hkv = wl.heads
    qkv, qw, kw, pos = synth.make_rope_inputs(wl.index, T)
    cache = rope_cache(wl.max_position, D, wl.rope_base).to(dev)
    rd, wr = rope_bytes(T, hq, hkv, D)
    qkv_bytes = qkv.numel() * 2
    nsets = max(2, math.ceil(FOOTPRINT_BYTES / qkv_bytes))
    qkv_d = qkv.to(dev)
    sets = [qkv_d.clone() for _ in range(nsets)]
    qw_d, kw_d, pos_d = qw.to(dev), kw.to(dev), pos.to(dev)
    if args.launch:
        hpb, hpl = (int(v) for v in args.launch.split(","))
    else:
        hpb, hpl, _ = B.rmsq_qk_norm_rope_query_launch(T, hq, hkv, D)
    lib = B.lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    status = []
    argsets = [(q.data_ptr(), qw_d.data_ptr(), kw_d.data_ptr(), cache.data_ptr(),
                pos_d.data_ptr(), float(wl.eps), T, hq, hkv, D, wl.max_position, 1, 0, hpb, hpl)
               for q in sets]

    def launch(a, e0, e1, hs):
        st = lib.rmsq_qk_norm_rope_ex(*a, e0, e1, hs)
        if st:
            status.append(st)

    for i in range(args.warmup):
        launch(argsets[i % nsets], None, None, sh)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        launch(argsets[i % nsets], None, None, sh)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    ms_per_step_graph = None
    if args.graph:
        g_ = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_, stream=torch.cuda.Stream()):
            hs = torch.cuda.current_stream().cuda_stream
            for i in range(args.steps):
                launch(argsets[i % nsets], None, None, hs)
        g_.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        g_.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms_per_step_graph = t0.elapsed_time(t1) / args.steps
        del g_
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a_, b_ in evs:
        a_.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()
    for i in range(args.warmup):  # lead-in: the timed dispatches do not start from an idle GPU
        launch(argsets[i % nsets], None, None, sh)
    for i in range(args.steps):
        launch(argsets[i % nsets], evs[i][0].cuda_event, evs[i][1].cuda_event, sh)
    torch.cuda.synchronize()
    if status:
        raise RuntimeError(f"rmsq_qk_norm_rope failed: {B.rmsq_status_string(status[0])}")
    per = sorted(a.elapsed_time(b) for a, b in evs)
    copy_gbs = copy_ceiling(dev, stream)
    return {"ms_per_step": ms_per_step, "ms_per_step_graph": ms_per_step_graph,
            "avg_launch_ms": sum(per) / len(per), "median_launch_ms": per[len(per) // 2],
            "p10_launch_ms": per[len(per) // 10], "p90_launch_ms": per[(9 * len(per)) // 10],
            "bytes": rd + wr, "read": rd, "write": wr, "sets": nsets, "launch": (hpb, hpl),
            "copy_gbs": copy_gbs, "device": torch.cuda.get_device_name(dev)}


def _probe_lib():
    import ctypes

    from rmsnorm_quantization_amd import build as hb

    if not os.path.exists(hb.PROBE_LIB):
        hb.build_probe_library()
    L = ctypes.CDLL(hb.PROBE_LIB)
    p = ctypes.c_void_p
    i32 = ctypes.c_int
    L.rmsq_probe_stream.argtypes = [p, p, p, p, p, ctypes.c_int64, ctypes.c_int64, i32, i32, i32,
                                    i32, i32, p, p, p]
    L.rmsq_probe_stream.restype = ctypes.c_int
    return L


def copy_ceiling(dev, stream):
    """The practical HBM ceiling for streaming: GB/s of a plain 128-bit copy kernel (the probe
    library with one input and one output) over two 256 MiB buffer pairs, 20 launches each
    stamped by its own dispatch; and, for context, torch's own device copy."""
    import torch

    L = _probe_lib()
    H = 4096
    rows = (256 << 20) // (2 * H)
    pairs = [(torch.empty((rows, H), dtype=torch.bfloat16, device=dev),
              torch.empty((rows, H), dtype=torch.bfloat16, device=dev)) for _ in range(2)]
    sh = stream.cuda_stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(20)]
    for a_, b_ in evs:
        a_.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()
    for i in range(4):  # lead-in, no host synchronization before the timed copies
        src, dst = pairs[i % 2]
        L.rmsq_probe_stream(src.data_ptr(), None, dst.data_ptr(), None, None, rows, H, 0, 0, 0,
                            256, 2, None, None, sh)
    for i, (a_, b_) in enumerate(evs):
        src, dst = pairs[i % 2]
        st = L.rmsq_probe_stream(src.data_ptr(), None, dst.data_ptr(), None, None, rows, H, 0,
                                 0, 0, 256, 2, a_.cuda_event, b_.cuda_event, sh)
        if st:
            raise RuntimeError(f"rmsq_probe_stream (copy) failed ({st})")
    torch.cuda.synchronize()
    per = sorted(a_.elapsed_time(b_) for a_, b_ in evs)
    probe_copy = 2 * rows * H * 2 / (per[len(per) // 2] * 1e-3) / 1e9

    copy_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    copy_dst = torch.empty_like(copy_src)
    for _ in range(3):
        copy_dst.copy_(copy_src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(10):
        copy_dst.copy_(copy_src)
    c1.record(stream)
    torch.cuda.synchronize()
    torch_copy = 2 * copy_src.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    return {"copy_GBs": probe_copy, "torch_copy_GBs": torch_copy}


def scale_layout(mode, T, H, G, flags):
    import torch

    if mode == 0:
        return None, None
    if mode == 1:
        return (T,), torch.float32
    if mode == 2:
        dt = torch.uint8 if flags & 4 else torch.float32
        return ((H // G, T) if flags & 1 else (T, H // G)), dt
    return (T, H // 16), torch.uint8


def gpu_leg(args, wl, T, H, mode, G, flags, with_copy=True):
    import torch

    from rmsnorm_quantization_amd import binding as B
    from rmsnorm_quantization_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    act = wl.kind == "act"
    pad = wl.kind == "pad"
    ld = -(-H // wl.pad_multiple) * wl.pad_multiple if pad else 0
    if act:
        x, r, w = synth.make_act_inputs(wl.index, T, H), None, torch.zeros(8, dtype=torch.bfloat16)
    else:
        x, r, w = synth.make_inputs(wl.index, T, H)
    residual = r is not None
    if pad:
        rd, wr = pad_bytes(T, H, ld, residual)
    else:
        rd, wr = algorithmic_bytes(mode, T, H, G, flags, residual, wl.kind)
    set_bytes = rd + wr
    # enough sets that the footprint dwarfs the last-level cache, and never more than the
    # launches that use them (every launch of a timed pass reads its own set)
    nsets = max(2, min(math.ceil(FOOTPRINT_BYTES / set_bytes), args.steps + args.warmup))
    xd, rdv, wd = x.to(dev), (r.to(dev) if residual else None), w.to(dev)
    sshape, sdt = scale_layout(mode, T, H, G, flags) if not pad else (None, None)
    qcols = H // 2 if mode == 3 else H
    sets = []
    for _ in range(nsets):
        s = {"x": xd.clone(), "r": rdv.clone() if residual else None,
             "ro": torch.empty_like(xd) if residual else None,
             "q": (torch.empty((T, ld), dtype=torch.bfloat16, device=dev) if pad else
                   torch.empty((T, qcols), dtype=torch.uint8, device=dev)),
             "s": torch.empty(sshape, dtype=sdt, device=dev) if sshape else None}
        if residual and args.inplace:
            s["ro"] = s["r"]  # the residual is updated in place, as the fused-add op does
        sets.append(s)
    wd = wd.contiguous()

    # per-tensor input scale: the static scale from the workload's warm-up batch (max|y|/448,
    # computed on the GPU with the per-token mode), the FP4 global scale 448*6/max|y|
    scale_in = None
    if pad:
        pass
    elif act and mode in (0, 3):
        # static scale: max|a|/448 of the warm-up batch; FP4 global scale 448*6/max|a| of the
        # batch itself -- both from the GPU's per-token launch
        src = synth.make_act_warmup(wl.index, H).to(dev) if mode == 0 else xd
        q = torch.empty((src.shape[0], H), dtype=torch.uint8, device=dev)
        st = torch.empty((src.shape[0],), dtype=torch.float32, device=dev)
        B.rmsq_silu_mul_quant(src, B.RMSQ_FP8_TOKEN, None, q, st)
        amax = float(st.max()) * 448.0
        scale_in = torch.tensor([amax / 448.0 if mode == 0 else 448.0 * 6.0 / amax],
                                dtype=torch.float32, device=dev)
    elif mode == 0:
        if wl.static_scale is not None:
            sval = wl.static_scale
        else:
            xw, rw = synth.make_warmup(wl.index, H)
            xw, rw = xw.to(dev), rw.to(dev)
            q = torch.empty(xw.shape, dtype=torch.uint8, device=dev)
            st = torch.empty((xw.shape[0],), dtype=torch.float32, device=dev)
            B.rmsq_fused(xw, rw, wd, wl.eps, B.RMSQ_FP8_TOKEN, None, q, st, torch.empty_like(xw))
            sval = float(st.max())
        scale_in = torch.tensor([sval], dtype=torch.float32, device=dev)
    elif mode == 3:
        q = torch.empty((T, H), dtype=torch.uint8, device=dev)
        st = torch.empty((T,), dtype=torch.float32, device=dev)
        B.rmsq_fused(xd, rdv, wd, wl.eps, B.RMSQ_FP8_TOKEN, None, q, st,
                     torch.empty_like(xd) if residual else None)
        amax = float(st.max()) * 448.0
        scale_in = torch.tensor([448.0 * 6.0 / amax], dtype=torch.float32, device=dev)

    launch = None
    if args.launch:
        vals = [int(v) for v in args.launch.split(",")]
        launch = B.rmsq_launch(*(vals + [0] * (4 - len(vals))))
    if launch:
        shape = launch.as_tuple()
    elif pad:
        shape = B.rmsq_rms_norm_pad_query_launch(T, H, ld)[0].as_tuple()
    elif act:
        shape = B.rmsq_silu_mul_query_launch(mode, T, H, 16 if mode == 3 else G)[0].as_tuple()
    else:
        shape = B.rmsq_query_launch(mode, T, H, G, flags)[0].as_tuple()
    if act and mode == 3:
        G = 16
    stream = torch.cuda.current_stream()

    # argument tuples marshalled once, so the launch loop is one C call per step
    import ctypes

    lib = B.lib()
    ptr = (lambda t: None if t is None else t.data_ptr())
    sh = stream.cuda_stream
    lref = ctypes.byref(launch) if launch is not None else None
    status = []
    if pad:
        argsets = [(ptr(s["x"]), ptr(s["r"]), wd.data_ptr(), float(wl.eps), ptr(s["q"]),
                    ptr(s["ro"]), T, H, ld, 0) for s in sets]

        def launch_on(a, hs):
            return lib.rmsq_rms_norm_pad_ex(*a, lref, None, None, hs)

        def launch_timed(a, e0, e1, hs):
            return lib.rmsq_rms_norm_pad_ex(*a, lref, e0, e1, hs)
    elif act:
        argsets = [(ptr(s["x"]), mode, ptr(scale_in), ptr(s["q"]), ptr(s["s"]), T, H, G, flags, 0)
                   for s in sets]

        def launch_on(a, hs):
            return lib.rmsq_silu_mul_quant_ex(*a, lref, None, None, hs)

        def launch_timed(a, e0, e1, hs):
            return lib.rmsq_silu_mul_quant_ex(*a, lref, e0, e1, hs)
    else:
        argsets = [(ptr(s["x"]), ptr(s["r"]), wd.data_ptr(), float(wl.eps), mode, ptr(scale_in),
                    ptr(s["q"]), ptr(s["s"]), ptr(s["ro"]), T, H, G, flags, 0) for s in sets]

        def launch_on(a, hs):
            return lib.rmsq_fused_with_launch(*a, lref, hs) if lref else lib.rmsq_fused(*a, hs)

        def launch_timed(a, e0, e1, hs):
            return lib.rmsq_fused_timed(*a, lref, e0, e1, hs)

    def step(i):
        st = launch_on(argsets[i % nsets], sh)
        if st:
            status.append(st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K back-to-back launches bracketed by one event pair
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # the same K launches captured once as a HIP graph and replayed: no host work and no
    # per-launch queue overhead between the kernels (how a serving loop would issue them)
    ms_per_step_graph = None
    if args.graph:
        g_ = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_, stream=torch.cuda.Stream()):
            hs = torch.cuda.current_stream().cuda_stream
            for i in range(args.steps):
                st = launch_on(argsets[i % nsets], hs)
                if st:
                    status.append(st)
        g_.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        g_.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms_per_step_graph = t0.elapsed_time(t1) / args.steps
        del g_

    # per-launch kernel durations: each launch carries its own event pair, stamped by the
    # dispatch itself at kernel start and end (rmsq_fused_timed)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a_, b_ in evs:  # create the underlying HIP events
        a_.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()
    # lead-in, untimed and with no host synchronization before the timed launches: the first
    # dispatches after an idle gap run slower (about 1.6x at the default workload), which is
    # the measurement's own synchronization, not the kernel
    for i in range(args.warmup):
        step(i)
    for i in range(args.steps):
        st = launch_timed(argsets[i % nsets], evs[i][0].cuda_event, evs[i][1].cuda_event, sh)
        if st:
            status.append(st)
    torch.cuda.synchronize()
    if status:
        raise RuntimeError(f"rmsq_fused failed: {B.rmsq_status_string(status[0])}")
    per = sorted(a.elapsed_time(b) for a, b in evs)
    avg_launch_ms = sum(per) / len(per)
    med_launch_ms = per[len(per) // 2]

    # the memory-only probe with the same traffic and launch shape (norm workloads, one row
    # per workgroup, exact fit): the practical ceiling for this exact access pattern
    ceiling = None
    if wl.kind == "norm" and shape[2] == 1 and shape[0] * shape[1] * 8 == H:
        ceiling = probe_leg(args, sets, T, H, mode, shape, stream, evs, G=G, flags=flags)

    # a plain device copy, for context (practical HBM ceiling)
    copy_gbs = copy_ceiling(dev, stream) if with_copy else None

    return {"ms_per_step": ms_per_step, "ms_per_step_graph": ms_per_step_graph,
            "avg_launch_ms": avg_launch_ms,
            "median_launch_ms": med_launch_ms, "p10_launch_ms": per[len(per) // 10],
            "p90_launch_ms": per[(9 * len(per)) // 10], "bytes": rd + wr, "read": rd, "write": wr,
            "sets": nsets, "launch": shape, "copy_gbs": copy_gbs, "ceiling": ceiling,
            "device": torch.cuda.get_device_name(dev)}


# The five configurations of the fused add + RMSNorm + quant family, each timed in the default
# run: (label, workload, tokens, hidden, group, scale flags).  The 1024-token shapes are the
# smallest batches the >= 80%-of-peak target is stated for (every wave of the launch resident at
# once).
CONFIG_LEGS = [
    ("rmsnorm_fp8_static 16 x 4096 (latency)", "w0", 16, 4096, 128, ""),
    ("add_rmsnorm_fp8_static 1024 x 4096", "w1", 1024, 4096, 128, ""),
    ("add_rmsnorm_fp8_static 4096 x 4096", "w1", 4096, 4096, 128, ""),
    ("add_rmsnorm_fp8_static 16384 x 4096", "w1", 16384, 4096, 128, ""),
    ("add_rmsnorm_fp8_per_token 8192 x 8192", "w2", 8192, 8192, 128, ""),
    ("add_rmsnorm_fp8_per_group G128 1024 x 5120", "w3", 1024, 5120, 128, ""),
    ("add_rmsnorm_fp8_per_group G128 1024 x 7168", "w3", 1024, 7168, 128, ""),
    ("add_rmsnorm_fp8_per_group G128 16384 x 7168", "w3", 16384, 7168, 128, ""),
    ("add_rmsnorm_fp4_block16 4096 x 2048", "w4", 4096, 2048, 128, ""),
]


CONFIG_STEPS = 200  # dispatch-stamped launches per configuration leg (at least)


def leg_summary(label, wl, T, H, mode, G, flags, g):
    """One configuration's line of the configs list: kernel time from dispatch-stamped events,
    algorithmic GB/s and fraction of 8 TB/s, graph-replay latency per launch, the memory-only
    probe's time on the same buffers and launch shape, HBM traffic when profiled."""
    kern_us = g["avg_launch_ms"] * 1e3
    gbs = g["bytes"] / (kern_us * 1e-6) / 1e9
    step_ms = g["ms_per_step_graph"] or g["ms_per_step"]
    key = f"w{wl.index}_T{T}_H{H}_{MODE_NAMES[mode]}_G{G}_f{flags}"
    tr = load_traffic(key)
    c = g.get("ceiling")
    return {
        "config": label, "workload": wl.name, "tokens": T, "hidden": H,
        "mode": MODE_NAMES[mode], "group_size": G, "flags": flags,
        "launch": list(g["launch"]), "bytes": g["bytes"],
        "kernel_us": {"mean": round(kern_us, 3), "median": round(g["median_launch_ms"] * 1e3, 3),
                      "p10": round(g["p10_launch_ms"] * 1e3, 3),
                      "p90": round(g["p90_launch_ms"] * 1e3, 3)},
        "GBs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(T / (kern_us * 1e-6), 1),
        "latency_us_per_launch": round(step_ms * 1e3, 3),
        "probe": None if not c else {
            "kernel_us": round(c["kernel_us"], 3), "median_us": round(c["median_us"], 3),
            "probe_time_over_kernel_time": round(c["kernel_us"] / kern_us, 4),
            "median_ratio": round(c["median_us"] / (g["median_launch_ms"] * 1e3), 4)},
        "traffic": None if tr is None else tr["bytes_per_launch"],
    }


def configs_leg(args, main):
    """Time every entry of CONFIG_LEGS (the main line's own configuration reuses its numbers)."""
    import torch

    out = []
    for label, w, T, H, G, fl in CONFIG_LEGS:
        a = argparse.Namespace(**vars(args))
        a.workload, a.tokens, a.hidden, a.group, a.flags, a.launch = w, T, H, G, fl, ""
        a.steps = max(args.steps, CONFIG_STEPS)  # a few ms each: enough launches for a median
        wl, T, H, mode, G, flags = workload_spec(a)
        if main is not None and (wl.index, T, H, mode, G, flags) == main[0] and \
                args.steps >= CONFIG_STEPS:
            g = main[1]
        else:
            g = gpu_leg(a, wl, T, H, mode, G, flags, with_copy=False)
            torch.cuda.empty_cache()
        out.append(leg_summary(label, wl, T, H, mode, G, flags, g))
        print(f"bench: {label}: {out[-1]['kernel_us']['mean']} us, "
              f"{out[-1]['frac_of_peak']:.3f} of peak", file=sys.stderr, flush=True)
    return out


def probe_scale_stream(mode, H, G, flags):
    """The probe's scale-like stream for a scheme: (shift, bytes per element) -- one f32 per row
    (per-token), per group of G/8 chunks (f32, or a byte for E8M0 bytes), a byte per two chunks
    (FP4 block-16) -- or None (static: no scales).  Column-major group scales are stored
    row-major by the probe (the same bytes, another pattern)."""
    if mode == 1:
        return (-1, 4)
    if mode == 2:
        return ((G // 8).bit_length() - 1, 1 if flags & 4 else 4)
    if mode == 3:
        return (1, 1)
    return None


def probe_leg(args, sets, T, H, mode, shape, stream, evs, G=0, flags=0):
    """Time librmsq_probe.so's memory-only kernel over the same buffer sets: it reads x and the
    residual and writes the new residual, codes-sized and scales-sized outputs in the fused
    kernel's layout, with no arithmetic.  Returns its mean dispatch-stamped duration and bytes."""
    L = _probe_lib()
    out1 = 4 if mode == 3 else 8
    sc = probe_scale_stream(mode, H, G, flags)
    shift, sbytes = sc if sc else (0, 0)
    ptr = (lambda t: None if t is None else t.data_ptr())
    sh = stream.cuda_stream
    argsets = [(ptr(s_["x"]), ptr(s_["r"]), ptr(s_["ro"]), ptr(s_["q"]),
                ptr(s_["s"]) if sc else None, T, H, out1, shift, sbytes, shape[0], shape[1])
               for s_ in sets]
    import torch

    torch.cuda.synchronize()
    for i in range(args.warmup):  # lead-in, as for the fused kernel
        st = L.rmsq_probe_stream(*argsets[i % len(sets)], None, None, sh)
        if st:
            raise RuntimeError(f"rmsq_probe_stream failed ({st})")
    for i in range(args.steps):
        st = L.rmsq_probe_stream(*argsets[i % len(sets)], evs[i][0].cuda_event,
                                 evs[i][1].cuda_event, sh)
        if st:
            raise RuntimeError(f"rmsq_probe_stream failed ({st})")
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    nbytes = T * (2 * H + (2 * H if sets[0]["r"] is not None else 0)
                  + (2 * H if sets[0]["ro"] is not None else 0) + H * out1 // 8)
    if sc:
        nbytes += T * sbytes * (1 if shift < 0 else (H // 8) >> shift)
    return {"kernel_us": sum(per) / len(per) * 1e3, "median_us": per[len(per) // 2] * 1e3,
            "bytes": nbytes}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def host_threads():
    """Threads the CPU leg may use: the CPUs this process may run on, at most 16 (one GPU's
    share of a host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_leg(wl, T, H, mode, G, flags, budget_s=12.0):
    """The oracle as it stands on whole rows of the same workload: first one thread, in chunks
    of 64 rows until about budget_s seconds of CPU work (or the whole batch); then the same rows
    split over host_threads() threads (the oracle is C called through ctypes, which releases the
    GIL).  GB/s with the same algorithmic byte count per row as the GPU leg."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle as O
    from rmsnorm_quantization_amd import synth

    if wl.kind == "rope":
        hq, hkv = wl.heads
        qkv, qw, kw, pos = synth.make_rope_inputs(wl.index, T)
        xb, qwb, kwb, posn = synth.bits(qkv), synth.bits(qw), synth.bits(kw), pos.numpy()
        cache = O.rope_cache(wl.max_position, H, wl.rope_base)

        def run_rows(lo, hi):
            O.qk_norm_rope(xb[lo:hi], qwb, kwb, cache, posn[lo:hi], wl.eps, hq, hkv, H)

        def nbytes(rows):
            return sum(rope_bytes(rows, hq, hkv, H))
        unit = "tokens"
    elif wl.kind == "act":
        xb = synth.bits(synth.make_act_inputs(wl.index, T, H))
        if mode == 0:
            s_in = float(np.abs(O.silu_mul(synth.bits(synth.make_act_warmup(wl.index, H)))).max()
                         / np.float32(448))
        elif mode == 3:
            s_in = float(np.float32(448 * 6) / np.abs(O.silu_mul(xb[:256])).max())
        else:
            s_in = 0.0
        G4 = 16 if mode == 3 else G

        def run_rows(lo, hi):
            O.silu_mul_quant(xb[lo:hi], mode, scale_in=s_in, group_size=G4, flags=flags & ~1)

        def nbytes(rows):
            return sum(algorithmic_bytes(mode, rows, H, G4, flags, False, "act"))
        unit = "rows"
    elif wl.kind == "fp4dyn":
        x, r, w = synth.make_inputs(wl.index, T, H)
        xb, rb, wb = synth.bits(x), synth.bits(r), synth.bits(w)

        def run_rows(lo, hi):  # each span takes its own batch scale: the same work per row
            O.fused_fp4_dynamic(xb[lo:hi], rb[lo:hi], wb, wl.eps)

        def nbytes(rows):
            return sum(fp4dyn_bytes(rows, H))
        unit = "rows"
    elif wl.kind == "pad":
        ld = -(-H // wl.pad_multiple) * wl.pad_multiple
        x, r, w = synth.make_inputs(wl.index, T, H)
        xb, rb, wb = synth.bits(x), synth.bits(r), synth.bits(w)

        def run_rows(lo, hi):
            O.rms_norm_pad(xb[lo:hi], rb[lo:hi], wb, wl.eps, ld)

        def nbytes(rows):
            return sum(pad_bytes(rows, H, ld))
        unit = "rows"
    else:
        x, r, w = synth.make_inputs(wl.index, T, H)
        xb, rb, wb = synth.bits(x), (synth.bits(r) if r is not None else None), synth.bits(w)
        if mode == 0:
            if wl.static_scale is not None:
                s_in = wl.static_scale
            else:
                xw, rw = synth.make_warmup(wl.index, H)
                y = O.rms_y(synth.bits(xw), synth.bits(rw), wb, wl.eps)
                s_in = float(np.abs(y).max() / np.float32(448))
        elif mode == 3:
            s_in = float(np.float32(448 * 6) / np.abs(
                O.rms_y(xb[:256], None if rb is None else rb[:256], wb, wl.eps)).max())
        else:
            s_in = 0.0

        def run_rows(lo, hi):
            O.fused(xb[lo:hi], None if rb is None else rb[lo:hi], wb, wl.eps, mode,
                    scale_in=s_in, group_size=G, flags=flags & ~1)

        def nbytes(rows):
            return sum(algorithmic_bytes(mode, rows, H, G, flags, rb is not None))
        unit = "rows"

    chunk = 64
    rows = 0
    t0 = time.perf_counter()
    while rows < T and time.perf_counter() - t0 < budget_s:
        n = min(chunk, T - rows)
        run_rows(rows, rows + n)
        rows += n
    dt1 = time.perf_counter() - t0
    nthr = min(host_threads(), rows)
    step = -(-rows // (4 * nthr))  # four spans per thread
    spans = [(lo, min(lo + step, rows)) for lo in range(0, rows, step)]
    times = []
    with ThreadPoolExecutor(max_workers=nthr) as ex:
        for _ in range(3):  # median of three threaded passes
            t0 = time.perf_counter()
            list(ex.map(lambda sp: run_rows(*sp), spans))
            times.append(time.perf_counter() - t0)
    dtn = sorted(times)[1]
    b = nbytes(rows)
    return {"value": b / dtn / 1e9, "unit": "GB/s", "cores": nthr, "kind": "oracle",
            "sample": f"first {rows} of {T} {unit}: {dt1:.1f} s on one thread, {dtn:.2f} s on "
                      f"{nthr} threads (median of 3; {os.cpu_count()} host CPUs visible, "
                      f"{cpu_model()})",
            "tokens_per_s": rows / dtn,
            "single_thread": {"value": b / dt1 / 1e9, "unit": "GB/s", "cores": 1,
                              "tokens_per_s": rows / dt1}}


def load_traffic(key):
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get(key)
    if not e or e.get("kernel_source") != kernel_source_hash():
        return None
    return e


# ---------------------------------------------------------------- rocprofv3 summaries
COPY_BYTES = 256 << 20  # the plain copy bench.py runs for calibration (copy_src above)


def _db_rows(db, sql):
    import sqlite3

    con = sqlite3.connect(db)
    try:
        return con.execute(sql).fetchall()
    finally:
        con.close()


def summarize(ktrace_db, fetch_db, write_db, key, title, commands, out_md, util=()):
    """Turn the three rocprofv3 databases of one bench configuration into a short text summary
    under profiles/ and the traffic entry bench.py reports.  Counters are KiB per dispatch;
    each is scaled by what it reads for the plain 256 MiB copy in the same run."""
    import statistics

    top = _db_rows(ktrace_db, "select name, total_calls, total_duration, average, percentage "
                              "from top_kernels")
    mine = [r for r in top if "rmsq::" in r[0]]
    # the benched instantiation has the most calls; a step of several launches (the FP4 path
    # with a batch scale) has several kernels with that count, and its figures are their sums
    ncalls = max(r[1] for r in mine)
    step_k = [r for r in mine if r[1] == ncalls]
    main_k = step_k[0] if len(step_k) == 1 else (
        " + ".join(r[0] for r in step_k), ncalls, sum(r[2] for r in step_k),
        sum(r[3] for r in step_k), sum(r[4] for r in step_k))
    durs = [r[0] for r in _db_rows(ktrace_db, "select duration from kernels where name = '%s'"
                                   % step_k[0][0].replace("'", "''"))]
    if len(step_k) > 1:  # per step: the sum of its kernels' durations, in dispatch order
        per = [[d for (d,) in _db_rows(ktrace_db, "select duration from kernels where name = "
                                       "'%s' order by start" % r[0].replace("'", "''"))]
               for r in step_k]
        durs = [sum(ds) for ds in zip(*per)]

    def counter(db, name):
        rows = _db_rows(db, "select kernel_name, value from counters_collection "
                            "where counter_name = '%s'" % name)
        med = [statistics.median([v for k, v in rows if k == r[0]]) for r in step_k]
        n = len([v for k, v in rows if k == step_k[0][0]])
        copies = sorted((v for k, v in rows if k.startswith("__amd_rocclr_copyBuffer")),
                        reverse=True)[:10]
        return sum(med), statistics.median(copies), n

    f_k, f_copy, nf = counter(fetch_db, "FETCH_SIZE")
    w_k, w_copy, nw = counter(write_db, "WRITE_SIZE")
    f_scale = (COPY_BYTES / 1024) / f_copy
    w_scale = (COPY_BYTES / 1024) / w_copy
    fetch_b = f_k * 1024 * f_scale
    write_b = w_k * 1024 * w_scale
    entry = {"kernel": main_k[0], "kernel_source": kernel_source_hash(),
             "bytes_per_launch": int(round(fetch_b + write_b)), "fetch_bytes": int(round(fetch_b)),
             "write_bytes": int(round(write_b)),
             "calibration": {"copy_bytes": COPY_BYTES, "fetch_kib_copy": f_copy,
                             "write_kib_copy": w_copy, "fetch_scale": round(f_scale, 5),
                             "write_scale": round(w_scale, 5)},
             "avg_duration_us": round(main_k[3], 3)}
    try:
        allt = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        allt = {}
    allt[key] = entry
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allt, fh, indent=1, sort_keys=True)
        fh.write("\n")

    lines = [f"# {title}", "", "Commands (from the repository root, on an MI355X host):", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for r in top[:8]:
        lines.append(f"| `{r[0][:90]}` | {r[1]} | {r[2]:.1f} | {r[3]:.3f} | {r[4]:.1f} |")
    what = ("Benched kernel" if len(step_k) == 1 else
            f"Benched step ({len(step_k)} kernels per step, figures summed over them)")
    lines += ["", f"{what} `{main_k[0]}`: {len(durs)} dispatches, average "
              f"{main_k[3]:.3f} us, median {statistics.median(durs) / 1e3:.3f} us, "
              f"min {min(durs) / 1e3:.3f} us, max {max(durs) / 1e3:.3f} us.", "",
              "## HBM traffic (rocprofv3 --pmc, one counter per run)", "",
              "| counter | benched kernel, KiB/dispatch (median of %d) | 256 MiB copy, KiB | scale "
              "| bytes/launch |" % nf, "|---|---|---|---|---|",
              f"| FETCH_SIZE | {f_k:.2f} | {f_copy:.2f} | {f_scale:.5f} | {fetch_b:,.0f} |",
              f"| WRITE_SIZE | {w_k:.2f} | {w_copy:.2f} | {w_scale:.5f} | {write_b:,.0f} |", "",
              f"Measured HBM traffic per launch: {fetch_b + write_b:,.0f} bytes.", ""]
    if util:
        lines += ["## Utilization (rocprofv3 derived metrics, one per run)", "",
                  "| metric | benched kernel, median over dispatches | dispatches |", "|---|---|---|"]
        for name, db in util:
            rows = _db_rows(db, "select kernel_name, value from counters_collection "
                                "where counter_name = '%s'" % name)
            for r in step_k:  # one row per kernel of the step
                vals = [v for k, v in rows if k == r[0]]
                label = name if len(step_k) == 1 else (
                    f"{name}, `{r[0].split('(')[0].replace('void ', '')}`")
                if vals:
                    lines.append(f"| {label} | {statistics.median(vals):.2f} | {len(vals)} |")
        med = {}
        for name, db in util:
            rows = _db_rows(db, "select kernel_name, value from counters_collection "
                                "where counter_name = '%s'" % name)
            vals = [v for k, v in rows if k == step_k[0][0]]
            if vals:
                med[name] = statistics.median(vals)
        if med.get("SQ_WAVES"):
            per_wave = [(n, med[n] / med["SQ_WAVES"]) for n in
                        ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_WAIT_ANY",
                         "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU") if n in med]
            if per_wave:
                lines += ["", "Per wave (the counter's median over dispatches / SQ_WAVES): " +
                          ", ".join(f"{n} {v:,.1f}" for n, v in per_wave) + "."]
        lines += ["", "VALUBusy: % of GPU time the vector ALUs issue; MemUnitStalled: % of GPU time "
                  "the texture/memory unit stalls on data; OccupancyPercent: resident waves as % "
                  "of the maximum.  SQ_* are raw counts per dispatch: waves launched, vector / "
                  "scalar / LDS instructions issued, wave-cycles waiting on anything / on an "
                  "instruction dependency, cycles the vector ALU was busy for a wave, and the "
                  "cycles the sequencers were busy.", ""]
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines))
    return entry


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="w1",
                    choices=["w0", "w1", "w2", "w3", "w4", "w5", "w6", "w7", "w8"],
                    help="w0-w4: (residual add ->) RMSNorm -> quant workloads; w5: SiLU+Mul -> "
                         "quant; w6: add+RMSNorm -> padded bf16; w7: QK-norm + RoPE; w8: add+RMSNorm "
                         "-> FP4 with the global scale from the batch (default w1: "
                         "add+RMSNorm -> FP8 "
                         "static, 4096 x 4096)")
    ap.add_argument("--quant", default="static", choices=["static", "token", "group", "fp4"],
                    help="quantization scheme of the SiLU+Mul workload (w5)")
    ap.add_argument("--tokens", type=int, default=0)
    ap.add_argument("--hidden", type=int, default=0)
    ap.add_argument("--group", type=int, default=128)
    ap.add_argument("--flags", default="")
    ap.add_argument("--launch", default="")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--inplace", action="store_true",
                    help="write the updated residual over the residual input")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="time eager back-to-back launches only (default: also a HIP-graph "
                         "replay of the same K launches, which is what value reports)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--configs", choices=["auto", "on", "off"], default="auto",
                    help="also time every configuration of the add + RMSNorm + quant family "
                         "and report them under 'configs' (auto: only for the default "
                         "workload with no size or launch override)")
    ap.add_argument("--summarize", nargs=3, metavar=("KTRACE_DB", "FETCH_DB", "WRITE_DB"),
                    help="write the profiles/ summary and traffic entry for this configuration "
                         "from three rocprofv3 databases, then exit")
    ap.add_argument("--summary-md", default="")
    ap.add_argument("--util", nargs="*", default=[], metavar="METRIC=DB",
                    help="with --summarize: rocprofv3 databases of derived-metric runs to add")
    ap.add_argument("--commands", default="", help="';;'-separated commands quoted in the summary")
    args = ap.parse_args()

    if args.summarize:
        from rmsnorm_quantization_amd import synth  # noqa: F401

        wl, T, H, mode, G, flags = workload_spec(args)
        key = f"{args.workload}_T{T}_H{H}_{MODE_NAMES[mode]}_G{G}_f{flags}"
        family = {"act": "silu_mul_kernel", "rope": "qk_norm_rope_kernel",
                  "fp4dyn": "fused_kernel_x2"}.get(wl.kind, "fused_kernel")
        md = args.summary_md or os.path.join(ROOT, "profiles", f"{family}_{key}.md")
        if wl.kind == "rope":
            title = (f"{family}, {wl.name}: {T} tokens x {wl.heads[0]} q + {wl.heads[1]} k heads "
                     f"of {H} (qkv in place)")
        else:
            title = (f"{family}, {wl.name}: {T} tokens x "
                     f"{'intermediate' if wl.kind == 'act' else 'hidden'}"
                     f" {H}, {MODE_NAMES[mode]}{' G=%d' % G if mode == 2 else ''}")
        util = [tuple(u.split("=", 1)) for u in args.util]
        e = summarize(*args.summarize, key, title, [c.strip() for c in args.commands.split(";;")
                                                     if c.strip()], md, util)
        print(json.dumps(e))
        return

    if args.gpus != 1:
        print(f"bench.py: runs on exactly one GPU; --gpus {args.gpus} is not "
              f"supported: token rows shard across GPUs with no exchange, and one GPU's share "
              f"is what this benchmark measures",
              file=sys.stderr)
        sys.exit(2)

    wl, T, H, mode, G, flags = workload_spec(args)
    rope = wl.kind == "rope"
    if rope:
        g = rope_leg(args, wl, T, H)
    elif wl.kind == "fp4dyn":
        g = fp4dyn_leg(args, wl, T, H)
    else:
        g = gpu_leg(args, wl, T, H, mode, G, flags)
    eager_gbs = g["bytes"] / (g["ms_per_step"] * 1e-3) / 1e9
    step_ms = g["ms_per_step_graph"] if g["ms_per_step_graph"] else g["ms_per_step"]
    gbs = g["bytes"] / (step_ms * 1e-3) / 1e9
    # the kernel's own average duration, from dispatch-stamped event pairs
    achieved = g["bytes"] / (g["avg_launch_ms"] * 1e-3) / 1e9
    key = f"{args.workload}_T{T}_H{H}_{MODE_NAMES[mode]}_G{G}_f{flags}"
    tr = load_traffic(key)
    out = {
        "metric": "fused add+RMSNorm+quant GB/s & % of MI355X HBM peak; tokens/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}: {T} tokens x ({wl.heads[0]} q + {wl.heads[1]} k + "
                         f"{wl.heads[1]} v heads) x head size {H}, positions in "
                         f"[0, {wl.max_position}), NeoX rotation, "
                         if rope else
                         f"{wl.name}: {T} tokens x intermediate {H} (input [T, 2I]), "
                         if wl.kind == "act" else
                         f"{wl.name}: {T} tokens x hidden {H}, "
                         f"{'residual add, ' if wl.residual else ''}")
                        + f"{MODE_NAMES[mode]}"
                        f"{f' G={G}' if mode == 2 else ''}{f' flags={flags}' if flags else ''}",
            "tokens": T, "hidden": H, "mode": MODE_NAMES[mode], "group_size": G,
            "flags": flags, "residual": wl.residual, "eps": wl.eps,
            "io": "bf16 in; " + {3: "e2m1 + e4m3 block scales out",
                                 6: "e2m1 + e4m3 block scales + f32 global scale out (two "
                                    "launches; the input is read twice)",
                                 4: f"bf16 out, rows padded to a multiple of {wl.pad_multiple}",
                                 5: "q and k heads rewritten in place (bf16), f32 cos/sin cache"
                                 }.get(mode, "e4m3fn out"),
            "launch": ("library default" if g["launch"] is None else
                       {"heads_per_block": g["launch"][0], "heads_per_lane": g["launch"][1]}
                       if rope else
                       {"threads_per_row": g["launch"][0], "chunks_per_thread": g["launch"][1],
                        "rows_per_block": g["launch"][2], "options": g["launch"][3]}),
            "rotating_sets": g["sets"], "parallelism": "single GPU",
        },
        "tokens_per_s": round(T / (step_ms * 1e-3), 1),
        "latency_us_per_launch": round(step_ms * 1e3, 3),
        "timing": ("one HIP graph of K launches" if g["ms_per_step_graph"]
                   else "K eager back-to-back launches"),
        "eager": {"ms_per_step": round(g["ms_per_step"], 5), "GBs": round(eager_gbs, 1)},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "bytes_per_step": g["bytes"],
        "kernel_us": {"mean": round(g["avg_launch_ms"] * 1e3, 3),
                      "median": round(g["median_launch_ms"] * 1e3, 3),
                      "p10": round(g["p10_launch_ms"] * 1e3, 3),
                      "p90": round(g["p90_launch_ms"] * 1e3, 3)},
        "copy_ceiling": {
            "kernel": "128-bit copy over 2 x 256 MiB (librmsq_probe.so), median of 20",
            "GBs": round(g["copy_gbs"]["copy_GBs"], 1),
            "frac_of_peak": round(g["copy_gbs"]["copy_GBs"] / HBM_PEAK_GBS, 4),
            "torch_copy_GBs": round(g["copy_gbs"]["torch_copy_GBs"], 1),
            "eighty_pct_of_peak_reachable": g["copy_gbs"]["copy_GBs"] >= 0.8 * HBM_PEAK_GBS},
        "device": g["device"],
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "timing": (f"achieved = algorithmic bytes / the mean kernel duration of {args.steps} "
                       "launches, each bracketed by a HIP event pair that its own dispatch "
                       "stamps (hipExtLaunchKernel) on the launch stream"),
            "kernel_us": round(g["avg_launch_ms"] * 1e3, 3),
            "frac_of_copy_ceiling": round(achieved / g["copy_gbs"]["copy_GBs"], 4),
            "traffic": None if tr is None else tr["bytes_per_launch"],
        },
        "cpu_baseline": None,
    }
    c = g.get("ceiling")
    if c:
        c_gbs = c["bytes"] / (c["kernel_us"] * 1e-6) / 1e9
        out["roofline"]["ceiling"] = {
            "kernel": "memory-only probe, same traffic and launch shape (librmsq_probe.so)",
            "kernel_us": round(c["kernel_us"], 3), "bytes": c["bytes"],
            "GBs": round(c_gbs, 1), "frac_of_peak": round(c_gbs / HBM_PEAK_GBS, 4),
            "probe_time_over_kernel_time": round(c["kernel_us"] / (g["avg_launch_ms"] * 1e3), 4),
            "median_us": round(c["median_us"], 3),
            "median_ratio": round(c["median_us"] / (g["median_launch_ms"] * 1e3), 4)}
    if tr is not None:
        out["roofline"]["traffic_detail"] = {k: tr[k] for k in ("fetch_bytes", "write_bytes",
                                                                "calibration") if k in tr}
    want_configs = args.configs == "on" or (
        args.configs == "auto" and args.workload == "w1" and not args.tokens and not args.hidden
        and not args.launch)
    if want_configs:
        main_key = (wl.index, T, H, mode, G, flags)
        out["configs"] = configs_leg(args, None if rope or wl.kind != "norm" else (main_key, g))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_leg(wl, T, H, mode, G, flags, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
