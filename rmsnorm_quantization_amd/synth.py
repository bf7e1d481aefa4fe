"""Seeded synthetic inputs shaped like LLM activations (no part of the method's arithmetic).

Both the GPU path and the CPU oracle are fed from here.  Values are drawn in float32 from a
seeded torch CPU generator and cast to bf16 by torch; nothing in this module normalizes,
scales or quantizes.  Seven workloads are defined, matching the shapes and distributions of
the fused RMSNorm + quantization (0-4), SiLU+Mul + quantization (5), RMSNorm + padding (6) and
QK-norm + RoPE (7) workloads this library is measured on:

  0  RMSNorm -> FP8 static        T=16,  H=4096, x~N(0,1), w~U(0.5,1.5), eps 1e-5, scale 0.05
  1  add+RMSNorm -> FP8 static    T in {1,64,512,4096}, H=4096, x,r~N(0,1), eps 1e-5,
                                  static scale from one fixed 512x4096 warm-up batch
  2  add+RMSNorm -> FP8 per-token T in {1,256,2048,8192}, H=8192, eps 1e-6; x~N(0,1) with
                                  round(0.001*H) fixed outlier channels multiplied by 50
  3  add+RMSNorm -> FP8 per-group T in {1,128,1024,16384}, H in {5120,7168}, G in {128,64},
                                  row/col-major, f32/E8M0 scales, eps 1e-6
  4  add+RMSNorm -> FP4 block-16  T in {1,32,256,4096}, H=2048, eps 1e-6, global scale
                                  448*6/max|y| of the same batch

  5  SiLU+Mul -> quant            T in {1,256,4096}, I=14336 (the intermediate size of the
                                  Llama-3.1-8B model the pages use in their examples);
                                  x = [gate | up] ~N(0,1), [T, 2I]; static scale from a fixed
                                  512 x 2I warm-up batch, FP4 global scale 448*6/max|a|

  6  add+RMSNorm -> padded bf16    T in {1,256,4096}, H=2880 (the hidden size the pages name for
                                  this fusion) padded to a multiple of 256 (3072), x,r~N(0,1),
                                  eps 1e-5

  7  QK-norm + RoPE                T in {1,256,4096}, qkv [T, (32 + 2*8) * 128] ~N(0,1) (the head
                                  layout of Qwen3-8B, a model of the family the pages name for
                                  this fusion: 32 q heads, 8 kv heads, head size 128), q/k weights
                                  ~U(0.5,1.5), positions ~ uniform integers in [0, 32768) (a
                                  batch of independent sequences), NeoX pairing, eps 1e-6; the
                                  cos/sin cache (base 1e6, 32768 positions) is built by the caller

Seeds: 1000*workload + tensor id (x=1, residual=2, weight=3, outlier channels=4,
warm-up x=5, warm-up residual=6, k weight=7, positions=8).  Unless stated otherwise, weight ~ U(0.5, 1.5) and the
residual ~ N(0,1) without outliers.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    tokens: Tuple[int, ...]
    hidden: Tuple[int, ...]
    eps: float
    residual: bool
    outlier_frac: float = 0.0
    outlier_gain: float = 50.0
    static_scale: Optional[float] = None   # fixed per-tensor scale, if the workload fixes one
    warmup_shape: Optional[Tuple[int, int]] = None  # batch the static scale is derived from
    group_sizes: Tuple[int, ...] = field(default_factory=tuple)
    kind: str = "norm"   # "norm": (residual add ->) RMSNorm -> quant; "act": SiLU+Mul -> quant;
    #                      "pad": (residual add ->) RMSNorm -> padded bf16; "rope": QK-norm + RoPE;
    #                      "fp4dyn": add + RMSNorm -> FP4 with the global scale from the batch
    pad_multiple: int = 0
    heads: Tuple[int, int] = (0, 0)   # (q heads, kv heads) of a "rope" workload; hidden = head size
    max_position: int = 0
    rope_base: float = 0.0


WORKLOADS = {
    0: Workload(0, "rmsnorm_fp8_static", (16,), (4096,), 1e-5, False, static_scale=0.05),
    1: Workload(1, "add_rmsnorm_fp8_static", (1, 64, 512, 4096), (4096,), 1e-5, True,
                warmup_shape=(512, 4096)),
    2: Workload(2, "add_rmsnorm_fp8_per_token", (1, 256, 2048, 8192), (8192,), 1e-6, True,
                outlier_frac=0.001),
    3: Workload(3, "add_rmsnorm_fp8_per_group", (1, 128, 1024, 16384), (5120, 7168), 1e-6, True,
                group_sizes=(128, 64)),
    4: Workload(4, "add_rmsnorm_fp4_block16", (1, 32, 256, 4096), (2048,), 1e-6, True),
    5: Workload(5, "silu_mul_quant", (1, 256, 4096), (14336,), 0.0, False,
                warmup_shape=(512, 14336), group_sizes=(128, 64), kind="act"),
    6: Workload(6, "add_rmsnorm_pad", (1, 256, 4096), (2880,), 1e-5, True, kind="pad",
                pad_multiple=256),
    7: Workload(7, "qk_norm_rope", (1, 256, 4096), (128,), 1e-6, False, kind="rope",
                heads=(32, 8), max_position=32768, rope_base=1e6),
    # the FP4 shapes of workload 4, with the global scale computed from the batch itself
    8: Workload(8, "add_rmsnorm_fp4_batch_scale", (1, 32, 256, 4096), (2048,), 1e-6, True,
                kind="fp4dyn"),
}

X, RESIDUAL, WEIGHT, OUTLIERS, WARM_X, WARM_R, K_WEIGHT, POSITIONS = 1, 2, 3, 4, 5, 6, 7, 8


def _gen(workload: int, tensor: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * workload + tensor)
    return g


def normal_bf16(shape, workload: int, tensor: int) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(workload, tensor), dtype=torch.float32).to(
        torch.bfloat16)


def uniform_bf16(shape, lo: float, hi: float, workload: int, tensor: int) -> torch.Tensor:
    u = torch.rand(shape, generator=_gen(workload, tensor), dtype=torch.float32)
    return (u * (hi - lo) + lo).to(torch.bfloat16)


def outlier_channels(hidden: int, frac: float, workload: int) -> torch.Tensor:
    """round(frac*hidden) distinct channel indices, the same for every token."""
    n = int(round(frac * hidden))
    perm = torch.randperm(hidden, generator=_gen(workload, OUTLIERS))
    return torch.sort(perm[:n]).values


def make_x(wl: Workload, T: int, H: int, tensor: int = X) -> torch.Tensor:
    x = torch.randn((T, H), generator=_gen(wl.index, tensor), dtype=torch.float32)
    if wl.outlier_frac > 0:
        ch = outlier_channels(H, wl.outlier_frac, wl.index)
        x[:, ch] *= wl.outlier_gain
    return x.to(torch.bfloat16)


def make_inputs(workload: int, T: int, H: Optional[int] = None):
    """(x, residual or None, weight) as CPU bf16 tensors for one workload shape."""
    wl = WORKLOADS[workload]
    H = H if H is not None else wl.hidden[0]
    x = make_x(wl, T, H)
    r = normal_bf16((T, H), wl.index, RESIDUAL) if wl.residual else None
    w = uniform_bf16((H,), 0.5, 1.5, wl.index, WEIGHT)
    return x, r, w


def make_warmup(workload: int, H: Optional[int] = None):
    """The fixed warm-up batch (x, residual or None) a static scale is derived from."""
    wl = WORKLOADS[workload]
    T, Hw = wl.warmup_shape
    H = H if H is not None else Hw
    x = make_x(wl, T, H, tensor=WARM_X)
    r = normal_bf16((T, H), wl.index, WARM_R) if wl.residual else None
    return x, r


def make_act_inputs(workload: int, T: int, I: Optional[int] = None, tensor: int = X):
    """x = [gate | up] as one [T, 2I] CPU bf16 tensor for a SiLU+Mul workload."""
    wl = WORKLOADS[workload]
    I = I if I is not None else wl.hidden[0]
    return normal_bf16((T, 2 * I), wl.index, tensor)


def make_act_warmup(workload: int, I: Optional[int] = None):
    wl = WORKLOADS[workload]
    T, Iw = wl.warmup_shape
    return make_act_inputs(workload, T, I if I is not None else Iw, tensor=WARM_X)


def make_rope_inputs(workload: int, T: int, hq: Optional[int] = None, hkv: Optional[int] = None,
                     D: Optional[int] = None, max_position: Optional[int] = None):
    """(qkv [T, (hq + 2 hkv) * D], q weight [D], k weight [D]) as CPU bf16 tensors and positions
    [T] int64 for a QK-norm + RoPE workload."""
    wl = WORKLOADS[workload]
    hq = hq if hq is not None else wl.heads[0]
    hkv = hkv if hkv is not None else wl.heads[1]
    D = D if D is not None else wl.hidden[0]
    mp = max_position if max_position is not None else wl.max_position
    qkv = normal_bf16((T, (hq + 2 * hkv) * D), wl.index, X)
    qw = uniform_bf16((D,), 0.5, 1.5, wl.index, WEIGHT)
    kw = uniform_bf16((D,), 0.5, 1.5, wl.index, K_WEIGHT)
    pos = torch.randint(0, mp, (T,), generator=_gen(wl.index, POSITIONS), dtype=torch.int64)
    return qkv, qw, kw, pos


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """numpy uint16 bit patterns -> CPU bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(np.int16)).view(torch.bfloat16)
