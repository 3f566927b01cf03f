"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and arranges them; it holds none of the
attention or softmax arithmetic, so the oracle and the HIP path can both be
fed from it without sharing any of the method.

Every tensor is drawn on the CPU with ``torch.Generator`` so the same bits
reach the GPU and the oracle on any machine:

* attention: Q, K, V drawn in that order as fp32 ``randn`` of shape
  [B, H, N, d], then cast round-to-nearest-even to bf16 for the bf16
  workloads; the causal N=4096 workload multiplies every 64th query row
  (i % 64 == 0, every batch and head) by 8 after the cast, which is exact
  in bf16, to force large jumps of the running row maximum;
* backward: the upstream gradient dO is N(0, 1) of Q's shape, drawn from a
  generator of its own, then cast to bf16;
* row softmax: fp32 ``randn`` of shape [B, N] times ``std``; the small
  workload overwrites row 0 with 1000 - j (a strictly falling row of huge
  values that overflows a softmax without the max subtraction).
"""
from __future__ import annotations

import dataclasses
import math

import torch

SEED_BASE = 20260000


@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    dtype: str            # "f32" or "bf16": element type of Q, K, V and O
    seed: int
    boost_every: int = 0  # >0: multiply query rows i % boost_every == 0 by boost
    boost: float = 8.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Counted FLOPs: two N x N x d products, 2 FLOPs per multiply-add,
        halved under the causal mask."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def describe(self) -> str:
        return (f"{self.name}: {self.dtype} B={self.B} H={self.H} N={self.N} "
                f"d={self.d} causal={int(self.causal)} seed={self.seed}")


@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    B: int
    N: int
    std: float
    seed: int
    falling_row0: bool = False  # row 0 := 1000 - j

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: each fp32 element read once and written once."""
        return 8 * self.B * self.N

    def describe(self) -> str:
        return f"{self.name}: f32 [{self.B},{self.N}] std={self.std} seed={self.seed}"


# The workloads the measurements and parity tests are defined on, named by
# what they are.
_ATTN_LIST = [
    AttnWorkload("attn_f32_B1H1N128d64", 1, 1, 128, 64, False, "f32", SEED_BASE + 1),
    AttnWorkload("attn_bf16_B2H8N1024d64", 2, 8, 1024, 64, False, "bf16", SEED_BASE + 2),
    AttnWorkload("attn_bf16_B4H16N2048d128", 4, 16, 2048, 128, False, "bf16",
                 SEED_BASE + 3),
    AttnWorkload("attn_bf16_B2H16N4096d128_causal_x8rows", 2, 16, 4096, 128, True,
                 "bf16", SEED_BASE + 4, boost_every=64),
    AttnWorkload("attn_bf16_B1H32N8192d128_causal", 1, 32, 8192, 128, True, "bf16",
                 SEED_BASE + 5),
]
_SOFTMAX_LIST = [
    SoftmaxWorkload("softmax_f32_4x128", 4, 128, 2.0, SEED_BASE + 101,
                    falling_row0=True),
    SoftmaxWorkload("softmax_f32_32768x8192", 32768, 8192, 1.0, SEED_BASE + 105),
]
ATTN = {w.name: w for w in _ATTN_LIST}
SOFTMAX = {w.name: w for w in _SOFTMAX_LIST}

# The headline pair: the causal B*H=32, N=4096, d=128 bf16 forward and the
# [32768, 8192] fp32 row softmax.
HEADLINE_ATTN = "attn_bf16_B2H16N4096d128_causal_x8rows"
HEADLINE_SOFTMAX = "softmax_f32_32768x8192"


def attn_inputs(w: AttnWorkload, *, B: int | None = None, H: int | None = None,
                N: int | None = None, d: int | None = None, seed: int | None = None):
    """Return CPU tensors (Q, K, V) for workload ``w`` (shape overrides allowed
    for edge-case tests; the recipe stays the same)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    d = w.d if d is None else d
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shape = (B, H, N, d)
    out = []
    for _ in range(3):
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        if w.dtype == "bf16":
            t = t.to(torch.bfloat16)
        out.append(t)
    q, k, v = out
    if w.boost_every > 0 and N > 0:
        q[:, :, ::w.boost_every, :] *= w.boost
    return q, k, v


def fp8_quantize(t: torch.Tensor):
    """Per-tensor FP8 (E4M3) storage of ``t``: the scale that maps the
    largest magnitude to 448 (1 for an all-zero tensor) and the codes of
    t / scale (round to nearest even), as uint8.  Returns (codes, scale)."""
    amax = float(t.abs().max()) if t.numel() else 0.0
    scale = amax / 448.0 if amax > 0 else 1.0
    codes = (t.to(torch.float32) / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale


def attn_inputs_fp8(w: AttnWorkload, *, B: int | None = None, H: int | None = None,
                    N: int | None = None, d: int | None = None, seed: int | None = None,
                    Hkv: int | None = None):
    """FP8 inputs for workload ``w``: the fp32 draws of attn_inputs (same
    seed, boosted rows included), each tensor stored as E4M3 codes with its own
    scale (fp8_quantize); K and V keep their first Hkv heads.  Returns
    ((q8, k8, v8), (q_scale, k_scale, v_scale)) as CPU tensors and floats."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    d = w.d if d is None else d
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shape = (B, H, N, d)
    q, k, v = (torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3))
    if w.boost_every > 0 and N > 0:
        q[:, :, ::w.boost_every, :] *= w.boost
    if Hkv is not None:
        k, v = k[:, :Hkv].contiguous(), v[:, :Hkv].contiguous()
    (q8, qs), (k8, ks), (v8, vs) = fp8_quantize(q), fp8_quantize(k), fp8_quantize(v)
    return (q8, k8, v8), (qs, ks, vs)


def hadamard_signs(d: int, seed: int) -> list:
    """d random signs (+1 or -1) for the Hadamard rotation, from a generator
    of their own; the rotation itself is the method's and is not here."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return [1 if b else -1 for b in torch.randint(0, 2, (d,), generator=g).tolist()]


def attn_inputs_outliers(*, B: int, H: int, N: int, d: int, seed: int, channels: int = 4,
                         factor: float = 20.0):
    """bf16 Q, K, V of N(0, 1) draws (attn_inputs' order) whose Q and K carry
    outlier head channels: ``channels`` columns, drawn from the same
    generator, multiplied by ``factor`` (the large, channel-aligned values
    that make one scale per tensor lose precision).  CPU tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, H, N, d)
    q, k, v = (torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3))
    ch = torch.randperm(d, generator=g)[:channels]
    q[..., ch] *= factor
    k[..., ch] *= factor
    return tuple(t.to(torch.bfloat16).contiguous() for t in (q, k, v))


def attn_inputs_blockwise(*, B: int, H: int, N: int, d: int, seed: int, Hkv: int | None = None):
    """bf16 Q, K, V of N(0, 1) draws whose 32-element blocks along each
    contracted axis (32 head columns of a Q or K row, 32 rows of a V column)
    are multiplied by powers of two from 2^-4 to 2^4, and with some blocks
    set to zero: inputs whose block scales all differ.  CPU tensors."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    shape = (B, H, N, d)
    q, k, v = (torch.randn(shape, generator=g, dtype=torch.float32) for _ in range(3))
    nb = (N + 31) // 32
    for t in (q, k):
        e = torch.randint(-4, 5, (B, H, N, d // 32), generator=g).to(torch.float32)
        e[torch.rand((B, H, N, d // 32), generator=g) < 0.02] = float("-inf")  # zero blocks
        t *= torch.exp2(e).repeat_interleave(32, dim=-1)
    e = torch.randint(-4, 5, (B, H, nb, d), generator=g).to(torch.float32)
    v *= torch.exp2(e).repeat_interleave(32, dim=2)[:, :, :N]
    if Hkv is not None:
        k, v = k[:, :Hkv], v[:, :Hkv]
    return tuple(t.to(torch.bfloat16).contiguous() for t in (q, k, v))


def grad_output(shape, seed: int, dtype: str = "bf16") -> torch.Tensor:
    """The upstream gradient dO for a backward test: N(0, 1) of ``shape`` from
    its own generator (seed), so Q, K, V stay those of the forward recipe."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def softmax_inputs(w: SoftmaxWorkload, *, B: int | None = None, N: int | None = None,
                   seed: int | None = None) -> torch.Tensor:
    B = w.B if B is None else B
    N = w.N if N is None else N
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    x = torch.randn((B, N), generator=g, dtype=torch.float32) * w.std
    if w.falling_row0 and B > 0:
        x[0] = 1000.0 - torch.arange(N, dtype=torch.float32)
    return x
