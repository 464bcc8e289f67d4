"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and lays them out in the shapes of the
workloads; it holds none of the quantization or forward arithmetic.  The pages
measure on real checkpoints (OLMoE-1B-7B, Qwen3-30B-A3B, gpt-oss-20b,
Mixtral-8x7B), none of which is available, so seeded tensors of the same
shapes and value distribution stand in for them.

Recipe (seed 0 throughout; per-tensor streams keyed by (seed, layer, tensor)):

* expert weights: N(0, 0.02) drawn in fp32, converted to bf16 by torch's
  round-to-nearest-even cast;
* Mixtral-shaped weights additionally carry 0.1 % outliers at +-20 sigma
  (+-0.4), positions drawn without replacement, random sign;
* hidden states: N(0, 1) -> bf16;
* routing: per token K distinct experts, uniform or Zipf(1.1)-skewed
  (expert 0 most popular); weights are the softmax of K N(0, 1) logits,
  formed in fp64 and stored as fp32.

Host generation uses ``numpy.random.default_rng``; device generation (for the
multi-GB weights of the large shapes) uses a seeded ``torch.Generator`` on the
device.  Either way the caller gets one set of bytes that both the GPU path
and the oracle read.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

GATE_UP, DOWN, HIDDEN, CHOICE, LOGITS, OUTLIERS, GRAD_OUT, ROUTER = range(8)


@dataclass(frozen=True)
class MoEShape:
    name: str
    E: int
    H: int
    I: int
    K: int
    fmt: str                      # "nf4" or "int8"
    routing: str = "uniform"      # "uniform" or "zipf"
    tokens: tuple = field(default_factory=tuple)
    layers: int = 1
    outliers: bool = False

    @property
    def gate_up_shape(self):
        return (self.E, 2 * self.I, self.H)

    @property
    def down_shape(self):
        return (self.E, self.H, self.I)


SHAPES = {
    "tiny": MoEShape("tiny", E=8, H=256, I=128, K=2, fmt="nf4", tokens=(64,)),
    "olmoe": MoEShape("olmoe", E=64, H=2048, I=1024, K=8, fmt="nf4",
                      tokens=(1, 32, 4096), layers=16),
    "qwen3": MoEShape("qwen3", E=128, H=2048, I=768, K=8, fmt="nf4", routing="zipf",
                      tokens=(1, 64, 8192), layers=48),
    "gptoss": MoEShape("gptoss", E=32, H=2880, I=2880, K=4, fmt="int8", tokens=(16, 2048)),
    "mixtral": MoEShape("mixtral", E=8, H=4096, I=14336, K=2, fmt="nf4", outliers=True,
                        tokens=(1, 512, 16384)),
}

OUTLIER_VALUE = 0.4           # 20 sigma of N(0, 0.02)
OUTLIER_FRACTION = 0.001


def _rng(seed, layer, tensor):
    return np.random.default_rng([seed, layer, tensor])


def _torch_gen(device, seed, layer, tensor):
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + layer) * 16 + tensor)
    return g


def expert_weights(shape, *, seed=0, layer=0, tensor=GATE_UP, std=0.02, outliers=False,
                   device="cpu"):
    """bf16 tensor of ``shape`` ~ N(0, std), optionally with 0.1 % +-20-sigma outliers."""
    shape = tuple(int(s) for s in shape)
    numel = int(np.prod(shape))
    dev = torch.device(device)
    if dev.type == "cpu":
        rng = _rng(seed, layer, tensor)
        w = torch.from_numpy(rng.standard_normal(numel, dtype=np.float32) * np.float32(std))
        if outliers:
            orng = _rng(seed, layer, OUTLIERS)
            n_out = int(round(OUTLIER_FRACTION * numel))
            pos = orng.choice(numel, n_out, replace=False)
            sign = np.where(orng.integers(0, 2, n_out) == 0, -1.0, 1.0).astype(np.float32)
            w[torch.from_numpy(pos)] = torch.from_numpy(sign * np.float32(OUTLIER_VALUE))
        return w.to(torch.bfloat16).reshape(shape)
    gen = _torch_gen(dev, seed, layer, tensor)
    w = torch.empty(numel, dtype=torch.bfloat16, device=dev)
    chunk = 1 << 28
    for s in range(0, numel, chunk):
        n = min(chunk, numel - s)
        w[s:s + n] = (torch.randn(n, generator=gen, device=dev, dtype=torch.float32) * std
                      ).to(torch.bfloat16)
    if outliers:
        ogen = _torch_gen(dev, seed, layer, OUTLIERS)
        n_out = int(round(OUTLIER_FRACTION * numel))
        pos = torch.randperm(numel, generator=ogen, device=dev)[:n_out]
        sign = torch.randint(0, 2, (n_out,), generator=ogen, device=dev).float() * 2 - 1
        w[pos] = (sign * OUTLIER_VALUE).to(torch.bfloat16)
    return w.reshape(shape)


def hidden_states(T, H, *, seed=0, layer=0, device="cpu"):
    """bf16 ``[T, H]`` ~ N(0, 1) (drawn on the host, then moved)."""
    rng = _rng(seed, layer, HIDDEN)
    x = torch.from_numpy(rng.standard_normal(T * H, dtype=np.float32)).to(torch.bfloat16)
    return x.reshape(T, H).to(device)


def router_weight(E, H, *, std=0.02, seed=0, layer=0, device="cpu"):
    """bf16 ``[E, H]`` ~ N(0, std^2): a router (gate) weight."""
    rng = _rng(seed, layer, ROUTER)
    g = torch.from_numpy(rng.standard_normal(E * H, dtype=np.float32) * np.float32(std)).to(torch.bfloat16)
    return g.reshape(E, H).to(device)


def grad_output(T, H, *, seed=0, layer=0, device="cpu"):
    """bf16 ``[T, H]`` ~ N(0, 1): an incoming gradient for the backward."""
    rng = _rng(seed, layer, GRAD_OUT)
    g = torch.from_numpy(rng.standard_normal(T * H, dtype=np.float32)).to(torch.bfloat16)
    return g.reshape(T, H).to(device)


def routing(T, K, E, *, kind="uniform", zipf_s=1.1, seed=0, layer=0, device="cpu"):
    """``(top_k_index int32 [T, K], top_k_weights float32 [T, K])``."""
    crng = _rng(seed, layer, CHOICE)
    lrng = _rng(seed, layer, LOGITS)
    if kind == "uniform":
        p = None
    elif kind == "zipf":
        p = (np.arange(1, E + 1, dtype=np.float64)) ** (-zipf_s)
        p = p / p.sum()
    else:
        raise ValueError(kind)
    idx = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        idx[t] = crng.choice(E, K, replace=False, p=p)
    logits = lrng.standard_normal((T, K))
    ex = np.exp(logits - logits.max(axis=1, keepdims=True))
    wts = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return (torch.from_numpy(idx).to(device), torch.from_numpy(wts).to(device))


def layer_inputs(shape: MoEShape, T, *, seed=0, layer=0, device="cpu"):
    """All inputs of one MoE layer: bf16 gate_up, down, hidden and the routing."""
    gu = expert_weights(shape.gate_up_shape, seed=seed, layer=layer, tensor=GATE_UP,
                        outliers=shape.outliers, device=device)
    dn = expert_weights(shape.down_shape, seed=seed, layer=layer, tensor=DOWN,
                        outliers=shape.outliers, device=device)
    x = hidden_states(T, shape.H, seed=seed, layer=layer, device=device)
    idx, wts = routing(T, shape.K, shape.E, kind=shape.routing, seed=seed, layer=layer,
                       device=device)
    return gu, dn, x, idx, wts


def bf16_bits(t):
    """A bf16 torch tensor as a numpy uint16 array of its bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
