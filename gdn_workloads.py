"""Seeded synthetic inputs for the gated delta rule prefill scan.

Shared by the tests, the smoke check and the benchmark; used to feed both the
HIP library and the CPU oracle with the same values.  This module holds the
input recipes only (shapes, length mixes, value distributions); it computes
nothing of the method itself.

Recipes (head_dim d = 128 everywhere; the pages fix d = 128 in every shape
on "flashinfer.cudnn.cudnn_chunk_gated_delta_rule", Parameters):

  tiny_fp32      2 sequences, cu_seqlens [0, 37, 128] (int32), Hqk = Hv = 2,
                 fp32 q/k/v; q, k ~ N(0,1) L2-normalised on the host
                 (variant "raw_l2": raw, normalised in-kernel); g ~ U[0.9, 1);
                 beta ~ U(0, 1); no initial state; fp32 final state.
  varlen_bf16    8 sequences, lengths ~ U{1..4096}; Hqk = 16, Hv = 32; bf16
                 q/k/v ~ N(0,1), in-kernel L2 norm; g = exp(-softplus(x)*0.1),
                 beta = sigmoid(y), x, y ~ N(0,1), fp32; fp32 initial state
                 ~ N(0, 0.01^2); int64 cu_seqlens.  Variants: "gates_bf16"
                 (g, beta stored bf16), "long_memory" (g ~ U[0.999, 1]).
  long_single    1 sequence of 65536 tokens, otherwise as varlen_bf16.
  many_short     256 sequences, lengths ~ U{0..256} with sequences 0, 127 and
                 255 forced empty; bf16 initial and final state; int32.
  large_batch    32 sequences x 8192 tokens (262144), int32; fp32 state.

  decode_batch   256 sequences of one token each (one decode step after a
                 prefill), Hqk = 16, Hv = 32, bf16 q/k/v, fp32 state ~ N(0, 0.01^2)
                 updated in place; gates as varlen_bf16.

Variant "alt_gates" (long_single, many_short, large_batch) draws
g ~ U[0.9, 1) and beta ~ U(0, 1) instead; variant "long_memory" of
long_single draws g ~ U[0.999, 1] (a memory of ~1000 tokens, so errors of the
state carried across chunks and segments are not hidden by fast decay).

Draw order per recipe: lengths, q, k, v, g source, beta source, state, from
torch.Generator(device).manual_seed(1000 + index).
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

D = 128
CONFIG_NAMES = ["tiny_fp32", "varlen_bf16", "long_single", "many_short", "large_batch"]


@dataclass
class Workload:
    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: Optional[torch.Tensor]
    beta: Optional[torch.Tensor]
    cu_seqlens: torch.Tensor
    initial_state: Optional[torch.Tensor]
    state_dtype: Optional[torch.dtype]          # dtype of output_state, None = not written
    use_qk_l2norm: bool
    scale: float = 0.0
    meta: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.q.shape[0]

    @property
    def N(self):
        return self.cu_seqlens.shape[0] - 1

    @property
    def Hqk(self):
        return self.q.shape[1]

    @property
    def Hv(self):
        return self.v.shape[1]

    def lengths(self):
        cu = self.cu_seqlens.cpu().to(torch.int64)
        return (cu[1:] - cu[:-1]).tolist()

    def to(self, device):
        mv = lambda t: None if t is None else t.to(device)
        return Workload(self.name, mv(self.q), mv(self.k), mv(self.v), mv(self.g), mv(self.beta),
                        mv(self.cu_seqlens), mv(self.initial_state), self.state_dtype,
                        self.use_qk_l2norm, self.scale, dict(self.meta))


def _gen(seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def _randn(shape, gen, device, dtype):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def _rand(shape, gen, device, lo, hi):
    return torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * (hi - lo) + lo


def build(lengths, Hqk, Hv, io_dtype, *, seed, device="cpu", cu_dtype=torch.int32,
          gate="sigmoid", gate_dtype=torch.float32, state_in=torch.float32,
          state_out=torch.float32, use_qk_l2norm=True, prenormalize=False,
          state_std=0.01, name="custom", with_g=True, with_beta=True, scale=0.0):
    """General recipe used by every named config (and by edge-case tests).

    gate: "sigmoid"   -> g = exp(-softplus(x) * 0.1), beta = sigmoid(y)
          "uniform"   -> g ~ U[0.9, 1), beta ~ U(0, 1)
          "long"      -> g ~ U[0.999, 1], beta = sigmoid(y)
    state_in / state_out: dtype or None (no initial state / no final state).
    """
    gen = _gen(seed, device)
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int64)
    cu[1:] = torch.tensor(lengths, dtype=torch.int64).cumsum(0) if lengths else cu[1:]
    q = _randn((T, Hqk, D), gen, device, torch.float32)
    k = _randn((T, Hqk, D), gen, device, torch.float32)
    v = _randn((T, Hv, D), gen, device, io_dtype)
    if prenormalize:
        q = torch.nn.functional.normalize(q, dim=-1)
        k = torch.nn.functional.normalize(k, dim=-1)
    q, k = q.to(io_dtype), k.to(io_dtype)
    x = _randn((T, Hv), gen, device, torch.float32)
    y = _randn((T, Hv), gen, device, torch.float32)
    if gate == "sigmoid":
        g = torch.exp(-torch.nn.functional.softplus(x) * 0.1)
        beta = torch.sigmoid(y)
    elif gate == "uniform":
        g = _rand((T, Hv), gen, device, 0.9, 1.0)
        beta = _rand((T, Hv), gen, device, 0.0, 1.0)
    elif gate == "long":
        g = _rand((T, Hv), gen, device, 0.999, 1.0)
        beta = torch.sigmoid(y)
    else:
        raise ValueError(gate)
    g, beta = g.to(gate_dtype), beta.to(gate_dtype)
    s0 = None
    if state_in is not None:
        s0 = (_randn((len(lengths), Hv, D, D), gen, device, torch.float32) * state_std).to(state_in)
    return Workload(name, q, k, v, g if with_g else None, beta if with_beta else None,
                    cu.to(cu_dtype).to(device), s0, state_out, use_qk_l2norm, scale,
                    dict(lengths=lengths, seed=seed, gate=gate))


def make(config, *, device="cpu", variant=None):
    """Named workload ``config`` (index or name), optionally a variant."""
    idx = config if isinstance(config, int) else CONFIG_NAMES.index(config)
    seed = 1000 + idx
    alt = variant == "alt_gates"
    if idx == 0:
        raw = variant == "raw_l2"
        return build([37, 91], 2, 2, torch.float32, seed=seed, device=device, gate="uniform",
                     state_in=None, state_out=torch.float32, use_qk_l2norm=raw,
                     prenormalize=not raw, name=CONFIG_NAMES[0] + ("/raw_l2" if raw else ""))
    if idx == 1:
        gen = _gen(seed, "cpu")
        lengths = torch.randint(1, 4097, (8,), generator=gen).tolist()
        return build(lengths, 16, 32, torch.bfloat16, seed=seed + 100, device=device,
                     cu_dtype=torch.int64,
                     gate="long" if variant == "long_memory" else "sigmoid",
                     gate_dtype=torch.bfloat16 if variant == "gates_bf16" else torch.float32,
                     name=CONFIG_NAMES[1] + (f"/{variant}" if variant else ""))
    if idx == 2:
        gate = "uniform" if alt else ("long" if variant == "long_memory" else "sigmoid")
        return build([65536], 16, 32, torch.bfloat16, seed=seed, device=device,
                     cu_dtype=torch.int64, gate=gate,
                     name=CONFIG_NAMES[2] + (f"/{variant}" if variant else ""))
    if idx == 3:
        gen = _gen(seed, "cpu")
        lengths = torch.randint(0, 257, (256,), generator=gen)
        lengths[[0, 127, 255]] = 0
        return build(lengths.tolist(), 16, 32, torch.bfloat16, seed=seed + 100, device=device,
                     cu_dtype=torch.int32, gate="uniform" if alt else "sigmoid",
                     state_in=torch.bfloat16, state_out=torch.bfloat16,
                     name=CONFIG_NAMES[3] + ("/alt_gates" if alt else ""))
    if idx == 4:
        return build([8192] * 32, 16, 32, torch.bfloat16, seed=seed, device=device,
                     cu_dtype=torch.int32, gate="uniform" if alt else "sigmoid",
                     name=CONFIG_NAMES[4] + ("/alt_gates" if alt else ""))
    raise ValueError(config)


def decode_batch(*, device="cpu", N=256):
    """One token for each of N sequences: the input of one decode step."""
    return build([1] * N, 16, 32, torch.bfloat16, seed=1100, device=device, name="decode_batch")


def slice_item(w: Workload, n: int, heads):
    """CPU copies of sequence n restricted to v-heads ``heads`` (and the q/k
    heads they read), as a one-sequence workload; used to check sampled
    outputs of full-size runs one by one."""
    cu = w.cu_seqlens.cpu().to(torch.int64)
    bos, eos = int(cu[n]), int(cu[n + 1])
    r = w.Hv // w.Hqk
    heads = list(heads)
    qk_heads = [h // r for h in heads]
    pick = lambda t, hs: None if t is None else t[bos:eos][:, hs].cpu()
    s0 = None if w.initial_state is None else w.initial_state[n:n + 1][:, heads].cpu()
    return Workload(f"{w.name}[n={n},h={heads}]", pick(w.q, qk_heads), pick(w.k, qk_heads),
                    pick(w.v, heads), pick(w.g, heads), pick(w.beta, heads),
                    torch.tensor([0, eos - bos], dtype=torch.int64), s0, w.state_dtype,
                    w.use_qk_l2norm, w.scale, dict(w.meta))
