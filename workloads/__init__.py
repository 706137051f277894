"""Seeded synthetic inputs for the DiLoCo outer-step merge.

This module builds the *inputs* of an outer step and nothing else: parameter-set
shapes, the global parameters theta_g, the learner replicas theta_i, the merge
weights and the learner presence pattern.  It holds none of the merge's own
arithmetic (no statistics, no quantizer, no codebook, no optimizer), so both the
CPU oracle and the HIP path can be fed from it without sharing any step of the
method.

Shapes follow the parameter sets the pages train or describe:
  * a single 4096x4096 fp32 projection (INTELLECT-1 notes, section 3.2 worked
    example, with pseudo-gradient std ~1.2e-3);
  * Llama-style transformer parameter lists (RMSNorm scale vectors, q/k/v/o with
    grouped KV heads, gated MLP, embedding and LM head);
  * an edge mix of many small vectors, mid-size matrices, a few large matrices
    and constant-pseudo-gradient tensors.

Random draws use torch generators seeded per (config, step, tensor, role), so
any tensor can be regenerated on its own.  Draws are made in fp32 on the target
device; learner replicas are formed as theta_i = fl32(theta_g - Delta_i), so the
pseudo-gradient a merge sees is fl32(theta_g - theta_i).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

ALIGN = 64  # element alignment of every tensor offset (256 bytes of fp32)

ROLE_THETA = 0          # theta_g of a tensor
ROLE_LEARNER0 = 1       # learner i uses role 1 + i
ROLE_CONFIG = 999       # config-level draws (per-tensor sigma, weights, absence)


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: tuple
    kind: str  # "matrix" | "embed" | "norm" | "vector" | "const"

    @property
    def numel(self) -> int:
        return int(math.prod(self.shape))


def llama_tensors(d: int, n_layers: int, ffn: int, n_heads: int, n_kv_heads: int,
                  vocab: int, tied: bool) -> List[TensorSpec]:
    """Llama-style parameter list: embedding, per-layer [attn_norm, q, k, v, o,
    mlp_norm, gate, up, down], final norm, then the LM head when untied."""
    head_dim = d // n_heads
    kv = n_kv_heads * head_dim
    out = [TensorSpec("embed", (vocab, d), "embed")]
    for layer in range(n_layers):
        p = f"layers.{layer}."
        out += [
            TensorSpec(p + "attn_norm", (d,), "norm"),
            TensorSpec(p + "q", (d, d), "matrix"),
            TensorSpec(p + "k", (kv, d), "matrix"),
            TensorSpec(p + "v", (kv, d), "matrix"),
            TensorSpec(p + "o", (d, d), "matrix"),
            TensorSpec(p + "mlp_norm", (d,), "norm"),
            TensorSpec(p + "gate", (ffn, d), "matrix"),
            TensorSpec(p + "up", (ffn, d), "matrix"),
            TensorSpec(p + "down", (d, ffn), "matrix"),
        ]
    out.append(TensorSpec("final_norm", (d,), "norm"))
    if not tied:
        out.append(TensorSpec("lm_head", (vocab, d), "embed"))
    return out


def edge_mix_tensors() -> List[TensorSpec]:
    """2000 vectors of 4096, 900 matrices 1024x1024, 90 matrices 4096x11008 and
    10 constant-pseudo-gradient vectors of 4096 (3000 tensors)."""
    out = [TensorSpec(f"vec.{i}", (4096,), "vector") for i in range(2000)]
    out += [TensorSpec(f"mat.{i}", (1024, 1024), "matrix") for i in range(900)]
    out += [TensorSpec(f"big.{i}", (4096, 11008), "matrix") for i in range(90)]
    out += [TensorSpec(f"const.{i}", (4096,), "const") for i in range(10)]
    return out


@dataclasses.dataclass(frozen=True)
class Config:
    key: str
    title: str
    tensors: tuple
    n_learners: int
    n_fragments: int
    delta: str            # "normal" | "student_t" | "normal_logu" | "normal_outlier" | "laplace"
    delta_scale: float
    weights: str          # "equal" | "dirichlet"
    steps: int = 1
    absent_p: float = 0.0
    lr: float = 0.7
    beta: float = 0.9


def _cfg(key: str) -> Config:
    if key == "c1":
        return Config("c1", "single fp32 4096x4096 tensor, K=3",
                      (TensorSpec("w", (4096, 4096), "matrix"),), 3, 1,
                      "normal", 1.2e-3, "equal")
    if key == "c2":
        return Config("c2", "135M Llama-style (tied), P=24 fragments, K=4",
                      tuple(llama_tensors(576, 30, 1536, 9, 3, 49152, tied=True)), 4, 24,
                      "student_t", 1e-3, "equal")
    if key == "c3":
        return Config("c3", "1B Llama-style (untied), K=8, Dirichlet weights, 10 steps",
                      tuple(llama_tensors(2048, 16, 5632, 32, 8, 32000, tied=False)), 8, 1,
                      "normal_logu", 0.0, "dirichlet", steps=10)
    if key == "c4":
        return Config("c4", "10B Llama-style (untied), P=24 fragments, K=14, outliers",
                      tuple(llama_tensors(4096, 42, 14336, 32, 8, 128256, tied=False)), 14, 24,
                      "normal_outlier", 1e-3, "equal")
    if key == "c5k1":
        return Config("c5k1", "edge mix of 3000 tensors, K=1",
                      tuple(edge_mix_tensors()), 1, 24, "laplace", 7e-4, "equal")
    if key == "c5k16":
        return Config("c5k16", "edge mix of 3000 tensors, K=16, absent learners",
                      tuple(edge_mix_tensors()), 16, 24, "laplace", 7e-4, "equal",
                      absent_p=0.25)
    raise KeyError(key)


CONFIG_KEYS = ("c1", "c2", "c3", "c4", "c5k1", "c5k16")
_CFG_IDS = {k: i + 1 for i, k in enumerate(CONFIG_KEYS)}


def config(key: str) -> Config:
    return _cfg(key)


def seed_of(cfg_key: str, step: int, tensor: int, role: int) -> int:
    """Deterministic 63-bit seed for one (config, step, tensor, role) stream."""
    h = _CFG_IDS.get(cfg_key, 0)
    for v in (step, tensor, role):
        h = (h * 1_000_003 + int(v) + 0x9E3779B1) % (1 << 61)
    return h


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def pack_offsets(numels: Sequence[int], align: int = ALIGN) -> tuple:
    """Offsets of tensors packed back to back, each rounded up to `align` elements.
    Returns (offsets, total_length)."""
    offs, pos = [], 0
    for n in numels:
        offs.append(pos)
        pos += (int(n) + align - 1) // align * align
    return offs, pos


# --- draws -----------------------------------------------------------------

def draw_theta(spec: TensorSpec, gen: torch.Generator, device) -> torch.Tensor:
    """theta_g for one tensor: RMSNorm scales and constant tensors are 1.0,
    everything else N(0, 0.02^2)."""
    n = spec.numel
    if spec.kind in ("norm", "const"):
        return torch.ones(n, dtype=torch.float32, device=device)
    return torch.randn(n, generator=gen, dtype=torch.float32, device=device).mul_(0.02)


def _uniform_open(n, gen, device):
    # U(0,1) strictly positive (log-safe)
    u = torch.rand(n, generator=gen, dtype=torch.float32, device=device)
    return u.clamp_(min=float.fromhex("0x1p-24"))


def draw_delta(cfg: Config, spec: TensorSpec, tensor_sigma: float, gen: torch.Generator,
               device) -> torch.Tensor:
    """One learner's pseudo-gradient for one tensor, fp32."""
    n = spec.numel
    if cfg.delta in ("normal", "normal_logu"):
        s = cfg.delta_scale if cfg.delta == "normal" else tensor_sigma
        return torch.randn(n, generator=gen, dtype=torch.float32, device=device).mul_(s)
    if cfg.delta == "student_t":
        # t_4 = Z / sqrt(chi2_4 / 4), chi2_4 = -2 ln(U1 U2); Var(t_4) = 2.
        z = torch.randn(n, generator=gen, dtype=torch.float32, device=device)
        u1 = _uniform_open(n, gen, device)
        u2 = _uniform_open(n, gen, device)
        chi2 = -2.0 * (torch.log(u1) + torch.log(u2))
        t = z / torch.sqrt(chi2 / 4.0)
        return t.mul_(cfg.delta_scale / math.sqrt(2.0))
    if cfg.delta == "normal_outlier":
        z = torch.randn(n, generator=gen, dtype=torch.float32, device=device).mul_(cfg.delta_scale)
        u = torch.rand(n, generator=gen, dtype=torch.float32, device=device)
        return torch.where(u < 1e-3, z * 50.0, z)
    if cfg.delta == "laplace":
        u = torch.rand(n, generator=gen, dtype=torch.float32, device=device) - 0.5
        mag = torch.neg(torch.log1p(-2.0 * u.abs())).clamp_(max=80.0)  # finite when u = -1/2
        return (torch.sign(u) * mag).mul_(cfg.delta_scale)
    raise ValueError(cfg.delta)


def tensor_sigmas(cfg: Config, n_tensors: int) -> List[float]:
    """Per-tensor pseudo-gradient std (log-uniform in [1e-4, 1e-2] for the 1B set)."""
    if cfg.delta != "normal_logu":
        return [cfg.delta_scale] * n_tensors
    g = generator(seed_of(cfg.key, 0, 0, ROLE_CONFIG), "cpu")
    u = torch.rand(n_tensors, generator=g, dtype=torch.float64)
    lo, hi = math.log(1e-4), math.log(1e-2)
    return [float(math.exp(lo + (hi - lo) * x)) for x in u.tolist()]


def base_weights(cfg: Config) -> List[float]:
    """Raw (unnormalised) learner weights for a run."""
    k = cfg.n_learners
    if cfg.weights == "equal":
        return [1.0 / k] * k
    g = generator(seed_of(cfg.key, 0, 1, ROLE_CONFIG), "cpu")
    e = -torch.log(torch.rand(k, generator=g, dtype=torch.float64).clamp_(min=1e-300))
    return (e / e.sum()).tolist()  # Dirichlet(1,...,1)


def presence(cfg: Config, fragment: int) -> List[int]:
    """Learner presence for one fragment: each learner absent with probability
    absent_p; if every learner is absent, learner 0 is forced present."""
    k = cfg.n_learners
    if cfg.absent_p <= 0.0:
        return [1] * k
    g = generator(seed_of(cfg.key, 0, 2 + fragment, ROLE_CONFIG), "cpu")
    u = torch.rand(k, generator=g, dtype=torch.float64).tolist()
    pres = [0 if x < cfg.absent_p else 1 for x in u]
    if not any(pres):
        pres[0] = 1
    return pres


def const_delta_value(cfg: Config, tensor: int, learner: int, const_index: int) -> float:
    """Constant pseudo-gradient of a constant tensor: 0 for the first one,
    Laplace(0, b) per (tensor, learner) otherwise."""
    if const_index == 0:
        return 0.0
    g = generator(seed_of(cfg.key, 0, tensor, ROLE_LEARNER0 + learner), "cpu")
    u = float(torch.rand(1, generator=g, dtype=torch.float64)) - 0.5
    return -math.copysign(1.0, u) * math.log1p(-2.0 * abs(u)) * cfg.delta_scale


# --- assembled inputs --------------------------------------------------------

@dataclasses.dataclass
class StepInputs:
    """Flat buffers and descriptors for one merge call.

    theta_g   : fp32 [global_len]           (tensor t at offsets[t])
    momentum  : fp32 [global_len]
    theta_L   : fp32 [K, learner_stride]    (tensor t at loffsets[t] in each row)
    tensors   : list of (offset, loffset, numel)
    weights   : raw learner weights (0 = absent)
    present   : 0/1 per learner
    """
    theta_g: torch.Tensor
    momentum: torch.Tensor
    theta_L: torch.Tensor
    tensors: list
    weights: list
    present: list
    tensor_ids: list
    learner_stride: int


def build_global(cfg: Config, tensor_ids: Sequence[int], device, step: int = 0,
                 offsets: Optional[Sequence[int]] = None):
    """theta_g and zero momentum for the listed tensors, packed (or at given offsets)."""
    specs = [cfg.tensors[t] for t in tensor_ids]
    if offsets is None:
        offsets, total = pack_offsets([s.numel for s in specs])
    else:
        total = max(o + s.numel for o, s in zip(offsets, specs))
        total = (total + ALIGN - 1) // ALIGN * ALIGN
    theta = torch.zeros(total, dtype=torch.float32, device=device)
    for t, s, off in zip(tensor_ids, specs, offsets):
        g = generator(seed_of(cfg.key, step, t, ROLE_THETA), device)
        theta[off:off + s.numel] = draw_theta(s, g, device)
    mom = torch.zeros(total, dtype=torch.float32, device=device)
    return theta, mom, list(offsets)


def learner_delta(cfg: Config, tensor: int, learner: int, step: int, sigma: float, device) -> torch.Tensor:
    """Learner `learner`'s pseudo-gradient draw for one tensor at one step: the
    draw build_learners subtracts from theta_g (fp32, on `device`)."""
    s = cfg.tensors[tensor]
    if s.kind == "const":
        const_rank = sum(1 for t in range(tensor) if cfg.tensors[t].kind == "const")
        c = const_delta_value(cfg, tensor, learner, const_rank)
        return torch.full((s.numel,), c, dtype=torch.float32, device=device)
    g = generator(seed_of(cfg.key, step, tensor, ROLE_LEARNER0 + learner), device)
    return draw_delta(cfg, s, sigma, g, device)


def build_learners(cfg: Config, tensor_ids: Sequence[int], theta_g: torch.Tensor,
                   offsets: Sequence[int], device, step: int = 0,
                   present: Optional[Sequence[int]] = None,
                   sigmas: Optional[Sequence[float]] = None):
    """Learner replicas theta_i = fl32(theta_g - Delta_i) for the listed tensors,
    packed per learner row.  Absent learners' rows are left zero (never read)."""
    specs = [cfg.tensors[t] for t in tensor_ids]
    loffs, stride = pack_offsets([s.numel for s in specs])
    k = cfg.n_learners
    if present is None:
        present = [1] * k
    if sigmas is None:
        all_s = tensor_sigmas(cfg, len(cfg.tensors))
        sigmas = [all_s[t] for t in tensor_ids]
    theta_L = torch.zeros((k, stride), dtype=torch.float32, device=device)
    const_rank = {}
    for t, s in enumerate(cfg.tensors):
        if s.kind == "const":
            const_rank[t] = len(const_rank)
    for j, (t, s, off, loff) in enumerate(zip(tensor_ids, specs, offsets, loffs)):
        tg = theta_g[off:off + s.numel]
        for i in range(k):
            if not present[i]:
                continue
            if s.kind == "const":
                c = const_delta_value(cfg, t, i, const_rank[t])
                delta = torch.full((s.numel,), c, dtype=torch.float32, device=device)
            else:
                g = generator(seed_of(cfg.key, step, t, ROLE_LEARNER0 + i), device)
                delta = draw_delta(cfg, s, sigmas[j], g, device)
            theta_L[i, loff:loff + s.numel] = tg - delta
    return theta_L, loffs, stride


def fragment_inputs(cfg: Config, tensor_ids: Sequence[int], device, step: int = 0,
                    fragment: int = 0) -> StepInputs:
    """All inputs for one merge call over the listed tensors."""
    theta_g, mom, offs = build_global(cfg, tensor_ids, device, step)
    pres = presence(cfg, fragment)
    theta_L, loffs, stride = build_learners(cfg, tensor_ids, theta_g, offs, device, step, pres)
    w = base_weights(cfg)
    w = [wi if p else 0.0 for wi, p in zip(w, pres)]
    tens = [(o, lo, cfg.tensors[t].numel) for o, lo, t in zip(offs, loffs, tensor_ids)]
    return StepInputs(theta_g, mom, theta_L, tens, w, pres, list(tensor_ids), stride)


def custom(key: str, sizes: Sequence[int], n_learners: int, delta: str = "normal",
           delta_scale: float = 1e-3, weights: str = "equal", absent_p: float = 0.0,
           kinds: Optional[Sequence[str]] = None) -> Config:
    """A parameter set of flat tensors of the given sizes (ragged sizes allowed)."""
    kinds = kinds or ["matrix"] * len(sizes)
    specs = tuple(TensorSpec(f"t{i}", (int(n),), k) for i, (n, k) in enumerate(zip(sizes, kinds)))
    return Config(key, f"custom {len(sizes)} tensors, K={n_learners}", specs, n_learners, 1,
                  delta, delta_scale, weights, absent_p=absent_p)
