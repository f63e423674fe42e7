"""Seeded synthetic inputs for segment state caching in linear-attention layers.

This module only draws random inputs: token tensors (q, k, v, log-gates,
beta), per-head decay constants and segment boundaries.  It holds none of the
method's arithmetic (no transitions, pairs, composition or seams), so both the
fp64 oracle and the HIP library may consume what it produces.

Shapes follow the HYPIC pages (codernav.top article, section on linear layers:
segments usually longer than 512 tokens, requests of 10^4..10^5 tokens made of
dozens to hundreds of segments) with the per-config distributions below.

Layout of every token tensor: token-major, ``x[token][chain][feature]``.  A
chain is one (layer, head) of one request.  Gates are log-gates ``g`` (the
per-token transition decays by ``exp(g)``): scalar ``g[token][chain]`` or
per-channel ``g[token][chain][dk]``.  ``beta[token][chain]`` is the delta-rule
write strength.

Derived quantities (L2 normalisation, sigmoid, softplus) are computed in the
generation precision (fp64 on the host, fp32 on a GPU) and the result is
rounded once to the storage dtype; consumers read the rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

FAMILIES = ("linear", "retnet", "mamba2", "gla", "deltanet", "gdn", "kda")
# families whose gate is a per-channel vector of length dk
VECTOR_GATE = ("gla", "kda")
# families that take a log-gate tensor at all
GATED = ("mamba2", "gla", "gdn", "kda")
# families with a delta-rule write strength beta
DELTA = ("deltanet", "gdn", "kda")

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "g": 3, "beta": 4, "lengths": 5, "cold": 6}


@dataclass
class Workload:
    name: str
    family: str
    dtype: str                      # "f32" or "bf16": storage dtype of q, k, v, g, beta
    n_chains: int
    dk: int
    dv: int
    w: int                          # seam width (first w tokens of every internal segment)
    q: torch.Tensor                 # [n_tok][n_chains][dk]
    k: torch.Tensor                 # [n_tok][n_chains][dk]
    v: torch.Tensor                 # [n_tok][n_chains][dv]
    g: Optional[torch.Tensor]       # [n_tok][n_chains] or [n_tok][n_chains][dk]
    beta: Optional[torch.Tensor]    # [n_tok][n_chains]
    gamma: Optional[torch.Tensor]   # [n_chains] fp32 (RetNet)
    requests: List[np.ndarray]      # per request: segment boundaries (global token index), len m+1
    cold: List[np.ndarray] = field(default_factory=list)  # per request: bool per segment (True = not cached)

    @property
    def n_tok(self) -> int:
        return int(self.k.shape[0])


def _seed(config_id: int, layer: int, tensor: str) -> int:
    return (config_id * 1_000_003 + layer * 10_007 + TENSOR_ID[tensor] * 101 + 17) & 0x7FFFFFFF


def _gen(device: str, config_id: int, layer: int, tensor: str) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(_seed(config_id, layer, tensor))
    return gen


def _store_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def _work_dtype(device: str) -> torch.dtype:
    # fp64 on the host (exact derived quantities before one rounding), fp32 on a GPU
    return torch.float64 if str(device).startswith("cpu") else torch.float32


def _draw(shape, law: str, device: str, config_id: int, layer: int, tensor: str,
          dtype: str, row_chunk: int = 2048) -> torch.Tensor:
    """Draw a token tensor of `shape` (token axis first) under `law`.

    Laws:  "l2n"  rows ~ N(0, I) then L2-normalised over the last axis
           "n01"  N(0, 1)
           "nsd"  N(0, std 1/sqrt(d)) with d the last-axis size
           "sig"  sigmoid(N(0, 1))
           "sp:mu:sigma"  -softplus(N(mu, sigma))  (a log-gate)
    The token axis is drawn in blocks of `row_chunk` rows so that GB-sized
    tensors never hold a full fp32 temporary.
    """
    gen = _gen(device, config_id, layer, tensor)
    wdt = _work_dtype(device)
    out = torch.empty(shape, dtype=_store_dtype(dtype), device=device)
    n = shape[0]
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        sub = (r1 - r0,) + tuple(shape[1:])
        if law.startswith("sp:"):
            _, mu, sigma = law.split(":")
            x = torch.randn(sub, generator=gen, dtype=wdt, device=device) * float(sigma) + float(mu)
            x = -torch.nn.functional.softplus(x)
        else:
            x = torch.randn(sub, generator=gen, dtype=wdt, device=device)
            if law == "l2n":
                x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True)
            elif law == "nsd":
                x = x / float(np.sqrt(shape[-1]))
            elif law == "sig":
                x = torch.sigmoid(x)
            elif law != "n01":
                raise ValueError(f"unknown law {law}")
        out[r0:r1] = x.to(out.dtype)
    return out


def lognormal_lengths(config_id: int, layer: int, n_tok: int, n_seg: int, min_len: int = 512) -> np.ndarray:
    """Segment lengths: min_len + floor(X_i * extra / sum X), X ~ LogNormal(0, 1),
    with the rounding remainder added to the longest segment so the lengths sum to n_tok."""
    rng = np.random.default_rng([config_id, layer, TENSOR_ID["lengths"]])
    x = rng.lognormal(0.0, 1.0, n_seg)
    extra = n_tok - min_len * n_seg
    if extra < 0:
        raise ValueError("n_tok too small for the minimum length")
    lens = min_len + np.floor(x * extra / x.sum()).astype(np.int64)
    lens[int(np.argmax(lens))] += n_tok - int(lens.sum())
    return lens


def uniform_lengths(config_id: int, layer: int, n_seg: int, lo: int, hi: int) -> np.ndarray:
    rng = np.random.default_rng([config_id, layer, TENSOR_ID["lengths"]])
    return rng.integers(lo, hi + 1, n_seg).astype(np.int64)


def make(name: str, *, config_id: int, family: str, dtype: str, n_chains: int, d: int,
         lens, w: int = 8, laws: Dict[str, str], gamma=None, device: str = "cpu",
         layer: int = 0, n_req: int = 1, n_cold: Optional[int] = None) -> Workload:
    """Build a workload.  `lens` is one list of segment lengths (shared by all
    requests) or a list of per-request lists.  Requests are laid out one after
    another on the token axis."""
    if family not in FAMILIES:
        raise ValueError(family)
    per_req = [np.asarray(l, dtype=np.int64) for l in lens] if isinstance(lens[0], (list, tuple, np.ndarray)) \
        else [np.asarray(lens, dtype=np.int64)] * n_req
    requests, start = [], 0
    for l in per_req:
        b = np.concatenate([[0], np.cumsum(l)]) + start
        requests.append(b.astype(np.int64))
        start = int(b[-1])
    n_tok = start
    dk = dv = d
    q = _draw((n_tok, n_chains, dk), laws["q"], device, config_id, layer, "q", dtype)
    k = _draw((n_tok, n_chains, dk), laws["k"], device, config_id, layer, "k", dtype)
    v = _draw((n_tok, n_chains, dv), laws["v"], device, config_id, layer, "v", dtype)
    g = beta = None
    if family in GATED:
        gshape = (n_tok, n_chains, dk) if family in VECTOR_GATE else (n_tok, n_chains)
        g = _draw(gshape, laws["g"], device, config_id, layer, "g", dtype)
    if family in DELTA:
        beta = _draw((n_tok, n_chains), laws.get("beta", "sig"), device, config_id, layer, "beta", dtype)
    gam = None
    if family == "retnet":
        gam = torch.tensor(np.asarray(gamma, dtype=np.float64), dtype=torch.float32, device=device)
    cold = []
    rng = np.random.default_rng([config_id, layer, TENSOR_ID["cold"]])
    for b in requests:
        m = len(b) - 1
        mask = np.ones(m, dtype=bool)
        if n_cold is not None:
            mask[:] = False
            mask[rng.choice(m, size=n_cold, replace=False)] = True
        cold.append(mask)
    return Workload(name, family, dtype, n_chains, dk, dv, w, q, k, v, g, beta, gam, requests, cold)


GDN_LAWS = {"q": "l2n", "k": "l2n", "v": "n01", "beta": "sig", "g": "sp:-3:0.5"}
SLOW_GDN_LAWS = dict(GDN_LAWS, g="sp:-7:0.5")
KDA_LAWS = {"q": "l2n", "k": "l2n", "v": "n01", "beta": "sig", "g": "sp:-4:1"}
DIAG_LAWS = {"q": "nsd", "k": "nsd", "v": "nsd", "g": "sp:-4:1"}


def retnet_gammas(n_heads: int) -> np.ndarray:
    """gamma_h = 1 - 2^(-5-h): RetNet's multi-scale per-head decays."""
    return 1.0 - 2.0 ** (-5.0 - np.arange(n_heads, dtype=np.float64))


def config(name: str, device: str = "cpu", layer: int = 0, **over) -> Workload:
    """Named workloads.

    c1            gated delta rule, fp32, 1 head, d=16, 2 x 64 tokens
    c1_deltanet   same shapes, DeltaNet (no decay)              (stressor)
    c1_slowgdn    same shapes, gates -softplus(N(-7, 0.5))      (stressor)
    c2            RetNet, fp32, 8 heads, d=64, 8 x 256 tokens
    c3            GLA-style per-channel decay, bf16, 16 heads, d=128, 32 segments U[512, 2048]
    c4            GDN, bf16, 960 chains (30 layers x 32 heads), d=128, one 32768-token request, 48 segments
    c5            KDA, bf16, per layer 32 heads, 16 requests x 100000 tokens x 128 segments, 13 cold each
    Small variants (``*_small``) keep a config's laws at sizes the oracle finishes in seconds.
    """
    if name in ("c1", "c1_deltanet", "c1_slowgdn"):
        fam = "deltanet" if name == "c1_deltanet" else "gdn"
        laws = SLOW_GDN_LAWS if name == "c1_slowgdn" else GDN_LAWS
        kw = dict(config_id=1, family=fam, dtype="f32", n_chains=1, d=16, lens=[64, 64], laws=laws)
    elif name == "c2":
        kw = dict(config_id=2, family="retnet", dtype="f32", n_chains=8, d=64, lens=[256] * 8,
                  laws=DIAG_LAWS, gamma=retnet_gammas(8))
    elif name == "c3":
        kw = dict(config_id=3, family="gla", dtype="bf16", n_chains=16, d=128,
                  lens=uniform_lengths(3, layer, 32, 512, 2048), laws=DIAG_LAWS)
    elif name in ("c4", "c4_deltanet", "c4_slowgdn"):
        fam = "deltanet" if name == "c4_deltanet" else "gdn"
        laws = SLOW_GDN_LAWS if name == "c4_slowgdn" else GDN_LAWS
        kw = dict(config_id=4, family=fam, dtype="bf16", n_chains=960, d=128,
                  lens=lognormal_lengths(4, layer, 32768, 48), laws=laws)
    elif name == "c5":
        lens = [lognormal_lengths(5, layer * 1000 + r, 100000, 128) for r in range(16)]
        kw = dict(config_id=5, family="kda", dtype="bf16", n_chains=32, d=128, lens=lens,
                  laws=KDA_LAWS, n_cold=13)
    else:
        raise KeyError(name)
    kw.update(over)
    return make(name, device=device, layer=layer, **kw)
