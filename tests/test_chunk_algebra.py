"""The chunked UT/WY form used by the kernels equals the token-by-token oracle
(fp64, CPU).  Chunk sizes 1, 8, 64 and lengths with ragged chunk tails."""
import numpy as np
import pytest

import oracle
from chunk_model import chunk_pair, chunk_pair_folded, chunk_pair_kda_inv, chunk_run

FAMS = ["linear", "retnet", "mamba2", "gla", "deltanet", "gdn", "kda"]


def _inputs(rng, fam, n, dk, dv):
    k = rng.normal(size=(n, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    q = rng.normal(size=(n, dk))
    v = rng.normal(size=(n, dv))
    g = None
    if fam in ("mamba2", "gdn"):
        g = -np.log1p(np.exp(rng.normal(-3, 0.5, size=n)))
    elif fam in ("gla", "kda"):
        g = -np.log1p(np.exp(rng.normal(-4, 1.0, size=(n, dk))))
    beta = 1 / (1 + np.exp(-rng.normal(size=n))) if fam in ("deltanet", "gdn", "kda") else None
    return q, k, v, g, beta, (0.97 if fam == "retnet" else 1.0)


@pytest.mark.parametrize("fam", FAMS)
@pytest.mark.parametrize("c", [1, 8, 64])
def test_chunk_pair_matches_oracle(fam, c):
    rng = np.random.default_rng(50 + FAMS.index(fam) * 3 + c)
    for n in (1, 9, 64, 65, 150):
        q, k, v, g, beta, gamma = _inputs(rng, fam, n, 8, 6)
        T, S = oracle.pair(fam, k, v, g, beta, gamma)
        Tc, Sc = chunk_pair(fam, k, v, g, beta, gamma, c)
        assert oracle.rel_fro(Tc, T) < 1e-11 and oracle.rel_fro(Sc, S) < 1e-11, (n, c)


@pytest.mark.parametrize("fam", FAMS)
@pytest.mark.parametrize("c", [8, 64])
def test_chunk_outputs_match_oracle(fam, c):
    rng = np.random.default_rng(90 + FAMS.index(fam))
    q, k, v, g, beta, gamma = _inputs(rng, fam, 77, 8, 6)
    S0 = rng.normal(size=(8, 6))
    S, O = oracle.run(fam, q, k, v, g, beta, gamma, S0)
    Sc, Oc = chunk_run(fam, q, k, v, g, beta, gamma, S0, c)
    assert oracle.rel_fro(Sc, S) < 1e-11
    assert oracle.rel_fro(Oc, O) < 1e-11


@pytest.mark.parametrize("fam", ["deltanet", "gdn"])
@pytest.mark.parametrize("law", ["moderate", "strong"])
def test_folded_decay_form_matches_oracle(fam, law):
    """The decay-folded block solve of the bf16 dense build equals the oracle,
    also under gates strong enough that exp(Gam_c) underflows fp32."""
    rng = np.random.default_rng(130 + (fam == "gdn") * 2 + (law == "strong"))
    for n in (1, 17, 64, 65, 150):
        q, k, v, g, beta, gamma = _inputs(rng, fam, n, 8, 6)
        if fam == "gdn" and law == "strong":
            g = -np.log1p(np.exp(rng.normal(1.5, 0.5, size=n)))
        T, S = oracle.pair(fam, k, v, g, beta, gamma)
        Tc, Sc = chunk_pair_folded(fam, k, v, g, beta)
        assert oracle.rel_fro(Tc, T) < 1e-11 or np.linalg.norm(T) < 1e-200, (n, law)
        assert oracle.rel_fro(Sc, S) < 1e-11, (n, law)


def test_gdn_transition_is_decay_times_deltanet():
    """With a scalar gate per token the decay commutes with every erasure, so
    the oracle's GDN T of a segment is exp(sum of its log-gates) times its
    DeltaNet T of the same keys and betas (a closed form tying the two
    families' transition products together)."""
    rng = np.random.default_rng(77)
    for n in (1, 9, 64, 65, 300):
        _, k, v, g, beta, _ = _inputs(rng, "gdn", n, 8, 6)
        T, _ = oracle.pair("gdn", k, v, g, beta)
        Tu, _ = oracle.pair("deltanet", k, v, None, beta)
        assert oracle.rel_fro(np.exp(g.sum()) * Tu, T) < 1e-12, n


@pytest.mark.parametrize("law", ["c5", "strong"])
def test_kda_inverse_decay_form_matches_oracle(law):
    """The bf16 KDA build's form (Gram as K_L K_i^T without reference tokens,
    update as diag(exp Gam_c)(X + K_i^T R)) equals the oracle, also with
    per-channel gates strong enough that exp(-Gam) reaches e^60 in a chunk."""
    rng = np.random.default_rng(140 + (law == "strong"))
    for n in (1, 17, 32, 33, 150):
        q, k, v, g, beta, gamma = _inputs(rng, "kda", n, 8, 6)
        if law == "strong":
            g = -np.log1p(np.exp(rng.normal(0.5, 0.3, size=(n, 8))))   # about -1 per token
        T, S = oracle.pair("kda", k, v, g, beta)
        Tc, Sc = chunk_pair_kda_inv(k, v, g, beta)
        assert oracle.rel_fro(Tc, T) < 1e-10 and oracle.rel_fro(Sc, S) < 1e-10, (n, law)
