"""fp64 CPU oracle for segment state caching in linear-attention layers (HYPIC).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are its only users.  The HIP library and its
Python binding never import it.  It shares no code with them; only the seeded
input generators in ``workloads`` feed both.

The arithmetic lives in ``hypic_oracle.c`` (plain loops, fp64, OpenMP across
chains); this module compiles it on demand with gcc and wraps it with numpy.
Every function works on fp64 numpy arrays of ONE chain unless it says
otherwise.  Families: linear, retnet, mamba2, gla, deltanet, gdn, kda.

Sources (HYPIC, codernav.top article, section on linear layers; xix.ai
article, paragraph on linear layers; codernav.top section on seam windows):
the pair (T_C, S(C|0)), the law S(C1.C2) = T(C2) S(C1) + S(C2), and the seam
advance through the first w tokens of each internal segment.

Every function here is pinned by a test against something other than itself
(brute-force matrix products, closed forms, the composition invariant, the
pages' 22% naive-addition figure); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hypic_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libhypic_oracle.so")

FAMILY_ID = {"linear": 0, "retnet": 1, "mamba2": 2, "gla": 3, "deltanet": 4, "gdn": 5, "kda": 6}

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math) into oracle/_build."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_run.argtypes = [i32, i32, i32, i64, P, P, P, P, P, f64, P, P]
        lib.oracle_pair.argtypes = [i32, i32, i32, i64, P, P, P, P, f64, P, P]
        lib.oracle_compose.argtypes = [i32, i32, P, P, P, P]
        lib.oracle_combine.argtypes = [i32, i32, P, P, P, P, P, P]
        lib.oracle_apply_transition.argtypes = [i32, i32, i32, i32, P, P, P, f64, f64]
        lib.oracle_request_batch.argtypes = [i32, i32, i32, i32, i64, i32, P, i32, P, P, P, P, P, P,
                                             P, P, P, P, i32]
        lib.oracle_gate_dim.argtypes = [i32, i32]
        lib.oracle_rope_matrix.argtypes = [i32, f64, f64, P]
        lib.oracle_rerotate.argtypes = [i32, i32, P, P, P, P, P]
        lib.oracle_conv.argtypes = [i64, i32, i32, P, P, i32, P]
        lib.oracle_max_threads.argtypes = []
        _lib = lib
    return _lib


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a) -> Optional[int]:
    return None if a is None else a.ctypes.data


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def apply_transition(family: str, X, k, g=None, beta: float = 1.0, gamma: float = 1.0) -> np.ndarray:
    """A_t X for one token (X is dk x ncols)."""
    X = _f64(X).copy()
    k = _f64(k)
    g = _f64(np.atleast_1d(g)) if g is not None else None
    _load().oracle_apply_transition(FAMILY_ID[family], X.shape[0], X.shape[1], X.shape[1], _ptr(X),
                                    _ptr(k), _ptr(g), float(beta), float(gamma))
    return X


def run(family: str, q, k, v, g=None, beta=None, gamma: float = 1.0, S0=None
        ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token recurrence S_t = A_t S_{t-1} + beta_t k_t v_t^T from S0
    (zero if None).  Returns (final state dk x dv, outputs o_t = S_t^T q_t as n x dv)."""
    k, v = _f64(k), _f64(v)
    n, dk = k.shape
    dv = v.shape[1]
    q = _f64(q) if q is not None else np.zeros((n, dk))
    g, beta = _f64(g), _f64(beta)
    S = np.zeros((dk, dv)) if S0 is None else _f64(S0).copy()
    O = np.zeros((n, dv))
    _load().oracle_run(FAMILY_ID[family], dk, dv, n, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                       float(gamma), _ptr(S), _ptr(O))
    return S, O


def pair(family: str, k, v, g=None, beta=None, gamma: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Cached pair of a segment: (T_C = A_n...A_1 as dk x dk, S(C|0) as dk x dv)."""
    k, v = _f64(k), _f64(v)
    n, dk = k.shape
    dv = v.shape[1]
    g, beta = _f64(g), _f64(beta)
    T = np.zeros((dk, dk))
    S = np.zeros((dk, dv))
    _load().oracle_pair(FAMILY_ID[family], dk, dv, n, _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                        float(gamma), _ptr(T), _ptr(S))
    return T, S


def compose(T, S_C, S_in) -> np.ndarray:
    """S(prefix . C) = T_C S(prefix) + S(C|0)."""
    T, S_C, S_in = _f64(T), _f64(S_C), _f64(S_in)
    out = np.zeros_like(S_C)
    _load().oracle_compose(T.shape[0], S_C.shape[1], _ptr(T), _ptr(S_C), _ptr(S_in), _ptr(out))
    return out


def combine(b, a) -> Tuple[np.ndarray, np.ndarray]:
    """(T_b, S_b) o (T_a, S_a) = (T_b T_a, T_b S_a + S_b): segment a, then b."""
    Tb, Sb = _f64(b[0]), _f64(b[1])
    Ta, Sa = _f64(a[0]), _f64(a[1])
    To = np.zeros_like(Ta)
    So = np.zeros_like(Sb)
    _load().oracle_combine(Tb.shape[0], Sb.shape[1], _ptr(Tb), _ptr(Sb), _ptr(Ta), _ptr(Sa), _ptr(To), _ptr(So))
    return To, So


def request_batch(family: str, bounds, w: int, q, k, v, g=None, beta=None, gamma=None,
                  want_pairs: bool = True, nthreads: int = 0):
    """Reuse path of one request for many chains.

    Token tensors are chain-major fp64: q, k [C][n][dk], v [C][n][dv],
    g [C][n] or [C][n][dk], beta [C][n]; gamma [C] (RetNet).  Segment j spans
    [bounds[j], bounds[j+1]) on the chain's token axis.  Segment 0 is cached
    whole; later segments cache their body [bounds[j]+w, bounds[j+1]) and
    their first w tokens are advanced token by token (seam window).
    Returns dict(T [m][C][dk][dk], S [m][C][dk][dv], state [C][dk][dv],
    O [m][w][C][dv]); T and S are None unless want_pairs."""
    k, v = _f64(k), _f64(v)
    C, n, dk = k.shape
    dv = v.shape[2]
    q = _f64(q) if q is not None else None
    g, beta = _f64(g), _f64(beta)
    gamma = _f64(gamma)
    b = np.ascontiguousarray(np.asarray(bounds, dtype=np.int64))
    m = len(b) - 1
    T = np.zeros((m, C, dk, dk)) if want_pairs else None
    S = np.zeros((m, C, dk, dv)) if want_pairs else None
    state = np.zeros((C, dk, dv))
    O = np.zeros((m, max(w, 1), C, dv))
    rc = _load().oracle_request_batch(FAMILY_ID[family], dk, dv, C, n, m, _ptr(b), w, _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(g), _ptr(beta), _ptr(gamma), _ptr(T), _ptr(S),
                                      _ptr(state), _ptr(O) if w > 0 else None, int(nthreads))
    if rc != 0:
        raise ValueError("every internal segment must be longer than the seam width")
    return {"T": T, "S": S, "state": state, "O": O if w > 0 else None}


def rel_fro(x, ref) -> float:
    """Relative Frobenius error ||x - ref||_F / ||ref||_F (inf-safe for ref = 0);
    infinite when x is not finite, so that a maximum over objects cannot pass
    over a NaN."""
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if not np.isfinite(x).all():
        return float("inf")
    nr = np.linalg.norm(ref)
    d = np.linalg.norm(x - ref)
    return float(d / nr) if nr > 0 else float(d)


# ---- variant patches (codernav.top, linear layers, last paragraph) ----------

def rope_matrix(d: int, p: float, base: float = 10000.0) -> np.ndarray:
    """R(p): channels (i, i + d/2) rotated by p * base^(-2i/d), as a d x d matrix."""
    R = np.zeros((d, d))
    _load().oracle_rope_matrix(d, float(p), float(base), _ptr(R))
    return R


def rerotate(T, S, p: float, base: float = 10000.0) -> Tuple[np.ndarray, np.ndarray]:
    """A pair cached at local positions, moved to offset p: (R T R^T, R S)."""
    T, S = _f64(T), _f64(S)
    dk, dv = S.shape
    R = rope_matrix(dk, p, base)
    To, So = np.zeros((dk, dk)), np.zeros((dk, dv))
    _load().oracle_rerotate(dk, dv, _ptr(R), _ptr(T), _ptr(S), _ptr(To), _ptr(So))
    return To, So


def conv(x, w, act: int = 0) -> np.ndarray:
    """Causal depthwise convolution of raw inputs x [n][d] with taps w [d][K]
    (zero before token 0); act 0: none, 1: SiLU."""
    x, w = _f64(x), _f64(w)
    n, d = x.shape
    y = np.zeros((n, d))
    _load().oracle_conv(n, d, w.shape[1], _ptr(x), _ptr(w), int(act), _ptr(y))
    return y

