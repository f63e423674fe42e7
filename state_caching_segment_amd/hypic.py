"""Python binding of libhypic (argument marshalling only).

Each function has the name and argument order of its C counterpart in
``include/hypic.h``; tensors are torch tensors whose data pointers are passed
through, and a negative status raises ``HypicError`` with the library's own
message.  All compute runs in the HIP kernels of ``libhypic.so``; nothing
here falls back to another implementation: without the built library every
call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhypic.so")

FAMILY = {"linear": 0, "retnet": 1, "mamba2": 2, "gla": 3, "deltanet": 4, "gdn": 5, "kda": 6}
DTYPE = {"f32": 0, "bf16": 1}
SEQ, TREE = 0, 1
OP_BUILD, OP_COMPOSE_SEQ, OP_COMPOSE_TREE, OP_SEAM = 0, 1, 2, 3
STATUS = {0: "HYPIC_OK", -1: "HYPIC_E_INVALID", -2: "HYPIC_E_UNSUPPORTED", -3: "HYPIC_E_WORKSPACE",
          -4: "HYPIC_E_DEVICE"}
EXPORTS = ("hypic_t_elems", "hypic_workspace_bytes", "hypic_segment_build", "hypic_segment_prefill",
           "hypic_compose", "hypic_compose_tree_noalloc", "hypic_seam_advance", "hypic_rerotate",
           "hypic_conv_warmup", "hypic_pair_compact", "hypic_compose_compact", "hypic_store_create", "hypic_store_destroy", "hypic_store_acquire",
           "hypic_store_evict", "hypic_store_stats", "hypic_content_key", "hypic_status_string", "hypic_last_error")
NOALLOC_WORKSPACE_BYTES = 64 << 20  # HYPIC_NOALLOC_WORKSPACE_BYTES


class HypicError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class hypic_layout(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("n_chains", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32)]


class hypic_tokens(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("tok_stride", ctypes.c_int64), ("chain_stride", ctypes.c_int64),
                ("g_tok_stride", ctypes.c_int64), ("g_chain_stride", ctypes.c_int64),
                ("b_tok_stride", ctypes.c_int64), ("b_chain_stride", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH, cache: bool = True) -> ctypes.CDLL:
    """Load libhypic.so from the package directory (raises if it is not built).
    cache=False loads another build of the library (e.g. for a same-process
    A/B timing) without making it the one the calls below use."""
    global _lib
    if cache and _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libhypic is not built ({path} missing); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.hypic_t_elems.argtypes = [i32, i32]
    lib.hypic_t_elems.restype = i64
    lib.hypic_workspace_bytes.argtypes = [P, i32, i32, i64, i32]
    lib.hypic_workspace_bytes.restype = sz
    lib.hypic_segment_build.argtypes = [P, P, i32, P, P, i64, P, P, P, sz, P]
    lib.hypic_segment_build.restype = ctypes.c_int
    lib.hypic_segment_prefill.argtypes = [P, P, i32, P, P, i64, P, P, P, i64, i64, P]
    lib.hypic_segment_prefill.restype = ctypes.c_int
    lib.hypic_compose.argtypes = [P, i32, i32, i32, P, P, i64, P, P, P, P, i32, P, P, P, P, sz, P]
    lib.hypic_compose.restype = ctypes.c_int
    lib.hypic_compose_tree_noalloc.argtypes = [P, i32, i32, P, P, i64, P, P, P, P, i32, P, P, P, P]
    lib.hypic_compose_tree_noalloc.restype = ctypes.c_int
    lib.hypic_seam_advance.argtypes = [P, P, i32, P, i32, P, P, P]
    lib.hypic_seam_advance.restype = ctypes.c_int
    lib.hypic_rerotate.argtypes = [P, i32, P, P, ctypes.c_double, P, P, P, P, P]
    lib.hypic_rerotate.restype = ctypes.c_int
    lib.hypic_conv_warmup.argtypes = [P, P, P, i32, i32, i32, P, i32, P, P, P, P]
    lib.hypic_conv_warmup.restype = ctypes.c_int
    lib.hypic_pair_compact.argtypes = [P, i32, P, P, P, P]
    lib.hypic_pair_compact.restype = ctypes.c_int
    lib.hypic_compose_compact.argtypes = [P, i32, i32, P, P, i64, P, P, P, P, P, i32, P, P, P, P]
    lib.hypic_compose_compact.restype = ctypes.c_int
    lib.hypic_store_create.argtypes = [i64]
    lib.hypic_store_create.restype = P
    lib.hypic_store_destroy.argtypes = [P]
    lib.hypic_store_destroy.restype = None
    lib.hypic_store_acquire.argtypes = [P, i32, P, P, P]
    lib.hypic_store_acquire.restype = ctypes.c_int
    lib.hypic_store_evict.argtypes = [P, ctypes.c_uint64]
    lib.hypic_store_evict.restype = ctypes.c_int
    lib.hypic_store_stats.argtypes = [P, P]
    lib.hypic_store_stats.restype = ctypes.c_int
    lib.hypic_content_key.argtypes = [P, sz]
    lib.hypic_content_key.restype = ctypes.c_uint64
    lib.hypic_status_string.argtypes = [ctypes.c_int]
    lib.hypic_status_string.restype = ctypes.c_char_p
    lib.hypic_last_error.argtypes = []
    lib.hypic_last_error.restype = ctypes.c_char_p
    if cache:
        _lib = lib
    return lib


def use(lib: ctypes.CDLL) -> None:
    """Route the calls below to `lib` (a library returned by load)."""
    global _lib
    _lib = lib


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(rc: int):
    if rc != 0:
        raise HypicError(rc, load().hypic_last_error().decode())


def layout(family: str, in_dtype: str, n_chains: int, dk: int, dv: Optional[int] = None) -> hypic_layout:
    return hypic_layout(FAMILY[family], DTYPE[in_dtype], n_chains, dk, dk if dv is None else dv)


def tokens(q=None, k=None, v=None, g=None, beta=None, gamma=None) -> hypic_tokens:
    """hypic_tokens from token-major tensors x[token][chain][feature] (any strides
    whose feature axis is contiguous); g is [token][chain] or [token][chain][dk],
    beta [token][chain], gamma [chain] fp32."""
    ref = k if k is not None else q
    tok = hypic_tokens()
    tok.q, tok.k, tok.v = _p(q), _p(k), _p(v)
    tok.g, tok.beta, tok.gamma = _p(g), _p(beta), _p(gamma)
    if ref is not None:
        tok.tok_stride, tok.chain_stride = ref.stride(0), ref.stride(1)
    if g is not None:
        tok.g_tok_stride, tok.g_chain_stride = g.stride(0), g.stride(1)
    if beta is not None:
        tok.b_tok_stride, tok.b_chain_stride = beta.stride(0), beta.stride(1)
    return tok


def hypic_t_elems(family: str, dk: int) -> int:
    return int(load().hypic_t_elems(FAMILY[family], dk))


def hypic_workspace_bytes(L: hypic_layout, op: int, n_items: int, max_len: int, w: int = 0) -> int:
    return int(load().hypic_workspace_bytes(ctypes.byref(L), op, n_items, max_len, w))


def hypic_segment_build(L: hypic_layout, x: hypic_tokens, n_seg: int, seg_begin, seg_end, max_seg_len: int,
                        T, S, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(load().hypic_segment_build(ctypes.byref(L), ctypes.byref(x), n_seg, _p(seg_begin), _p(seg_end),
                                      int(max_seg_len), _p(T), _p(S), _p(ws), ws_bytes, _stream(stream)))


def hypic_segment_prefill(L: hypic_layout, x: hypic_tokens, n_seg: int, seg_begin, seg_end, max_seg_len: int,
                          T, S, out, stream=None) -> None:
    """out: token-major [token][chain][dv] tensor (any strides with a contiguous
    feature axis) in the input dtype."""
    _check(load().hypic_segment_prefill(ctypes.byref(L), ctypes.byref(x), n_seg, _p(seg_begin), _p(seg_end),
                                        int(max_seg_len), _p(T), _p(S), _p(out), out.stride(0), out.stride(1),
                                        _stream(stream)))


def hypic_compose(L: hypic_layout, mode: int, n_req: int, max_list_len: int, list_off, pair_id, n_slots: int,
                  T, S, seam: Optional[hypic_tokens], seam_begin, w: int, state, o, prefix_states=None, ws=None,
                  ws_bytes: int = 0, stream=None) -> None:
    _check(load().hypic_compose(ctypes.byref(L), mode, n_req, max_list_len, _p(list_off), _p(pair_id), n_slots,
                                _p(T), _p(S), ctypes.byref(seam) if seam is not None else None, _p(seam_begin), w,
                                _p(state), _p(o), _p(prefix_states), _p(ws), ws_bytes, _stream(stream)))


def hypic_compose_tree_noalloc(L: hypic_layout, n_req: int, max_list_len: int, list_off, pair_id, n_slots: int,
                               T, S, seam: Optional[hypic_tokens], seam_begin, w: int, state, o,
                               prefix_states=None, stream=None) -> None:
    _check(load().hypic_compose_tree_noalloc(ctypes.byref(L), n_req, max_list_len, _p(list_off), _p(pair_id),
                                             n_slots, _p(T), _p(S), ctypes.byref(seam) if seam is not None else None,
                                             _p(seam_begin), w, _p(state), _p(o), _p(prefix_states),
                                             _stream(stream)))


def hypic_seam_advance(L: hypic_layout, x: hypic_tokens, n_items: int, tok_begin, w: int, state, o,
                       stream=None) -> None:
    _check(load().hypic_seam_advance(ctypes.byref(L), ctypes.byref(x), n_items, _p(tok_begin), w, _p(state), _p(o),
                                     _stream(stream)))


def hypic_rerotate(L: hypic_layout, n_items: int, slot, offset, rope_base: float, T, S, T_out, S_out,
                   stream=None) -> None:
    _check(load().hypic_rerotate(ctypes.byref(L), n_items, _p(slot), _p(offset), float(rope_base), _p(T), _p(S),
                                 _p(T_out), _p(S_out), _stream(stream)))


def hypic_conv_warmup(L: hypic_layout, raw: hypic_tokens, taps, conv_k: int, act: int, n_items: int, tok_begin,
                      w: int, q_out, k_out, v_out, stream=None) -> None:
    _check(load().hypic_conv_warmup(ctypes.byref(L), ctypes.byref(raw), _p(taps), conv_k, act, n_items,
                                    _p(tok_begin), w, _p(q_out), _p(k_out), _p(v_out), _stream(stream)))


def hypic_pair_compact(L: hypic_layout, n_slots: int, T, Tc, Tscale, stream=None) -> None:
    _check(load().hypic_pair_compact(ctypes.byref(L), n_slots, _p(T), _p(Tc), _p(Tscale), _stream(stream)))


def hypic_compose_compact(L: hypic_layout, n_req: int, max_list_len: int, list_off, pair_id, n_slots: int, Tc,
                          Tscale, S, seam: Optional[hypic_tokens], seam_begin, w: int, state, o, prefix_states=None,
                          stream=None) -> None:
    _check(load().hypic_compose_compact(ctypes.byref(L), n_req, max_list_len, _p(list_off), _p(pair_id), n_slots,
                                        _p(Tc), _p(Tscale), _p(S), ctypes.byref(seam) if seam is not None else None,
                                        _p(seam_begin), w, _p(state), _p(o), _p(prefix_states), _stream(stream)))


class Store:
    """A pair store (hypic_store_*): content keys to slots of a caller-owned
    pool of pairs."""

    def __init__(self, n_slots: int):
        self._lib = load()
        self.h = self._lib.hypic_store_create(int(n_slots))
        if not self.h:
            raise HypicError(-1, f"cannot create a store of {n_slots} slots")
        self.n_slots = int(n_slots)

    def acquire(self, keys):
        """-> (slots int32 array, miss bool array); raises HypicError."""
        import numpy as np
        k = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
        slots = np.empty(len(k), np.int32)
        miss = np.empty(len(k), np.uint8)
        rc = self._lib.hypic_store_acquire(self.h, len(k), k.ctypes.data, slots.ctypes.data, miss.ctypes.data)
        if rc < 0:
            raise HypicError(rc, "store acquire refused (more distinct keys than slots)" if rc == -3 else "bad store call")
        return slots, miss.astype(bool)

    def evict(self, key) -> bool:
        return self._lib.hypic_store_evict(self.h, int(key)) == 1

    def stats(self):
        import numpy as np
        out = np.zeros(4, np.int64)
        _check(self._lib.hypic_store_stats(self.h, out.ctypes.data))
        return dict(zip(("entries", "hits", "misses", "evictions"), (int(x) for x in out)))

    def close(self):
        if self.h:
            self._lib.hypic_store_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def hypic_content_key(data) -> int:
    """FNV-1a 64 of a bytes-like object or a numpy array's bytes."""
    import numpy as np
    b = np.ascontiguousarray(data).tobytes() if not isinstance(data, (bytes, bytearray)) else bytes(data)
    buf = ctypes.create_string_buffer(b, len(b))
    return int(load().hypic_content_key(buf, len(b)))


def hypic_status_string(status: int) -> str:
    return load().hypic_status_string(status).decode()


def hypic_last_error() -> str:
    return load().hypic_last_error().decode()
