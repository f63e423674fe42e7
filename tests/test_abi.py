"""C ABI checks that need no GPU: the library loads, exports every function
include/hypic.h declares, and rejects bad arguments with the documented
status before making any HIP call.  Also the host-side request plan."""
import ctypes
import os
import re

import numpy as np
import pytest

import state_caching_segment_amd as hy
from state_caching_segment_amd.plan import request_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hypic.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hypic_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = hy.load()
    names = declared()
    assert set(names) == set(hy.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_t_elems_and_status_strings():
    assert hy.hypic_t_elems("retnet", 64) == 1
    assert hy.hypic_t_elems("gla", 64) == 64
    assert hy.hypic_t_elems("kda", 128) == 128 * 128
    assert hy.hypic_status_string(0) == "ok"
    assert hy.hypic_status_string(-2) == "unsupported"
    assert hy.load().hypic_t_elems(99, 16) == 0


def _fake_tokens(family, dtype="bf16", align=0, ts=None, cs=128):
    base = 1 << 20  # never dereferenced: validation fails or returns before any HIP call
    t = hy.hypic_tokens()
    t.q = t.k = t.v = base + align
    t.g = base if family in ("mamba2", "gdn", "gla", "kda") else None
    t.beta = base if family in ("deltanet", "gdn", "kda") else None
    t.gamma = base if family == "retnet" else None
    t.tok_stride = ts if ts is not None else 4 * cs
    t.chain_stride = cs
    t.g_tok_stride, t.g_chain_stride = 4 * 128, 128
    t.b_tok_stride, t.b_chain_stride = 4, 1
    return t


# a stand-in device pointer (never dereferenced: every call here fails or
# returns before a launch), aligned as the calls require
P = 256


def expect(status, fn, *args):
    with pytest.raises(hy.HypicError) as e:
        fn(*args)
    assert e.value.status == status, str(e.value)
    assert hy.hypic_last_error() != ""


def test_build_validation():
    L = hy.layout("gdn", "bf16", 4, 128)
    x = _fake_tokens("gdn")
    b = hy.hypic_segment_build
    expect(-1, b, hy.layout("gdn", "bf16", 4, 100), x, 1, 8, 8, 10, 8, 8)       # bad dk
    expect(-2, b, hy.layout("gdn", "bf16", 4, 128, 64), x, 1, 8, 8, 10, 8, 8)   # dv != dk
    expect(-1, b, hy.layout("gdn", "bf16", 0, 128), x, 1, 8, 8, 10, 8, 8)      # no chains
    bad = hy.hypic_layout(9, 1, 4, 128, 128)
    expect(-1, b, bad, x, 1, 8, 8, 10, 8, 8)                                    # family
    bad = hy.hypic_layout(5, 7, 4, 128, 128)
    expect(-1, b, bad, x, 1, 8, 8, 10, 8, 8)                                    # dtype
    expect(-1, b, L, _fake_tokens("gdn", align=2), 1, 8, 8, 10, 8, 8)          # misaligned k
    expect(-1, b, L, _fake_tokens("gdn", ts=4 * 128 + 1), 1, 8, 8, 10, 8, 8)   # stride not 16 B
    expect(-1, b, L, _fake_tokens("gdn", cs=64), 1, 8, 8, 10, 8, 8)           # chain stride < dk
    x2 = _fake_tokens("gdn")
    x2.g = None
    expect(-1, b, L, x2, 1, 8, 8, 10, 8, 8)                                    # missing gate
    x3 = _fake_tokens("gdn")
    x3.beta = None
    expect(-1, b, L, x3, 1, 8, 8, 10, 8, 8)                                    # missing beta
    expect(-1, b, hy.layout("retnet", "f32", 4, 128), _fake_tokens("linear", "f32"), 1, 8, 8, 10, 8, 8)  # gamma
    expect(-1, b, L, x, -1, 8, 8, 10, 8, 8)                                    # n_seg < 0
    expect(-1, b, L, x, 2, None, 8, 10, 8, 8)                                  # NULL begin
    expect(-1, b, L, x, 2, 8, 8, 10, None, 8)                                  # NULL T
    b(L, x, 0, None, None, 0, None, None)  # nothing to do: OK without touching the device


def test_compose_and_seam_validation():
    L = hy.layout("gdn", "bf16", 4, 64)
    x = _fake_tokens("gdn", cs=64)
    c = hy.hypic_compose
    expect(-1, c, L, 5, 1, 2, P, P, 2, P, P, None, None, 0, P, None)           # mode
    expect(-1, c, L, hy.SEQ, 1, 2, P, P, 2, P, P, x, P, -1, P, P)              # w < 0
    expect(-1, c, L, hy.SEQ, 1, 2, None, P, 2, P, P, None, None, 0, P, None)   # NULL list
    expect(-1, c, L, hy.SEQ, 1, 2, P, P, 2, P, P, x, None, 8, P, P)            # seams without begin
    expect(-1, c, L, hy.SEQ, 1, 2, P, P, 2, P, P, x, P, 8, P, None)            # seams without outputs
    xq = _fake_tokens("gdn", cs=64)
    xq.q = None
    expect(-1, c, L, hy.SEQ, 1, 2, P, P, 2, P, P, xq, P, 8, P, P)              # seams need q
    expect(-3, c, L, hy.TREE, 1, 2, P, P, 2, P, P, None, None, 0, P, None)     # tree needs a workspace
    # pairs 16-byte, states and outputs 4-byte aligned
    expect(-1, c, L, hy.SEQ, 1, 2, P, P, 2, P + 8, P, None, None, 0, P, None)  # T
    expect(-1, c, L, hy.SEQ, 1, 2, P, P, 2, P, P + 8, None, None, 0, P, None)  # S
    expect(-1, c, L, hy.SEQ, 1, 2, P, P, 2, P, P, None, None, 0, P + 2, None)  # state
    expect(-1, c, L, hy.SEQ, 1, 2, P, P, 2, P, P, x, P, 8, P, P + 2)           # outputs
    c(L, hy.SEQ, 0, 0, None, None, 0, None, None, None, None, 0, None, None)   # empty: OK
    s = hy.hypic_seam_advance
    expect(-1, s, L, x, 2, None, 8, 8, 8)
    expect(-1, s, L, x, 2, 8, -3, 8, 8)
    s(L, x, 0, None, 8, None, None)


def test_token_stride_bound():
    """Token strides above 2^24 elements are refused by every call that reads
    tokens: offsets inside a chunk or seam window are 32-bit in the kernels."""
    L = hy.layout("gdn", "f32", 4, 64)
    big = (1 << 24) + 64
    expect(-2, hy.hypic_segment_build, L, _fake_tokens("gdn", "f32", ts=big, cs=64), 1, 8, 8, 10, 8, 8)
    expect(-2, hy.hypic_compose, L, hy.SEQ, 1, 2, P, P, 2, P, P, _fake_tokens("gdn", "f32", ts=big, cs=64), P, 8, P, P)
    expect(-2, hy.hypic_seam_advance, L, _fake_tokens("gdn", "f32", ts=big, cs=64), 2, 8, 8, 8, 8)
    xg = _fake_tokens("gdn", "f32", cs=64)
    xg.g_tok_stride = big
    expect(-2, hy.hypic_compose, L, hy.SEQ, 1, 2, P, P, 2, P, P, xg, P, 8, P, P)
    xb = _fake_tokens("gdn", "f32", cs=64)
    xb.b_tok_stride = big
    expect(-2, hy.hypic_seam_advance, L, xb, 2, 8, 8, 8, 8)
    # at the bound the checks pass: the fault-injection switch stops the call before any launch
    ok = _fake_tokens("gdn", "f32", ts=1 << 24, cs=64)
    os.environ["HYPIC_FAULT_INJECT"] = "all"
    try:
        expect(-4, hy.hypic_compose, L, hy.SEQ, 1, 2, P, P, 2, P, P, ok, P, 8, P, P)
    finally:
        del os.environ["HYPIC_FAULT_INJECT"]


def test_fault_injection():
    """HYPIC_FAULT_INJECT fails a valid call with HYPIC_E_DEVICE after its
    arguments are checked and before anything is enqueued; bad arguments still
    report their own status first."""
    L = hy.layout("gdn", "bf16", 4, 64)
    x = _fake_tokens("gdn", cs=64)
    try:
        for val in ("1", "all", "build"):
            os.environ["HYPIC_FAULT_INJECT"] = val
            expect(-4, hy.hypic_segment_build, L, x, 1, 8, 8, 10, 8, 8)
            assert "fault injected" in hy.hypic_last_error()
            expect(-1, hy.hypic_segment_build, L, x, -1, 8, 8, 10, 8, 8)   # validation first
        for val in ("1", "compose"):
            os.environ["HYPIC_FAULT_INJECT"] = val
            expect(-4, hy.hypic_compose, L, hy.SEQ, 1, 2, P, P, 2, P, P, x, P, 8, P, P)
            # tree mode: the workspace check comes before the injected fault
            expect(-3, hy.hypic_compose, L, hy.TREE, 1, 2, P, P, 2, P, P, None, None, 0, P, None)
            expect(-4, hy.hypic_compose, L, hy.TREE, 1, 2, P, P, 2, P, P, None, None, 0, P, None, None, P,
                   1 << 30)
        for val in ("1", "seam"):
            os.environ["HYPIC_FAULT_INJECT"] = val
            expect(-4, hy.hypic_seam_advance, L, x, 2, 8, 8, 8, 8)
        os.environ["HYPIC_FAULT_INJECT"] = "seam"   # other calls unaffected: they reach their own checks
        expect(-1, hy.hypic_compose, L, hy.SEQ, 1, 2, P, P, 2, P, P, x, P, -1, P, P)
        os.environ["HYPIC_FAULT_INJECT"] = "0"
        expect(-1, hy.hypic_seam_advance, L, x, 2, 8, -3, 8, 8)
    finally:
        os.environ.pop("HYPIC_FAULT_INJECT", None)


def test_workspace_query():
    L = hy.layout("gdn", "bf16", 4, 128)
    assert hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_SEQ, 4, 48, 8) == 0
    assert hy.hypic_workspace_bytes(L, hy.OP_BUILD, 4, 48, 8) == 0
    # tree: 3 block-aggregate arrays of n_req x NB x chains x dk^2 fp32, plus seam queries; 16 chains
    # cannot fill the GPU, so blocks of ceil(sqrt(48 / 2)) = 5 entries, NB = 10
    # (the last term: the block entry offsets, n_req x NB + 1 int32, in whole 256-byte units)
    nb, agg = 10, 4 * 10 * 4 * 128 * 128 * 4
    pv = 4 * 48 * 8 * 4 * 128 * 4
    assert hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, 4, 48, 8) == 3 * agg + pv + 256
    assert hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, 4, 48, 0) == 3 * agg + 256
    assert hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, 4, 48, -1) == 0
    assert hy.hypic_workspace_bytes(hy.layout("gdn", "bf16", 4, 100), hy.OP_COMPOSE_TREE, 4, 48, 8) == 0
    # 16 requests x 32 chains (one KDA layer) of 128 entries: the chains fill the GPU, so 4 blocks
    # of 32 entries (8 block workgroups per compute unit) instead of 11 blocks of 12
    L = hy.layout("kda", "bf16", 32, 128)
    agg = 16 * 4 * 32 * 128 * 128 * 4
    pv = 16 * 128 * 8 * 32 * 128 * 4
    assert hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, 16, 128, 8) == 3 * agg + pv + 512
    # one request of 32 entries on 16 GLA chains: 16 x 6 blocks cannot fill the GPU, so blocks of
    # ceil(sqrt(32 / 2)) = 4 entries, NB = 8 (GLA's aggregates are still dk x dk fp32 states)
    L = hy.layout("gla", "bf16", 16, 128)
    assert hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, 1, 32, 0) == 3 * (1 * 8 * 16 * 128 * 128 * 4) + 256
    # 5000 entries on 512 chains: longer blocks are capped at 64 entries, NB = ceil(5000 / 64) = 79
    L = hy.layout("gdn", "bf16", 32, 64)
    assert hy.hypic_workspace_bytes(L, hy.OP_COMPOSE_TREE, 16, 5000, 0) == 3 * (16 * 79 * 32 * 64 * 64 * 4) + 5120


def test_request_plan():
    reqs = [np.array([0, 100, 150, 300]), np.array([300, 420, 500])]
    p = request_plan(reqs, 8)
    assert p.n_slots == 5 and p.n_req == 2
    assert p.seg_begin.tolist() == [0, 108, 158, 300, 428]
    assert p.seg_end.tolist() == [100, 150, 300, 420, 500]
    assert p.seam_begin.tolist() == [-1, 100, 150, -1, 420]
    assert p.list_off.tolist() == [0, 3, 5]
    assert p.max_seg_len == 142 and p.max_list_len == 3
    p0 = request_plan(reqs, 0)
    assert p0.seg_begin.tolist() == [0, 100, 150, 300, 420] and (p0.seam_begin == -1).all()
    with pytest.raises(ValueError):
        request_plan([np.array([0, 100, 108])], 8)
    assert p.seg_index.tolist() == [0, 1, 2, 3, 4]


def test_request_plan_longest_first():
    """Slots numbered by decreasing body length; every entry still reaches the
    same token range through pair_id, and nothing else changes."""
    rng = np.random.default_rng(5)
    reqs, t = [], 0
    for _ in range(4):
        b = np.concatenate([[t], t + np.cumsum(rng.integers(20, 300, size=rng.integers(1, 7)))])
        reqs.append(b)
        t = int(b[-1])
    p = request_plan(reqs, 8)
    q = request_plan(reqs, 8, slot_order="longest_first")
    lens = q.seg_end - q.seg_begin
    assert (np.diff(lens) <= 0).all()
    assert sorted(q.seg_index.tolist()) == list(range(p.n_slots))
    assert (q.seg_begin == p.seg_begin[q.seg_index]).all() and (q.seg_end == p.seg_end[q.seg_index]).all()
    assert (q.seg_begin[q.pair_id] == p.seg_begin[p.pair_id]).all()
    assert (q.seg_end[q.pair_id] == p.seg_end[p.pair_id]).all()
    assert (q.list_off == p.list_off).all() and (q.seam_begin == p.seam_begin).all()
    with pytest.raises(ValueError):
        request_plan(reqs, 8, slot_order="random")


def test_prefill_output_layout_validation():
    """hypic_segment_prefill refuses an output it cannot write in four-element
    row pieces (strides not multiples of 4 elements, or d_out not 8-byte
    aligned), before any HIP call."""
    L = hy.layout("gdn", "bf16", 4, 128)
    x = _fake_tokens("gdn", "bf16")
    fn = hy.load().hypic_segment_prefill
    base = 1 << 21
    args = lambda out, ts, cs: (ctypes.byref(L), ctypes.byref(x), 1, ctypes.c_void_p(base), ctypes.c_void_p(base),
                                64, ctypes.c_void_p(base), ctypes.c_void_p(base), ctypes.c_void_p(out), ts, cs, None)
    assert fn(*args(base + 4, 512, 128)) == -1    # d_out misaligned
    assert fn(*args(base, 514, 128)) == -1        # token stride
    assert fn(*args(base, 512, 130)) == -1        # chain stride


def test_variant_calls_validation():
    """hypic_rerotate and hypic_conv_warmup reject bad arguments before any
    HIP call; families whose per-channel decay does not commute with the
    rotation are refused."""
    rr = hy.hypic_rerotate
    L = hy.layout("gdn", "f32", 4, 64)
    expect(-2, rr, hy.layout("gla", "bf16", 4, 64), 1, 8, 8, 10000.0, 16, 16, 16, 16)
    expect(-2, rr, hy.layout("kda", "bf16", 4, 64), 1, 8, 8, 10000.0, 16, 16, 16, 16)
    expect(-1, rr, L, 1, 8, 8, 1.0, 16, 16, 16, 16)           # base not above 1
    expect(-1, rr, L, -1, 8, 8, 10000.0, 16, 16, 16, 16)      # n_items < 0
    expect(-1, rr, L, 1, None, 8, 10000.0, 16, 16, 16, 16)    # NULL slot
    expect(-1, rr, L, 1, 8, 8, 10000.0, 16, 16, 18, 16)       # misaligned output
    rr(L, 0, None, None, 10000.0, None, None, None, None)     # nothing to do
    cw = hy.hypic_conv_warmup
    x = _fake_tokens("gdn", "f32", cs=64)
    expect(-2, cw, L, x, 16, 9, 1, 1, 8, 8, 16, 16, 16)       # conv_k > 8
    expect(-2, cw, L, x, 16, 0, 1, 1, 8, 8, 16, 16, 16)       # conv_k < 1
    expect(-1, cw, L, x, 16, 4, 2, 1, 8, 8, 16, 16, 16)       # act
    expect(-1, cw, L, x, None, 4, 1, 1, 8, 8, 16, 16, 16)     # NULL taps
    xq = _fake_tokens("gdn", "f32", cs=64)
    xq.q = None
    expect(-1, cw, L, xq, 16, 4, 1, 1, 8, 8, 16, 16, 16)      # raw q required
    cw(L, x, None, 4, 1, 0, None, 8, None, None, None)        # nothing to do
    expect(-1, cw, L, _fake_tokens("gdn", "f32", align=4, cs=64), 16, 4, 1, 1, 8, 8, 16, 16, 16)  # raw misaligned
    expect(-1, cw, L, _fake_tokens("gdn", "f32", cs=66), 16, 4, 1, 1, 8, 8, 16, 16, 16)  # raw stride
    expect(-1, cw, L, x, 16, 4, 1, 1, 8, 8, 16, 24, 16)       # output misaligned
    os.environ["HYPIC_FAULT_INJECT"] = "rerotate"
    try:
        expect(-4, rr, L, 1, 8, 8, 10000.0, 16, 16, 16, 16)
        os.environ["HYPIC_FAULT_INJECT"] = "conv"
        expect(-4, cw, L, x, 16, 4, 1, 1, 8, 8, 16, 16, 16)
    finally:
        del os.environ["HYPIC_FAULT_INJECT"]


def test_compact_pair_validation():
    """hypic_pair_compact and hypic_compose_compact refuse what they cannot
    run, and misaligned pointers, before any launch; with aligned stand-in
    pointers the checks pass and the fault-injection switch stops the call."""
    L = hy.layout("gdn", "bf16", 4, 128)
    pc, cc = hy.hypic_pair_compact, hy.hypic_compose_compact
    expect(-2, pc, hy.layout("gla", "bf16", 4, 128), 2, P, P, P)               # diagonal T
    expect(-1, pc, L, -1, P, P, P)                                             # n_slots < 0
    expect(-1, pc, L, 2, None, P, P)                                           # NULL T
    expect(-1, pc, L, 2, P + 8, P, P)                                          # T not 16-byte aligned
    expect(-1, pc, L, 2, P, P + 4, P)                                          # compact T not 8-byte aligned
    pc(L, 0, None, None, None)                                                 # nothing to do
    expect(-2, cc, hy.layout("kda", "bf16", 4, 128), 1, 2, P, P, 2, P, P, P, None, None, 0, P, None)
    expect(-2, cc, hy.layout("gdn", "f32", 4, 128), 1, 2, P, P, 2, P, P, P, None, None, 0, P, None)
    expect(-1, cc, L, 1, 2, P, P, 2, None, P, P, None, None, 0, P, None)      # NULL compact T
    expect(-1, cc, L, 1, 2, P, P, 2, P + 4, P, P, None, None, 0, P, None)     # compact T misaligned
    expect(-1, cc, L, 1, 2, P, P, 2, P, P, P + 8, None, None, 0, P, None)     # S misaligned
    expect(-1, cc, L, 1, 2, P, P, 2, P, P, P, None, None, 0, P + 2, None)     # state misaligned
    x = _fake_tokens("gdn", cs=128)
    expect(-1, cc, L, 1, 2, P, P, 2, P, P, P, x, P, 8, P, None)               # seams without outputs
    os.environ["HYPIC_FAULT_INJECT"] = "all"
    try:
        expect(-4, pc, L, 2, P, P, P)
        expect(-4, cc, L, 1, 2, P, P, 2, P, P, P, x, P, 8, P, P)
    finally:
        del os.environ["HYPIC_FAULT_INJECT"]
