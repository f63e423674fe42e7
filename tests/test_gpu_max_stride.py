"""GPU parity at the largest token stride the C ABI accepts (2^24 elements):
the inputs of a few requests' tokens sit 2^24 elements apart (32 MiB per bf16
token row, 64 MiB per fp32 row), so every offset the kernels form inside a
chunk or a seam window is at its 32-bit bound.  Builds, compose (sequential
and tree) and seam outputs against the oracle, per family and dtype."""
import dataclasses

import pytest
import torch

import workloads
from gpu_harness import TOL, assert_close, compare, gpu_request, oracle_request

pytestmark = pytest.mark.gpu

TS = 1 << 24
LAWS = {"gdn": workloads.GDN_LAWS, "deltanet": workloads.GDN_LAWS, "kda": workloads.KDA_LAWS}


def _spread(t):
    """t [n_tok][chains](...) contiguous -> the same values with token stride TS."""
    if t is None:
        return None
    n = t.shape[0]
    m = t[0].numel()
    big = torch.zeros(n, TS, dtype=t.dtype, device=t.device)
    big[:, :m] = t.reshape(n, m)
    return big[:, :m].view(t.shape)


@pytest.mark.parametrize("fam,dtype,d,mode", [("gdn", "bf16", 128, "seq"), ("deltanet", "f32", 32, "tree"),
                                              ("kda", "bf16", 64, "seq"), ("gla", "bf16", 64, "tree"),
                                              ("retnet", "f32", 32, "seq")])
def test_largest_token_stride(fam, dtype, d, mode):
    import state_caching_segment_amd as hy
    lens = [70, 9, 66]   # a full chunk and ragged tails, w = 8 seams on the internal segments
    wl = workloads.make(f"stride_{fam}_{dtype}_{d}", config_id=93, family=fam, dtype=dtype, n_chains=1, d=d,
                        lens=lens, w=8, laws=LAWS.get(fam, workloads.DIAG_LAWS),
                        gamma=workloads.retnet_gammas(1) if fam == "retnet" else None, device="cuda")
    wide = dataclasses.replace(wl, q=_spread(wl.q), k=_spread(wl.k), v=_spread(wl.v), g=_spread(wl.g),
                               beta=_spread(wl.beta))
    assert wide.k.stride(0) == TS and (wide.g is None or wide.g.stride(0) == TS)
    gpu = gpu_request(wide, mode=hy.TREE if mode == "tree" else hy.SEQ)
    ref = oracle_request(wl, [0])
    err = compare(wl, gpu, ref, [0])
    print(wl.name, {k: (f"{v:.2e}" if isinstance(v, float) else v) for k, v in err.items()}, flush=True)
    assert_close(err, TOL[dtype], wl.name)
    del wide, gpu
    torch.cuda.empty_cache()
