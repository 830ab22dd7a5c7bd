"""The allocation-free attention forward (ttt_k_attn_fwd_noalloc, for callers
that cannot allocate device memory) against the workspace entry point
ttt_k_attn_fwd: the same kernels on the same inputs, so the outputs must be
bit for bit equal. Two calls in a row share the static scratch, the second
with a smaller input; an input whose partials exceed the scratch is rejected
before any launch."""
import math

import numpy as np
import pytest
import torch

from long_context_lm_token_amd import binding as bd
from tests.gpu_util import kdt, to_dev

pytestmark = pytest.mark.gpu

SCRATCH_FLOATS = 16 << 20


def case(dtype, B, M, H, hd, pos0, window, seed):
    rng = np.random.default_rng(seed)
    cap = ((window + M + 63) // 64) * 64
    HD = H * hd
    q = to_dev(rng.standard_normal((B * M, HD)), dtype)
    kc = to_dev(rng.standard_normal((B, cap, HD)), dtype)
    vc = to_dev(rng.standard_normal((B, cap, HD)), dtype)
    return cap, q, kc, vc


def run(lib, fn, dtype, B, M, H, hd, pos0, window, nsplit, c, with_ws):
    cap, q, kc, vc = c
    HD = H * hd
    o = torch.full((B * M, HD), 3.0, dtype=dtype, device="cuda")
    lse = torch.full((B, H, M), 3.0, dtype=torch.float32, device="cuda")
    args = [kdt(dtype), bd.ptr(q), bd.ptr(kc), bd.ptr(vc), cap, bd.ptr(o), bd.ptr(lse), B, M, H, hd, pos0, window,
            1.0 / math.sqrt(hd), nsplit]
    if with_ws:
        ws = torch.empty(max(1, nsplit * B * M * (HD + 2 * H)), device="cuda")
        args.append(bd.ptr(ws))
    rc = fn(*args, bd.stream_ptr())
    torch.cuda.synchronize()
    return rc, o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("dtype,hd", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_noalloc_matches_workspace_entry_point(dtype, hd):
    lib = bd.load()
    # a chunk-sized call with 4 key splits (the 3B chunk loop's shape: 12.8 Mi
    # floats of partials), then a smaller few-query call with 16 splits
    shapes = [(1, 1024, 24, 9216 - 1024, 8192, 4), (2, 5, 3, 3000, 2048, 16)]
    if dtype == torch.float32:
        shapes = [(1, 512, 8, 3000, 2048, 4), (2, 5, 3, 3000, 2048, 16)]
    for i, (B, M, H, pos0, window, nsplit) in enumerate(shapes):
        c = case(dtype, B, M, H, hd, pos0, window, seed=10 + i)
        rc, o_ref, l_ref = run(lib, lib.ttt_k_attn_fwd, dtype, B, M, H, hd, pos0, window, nsplit, c, True)
        assert rc == 0, lib.ttt_k_last_error()
        rc, o, l = run(lib, lib.ttt_k_attn_fwd_noalloc, dtype, B, M, H, hd, pos0, window, nsplit, c, False)
        assert rc == 0, lib.ttt_k_last_error()
        np.testing.assert_array_equal(o, o_ref)
        np.testing.assert_array_equal(l, l_ref)
        assert np.isfinite(o).all()


def test_noalloc_rejects_partials_beyond_the_scratch():
    """Every buffer is sized for the call, so only the scratch is too small."""
    lib = bd.load()
    B, M, H, hd, nsplit, window = 2, 1024, 24, 128, 4, 8192   # 2 * 4 * 1024 * (3072 + 48) > 16 Mi
    assert nsplit * B * M * (H * hd + 2 * H) > SCRATCH_FLOATS
    cap, q, kc, vc = case(torch.bfloat16, B, M, H, hd, window, window, seed=3)
    o = torch.full((B * M, H * hd), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, H, M), device="cuda")
    rc = lib.ttt_k_attn_fwd_noalloc(1, bd.ptr(q), bd.ptr(kc), bd.ptr(vc), cap, bd.ptr(o), bd.ptr(lse), B, M, H,
                                    hd, window, window, 0.1, nsplit, bd.stream_ptr())
    assert rc == -1 and b"static scratch" in lib.ttt_k_last_error()
    torch.cuda.synchronize()
    assert (o.float().cpu().numpy() == 3.0).all()   # nothing was launched
