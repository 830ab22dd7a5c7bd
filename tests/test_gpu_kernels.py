"""Kernel-level parity: each HIP kernel of the hot path against the oracle's
definition of the same operation (fp64, on the same bf16/fp32 inputs)."""
import math

import numpy as np
import pytest
import torch

from long_context_lm_token_amd import binding as bd
from oracle import ttt_oracle as O
from tests.gpu_util import kdt, to_dev

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.bfloat16]


def rnd(shape, seed, dtype, scale=1.0):
    a = np.random.default_rng(seed).standard_normal(shape) * scale
    t = torch.as_tensor(a, dtype=torch.float32).to(dtype)
    return t.float().numpy().astype(np.float64), t.cuda()


def sync():
    torch.cuda.synchronize()


# ------------------------------- GEMM ---------------------------------------

def run_gemm(dtype, epi, M, N, K, batch=1, out_f32=True, lr=0.0, tile=0, ws_elems=0, sr_seed=0):
    """C = A . B^T with both operands K-contiguous, against fp64 numpy."""
    lib = bd.load()
    A, Ad = rnd((batch, M, K), 1, dtype)
    Bm, Bd = rnd((batch, N, K), 2, dtype)
    ref = np.einsum("zmk,znk->zmn", A, Bm)
    R = Rd = Wm = Wd = C2 = None
    cdt = torch.float32 if (out_f32 or epi == 1) else dtype
    C = torch.zeros((batch, M, N), dtype=cdt, device="cuda")
    if epi == 1:
        R, Rd = rnd((batch, M, N), 3, torch.float32)
        ref = R + ref
    if epi == 2:
        Wm, Wd = rnd((batch, M, N), 4, torch.float32)
        ref = Wm - lr * ref
        C = torch.zeros((batch, M, N), dtype=dtype, device="cuda")
        C2 = torch.zeros((batch, N, M), dtype=dtype, device="cuda")
    ws = torch.zeros(max(ws_elems, 1), device="cuda") if ws_elems else None
    lib.ttt_k_gemm_tile(tile)
    try:
        rc = lib.ttt_k_gemm(kdt(dtype), epi, int(out_f32), M, N, K, bd.ptr(Ad), K, M * K, bd.ptr(Bd), K, N * K,
                            bd.ptr(C), N, M * N, bd.ptr(C2), M, M * N, bd.ptr(Rd), N, M * N, bd.ptr(Wd), N, M * N,
                            lr, sr_seed, batch, bd.ptr(ws), ws_elems, bd.stream_ptr())
        bd.check(rc, kernel=True)
        sync()
    finally:
        lib.ttt_k_gemm_tile(0)
    return (ref, C.float().cpu().numpy(), (Wd.cpu().numpy() if Wd is not None else None),
            (C2.float().cpu().numpy() if C2 is not None else None))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("tile", [0, 1, 3])
@pytest.mark.parametrize("shape", [(200, 136, 72), (1, 64, 96), (256, 256, 512), (300, 328, 1000)])
def test_gemm_store(dtype, tile, shape):
    M, N, K = shape
    ref, got, _, _ = run_gemm(dtype, 0, M, N, K, batch=2, tile=tile)
    err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err < 4e-5 * math.sqrt(K), err


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("shape", [(130, 136, 4096), (1, 3072, 3072), (64, 256, 8192)])
def test_gemm_split_k(dtype, shape):
    """Few output tiles and a long K: the 128x128 tile splits K (fixed-order sum)."""
    M, N, K = shape
    ref, got, _, _ = run_gemm(dtype, 1, M, N, K, tile=3, ws_elems=1 << 24)
    err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err < 4e-5 * math.sqrt(K), err


@pytest.mark.parametrize("tile", [4, 5, 6, 7, 8, 9])
@pytest.mark.parametrize("epi,shape,ws", [(0, (300, 328, 1024), 0), (1, (257, 520, 2048), 0), (0, (130, 136, 4096), 1 << 24),
                                          (1, (64, 3072, 3072), 1 << 24), (0, (512, 512, 96), 0)])
def test_gemm_direct_to_lds(tile, epi, shape, ws):
    """bf16 tiles loaded straight into an LDS ring (ragged M/N, split-K;
    K not a multiple of the tile depth falls back to the register-staged kernel)."""
    M, N, K = shape
    ref, got, _, _ = run_gemm(torch.bfloat16, epi, M, N, K, batch=2, tile=tile, ws_elems=ws)
    err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err < 4e-5 * math.sqrt(K), err


@pytest.mark.parametrize("epi,shape,ws", [
    (0, (1024, 8448, 192), 0),        # 128x128 tiles would take more than one round: 256x256, unsplit
    (0, (256, 384, 8192), 1 << 22),   # long K over few tiles: 256x256 split over K to fill the CUs
    (1, (300, 520, 8256), 1 << 22),   # the same with ragged M / N, an uneven split and the residual
])
def test_gemm_automatic_tile_rules(epi, shape, ws):
    """The automatic tile choice at the shapes whose rules the chunk loop's
    products (Q/K/V, dn, dx, MLP down) fall under."""
    M, N, K = shape
    ref, got, _, _ = run_gemm(torch.bfloat16, epi, M, N, K, tile=0, ws_elems=ws)
    err = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert err < 4e-5 * math.sqrt(K), err


@pytest.mark.parametrize("N", [640, 645, 40001])
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("epi,out_f32", [(0, True), (0, False), (1, True), (3, False), (4, True)])
def test_gemm_skinny(M, epi, out_f32, N):
    """A few rows of A (decode): the streaming skinny-product kernel, batched,
    against fp64 for every epilogue but SGD. Odd N leaves a wave with one of
    its two outputs; N = 40001 makes the 4096-workgroup grid stride over the
    outputs."""
    if epi == 3 and N % 64:
        pytest.skip("SwiGLU needs N a multiple of 64")
    if N > 1000 and (M, epi, out_f32) != (3, 0, True):
        pytest.skip("one combination covers the grid stride")
    lib = bd.load()
    # K = 4104: two full groups of loads in flight per lane and a one-lane tail
    K, batch = (4104 if N == 645 else 1000), 2
    A, Ad = rnd((batch, M, K), 1, torch.bfloat16)
    Bm, Bd = rnd((batch, N, K), 2, torch.bfloat16)
    z = np.einsum("zmk,znk->zmn", A, Bm)
    R = Rd = None
    if epi == 0:
        ref = z
    elif epi == 1:
        R, Rd = rnd((batch, M, N), 3, torch.float32)
        ref = R + z
    elif epi == 3:
        u = np.arange(N // 2)
        gc = (u // 32) * 64 + u % 32
        ref = _silu(z[:, :, gc]) * z[:, :, gc + 32]
    else:
        ref = _gelu(z)
    NO = ref.shape[2]
    cdt = torch.float32 if (out_f32 or epi == 1) else torch.bfloat16
    C = torch.zeros((batch, M, NO), dtype=cdt, device="cuda")
    bd.check(lib.ttt_k_gemm(1, epi, int(out_f32), M, N, K, bd.ptr(Ad), K, M * K, bd.ptr(Bd), K, N * K,
                            bd.ptr(C), NO, M * NO, None, 0, 0, bd.ptr(Rd), N, M * N, None, 0, 0, 0.0, 0, batch,
                            None, 0, bd.stream_ptr()), kernel=True)
    sync()
    got = C.float().cpu().numpy()
    scale = max(np.abs(ref).max(), 1.0)
    tol = (4e-5 * math.sqrt(K) if cdt == torch.float32 else 2 ** -8 * 2) * scale
    assert np.abs(got - ref).max() <= tol


@pytest.mark.parametrize("dtype", DTYPES)
def test_gemm_store_compute_dtype(dtype):
    ref, got, _, _ = run_gemm(dtype, 0, 130, 64, 64, out_f32=False)
    rt = 1e-6 if dtype == torch.float32 else 2 ** -8
    np.testing.assert_allclose(got, ref, rtol=rt, atol=rt * np.abs(ref).max())


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("tile", [0, 1, 3])
def test_gemm_residual_add(dtype, tile):
    ref, got, _, _ = run_gemm(dtype, 1, 150, 96, 200, tile=tile)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("tile,ws", [(0, 0), (1, 0), (3, 1 << 22), (6, 0), (7, 1 << 22)])
@pytest.mark.parametrize("sr_seed", [0, 12345])
@pytest.mark.parametrize("M,N", [(96, 136), (256, 392)])
def test_gemm_sgd_epilogue(dtype, tile, ws, sr_seed, M, N):
    """W <- W - lr * (gradient); both compute copies = the same rounding of W.
    256 x 392 has whole 128 x 128 tiles (the wide-access epilogue of the
    direct-to-LDS kernels) beside a ragged column edge."""
    lr = 0.37
    ref, got_c, got_w, got_c2 = run_gemm(dtype, 2, M, N, 1024, batch=2, lr=lr, tile=tile, ws_elems=ws,
                                         sr_seed=sr_seed)
    np.testing.assert_allclose(got_w, ref, rtol=1e-5, atol=1e-4)
    np.testing.assert_array_equal(got_c2, got_c.transpose(0, 2, 1))
    if dtype == torch.float32:
        np.testing.assert_allclose(got_c, got_w, rtol=1e-7, atol=0)
    elif sr_seed == 0:
        np.testing.assert_allclose(got_c, got_w, rtol=2 ** -8, atol=0)
    else:
        # stochastic rounding: within one bf16 ulp, to one of the two neighbours, unbiased
        np.testing.assert_allclose(got_c, got_w, rtol=2 ** -7, atol=0)
        err = (got_c - got_w) / np.abs(got_w)
        assert abs(err.mean()) < 0.05 * np.abs(err).mean()


@pytest.mark.parametrize("epi,out_f32,sr_seed", [(0, True, 0), (0, False, 0), (2, False, 0), (2, False, 5)])
@pytest.mark.parametrize("shape,batch", [((128, 128, 64), 2), ((256, 384, 192), 2), ((4096, 3072, 1024), 1)])
def test_gemm_mn_major_operands(epi, out_f32, sr_seed, shape, batch):
    """Both operands stored MN-major (as the weight-gradient products read
    their activations): C = A^T-layout . B^T-layout, plain store and the SGD
    epilogue, against fp64."""
    lib = bd.load()
    M, N, K = shape
    At, Atd = rnd((batch, K, M), 1, torch.bfloat16)
    Bt, Btd = rnd((batch, K, N), 2, torch.bfloat16)
    z = np.einsum("zkm,zkn->zmn", At, Bt)
    lr = 0.37
    C = torch.zeros((batch, M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device="cuda")
    C2 = Wd = None
    if epi == 2:
        Wm, Wd = rnd((batch, M, N), 4, torch.float32)
        ref = Wm - lr * z
        C2 = torch.zeros((batch, N, M), dtype=torch.bfloat16, device="cuda")
    else:
        ref = z
    lib.ttt_k_gemm_operands(1)
    try:
        bd.check(lib.ttt_k_gemm(1, epi, int(out_f32), M, N, K, bd.ptr(Atd), M, K * M, bd.ptr(Btd), N, K * N,
                                bd.ptr(C), N, M * N, bd.ptr(C2), M, M * N, None, 0, 0, bd.ptr(Wd), N, M * N,
                                lr, sr_seed, batch, None, 0, bd.stream_ptr()), kernel=True)
        sync()
    finally:
        lib.ttt_k_gemm_operands(0)
    got = C.float().cpu().numpy()
    if epi == 2:
        got_w = Wd.cpu().numpy()
        np.testing.assert_allclose(got_w, ref, rtol=1e-5, atol=1e-4)
        np.testing.assert_array_equal(C2.float().cpu().numpy(), got.transpose(0, 2, 1))
        np.testing.assert_allclose(got, got_w, rtol=2 ** -7 if sr_seed else 2 ** -8, atol=0)
    else:
        scale = max(np.abs(ref).max(), 1.0)
        tol = (4e-5 * math.sqrt(K) if out_f32 else 2 ** -7) * scale
        assert np.abs(got - ref).max() <= tol


def test_gemm_mn_major_rejects_ragged_shapes():
    lib = bd.load()
    A = torch.zeros(64 * 200, dtype=torch.bfloat16, device="cuda")
    C = torch.zeros(200 * 128, dtype=torch.float32, device="cuda")
    lib.ttt_k_gemm_operands(1)
    try:
        rc = lib.ttt_k_gemm(1, 0, 1, 200, 128, 64, bd.ptr(A), 200, 0, bd.ptr(A), 128, 0, bd.ptr(C), 128, 0, None, 0,
                            0, None, 0, 0, None, 0, 0, 0.0, 0, 1, None, 0, bd.stream_ptr())
    finally:
        lib.ttt_k_gemm_operands(0)
    assert rc != 0


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _gelu(x):
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("epi", [3, 4])
@pytest.mark.parametrize("tile,ws,shape", [(0, 0, (200, 384, 264)), (1, 0, (300, 640, 200)),
                                           (3, 1 << 24, (130, 128, 4096)), (3, 0, (70, 192, 96)),
                                           (5, 0, (300, 640, 256)), (4, 1 << 24, (130, 256, 4096))])
@pytest.mark.parametrize("out_f32", [True, False])
def test_gemm_activation_epilogue(dtype, epi, tile, ws, shape, out_f32):
    """Up-projection with the MLP activation in the epilogue (SwiGLU: gate/up
    columns interleaved in blocks of 32; GELU: elementwise), incl. split-K."""
    lib = bd.load()
    M, N, K = shape
    batch = 2
    A, Ad = rnd((batch, M, K), 1, dtype)
    Bm, Bd = rnd((batch, N, K), 2, dtype)
    z = np.einsum("zmk,znk->zmn", A, Bm)
    if epi == 3:
        u = np.arange(N // 2)
        gc = (u // 32) * 64 + u % 32
        ref = _silu(z[:, :, gc]) * z[:, :, gc + 32]
    else:
        ref = _gelu(z)
    NO = ref.shape[2]
    C = torch.zeros((batch, M, NO), dtype=torch.float32 if out_f32 else dtype, device="cuda")
    wsb = torch.zeros(ws, device="cuda") if ws else None
    lib.ttt_k_gemm_tile(tile)
    try:
        bd.check(lib.ttt_k_gemm(kdt(dtype), epi, int(out_f32), M, N, K, bd.ptr(Ad), K, M * K, bd.ptr(Bd), K, N * K,
                                bd.ptr(C), NO, M * NO, None, 0, 0, None, 0, 0, None, 0, 0, 0.0, 0, batch,
                                bd.ptr(wsb), ws, bd.stream_ptr()), kernel=True)
        sync()
    finally:
        lib.ttt_k_gemm_tile(0)
    got = C.float().cpu().numpy()
    scale = np.abs(ref).max()
    if out_f32:
        tol = (4e-5 * math.sqrt(K) if dtype == torch.float32 else 2e-3) * max(scale, 1.0)
    else:
        tol = (1e-4 if dtype == torch.float32 else 2 ** -8) * max(scale, 1.0) * 2
    err = np.abs(got - ref).max()
    assert err <= tol, (err, tol)


def test_swiglu_epilogue_rejects_ragged_n():
    lib = bd.load()
    rc = lib.ttt_k_gemm(1, 3, 1, 64, 96, 64, None, 64, 0, None, 64, 0, None, 48, 0, None, 0, 0, None, 0, 0,
                        None, 0, 0, 0.0, 0, 1, None, 0, bd.stream_ptr())
    assert rc != 0


def test_stochastic_rounding_is_unbiased():
    """Equal masters 1 + 2^-10, an eighth of a bf16 ulp (2^-7 at 1.0) above 1, round up 1/8 of the time."""
    lib = bd.load()
    M, N, K = 64, 512, 8
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    W = torch.full((M, N), 1.0 + 2.0 ** -10, device="cuda")
    C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    bd.check(lib.ttt_k_gemm(1, 2, 0, M, N, K, bd.ptr(A), K, 0, bd.ptr(B), K, 0, bd.ptr(C), N, 0, None, 0, 0,
                            None, 0, 0, bd.ptr(W), N, 0, 0.0, 777, 1, None, 0, bd.stream_ptr()), kernel=True)
    sync()
    c = C.float().cpu().numpy()
    up = np.mean(c > 1.0)
    assert set(np.unique(c)) <= {1.0, 1.0 + 2.0 ** -7}
    assert abs(up - 0.125) < 0.01, up


# ---------------------------- attention --------------------------------------

def attn_case(dtype, B, M, H, hd, pos0, window, seed=0):
    cap = ((window + M + 63) // 64) * 64
    HD = H * hd
    lo = max(0, pos0 - window + 1)
    npos = pos0 + M - lo
    K, _ = rnd((B, npos, H, hd), seed + 1, dtype)
    V, _ = rnd((B, npos, H, hd), seed + 2, dtype)
    q, qd = rnd((B, M, H, hd), seed + 3, dtype)
    # slots outside the window hold unrelated finite values: they must get weight 0
    junk = np.random.default_rng(seed + 4)
    kc = junk.standard_normal((B, cap, HD)) * 3
    vc = junk.standard_normal((B, cap, HD)) * 3
    for i, p in enumerate(range(lo, pos0 + M)):
        kc[:, p % cap] = K[:, i].reshape(B, HD)
        vc[:, p % cap] = V[:, i].reshape(B, HD)
    kcd, vcd = to_dev(kc, dtype), to_dev(vc, dtype)
    return dict(cap=cap, K=K, V=V, q=q, qd=qd.reshape(B * M, HD).contiguous(), kcd=kcd, vcd=vcd, lo=lo)


@pytest.mark.parametrize("dtype,hd,dl", [(torch.float32, 16, 1), (torch.float32, 64, 1), (torch.bfloat16, 64, 1),
                                         (torch.bfloat16, 128, 1), (torch.bfloat16, 128, 0),
                                         (torch.bfloat16, 128, 2)])
@pytest.mark.parametrize("B,M,H,pos0,window,nsplit", [(1, 100, 2, 0, 128, 1), (2, 64, 3, 300, 96, 1),
                                                      (1, 200, 2, 1000, 64, 1), (1, 1, 2, 517, 256, 1),
                                                      (1, 130, 2, 900, 512, 4), (2, 64, 3, 1500, 1024, 8),
                                                      (1, 1, 2, 2000, 1024, 8), (1, 100, 2, 0, 128, 2),
                                                      (1, 1, 3, 4000, 2048, 16), (2, 33, 2, 3000, 2048, 16),
                                                      (2, 5, 3, 3000, 2048, 4), (1, 8, 2, 70, 1024, 1),
                                                      (1, 3, 2, 200, 64, 2), (1, 1, 2, 0, 64, 1),
                                                      (1, 2, 2, 10, 64, 4), (2, 1, 2, 40, 128, 16),
                                                      (1, 520, 2, 3000, 2048, 4), (1, 700, 2, 5000, 256, 2)])
def test_attention_fwd_bwd(dtype, hd, dl, B, M, H, pos0, window, nsplit):
    """dl: forward kernels of bf16 head dim 128 (1 default: direct-to-LDS tiles,
    the one-query kernel for at most 8 queries; 2 direct-to-LDS tiles for any
    number of queries; 0 register-staged)."""
    lib = bd.load()
    c = attn_case(dtype, B, M, H, hd, pos0, window)
    HD = H * hd
    scale = 1.0 / math.sqrt(hd)
    o = torch.zeros((B * M, HD), dtype=dtype, device="cuda")
    lse = torch.zeros((B, H, M), dtype=torch.float32, device="cuda")
    ws = torch.zeros(nsplit * B * M * (HD + 2 * H), device="cuda")
    lib.ttt_k_attn_fwd_kernel(dl)
    try:
        bd.check(lib.ttt_k_attn_fwd(kdt(dtype), bd.ptr(c["qd"]), bd.ptr(c["kcd"]), bd.ptr(c["vcd"]), c["cap"],
                                    bd.ptr(o), bd.ptr(lse), B, M, H, hd, pos0, window, scale, nsplit, bd.ptr(ws),
                                    bd.stream_ptr()),
                 kernel=True)
    finally:
        lib.ttt_k_attn_fwd_kernel(1)
    do, dod = rnd((B, M, H, hd), 9, dtype)
    dod = dod.reshape(B * M, HD).contiguous()
    delta = torch.zeros((B, H, M), dtype=torch.float32, device="cuda")
    bd.check(lib.ttt_k_attn_delta(kdt(dtype), bd.ptr(o), bd.ptr(dod), B, M, H, hd, bd.ptr(delta),
                                  bd.stream_ptr()), kernel=True)
    dqs = torch.zeros((nsplit, B * M, HD), dtype=torch.float32, device="cuda")
    dk = torch.zeros((B * M, HD), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    bd.check(lib.ttt_k_attn_bwd(kdt(dtype), bd.ptr(c["qd"]), bd.ptr(c["kcd"]), bd.ptr(c["vcd"]), c["cap"],
                                bd.ptr(lse), bd.ptr(dod), bd.ptr(delta), bd.ptr(dqs), bd.ptr(dk), bd.ptr(dv),
                                B, M, H, hd, pos0, window, scale, nsplit, bd.stream_ptr()), kernel=True)
    sync()
    dq = dqs.sum(0)
    qpos = np.arange(pos0, pos0 + M)
    kpos = np.arange(c["lo"], pos0 + M)
    o_g = o.float().cpu().numpy().reshape(B, M, H, hd)
    dq_g = dq.cpu().numpy().reshape(B, M, H, hd)
    dk_g = dk.cpu().numpy().reshape(B, M, H, hd)
    dv_g = dv.cpu().numpy().reshape(B, M, H, hd)
    lse_g = lse.cpu().numpy()
    bf = dtype == torch.bfloat16
    for s in range(B):
        o_r, P = O.window_attention(c["q"][s], c["K"][s], c["V"][s], qpos, kpos, window)
        tol = 3e-2 if bf else 2e-5
        np.testing.assert_allclose(o_g[s], o_r, atol=tol * np.abs(o_r).max(), rtol=0)
        # lse of the scaled scores
        sc = np.einsum("mhd,nhd->hmn", c["q"][s], c["K"][s]) * scale
        sc = np.where(O.window_mask(qpos, kpos, window)[None], sc, -np.inf)
        mx = sc.max(-1, keepdims=True)
        lse_r = (np.log(np.exp(sc - mx).sum(-1, keepdims=True)) + mx)[..., 0]
        np.testing.assert_allclose(lse_g[s], lse_r, atol=1e-2 if bf else 1e-5, rtol=0)
        dq_r, dK_r, dV_r = O.window_attention_bwd(c["q"][s], c["K"][s], c["V"][s], P,
                                                  do[s] if not bf else do[s])
        # with bf16, O is rounded before it enters delta: compare with loose bounds
        tb = 5e-2 if bf else 5e-5
        # dQ and dK vanish where a query sees a single key (its weight is 1):
        # there the bound falls back to a small fraction of the scale of
        # scale * dO * V * K instead of the (zero) reference maximum
        floor = 1e-2 * scale * np.abs(do[s]).max() * np.abs(c["V"][s]).max() * np.abs(c["K"][s]).max()
        np.testing.assert_allclose(dq_g[s], dq_r, atol=tb * max(np.abs(dq_r).max(), floor), rtol=0)
        np.testing.assert_allclose(dk_g[s], dK_r[-M:], atol=tb * max(np.abs(dK_r[-M:]).max(), floor), rtol=0)
        np.testing.assert_allclose(dv_g[s], dV_r[-M:], atol=tb * np.abs(dV_r[-M:]).max(), rtol=0)


# ------------------------------ CE -------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("V,rows", [(256, 37), (32000, 37), (32000, 600)])
def test_cross_entropy(dtype, V, rows):
    """Against the oracle's softmax cross entropy, at a chunk-like row count
    too (600 rows of the 32000-word vocabulary)."""
    lib = bd.load()
    z, zd = rnd((rows, V), 5, torch.float32, scale=3.0)
    rng = np.random.default_rng(6)
    labels = rng.integers(0, V, rows)
    z[3, [10, 20]] = z[3].max() + 1.0          # planted tie: argmax must be 10
    zd = to_dev(z, torch.float32)
    ids2 = to_dev(np.stack([np.zeros(rows), labels], 1), torch.int32)
    losses = torch.zeros(rows, device="cuda")
    dz = torch.zeros((rows, V), dtype=dtype, device="cuda")
    scale = 1.0 / 512
    bd.check(lib.ttt_k_ce(kdt(dtype), bd.ptr(zd), rows, V, bd.ptr(ids2), 1, bd.ptr(losses), bd.ptr(dz), scale,
                          None, None, None, bd.stream_ptr()), kernel=True)
    lse = torch.zeros(rows, device="cuda")
    mx = torch.zeros(rows, device="cuda")
    am = torch.zeros(rows, dtype=torch.int32, device="cuda")
    bd.check(lib.ttt_k_ce(kdt(dtype), bd.ptr(zd), rows, V, bd.ptr(ids2), 0, None, None, scale, bd.ptr(lse),
                          bd.ptr(mx), bd.ptr(am), bd.stream_ptr()), kernel=True)
    sync()
    l_r, g_r = O.cross_entropy(z, labels)
    np.testing.assert_allclose(losses.cpu().numpy(), l_r, atol=1e-4, rtol=0)
    rt = 1e-5 if dtype == torch.float32 else 2 ** -8
    np.testing.assert_allclose(dz.float().cpu().numpy(), g_r * scale, rtol=rt, atol=rt * scale * 1e-3)
    assert am.cpu().numpy()[3] == 10
    np.testing.assert_array_equal(am.cpu().numpy(), np.argmax(z, axis=1))
    np.testing.assert_allclose(lse.cpu().numpy(), l_r + z[np.arange(rows), labels], atol=1e-4)
    np.testing.assert_allclose(mx.cpu().numpy(), z.max(1), atol=0)


# ----------------------------- RMSNorm ---------------------------------------

@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 2048, 3072, 4096, 4100])
def test_rmsnorm(dtype, d):
    """Rows of up to 4096 columns are held in registers (1 to 4 float4 per
    thread); wider rows take the two-pass kernel (4100)."""
    lib = bd.load()
    rows = 19
    x, xd = rnd((rows, d), 7, torch.float32, scale=2.0)
    g, gd = rnd((d,), 8, dtype)
    y = torch.zeros((rows, d), dtype=dtype, device="cuda")
    r = torch.zeros(rows, device="cuda")
    bd.check(lib.ttt_k_rmsnorm_fwd(kdt(dtype), bd.ptr(xd), rows, d, bd.ptr(gd), 1e-6, bd.ptr(y), bd.ptr(r),
                                   bd.stream_ptr()), kernel=True)
    dn, dnd = rnd((rows, d), 9, torch.float32)
    res0, res = rnd((rows, d), 10, torch.float32)
    bd.check(lib.ttt_k_rmsnorm_bwd(kdt(dtype), bd.ptr(xd), bd.ptr(r), bd.ptr(gd), bd.ptr(dnd), rows, d, bd.ptr(res),
                                   1, bd.stream_ptr()), kernel=True)
    sync()
    y_r, r_r = O.rmsnorm_fwd(x, g, 1e-6)
    rt = 1e-5 if dtype == torch.float32 else 2 ** -8
    np.testing.assert_allclose(y.float().cpu().numpy(), y_r, rtol=rt, atol=rt * np.abs(y_r).max() * 1e-2)
    np.testing.assert_allclose(r.cpu().numpy(), r_r[:, 0], rtol=1e-5)
    dx_r = O.rmsnorm_bwd(x, g, r_r, dn) + res0
    np.testing.assert_allclose(res.cpu().numpy(), dx_r, rtol=1e-4, atol=1e-4)


# ------------------------ rotary Q/K/V projection -----------------------------

def _permute_qkv_rows(Wt, H, hd):
    """Rows [3*H*hd][K] of W^T, each head's hd rows reordered in 32-row blocks
    as [0, nb/2, 1, nb/2 + 1, ...] (the layout ttt_k_qkv_rope documents)."""
    nb = hd // 32
    order = []
    for b in range(nb // 2):
        order += [b, nb // 2 + b]
    out = np.empty_like(Wt)
    for part in range(3):
        for h in range(H):
            base = (part * H + h) * hd
            for k, b in enumerate(order):
                out[base + 32 * k: base + 32 * k + 32] = Wt[base + 32 * b: base + 32 * b + 32]
    return out


@pytest.mark.parametrize("rows,S,p0,cap,rope", [(200, 100, 0, 192, True),     # tiles, two sequences
                                                (3, 3, 131000, 64, True),     # skinny product, ring wrap
                                                (256, 256, 4100, 320, True),  # slots wrap inside the block
                                                (130, 130, 7, 192, False)])   # no rotation
@pytest.mark.parametrize("hd", [64, 128])
def test_qkv_rope_epilogue(rows, S, p0, cap, rope, hd):
    """The Q/K/V product with RoPE applied to its fp32 accumulators and k / v
    written to ring-cache slots, against the oracle's rope of the fp64
    product (bf16 outputs rounded once)."""
    lib = bd.load()
    H, K, theta = 3, 256, 10000.0
    HD = H * hd
    B = rows // S
    A, Ad = rnd((rows, K), 11, torch.bfloat16)
    W, _ = rnd((K, 3 * HD), 12, torch.bfloat16, scale=0.05)
    Bp = torch.as_tensor(_permute_qkv_rows(np.ascontiguousarray(W.T), H, hd), dtype=torch.float32)
    Bp = Bp.to(torch.bfloat16).cuda()
    tab = None
    if rope:
        ang = O.rope_angles(np.arange(p0 + S), hd, theta)
        t = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
        tab = torch.as_tensor(t).cuda()
    q = torch.zeros((rows, HD), dtype=torch.bfloat16, device="cuda")
    kc = torch.full((B, cap, HD), 7.0, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((B, cap, HD), 7.0, dtype=torch.bfloat16, device="cuda")
    bd.check(lib.ttt_k_qkv_rope(rows, S, H, hd, K, bd.ptr(Ad), K, bd.ptr(Bp), bd.ptr(tab), p0, bd.ptr(q),
                                bd.ptr(kc), bd.ptr(vc), cap, bd.stream_ptr()), kernel=True)
    sync()
    z = A @ W
    pos = np.tile(np.arange(p0, p0 + S), B)
    qr = z[:, :HD].reshape(rows, H, hd)
    kr = z[:, HD:2 * HD].reshape(rows, H, hd)
    vr = z[:, 2 * HD:].reshape(rows, H, hd)
    if rope:
        qr, kr = O.rope(qr, pos, theta), O.rope(kr, pos, theta)
    tol = 2 ** -8 * np.abs(z).max()
    np.testing.assert_allclose(q.float().cpu().numpy(), qr.reshape(rows, HD), rtol=0, atol=tol)
    kg, vg = kc.float().cpu().numpy(), vc.float().cpu().numpy()
    slots = pos % cap
    for s in range(B):
        sl = slots[s * S:(s + 1) * S]
        np.testing.assert_allclose(kg[s, sl], kr[s * S:(s + 1) * S].reshape(S, HD), rtol=0, atol=tol)
        np.testing.assert_allclose(vg[s, sl], vr[s * S:(s + 1) * S].reshape(S, HD), rtol=0, atol=tol)
        untouched = np.setdiff1d(np.arange(cap), sl)
        assert (kg[s, untouched] == 7.0).all() and (vg[s, untouched] == 7.0).all()
