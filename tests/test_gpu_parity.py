"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case prints its name, shapes and seed before touching the GPU.
Tolerances are those of ``tests/parity.py``.
"""
import numpy as np
import pytest

import oracle
import parity
import workloads as wl

pytestmark = pytest.mark.gpu

F32 = np.float32


def _torch():
    import torch
    return torch


def dev(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def say(*a):
    print("[case]", *a, flush=True)


def _problem(d_out, d_in, n, seed, xdtype=np.float32, wdtype=np.float32, dead=(), rank=4):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((d_in, n)) + rng.standard_normal((d_in, rank)) @ rng.standard_normal((rank, n)) / np.sqrt(rank)
    for d in dead:
        X[d] = 0.0
    W = rng.standard_normal((d_out, d_in)) * 0.02
    return W.astype(wdtype), X.astype(xdtype)


def _quant_dict(qz):
    return {"codes": host(qz.codes), "scales": host(qz.scales), "zeros": host(qz.zeros),
            "err_row": host(qz.err_row), "minmax": host(qz.minmax)}


# ---------------------------------------------------------------------------
# stage 1
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,N,xdtype,chunk", [
    (64, 512, np.float32, None),
    (128, 100, np.float32, 7),        # ragged token tail, unaligned chunk views
    (200, 333, np.float16, None),     # ragged tiles
    (130, 1000, np.float16, 300),     # chunk views at unaligned offsets
    (256, 2048, np.float16, 1024),
    (1, 5, np.float16, None),
    (4000, 333, np.float16, None),    # 192-wide tiles (21 per side): ragged tiles, unaligned rows
    (4000, 1000, np.float16, None),   # 192-wide tiles: 13 steady slabs, then the generic part and a ragged tail
    (4096, 700, np.float16, 300),     # 192-wide tiles, ragged last tile row, unaligned chunk views
    (4500, 96, np.float16, None),     # 192-wide tiles (24 per side), one full slab and a tail
    (3904, 700, np.float16, 300),     # 192-wide tiles: chunk views at unaligned offsets
    (8000, 200, np.float16, None),    # 256-wide tiles (32 per side: two rounds on 256 CUs), ragged
])
def test_hessian(lib, n, N, xdtype, chunk):
    from post_weight_quantization_04_amd import layer
    say("hessian", n, N, xdtype.__name__, chunk)
    _, X = _problem(1, n, N, seed=n + N, xdtype=xdtype)
    H = layer.hessian(dev(X), chunk=chunk)
    _torch().cuda.synchronize()
    Hd = host(H)
    step = chunk or N
    H_ref = oracle.hessian([X[:, t:t + step] for t in range(0, N, step)])
    parity.check_h(Hd, H_ref)
    assert np.all(np.triu(Hd, 1) == 0)  # upper triangle untouched (zeroed by the caller)


@pytest.mark.parametrize("n,N,xdtype,chunk", [
    (300, 200, np.float16, 64),       # 128-wide tiles: set, then three accumulating chunks
    (4000, 333, np.float16, None),    # 192-wide tiles
    (8000, 100, np.float16, 40),      # 256-wide tiles
    (200, 150, np.float32, 50),       # float32 inputs
])
def test_hessian_set_then_accumulate(lib, n, N, xdtype, chunk):
    """Setting H from the first chunk (old values neither read nor needed)
    and accumulating the rest gives, bit for bit, the H of accumulating every
    chunk into a zeroed H; the strictly upper triangle is not written."""
    import torch
    say("hessian set", n, N, xdtype.__name__, chunk)
    _, X = _problem(1, n, N, seed=n + 7 * N, xdtype=xdtype)
    Xd = dev(X)
    step = chunk or N
    H0 = torch.zeros((n, n), dtype=torch.float32, device=Xd.device)
    for t0 in range(0, N, step):
        _lib_mod().hessian_accumulate(H0, Xd[:, t0:t0 + step])
    H1 = torch.full((n, n), 7.0, dtype=torch.float32, device=Xd.device)
    _lib_mod().hessian_set(H1, Xd[:, 0:step])
    for t0 in range(step, N, step):
        _lib_mod().hessian_accumulate(H1, Xd[:, t0:t0 + step])
    torch.cuda.synchronize()
    a, b = host(H0), host(H1)
    np.testing.assert_array_equal(np.tril(b), np.tril(a))
    assert np.all(b[np.triu_indices(n, 1)] == 7.0)


@pytest.mark.parametrize("ldx", [530_000, 540_000])
def test_hessian_large_row_stride(lib, ldx):
    """A chunk of a very long X (rows 1 MB apart): with byte offsets below
    4 GiB the 192-wide kernel takes d_in = 4000, above it the 128-wide one;
    either gives, bit for bit, the H of the same chunk stored contiguously."""
    import torch
    n, N = 4000, 96
    say("hessian large row stride", n, N, ldx)
    g = torch.Generator(device="cuda").manual_seed(11)
    big = torch.empty((n, ldx), dtype=torch.float16, device="cuda")
    big[:, :N] = torch.randn((n, N), generator=g, device="cuda").to(torch.float16)
    Xv = big[:, :N]
    Xc = Xv.contiguous()
    H0 = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    H1 = torch.zeros((n, n), dtype=torch.float32, device="cuda")
    _lib_mod().hessian_accumulate(H0, Xc)
    _lib_mod().hessian_accumulate(H1, Xv)
    torch.cuda.synchronize()
    assert torch.equal(H0, H1)
    del big, Xv


@pytest.mark.parametrize("n,nc,ntok,set_first", [
    (300, 4, 64, True),       # 128-wide tiles
    (4096, 3, 128, True),     # 192-wide tiles
    (4000, 5, 64, False),     # 192-wide tiles, ragged d_in, adding into H
    (8000, 2, 64, True),      # 256-wide tiles
    (300, 35, 64, False),     # two launches: 32 chunks, then 3
])
def test_hessian_chunks_match_contiguous(lib, n, nc, ntok, set_first):
    """Chunks in separate buffers summed by one call give, bit for bit, the
    H of single calls over the same tokens stored contiguously, one per group
    of 32 chunks."""
    import torch
    say("hessian chunks", n, nc, ntok, set_first)
    g = torch.Generator(device="cuda").manual_seed(n + nc)
    Xs = [torch.randn((n, ntok), generator=g, device="cuda").to(torch.float16) for _ in range(nc)]
    init = 0.0 if set_first else 0.5
    H0 = torch.full((n, n), init, dtype=torch.float32, device="cuda")
    H1 = torch.full((n, n), init, dtype=torch.float32, device="cuda")
    _lib_mod().hessian_chunks(H1, Xs, set_first=set_first)
    for c0 in range(0, nc, 32):
        Xcat = torch.cat(Xs[c0:c0 + 32], dim=1).contiguous()
        if set_first and c0 == 0:
            _lib_mod().hessian_set(H0, Xcat)
        else:
            _lib_mod().hessian_accumulate(H0, Xcat)
    torch.cuda.synchronize()
    assert torch.equal(torch.tril(H0), torch.tril(H1))
    iu = torch.triu_indices(n, n, 1, device="cuda")
    assert torch.all(H1[iu[0], iu[1]] == init)  # strictly upper triangle not written
    if n <= 4096:
        Xall = np.concatenate([host(X) for X in Xs], axis=1)
        ref = oracle.hessian([Xall])
        if not set_first:
            ref = ref + np.tril(np.full((n, n), init))
        parity.check_h(host(H1), ref)


@pytest.mark.parametrize("n,nc,ntok,xdtype,offset", [
    (300, 3, 100, "f16", 0),                 # ragged chunks: one call per chunk
    (300, 3, 64, "f16", 1),                  # unaligned rows: one call per chunk
    (200, 3, 50, "f32", 0),                  # float32 inputs: one call per chunk
])
def test_hessian_chunks_fallback(lib, n, nc, ntok, xdtype, offset):
    """Chunks the batched launch does not take are added one call per chunk:
    the H of gptq_hessian_set on the first and gptq_hessian_accumulate on
    the others, bit for bit."""
    import torch
    say("hessian chunks fallback", n, nc, ntok, xdtype, offset)
    dt = torch.float16 if xdtype == "f16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(3 * n + nc)
    Xs = [torch.randn((n, ntok + offset), generator=g, device="cuda").to(dt)[:, offset:] for _ in range(nc)]
    H0 = torch.full((n, n), 9.0, dtype=torch.float32, device="cuda")
    H1 = torch.full((n, n), 9.0, dtype=torch.float32, device="cuda")
    _lib_mod().hessian_chunks(H1, Xs, set_first=True)
    _lib_mod().hessian_set(H0, Xs[0])
    for X in Xs[1:]:
        _lib_mod().hessian_accumulate(H0, X)
    torch.cuda.synchronize()
    assert torch.equal(H0, H1)


def test_hessian_set_empty_writes_zero(lib):
    import torch
    say("hessian set, no tokens")
    H = torch.full((70, 70), 3.0, dtype=torch.float32, device="cuda")
    X = torch.zeros((70, 0), dtype=torch.float16, device="cuda")
    _lib_mod().hessian_set(H, X)
    torch.cuda.synchronize()
    h = host(H)
    assert np.all(h[np.tril_indices(70)] == 0.0) and np.all(h[np.triu_indices(70, 1)] == 3.0)


def _lib_mod():
    from post_weight_quantization_04_amd import _lib
    return _lib


def test_hessian_fp16_products_exact(lib):
    """Each f16 x f16 product is exact in fp32: a single-token X gives
    H = 2 x x^T exactly."""
    from post_weight_quantization_04_amd import layer
    say("hessian single token")
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 1)).astype(np.float16)
    H = host(layer.hessian(dev(x)))
    xf = x.astype(np.float64)
    ref = np.tril(2 * xf @ xf.T).astype(np.float32)
    np.testing.assert_array_equal(np.tril(H), ref)


# ---------------------------------------------------------------------------
# stages 2 + 3
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,N,dead", [
    (1, 4, ()), (16, 40, ()), (64, 200, (3,)), (100, 300, (0, 99)), (200, 150, ()),
    (333, 700, (5, 6, 300)), (512, 1024, ()),
])
def test_prepare(lib, n, N, dead):
    from post_weight_quantization_04_amd import layer
    say("prepare", n, N, dead)
    _, X = _problem(1, n, N, seed=7 * n + N, dead=dead)
    H32 = np.tril(oracle.hessian([X])).astype(F32)
    f = layer.prepare(dev(H32), 0.01)
    _torch().cuda.synchronize()
    assert int(host(f.info)[0]) == 0
    U = host(f.U)
    e, U_ref, dead_ref, lam_ref = parity.check_u(U, H32, 0.01)
    np.testing.assert_array_equal(host(f.dead).astype(bool), dead_ref)
    assert host(f.lam)[0] == pytest.approx(lam_ref, rel=1e-12)


@pytest.mark.parametrize("n,N,dead", [
    (333, 700, (5, 6, 300)),     # 6 tiles, ragged last tile
    (640, 1200, (7,)),           # 10 tiles
    (200, 150, ()),              # 4 tiles, rank-deficient X
])
def test_prepare_paired_steps(lib, monkeypatch, n, N, dead):
    """Steps paired at widths that would not pair them (GPTQ_SCHED_PAIR=1):
    every even step's update of the rest deferred into the next launch, the
    odd launches' diagonal-block workgroups applying both steps; U the same
    within the bar."""
    from post_weight_quantization_04_amd import layer
    say("prepare paired steps", n, N, dead)
    monkeypatch.setenv("GPTQ_SCHED_PAIR", "1")
    _, X = _problem(1, n, N, seed=7 * n + N, dead=dead)
    H32 = np.tril(oracle.hessian([X])).astype(F32)
    f = layer.prepare(dev(H32), 0.01)
    _torch().cuda.synchronize()
    assert int(host(f.info)[0]) == 0
    e, U_ref, dead_ref, lam_ref = parity.check_u(host(f.U), H32, 0.01)
    np.testing.assert_array_equal(host(f.dead).astype(bool), dead_ref)


def test_prepare_not_positive_definite(lib):
    from post_weight_quantization_04_amd import layer
    say("prepare non-PD")
    _, X = _problem(1, 96, 20, seed=3)  # rank 20 < 96
    H32 = np.tril(oracle.hessian([X])).astype(F32)
    with pytest.raises(oracle.NotPositiveDefinite):
        oracle.prepare(H32.astype(np.float64) + np.tril(H32, -1).T.astype(np.float64), lam=0.0)
    f = layer.prepare(dev(H32), 0.0)
    _torch().cuda.synchronize()
    info = int(host(f.info)[0])
    assert 0 < info <= 96
    f2 = layer.prepare(dev(H32), 0.01)
    _torch().cuda.synchronize()
    assert int(host(f2.info)[0]) == 0


# ---------------------------------------------------------------------------
# stage 4 (fed the oracle's U rounded to fp32)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d_out,d_in,bits,group,block,dead", [
    (64, 128, 4, 0, 32, ()),
    (100, 200, 3, 0, 48, ()),        # ragged rows, ragged last block
    (33, 160, 4, 32, 64, ()),        # groups inside a block
    (70, 256, 4, 128, 64, ()),       # group wider than a block
    (1, 16, 2, 0, 1, ()),            # B = 1
    (65, 300, 8, 0, 128, ()),        # widest block, ragged tail
    (16, 96, 4, 16, 16, ()),
    (50, 128, 4, 0, 32, (2, 64, 127)),  # dead channels
    (130, 128, 3, 128, 128, (10,)),
    (16448, 384, 4, 0, 128, ()),     # more sweeping workgroups than CUs: they take the whole update
])
def test_quantize(lib, d_out, d_in, bits, group, block, dead):
    from post_weight_quantization_04_amd import layer
    say("quantize", d_out, d_in, bits, group, block, dead)
    W, X = _problem(d_out, d_in, 3 * d_in, seed=d_out * 31 + d_in, dead=dead)
    U_ref, dmask, _ = oracle.prepare(oracle.hessian([X]))
    U32 = U_ref.astype(F32)
    fac = layer.Factor(dev(U32), dev(dmask.astype(np.uint8)), None, None)
    qz = layer.quantize(dev(W), fac, bits, group, block)
    _torch().cuda.synchronize()
    q = _quant_dict(qz)
    parity.check_codes(W.astype(np.float64), U32, dmask, q, bits, group, block)


@pytest.mark.parametrize("d_out,d_in,bits,group,block,dead", [
    (70, 300, 4, 0, 128, (3, 150)),   # f16 rows not a multiple of 8: element path of the working copy
    (64, 200, 4, 0, 64, (7,)),        # f16, 16-byte pieces with dead flags
])
def test_quantize_fp16_weights(lib, d_out, d_in, bits, group, block, dead):
    from post_weight_quantization_04_amd import layer
    say("quantize f16", d_out, d_in, bits, group, block, dead)
    W, X = _problem(d_out, d_in, 3 * d_in, seed=d_out * 37 + d_in, dead=dead, wdtype=np.float16)
    U_ref, dmask, _ = oracle.prepare(oracle.hessian([X]))
    U32 = U_ref.astype(F32)
    fac = layer.Factor(dev(U32), dev(dmask.astype(np.uint8)), None, None)
    qz = layer.quantize(dev(W), fac, bits, group, block)
    _torch().cuda.synchronize()
    q = _quant_dict(qz)
    parity.check_codes(W.astype(np.float64), U32, dmask, q, bits, group, block)


def test_quantize_fp16_weights_exact_conversion(lib):
    """All finite f16 values (subnormals included) survive the working copy:
    with U = I every column rounds independently, so the per-row grid and the
    codes equal those of the exact values."""
    from post_weight_quantization_04_amd import layer
    say("quantize all f16 values")
    bits = np.arange(0, 0x7C00, dtype=np.uint16)  # every finite non-negative f16
    vals = bits.view(np.float16)
    vals = np.concatenate([vals, -vals])[: 64 * 960].reshape(64, 960)
    U = np.eye(960, dtype=F32)
    fac = layer.Factor(dev(U), dev(np.zeros(960, np.uint8)), None, None)
    qz = layer.quantize(dev(vals), fac, 8, 0, 128)
    _torch().cuda.synchronize()
    r = oracle.quantize(vals.astype(np.float64), U.astype(np.float64), 8, 0, 128)
    np.testing.assert_array_equal(host(qz.scales), r.scales)
    np.testing.assert_array_equal(host(qz.codes), r.codes)


# ---------------------------------------------------------------------------
# the whole path
# ---------------------------------------------------------------------------
def _run_layer(W, X, bits, group, block, damp=0.01, chunk=None):
    from post_weight_quantization_04_amd import layer
    H = layer.hessian(dev(X), chunk=chunk)
    f = layer.prepare(H, damp)
    qz = layer.quantize(dev(W), f, bits, group, block)
    _torch().cuda.synchronize()
    return host(H), f, qz


@pytest.mark.parametrize("case", ["tiny", "ragged", "ragged_groups"])
def test_layer_end_to_end_small(lib, case):
    if case == "tiny":
        w = wl.get("tiny")
    elif case == "ragged":
        w = wl.custom(77, 200, 450, bits=3, block_size=48, xdtype="float16", wdtype="float16", rank=8, seed=2,
                      dead_frac=0.02)
    else:
        w = wl.custom(90, 192, 600, bits=4, group_size=32, block_size=64, xdtype="float16", wdtype="float32",
                      rank=8, seed=4)
    say("layer", case, w.layers[0], w.bits, w.group_size, w.block_size)
    W = wl.make_weight(w)
    X = wl.x_full(w)
    Hd, f, qz = _run_layer(W, X, w.bits, w.group_size, w.block_size, w.damp)
    H_ref = oracle.hessian(wl.x_chunks(w))
    parity.check_h(Hd, H_ref)
    assert int(host(f.info)[0]) == 0
    U = host(f.U)
    _, U_ref_dev, dead_ref, _ = parity.check_u(U, Hd, w.damp)
    q = _quant_dict(qz)
    parity.check_codes(W.astype(np.float64), U, dead_ref, q, w.bits, w.group_size, w.block_size)
    # end to end: the oracle's own independent run from X
    _, U_o, dead_o, _, res = oracle.layer(W.astype(np.float64), wl.x_chunks(w), w.bits, w.group_size,
                                          w.block_size, w.damp)
    e_dev, e_ref = parity.output_errors(W, q["codes"], q["scales"], q["zeros"], w.group_size,
                                        wl.x_chunks(w), res.w_hat)
    assert abs(e_dev - e_ref) <= parity.OUT_TOL * e_ref, (e_dev, e_ref)


def test_layer_attn_proj_full(lib):
    """The 4096x4096 fp16 layer with 2048 tokens, at full size: H and U in
    full, codes on 512 sampled rows (rows decouple), output error in full."""
    w = wl.get("attn_proj")
    say("layer attn_proj 4096x4096 N=2048 4-bit B=128")
    W = wl.make_weight(w)
    X = wl.x_full(w)
    Hd, f, qz = _run_layer(W, X, w.bits, w.group_size, w.block_size, w.damp)
    H_ref = oracle.hessian([X])
    parity.check_h(Hd, H_ref)
    assert int(host(f.info)[0]) == 0
    U = host(f.U)
    _, _, dead_ref, _ = parity.check_u(U, Hd, w.damp)
    q = _quant_dict(qz)
    rows = np.sort(np.random.default_rng(0).choice(W.shape[0], 512, replace=False))
    parity.check_codes(W.astype(np.float64), U, dead_ref, q, w.bits, 0, w.block_size, rows=rows)
    U_o, dead_o, _ = oracle.prepare(H_ref, w.damp)
    res = oracle.quantize(W.astype(np.float64), U_o, w.bits, 0, w.block_size, dead=dead_o)
    e_dev, e_ref = parity.output_errors(W, q["codes"], q["scales"], q["zeros"], 0, [X], res.w_hat)
    assert abs(e_dev - e_ref) <= parity.OUT_TOL * e_ref, (e_dev, e_ref)


# ---------------------------------------------------------------------------
# invariants and edge cases
# ---------------------------------------------------------------------------
def test_determinism_and_row_permutation(lib):
    from post_weight_quantization_04_amd import layer
    say("determinism + permutation")
    W, X = _problem(150, 256, 800, seed=12, xdtype=np.float16)
    a = _run_layer(W, X, 4, 0, 64)
    b = _run_layer(W, X, 4, 0, 64)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(host(a[1].U), host(b[1].U))
    np.testing.assert_array_equal(host(a[2].codes), host(b[2].codes))
    perm = np.random.default_rng(1).permutation(150)
    qz = layer.quantize(dev(W[perm]), a[1], 4, 0, 64)
    _torch().cuda.synchronize()
    np.testing.assert_array_equal(host(qz.codes), host(a[2].codes)[perm])
    np.testing.assert_array_equal(host(qz.scales), host(a[2].scales)[perm])


@pytest.mark.parametrize("group,split", [(0, False), (0, True), (32, False)])
def test_block_size_invariance(lib, group, split):
    """Lazy batching is exact (aicassindra.com "tm_gptq_math", "GPTQ's
    speedups: fixed order and lazy batches"): the codes found with block
    width B are a valid run of the sweep at any other width.  The codes of
    every B are replayed by the oracle at B = 128: no hard mismatch, ties in
    at most 0.01% of entries, grids as in every parity case; and two widths
    differ only in rows where one of them took a tie."""
    from post_weight_quantization_04_amd import layer
    say("block invariance", group, split)
    W, X = _problem(192, 384, 1200, seed=21)
    H, f, _ = _run_layer(W, X, 4, 0, 128)
    U = host(f.U)
    _, _, dead, _ = parity.check_u(U, H, 0.01)
    W64 = W.astype(np.float64)
    q = {}
    widths = (1, 7, 32, 48, 64, 128) if group == 0 else (1, 16, 32, 64, 96, 128)
    for B in widths:
        q[B] = _quant_dict(layer.quantize(dev(W), f, 4, group, B, split=split))
        _torch().cuda.synchronize()
    # each run replayed at B = 128: rows where the replay adopted nothing
    # are the oracle's own codes, so they are equal across widths
    tied = {B: parity.check_codes(W64, U, dead, qb, 4, group, 128).mismatch_rows for B, qb in q.items()}
    for B, qb in q.items():
        rows = np.any(qb["codes"] != q[128]["codes"], axis=1)
        assert not np.any(rows & ~(tied[B] | tied[128])), (B, np.nonzero(rows)[0])
        keep = ~(tied[B] | tied[128])
        if group == 0:  # per-row grids come from the input W alone
            np.testing.assert_array_equal(qb["scales"][keep], q[128]["scales"][keep])
            np.testing.assert_array_equal(qb["zeros"][keep], q[128]["zeros"][keep])
        else:  # group grids see the compensated weights, rounded in a B-dependent order
            np.testing.assert_allclose(qb["scales"][keep], q[128]["scales"][keep], rtol=1e-5)
            assert np.mean(qb["zeros"] != q[128]["zeros"]) <= 1e-4


def test_empty_and_invalid(lib):
    import ctypes
    torch = _torch()
    say("empty and invalid")
    H = torch.zeros((4, 4), device="cuda")
    X = torch.zeros((4, 0), device="cuda")
    assert lib.gptq_hessian_accumulate(H.data_ptr(), 4, X.data_ptr(), 1, 0, 0, None) == 0
    assert lib.gptq_prepare_hinv(None, 0, 0.01, None, None, None, None, None, 0, None) == 0
    assert lib.gptq_quantize_layer(None, 1, 0, 16, None, None, 4, 0, 16, None, None, None, None, None, None, 0,
                                   None) == 0
    assert lib.gptq_quantize_layer(None, 1, 4, 16, None, None, 1, 0, 16, None, None, None, None, None, None, 0,
                                   None) == 1
    torch.cuda.synchronize()
