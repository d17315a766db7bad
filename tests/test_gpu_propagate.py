"""GPU parity of the propagation to the next layer, Y = act(What X)
(gptq_propagate), against the fp64 oracle, and a two-layer chain quantized
one layer at a time with the second layer's inputs taken from the first
quantized layer's output (math4ai "GPTQ Hessian", opening paragraph).

Tolerance, from the arithmetic: each f16 x f16 product is exact in fp32, the
K products of an output are summed in fp32 (error at most about
K 2^-24 sum_k |w_k x_k|), and the result is rounded once to f16 (at most
2^-11 of it, or 2^-25 absolute in the subnormal range).  The test bound
doubles each term.
"""
import numpy as np
import pytest

import oracle
import parity

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def say(*a):
    print("[propagate]", *a, flush=True)


def bound(W, X, Y_ref):
    K = W.shape[1]
    absprod = np.abs(W.astype(np.float64)) @ np.abs(X.astype(np.float64))
    return 2.0 * (2.0 ** -11 * np.abs(Y_ref) + K * 2.0 ** -24 * absprod + 2.0 ** -25)


@pytest.mark.parametrize("M,K,N,relu,ld_pad,offset", [
    (1, 1, 1, False, 0, 0),
    (64, 128, 512, True, 0, 0),
    (130, 70, 200, True, 8, 0),       # ragged tiles and slab, strided X and Y
    (257, 300, 129, False, 0, 3),     # ragged everywhere, X and Y at an unaligned offset
    (128, 1000, 256, True, 64, 0),
    (96, 256, 100, False, 0, 0),      # 16-byte What runs, element loads of X (tokens not a multiple of 8)
    (384, 200, 1024, True, 0, 0),     # 24 tiles: the XCD-banded tile order (bands of rows)
    (512, 72, 512, False, 0, 0),      # 16 tiles in a 4 x 4 grid, K one ragged slab
    (1000, 136, 4088, True, 0, 0),    # 256 tiles, ragged rows, tokens and last slab
    (5, 0, 7, True, 0, 0),            # d_in = 0: Y = act(0)
])
def test_propagate_matches_oracle(lib, M, K, N, relu, ld_pad, offset):
    from post_weight_quantization_04_amd import layer
    torch = _torch()
    say(M, K, N, "relu" if relu else "none", ld_pad, offset)
    rng = np.random.default_rng(M * 7 + K * 3 + N)
    W = (rng.standard_normal((M, K)) * 0.05).astype(np.float16)
    X = rng.standard_normal((K, N)).astype(np.float16)
    ldx, ldy = N + ld_pad + offset, N + ld_pad + offset
    Xbuf = torch.zeros((max(K, 1) * ldx + offset,), dtype=torch.float16, device="cuda")
    Ybuf = torch.full((M * ldy + offset,), 7.0, dtype=torch.float16, device="cuda")
    Xd = Xbuf[offset:offset + K * ldx].view(K, ldx)[:, :N] if K else Xbuf[:0].view(0, N)
    if K:
        Xd.copy_(torch.from_numpy(X))
    Yd = Ybuf[offset:offset + M * ldy].view(M, ldy)[:, :N]
    layer.propagate(torch.from_numpy(W).cuda(), Xd, relu=relu, out=Yd)
    torch.cuda.synchronize()
    Y = Yd.cpu().numpy().astype(np.float64)
    Y_ref = oracle.propagate(W, X, "relu" if relu else "none")
    err = np.abs(Y - Y_ref)
    assert np.all(err <= bound(W, X, Y_ref)), float((err / bound(W, X, Y_ref)).max())
    if relu:
        assert np.all(Y >= 0.0)
    # nothing outside the output view was written
    Yall = Ybuf.cpu().numpy()
    mask = np.ones(Yall.shape, bool)
    for r in range(M):
        mask[offset + r * ldy: offset + r * ldy + N] = False
    assert np.all(Yall[mask] == 7.0)


def test_propagate_rounds_exactly_representable_results(lib):
    """Small integers: every product and partial sum is exact in fp32 and
    every result is an f16 integer, so Y is bit-exact."""
    from post_weight_quantization_04_amd import layer
    torch = _torch()
    rng = np.random.default_rng(3)
    W = rng.integers(-3, 4, size=(200, 96)).astype(np.float16)
    X = rng.integers(-2, 3, size=(96, 300)).astype(np.float16)
    Y = layer.propagate(torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Y.cpu().numpy().astype(np.float64), oracle.propagate(W, X))


def test_two_layer_chain(lib):
    """Layer A quantized against X1; layer B's inputs are ReLU(What_A X1)
    from the device; B quantized against them.  Each stage is checked with
    the oracle fed the device's previous-stage output."""
    from post_weight_quantization_04_amd import layer
    torch = _torch()
    d0, d1, d2, N, bits, block = 256, 192, 128, 1024, 4, 64
    say("chain", d0, d1, d2, N)
    rng = np.random.default_rng(11)
    X1 = (rng.standard_normal((d0, N)) + rng.standard_normal((d0, 8)) @ rng.standard_normal((8, N)) / np.sqrt(8)
          ).astype(np.float16)
    WA = (rng.standard_normal((d1, d0)) * 0.05).astype(np.float16)
    WB = (rng.standard_normal((d2, d1)) * 0.05).astype(np.float16)
    X1d = torch.from_numpy(X1).cuda()
    HA = layer.hessian(X1d)
    fA = layer.prepare(HA, 0.01)
    qA = layer.quantize(torch.from_numpy(WA).cuda(), fA, bits, 0, block)
    packed = layer.pack(qA.codes, bits)
    WA_hat = layer.dequantize(packed, bits, d0, qA.scales, qA.zeros, 0, dtype=torch.float16)
    X2d = layer.propagate(WA_hat, X1d, relu=True)
    HB = layer.hessian(X2d)
    fB = layer.prepare(HB, 0.01)
    qB = layer.quantize(torch.from_numpy(WB).cuda(), fB, bits, 0, block)
    torch.cuda.synchronize()
    # stage A: the dequantized weights are the oracle's dequantization of the device codes
    codesA = qA.codes.cpu().numpy()
    WA_ref = oracle.dequantize(codesA, qA.scales.cpu().numpy(), qA.zeros.cpu().numpy())
    WA_dev = WA_hat.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(WA_dev, WA_ref.astype(np.float16).astype(np.float64))
    # propagation, from the device's own What_A
    X2 = X2d.cpu().numpy()
    X2_ref = oracle.propagate(WA_dev, X1, "relu")
    assert np.all(np.abs(X2 - X2_ref) <= bound(WA_dev, X1, X2_ref))
    # layer B's Hessian from the device's X2, then its factor and codes
    HB_ref = oracle.hessian([X2])
    HBd = HB.cpu().numpy().astype(np.float64)
    parity.check_h(HBd, HB_ref)
    UB = fB.U.cpu().numpy()
    _, UB_ref, deadB, _ = parity.check_u(UB, HBd, 0.01)
    q = {"codes": qB.codes.cpu().numpy(), "scales": qB.scales.cpu().numpy(), "zeros": qB.zeros.cpu().numpy(),
         "err_row": qB.err_row.cpu().numpy(), "minmax": qB.minmax.cpu().numpy()}
    parity.check_codes(WB.astype(np.float64), UB.astype(np.float32), deadB, q, bits, 0, block)


def test_propagate_full_size_sampled(lib):
    """The 4096 x 4096 layer by 2048 tokens, the shape the benchmark times,
    in the launch configuration it uses (16-byte loads, XCD-banded tiles):
    sampled 32 x 32 blocks of Y against the oracle on the same rows of What
    and columns of X, within the bound of the arithmetic."""
    from post_weight_quantization_04_amd import layer
    torch = _torch()
    M, K, N = 4096, 4096, 2048
    say("full size", M, K, N)
    rng = np.random.default_rng(2048)
    W = (rng.standard_normal((M, K), dtype=np.float32) * 0.02).astype(np.float16)
    X = rng.standard_normal((K, N), dtype=np.float32).astype(np.float16)
    Yd = layer.propagate(torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda(), relu=True)
    torch.cuda.synchronize()
    Y = Yd.cpu().numpy().astype(np.float64)
    for trial in range(4):
        rows = np.sort(rng.choice(M, 32, replace=False))
        cols = np.sort(rng.choice(N, 32, replace=False))
        Wr, Xc = W[rows], X[:, cols]
        ref = oracle.propagate(Wr, Xc, "relu")
        got = Y[np.ix_(rows, cols)]
        assert np.all(np.abs(got - ref) <= bound(Wr, Xc, ref)), trial
    assert np.all(Y >= 0.0) and np.isfinite(Y).all()
