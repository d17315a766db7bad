"""The no-allocation factorization entry point against the ordinary one.

``gptq_prepare_hinv_noalloc`` runs the same kernels as ``gptq_prepare_hinv``
on a fixed device array inside the library, so every output must be
identical bit for bit: U, the dead flags, lambda and info.  Two calls in a
row, the second smaller than the first, show that what the first call left
in the shared array does not leak into the second; the U of each is also
checked against the fp64 oracle fed the same H (relative error <= 1e-4).
"""
import numpy as np
import pytest

import oracle
from post_weight_quantization_04_amd import _lib, layer

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _hessian(torch, d_in, n, seed, dead=()):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((d_in, n)) + rng.standard_normal((d_in, 8)) @ rng.standard_normal((8, n)) / np.sqrt(8)
    for d in dead:
        X[d] = 0.0
    Xd = torch.from_numpy(X.astype(np.float16)).cuda()
    return layer.hessian(Xd)


def _outputs(torch, d_in):
    return (torch.full((d_in, d_in), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((d_in,), 7, dtype=torch.uint8, device="cuda"),
            torch.full((1,), -5, dtype=torch.int32, device="cuda"),
            torch.full((1,), float("nan"), dtype=torch.float64, device="cuda"))


def test_noalloc_matches_prepare_hinv_on_two_calls(lib):
    import torch
    assert _lib.prepare_hinv_noalloc_max_din() == 4096
    # the largest order first, then a smaller ragged one with dead channels
    for d_in, n, seed, dead in ((4096, 2048, 11, ()), (1000, 1500, 12, (3, 500, 999))):
        say(f"noalloc prepare d_in={d_in} tokens={n} seed={seed} dead={dead}")
        H = _hessian(torch, d_in, n, seed, dead)
        U0, dead0, info0, lam0 = _outputs(torch, d_in)
        ws = torch.empty(_lib.prepare_hinv_workspace(d_in), dtype=torch.uint8, device="cuda")
        _lib.prepare_hinv(H, 0.01, U0, dead0, info0, lam0, ws)
        U1, dead1, info1, lam1 = _outputs(torch, d_in)
        _lib.prepare_hinv_noalloc(H, 0.01, U1, dead1, info1, lam1)
        torch.cuda.synchronize()
        assert int(info0.item()) == 0 and int(info1.item()) == 0
        assert torch.equal(U0.view(torch.int32), U1.view(torch.int32)), "U differs"
        assert torch.equal(dead0, dead1)
        assert lam0.item() == lam1.item()
        assert int(dead1.sum().item()) == len(dead)
        # against the oracle fed the same H (stage isolation)
        Hh = H.cpu().numpy().astype(np.float64)
        Hs = np.tril(Hh) + np.tril(Hh, -1).T
        U_ref, dead_ref, lam_ref = oracle.prepare(Hs, 0.01)
        U = U1.cpu().numpy().astype(np.float64)
        err = np.linalg.norm(U - U_ref) / np.linalg.norm(U_ref)
        say(f"  U rel err vs oracle {err:.2e}")
        assert err <= 1e-4
        np.testing.assert_array_equal(dead1.cpu().numpy().astype(bool), dead_ref)
        assert lam1.item() == pytest.approx(lam_ref, rel=1e-12)
        del ws


def test_noalloc_rejects_orders_above_its_scratch(lib):
    import torch
    d_in = _lib.prepare_hinv_noalloc_max_din() + 1
    say(f"noalloc prepare d_in={d_in}: rejected before any launch")
    H = torch.zeros((8, 8), dtype=torch.float32, device="cuda")  # never read: the size check comes first
    U = torch.zeros((8, 8), dtype=torch.float32, device="cuda")
    info = torch.zeros((1,), dtype=torch.int32, device="cuda")
    rc = lib.gptq_prepare_hinv_noalloc(H.data_ptr(), d_in, 0.01, U.data_ptr(), None, info.data_ptr(), None, None)
    assert rc == _lib.GPTQ_ESCRATCH
    assert b"no-allocation" in lib.gptq_status_string(rc)
