"""Host checks of bench.py (no GPU): the one-GPU refusal, the algorithmic
work it divides by measured time, and the gate on the recorded HBM traffic.

The flop counts are checked against closed forms, not against the
formulas they are written with:
  - H = 2 X X^T as a symmetric rank-N update: d_in (d_in + 1) N flops
    (aicassindra.com "tm_gptq_math", "Why it is second-order");
  - the lazy trailing update W[:, b1:] -= E U[b0:b1, b1:] summed over the
    blocks of width B: d_out * d_in * (d_in - B) when B divides d_in
    ("GPTQ's speedups: fixed order and lazy batches");
  - the factorization and the inverse factor together: 2 d^3 / 3 to leading
    order ("The Cholesky trick for the inverse Hessian").
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


@pytest.mark.parametrize("d_in,n_tok", [(64, 512), (4096, 2048), (11008, 16384)])
def test_hessian_flops_are_a_symmetric_rank_n_update(d_in, n_tok):
    assert bench.algorithmic_flops("hessian_f16", 7, d_in, n_tok, 128) == d_in * (d_in + 1) * n_tok


@pytest.mark.parametrize("d_out,d_in,block", [(4096, 4096, 128), (4096, 11008, 128), (64, 128, 32), (5, 96, 32)])
def test_trailing_update_flops_closed_form(d_out, d_in, block):
    assert d_in % block == 0
    got = bench.algorithmic_flops("q_step", d_out, d_in, 2048, block)
    assert got == d_out * d_in * (d_in - block)
    assert bench.algorithmic_flops("q_trail", d_out, d_in, 2048, block) == 0.0


def test_group_starts_move_their_update_to_the_trail_kernel():
    """Groups wider than the block: the update at each group start is
    counted under q_trail, and the two parts add up to the whole."""
    d_out, d_in, block, group = 64, 1024, 128, 256
    step = bench.algorithmic_flops("q_step", d_out, d_in, 0, block, group)
    trail = bench.algorithmic_flops("q_trail", d_out, d_in, 0, block, group)
    assert trail > 0 and step + trail == d_out * d_in * (d_in - block)


def test_factorization_flops_leading_order():
    ratios = []
    for n in (1024, 4096, 16384):
        r = bench.algorithmic_flops("chol_step", 1, n, 0, 128) / (2.0 * n ** 3 / 3.0)
        assert 1.0 <= r < 1.0 + 6.0 * bench.NB / n
        ratios.append(r)
    assert ratios[0] > ratios[1] > ratios[2]  # lower-order terms fade as d grows


def test_recorded_traffic_needs_a_matching_source_hash_and_workload(tmp_path, monkeypatch):
    rec = {"workload": "attn_proj: 4096x4096 layer",
           "kernels": {"chol_step": {"bytes_per_launch": 12345,
                                     "source_sha256": bench.kernel_source_sha("chol_step")}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic("chol_step", "attn_proj") == 12345
    assert bench.recorded_traffic("chol_step", "mlp_down") is None         # taken on another workload
    assert bench.recorded_traffic("q_step", "attn_proj") is None           # not in the record
    assert bench.recorded_traffic("no_such_kernel", "attn_proj") is None   # not a known class
    monkeypatch.setattr(bench, "kernel_source_sha", lambda name: "0" * 64)
    assert bench.recorded_traffic("chol_step", "attn_proj") is None        # source changed since the counters


def test_committed_traffic_record_names_its_workload():
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert rec["workload"].split(":")[0].strip() == "attn_proj"


def test_every_traffic_class_names_an_existing_kernel():
    csrc = os.path.join(ROOT, "post_weight_quantization_04_amd", "csrc")
    for name, (src, symbol) in bench.KERNEL_SOURCE.items():
        with open(os.path.join(csrc, src)) as fh:
            assert symbol in fh.read(), (name, src, symbol)
