"""Host logic of bench.py (no GPU): the algorithmic byte counts behind the
roofline object, the one-GPU guard, and the source-hash check that keeps
counter summaries from being used once their kernel has changed."""
import hashlib
import os
import subprocess
import sys

import pytest

import bench
from workload import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("weights", ["mxfp4", "bf16"])
@pytest.mark.parametrize("shared", [False, True])
def test_kernel_bytes_reads_each_expert_once(weights, shared):
    """Weights: the two kernels together read every looked-up expert once,
    plus the shared expert once per call, split 2:1 (gate and up against
    down, three matrices of equal size).  Activations: x once, h written and
    read back as two bf16 planes, fp32 outputs written once."""
    sh = gen.Shape(H=256, I=512, E=8, k=2, shared=shared, weights=weights)
    lookups, calls, pairs, T_total = 7, 3, 12, 6
    gu, dn = bench.kernel_bytes(sh, lookups, calls, pairs, T_total)
    experts = lookups + (calls if shared else 0)
    rows = pairs + (T_total if shared else 0)
    b_e = sh.expert_bytes()
    w_gu = gu - T_total * sh.H * 2 - rows * sh.I * 4
    w_dn = dn - rows * sh.I * 4 - rows * sh.H * 4
    assert w_gu + w_dn == experts * b_e
    assert w_gu == 2 * w_dn
    # one matrix of H x I: 4.25 bits per weight in MXFP4, 16 in bf16
    per_matrix = sh.H * sh.I * (17 / 32 if weights == "mxfp4" else 2)
    assert w_dn == experts * per_matrix


def test_expert_bytes_at_the_stand_in_shapes():
    # three H x I matrices at 4 bits per weight plus one scale byte per 32
    want = {"tiny": 208_896, "a3b_decode": 1_671_168, "dsv4_decode": 13_369_344,
            "glm_decode": 20_054_016}
    for name, b in want.items():
        assert gen.WORKLOADS[name].shape.expert_bytes() == b


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_profile_fields_follow_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    (tmp_path / "profiles").mkdir()
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles" / "traffic_k_w.md").write_text(
        "# summary\n\n- source: `k.hip`\n- source_sha256: `%s`\n"
        "- hbm_bytes_per_launch: `1234`\n" % sha)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("k", "w") == 1234
    src.write_text("kernel v2\n")  # the kernel changed after the counters were taken
    assert bench.traffic_from_profile("k", "w") is None
    assert bench.traffic_from_profile("other", "w") is None  # no such summary
    assert bench.mfma_busy_from_profile() is None


def test_layer_bytes_adds_router_and_combine():
    """The layer's bytes are the expert kernels' plus the router (W_r once
    per call, token rows, bias, logits) and the combine (every fp32 expert
    row read once, y written in bf16)."""
    sh = gen.Shape(H=256, I=512, E=8, k=2, shared=True)
    lookups, calls, pairs, T_total = 7, 3, 12, 6
    gu, dn = bench.kernel_bytes(sh, lookups, calls, pairs, T_total)
    rows = pairs + T_total
    router = calls * sh.H * sh.E * 4 + T_total * (sh.H * 2 + 2 * sh.E * 4)
    combine = rows * sh.H * 4 + T_total * sh.H * 2
    assert bench.layer_bytes(sh, lookups, calls, pairs, T_total) == gu + dn + router + combine
    no_bias = bench.layer_bytes(sh, lookups, calls, pairs, T_total, bias=False)
    assert no_bias == gu + dn + router + combine - T_total * sh.E * 4


def test_check_pairs_lie_in_the_timed_steps():
    wl = gen.WORKLOADS["glm_decode"]
    for W, K, n in ((5, 20, 4), (0, 1024, 4), (3, 1, 4), (0, 7, 1)):
        pairs = bench.check_pairs_of(wl, W, K, n)
        assert pairs and all(W <= s < W + K and 0 <= l < wl.shape.layers for s, l in pairs)
        assert (W + K - 1) in {s for s, _ in pairs}
    assert bench.check_pairs_of(wl, 5, 20, 0) == []
