"""bench.py's byte model, the numerator of the roofline figure, checked on
the CPU against a hand count of its terms at the headline shape (batch 8,
12 heads, n 4096, d 64, bf16, one graph per batch element of 1,294,208
edges each, K = 5):

- every edge weight of every (b, h) pair is read once per diffusion step
  and written once by the score pass, 2 bytes each;
- each graph's CSR (4-byte column, 8-byte row offset) is read once per pass;
- the score pass reads Q and K; each diffusion step reads Z_k and V and
  writes Z_{k+1}, except that the first step's Z_0 is V itself, read once.
"""
from __future__ import annotations

import bench


class _Graph:
    def __init__(self, nnz, num_graphs):
        self.nnz = [nnz] * num_graphs

    def edges(self, B, H):
        return sum(H * self.nnz[b if len(self.nnz) == B else 0] for b in range(B))


class _Workload:
    B, H, n, d, dtype = 8, 12, 4096, 64, "bf16"


def test_headline_byte_model():
    g = _Graph(1_294_208, 8)
    score, diffusion = bench.algorithmic_bytes(_Workload, g, 5)
    weights = 8 * 12 * 1_294_208 * 2            # 248,487,936
    csr = 8 * (1_294_208 * 4 + 4097 * 8)        # 41,676,864
    tensor = 8 * 12 * 4096 * 64 * 2             # one of Q, K, V, Z: 50,331,648
    assert weights == 248_487_936 and csr == 41_676_864 and tensor == 50_331_648
    assert score == 2 * tensor + weights + csr == 390_828_096
    # steps 1..4: Z_k, V in and Z_{k+1} out; step 0: V (= Z_0) in once, Z_1 out
    assert diffusion == 5 * (weights + csr) + 4 * 3 * tensor + 2 * tensor == 2_155_467_072
    assert diffusion / 5 == 431_093_414.4


def test_byte_model_fp32_shared_graph():
    """fp32 storage doubles the tensor and weight terms, not the graph's;
    one graph shared by the whole batch is counted once."""
    class W32(_Workload):
        B, dtype = 2, "f32"
    g = _Graph(1000, 1)
    score, diffusion = bench.algorithmic_bytes(W32, g, 1)
    tensor = 2 * 12 * 4096 * 64 * 4
    weights = 2 * 12 * 1000 * 4
    csr = 1000 * 4 + 4097 * 8
    assert score == 2 * tensor + weights + csr
    assert diffusion == weights + csr + 2 * tensor


def test_multi_gpu_request_exits_with_message():
    """The path runs on one GPU; asking bench.py for more exits (status 2)
    with a message, before anything touches a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "8"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_cpu_baseline_legs(monkeypatch):
    """The CPU baseline times the oracle on one thread and on every core the
    process may use, stages apart, and reports that core count."""
    from workloads import WORKLOADS, make_qkv
    monkeypatch.setenv("OMP_NUM_THREADS", "2")
    assert bench.host_cores() <= 2
    w = WORKLOADS["small_f32"]
    q, k, v = make_qkv(w)
    out = bench.cpu_baseline(w, q, k, v, budget_s=0.01, max_pairs=1)
    cores = bench.host_cores()
    assert out["kind"] == "oracle" and out["unit"] == "edges/s" and out["cores"] == cores
    assert out["one_thread"]["threads"] == 1 and out["one_thread"]["pairs"] == 1
    assert out["all_cores"]["threads"] == cores and out["value"] == out["all_cores"]["value"]
    for leg in (out["one_thread"], out["all_cores"]):
        assert leg["value"] > 0
        assert leg["score_softmax_s_per_pair"] > 0 and leg["diffusion_s_per_pair"] > 0
