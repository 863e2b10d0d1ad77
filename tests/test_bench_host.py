"""Host checks of bench.py's contract and byte accounting (no GPU).

The algorithmic bytes per op are the roofline's numerator; the figures
below are the per-config budgets derived from the workload sizes (inputs
read once, outputs written once) and must stay what bench.py reports."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench as b

    return b


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("op,alg", [
    ("uniform_enc", 852_096),          # 65,536 x (4 g + 4 e + 4 e' + 1 code) + 16 x 8 B of scale/zero
    ("uniform_dec", 327_808),
    ("fp8_enc", 644_000_000),          # 512 MB in -> 128 MB codes + 4 MB scales
    ("fp8_dec", 644_000_000),
    ("qsgd_enc", 12_507_812_500),      # 1e9 x 12.5 B + 1,953,125 norms
    ("qsgd_dec", 4_507_812_500),
    ("sign_enc", 2_718_171_136),       # 2^28 x (2 + 4 + 4 + 1/8) + 65,536 scales
    ("sign_vote", 570_425_344),        # 16 x 2^28 / 8 in + 2^28 / 8 out
    ("sign_dec", 1_107_558_400),
    ("acc_requant", 4_647_550_976),    # 64 x (2^26 + 32,768 x 8) + 4 x 2^26 + 2^26 + 32,768 x 8
])
def test_algorithmic_bytes(bench, op, alg):
    assert bench.op_bytes()[op][1] == alg


def test_input_bytes_of_the_step(bench):
    b = bench.op_bytes()
    assert b["qsgd_enc"][0] == 4 * 10 ** 9
    assert b["sign_enc"][0] == 2 * 2 ** 28          # bf16 input
    assert b["acc_requant"][0] == 4 * 64 * 2 ** 26  # M x n fp32 terms
    assert b["sign_vote"][0] == 16 * 2 ** 28 // 8   # packed bits of 16 workers


def test_tensor_list_is_a_24_layer_width_1024_transformer(bench):
    sizes = bench.tensor_list_sizes()
    assert len(sizes) == 288
    assert sum(sizes) == 302_309_376
    d = 1024
    assert sum(sizes[:12]) == 12 * d * d + 13 * d  # qkv, proj, two MLP weights; their biases and two norms


def test_counter_traffic_is_dropped_when_a_kernel_changes(bench, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert set(t["ops"]) == set(bench.ORDER + bench.EXT_ORDER)
    for op, e in t["ops"].items():
        assert e["algorithmic_bytes"] == bench.op_bytes()[op][1], op
        assert e["hbm_bytes"] == e["fetch_bytes"] + e["write_bytes"] or abs(
            e["hbm_bytes"] - e["fetch_bytes"] - e["write_bytes"]) <= 1, op
    monkeypatch.setattr(bench, "source_hash", lambda op: "0" * 16)
    assert all(bench.load_traffic(op) is None for op in t["ops"])


def test_host_cpu_is_reported(bench):
    n, model = bench.host_cpu()
    assert isinstance(n, int) and n >= 1
    assert isinstance(model, str) and model
