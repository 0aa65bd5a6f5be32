"""Host-side logic of bench.py (CPU only): the byte models, the lookup of committed
counter traffic, the budget statistics and the one-GPU guard."""
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from adaptive_kv_cache_amd.workloads import WORKLOADS  # noqa: E402


def _per_array_bytes(wl, n8, nw):
    """The attention's algorithmic bytes of one (layer, sequence), array by array."""
    H, d, Hq = wl.n_kv_heads, wl.head_dim, wl.n_q_heads
    k8 = v8 = H * n8 * d                      # INT8 codes
    k16 = v16 = H * nw * d * 2                # 16-bit window
    new_in = 2 * H * d * 2                    # this step's k and v read
    new_out = 2 * H * d * 2                   # and appended to the window
    amax = 2 * H * d * 4                      # the K and V absmax rows
    q_in, o_out = Hq * d * 2, Hq * d * 4
    return k8 + v8 + k16 + v16 + new_in + new_out + amax + q_in + o_out


def test_attn_bytes_sums_every_stream():
    wl = WORKLOADS["qwen32b_gqa_b8_32k"].scaled(n_layers=2, batch=3)
    n8 = torch.tensor([[3585, 3584, 100], [0, 1, 64]], dtype=torch.int64)
    nw = torch.tensor([[512, 511, 7], [0, 513, 32]], dtype=torch.int64)
    want = sum(_per_array_bytes(wl, int(a), int(b)) for a, b in zip(n8.flatten(), nw.flatten()))
    assert bench.attn_bytes(wl, n8, nw) == want


def test_step_bytes_adds_moves_and_demotion():
    wl = WORKLOADS["gpt2_12layer_b8_pyramid"].scaled(n_layers=1, batch=2)
    n8 = torch.tensor([[300, 10]], dtype=torch.int64)
    nw = torch.tensor([[128, 5]], dtype=torch.int64)
    plan = torch.zeros(1, 2, 16, dtype=torch.int64)
    plan[..., 5] = -1
    base = bench.step_bytes(wl, n8, nw, plan)
    plan[0, 0, 1] = 3       # three INT8 moves
    plan[0, 1, 3] = 2       # two window moves
    plan[0, 1, 5] = 7       # one demotion
    H, d = wl.n_kv_heads, wl.head_dim
    extra = 3 * (2 * 2 * H * d + 16) + 2 * (2 * 2 * H * d * 2 + 16) + (2 * H * d * 3 + 8)
    assert bench.step_bytes(wl, n8, nw, plan) == base + extra
    # the attention part is attn_bytes; the rest is the logits, the EMA and the positions
    n = n8 + nw + 1
    assert base == (bench.attn_bytes(wl, n8, nw) + wl.batch * wl.vocab * 4
                    + int((8 * n + 4).sum()) + int((4 * n).sum()))


def test_ingest_bytes():
    wl = WORKLOADS["qwen14b_gqa_b8_8k"].scaled(n_layers=3, batch=2)
    st = bench.ingest_stats(wl, 2.0)
    units = 3 * 2 * wl.n_kv_heads
    n8, nw = wl.prefill - wl.window, wl.window
    # the 16-bit prefill read once, the INT8 codes and the 16-bit window written
    want = units * wl.head_dim * (2 * 2 * (n8 + nw) + 2 * n8 + 2 * 2 * nw)
    assert st["bytes"] == want
    assert st["GBs"] == round(want / 2e-3 / 1e9, 1)


def test_budget_stats():
    wl = WORKLOADS["qwen32b_gqa_b8_32k"]
    b0 = torch.tensor([[wl.n_high, wl.n_low], [wl.n_high, wl.n_high], [wl.n_low, wl.n_high]])
    s = bench.budget_stats(b0, wl)
    assert s["confident_fraction"] == round(4 / 6, 4)
    assert s["flip_rate"] == 0.5          # one of the two sequences changes at each step


def test_stored_traffic_matches_only_its_regime(tmp_path, monkeypatch):
    h = bench.attn_source_hash()
    (tmp_path / "attn_traffic_x.md").write_text(
        "text\n"
        f"traffic: workload=w1 steps=20 warmup=5 tokens=4097.0 source={h} bytes_per_launch=123\n"
        f"traffic: workload=w1 steps=384 warmup=128 tokens=2065.3 source=0000 bytes_per_launch=9\n")
    (tmp_path / "other.md").write_text(
        f"traffic: workload=w2 steps=1 warmup=1 tokens=1.0 source={h} bytes_per_launch=7\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic("w1", 20, 5, 4097.0) == 123
    assert bench.stored_traffic("w1", 21, 5, 4097.0) is None     # other timed steps
    assert bench.stored_traffic("w1", 20, 6, 4097.0) is None     # other warm-up
    assert bench.stored_traffic("w1", 20, 5, 4096.9) is None     # other cache size
    assert bench.stored_traffic("w1", 384, 128, 2065.3) is None  # other attention sources
    assert bench.stored_traffic("w2", 1, 1, 1.0) is None         # not an attn_traffic_ file
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "missing"))
    assert bench.stored_traffic("w1", 20, 5, 4097.0) is None


def test_committed_traffic_lines_name_the_current_sources():
    """Every committed counter line of the headline workload is for the attention
    sources as they are (a stale line would be reported as null, not as traffic)."""
    assert bench.stored_traffic("qwen32b_gqa_b8_32k", 20, 5, 4097.0) is not None
    assert bench.stored_traffic("qwen32b_gqa_b8_32k", 384, 128, 2065.3) is not None
    assert bench.stored_traffic("gptoss20b_gqa_b32_16k", 384, 128, 1036.4) is not None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
