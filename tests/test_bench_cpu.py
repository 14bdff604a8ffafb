"""bench.py's byte accounting (the denominator of every bandwidth it
reports) against sizes worked out by hand for the named workloads, and its
one-GPU contract.  No GPU needed."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _spec_only(name):
    """The layer specs of a workload without building its tensors."""
    r = synth.WORKLOADS[name]
    d = r["dims"]
    return dict(hidden=d["hidden"], n_q_heads=d["n_q_heads"], n_kv_heads=d["n_kv_heads"],
                head_dim=d["head_dim"], n_experts=d["n_experts"], top_k=d["top_k"],
                ffn_dim=d["ffn_dim"], window=r["windows"][0], dense_dtype=r["dense"],
                expert_dtype=r["expert"], kv_dtype=r["kv"])


def test_decode_bytes_by_hand():
    """hidden 6144, 48 q / 8 kv heads of 128, 256 experts of FFN 2048, bf16;
    one token with 8 distinct experts over a 2048-position window of a
    2048-position bf16 cache."""
    spec = _spec_only("decode-bf16")
    topk = [np.arange(8).reshape(1, 8)]
    total, parts = bench.algorithmic_bytes([spec], [2048], 1, topk)
    # wq + wk + wv: 8192 x 6144 bf16; wo: 6144 x 6144; router: 256 x 6144;
    # gains: attn and ffn norms (2 x 6144 fp32), q and k norms (2 x 128)
    dense = 100_663_296 + 75_497_472 + 3_145_728 + 50_176
    assert parts["dense"] == dense == 179_356_672
    # 8 experts x (gate + up + down) x 2048 x 6144 bf16
    assert parts["experts"] == 603_979_776
    # the window covers positions 1 .. 2048 (the new token at 2048): 2048
    # positions x 8 heads x 128 x 2 B, K and V
    assert parts["kv"] == 8_388_608
    assert total == dense + 603_979_776 + 8_388_608


def test_nvfp4_expert_bytes_by_hand():
    """An NVFP4 matrix of 2048 x 6144: 4-bit codes, one e4m3 scale per 16
    elements and one fp32 scale."""
    spec = _spec_only("stack4-nvfp4")
    gu, dn = bench.expert_bytes(spec)
    one = 6_291_456 + 786_432 + 4
    assert (gu, dn) == (2 * one, one)


def test_window_union_by_hand():
    """8 drafts after 65536 cached positions under a 2048 window: the first
    draft's window starts at 65536 - 2047, the last draft sits at 65543."""
    spec = dict(window=2048)
    assert bench.union_kv_positions(spec, [65536], 8) == 65543 - 63489 + 1
    spec = dict(window=0)
    assert bench.union_kv_positions(spec, [0, 5], 3) == 3 + 8


def test_distinct_experts_counted_once():
    spec = _spec_only("verify-bf16-128k")
    topk = [np.array([[1, 2, 3, 4, 5, 6, 7, 8], [8, 7, 6, 5, 4, 3, 2, 1]])]
    _, parts = bench.algorithmic_bytes([spec], [131072, 131072], 1, topk)
    assert parts["experts"] == 8 * sum(bench.expert_bytes(spec))


def test_prefill_accounting_by_hand():
    """Hidden 6144, FFN 2048: 300 slots on expert 0, 128 on expert 1, 161 on
    expert 5, none elsewhere.  NVFP4 experts take chunks of up to 160 slots
    (two, one and two chunks), bf16 experts chunks of up to 128 (three, one,
    two)."""
    spec = _spec_only("stack4-nvfp4")
    counts = np.zeros(256, dtype=np.int64)
    counts[[0, 1, 5]] = [300, 128, 161]
    flops, distinct, streamed = bench.prefill_accounting(spec, counts)
    # gate and up: 2 flops x 589 slots x 4096 rows x 6144; down: x 6144 x 2048
    assert flops["gateup"] == 2 * 589 * 4096 * 6144
    assert flops["down"] == 2 * 589 * 6144 * 2048
    one = 6_291_456 + 786_432 + 4          # one NVFP4 matrix of 2048 x 6144
    assert distinct == 3 * 3 * one
    assert streamed == (2 + 1 + 2) * 3 * one
    spec = dict(spec, expert_dtype="bf16")
    one = 2048 * 6144 * 2                  # one bf16 matrix
    _, distinct, streamed = bench.prefill_accounting(spec, counts)
    assert distinct == 3 * 3 * one
    assert streamed == (3 + 1 + 2) * 3 * one


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
