"""Host-side logic of bench.py, checked on the CPU: the algorithmic bytes and
flops that the roofline figures divide by (against closed forms written out
from the workload shapes), which steps write inside the decode launch, and
the hash gate of the committed HBM-traffic record."""

import json
import math
import os

import pytest

import bench
import workloads as wl

PER_TOKEN_BYTES = 128 + 128 + 4 + 4  # K and V codes, K and V scales per (token, KV head)


def test_algorithmic_bytes_128k_dense():
    # 32 requests of 131072 tokens, one KV head: every token's K/V codes and
    # scales, q and out (bf16, 16 query heads x 128), 1024 table entries and
    # one context length per request
    kv, total = bench.algorithmic_bytes(bench.CONFIGS["c3"]())
    assert kv == 32 * 131072 * PER_TOKEN_BYTES
    assert total == kv + 2 * 32 * 16 * 128 * 2 + 4 * 32 * 1024 + 4 * 32 == 1_107_689_600


def test_algorithmic_bytes_8k_dense():
    w = bench.CONFIGS["c2"]()
    kv, total = bench.algorithmic_bytes(w)
    ctx = [int(c) for c in w.ctx]
    assert kv == sum(ctx) * PER_TOKEN_BYTES
    pages = sum(math.ceil(c / 128) for c in ctx)
    assert total == kv + 2 * 4 * 16 * 128 * 2 + 4 * pages + 4 * 4


def test_algorithmic_bytes_block_sparse():
    # 16 rows, each listing 32 full pages of its 131072-token request: the
    # listed pages' tokens, q/out, the list entries (read) and their table
    # entries, and the context lengths
    w = bench.CONFIGS["c5"]()
    kv, total = bench.algorithmic_bytes(w)
    assert kv == 16 * 32 * 128 * PER_TOKEN_BYTES
    assert total == kv + 2 * 16 * 16 * 128 * 2 + 4 * 512 + 4 * 16 + 4 * 512


def test_algorithmic_flops_16k_prompt():
    # row i of a 16384-row prompt sees i + 1 tokens: T(T+1)/2 (row, token)
    # pairs, each 16 heads x (128 multiply-adds for the score + 128 for V)
    T = 16384
    assert bench.algorithmic_flops(bench.CONFIGS["p16k"]()) == T * (T + 1) // 2 * 16 * 128 * 4


@pytest.mark.parametrize("kw, sparse, separate, expect", [
    (dict(ctx=[300], q_lens=[1]), 0, False, True),
    (dict(ctx=[300, 400], q_lens=[16, 16]), 0, False, True),
    (dict(ctx=[300, 400], q_lens=[17, 17]), 0, False, False),    # above the fused limit
    (dict(ctx=[300, 400], q_lens=[1, 1]), 0, True, False),       # the separate writer asked for
    (dict(ctx=[3000, 4000], q_lens=[1, 1]), 3, False, True),     # block-sparse, one row per request
    (dict(ctx=[3000, 4000], q_lens=[2, 2]), 3, False, False),    # block-sparse, two rows
])
def test_which_steps_write_inside_the_decode(kw, sparse, separate, expect):
    w = wl.small_case(seed=1, sparse_topk=sparse, **kw)
    assert bench.write_in_decode(w, separate, 0) is expect
    assert bench.write_in_decode(wl.bf16_kv(w), separate, 0) is expect  # over a bf16 cache too


def test_traffic_record_is_current():
    """Every workload in the committed record carries a kernel whose sources
    still hash to the recorded digest, so the bench reports its traffic."""
    rec = json.load(open(os.path.join(bench.ROOT, "profiles", "pa_decode_main_traffic.json")))
    assert rec["workloads"]
    for name, e in rec["workloads"].items():
        assert e["kernel"] in bench.KERNEL_SOURCES, name
        assert e["source_sha256"] == bench.sources_sha256(e["kernel"]), f"{name}: counters predate the sources"
        fetch, write = e["fetch_kib"], e["write_kib"]
        expect = int(round((fetch * rec["fetch_scale"] + write * rec["write_scale"]) * 1024))
        assert e["traffic_bytes_per_launch"] == expect, name
        assert bench.recorded_traffic(name) == expect, name


def test_traffic_record_gate(tmp_path, monkeypatch):
    """The bench reports a recorded workload's traffic while its kernel's
    sources hash to the recorded digest, and none once a source byte
    changes or for a workload the record does not hold."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "k.hip").write_text("kernel A\n")
    monkeypatch.setitem(bench.KERNEL_SOURCES, "probe_kernel", ("k.hip",))
    (tmp_path / "profiles").mkdir()
    rec = {"fetch_scale": 2.0, "write_scale": 1.0, "workloads": {"w": {
        "kernel": "probe_kernel", "source_sha256": bench.sources_sha256("probe_kernel"),
        "fetch_kib": 1.0, "write_kib": 1.0, "traffic_bytes_per_launch": 3072}}}
    (tmp_path / "profiles" / "pa_decode_main_traffic.json").write_text(json.dumps(rec))
    assert bench.recorded_traffic("w") == 3072
    assert bench.recorded_traffic("no_such_workload") is None
    (tmp_path / "k.hip").write_text("kernel B\n")
    assert bench.recorded_traffic("w") is None
