"""Host-side pieces of bench.py: counter summaries and the traffic lookup."""
import json
import os

import bench


def _write_summary(tmp_path, config, sha, traffic=123):
    rec = {"kernel_source_sha256": sha, "traffic_bytes": traffic}
    p = tmp_path / f"{bench.ATTN_KERNEL}_{config}_pmc.md"
    p.write_text("# x\n\n```json pmc-summary\n" + json.dumps(rec) + "\n```\n")


def test_traffic_used_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.profile_traffic("c3") is None                     # no summary
    _write_summary(tmp_path, "c3", bench.kernel_source_sha256(), 777)
    assert bench.profile_traffic("c3")["traffic_bytes"] == 777
    _write_summary(tmp_path, "c3", "0" * 64)                       # kernel changed since
    assert bench.profile_traffic("c3") is None


def test_committed_summaries_parse():
    for name in os.listdir(bench.PROFILES):
        if name.endswith("_pmc.md"):
            text = open(os.path.join(bench.PROFILES, name)).read()
            start = text.index("```json pmc-summary")
            body = text[text.index("\n", start) + 1:text.index("```", start + 3)]
            rec = json.loads(body)
            assert abs(rec["traffic_bytes"] - rec["fetch_bytes"] - rec["write_bytes"]) <= 1
            assert 0.9 < rec["traffic_over_algorithmic"] < 2.0


def test_algorithmic_bytes_c3():
    from prefix_shared_kv_tree_amd import binding as B
    from prefix_shared_kv_tree_amd import workloads as W
    w = W.make_config("c3", with_kv=False)
    t = B.pkvt_tree_create(w.h, w.d, w.c, 1 << 16)
    ids, _ = B.pkvt_tree_build(t, w.all_seq_tokens())
    B.pkvt_plan(t, ids)
    info = B.pkvt_plan_info_get(t)
    B.pkvt_tree_destroy(t)
    unique, attn = bench.algorithmic_bytes(w, info)
    assert unique == W.unique_tokens(w) * 32 * 128 * 4          # 16 KiB per distinct token
    assert attn == unique + 64 * 32 * 128 * 2 + info["slots"] * 32 * 130 * 4 + \
        (64 - info["merge_rows"]) * 32 * 128 * 2


def test_cpu_baseline_single_and_all_cores():
    """The oracle's CPU baseline: a single-thread figure on a sample and an
    all-cores figure over every sequence, both for the same layer."""
    from prefix_shared_kv_tree_amd import workloads as W
    w = W.make_config("tiny")
    unique = W.unique_tokens(w) * w.h * w.d * 4
    r = bench.cpu_baseline(w, unique, 0.05)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert 1 <= r["cores"] <= min(bench.oracle_cores(), w.b)
    assert r["value"] > 0 and r["single_thread_value"] > 0
    assert r["ms_per_layer"] > 0
