"""Host logic of bench.py (CPU only): the kernel-source hash that keeps the
committed HBM counters tied to the code they were taken on, the rule that
`traffic` is reported only while that hash (and the element count or GEMM
shape) match, and the rank-share split of the Llama-3-8B list."""

import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _hash_of(tmp_path, monkeypatch, text):
    f = tmp_path / "k.hip"
    f.write_text(text)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(f)])
    return bench.source_hash()


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    code = "int f(int x) {\n  return x + 1;\n}\n"
    h0 = _hash_of(tmp_path, monkeypatch, code)
    assert _hash_of(tmp_path, monkeypatch, "// a comment\n" + code) == h0
    assert _hash_of(tmp_path, monkeypatch, "/* block\n comment */ " + code.replace("  ", "    ")) == h0
    assert _hash_of(tmp_path, monkeypatch, code.replace("x + 1", "x + 2")) != h0


def test_traffic_only_for_matching_code_and_size(tmp_path, monkeypatch):
    doc = {"source_hash": "abc", "n_elems": 100, "hbm_bytes_per_launch": 2200.0}
    (tmp_path / "adamw_sr_w_hbm_counters.json").write_text(json.dumps(doc))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda: "abc")
    assert bench.traffic_from_profile("w", 100) == 2200.0
    assert bench.traffic_from_profile("w", 101) is None        # another workload size
    assert bench.traffic_from_profile("other", 100) is None    # no counters for it
    monkeypatch.setattr(bench, "source_hash", lambda: "def")
    assert bench.traffic_from_profile("w", 100) is None        # kernel code changed


def test_gemm_traffic_only_for_matching_code_and_shape(tmp_path, monkeypatch):
    doc = {"source_hash": "abc", "shape": [8, 16, 32], "hbm_bytes_per_launch": 1234.0}
    (tmp_path / "gemm_bf16_sr_8x16x32_hbm_counters.json").write_text(json.dumps(doc))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "abc")
    assert bench.gemm_traffic_from_profile(8, 16, 32) == 1234.0
    assert bench.gemm_traffic_from_profile(8, 16, 40) is None     # no counters for that shape
    monkeypatch.setattr(bench, "gemm_source_hash", lambda: "def")
    assert bench.gemm_traffic_from_profile(8, 16, 32) is None     # kernel code changed


def test_committed_gemm_counters_are_consistent():
    path = os.path.join(ROOT, "profiles", "gemm_bf16_sr_8192x14336x4096_hbm_counters.json")
    with open(path) as fh:
        doc = json.load(fh)
    m, n, k = doc["shape"]
    assert doc["algorithmic_bytes_per_launch"] == 2 * (m * k + n * k + m * n)
    total = doc["read_bytes_per_launch"]["sr"] + doc["write_bytes_per_launch"]["sr"]
    assert abs(doc["hbm_bytes_per_launch"] - total) <= 2
    # at least the output is written, and at least A and B are read
    assert doc["write_bytes_per_launch"]["sr"] >= 2 * m * n
    assert doc["read_bytes_per_launch"]["sr"] >= 2 * (m + n) * k


def test_committed_counters_describe_the_llama_list():
    path = os.path.join(ROOT, "profiles", "adamw_sr_llama3_8b_hbm_counters.json")
    with open(path) as fh:
        doc = json.load(fh)
    assert doc["n_elems"] == 8030261248
    # scaled counter bytes equal the algorithmic 22 B/element to within 0.1%
    assert abs(doc["hbm_bytes_per_launch"] / (22 * doc["n_elems"]) - 1) < 1e-3


@pytest.mark.parametrize("name,hash_fn,per_elem", [
    ("cvt_f32_bf16_sr_2pow30_hbm_counters.json", "source_hash", 6),
    ("rng_dropout_2pow30_hbm_counters.json", "rng_source_hash", 9)])
def test_committed_streaming_counters_are_current_and_reported(name, hash_fn, per_elem):
    """The conversion's and dropout's counter summaries were taken on the
    current sources, their scaled bytes match the algorithmic ones to within
    0.1%, and the benchmark reports them; a stale hash or another size gives
    None."""
    import bench
    path = os.path.join(ROOT, "profiles", name)
    with open(path) as fh:
        doc = json.load(fh)
    n = doc["n_elems"]
    assert doc["algorithmic_bytes_per_launch"] == per_elem * n
    assert abs(doc["hbm_bytes_per_launch"] / (per_elem * n) - 1) < 1e-3
    assert abs(doc["read_bytes_per_launch"] + doc["write_bytes_per_launch"]
               - doc["hbm_bytes_per_launch"]) <= 2
    now = getattr(bench, hash_fn)()
    assert doc["source_hash"] == now
    assert bench.stream_traffic_from_profile(name, now, n) == doc["hbm_bytes_per_launch"]
    assert bench.stream_traffic_from_profile(name, "0" * 16, n) is None
    assert bench.stream_traffic_from_profile(name, now, n + 1) is None


def test_rank_pieces_partition_the_list():
    """The ranks' pieces cover the flattened Llama-3-8B list exactly once,
    in order, each piece inside its tensor with base_index = the tensor's
    running total of numel + the piece's offset."""
    from adamw_optimizer_stochastic_amd import workloads as wl
    shapes = wl.llama3_8b_shapes()
    starts, pos = {}, 0
    for name, shape in shapes:
        starts[name] = (pos, wl.numel(shape))
        pos += wl.numel(shape)
    for ranks in (1, 3, 8):
        nxt = 0
        for r in range(ranks):
            pieces = wl.llama3_8b_rank_pieces(r, ranks)
            assert sum(p[3] for p in pieces) in (pos // ranks, pos // ranks + 1)
            for name, shape, off, n, base in pieces:
                t0, tn = starts[name]
                assert 0 <= off and off + n <= tn and n > 0
                assert base == t0 + off == nxt
                nxt = base + n
        assert nxt == pos
    assert len(wl.llama3_8b_rank_pieces(3, 8)) == 42
