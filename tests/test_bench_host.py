"""Host-side logic of bench.py (no GPU): the HIP-graph step count and the
lookup of committed HBM counters, which must only be reported for the kernel
sources they were taken on."""
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_graph_steps_divide_k():
    b = _bench()
    for K in (1, 2, 7, 20, 50, 99, 200, 1000):
        g = b.graph_steps(K)
        assert 1 <= g <= b.GRAPH_STEPS and K % g == 0
    assert b.graph_steps(200) == 20 and b.graph_steps(50) == 10 and b.graph_steps(7) == 7


def test_traffic_entries_match_their_sources(tmp_path):
    b = _bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for key, ent in rec.items():
        srcs = tuple(ent.get("sources", b.KERNEL_SOURCES))
        for rel in srcs:
            assert os.path.exists(os.path.join(ROOT, rel)), (key, rel)
        assert ent["read_bytes"] > 0 and ent["write_bytes"] > 0
    # an entry is reported only while its hash matches its own sources
    b.ROOT = str(tmp_path)
    os.makedirs(tmp_path / "profiles")
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    ent = {"read_bytes": 10, "write_bytes": 5, "sources": ["k.hip"]}
    ent["source_sha256_16"] = b.kernel_source_hash(("k.hip",))
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"radial/generation/sorted/0": ent}))
    assert b.measured_traffic("radial", "generation", False, 0) == 15
    assert b.measured_traffic("mid", "generation", False, 0) is None
    src.write_text("kernel v2")
    assert b.measured_traffic("radial", "generation", False, 0) is None
