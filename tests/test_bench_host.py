"""Host-side behaviour of bench.py (no GPU): more than one GPU is refused with a
message, and the HBM traffic records are used only while the kernel source they were
measured on is unchanged as the library compiles it (the timeline build's marks aside)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_traffic_records_follow_the_source_hash(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    key = "decode1/gate_up"
    import hashlib
    text = open(os.path.join(ROOT, recs[key]["source"])).read()
    cur = hashlib.sha256(bench.library_source(text).encode()).hexdigest()
    got = bench.traffic_record(key)
    if cur == recs[key]["source_sha256"]:                 # counters taken on this source
        assert got is not None and got["bytes_per_launch"] == recs[key]["bytes_per_launch"]
    else:
        assert got is None
    # the same record against another copy of the source: no longer valid
    src = tmp_path / "src.hip"
    src.write_bytes(open(os.path.join(ROOT, recs[key]["source"]), "rb").read() + b"\n// changed\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = dict(recs[key], source=str(src))
    (prof / "traffic.json").write_text(json.dumps({key: rec}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_record(key) is None
    # timeline marks added or removed leave the compiled source, and the record, as they were
    src.write_text(bench.library_source(text).replace("\n}\n", "\n    MQ_TL(GU, 0, 0);\n}\n", 1) +
                   "#ifdef MQ_WG_TIMELINE\nint x;\n#if 1\n#endif\n#endif\n")
    assert bench.library_source(src.read_text()) == bench.library_source(text)
    assert (bench.traffic_record(key) is not None) == (cur == recs[key]["source_sha256"])
    assert bench.traffic_record("no/such") is None
