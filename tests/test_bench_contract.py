"""bench.py contract checks that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr and r.stdout == ""


def test_counter_summary_is_tied_to_kernel_source():
    sys.path.insert(0, ROOT)
    import bench
    data = json.load(open(os.path.join(ROOT, "profiles", "hbm_counters.json")))
    rec = data["adam_update"]["gpt_1t_nd1024_last_rank"]
    # the algorithmic bytes recorded with the counters are 28 B/param of the shard
    assert rec["algorithmic_bytes"] == 28 * 976077312
    if rec["kernel_code_sha256_16"] == bench.kernel_source_hash():
        assert bench.measured_traffic("gpt_1t_nd1024_last_rank") == rec["bytes_per_launch"]
    else:
        assert bench.measured_traffic("gpt_1t_nd1024_last_rank") is None


def test_code_hash_ignores_comments_only():
    sys.path.insert(0, ROOT)
    import bench
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    b = "/* header */\nint f(int x) {\n\n    return x + 1;  // a different comment\n}\n"
    c = "int f(int x) {\n    return x + 2;  // one more\n}\n"
    assert bench.code_hash(a) == bench.code_hash(b) != bench.code_hash(c)


class _FakeEvent:
    """Stands in for a timing event: record() stamps the next tick."""
    clock = 0

    def __init__(self):
        self.t = None

    def record(self):
        _FakeEvent.clock += 1
        self.t = _FakeEvent.clock

    def elapsed_time(self, other):
        return float(other.t - self.t)


def test_step_marks_record_only_after_work():
    """A mark records a new event only when work was enqueued since the last
    recorded one; a step can start at the previous step's last event."""
    import bench
    pool = [_FakeEvent() for _ in range(8)]
    a = bench.StepMarks(pool)
    a.mark("start")
    a.mark("norm0")                           # nothing enqueued: the same event
    assert a.ev["start"] is a.ev["norm0"] and len(pool) == 7
    a.enqueued()
    a.mark("norm1")
    a.mark("upd0")
    assert a.ev["norm1"] is a.ev["upd0"] is not a.ev["norm0"] and len(pool) == 6
    a.enqueued()
    a.mark("upd1")
    assert a.ms("start", "upd1") == 2.0 and a.ms("norm0", "norm1") == 1.0 and a.ms("upd0", "upd1") == 1.0
    b = bench.StepMarks(pool, a.ev["upd1"])   # the next step starts where this one ended
    b.mark("start")
    assert b.ev["start"] is a.ev["upd1"] and len(pool) == 5
    b.enqueued()
    b.mark("upd1")
    assert b.ms("start", "upd1") == 1.0 and len(pool) == 4
