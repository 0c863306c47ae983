"""The benchmark's command line on a host (no GPU needed): more than one GPU
is refused with an explanation before any GPU work, whether asked for with
--gpus or by a multi-process launcher's WORLD_SIZE."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    res = _run(["--gpus", "2"])
    assert res.returncode == 2, res.stderr
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def test_multi_process_launch_is_refused():
    res = _run([], {"WORLD_SIZE": "4"})
    assert res.returncode == 2, res.stderr
    assert "--gpus 4 is not supported" in res.stderr


# --------------------------------------------- the bench's host-side helpers
sys.path.insert(0, ROOT)


def test_launch_stats_flags_outliers():
    import bench
    per_ms = [0.0636] * 19 + [1.2]  # one launch 19x slower than the rest
    st = bench.launch_stats(per_ms)
    assert st["launches"] == 20 and st["median"] == 63.6 and st["min"] == 63.6 and st["max"] == 1200.0
    assert st["outliers"]["count"] == 1 and st["outliers"]["index_us"] == [(19, 1200.0)]
    assert st["mean"] > 100 and st["mean_without_outliers"] == 63.6


def test_comparison_rules_of_the_bench():
    """Bitwise for sums and pre-norm sums, ulp distance across zero for the
    normed output (+0 and -0 are the same value)."""
    import numpy as np

    import bench
    from tensor_all_reduce_ar_amd import inputs
    w = inputs.random_fused("bf16", 2, 3, 16, 5)
    ref = np.array([0x3F80, 0x8000, 0x0001] * 16, np.uint16)
    got = ref.copy()
    got[1] = 0x0000           # -0 vs +0: 0 ulp
    got[2] = 0x8001           # smallest subnormals of either sign: 2 ulp apart
    rec = bench.compare_to_oracle(w, got, ref.copy(), ref, ref)
    # relative error floored at the smallest normal: 2^-132 apart / 2^-126
    assert rec == {"intermediate_bitexact": True, "output_max_ulp": 2, "output_max_rel": 2.0 ** -6,
                   "within_tolerance": True}
    got[0] = 0x3F83           # 3 ulp above 1.0
    rec = bench.compare_to_oracle(w, got, ref.copy(), ref, ref)
    assert not rec["within_tolerance"] and rec["output_max_rel"] == 3 * 2.0 ** -7
    s = inputs.random_sum("fp32", 2, 8, 5)
    r32 = np.arange(8, dtype=np.float32)
    g = r32.view(np.uint32).copy()
    assert bench.compare_to_oracle(s, g, None, r32, None) == {"bitexact": True, "max_ulp": 0, "max_rel": 0.0}
    g[3] += 1                 # one ulp above 3.0
    assert bench.compare_to_oracle(s, g, None, r32, None) == {"bitexact": False, "max_ulp": 1,
                                                              "max_rel": 2.0 ** -22 / 3}


def test_all_core_oracle_leg_matches_one_thread():
    """The all-core leg splits rows (fused) or elements (sum) into blocks; the
    result must be bitwise the one-thread result."""
    import bench
    from tensor_all_reduce_ar_amd import inputs
    for w in (inputs.random_fused("fp16", 3, 37, 640, 9), inputs.random_sum("bf16", 5, 10007, 9)):
        o = bench.oracle_timed(w, 2, 2, 5.0)
        assert o["nt_bitexact"] and o["n1"] == 2 and o["nn"] == 2 and o["threads"] >= 1


def test_source_hash_follows_code_not_comments():
    """The traffic figures in the bench line are tied to this hash: a comment
    edit keeps it, any change to the code changes it."""
    import bench
    base = ["int f(int x) { return x + 1; } // one\n/* two */\n", "#define A 1\n", "x"]
    h = bench.source_hash(base)
    assert bench.source_hash(["int f(int x)  {\n return x + 1; }  // changed\n", "#define A 1 /* c */\n", "x"]) == h
    assert bench.source_hash(["int f(int x) { return x + 2; }\n", "#define A 1\n", "x"]) != h
    assert bench.source_hash(["int f(int x) { return x + 1; }\n", "#define A 2\n", "x"]) != h
