"""Host-side pieces of bench.py that decide what it reports: the code hash
that ties the committed HBM counters to the kernel sources, and the lookup
of those counters.  CPU only."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _bench():
    argv, sys.argv = sys.argv, ["bench.py"]
    try:
        import bench
    finally:
        sys.argv = argv
    return bench


def test_code_tokens_drop_comments_and_layout_only():
    t = _bench().code_tokens
    assert t('a = 1; // c\nb = "x // y"; /* z */ c') == 'a = 1; b = "x // y"; c'
    assert t("x = '\\'';  // q") == "x = '\\'';"
    assert t("a\n\n   b\t c") == "a b c"
    assert t('s = "/* not a comment */";') == 's = "/* not a comment */";'
    # a change of code changes the tokens
    assert t("a = 1;") != t("a = 2;")


def test_hash_ignores_comments_but_not_code():
    b = _bench()
    src = {p: open(p, encoding="utf-8").read() for p in b.KERNEL_SRCS}
    base = b.kernel_src_sha(lambda p: src[p])
    k = b.KERNEL_SRCS[0]
    assert b.kernel_src_sha(lambda p: src[p] + ("\n// a new comment\n" if p == k else "")) == base
    assert b.kernel_src_sha(lambda p: src[p] + ("\nstatic int zz_extra;\n" if p == k else "")) != base


def test_traffic_lookup_requires_matching_hash(tmp_path, monkeypatch):
    b = _bench()
    f = tmp_path / "hbm_traffic_w1.md"
    sha = b.kernel_src_sha()
    f.write_text(f"traffic: kernel=zs_adam_kernel workload=w1 src_sha256={sha} hbm_bytes_per_launch=123\n"
                 f"traffic: kernel=zs_reduce_kernel workload=w1 src_sha256=0000000000000000 hbm_bytes_per_launch=456\n")
    monkeypatch.setattr(b, "TRAFFIC_GLOB", str(tmp_path / "hbm_traffic_*.md"))
    assert b.measured_traffic("zs_adam_kernel", "w1") == 123.0
    assert b.measured_traffic("zs_reduce_kernel", "w1") is None      # taken on other code
    assert b.measured_traffic("zs_adam_kernel", "w2") is None        # another workload


def test_committed_counters_match_the_current_kernels():
    """profiles/hbm_traffic_*.md were taken on the kernels as they are now, so
    the default bench line carries measured HBM traffic for both kernels of
    the step, and the N_d = 8 shard and the Llama-7B list for their Adam
    step (re-take the counters after any change to the kernels' code)."""
    b = _bench()
    for k in ("zs_reduce_kernel", "zs_adam_kernel"):
        assert b.measured_traffic(k, "flat_7p5b_nd64") is not None, k
    for w in ("flat_7p5b_nd8", "llama_7b"):
        assert b.measured_traffic("zs_adam_kernel", w) is not None, w


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""
