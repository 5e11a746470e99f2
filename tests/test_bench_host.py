"""Host-side pieces of bench.py that decide its reported numbers (CPU only).

allowed_pairs counts the algorithmic FLOPs behind every TFLOP/s figure; it is
checked against a brute-force count of the allowed (query, key) pairs of the
band rule and against closed forms. recorded_traffic must refuse a counter
summary taken on other kernel sources.
"""
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def brute_pairs(N, causal, window):
    n = 0
    for i in range(N):
        for j in range(N):
            ok = True
            if causal and j > i:
                ok = False
            if window >= 0 and (j < i - window or (not causal and j > i + window)):
                ok = False
            n += ok
    return n


@pytest.mark.parametrize("N", [1, 2, 7, 64, 129])
@pytest.mark.parametrize("causal,window", [(False, -1), (True, -1), (True, 0), (True, 5), (False, 0),
                                           (False, 3), (True, 200), (False, 200)])
def test_allowed_pairs_brute_force(N, causal, window):
    assert bench.allowed_pairs(N, causal, window) == brute_pairs(N, causal, window)


def test_allowed_pairs_closed_forms():
    assert bench.allowed_pairs(8192, False, -1) == 8192 * 8192
    assert bench.allowed_pairs(2048, True, -1) == 2048 * 2049 // 2
    # causal window w: row i sees min(i, w) + 1 keys
    N, w = 16384, 1024
    assert bench.allowed_pairs(N, True, w) == (w + 1) * (w + 2) // 2 - (w + 1) + (N - w) * (w + 1)
    # the headline workload's algorithmic FLOP: 4 d N^2 B H
    assert bench.workload_flop(bench_workload("noncausal_b16h16n8192d128_bf16")) == 4.0 * 128 * 8192 ** 2 * 256


def bench_workload(name):
    from attn_inputs import BY_NAME
    return BY_NAME[name]


def test_spread_heads_distinct_and_spread():
    hs = bench.spread_heads(8, 16, 8)
    assert len(set(hs)) == 8 and {b for b, _ in hs} == set(range(8))
    assert len(set(bench.spread_heads(2, 32, 4))) == 4


def test_recorded_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    # a summary is used only when its recorded hash is that of the current
    # kernel sources; otherwise (or with no summary at all) traffic is None
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kind="bf16": "abcd1234abcd1234")
    assert bench.recorded_traffic("w", "bf16") is None
    (prof / "traffic_w.txt").write_text("hbm_bytes_per_launch: 1.5e9\nkernel_source_hash: 0000\n")
    assert bench.recorded_traffic("w", "bf16") is None
    (prof / "traffic_w.txt").write_text("hbm_bytes_per_launch: 1.5e9\nkernel_source_hash: abcd1234abcd1234\n")
    assert bench.recorded_traffic("w", "bf16") == 1.5e9


def test_kernel_source_hash_tracks_the_sources():
    h = bench.kernel_source_hash("bf16")
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_source_hash("bf16") == h
    assert bench.kernel_source_hash("fp8") != h


def test_strip_c_comments_keeps_code_and_literals():
    src = 'int a = 1; // note\n/* block\n comment */ const char* s = "a // b /* c */";\nchar q = \'"\';  int  b;\n'
    assert bench.strip_c_comments(src) == 'int a = 1; const char* s = "a // b /* c */"; char q = \'"\'; int b;'
    # an escaped quote inside a literal does not end it
    assert bench.strip_c_comments('x = "a\\" // b"; // c') == 'x = "a\\" // b";'


def test_kernel_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    csrc = tmp_path / "tiled_attention_forward_attn_amd" / "csrc"
    csrc.mkdir(parents=True)
    src_root = os.path.join(ROOT, "tiled_attention_forward_attn_amd")
    for f in bench.KERNEL_SOURCES["bf16"]:
        path = os.path.normpath(os.path.join(src_root, "csrc", f))
        dst = os.path.normpath(os.path.join(str(csrc), f))
        with open(path) as fh, open(dst, "w") as out:
            out.write(fh.read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash("bf16")
    main = csrc / "attn_fwd_bf16.hip"
    text = main.read_text()
    main.write_text("// an added comment line\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash("bf16") == h0
    main.write_text(text.replace("kRescaleSlack = 8.f", "kRescaleSlack = 7.f"))
    assert bench.kernel_source_hash("bf16") != h0
