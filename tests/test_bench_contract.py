"""CPU checks of the benchmark's bookkeeping (no GPU)."""
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {\n  // scale it\n  return 2 * x;  /* doubled */\n}\n"
    b = "int f(int x) { return 2 * x; }  // one line now"
    c = "int f(int x) { return 3 * x; }"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)


def test_kernel_hash_follows_code_not_comments():
    paths = [os.path.join("exact_tiled_attention_21_amd", "csrc", f) for f in bench.KERNEL_SOURCES]
    texts = {p: open(os.path.join(ROOT, p), encoding="utf-8").read() for p in paths}
    h = bench.kernel_source_hash()
    assert bench.kernel_source_hash(lambda p: texts[p] + "\n// a new comment\n") == h
    first = paths[0]
    changed = dict(texts)
    changed[first] = texts[first].replace("constexpr float kLazy = 8.0f;", "constexpr float kLazy = 7.0f;")
    assert changed[first] != texts[first]
    assert bench.kernel_source_hash(lambda p: changed[p]) != h


def test_launch_header_hash_covers_forward_arguments_only():
    h = bench.kernel_source_hash()
    path = os.path.join("exact_tiled_attention_21_amd", "csrc", "fa_launch.h")

    def read(p, edit=None):
        text = open(os.path.join(ROOT, p), encoding="utf-8").read()
        return edit(text) if (edit and p == path) else text

    # another kernel's argument struct changes: the forward kernel's hash does not
    assert bench.kernel_source_hash(lambda p: read(p, lambda t: t.replace(
        "struct DecodeArgs {", "struct DecodeArgs {\n  int unused_field;"))) == h
    # a forward argument changes: the hash does
    assert bench.kernel_source_hash(lambda p: read(p, lambda t: t.replace(
        "struct FwdArgs {", "struct FwdArgs {\n  int unused_field;"))) != h


def test_committed_traffic_is_reported_only_for_the_kernel_it_measured():
    """The bench line carries the committed counter runs' traffic when they describe
    the forward kernel in the tree, and null once its code has changed since."""
    with open(os.path.join(ROOT, "profiles", "fa_fwd_headline_traffic.json")) as f:
        t = json.load(f)
    if t["kernel_source_sha"] == bench.kernel_source_hash():
        assert bench.measured_traffic() == t["bytes_per_launch"]
    else:
        assert bench.measured_traffic() is None
    # HBM bytes per launch stay within 1% of the algorithmic bytes (Q, K, V read, O, LSE written once)
    assert abs(t["bytes_per_launch"] - t["algorithmic_bytes"]) <= 0.01 * t["algorithmic_bytes"]
