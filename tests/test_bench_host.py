"""Host logic of bench.py (CPU only): the work count, the kernel-source digest and the
rule that counter-derived figures (HBM traffic, core clock) are used only for the kernel
sources they were measured on."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _pairs_brute(seqlens, causal, window):
    total = 0
    for n in seqlens:
        for i in range(n):
            for j in range(n):
                if causal and j > i:
                    continue
                if window > 0 and j <= i - window:
                    continue
                total += 1
    return total


@pytest.mark.parametrize("seqlens,causal,window", [
    ((1,), True, 0), ((64,), True, 0), ((70, 5, 0, 33), True, 0), ((50,), False, 0),
    ((90,), True, 16), ((40, 7), True, 128), ((30,), True, 1), ((25, 9), False, 0),
])
def test_count_pairs_matches_brute_force(seqlens, causal, window):
    assert bench.count_pairs(list(seqlens), causal, window) == _pairs_brute(seqlens, causal, window)


def test_count_pairs_closed_forms():
    # full causal: N (N + 1) / 2 per sequence; a window W: sum_i min(i + 1, W)
    assert bench.count_pairs([4096], True, 0) == 4096 * 4097 // 2 == 8_390_656
    assert bench.count_pairs([16384], True, 128) == sum(min(i + 1, 128) for i in range(16384)) == 2_089_024
    assert bench.count_pairs([300], False, 0) == 300 * 300


def _write(path, text):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", encoding="utf-8") as f:
        f.write(text)


def test_code_only_drops_comments_and_blank_lines():
    src = "// header\nint a = 1;  // trailing\n\n/* block\n comment */ int b = 2;\n   \nint c;\n"
    assert bench._code_only(src) == "int a = 1;\n int b = 2;\nint c;"


def test_digest_ignores_comment_edits_but_not_code_edits(tmp_path):
    f = tmp_path / "k.hip"
    _write(str(f), "// v1\nint x = 1;\n")
    d1 = bench.source_digest([str(f)])
    _write(str(f), "// v2, reworded\n\nint x = 1;   // note\n")
    assert bench.source_digest([str(f)]) == d1
    _write(str(f), "// v2\nint x = 2;\n")
    assert bench.source_digest([str(f)]) != d1


def _fake_tree(root, kernel_text):
    for rel in set(bench.KERNEL_SOURCES + bench.DECODE_SOURCES):
        _write(os.path.join(root, rel), kernel_text)


def test_counter_figures_follow_the_source_digest(tmp_path, monkeypatch):
    root = str(tmp_path)
    monkeypatch.setattr(bench, "ROOT", root)
    _fake_tree(root, "int kernel_v1;\n")
    digest = bench.source_digest(bench.KERNEL_SOURCES)
    name = "_ZN9attn_sink15bwd_dkdv_kernelIDF16bLi64EEEvNS_7BwdArgsE"
    _write(os.path.join(root, "profiles", "traffic_attn_sink_bwd_dkdv_kernel_w.txt"),
           f"# summary\nsource_digest: {digest}\ntraffic_bytes_per_launch: 123456\n")
    _write(os.path.join(root, "profiles", "counters_w.txt"),
           f"kernel_source_digest {digest} (training kernels), x (decoding kernels)\nsclk_ghz {name} 1.900\n")
    assert bench.read_traffic("w", "attn_sink_bwd_dkdv_kernel") == 123456.0
    assert bench.read_sclk("w", "attn_sink_bwd_dkdv_kernel") == 1.9
    assert bench.read_sclk("w", "attn_sink_fwd_kernel") is None          # no line for it
    assert bench.read_traffic("other", "attn_sink_bwd_dkdv_kernel") is None  # no summary
    _fake_tree(root, "int kernel_v1;  // a comment changes nothing\n")
    assert bench.read_traffic("w", "attn_sink_bwd_dkdv_kernel") == 123456.0
    _fake_tree(root, "int kernel_v2;\n")                                  # the kernel changed
    assert bench.read_traffic("w", "attn_sink_bwd_dkdv_kernel") is None
    assert bench.read_sclk("w", "attn_sink_bwd_dkdv_kernel") is None


def test_bench_refuses_more_than_one_gpu(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
