"""bench.py's command line on the host: one GPU only (no device needed for this check)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_work_of_the_headline_decode():
    """The roofline's algorithmic bytes and flops, worked by hand for 8 sequences of 131,072 tokens
    and 128 heads: per packed token 256 B of 4-bit content, 32 B of 4-bit RoPE key and 9 x 4 B of
    bf16 scale / zero; 132 tokens per sequence read as 1152 B bf16 rows; one 4 B page id per
    64 tokens; per head the bf16 query (1152 B) and output (1024 B) and the fp32 lse; two flops per
    multiply-add over 576 score and 512 output channels."""
    b = _bench_module()
    assert b.kv_bytes_per_token(4) == 324 and b.kv_bytes_per_token(2) == 196
    per_seq = 324 * (131072 - 132) + 1152 * 132 + 4 * 2048 + 128 * (1152 + 1024 + 4)
    assert per_seq == 42_863_856
    by, fl = b.algorithmic([131072] * 8, 128, 4)
    assert by == 8 * per_seq == 342_910_848
    assert fl == 8 * 2 * 128 * (576 + 512) * 131072 == 292_057_776_128
    # short sequences are read from bf16 only
    by_s, fl_s = b.algorithmic([100], 16, 2)
    assert by_s == 1152 * 100 + 4 * 2 + 16 * 2180 and fl_s == 2 * 16 * 1088 * 100


def test_source_digest_ignores_comments_only():
    """The digest that ties a committed counter summary to the kernel code it was taken on changes
    with the code, not with its comments or blank lines; string literals are kept whole."""
    b = _bench_module()
    code = 'int a = 1;\nasm volatile("s_nop 0" ::: "memory");\nint b = a + 2;\n'
    commented = ('// header\nint a = 1;  // one\n\n/* block\n   comment */\n'
                 'asm volatile("s_nop 0" ::: "memory");\nint b = a + 2;  /* two */\n')
    assert b._code_only(code) == b._code_only(commented)
    assert b._code_only(code) != b._code_only(code.replace("a + 2", "a + 3"))
    assert b._code_only('const char* s = "x // y /* z */";') == 'const char* s = "x // y /* z */";'
    assert len(b.source_digest()) == 16


def test_committed_counter_summaries_match_the_current_kernels():
    """The bench line's traffic and MFMA-busy figures come from the committed rocprofv3 summaries; they
    are taken on the current decode source, so both are present for the headline workload and agree
    with the table rows they are read from."""
    b = _bench_module()
    traffic = b.committed_traffic("dsv3_c4r4_128k")
    busy = b.committed_mfma_busy("dsv3_c4r4_128k")
    assert traffic is not None and 3.0e8 < traffic < 6.0e8
    assert busy is not None and 0.0 < busy < 1.0
    assert b.committed_mfma_busy("dsv2lite_c4r4_128k") is not None
    assert b.committed_mfma_busy("no_such_workload") is None
