"""Host logic of bench.py that runs without a GPU: the algorithmic work model,
the mapping from kernel names to their sources, the stored-traffic lookup and
the one-GPU contract."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_decode_gemv_bytes_match_the_documented_figure():
    # down_proj at the 1.3B shape, batch 16: weights 2048*5632/4, codes 16*5632 + 8*16,
    # residual (fp32) read and output (bf16) written per output
    ops, nbytes = bench.algorithmic("tgemv<resid>", 16, 2048, 5632)
    assert ops == 2.0 * 16 * 2048 * 5632
    assert nbytes == 2048 * 5632 / 4 + 16 * 5632 + 8 * 16 + 16 * 2048 * (4 + 2)
    assert nbytes == 3170432


def test_gate_groups_share_their_epilogue_bytes():
    # n counts all groups' outputs; the epilogue bytes are per channel of one group
    _, gates = bench.algorithmic("tgemv<gates_step>", 16, 3 * 2048, 2048)
    assert gates == 3 * 2048 * 2048 / 4 + 16 * 2048 + 8 * 16 + 16 * 2048 * 12
    _, glu = bench.algorithmic("tgemm_dma<glu>", 1024, 2 * 5632, 2048)
    assert glu == 2 * 5632 * 2048 / 4 + 1024 * 2048 + 8 * 1024 + 1024 * 5632 * 4


def test_self_quantising_contractions_read_rows_not_codes():
    # gate_proj + up_proj at the 1.3B shape, 16 fp32 rows; i/f/g from 16 bf16 rows
    _, glu = bench.algorithmic("tgemv_row<glu,f32>", 16, 2 * 5632, 2048)
    assert glu == 2 * 5632 * 2048 / 4 + 16 * 2048 * 4 + 16 * 5632 * 4
    _, gates = bench.algorithmic("tgemv_row<gates_step,bf16>", 16, 3 * 2048, 2048)
    assert gates == 3 * 2048 * 2048 / 4 + 16 * 2048 * 2 + 16 * 2048 * 12
    assert bench.kernel_files("tgemv_row<resid,bf16> m=1 n=2 k=3") == bench.kernel_files("tgemv<resid>")
    # o_proj over the gated g_norm of one row: h, g and the gain read, residual and sum per output
    _, o = bench.algorithmic("tgemv_row<resid,gnorm,f32>", 1, 2048, 2048)
    assert o == 2048 * 2048 / 4 + 2048 * (4 + 4) + 4 * 2048 + 2048 * (4 + 2)


def test_split_activation_codes_counted_per_group():
    _, shared = bench.algorithmic("tgemm<gates>", 256, 3 * 512, 512)
    _, split = bench.algorithmic("tgemm<gates,split_a>", 256, 3 * 512, 512)
    assert split - shared == 2 * (256 * 512 + 8 * 256)


def test_elementwise_kernels():
    assert bench.algorithmic("scan_tiled", 100, 7, 64) == (0.0, 12.0 * 100 * 64)
    # the derivative: dh, f, h read and dx, df written
    assert bench.algorithmic("scan_bwd_tiled", 100, 64, 64) == (0.0, 20.0 * 100 * 64)
    assert bench.kernel_files("scan_bwd_recurrent m=1 n=2 k=2") == bench.kernel_files("scan_tiled")
    assert bench.algorithmic("norm_quant<f32>", 10, 0, 256) == (0.0, 10 * 256 * 5 + 80)
    assert bench.algorithmic("norm_quant<bf16>", 10, 0, 256) == (0.0, 10 * 256 * 3 + 80)
    assert bench.algorithmic("gnorm_quant<bf16>", 10, 0, 256) == (0.0, 10 * 256 * 7 + 80)


def test_every_kernel_name_maps_to_its_sources():
    names = ["tgemv<resid>", "tgemv_row<glu,f32>", "tgemm<gates,split_a>", "tgemm_dma<glu>",
             "norm_quant<f32>", "gnorm_quant<bf16>", "scan_tiled", "scan_chunk", "scan_recurrent"]
    csrc = os.path.join(ROOT, "ternary_weight_matmul_amd", "csrc")
    for n in names:
        files = bench.kernel_files(n + " m=1 n=2 k=3")
        assert files, n
        for f in files:
            assert os.path.exists(os.path.join(csrc, f)), (n, f)


def test_digest_changes_with_its_files_only():
    files = bench.kernel_files("scan_tiled")
    assert bench.source_digest(files) == bench.source_digest(list(reversed(files)))
    assert bench.source_digest(files) != bench.source_digest(bench.kernel_files("tgemv<resid>"))


def test_stored_traffic_applies_only_to_the_measured_sources():
    pdir = os.path.join(ROOT, "profiles")
    found = 0
    for name in sorted(os.listdir(pdir)):
        if not (name.startswith("traffic_") and name.endswith(".txt")):
            continue
        text = open(os.path.join(pdir, name)).read()
        key = re.search(r"^kernel: (.+)$", text, re.M).group(1).strip()
        digest = re.search(r"^sources: (\w+)$", text, re.M).group(1)
        value = float(re.search(r"^hbm_bytes_per_launch: ([0-9.]+)$", text, re.M).group(1))
        current = bench.source_digest(bench.kernel_files(key))
        assert bench.stored_traffic(key) == (value if digest == current else None)
        found += 1
    assert found >= 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_digest_ignores_comments_and_layout():
    a = "int f(int x) { // doubles x\n  return 2 * x; /* plain */ }\n"
    b = "int f(int x) {\n    return 2 * x;\n}  // edited note\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("2 * x", "3 * x"))
