"""Host-side checks of bench.py (no GPU): the attention kernel it names in
the roofline object follows the library's launch rule, and a request for
more than one GPU ends with a message before anything touches a device."""

import os
import re
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_kernel_name_follows_the_launch_rule():
    # the rule in the library: the key-split kernel when the 256-row query
    # tiles number fewer than twice the CUs
    src = open(os.path.join(ROOT, "learned_token_pruning_score_amd", "csrc", "attn.hip")).read()
    assert re.search(r"if \(\(int64_t\)Hq \* \(\(Kt \+ 255\) / 256\) < 2 \* \(int64_t\)n_cu\)", src), \
        "the attention launch rule changed: update bench.attn_kernel_name"
    n_cu = 256
    assert bench.attn_kernel_name(torch.bfloat16, 16, 128, 8448, n_cu) == "attn_bf16_kernel<128, 8>"
    assert bench.attn_kernel_name(torch.bfloat16, 16, 128, 17442, n_cu) == "attn_bf16_kernel<128, 8>"
    assert bench.attn_kernel_name(torch.bfloat16, 16, 128, 2304, n_cu) == "attn_bf16_ks_kernel<128>"
    assert bench.attn_kernel_name(torch.bfloat16, 16, 128, 4352, n_cu) == "attn_bf16_ks_kernel<128>"
    assert bench.attn_kernel_name(torch.bfloat16, 16, 64, 32 * 256, n_cu) == "attn_bf16_kernel<64, 8>"
    assert bench.attn_kernel_name(torch.bfloat16, 16, 64, 32 * 256 - 256, n_cu) == "attn_bf16_ks_kernel<64>"
    assert bench.attn_kernel_name(torch.float32, 4, 64, 192, n_cu) == "attn_f32_kernel<64>"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
