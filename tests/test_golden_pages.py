"""The benchmark's work accounting against figures printed on the pages."""
import json
import os

import torch

import oracle.mla_verify_oracle as orc
from mla_tree_verify_amd import gen

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_work_figures.json")))


def _close(x, key):
    ref = GOLD[key]
    return abs(x - ref["value"]) <= ref["rel_tol"] * ref["value"]


def test_fma_count_headline_shape():
    parent = gen.random_tree(9, torch.Generator().manual_seed(16))
    fma = orc.algorithmic_flops(parent, 16384) / 2
    assert _close(fma, "fma_count_q9_p16384")


def test_per_key_width_576():
    # 64 heads each reading the whole KV: 576 values (512 latent + 64 rope) per token, fp32
    per_key_bf16 = orc.algorithmic_bytes(0, 1)  # one KV row, no queries or outputs
    assert per_key_bf16 == 576 * 2
    assert _close(16384 * (per_key_bf16 // 2) * 4 * 64, "per_head_kv_bytes_p16384_fp32")


def test_naive_score_row():
    assert _close(65536 * 4, "naive_score_row_bytes_p65536")
