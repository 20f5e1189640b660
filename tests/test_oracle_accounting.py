"""Pins of the accounting functions against the figures the pages print
(tests/golden/page_figures.json, each with its citation)."""
import json
import os
from fractions import Fraction

from oracle import accounting as A

with open(os.path.join(os.path.dirname(__file__), "golden",
                       "page_figures.json")) as f:
    G = {k: v["value"] for k, v in json.load(f).items() if k != "_sources"}


def test_entry_bytes():
    assert A.main_entry_bytes() == G["main_entry_bytes"]
    assert A.idx_entry_bytes() == G["idx_entry_bytes"]
    assert A.entry_bytes() == G["entry_bytes"]
    # 4.5 bits per channel for the main entry
    assert Fraction(A.main_entry_bytes() * 8, 512) == Fraction(9, 2)


def test_layer_plan_matches_pages():
    plan = A.layer_plan()
    modes = [m for m, _ in plan]
    full = [i for i, m in enumerate(modes) if m == "full"]
    reindex = [i for i, m in enumerate(modes) if m == "reindex"]
    assert full == G["full_layers"]
    assert reindex == G["reindex_layers"]
    assert sum(m != "swa" for m in modes) == G["csa2_layers"]
    assert modes.count("full") == G["full_count"]
    assert modes.count("reindex") == G["reindex_count"]
    assert modes.count("reuse") == G["reuse_count"]
    assert len(full) + len(reindex) == G["indexer_layers"]


def test_global_kv_890():
    b = A.global_kv_bytes_per_token()
    assert b == G["global_kv_bytes_per_token"]
    enc = sum(Fraction(A.entry_bytes(), m) for mode, m in A.layer_plan()
              if mode == "full" and m == 2)
    assert enc == G["encoder_full_share"]
    assert b * 10 ** 6 / 10 ** 6 == G["global_kv_1m_context_MB"]


def test_other_models_per_token():
    assert A.v1_bytes_per_token() == G["v1_bytes_per_token"]
    assert A.v32_bytes_per_token() == G["v32_bytes_per_token"]
    assert round(A.v32_bytes_per_token() * 10 ** 6 / 1e9) == \
        G["v32_global_kv_1m_context_GB"]
    # V4.1 is about a quarter of V4-Flash
    assert round(G["v4flash_bytes_per_token"] / 890) == 4


def test_decode_indexer_macs():
    f = A.decode_indexer_macs
    lin = f(2) - f(1)
    assert lin == G["mac_linear_coeff"]
    assert f(0) == 4 * G["macs_per_entry"] * G["pool_positions"]
    assert round(float(f(0)) / 1e9, 2) == G["mac_constant_G"]
    flat = f(2, hierarchical=False) - f(1, hierarchical=False)
    assert flat == G["mac_linear_coeff_flat"]
    lin1m = lin * 10 ** 6
    assert round(float(lin1m) / 1e9, 1) == G["mac_linear_at_1M_G"]
    assert round(2 * float(lin1m) / 1e9, 1) == G["gflops_linear_at_1M"]
    assert G["pool_blocks"] * G["pool_block_size"] == G["pool_positions"]
