"""Byte and operation accounting of the CSA2 cache, written from the pages'
definitions.

TEST INFRASTRUCTURE ONLY (see oracle/csa2.py).

Sources (web pages, cited by title):
  [KVC]  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
         (mer.run post): section 2 "890 bytes/token" (B_global sum, b_main,
         layer arrangement, per-model table), 4.2 (layer counts), 4.4
         (decode indexer MAC estimate).
  [ARCH] "DeepSeek-V4.1-Flash, 2. Architecture" course notes, 2.1 and 2.3.1.
"""
from fractions import Fraction

# Entry sizes from the formats: bits per element x elements + scale bytes.
MAIN_CHANNELS, MAIN_GROUP = 512, 16          # E2M1 + E4M3 per 16  [KVC] 2
IDX_DIMS, IDX_GROUP = 128, 32                # MXFP4, E8M0 per 32   [KVC] 2


def main_entry_bytes():
    return MAIN_CHANNELS * 4 // 8 + MAIN_CHANNELS // MAIN_GROUP


def idx_entry_bytes():
    return IDX_DIMS * 4 // 8 + IDX_DIMS // IDX_GROUP


def entry_bytes():
    return main_entry_bytes() + idx_entry_bytes()


def layer_plan(n_layers=40):
    """Mode of each of the 40 layers, [KVC] 2 arrangement list and 4.2:
    layers 0-1 SWA only; encoder (layers 2-19) = 3 groups of 1 Full + 5
    Reuse with m = 2; decoder (layers 20-39) = 5 groups of 4, the first
    1 Full + 3 Reuse, the other four 1 Reindex + 3 Reuse, with m = 1.
    Returns a list of (mode, m) with mode in {"swa", "full", "reindex",
    "reuse"}."""
    plan = [("swa", None), ("swa", None)]
    for _ in range(3):
        plan += [("full", 2)] + [("reuse", 2)] * 5
    plan += [("full", 1)] + [("reuse", 1)] * 3
    for _ in range(4):
        plan += [("reindex", 1)] + [("reuse", 1)] * 3
    assert len(plan) == n_layers
    return plan


def global_kv_bytes_per_token(plan=None):
    """B_global = sum over layers that produce KV (the Full layers) of
    b_entry / m_l, [KVC] 2.  Returned as an exact Fraction."""
    plan = layer_plan() if plan is None else plan
    return sum(Fraction(entry_bytes(), m) for mode, m in plan
               if mode == "full")


def v1_bytes_per_token():
    """[KVC] 2 table: 95 layers x (K and V) x 8 KV heads x 128 dims x 2 B."""
    return 95 * 2 * 8 * 128 * 2


def v32_bytes_per_token():
    """[KVC] 2 table: 61 layers x [(512 B FP8 latent + 16 B scale + 128 B RoPE
    part) + (128 B indexer K + 4 B scale)]."""
    return 61 * ((512 + 16 + 128) + (128 + 4))


def decode_indexer_macs(n_tokens, pool=2048 * 8, hierarchical=True,
                        plan=None):
    """Indexer multiply-adds per decode token, [KVC] 4.4: every indexing
    layer scores its visible entries at 32 heads x 128 dims per entry; Full
    layers see n/m entries; Reindex layers see the pool when the
    hierarchical indexer is on, else n/m entries."""
    plan = layer_plan() if plan is None else plan
    per_entry = 32 * 128
    macs = Fraction(0)
    for mode, m in plan:
        if mode == "full":
            macs += per_entry * Fraction(n_tokens, m)
        elif mode == "reindex":
            macs += per_entry * (pool if hierarchical
                                 else Fraction(n_tokens, m))
    return macs
