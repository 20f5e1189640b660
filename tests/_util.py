"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch

from oracle import csa2 as O

REL_L2_TOL = 5e-3          # attention output vs the float64 oracle
GAP_TOL = 1e-5             # top-k near-tie band (relative)
SCORE_RTOL = 2e-6          # float32-accumulated scores vs float64


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def head_rel_l2_max(a, b):
    """The largest per-head relative L2 error of a [64][512] output (the
    per-sequence tolerance's diagnostic); heads whose reference is all zero
    are skipped."""
    a = np.asarray(a, np.float64).reshape(64, -1)
    b = np.asarray(b, np.float64).reshape(64, -1)
    nb = np.linalg.norm(b, axis=1)
    e = np.linalg.norm(a - b, axis=1)[nb > 0] / nb[nb > 0]
    return float(e.max()) if e.size else 0.0


def bf16_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def topk_set_ok(gpu_ids, ref_scores, k, ids=None):
    """The gap rule for one row: with s_(k) the oracle's k-th score, the GPU
    set must contain every id scoring above s_(k)(1 + tol) and only ids
    scoring at least s_(k)(1 - tol); when the (k, k+1) gap is >= tol it must
    equal the oracle's set.  Returns (ok, message)."""
    s = np.asarray(ref_scores, np.float64)
    ids = np.arange(len(s)) if ids is None else np.asarray(ids)
    g = np.asarray(gpu_ids)
    g = g[g >= 0]
    want = O.topk(s, k, ids)
    want = want[want >= 0]
    if len(g) != len(want):
        return False, f"size {len(g)} != {len(want)}"
    if np.array_equal(np.sort(g), want):
        return True, "equal"
    gap = O.topk_gap(s, k)
    if gap >= GAP_TOL:
        return False, f"sets differ with gap {gap:.3g}"
    pos = {int(i): j for j, i in enumerate(ids)}
    sg = np.array([s[pos[int(i)]] for i in g])
    kth = np.sort(s)[::-1][k - 1]
    must = ids[s > kth * (1 + GAP_TOL)]
    if not set(must.tolist()) <= set(g.tolist()):
        return False, "missing a clear winner"
    if np.any(sg < kth * (1 - GAP_TOL)):
        return False, "contains a clear loser"
    return True, f"near-tie (gap {gap:.3g})"


def planned_splits(B, k):
    """Workgroups per sequence the attention plans for B sequences and k
    chosen entries (k + 128 slots in 32-slot tiles): about one per compute
    unit, at least 3 tiles each with 16 or more sequences, at most 16, and
    the same number of tiles in every split."""
    n_tiles = (k + 128 + 31) // 32
    s = (256 + B - 1) // B
    max_s = (n_tiles + 2) // 3 if B >= 16 else n_tiles
    s = max(1, min(s, max_s, 16))
    tps = -(-n_tiles // s)
    return -(-n_tiles // tps)


def split_parts_bytes(B, S):
    """Workspace of S split partials: fp16 outputs [B][S][64][512] and
    float32 (max, sum) [B][S][64][2], each 256-byte aligned; none for S = 1."""
    if S <= 1:
        return 0
    a = lambda x: (x + 255) & ~255
    return a(B * S * 64 * 512 * 2) + a(B * S * 64 * 2 * 4)
