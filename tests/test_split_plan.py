"""Host logic: the attention's split plan, read back through the library's
workspace size, follows its rule and never exceeds the 16 partials the merge
kernel is instantiated for."""
from fp4_kv_cache_amd import csa2
from _util import planned_splits, split_parts_bytes


def test_split_plan_matches_library():
    seen = set()
    for B in list(range(1, 70)) + [96, 128, 255, 256, 257, 1000]:
        for k in (1, 16, 31, 32, 33, 48, 96, 100, 128, 160, 192, 224, 256, 288,
                  320, 352,
                  384, 512, 513, 1000, 1024, 1280, 1536, 2047, 2048):
            S = planned_splits(B, k)
            assert 1 <= S <= 16, (B, k, S)
            assert csa2.workspace_size(csa2.OP_REUSE, B, 4096, k) == \
                split_parts_bytes(B, S), (B, k, S)
            seen.add(S)
    assert seen == set(range(1, 17)), sorted(seen)
