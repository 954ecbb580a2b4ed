"""Split-KV planner (host C++ through the C-ABI): coverage, slots, balance (CPU only)."""
import numpy as np
import pytest

from mla_decode_attention_paged_amd import binding as B

BLOCK = 16


def make_plan(lens, heads=16, q_len=1, page=64, num_cus=256, force=0):
    lens = np.asarray(lens, dtype=np.int32)
    maxp = max(1, int(max((int(l) + page - 1) // page for l in lens)))
    num_pages = max(1, int(sum((int(l) + page - 1) // page for l in lens)))
    prob = B.make_problem(len(lens), q_len, heads, page, num_pages, maxp)
    return B.Plan(prob, lens, num_cus=num_cus, force_splits=force)


def check_plan(plan, lens):
    seg, off = plan.segments()
    info = plan.info()
    assert off[0] == 0 and off[-1] == len(seg) and np.all(np.diff(off) >= 0)
    assert info["num_workers"] == len(off) - 1
    by_seq = {}
    for s in seg:
        by_seq.setdefault(int(s[0]), []).append(s)
    assert sorted(by_seq) == list(range(len(lens)))
    slots_used = []
    for b, pieces in by_seq.items():
        L = int(lens[b])
        pos = 0
        for p in pieces:               # listed in token order
            assert p[1] == pos, f"seq {b}: gap or overlap at {pos}"
            assert p[1] % BLOCK == 0
            assert p[2] >= p[1]
            assert p[2] == L or p[2] % BLOCK == 0
            pos = int(p[2])
        assert pos == L, f"seq {b}: covered up to {pos} of {L}"
        if len(pieces) == 1:
            assert pieces[0][3] == -1
        else:
            sl = [int(p[3]) for p in pieces]
            assert sl == list(range(sl[0], sl[0] + len(sl)))
            assert all(p[2] > p[1] for p in pieces), "a split sequence has an empty piece"
            slots_used += sl
    assert sorted(slots_used) == list(range(info["num_partials"]))
    assert info["num_combine"] == sum(1 for v in by_seq.values() if len(v) > 1)
    return seg, off, info


CASES = {
    "tiny": [1024],
    "paged": [4096] * 16,
    "two_token": [16384] * 32,
    "long": [65536] * 16,
    "ragged": list(np.random.default_rng(4).integers(1024, 65536, endpoint=True, size=64)),
    "one_long_many_short": [65536] + [1024] * 63,
    "edges": [0, 1, 15, 16, 17, 63, 64, 65, 1000],
    "many_short": [33] * 1000,
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_plan_covers_every_token_once(name):
    lens = CASES[name]
    for heads, q_len in ((16, 1), (16, 2), (128, 1), (128, 2)):
        plan = make_plan(lens, heads=heads, q_len=q_len)
        seg, off, info = check_plan(plan, lens)
        R = heads * q_len
        # bf16 cache: 128 rows per work-group when they fit, else 64, else 32, else 16
        assert info["rows_per_group"] == (128 if R % 128 == 0 else 64 if R % 64 == 0 else 32 if R % 32 == 0 else 16)
        assert info["row_groups"] == R // info["rows_per_group"]
        workers = 256 // info["row_groups"]
        assert info["num_workers"] <= max(1, workers)


@pytest.mark.parametrize("name", ["long", "ragged", "one_long_many_short", "paged", "two_token"])
def test_plan_balance(name):
    lens = np.asarray(CASES[name])
    plan = make_plan(lens)
    info = plan.info()
    nblk = int(sum((l + 15) // 16 for l in lens))
    budget = -(-(nblk + 6 * len(lens)) // 256)
    # no work-group more than one piece's overhead plus a sliver over the even share
    assert info["max_worker_cost"] <= budget + 6 + 4, info
    # and the work fills the machine
    assert info["num_workers"] >= 250


def test_plan_long_context_shape():
    plan = make_plan(CASES["long"])
    info = plan.info()
    assert info["num_workers"] == 256
    assert info["num_combine"] == 16
    assert info["num_partials"] == info["num_segments"]


@pytest.mark.parametrize("k", [1, 2, 3, 7, 1000])
def test_force_splits(k):
    lens = [1, 16, 17, 100, 1000, 4096]
    plan = make_plan(lens, force=k)
    seg, off, info = check_plan(plan, lens)
    counts = np.bincount(seg[:, 0], minlength=len(lens))
    for b, L in enumerate(lens):
        assert counts[b] == max(1, min(k, (L + 15) // 16))
    assert info["num_workers"] == len(seg)


def test_empty_sequence_gets_an_empty_piece():
    lens = [0, 50, 0]
    plan = make_plan(lens)
    seg, _, _ = check_plan(plan, lens)
    empties = [s for s in seg if s[0] in (0, 2)]
    assert len(empties) == 2 and all(s[1] == 0 and s[2] == 0 and s[3] == -1 for s in empties)


def test_grid_padding_for_row_groups():
    plan = make_plan([5000] * 3, heads=48)
    info = plan.info()
    assert info["row_groups"] == 3 and info["rows_per_group"] == 16
    assert info["grid_size"] % 8 == 0
    assert info["grid_size"] == ((info["num_workers"] + 7) // 8 * 8) * 3


@pytest.mark.parametrize("heads,q_len,rpg", [(32, 1, 32), (64, 1, 64), (16, 4, 64), (128, 1, 32), (128, 1, 64),
                                          (128, 2, 128), (64, 2, 128)])
def test_forced_rows_per_group(heads, q_len, rpg):
    lens = [5000, 300]
    maxp = max((l + 63) // 64 for l in lens)
    prob = B.make_problem(len(lens), q_len, heads, 64, sum((l + 63) // 64 for l in lens), maxp)
    plan = B.Plan(prob, lens, num_cus=256, rows_per_group=rpg)
    seg, off, info = check_plan(plan, lens)
    assert info["rows_per_group"] == rpg and info["row_groups"] == heads * q_len // rpg


def test_rows_per_group_rejected():
    prob = B.make_problem(1, 1, 16, 64, 1, 1)
    with pytest.raises(B.MlaError):
        B.Plan(prob, [10], num_cus=256, rows_per_group=32)      # R = 16 is not a multiple of 32
    with pytest.raises(B.MlaError):
        B.Plan(prob, [10], num_cus=256, rows_per_group=24)
    fp8 = B.make_problem(1, 1, 128, 64, 1, 1, kv_fp8=True)
    with pytest.raises(B.MlaError) as ei:
        B.Plan(fp8, [10], num_cus=256, rows_per_group=32)       # the 32-row kernel reads bf16 rows only
    assert ei.value.status == B.MLA_ERR_UNSUPPORTED
    for rpg in (16, 64, 128):                                   # FP8 rows: the 16-row and the wide kernel
        assert B.Plan(fp8, [10], num_cus=256, rows_per_group=rpg).info()["rows_per_group"] == rpg
    with pytest.raises(B.MlaError) as ei:
        B.Plan(B.make_problem(1, 1, 64, 64, 1, 1), [10], num_cus=256, rows_per_group=128)   # R = 64
    assert ei.value.status == B.MLA_ERR_UNSUPPORTED


def test_default_rows_per_group():
    """128 rows per work-group when R is a multiple of 128, else 64 when R is a multiple of 64; else,
    with a bf16 cache, 32 when R is a multiple of 32; else 16."""
    for heads, q_len, kv, want in [(16, 1, 0, 16), (16, 2, 0, 32), (48, 1, 0, 16), (64, 1, 0, 64), (128, 1, 0, 128),
                                   (32, 2, 0, 64), (64, 1, 1, 64), (128, 1, 1, 128), (128, 2, 0, 128), (128, 2, 1, 128),
                                   (64, 2, 0, 128), (64, 2, 1, 128), (96, 2, 0, 64), (96, 2, 1, 64), (16, 2, 1, 16),
                                   (48, 2, 1, 16),
                                   (32, 1, 0, 32), (48, 2, 0, 32), (8, 4, 0, 32)]:
        prob = B.make_problem(1, q_len, heads, 64, 1, 1, kv_fp8=bool(kv))
        info = B.Plan(prob, [10], num_cus=256).info()
        assert info["rows_per_group"] == want, (heads, q_len, kv, info["rows_per_group"])
