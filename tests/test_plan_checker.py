"""Host test of the tile-plan checker the GPU parity tests apply to the plan the
kernels used: it accepts the oracle's plan (with the tile-group field filled in
as documented) and rejects each kind of broken plan."""
import numpy as np
import pytest

import oracle
from parity import check_plan


def _with_groups(blocks):
    """(expert, row0, rows) blocks in expert order -> int32 [n][4] with the group field:
    runs of up to 8 consecutive blocks of one expert, (first block << 4) | size."""
    out = []
    i = 0
    while i < len(blocks):
        j = i
        while j < len(blocks) and blocks[j][0] == blocks[i][0]:
            j += 1
        for g0 in range(i, j, 8):
            gs = min(8, j - g0)
            out += [[e, r0, rows, (g0 << 4) | gs] for e, r0, rows in blocks[g0:g0 + gs]]
        i = j
    return np.array(out, np.int64)


COUNTS = [300, 0, 17, 256, 2049, 1, 0, 513]


@pytest.mark.parametrize("beta", [128, 256])
def test_accepts_the_oracle_plan(beta):
    counts = np.array(COUNTS)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    plan = _with_groups(oracle.block_plan(counts, beta))
    check_plan(plan, counts, offsets, beta, int(counts.sum()))


@pytest.mark.parametrize("damage", ["duplicate", "drop", "two_partials", "wrong_expert", "too_big", "group"])
def test_rejects_broken_plans(damage):
    beta = 256
    counts = np.array(COUNTS)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    blocks = list(oracle.block_plan(counts, beta))
    big = [i for i, b in enumerate(blocks) if b[0] == 4]     # expert 4: 2049 rows, 9 blocks
    if damage == "duplicate":
        blocks.insert(big[1], blocks[big[1]])
    elif damage == "drop":
        del blocks[big[2]]
    elif damage == "two_partials":
        e, r0, rows = blocks[big[0]]
        blocks[big[0]:big[0] + 1] = [(e, r0, 100), (e, r0 + 100, rows - 100)]
    elif damage == "wrong_expert":
        e, r0, rows = blocks[big[3]]
        blocks[big[3]] = (3, r0, rows)
    elif damage == "too_big":
        e, r0, rows = blocks[big[0]]
        e2, r1, rows2 = blocks[big[0] + 1]
        blocks[big[0]:big[0] + 2] = [(e, r0, rows + rows2)]
    plan = _with_groups(blocks)
    if damage == "group":
        plan[big[8], 3] = (big[0] << 4) | 8                   # block 9 of the expert claims the first group
    with pytest.raises(AssertionError):
        check_plan(plan, counts, offsets, beta, int(counts.sum()))
