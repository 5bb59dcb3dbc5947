"""Host build of the decode kernels' visibility helpers, checked bit for bit.

The decode kernels decide which cached tokens a query row sees from two
helpers in csrc/mla_common.h: tree_branch_mask (bit i set when drafted token i
lies on query j's branch; "The Architecture of Memory", "Tree Attention
Verification") and tile_visible (the 64-bit mask of one tile's tokens: the
prefix up to the row's limit, plus the branch's drafted tokens below the
partition end). Both are compiled for the host here (no GPU needed) and
compared with the per-token definition and with the oracle's tree ancestry.
"""
import os
import random
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, os.pardir, "mla_latent_kv_03_amd", "csrc")
M64 = (1 << 64) - 1


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cc = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        cc = shutil.which("hipcc")
    if not cc:
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("mask") / "mask_check")
    subprocess.run([cc, "--offload-host-only", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(HERE, "host", "mask_check.hip"), "-o", exe], check=True)

    def run(lines):
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True,
                             text=True, check=True).stdout
        return out.splitlines()
    return run


def visible_by_definition(ts, lim, t_draft, t1, branch):
    m = 0
    for o in range(64):
        t = ts + o
        d = t - t_draft
        if t <= lim or (0 <= d < 64 and t < t1 and (branch >> d) & 1):
            m |= 1 << o
    return m


def _cases(rng, n):
    out = []
    for _ in range(n):
        Q = rng.randint(1, 64)
        L = rng.randint(Q, 600)
        t_draft = L - Q
        t0 = rng.randrange(0, L)
        t1 = rng.randint(t0 + 1, L)
        ts = t0 + 64 * rng.randint(0, (t1 - t0 - 1) // 64)
        tree = rng.random() < 0.7
        j = rng.randrange(Q)
        branch = (rng.getrandbits(Q) | (1 << j)) if tree else 0
        lim = min(t_draft - 1 if tree else t_draft + j, t1 - 1)
        out.append((ts, lim, t_draft, t1, branch))
    # edges: drafts wholly before / after the tile, a full 64-draft branch,
    # a limit below the tile, a partition that ends inside the drafts
    out += [(0, -1, 0, 64, M64), (128, 127, 64, 192, M64), (0, 63, 200, 264, 5),
            (64, 63, 130, 150, M64), (0, -5, 10, 20, 0), (64, 100, 90, 101, 1 << 10),
            (0, 63, 0, 64, 0), (192, 199, 200, 264, (1 << 64) - 2)]
    return out


def test_tile_visible_matches_the_per_token_definition(driver):
    cases = _cases(random.Random(5), 4000)
    got = driver([f"V {ts} {lim} {td} {t1} {br}" for ts, lim, td, t1, br in cases])
    assert len(got) == len(cases)
    for c, g in zip(cases, got):
        assert int(g) == visible_by_definition(*c), c


def _random_tree(rng, Q):
    return [-1] + [rng.randint(-1, i - 1) for i in range(1, Q)]


def test_branch_masks_match_the_oracle_ancestry(driver):
    rng = random.Random(9)
    trees = [_random_tree(rng, rng.randint(1, 64)) for _ in range(200)]
    trees += [[i - 1 for i in range(64)], [-1] * 64, [-1, 0, 0, 1, 1, 2, 2, 3]]
    got = driver([f"T {len(p)} " + " ".join(map(str, p)) for p in trees])
    for p, line in zip(trees, got):
        vals = [int(x) for x in line.split()]
        Q = len(p)
        masks, ok = vals[:Q], vals[Q:]
        anc = oracle.tree_ancestry(p)
        for j in range(Q):
            want = sum(1 << int(i) for i in np.flatnonzero(anc[j]))
            assert masks[j] == want, (p, j)
        assert ok == [1] * Q


def test_malformed_entries_are_flagged_and_the_walk_ends(driver):
    bad = [[0], [-1, 1], [-1, 0, 3], [-2, -1], [-1, 2, 1]]
    got = driver([f"T {len(p)} " + " ".join(map(str, p)) for p in bad])
    for p, line in zip(bad, got):
        vals = [int(x) for x in line.split()]
        Q = len(p)
        ok = vals[Q:]
        assert ok == [1 if -1 <= e < i else 0 for i, e in enumerate(p)], p
        for m in vals[:Q]:
            assert 0 <= m < (1 << Q)  # bounded walk, bits only inside the draft


def test_tiles_needed_stops_at_the_blocks_last_visible_token(driver):
    rng = random.Random(21)
    cases = []
    for _ in range(3000):
        Q = rng.randint(1, 5000)
        L = rng.randint(Q, 40000)
        t0 = rng.randrange(0, L)
        t1 = rng.randint(t0, L)
        tile = rng.choice([16, 32, 64])
        tree = int(rng.random() < 0.2)
        jmax = rng.randrange(Q)
        cases.append((t0, t1, tile, tree, L - Q, jmax))
    out = driver([f"N {a} {b} {c} {d} {e} {f}" for a, b, c, d, e, f in cases])
    for (t0, t1, tile, tree, t_draft, jmax), g in zip(cases, out):
        # tokens the block's rows can see in [t0, t1): up to t_draft + jmax
        # for a chain, everything for a tree
        last = t1 - 1 if tree else min(t1 - 1, t_draft + jmax)
        want = 0 if last < t0 else -(-(last - t0 + 1) // tile)
        assert int(g) == want, (t0, t1, tile, tree, t_draft, jmax)
