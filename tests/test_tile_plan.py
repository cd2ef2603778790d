"""The tile-range and K-split plan of the persistent grouped GEMMs (csrc/tile_plan.h), compiled
for the host and checked exhaustively over launch shapes (CPU only): every tile of a launch is
computed exactly once, either whole or as pieces whose K ranges partition [0, KT) and which share
one arrival counter; partial-tile slots and counters stay inside their workspace regions; every
range is drained by its own workgroups, whatever XCD they run on."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "mixture_experts_layer_07_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
MAX_ITEMS, MAX_PIECES, QUEUES = 512, 4, 8


@pytest.fixture(scope="module")
def dump(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "tile_plan_dump")
    r = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", "-I" + CSRC,
                        os.path.join(HERE, "tile_plan_dump.cpp"), "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

    def run(launches):
        text = "".join(f"{t} {kt} {ms} {sl} {c}\n" for t, kt, ms, sl, c in launches)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        res, cur = [], None
        for line in out.splitlines():
            f = line.split()
            if f[0] == "L":
                cur = {"total": int(f[1]), "KT": int(f[2]), "C": int(f[3]), "items": []}
                res.append(cur)
            else:
                cur["items"].append(tuple(int(v) for v in f))
        return res
    return run


def check_launch(L, max_slots):
    total, KT, C = L["total"], L["KT"], L["C"]
    seen = {}
    split = 0
    for q, it, tile, piece, k0, k1, slot, first, S in L["items"]:
        if tile < 0:
            continue
        per = (total + QUEUES - 1) // QUEUES
        assert q * per <= tile < min(total, (q + 1) * per), "tile outside its range"
        seen.setdefault(tile, []).append((piece, k0, k1, slot, first, S, q))
    assert sorted(seen) == list(range(total)), "a tile is missing or out of range"
    for tile, parts in seen.items():
        if parts[0][0] < 0:
            assert len(parts) == 1 and parts[0][1:3] == (0, KT), (tile, parts)
            continue
        split += 1
        S = parts[0][5]
        assert 2 <= S <= MAX_PIECES and len(parts) == S
        parts.sort()
        assert [p[0] for p in parts] == list(range(S))
        assert parts[0][1] == 0 and parts[-1][2] == KT
        for a, b in zip(parts, parts[1:]):
            assert a[2] == b[1], "pieces leave a gap or overlap in K"
        for p in parts:
            assert p[2] > p[1] and (p[0] == S - 1 or (p[2] - p[1]) % 2 == 0)
            assert p[4] == parts[0][3] and p[3] == p[4] + p[0], "slot / counter mismatch"
            assert 0 <= p[3] < min(max_slots, QUEUES * C, MAX_ITEMS), "partial-tile slot out of range"
            assert p[3] // C == p[6], "slot outside the range's block"
    slots = [p[3] for parts in seen.values() if parts[0][0] >= 0 for p in parts]
    assert len(slots) == len(set(slots)), "two pieces share a partial-tile slot"
    # after its items the range's counter yields only "drained"
    for q in range(QUEUES):
        its = [i for i in L["items"] if i[0] == q]
        n = sum(1 for i in its if i[2] >= 0)
        assert all(i[2] < 0 for i in its[n:]) and all(i[2] >= 0 for i in its[:n])
    return split


def test_every_tile_once_and_pieces_partition_k(dump):
    launches = []
    for C in (32, 64):
        for KT in (2, 8, 28, 32, 56, 112, 128, 224):
            for ms in (7, 16):
                for slots in (256, 512):
                    for total in list(range(0, 70)) + [200, 255, 256, 257, 300, 320, 401 * 16 // 3, 6416]:
                        launches.append((total, KT, ms, slots, C))
    n_split = 0
    for L, (total, KT, ms, slots, C) in zip(dump(launches), launches):
        n_split += check_launch(L, slots)
    assert n_split > 1000   # the split path is exercised, with full rounds and without


def test_split_tail_after_full_rounds(dump):
    # 8 ranges of 40 tiles, 32 workgroups each: one full round, 8 tail tiles cut into 4 pieces
    (L,) = dump([(320, 128, 16, 256, 32)])
    assert check_launch(L, 256) == 64
    pieces = [i for i in L["items"] if i[2] >= 0 and i[3] >= 0]
    assert {i[8] for i in pieces} == {4}
    assert sorted({(i[4], i[5]) for i in pieces}) == [(0, 32), (32, 64), (64, 96), (96, 128)]
