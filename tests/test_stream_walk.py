"""CPU replay of the weight-stream kernels' walks (no GPU).

`rowstream_kernel` (csrc/stream.hip) walks K in 128-wide super-chunks through
a ring of D register buffers, D - 1 super-chunks ahead of the products, in
either direction, and stages the activation panel one k slice at a time
whenever the walk enters a slice.  `rowpersist_kernel` walks a wave's row
units one after another as one stream of super-chunks, its prefetch cursor
D - 1 super-chunks ahead, with clamped rows past the wave's last unit.  A
mistake in either walk reads the wrong ring slot or panel slice (wrong
logits) or reads outside a buffer (a fault).  These tests replay the loops
statement for statement and check, for every schedule the launchers can
choose: each super-chunk is multiplied exactly once, from the ring slot that
holds it and the panel slice that is staged; every load index, clamped row,
staged record and panel offset lies inside its buffer.
"""
import itertools
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "gru_corrected_draft_amd", "csrc")


def _constant(name):
    text = open(os.path.join(CSRC, "stream.hip")).read()
    m = re.search(rf"constexpr int {name} = (\d+);", text)
    assert m, name
    return int(m.group(1))


KSC = _constant("kSC")            # k per super-chunk
PAD = _constant("kPanelPad")      # panel row padding (elements)
UNIT_ROWS = _constant("kUnionUnitRows")
LANE_K_SPAN = 3 * 32 + 3 * 8 + 8  # last element a lane reads in a super-chunk: c = 3, q = 3, 8 wide


def pick_slice(K, ncols, planes, budget):
    """The launcher's slice choice: the largest multiple of 128 dividing K
    whose panel slice fits the budget (128 when none does)."""
    best = 128
    for ks in range(128, K + 1, 128):
        if K % ks == 0 and planes * ncols * (ks + PAD) * 2 <= budget:
            best = ks
    return best


def replay_rowstream(K, KS, D, rev, straight=True, clamp=True, ahead=None):
    """clamp / ahead plant mistakes for the self-test: an unclamped
    prefetch index, or a prefetch distance other than D - 1."""
    nsc, per_slice = K // KSC, KS // KSC
    ahead = D - 1 if ahead is None else ahead
    lim = (lambda x: min(x, nsc - 1)) if clamp else (lambda x: x)
    assert K % KSC == 0 and KS % KSC == 0 and K % KS == 0

    def chunk(i):
        return nsc - 1 - i if rev else i

    def enters_slice(i):
        sc = chunk(i)
        return sc % per_slice == per_slice - 1 if rev else sc % per_slice == 0

    ring = [None] * D
    staged = [None]
    computed = []

    def stage(sc):
        assert 0 <= sc < nsc
        slice0 = (sc // per_slice) * KS
        # the copy reads act[row, slice0 + 8 p .. + 8) for p < KS / 8
        assert 0 <= slice0 and slice0 + KS <= K
        staged[0] = slice0

    def load(slot, sc):
        assert 0 <= slot < D
        assert 0 <= sc < nsc, f"super-chunk {sc} outside 0..{nsc - 1}"
        assert sc * KSC + LANE_K_SPAN <= K
        ring[slot] = sc

    def compute(slot, i, kk):
        sc = chunk(i)
        assert ring[slot] == sc, f"slot {slot} holds {ring[slot]}, step {i} needs {sc}"
        assert staged[0] is not None and staged[0] <= sc * KSC < staged[0] + KS, "slice not staged"
        assert kk == sc * KSC - staged[0], "panel offset"
        assert 0 <= kk and kk + LANE_K_SPAN <= KS  # inside the staged row (its pad excluded)
        computed.append(sc)

    stage(chunk(0))
    for p in range(D - 1):
        load(p, chunk(lim(p)))
    if straight and per_slice == nsc and nsc % D == 0:
        i0 = 0
        while True:
            for d in range(D):
                load((d + D - 1) % D, chunk(lim(i0 + d + ahead)))
                compute(d, i0 + d, chunk(i0 + d) * KSC)
            i0 += D
            if i0 >= nsc:
                break
    else:
        for i0 in range(0, nsc, D):
            for d in range(D):
                i = i0 + d
                if i >= nsc:
                    break
                if i > 0 and enters_slice(i):
                    stage(chunk(i))
                load((d + D - 1) % D, chunk(lim(i + ahead)))
                compute(d, i, (chunk(i) % per_slice) * KSC)
    assert sorted(computed) == list(range(nsc))
    order = [chunk(i) for i in range(nsc)]
    assert computed == order


def replay_rowpersist(K, D, N, RT, w, stride, rev, mode, umaxu=None):
    """mode: 'rows' (row-major W), 'tiles' (W in tile order), 'union' (rows
    through staged records; N is the union size)."""
    nsc = K // KSC
    assert nsc % D == 0  # persist_fits
    units = ((N + 15) // 16 + RT - 1) // RT
    my_n = (units - w + stride - 1) // stride if units > w else 0
    if mode == "union":
        assert umaxu is not None
        my_n = min(my_n, umaxu)
    ntiles = (N + 15) // 16

    def unit_of(j):
        return w + ((my_n - 1 - j) if rev else j) * stride

    def kchunk(ci):
        return nsc - 1 - ci if rev else ci

    srec_len = (umaxu or 0) * UNIT_ROWS
    if mode == "union":  # record staging: srec[e] = rec[min(unit_of(j) * 32 + rr, N - 1)]
        for e in range(my_n * UNIT_ROWS):
            j, rr = divmod(e, UNIT_ROWS)
            src = min(unit_of(j) * UNIT_ROWS + rr, N - 1)
            assert 0 <= src < N and e < srec_len

    def rows_of(j):
        out = []
        for row in range(16):
            if mode == "tiles":
                u = unit_of(j)
                r = (min(max(u * RT, 0), ntiles - 1), min(max(u * RT + 1, 0), ntiles - 1))
                assert all(0 <= x < ntiles for x in r)
            elif mode == "union":
                jj = min(j, my_n - 1)
                if jj >= 0:
                    i0, i1 = jj * UNIT_ROWS + row, jj * UNIT_ROWS + 16 + row
                    assert 0 <= i0 < srec_len and 0 <= i1 < srec_len
                r = ("rec", jj)
            else:
                u = unit_of(j)
                r = (min(max((u * RT) * 16 + row, 0), N - 1), min(max((u * RT + 1) * 16 + row, 0), N - 1))
                assert all(0 <= x < N for x in r)
            out.append(r)
        return out

    cur = {"pj": 0, "pci": 0}
    rows_of(0)
    ring = [None] * D

    def load_next(slot):
        sc = kchunk(cur["pci"])
        assert 0 <= sc < nsc and sc * KSC + LANE_K_SPAN <= K
        ring[slot] = (cur["pj"], sc)
        cur["pci"] += 1
        if cur["pci"] == nsc:
            cur["pci"] = 0
            cur["pj"] += 1
            rows_of(cur["pj"])

    for p in range(D - 1):
        load_next(p)
    done = []
    for j in range(my_n):
        u = unit_of(j)
        assert 0 <= u < units
        ci0 = 0
        while True:
            for d in range(D):
                load_next((d + D - 1) % D)
                want = (j, kchunk(ci0 + d))
                assert ring[d] == want, f"slot {d} holds {ring[d]}, unit step {j} needs {want}"
                done.append(want)
            ci0 += D
            if ci0 >= nsc:
                break
    assert done == [(j, kchunk(ci)) for j in range(my_n) for ci in range(nsc)]
    return my_n


KS_ALL = [k for k in range(128, 8193, 128)]


@pytest.mark.parametrize("D", [2, 3, 4])
@pytest.mark.parametrize("rev", [False, True])
def test_rowstream_every_slice_schedule(D, rev):
    """Every K up to 8192 with every slice width that divides it."""
    n = 0
    for K in KS_ALL:
        for KS in range(128, K + 1, 128):
            if K % KS:
                continue
            replay_rowstream(K, KS, D, rev)
            replay_rowstream(K, KS, D, rev, straight=False)
            n += 1
    assert n == 280  # (K, slice) pairs: every divisor of every K up to 8192


def test_rowstream_launcher_slices():
    """The slices the launchers pick for the store and argmax paths."""
    for K in (1024, 2048, 2560, 3072, 4096, 5120, 5376, 8192):
        for ncols in range(1, 129):
            for planes, budget, D in ((1, 32 * 1024, 3), (1, 32 * 1024, 2), (2, 32 * 1024, 2)):
                KS = pick_slice(K, ncols, planes, budget)
                for rev in (False, True):
                    replay_rowstream(K, KS, D, rev)


def test_pick_slice_fits_budget_or_is_minimal():
    for K, ncols, planes, budget in itertools.product((1024, 4096, 5376), (1, 15, 120, 128), (1, 2),
                                                      (32 * 1024,)):
        KS = pick_slice(K, ncols, planes, budget)
        assert K % KS == 0 and KS % 128 == 0
        fits = planes * ncols * (KS + PAD) * 2 <= budget
        assert fits or KS == 128


@pytest.mark.parametrize("mode", ["rows", "tiles"])
@pytest.mark.parametrize("D", [2, 3, 4])
def test_rowpersist_prefetch_cursor(mode, D):
    """Waves with several units, one, or none; ragged last tiles; both
    directions; the cursor runs D - 1 super-chunks past the last unit."""
    for K in (128 * D, 1024, 3072, 4096):
        if (K // KSC) % D:
            continue
        for N in (1, 15, 16, 17, 100, 5003, 151936):
            for stride in (1, 3, 8, 2048):
                for w in sorted({0, 1, stride - 1, min(stride, 5)}):
                    if w >= stride:
                        continue
                    for rev in (False, True):
                        replay_rowpersist(K, D, N, 2, w, stride, rev, mode)


def test_rowpersist_union_records():
    """Union stream: rows through the staged records, a wave's unit count
    capped at the staged record count."""
    for K in (1024, 4096):
        for N in (1, 31, 32, 33, 2048, 65536):
            for stride, umaxu in ((8, 1), (16, 2), (2048, 1), (2048, 4), (3, 1000)):
                for w in (0, 1, stride - 1):
                    for rev in (False, True):
                        my_n = replay_rowpersist(K, 2, N, 2, w, stride, rev, "union", umaxu)
                        assert my_n <= umaxu


@pytest.mark.parametrize("straight", [True, False])
def test_replay_catches_a_wrong_walk(straight):
    """The checks are live: the reversed walk without the clamp of its
    prefetch index (it reads super-chunk -1, before the matrix) and a walk
    whose prefetch runs one super-chunk too far ahead both fail them."""
    with pytest.raises(AssertionError):
        replay_rowstream(4096, 4096, 2, True, straight=straight, clamp=False)
    with pytest.raises(AssertionError):
        replay_rowstream(4096, 1024, 2, False, straight=straight, ahead=2)
    replay_rowstream(4096, 1024, 2, True, straight=straight)
