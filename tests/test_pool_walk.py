"""CPU replay of the pool selection's collect and select kernels (no GPU).

After two radix passes fix the top 22 bits of the K-th largest key,
`pool_collect_kernel` (csrc/kernels.hip) keeps every id whose key's top 22
bits are at least that prefix, compacted per 1024-id chunk in (load, wave,
lane) order, with a count per chunk, and adds the prefix's own ids to the
last 10-bit histogram; `pool_select_kernel` gives each of its 256 threads a
run of consecutive chunks, loads up to 24 candidates of the first one at
clamped places before the threshold is known (the rest 4 at a time, also
clamped), counts the keys above and
equal to the threshold, and writes its selected ids from place
gt + min(eq, need) on.  A mistake in the ordering, the clamps, the chunk
ownership or the placement gives a pool out of id order, a wrong member at
the cutoff, or a read outside the candidate buffer.  This replay follows the
kernels' index arithmetic and checks, for vocabularies, pool sizes, chunk
widths and tie patterns the launcher can meet, that the pool is the K best
keys, lowest id on ties, in id order, and that every read stays inside the
request's stretch of the candidate buffer; planted mistakes must fail it.
"""
import os
import re

import numpy as np
import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "gru_corrected_draft_amd", "csrc")


def _constant(name, fname):
    m = re.search(rf"constexpr int {name} = (\d+);", open(os.path.join(SRC, fname)).read())
    assert m, name
    return int(m.group(1))


CHUNK = _constant("kPoolChunk", "launch.h")
PRE = _constant("kSelectPre", "kernels.hip")
THREADS = 256


def orderable(scores):
    """Order-preserving uint32 keys of float32 scores (-0 as +0)."""
    u = np.asarray(scores, np.float32).view(np.uint32).astype(np.uint64)
    u = np.where((u & 0x7FFFFFFF) == 0, 0, u)
    return np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000).astype(np.uint64)


def select_bin(hist, prefix, need, bits):
    """The bin (from the top) holding the need-th largest key: the extended
    prefix and the rank left inside that bin."""
    above = 0
    for b in range(len(hist) - 1, -1, -1):
        c = int(hist[b])
        if above < need <= above + c:
            return (prefix << bits) | b, need - above
        above += c
    raise AssertionError("need beyond the histogram")


def radix_prefix(keys, K):
    """The two histogram passes: the 22-bit prefix and the rank in it."""
    h0 = np.bincount((keys >> 21).astype(np.int64), minlength=2048)
    p11, r0 = select_bin(h0, 0, K, 11)
    m = (keys >> 21) == p11
    h1 = np.bincount(((keys[m] >> 10) & 2047).astype(np.int64), minlength=2048)
    return select_bin(h1, p11, r0, 11)


def collect(keys, p22, F, order="jwl"):
    """pool_collect_kernel for one request: the candidate stretch (key, id)
    per 1024-id chunk (unused places hold garbage), the counts, and the last
    histogram."""
    V = len(keys)
    nsub = (V + CHUNK - 1) // CHUNK
    rng = np.random.default_rng(V)
    cand = rng.integers(0, 2 ** 32, size=(V, 2), dtype=np.uint64)  # stale contents
    cnt = np.zeros(nsub, np.int64)
    hist2 = np.zeros(1024, np.int64)
    per = CHUNK // 256
    for blk in range((V + F * CHUNK - 1) // (F * CHUNK)):
        v0 = blk * F * CHUNK
        for f in range(F):
            sub = v0 + f * CHUNK
            if sub >= V:
                continue
            ids = []
            js = range(f * per, (f + 1) * per)
            if order == "jwl":   # the kernel's order: load, then wave, then lane
                for j in js:
                    ids.extend(v0 + j * 256 + t for t in range(256))
            else:                # a planted mistake: wave before load
                for w in range(4):
                    for j in js:
                        ids.extend(v0 + j * 256 + w * 64 + l for l in range(64))
            ids = np.array([i for i in ids if i < V], np.int64)
            take = ids[(keys[ids] >> 10) >= p22]
            n = len(take)
            assert n <= min(CHUNK, V - sub)
            cand[sub:sub + n, 0] = keys[take]
            cand[sub:sub + n, 1] = take
            cnt[sub // CHUNK] = n
        eqp = np.arange(v0, min(v0 + F * CHUNK, V))
        eqp = eqp[(keys[eqp] >> 10) == p22]
        np.add.at(hist2, (keys[eqp] & 1023).astype(np.int64), 1)
    return cand, cnt, hist2


def select(cand, cnt, hist2, p22, r1, V, K, clamp=True, cap=True):
    """pool_select_kernel for one request; returns the pool (K ids)."""
    nch = len(cnt)
    T, need = select_bin(hist2, p22, r1, 10)
    cpt = (nch + THREADS - 1) // THREADS

    def rd(i):
        assert 0 <= i < V, f"candidate read {i} outside the request's stretch"
        return int(cand[i, 0]), int(cand[i, 1])

    runs = []
    for t in range(THREADS):
        c0, c1 = min(t * cpt, nch), min(t * cpt + cpt, nch)
        first = min(c0, nch - 1)
        src0 = first * CHUNK
        last = min(CHUNK, V - first * CHUNK) - 1
        pre = [rd(src0 + (min(j, last) if clamp else j)) for j in range(PRE)]
        n0 = int(cnt[c0]) if c0 < c1 else 0
        items = [pre[j] for j in range(min(PRE, n0))]

        def tail(src, j0, n):  # 4 loads at a time, clamped to the chunk's last candidate
            got = []
            for j in range(j0, n, 4):
                batch = [rd(src + min(j + i, n - 1)) for i in range(4)]
                got += [batch[i] for i in range(4) if j + i < n]
            return got

        items += tail(src0, PRE, n0)
        for c in range(c0 + 1, c1):
            items += tail(c * CHUNK, 0, int(cnt[c]))
        runs.append(items)
    gt = [sum(k > T for k, _ in it) for it in runs]
    eq = [sum(k == T for k, _ in it) for it in runs]
    out = np.full(K, -1, np.int64)
    gtb = eqb = 0
    for t, items in enumerate(runs):
        pos = gtb + (min(eqb, need) if cap else eqb)
        e = eqb
        for k, i in items:
            sel = k > T or (k == T and e < need)
            e += k == T
            if sel:
                if pos < K:
                    out[pos] = i
                pos += 1
        gtb += gt[t]
        eqb += eq[t]
    return out


def reference_pool(keys, K):
    order = np.lexsort((np.arange(len(keys)), -keys.astype(np.int64)))
    return np.sort(order[:K])


def run_case(scores, K, F, **mistakes):
    keys = orderable(scores)
    p22, r1 = radix_prefix(keys, K)
    cand, cnt, hist2 = collect(keys, p22, F, order=mistakes.pop("order", "jwl"))
    got = select(cand, cnt, hist2, p22, r1, len(keys), K, **mistakes)
    return got, reference_pool(keys, K)


def _scores(V, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal(V).astype(np.float32)
    if kind == "coarse":      # many exact ties, some across chunk borders
        return (np.round(rng.standard_normal(V) * 8) / 8).astype(np.float32)
    if kind == "flat":        # every score equal
        return np.full(V, 1.5, np.float32)
    if kind == "signed":      # negative scores and both zeros
        s = np.round(rng.standard_normal(V) * 2) / 2
        s[rng.integers(0, V, V // 10)] = -0.0
        return s.astype(np.float32)
    raise ValueError(kind)


CASES = [(37, 5, 1, "normal"), (37, 36, 4, "coarse"), (1000, 1, 1, "normal"),
         (1024, 1023, 1, "coarse"), (1025, 300, 2, "signed"), (5003, 300, 1, "coarse"),
         (5003, 700, 4, "flat"), (5003, 5002, 2, "flat"), (20011, 2048, 4, "coarse"),
         (151936, 2048, 1, "normal"), (300007, 9000, 1, "coarse"), (300007, 2048, 4, "normal")]


@pytest.mark.parametrize("V,K,F,kind", CASES)
def test_selection_replay(V, K, F, kind):
    got, want = run_case(_scores(V, kind, V + K), K, F)
    assert np.array_equal(got, want)


def test_planted_uncapped_place_fails():
    """Placing a thread's first id at gt + eq (without the min with need)
    shifts every later id once earlier runs hold more keys equal to the
    threshold than are taken: here the first two chunks tie at the threshold
    and 200 larger keys sit in later chunks, which the mistake drops."""
    scores = np.full(5003, 1.0, np.float32)
    rng = np.random.default_rng(4)
    scores[2048 + rng.choice(5003 - 2048, 200, replace=False)] = 2.0
    got, want = run_case(scores, 500, 1)
    assert np.array_equal(got, want)
    got, want = run_case(scores, 500, 1, cap=False)
    assert not np.array_equal(got, want)


def test_planted_unclamped_preload_fails():
    """Without the clamp to the chunk's last id, the preload of a short last
    chunk reads past the vocabulary."""
    with pytest.raises(AssertionError, match="outside"):
        run_case(_scores(1025, "normal", 2), 300, 1, clamp=False)


def test_planted_wave_major_order_fails():
    """Compacting in (wave, load, lane) order instead of (load, wave, lane)
    leaves a chunk's candidates out of id order."""
    got, want = run_case(_scores(5003, "normal", 3), 2000, 1, order="wjl")
    assert not np.array_equal(got, want)
