"""Pins of the oracle's verification index-set selection (Dustin page,
methodology 1: sinks and a recent window kept, then the top-m positions by
the draft-lookahead signal, then the best remaining positions by the
target-historical signal) and of the recall-rate identity."""

import itertools

import numpy as np

import oracle


def _py_select(draft, target, c, n_sel, n_sink, n_recent, m):
    """Independent pure-Python statement of the same rule (tuple-key sort)."""
    c = max(0, min(c, len(draft)))
    lo = min(n_sink, c)
    hi = max(c - n_recent, lo)
    keep = set(range(lo)) | set(range(hi, c))
    fill = n_sel - len(keep)

    def key(scores, p):
        s = float(scores[p])
        return (s != s, 0.0 if s != s else -s, p)   # NaN last, then higher score, then lower p

    cand = list(range(lo, hi))
    by_d = sorted(cand, key=lambda p: key(draft, p))[:min(m, fill, len(cand))]
    left = [p for p in cand if p not in set(by_d)]
    by_t = sorted(left, key=lambda p: key(target, p))[:min(fill - len(by_d), len(left))]
    sel = sorted(keep | set(by_d) | set(by_t))
    return sel + [-1] * (n_sel - len(sel))


def test_worked_example():
    d = np.array([[[5, 1, 9, 9, 0, 3, 7, 2, 8, 6]]], np.float32)
    t = np.array([[[0, 9, 1, 2, 8, 3, 4, 5, 6, 7]]], np.float32)
    # sink {0}, recent {8, 9}; draft top-2 of 1..7: 2 and 3 (tie at 9 -> lower
    # position first); target best of the rest {1, 4, 5, 6, 7}: 1
    got = oracle.select_kv_idx(d, t, np.array([10]), 6, 1, 2, 2)
    assert got.tolist() == [[[0, 1, 2, 3, 8, 9]]]


def test_matches_independent_statement_on_random_small_cases():
    rng = np.random.default_rng(7)
    for _ in range(400):
        S = int(rng.integers(1, 24))
        n_sel = int(rng.integers(1, 12))
        n_sink = int(rng.integers(0, n_sel + 1))
        n_recent = int(rng.integers(0, n_sel - n_sink + 1))
        m = int(rng.integers(0, n_sel + 2))
        c = int(rng.integers(0, S + 3))
        # few distinct values so that ties are common; some NaN and -0
        pool = np.array([0.0, -0.0, 1.0, 2.0, -1.0, np.nan, np.inf, -np.inf], np.float32)
        d = rng.choice(pool, size=(1, 2, S))
        t = rng.choice(pool, size=(1, 2, S))
        got = oracle.select_kv_idx(d, t, np.array([c]), n_sel, n_sink, n_recent, m)
        for g in range(2):
            want = _py_select(d[0, g], t[0, g], c, n_sel, n_sink, n_recent, m)
            assert got[0, g].tolist() == want, (S, n_sel, n_sink, n_recent, m, c, g)


def test_invariants_and_ranking_property():
    rng = np.random.default_rng(3)
    B, H, S = 3, 4, 500
    d = rng.standard_normal((B, H, S)).astype(np.float32)
    t = rng.standard_normal((B, H, S)).astype(np.float32)
    ctx = np.array([500, 37, 260])
    n_sel, n_sink, n_recent, m = 64, 4, 16, 20
    out = oracle.select_kv_idx(d, t, ctx, n_sel, n_sink, n_recent, m)
    for b in range(B):
        c = int(ctx[b])
        for g in range(H):
            row = out[b, g]
            valid = row[row >= 0]
            assert valid.size == min(n_sel, c)
            assert (np.diff(valid) > 0).all() and (valid < c).all()
            s = set(valid.tolist())
            assert set(range(min(n_sink, c))) <= s
            assert set(range(max(c - n_recent, min(n_sink, c)), c)) <= s
            if c > n_sel:
                mid = [p for p in range(n_sink, c - n_recent)]
                chosen = [p for p in mid if p in s]
                # the draft-top positions are the m best draft scores of the middle
                best_d = sorted(mid, key=lambda p: -d[b, g, p])[:m]
                assert set(best_d) <= s
                # every other chosen middle position beats every unchosen one
                # on the target score
                others = [p for p in chosen if p not in set(best_d)]
                unchosen = [p for p in mid if p not in s]
                if others and unchosen:
                    assert min(t[b, g, p] for p in others) >= max(t[b, g, p] for p in unchosen)


def test_special_cases():
    S = 16
    flat = np.zeros((1, 1, S), np.float32)
    # all scores equal: the lowest positions win
    got = oracle.select_kv_idx(flat, flat, np.array([S]), 5, 0, 0, 2)
    assert got.tolist() == [[[0, 1, 2, 3, 4]]]
    # m = 0: target ranking only
    t = np.arange(S, dtype=np.float32)[None, None]
    got = oracle.select_kv_idx(flat, t, np.array([S]), 3, 0, 0, 0)
    assert got.tolist() == [[[13, 14, 15]]]
    # protected positions only (context shorter than sinks + window)
    got = oracle.select_kv_idx(flat, flat, np.array([5]), 8, 4, 4, 0)
    assert got.tolist() == [[[0, 1, 2, 3, 4, -1, -1, -1]]]
    # budget larger than the context: everything, then -1
    got = oracle.select_kv_idx(flat, t, np.array([6]), 9, 1, 1, 2)
    assert got.tolist() == [[[0, 1, 2, 3, 4, 5, -1, -1, -1]]]
    # NaN ranks below -inf; -0 ties with +0 (lower position first)
    d = np.array([[[np.nan, -np.inf, -0.0, 0.0, np.nan]]], np.float32)
    got = oracle.select_kv_idx(d, d, np.array([5]), 3, 0, 0, 3)
    assert got.tolist() == [[[1, 2, 3]]]
    got = oracle.select_kv_idx(d, d, np.array([5]), 1, 0, 0, 1)
    assert got.tolist() == [[[2]]]


def test_recall_rate_identity():
    # recall of a subset = its share of the softmax mass
    rng = np.random.default_rng(5)
    s = rng.standard_normal(50)
    subset = rng.choice(50, size=12, replace=False)
    lse_full = np.log(np.exp(s).sum())
    lse_sub = np.log(np.exp(s[subset]).sum())
    share = np.exp(s[subset]).sum() / np.exp(s).sum()
    assert abs(oracle.recall_rate(lse_sub, lse_full) - share) < 1e-12
