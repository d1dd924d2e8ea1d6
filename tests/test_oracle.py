"""Pins of the CPU oracle to things other than itself (runs without a GPU).

Each test names what fixes the expected value: a worked example printed on the
pages (tests/golden), a library routine the definition reduces to (torch's
scaled_dot_product_attention in float64, scipy's logsumexp), a brute-force
pure-Python evaluation on tiny inputs, or an identity / invariant that the
pages state.  The last group plants mistakes into the oracle (on the CPU) and
checks that some pin catches each one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import MASK_CAUSAL, MASK_NONE, MASK_PREFIX_CAUSAL, SeqSpec
from oracle import splitkv as osk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "split_counts_worked_examples.json")
MASKS = {"none": MASK_NONE, "causal": MASK_CAUSAL, "prefix_causal": MASK_PREFIX_CAUSAL}


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _spec_from_case(c):
    return SeqSpec(
        sq=c["sq"], sk=c["sk"], split_kv=c["split_kv"], n_per_block=c["n_per_block"],
        mask=MASKS[c["mask"]], prefix_offset=c["prefix_offset"], last_valid=c["last_valid"],
    )


def _expected_counts(c):
    if "expected" in c:
        return np.array(c["expected"])
    return np.concatenate([np.full(n, v) for v, n in c["expected_runs"]])


# ---------------------------------------------------------------------------
# Counts: worked examples printed on the pages
# ---------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_counts_worked_examples(case):
    """Recombine fully masked split-KV partials on the host: CHECK / STRADDLE /
    MULTITILE / decode counts as printed in the review rounds."""
    spec = _spec_from_case(case)
    got = oracle.valid_split_counts(spec)
    np.testing.assert_array_equal(got, _expected_counts(case))


def test_straddle_needs_key_tile_32():
    """The STRADDLE counts fix the reading n_per_block = 32: 16 and 64 give other counts."""
    base = dict(sq=4, sk=128, split_kv=4, mask=MASK_PREFIX_CAUSAL, prefix_offset=62)
    assert list(oracle.valid_split_counts(SeqSpec(n_per_block=32, **base))) == [2, 2, 3, 3]
    assert list(oracle.valid_split_counts(SeqSpec(n_per_block=16, **base))) != [2, 2, 3, 3]
    assert list(oracle.valid_split_counts(SeqSpec(n_per_block=64, **base))) != [2, 2, 3, 3]


# ---------------------------------------------------------------------------
# Counts: brute force and the invariants the pages state
# ---------------------------------------------------------------------------

def _count_brute(row_last, nPB, S):
    """Enumerate the row's keys 0..rowLast, deal its key tiles into S equal
    runs of whole tiles (the fewest tiles per run that covers them all), and
    count the runs that receive a key.  Pure Python, no closed form."""
    n_keys = row_last + 1
    n_tiles = 0
    while n_tiles * nPB < n_keys:
        n_tiles += 1
    per = 0
    while per * S < n_tiles:
        per += 1
    used = set()
    for k in range(n_keys):
        used.add((k // nPB) // per)
    return len(used)


def _sweep_specs():
    for sq, sk, S, nPB, mask in itertools.product(
        (1, 5, 33), (0, 1, 7, 64, 100), (1, 2, 3, 4, 7), (1, 4, 16, 32), (MASK_NONE, MASK_CAUSAL, MASK_PREFIX_CAUSAL)
    ):
        offs = (0,) if mask != MASK_PREFIX_CAUSAL else (-40, -3, 0, 5, 62, 99)
        for off in offs:
            for lv in (-1, 0, sk // 2, sk + 10):
                yield SeqSpec(sq, sk, S, nPB, mask, off, lv)


def test_counts_brute_force_and_bounds():
    """count equals the number of non-empty runs found by enumeration, and
    1 <= count <= split_kv (the reviewer's bound)."""
    n = 0
    for spec in _sweep_specs():
        counts = oracle.valid_split_counts(spec)
        rl = oracle.row_last(np.arange(spec.sq), spec)
        for q in range(spec.sq):
            assert counts[q] == _count_brute(int(rl[q]), spec.n_per_block, spec.split_kv), (spec, q)
            assert 1 <= counts[q] <= spec.split_kv
            n += 1
    assert n > 10000


def test_counts_are_conservative_for_every_block_size():
    """The host count never drops a split holding the row's data: every split
    s >= count of the row's block partition holds no key the row sees
    (conservativeness argument of the reviewer rounds)."""
    for spec in _sweep_specs():
        counts = oracle.valid_split_counts(spec)
        vis = oracle.visible_last_key(np.arange(spec.sq), spec)
        for mpb in (1, 2, 8, 16, 64):
            for j in range(-(-spec.sq // mpb)):
                ranges = oracle.block_split_ranges(spec, mpb, j)
                for q in range(j * mpb, min((j + 1) * mpb, spec.sq)):
                    holding = [s for s, (a, b) in enumerate(ranges) if b > a and a <= vis[q]]
                    assert all(s < counts[q] for s in holding), (spec, mpb, q)


def test_block_partition_covers_every_visible_key_once():
    """Union of a block's split ranges = keys 0..rowLast of the block's last row,
    disjoint and in order; every row of the block sees only keys inside it."""
    for spec in _sweep_specs():
        vis = oracle.visible_last_key(np.arange(spec.sq), spec)
        for mpb in (1, 3, 16):
            for j in range(-(-spec.sq // mpb)):
                ranges = oracle.block_split_ranges(spec, mpb, j)
                covered = []
                for a, b in ranges:
                    covered.extend(range(a, b))
                assert covered == list(range(len(covered)))
                rows = range(j * mpb, min((j + 1) * mpb, spec.sq))
                for q in rows:
                    assert vis[q] < len(covered)


def _brute_window_attention(Q, K, V, scale, q, lo, hi):
    """Pure-Python softmax attention of row q over keys lo..hi (inclusive)."""
    keys = [k for k in range(len(K)) if lo <= k <= hi]
    if not keys:
        return [0.0] * len(V[0]), -math.inf
    x = [scale * sum(a * b for a, b in zip(Q[q], K[k])) for k in keys]
    m = max(x)
    e = [math.exp(v - m) for v in x]
    z = sum(e)
    return [sum(e[i] * V[k][d] for i, k in enumerate(keys)) / z for d in range(len(V[0]))], m + math.log(z)


@pytest.mark.parametrize("mask,off,win,lv", [
    (MASK_CAUSAL, 0, 3, -1), (MASK_CAUSAL, 0, 0, -1), (MASK_PREFIX_CAUSAL, 9, 5, -1),
    (MASK_PREFIX_CAUSAL, -3, 4, 20), (MASK_NONE, 0, 6, -1), (MASK_PREFIX_CAUSAL, 2, 40, 12),
])
def test_sliding_window_matches_brute_force(mask, off, win, lv):
    """Left window: row q sees keys q + off - win .. vis(q), checked against
    explicit loops; split -> merge reproduces it for several split shapes."""
    rng = np.random.default_rng(31)
    sq, sk, d = 14, 26, 3
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, 2)
    spec = SeqSpec(sq, sk, 3, 4, mask, off, lv, window_left=win)
    O, lse = oracle.unsplit(Q, K, V, 0.7, spec)
    last = spec.last_valid_index
    for q in range(sq):
        hi = min(q + spec.offset, last) if mask != MASK_NONE else last
        o, l = _brute_window_attention(Q.tolist(), K.tolist(), V.tolist(), 0.7, q, q + spec.offset - win, hi)
        np.testing.assert_allclose(O[q], o, rtol=1e-12, atol=1e-12)
        assert (lse[q] == l) if l == -math.inf else abs(lse[q] - l) < 1e-12
    for S, nPB, mpb in ((1, 4, 4), (3, 4, 8), (5, 2, 16), (9, 1, 3)):
        sp = SeqSpec(sq, sk, S, nPB, mask, off, lv, window_left=win)
        O2, lse2, *_ = oracle.split_attention(Q, K, V, 0.7, sp, mpb)
        np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(lse2), np.isneginf(lse))


def test_sliding_window_matches_torch_sdpa_with_explicit_mask():
    rng = np.random.default_rng(32)
    sq, sk, d = 40, 70, 16
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, 8)
    spec = SeqSpec(sq, sk, 4, 8, MASK_PREFIX_CAUSAL, 30, window_left=12)
    O, _ = oracle.unsplit(Q, K, V, 0.25, spec)
    q = np.arange(sq)[:, None]
    k = np.arange(sk)[None, :]
    allowed = torch.from_numpy((k <= q + 30) & (k >= q + 30 - 12))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
        attn_mask=allowed[None, None], scale=0.25)[0, 0].numpy()
    np.testing.assert_allclose(O, ref, rtol=1e-12, atol=1e-12)
    # the window leaves the count formula alone: it is conservative still
    assert np.array_equal(oracle.valid_split_counts(spec),
                          oracle.valid_split_counts(SeqSpec(sq, sk, 4, 8, MASK_PREFIX_CAUSAL, 30)))
    assert oracle.visible_pairs(spec) == sq * 13


@pytest.mark.parametrize("mask,off,win,lv", [
    (MASK_NONE, 0, -1, -1), (MASK_CAUSAL, 0, -1, -1), (MASK_PREFIX_CAUSAL, 6, -1, 15),
    (MASK_PREFIX_CAUSAL, -4, -1, -1), (MASK_CAUSAL, 0, 3, -1),
])
def test_backward_matches_torch_autograd_f64(mask, off, win, lv):
    """The gradient formulas against torch autograd through float64 SDPA with
    the same explicit visibility mask (rows with no visible key are given a
    zero gradient on both sides)."""
    rng = np.random.default_rng(41)
    sq, sk, d, dv = 13, 22, 6, 5
    Q, K, V, dO = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, dv), _rand(rng, sq, dv)
    spec = SeqSpec(sq, sk, 3, 4, mask, off, lv, window_left=win)
    dQ, dK, dV = oracle.unsplit_backward(Q, K, V, dO, 0.6, spec)
    vis = torch.from_numpy(osk.visible_keys(np.arange(sq), spec, np.arange(sk)))
    has = vis.any(dim=1)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_() for a in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[has][None, None], tk[None, None], tv[None, None], attn_mask=vis[has][None, None], scale=0.6)[0, 0]
    o.backward(torch.from_numpy(dO)[has])
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_matches_finite_differences():
    """Central differences of <dO, unsplit(...)> in a few coordinates of Q, K and V."""
    rng = np.random.default_rng(42)
    sq, sk, d, dv = 5, 9, 3, 2
    Q, K, V, dO = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, dv), _rand(rng, sq, dv)
    spec = SeqSpec(sq, sk, 2, 4, MASK_PREFIX_CAUSAL, 2, window_left=4)
    grads = oracle.unsplit_backward(Q, K, V, dO, 0.9, spec)

    def f(Q, K, V):
        return float((oracle.unsplit(Q, K, V, 0.9, spec)[0] * dO).sum())

    h = 1e-6
    for which, (i, j) in ((0, (1, 2)), (0, (4, 0)), (1, (3, 1)), (1, (6, 2)), (2, (2, 0)), (2, (5, 1))):
        args = [Q.copy(), K.copy(), V.copy()]
        args[which][i, j] += h
        fp = f(*args)
        args[which][i, j] -= 2 * h
        fm = f(*args)
        assert abs((fp - fm) / (2 * h) - grads[which][i, j]) < 1e-7


@pytest.mark.parametrize("mask,off,win", [(MASK_NONE, 0, -1), (MASK_PREFIX_CAUSAL, 20, 9), (MASK_CAUSAL, 0, -1)])
def test_sampled_backward_matches_torch_autograd_f64(mask, off, win):
    """The chunked form used at full size: rows spread over several chunks
    (including a ragged last one), against torch autograd through float64
    SDPA with the explicit visibility mask."""
    rng = np.random.default_rng(43)
    sq, sk, d, dv = 37, 50, 5, 4
    Q, K, V, dO = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, dv), _rand(rng, sq, dv)
    spec = SeqSpec(sq, sk, 2, 4, mask, off, window_left=win)
    rows = np.array([0, 1, 7, 8, 9, 30, 36])
    keys = np.array([0, 5, 17, 31, 49])
    dQ, dK, dV = oracle.sampled_backward(Q, K, V, dO, 0.45, spec, rows, keys, chunk=8)
    vis = torch.from_numpy(osk.visible_keys(np.arange(sq), spec, np.arange(sk)))
    has = vis.any(dim=1)
    tq, tk, tv = (torch.from_numpy(a).requires_grad_() for a in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[has][None, None], tk[None, None], tv[None, None], attn_mask=vis[has][None, None], scale=0.45)[0, 0]
    o.backward(torch.from_numpy(dO)[has])
    np.testing.assert_allclose(dQ, tq.grad.numpy()[rows], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy()[keys], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy()[keys], rtol=1e-11, atol=1e-12)


def test_block_populated_splits_hold_every_key_the_block_sees():
    """Real early exit: the splits a block still writes (populated) include
    every split holding a key that any row of the block sees, and every other
    split is (0, -inf) for all the block's rows, so a merge over
    s < min(count, populated) is the merge over s < count."""
    rng = np.random.default_rng(11)
    n = 0
    for spec in _sweep_specs():
        if spec.sq > 40 or spec.sk > 60:
            continue
        Q, K, V = _rand(rng, spec.sq, 4), _rand(rng, spec.sk, 4), _rand(rng, spec.sk, 3)
        counts = oracle.valid_split_counts(spec)
        for mpb in (1, 8, 16):
            pop = np.array([oracle.block_populated_splits(spec, mpb, q) for q in range(spec.sq)])
            for q in range(spec.sq):
                assert oracle.kernel_nonempty_splits(spec, mpb, q) <= pop[q] <= spec.split_kv, (spec, mpb, q)
            O_s, L_s = oracle.partials(Q, K, V, 0.5, spec, mpb)
            for q in range(spec.sq):
                assert np.isneginf(L_s[pop[q]:, q]).all() and (O_s[pop[q]:, q] == 0).all(), (spec, mpb, q)
            O1, l1 = oracle.combine(O_s, L_s, counts)
            O2, l2 = oracle.combine(O_s, L_s, np.minimum(counts, pop))
            np.testing.assert_array_equal(O1, O2)
            np.testing.assert_array_equal(l1, l2)
            n += 1
    assert n > 100


def test_block_populated_splits_special_cases():
    # every row sees every key: one partition, populated = count = ceil(Sk / kps)
    spec = SeqSpec(40, 300, 4, 32, MASK_NONE)
    kps = 32 * math.ceil(math.ceil(300 / 32) / 4)  # 96
    assert all(oracle.block_populated_splits(spec, 16, q) == math.ceil(300 / kps) == 4 for q in range(40))
    # no key at all (lastValid = -1 after clamping an empty K): nothing to write
    assert oracle.block_populated_splits(SeqSpec(5, 0, 3, 16, MASK_NONE), 4, 2) == 0
    # causal, first block of 16 rows (keys 0..15): key tile 4 gives kps = 4 and
    # all 4 splits hold keys; key tile 16 gives kps = 16 and only split 0 does
    assert oracle.block_populated_splits(SeqSpec(64, 64, 4, 4, MASK_CAUSAL), 16, 0) == 4
    assert oracle.block_populated_splits(SeqSpec(64, 64, 4, 16, MASK_CAUSAL), 16, 3) == 1


def test_noncausal_counts_are_per_sequence():
    """Non-causal configs keep one count per batch-head (every row equal)."""
    for spec in _sweep_specs():
        if spec.mask == MASK_NONE and spec.sq > 0:
            c = oracle.valid_split_counts(spec)
            assert (c == c[0]).all()


def test_aiter_count_shape():
    """The count-test shape of the aiter split-KV tests (sq=129, sk=2048, splits
    2..8), non-causal: with a key tile that divides 2048 every split holds keys."""
    for S in range(2, 9):
        for nPB in (32, 64):
            c = oracle.valid_split_counts(SeqSpec(129, 2048, S, nPB))
            assert (c == S).all()


# ---------------------------------------------------------------------------
# Attention: the plain definition against library routines and brute force
# ---------------------------------------------------------------------------

def _sdpa_f64(Q, K, V, scale, causal):
    q = torch.from_numpy(Q)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    return o[0, 0].numpy()


@pytest.mark.parametrize("sq,sk,d,dv", [(8, 8, 16, 16), (17, 40, 32, 24), (64, 256, 64, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_unsplit_matches_torch_sdpa_f64(sq, sk, d, dv, causal):
    """Unmasked and top-left causal attention reduce to torch's SDPA (float64, CPU)."""
    rng = np.random.default_rng(1)
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, dv)
    scale = 1 / math.sqrt(d)
    spec = SeqSpec(sq, sk, 1, 16, MASK_CAUSAL if causal else MASK_NONE)
    O, _ = oracle.unsplit(Q, K, V, scale, spec)
    np.testing.assert_allclose(O, _sdpa_f64(Q, K, V, scale, causal), rtol=1e-12, atol=1e-12)


def test_unsplit_lse_matches_scipy_logsumexp():
    rng = np.random.default_rng(2)
    sq, sk, d = 9, 50, 8
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, 3)
    spec = SeqSpec(sq, sk, 1, 8, MASK_PREFIX_CAUSAL, prefix_offset=20, last_valid=40)
    _, lse = oracle.unsplit(Q, K, V, 0.3, spec)
    for q in range(sq):
        last = min(q + 20, 40)
        x = 0.3 * (K[: last + 1] @ Q[q])
        assert abs(lse[q] - scipy.special.logsumexp(x)) < 1e-12


def _attention_brute(Q, K, V, scale, spec):
    """Pure-Python loops, math.exp, no max subtraction (tiny inputs only)."""
    out, lses = [], []
    for q in range(spec.sq):
        if spec.mask == MASK_NONE:
            last = spec.last_valid_index
        else:
            last = min(q + spec.offset, spec.last_valid_index)
        ws, acc = 0.0, [0.0] * V.shape[1]
        for k in range(0, last + 1):
            x = scale * sum(float(Q[q, d]) * float(K[k, d]) for d in range(Q.shape[1]))
            w = math.exp(x)
            ws += w
            for c in range(V.shape[1]):
                acc[c] += w * float(V[k, c])
        if ws == 0.0:
            out.append([0.0] * V.shape[1])
            lses.append(-math.inf)
        else:
            out.append([a / ws for a in acc])
            lses.append(math.log(ws))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize(
    "mask,off,lv",
    [(MASK_NONE, 0, -1), (MASK_NONE, 0, 9), (MASK_CAUSAL, 0, -1), (MASK_PREFIX_CAUSAL, 4, -1),
     (MASK_PREFIX_CAUSAL, -3, -1), (MASK_PREFIX_CAUSAL, 6, 11), (MASK_CAUSAL, 0, 2)],
)
def test_unsplit_matches_brute_force(mask, off, lv):
    rng = np.random.default_rng(3)
    sq, sk, d, dv = 7, 15, 5, 4
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, dv)
    spec = SeqSpec(sq, sk, 1, 4, mask, off, lv)
    O, lse = oracle.unsplit(Q, K, V, 0.7, spec)
    Ob, lseb = _attention_brute(Q, K, V, 0.7, spec)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(lseb))
    fin = np.isfinite(lseb)
    np.testing.assert_allclose(lse[fin], lseb[fin], rtol=1e-12, atol=1e-13)


def test_single_visible_key_gives_that_value_row():
    """A row that sees exactly one key returns that V row exactly, LSE = its score."""
    rng = np.random.default_rng(4)
    sq, sk, d = 6, 20, 8
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, 8)
    spec = SeqSpec(sq, sk, 3, 4, MASK_CAUSAL)
    O, lse, *_ = oracle.split_attention(Q, K, V, 0.5, spec, m_per_block=4)
    np.testing.assert_array_equal(O[0], V[0])
    assert lse[0] == 0.5 * float(Q[0] @ K[0])


def test_fully_masked_rows_are_exactly_zero():
    """Rows whose every split is empty give 0 output and -inf LSE, never NaN
    (NaN-safe merge)."""
    rng = np.random.default_rng(5)
    sq, sk, d = 40, 64, 16
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, 16)
    spec = SeqSpec(sq, sk, 4, 8, MASK_PREFIX_CAUSAL, prefix_offset=-16)
    O, lse, counts, O_s, L_s = oracle.split_attention(Q, K, V, 0.25, spec, m_per_block=16)
    assert not np.isnan(O).any() and not np.isnan(lse).any()
    assert (O[:16] == 0).all() and np.isneginf(lse[:16]).all()
    assert np.isfinite(lse[16:]).all()
    assert (O_s[:, :16] == 0).all() and np.isneginf(L_s[:, :16]).all()


def test_offsets_beyond_32_bits_reduce_to_the_plain_cases():
    """A prefix offset of +2^40 makes every key visible (no mask), -2^40 none
    (every row fully masked, count 1), and +2^40 with a window of w puts
    every window's start past the last key."""
    rng = np.random.default_rng(12)
    sq, sk, d = 9, 40, 6
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, 5)
    plain = oracle.unsplit(Q, K, V, 0.4, SeqSpec(sq, sk, 3, 8, MASK_NONE))
    far = oracle.unsplit(Q, K, V, 0.4, SeqSpec(sq, sk, 3, 8, MASK_PREFIX_CAUSAL, 1 << 40))
    np.testing.assert_array_equal(far[0], plain[0])
    np.testing.assert_array_equal(far[1], plain[1])
    below = SeqSpec(sq, sk, 3, 8, MASK_PREFIX_CAUSAL, -(1 << 40))
    O, lse = oracle.unsplit(Q, K, V, 0.4, below)
    assert (O == 0).all() and np.isneginf(lse).all()
    assert (oracle.valid_split_counts(below) == 1).all()
    win = SeqSpec(sq, sk, 3, 8, MASK_PREFIX_CAUSAL, 1 << 40, window_left=5)
    O, lse = oracle.unsplit(Q, K, V, 0.4, win)
    assert (O == 0).all() and np.isneginf(lse).all()
    assert (oracle.valid_split_counts(win) == oracle.valid_split_counts(SeqSpec(sq, sk, 3, 8, MASK_NONE))).all()


def test_empty_key_sequence():
    """Empty K returns zero output and -inf LSE instead of an error (aiter review)."""
    Q = np.ones((3, 4))
    K = np.zeros((0, 4))
    V = np.zeros((0, 2))
    for mask in (MASK_NONE, MASK_CAUSAL):
        spec = SeqSpec(3, 0, 2, 8, mask)
        O, lse, counts, _, _ = oracle.split_attention(Q, K, V, 1.0, spec, m_per_block=2)
        assert (O == 0).all() and np.isneginf(lse).all()
        assert (counts == 1).all()


# ---------------------------------------------------------------------------
# The method: merged partials equal the plain definition (closed-form identity)
# ---------------------------------------------------------------------------

def _identity_cases():
    for S, nPB, mpb in itertools.product((1, 2, 3, 5, 9), (1, 4, 16, 32), (1, 8, 16, 64)):
        for mask, off, lv in ((MASK_NONE, 0, -1), (MASK_NONE, 0, 50), (MASK_CAUSAL, 0, -1),
                              (MASK_PREFIX_CAUSAL, 30, -1), (MASK_PREFIX_CAUSAL, -7, 70)):
            yield S, nPB, mpb, mask, off, lv


def test_split_merge_equals_unsplit():
    """split -> merge reproduces plain attention for every split count, key tile,
    block size and mask (the identity the NaN-safe merge implements)."""
    rng = np.random.default_rng(6)
    sq, sk, d, dv = 37, 90, 12, 10
    Q, K, V = _rand(rng, sq, d), _rand(rng, sk, d), _rand(rng, sk, dv)
    for S, nPB, mpb, mask, off, lv in _identity_cases():
        spec = SeqSpec(sq, sk, S, nPB, mask, off, lv)
        O, lse, *_ = oracle.split_attention(Q, K, V, 0.4, spec, mpb)
        Ou, lseu = oracle.unsplit(Q, K, V, 0.4, spec)
        np.testing.assert_allclose(O, Ou, rtol=1e-12, atol=1e-12, err_msg=str(spec))
        np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lseu))
        fin = np.isfinite(lseu)
        np.testing.assert_allclose(lse[fin], lseu[fin], rtol=1e-12, atol=1e-12)


def test_split_one_is_plain_attention_partial():
    """With split_kv = 1 the single partial is the plain attention itself."""
    rng = np.random.default_rng(7)
    Q, K, V = _rand(rng, 20, 8), _rand(rng, 30, 8), _rand(rng, 30, 8)
    spec = SeqSpec(20, 30, 1, 16, MASK_CAUSAL)
    O_s, L_s = oracle.partials(Q, K, V, 0.3, spec, 8)
    Ou, lseu = oracle.unsplit(Q, K, V, 0.3, spec)
    np.testing.assert_allclose(O_s[0], Ou, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(L_s[0], lseu, rtol=1e-13, atol=1e-13)


def test_row_subsets_match_full_evaluation():
    rng = np.random.default_rng(8)
    sq, sk = 50, 80
    Q, K, V = _rand(rng, sq, 8), _rand(rng, sk, 8), _rand(rng, sk, 6)
    spec = SeqSpec(sq, sk, 3, 8, MASK_PREFIX_CAUSAL, prefix_offset=10)
    rows = np.array([0, 7, 16, 31, 49])
    O, lse, counts, O_s, L_s = oracle.split_attention(Q, K, V, 0.2, spec, 16)
    o, l, c, o_s, l_s = oracle.split_attention(Q[rows], K, V, 0.2, spec, 16, rows=rows)
    # BLAS may block a row subset differently: equal up to f64 rounding
    np.testing.assert_allclose(O[rows], o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[rows], l, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(counts[rows], c)
    np.testing.assert_allclose(O_s[:, rows], o_s, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(L_s[:, rows], l_s, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# The merge on its own
# ---------------------------------------------------------------------------

def test_merge_clamps_are_noops_when_a_split_is_finite():
    """With at least one finite L_s the clamped merge equals the unclamped formula."""
    rng = np.random.default_rng(9)
    S, rows, dv = 5, 30, 4
    O_s = rng.standard_normal((S, rows, dv))
    L_s = rng.standard_normal((S, rows)) * 3
    L_s[rng.random((S, rows)) < 0.4] = -np.inf
    L_s[0] = rng.standard_normal(rows)  # at least one finite split per row
    O_s[np.isneginf(L_s)] = 0.0
    counts = np.full(rows, S)
    O, lse = oracle.combine(O_s, L_s, counts)
    m = L_s.max(axis=0)
    w = np.exp(L_s - m)
    ref = (w[..., None] * O_s).sum(0) / w.sum(0)[:, None]
    np.testing.assert_allclose(O, ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(L_s, axis=0), rtol=1e-13, atol=1e-13)


def test_merge_all_empty_and_invalid_splits():
    S, rows, dv = 4, 6, 3
    O_s = np.full((S, rows, dv), np.nan)
    L_s = np.full((S, rows), np.nan)
    # rows 0..2: every valid split empty; rows 3..5: valid split 0 only, rest garbage
    O_s[:2, :3] = 0.0
    L_s[:2, :3] = -np.inf
    O_s[0, 3:] = 2.0
    L_s[0, 3:] = 1.5
    counts = np.array([2, 2, 2, 1, 1, 1])
    O, lse = oracle.combine(O_s, L_s, counts)
    assert (O[:3] == 0).all() and np.isneginf(lse[:3]).all()
    assert (O[3:] == 2.0).all() and (lse[3:] == 1.5).all()


def test_merge_is_order_independent():
    rng = np.random.default_rng(10)
    S, rows, dv = 6, 10, 5
    O_s = rng.standard_normal((S, rows, dv))
    L_s = rng.standard_normal((S, rows))
    perm = rng.permutation(S)
    a = oracle.combine(O_s, L_s, np.full(rows, S))
    b = oracle.combine(O_s[perm], L_s[perm], np.full(rows, S))
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13)


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by one of the pins above
# ---------------------------------------------------------------------------

def _golden_ok():
    try:
        for case in _golden_cases():
            test_counts_worked_examples(case)
        return True
    except AssertionError:
        return False


def _identity_ok():
    try:
        test_split_merge_equals_unsplit()
        return True
    except AssertionError:
        return False


@pytest.mark.filterwarnings("ignore:divide by zero")
def test_planted_count_mistakes_are_caught(monkeypatch):
    true_kps = osk.keys_per_split
    mistakes = {
        "rowLast instead of rowLast+1": lambda rl, spec: true_kps(np.asarray(rl) - 1, spec),
        "no key-tile rounding": lambda rl, spec: osk._ceil_div(np.asarray(rl) + 1, spec.split_kv),
        "floor of tiles / split": lambda rl, spec: spec.n_per_block
        * np.maximum(1, osk._ceil_div(np.asarray(rl) + 1, spec.n_per_block) // spec.split_kv),
    }
    for name, wrong in mistakes.items():
        monkeypatch.setattr(osk, "keys_per_split", wrong)
        assert not _golden_ok(), name
        monkeypatch.setattr(osk, "keys_per_split", true_kps)
    assert _golden_ok()


def test_planted_merge_and_partition_mistakes_are_caught(monkeypatch):
    true_ranges = osk.block_split_ranges

    def first_row_partition(spec, mpb, block):
        # uses the block's FIRST row instead of its last
        rl = int(osk.row_last([block * mpb], spec)[0])
        kps = int(osk.keys_per_split(rl, spec))
        return [(min(s * kps, rl + 1), min((s + 1) * kps, rl + 1)) for s in range(spec.split_kv)]

    def off_by_one_end(spec, mpb, block):
        return [(a, max(a, b - 1)) if s == 0 else (a, b) for s, (a, b) in enumerate(true_ranges(spec, mpb, block))]

    for wrong in (first_row_partition, off_by_one_end):
        monkeypatch.setattr(osk, "block_split_ranges", wrong)
        assert not _identity_ok(), wrong.__name__
        monkeypatch.setattr(osk, "block_split_ranges", true_ranges)

    true_combine = osk.combine

    def sign_flip(O_s, L_s, counts):
        return true_combine(O_s, -np.asarray(L_s), counts)

    def no_normalise(O_s, L_s, counts):
        O, lse = true_combine(O_s, L_s, counts)
        return O * 1.01, lse

    for wrong in (sign_flip, no_normalise):
        monkeypatch.setattr(osk, "combine", wrong)
        assert not _identity_ok(), wrong.__name__
        monkeypatch.setattr(osk, "combine", true_combine)
    assert _identity_ok()
