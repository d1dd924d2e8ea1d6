"""Plain CPU oracle for split-KV attention forward, in float64.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module; the library and its Python binding
never do, and nothing here is shared with the HIP path.

Sources (titles of the pages this follows):

[R]  "Recombine fully masked split-KV attention partials on the host"
     (rocmlirTriton pull request #535):
       - Summary (partials O_s / L_s per split, empty splits give 0 / -inf),
       - "Per-row valid-split counts", "Per-row mask layout",
       - "NaN-safe merge", "f32 merge for f16/bf16",
       - the reviewer notes on conservativeness and the block partition.
[A]  "[ASM][HIP][JIT][gfx942] Optimize long-context FMHA with split-KV"
     (aiter pull request #5592): Technical Details (num_splits, packed varlen),
     and the review note that empty K returns zero output instead of raising.

Everything is computed in float64 from the stored inputs (bf16 and f32 convert
to f64 exactly).  Where the pages leave a step open the reading taken is stated
next to the code that takes it.

Functions
---------
visible_last_key   last key a query row may see (vis(q)); < 0 means none
visible_first_key  first key a query row may see (0 without a sliding window)
valid_split_counts per-row valid-split counts [R, Per-row valid-split counts]
block_split_ranges the key range of every split for one M block
                   [R, Per-row valid-split counts, the block's last row]
unsplit            plain softmax attention over the visible keys (the definition)
partials           per-split partial O_s and L_s [R, Summary]
combine            NaN-safe merge of the partials [R, NaN-safe merge]
split_attention    counts -> partials -> combine
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_PREFIX_CAUSAL = 2

# "lowest finite" of the NaN-safe merge [R, NaN-safe merge], at the oracle's
# precision.  The GPU merge uses the f32 value; the result is the same because
# the clamp only acts when every split is -inf.
LOWEST_FINITE = -np.finfo(np.float64).max


@dataclass(frozen=True)
class SeqSpec:
    """One sequence of a (possibly packed) batch, with its split parameters.

    sq, sk        query rows and keys of this sequence
    split_kv      number of splits S (>= 1) [A, Technical Details: num_splits]
    n_per_block   split granularity in keys: GEMM0's key tile [R, Per-row
                  valid-split counts]
    mask          MASK_NONE, MASK_CAUSAL or MASK_PREFIX_CAUSAL
    prefix_offset used by MASK_PREFIX_CAUSAL; plain causal uses 0 [R]
    last_valid    last_valid_kv_index; < 0 selects the default sk - 1 [R].
                  Reading: a value beyond the sequence is clamped to sk - 1,
                  because keys past the end do not exist.
    window_left   sliding window: [A, Technical Details] lets the split path
                  take the caller's window without defining it.  Reading: a
                  left window of that many keys behind the row's position
                  q + offset (the position the causal rule uses; offset 0
                  without a prefix), i.e. keys k >= q + offset - window_left;
                  < 0 means no window.  The count formula is unchanged: it
                  depends only on the last visible key.
    """

    sq: int
    sk: int
    split_kv: int
    n_per_block: int
    mask: int = MASK_NONE
    prefix_offset: int = 0
    last_valid: int = -1
    window_left: int = -1

    def __post_init__(self):
        if self.sq < 0 or self.sk < 0:
            raise ValueError("sequence lengths must be >= 0")
        if self.split_kv < 1:
            raise ValueError("split_kv must be >= 1")
        if self.n_per_block < 1:
            raise ValueError("n_per_block must be >= 1")
        if self.mask not in (MASK_NONE, MASK_CAUSAL, MASK_PREFIX_CAUSAL):
            raise ValueError("unknown mask mode")

    @property
    def last_valid_index(self) -> int:
        if self.last_valid < 0:
            return self.sk - 1
        return min(self.last_valid, self.sk - 1)

    @property
    def offset(self) -> int:
        if self.mask == MASK_PREFIX_CAUSAL:
            return self.prefix_offset
        return 0


def _ceil_div(a, b):
    """Ceiling division of non-negative integers (numpy arrays or ints)."""
    return -((-np.asarray(a)) // b)


def visible_last_key(rows, spec: SeqSpec) -> np.ndarray:
    """vis(q): the last key index row q may attend to; keys 0..vis(q) are visible.

    Reading of [R, Per-row valid-split counts]: under causal and prefix-causal
    masking a row sees keys k <= q + prefix_offset, and in every mode no key
    past last_valid_kv_index.  Plain causal is top-left aligned (offset 0).
    A negative value means the row sees no key at all (fully masked row).
    """
    rows = np.asarray(rows, dtype=np.int64)
    lv = spec.last_valid_index
    if spec.mask == MASK_NONE:
        return np.full(rows.shape, lv, dtype=np.int64)
    return np.minimum(rows + spec.offset, lv)


def visible_first_key(rows, spec: SeqSpec) -> np.ndarray:
    """The first key index row q may attend to: q + offset - window_left with a
    window (see SeqSpec), else 0.  Keys below 0 do not exist, so values <= 0
    all mean "from the first key"."""
    rows = np.asarray(rows, dtype=np.int64)
    if spec.window_left < 0:
        return np.zeros(rows.shape, dtype=np.int64)
    return np.maximum(rows + spec.offset - spec.window_left, 0)


def visible_keys(rows, spec: SeqSpec, keys) -> np.ndarray:
    """Boolean [rows, keys]: key k is visible to row q iff
    visible_first_key(q) <= k <= visible_last_key(q)."""
    keys = np.asarray(keys, dtype=np.int64)
    lo = visible_first_key(rows, spec)
    hi = visible_last_key(rows, spec)
    return (keys[None, :] >= lo[:, None]) & (keys[None, :] <= hi[:, None])


def row_last(rows, spec: SeqSpec) -> np.ndarray:
    """rowLast = clamp(q + prefix_offset, 0, lastValid) [R].

    Reading: the lower clamp is applied last, max(0, min(q + off, lastValid)),
    so that an empty key range (lastValid = -1) still gives rowLast = 0 and a
    count of 1 instead of a division by zero.  With lastValid >= 0 both orders
    give the same value.  Non-causal rows all use lastValid.
    """
    return np.maximum(0, visible_last_key(rows, spec))


def keys_per_split(rl, spec: SeqSpec):
    """keysPerSplit = nPerBlock * ceil(ceil((rowLast + 1) / nPerBlock) / split_kv) [R]."""
    tiles = _ceil_div(np.asarray(rl) + 1, spec.n_per_block)
    return spec.n_per_block * _ceil_div(tiles, spec.split_kv)


def valid_split_counts(spec: SeqSpec, rows=None) -> np.ndarray:
    """Per-row valid-split counts [R, Per-row valid-split counts].

    count = ceil((rowLast + 1) / keysPerSplit), one value per query row.  Under
    no mask every row of the sequence has the same count (the pages' per
    batch-head count, broadcast over the rows).
    """
    rows = np.arange(spec.sq) if rows is None else np.asarray(rows)
    rl = row_last(rows, spec)
    return _ceil_div(rl + 1, keys_per_split(rl, spec)).astype(np.int64)


def block_split_ranges(spec: SeqSpec, m_per_block: int, block: int):
    """Key range [start, end) of every split for query block `block`.

    One partition serves every row of an M block: keysPerSplit is taken
    from the count formula at the block's final row, and split s then holds
    keys [s * kps, min((s + 1) * kps, rowLast + 1)) of that row's visible
    range [R, Per-row valid-split counts, the paragraph on conservative
    counts].  Reading: the final row is the last one that exists,
    min(start + mPB, sq) - 1.
    """
    last = min((block + 1) * m_per_block, spec.sq) - 1
    rl = int(row_last([last], spec)[0])
    kps = int(keys_per_split(rl, spec))
    return [(min(s * kps, rl + 1), min((s + 1) * kps, rl + 1)) for s in range(spec.split_kv)]


def _softmax_attention(Q, K, V, scale, visible):
    """Softmax attention of the rows of Q over the keys marked in `visible`.

    x = scale * Q K^T; LSE = ln sum_k exp(x_k); O = sum_k softmax(x)_k V_k,
    over the visible keys only.  A row with no visible key gives O = 0 and
    LSE = -inf (the empty-split / fully-masked convention [R, Summary]).
    The max subtraction only keeps exp() in range; it does not change the
    value in exact arithmetic.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    nq, dv = Q.shape[0], V.shape[1]
    O = np.zeros((nq, dv))
    lse = np.full(nq, -np.inf)
    if nq == 0 or K.shape[0] == 0:
        return O, lse
    x = scale * (Q @ K.T)
    x = np.where(visible, x, -np.inf)
    m = x.max(axis=1)
    has = np.isfinite(m)
    if not has.any():
        return O, lse
    e = np.exp(x[has] - m[has, None])
    z = e.sum(axis=1)
    O[has] = (e @ V) / z[:, None]
    lse[has] = m[has] + np.log(z)
    return O, lse


def unsplit(Q, K, V, scale, spec: SeqSpec, rows=None):
    """Plain softmax attention over each row's visible keys (no split at all).

    Q: [len(rows), Dqk] (the rows listed in `rows`, default all sq rows),
    K: [sk, Dqk], V: [sk, Dv].  Returns O [len(rows), Dv] and LSE [len(rows)]
    (natural log).  This is the result the split method must reproduce
    [R, Summary and NaN-safe merge: the merged output equals attention].
    """
    rows = np.arange(spec.sq) if rows is None else np.asarray(rows)
    visible = visible_keys(rows, spec, np.arange(spec.sk))
    return _softmax_attention(Q, K[: spec.sk], V[: spec.sk], scale, visible)


def unsplit_backward(Q, K, V, dO, scale, spec: SeqSpec):
    """Gradients dQ [sq, Dqk], dK [sk, Dqk], dV [sk, Dv] of the plain softmax
    attention of `unsplit` for the output gradient dO [sq, Dv] (f64).

    [A] leaves backward coverage of split-KV long-K attention open; the
    method's output is plain attention over the visible keys, so its gradient
    is that of attention: with P = softmax(x) over the visible keys,
        D_q = sum_v dO[q, v] O[q, v]
        dP  = dO V^T,   dS = P * (dP - D_q)
        dQ  = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO
    A row with no visible key has P = 0 and contributes nothing.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)[: spec.sk]
    V = np.asarray(V, dtype=np.float64)[: spec.sk]
    dO = np.asarray(dO, dtype=np.float64)
    rows = np.arange(spec.sq)
    visible = visible_keys(rows, spec, np.arange(spec.sk))
    x = scale * (Q @ K.T)
    x = np.where(visible, x, -np.inf)
    has = visible.any(axis=1)
    m = np.where(has, x.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(visible, np.exp(x - m[:, None]), 0.0)
    z = e.sum(axis=1)
    P = np.where(has[:, None], e / np.where(has, z, 1.0)[:, None], 0.0)
    O = P @ V
    D = (dO * O).sum(axis=1)
    dP = dO @ V.T
    dS = P * (dP - D[:, None])
    return scale * (dS @ K), scale * (dS.T @ Q), P.T @ dO


def sampled_backward(Q, K, V, dO, scale, spec: SeqSpec, rows, keys, chunk: int = 256):
    """dQ at query rows `rows` and dK, dV at key indices `keys` of
    `unsplit_backward`, for inputs whose whole score matrix does not fit in
    memory.  Each step of that definition is row-wise except the sums over
    rows that make dK and dV, so the rows are taken `chunk` at a time and those
    two sums are added up chunk by chunk (only the f64 summation order differs
    from `unsplit_backward`).  Q, dO: all sq rows; K, V: all sk keys."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)[: spec.sk]
    V = np.asarray(V, dtype=np.float64)[: spec.sk]
    dO = np.asarray(dO, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    dQ = np.zeros((len(rows), Q.shape[1]))
    dK = np.zeros((len(keys), Q.shape[1]))
    dV = np.zeros((len(keys), V.shape[1]))
    all_keys = np.arange(spec.sk)
    for c0 in range(0, spec.sq, chunk):
        cr = np.arange(c0, min(c0 + chunk, spec.sq))
        visible = visible_keys(cr, spec, all_keys)
        x = np.where(visible, scale * (Q[cr] @ K.T), -np.inf)
        has = visible.any(axis=1)
        m = np.where(has, x.max(axis=1, initial=-np.inf), 0.0)
        e = np.where(visible, np.exp(x - m[:, None]), 0.0)
        z = e.sum(axis=1)
        P = np.where(has[:, None], e / np.where(has, z, 1.0)[:, None], 0.0)
        O = P @ V
        D = (dO[cr] * O).sum(axis=1)
        dS = P * (dO[cr] @ V.T - D[:, None])
        dK += scale * (dS[:, keys].T @ Q[cr])
        dV += P[:, keys].T @ dO[cr]
        hit = (rows >= c0) & (rows < c0 + len(cr))
        if hit.any():
            dQ[hit] = scale * (dS[rows[hit] - c0] @ K)
    return dQ, dK, dV


def partials(Q, K, V, scale, spec: SeqSpec, m_per_block: int, rows=None):
    """Per-split partial outputs O_s [S, rows, Dv] and LSE L_s [S, rows].

    Each split is attention restricted to (split key range of the row's
    block) intersected with (keys the row may see).  An empty intersection
    gives O_s = 0 and L_s = -inf [R, Summary: empty splits write zero output
    and -inf LSE].  Reading: this also holds when the split is non-empty for
    the block but empty for this row.
    """
    rows = np.arange(spec.sq) if rows is None else np.asarray(rows)
    S = spec.split_kv
    Q = np.asarray(Q, dtype=np.float64)
    dv = V.shape[1]
    O = np.zeros((S, len(rows), dv))
    L = np.full((S, len(rows)), -np.inf)
    blocks = rows // m_per_block
    for j in np.unique(blocks):
        sel = np.nonzero(blocks == j)[0]
        for s, (a, b) in enumerate(block_split_ranges(spec, m_per_block, int(j))):
            if b <= a:
                continue
            visible = visible_keys(rows[sel], spec, np.arange(a, b))
            o, l = _softmax_attention(Q[sel], K[a:b], V[a:b], scale, visible)
            O[s, sel] = o
            L[s, sel] = l
    return O, L


def combine(O_s, L_s, counts):
    """NaN-safe merge of split partials [R, NaN-safe merge; Per-row mask layout].

    O_s [S, rows, Dv], L_s [S, rows], counts [rows].  Split s is valid for a
    row when s < count; invalid splits get LSE -inf and contribute zero.
        m   = max(max_s L_s, lowest finite)
        w_s = exp(L_s - m)
        O   = sum_s w_s O_s / max(sum_s w_s, 1)
    The merged LSE is not given on the pages.  Reading: m + ln(sum_s w_s),
    which equals ln sum_s exp(L_s), and -inf when every weight is 0.
    """
    O_s = np.asarray(O_s, dtype=np.float64)
    L_s = np.asarray(L_s, dtype=np.float64)
    S = L_s.shape[0]
    valid = np.arange(S)[:, None] < np.asarray(counts)[None, :]
    L = np.where(valid, L_s, -np.inf)
    m = np.maximum(L.max(axis=0), LOWEST_FINITE)
    w = np.where(valid, np.exp(L - m[None, :]), 0.0)
    num = np.where(valid[..., None], w[..., None] * O_s, 0.0).sum(axis=0)
    den = w.sum(axis=0)
    O = num / np.maximum(den, 1.0)[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(den > 0, m + np.log(den), -np.inf)
    return O, lse


def split_attention(Q, K, V, scale, spec: SeqSpec, m_per_block: int, rows=None):
    """The whole method for one (sequence, head): counts, partials, merge."""
    counts = valid_split_counts(spec, rows)
    O_s, L_s = partials(Q, K, V, scale, spec, m_per_block, rows)
    O, lse = combine(O_s, L_s, counts)
    return O, lse, counts, O_s, L_s


def visible_pairs(spec: SeqSpec) -> int:
    """Number of visible (query, key) pairs of one head: the algorithmic work unit."""
    rows = np.arange(spec.sq)
    vis = visible_last_key(rows, spec)
    first = visible_first_key(rows, spec)
    return int(np.clip(vis + 1 - first, 0, None).sum())


def kernel_nonempty_splits(spec: SeqSpec, m_per_block: int, row: int) -> int:
    """Number of splits of `row`'s block whose range holds a key the row sees."""
    vis = int(visible_last_key([row], spec)[0])
    first = int(visible_first_key([row], spec)[0])
    n = 0
    for a, b in block_split_ranges(spec, m_per_block, row // m_per_block):
        if b > a and a <= vis and b - 1 >= first:
            n += 1
    return n


def block_populated_splits(spec: SeqSpec, m_per_block: int, row: int) -> int:
    """Number of splits of `row`'s query block whose key range holds a key
    that exists (index <= lastValid).  These are the splits a kernel with
    real early exit still writes [R, the review note on real early exit: a
    workgroup with no work exits without writing, and the host side must then
    stop assuming those slots are initialised]; every other split of the
    block is (0, -inf) for all its rows, so a merge may leave it out.
    """
    lv = spec.last_valid_index
    n = 0
    for a, b in block_split_ranges(spec, m_per_block, row // m_per_block):
        if b > a and a <= lv:
            n += 1
    return n


__all__ = [
    "MASK_NONE",
    "MASK_CAUSAL",
    "MASK_PREFIX_CAUSAL",
    "LOWEST_FINITE",
    "SeqSpec",
    "visible_last_key",
    "visible_first_key",
    "visible_keys",
    "row_last",
    "keys_per_split",
    "valid_split_counts",
    "block_split_ranges",
    "unsplit",
    "unsplit_backward",
    "sampled_backward",
    "partials",
    "combine",
    "split_attention",
    "visible_pairs",
    "kernel_nonempty_splits",
    "block_populated_splits",
]
