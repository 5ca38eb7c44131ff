"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each pin checks one oracle function against mathematics or a hand derivation
(closed forms, error bounds, brute force, an independent formulation, a hand
simulated trace, invariants stated on the pages).  ``test_planted_mistakes``
then plants plausible slips in the oracle (its mutation switch, CPU only) and
asserts that some pin rejects every one of them.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24


def bf(x):
    return synth.f64_to_bf16(np.asarray(x, dtype=np.float64))


def f(x):
    return synth.bf16_to_f32(np.asarray(x, dtype=np.uint16)).astype(np.float64)


def rand_bf16(rng, *shape, scale=1.0):
    return bf(rng.standard_normal(shape) * scale)


# --------------------------------------------------------------------- score

def pin_score_error_bound():
    """Recursive-summation bound (Higham, Accuracy and Stability, Thm 4.4 /
    eq. 4.4): |fl(sum) - sum| <= gamma_{n-1} sum |x_i|, with exact products
    (bf16 x bf16 fits binary32) and n = 64 terms."""
    rng = np.random.default_rng(1)
    g = 63 * U32 / (1 - 63 * U32)
    for _ in range(300):
        q, k = rand_bf16(rng, 64), rand_bf16(rng, 64)
        exact = float(np.dot(f(q), f(k)))  # products and 64-term sum exact enough in fp64
        bound = g * float(np.sum(np.abs(f(q) * f(k))))
        s = oracle.score_one(q, k)
        assert abs(s - exact) <= bound + 1e-300, (s, exact, bound)


def pin_score_special_cases():
    z = np.zeros(64, dtype=np.uint16)
    rng = np.random.default_rng(2)
    k = rand_bf16(rng, 64)
    s = oracle.score_one(z, k)
    assert s == 0.0 and np.signbit(np.float32(s)) == False  # q = 0 -> +0
    # one-hot query picks the key component exactly
    for j in (0, 17, 63):
        e = np.zeros(64, dtype=np.uint16)
        e[j] = bf([1.0])[0]
        assert oracle.score_one(e, k) == float(f(k[j]))
    # negative zero products sum to +0
    kz = np.zeros(64, dtype=np.uint16)
    qn = rand_bf16(rng, 64)
    s = oracle.score_one(qn, kz | np.uint16(0x8000))
    assert s == 0.0 and not np.signbit(np.float32(s))


def pin_score_order():
    """Index-order binary32 accumulation from +0: with terms 2^24, 1, -2^24
    the running sum is 2^24, then 2^24 (1 is lost to round-half-even), then 0;
    any other order or a wider accumulator gives 1."""
    q = np.zeros(64, dtype=np.uint16)
    k = np.zeros(64, dtype=np.uint16)
    q[:3] = bf([1.0, 1.0, 1.0])
    k[:3] = bf([2.0 ** 24, 1.0, -(2.0 ** 24)])
    assert oracle.score_one(q, k) == 0.0
    # reversed placement: -2^24, 1, 2^24 -> -2^24, then -2^24+1 exact? no:
    # -2^24 + 1 = -16777215 is representable, + 2^24 = 1
    k2 = np.zeros(64, dtype=np.uint16)
    k2[:3] = bf([-(2.0 ** 24), 1.0, 2.0 ** 24])
    assert oracle.score_one(q, k2) == 1.0


def pin_ordered_key_monotone():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000),
                           [0.0, 1e-45, -1e-45, 3.4e38, -3.4e38, 1.0, -1.0]]).astype(np.float32)
    vals = np.unique(vals[np.isfinite(vals)])
    keys = np.array([oracle.ordered_key(float(v)) for v in vals], dtype=np.uint64)
    assert np.all(np.diff(keys.astype(np.int64)) > 0)
    assert oracle.ordered_key(0.0) == 0x80000000


# --------------------------------------------------------------------- top-k

def brute_topk_ok(scores, k, sel):
    """Set property of top-k by pairwise comparison (score desc, index asc)."""
    n = len(scores)
    kk = min(k, n)
    sel = list(sel)
    assert len(sel) == kk and len(set(sel)) == kk
    chosen = set(sel)
    for a in chosen:
        for b in range(n):
            if b in chosen:
                continue
            better = scores[a] > scores[b] or (scores[a] == scores[b] and a < b)
            assert better, (a, b, scores[a], scores[b])


def pin_topk_bruteforce():
    rng = np.random.default_rng(4)
    for trial in range(400):
        n = int(rng.integers(1, 14))
        pool = np.float32(rng.standard_normal(3))  # few distinct values -> many ties
        s = rng.choice(pool, n).astype(np.float32) if trial % 2 else rng.standard_normal(n).astype(np.float32)
        for k in (1, 2, 5, n, n + 3):
            brute_topk_ok(s, k, oracle.topk(s, k))


def pin_topk_all_equal():
    s = np.zeros(50, dtype=np.float32)
    assert list(oracle.topk(s, 7)) == list(range(7))


# --------------------------------------------------------------------- LRU

def pin_lru_golden_trace():
    g = json.load(open(os.path.join(GOLDEN, "lru_trace_s4.json")))
    st = oracle.LRUState(g["capacity"], g["hot_slots"])
    for step in g["steps"]:
        r = st.apply(step["selected"])
        assert r["hits"] == step["hits"]
        assert list(r["misses"]) == step["misses"]
        assert list(r["victims"]) == step["victims"]
        assert list(r["evict_old"]) == step["evict_old"]
    assert list(st.slot_token) == g["final_slot_token"]
    assert list(st.last_use) == g["final_last_use"]


class ListLRU:
    """Independent formulation: an explicit recency list of slots.  Slots
    touched this step (hits and refilled victims) move to the back in slot
    order; victims come from the front, skipping this step's hit slots.  The
    step number of each slot's last touch is kept only for comparison; the
    list order alone decides the victims."""

    def __init__(self, S):
        self.order = list(range(S))
        self.slot_of = {}
        self.owner = [-1] * S
        self.stamp = [-1] * S
        self.t = 0

    def apply(self, selected):
        U = sorted(set(int(x) for x in selected))
        hits = [u for u in U if u in self.slot_of]
        misses = [u for u in U if u not in self.slot_of]
        hit_slots = {self.slot_of[u] for u in hits}
        free = [s for s in self.order if s not in hit_slots]
        victims = free[:len(misses)]
        olds = []
        for m, v in zip(misses, victims):
            old = self.owner[v]
            olds.append(old)
            if old >= 0:
                del self.slot_of[old]
            self.slot_of[m] = v
            self.owner[v] = m
        touched = sorted(hit_slots | set(victims))
        self.order = [s for s in self.order if s not in set(touched)] + touched
        for s in touched:
            self.stamp[s] = self.t
        self.t += 1
        return misses, victims, olds, len(hits)


def pin_lru_matches_list_formulation():
    rng = np.random.default_rng(5)
    for trial in range(30):
        S = int(rng.integers(4, 40))
        k = int(rng.integers(1, S // 2 + 1))
        D = int(rng.integers(1, max(2, S // k) + 1))
        D = max(1, min(D, S // k))
        cap = int(rng.integers(k + 1, 4 * S + 2))
        st = oracle.LRUState(cap, S)
        ref = ListLRU(S)
        for t in range(25):
            sel = np.concatenate([rng.choice(min(cap, max(k, int(rng.integers(k, cap + 1)))), k, replace=False)
                                  for _ in range(D)])
            r = st.apply(sel)
            m, v, o, nh = ref.apply(sel)
            assert list(r["misses"]) == m and list(r["victims"]) == v and list(r["evict_old"]) == o
            assert r["hits"] == nh
            # reverse index and slot table are mutual inverses
            for s in range(S):
                if st.slot_token[s] >= 0:
                    assert st.cache_slots[st.slot_token[s]] == s
            assert int(np.sum(st.cache_slots >= 0)) == int(np.sum(st.slot_token >= 0))


# --------------------------------------------------------------------- attention

SCALE = float(np.float32(1.0 / 24.0))


def pin_attention_single_row():
    rng = np.random.default_rng(6)
    qa, row = rand_bf16(rng, 3, 576), rand_bf16(rng, 1, 576)
    out = oracle.attention(qa, row, SCALE)
    assert np.array_equal(out, np.broadcast_to(f(row[0, :512]), (3, 512)))


def pin_attention_uniform_mean():
    """Equal scores for every row -> the output is the mean of the V (first
    512) columns.  The query lives only in the rope columns, where all rows
    agree, while the latent columns differ."""
    rng = np.random.default_rng(7)
    rows = rand_bf16(rng, 9, 576)
    rows[:, 512:] = rows[0, 512:]
    qa = np.zeros((2, 576), dtype=np.uint16)
    qa[:, 512:] = rand_bf16(rng, 2, 64)
    out = oracle.attention(qa, rows, SCALE)
    mean = f(rows[:, :512]).mean(axis=0)
    assert np.allclose(out, mean[None, :], rtol=0, atol=1e-12)


def pin_attention_textbook():
    rng = np.random.default_rng(8)
    for n in (2, 5, 33):
        qa, rows = rand_bf16(rng, 4, 576, scale=2.0), rand_bf16(rng, n, 576)
        z = (f(qa) @ f(rows).T) * np.float64(np.float32(1.0 / 24.0))
        want = softmax(z, axis=1) @ f(rows[:, :512])
        out = oracle.attention(qa, rows, SCALE)
        assert np.allclose(out, want, rtol=1e-12, atol=1e-13)


def pin_attention_peaked():
    rng = np.random.default_rng(9)
    rows = rand_bf16(rng, 16, 576)
    qa = bf(f(rows[5:6]) * 40.0)  # q = c K_5, c large -> weight ~ 1 on row 5
    out = oracle.attention(qa, rows, SCALE)
    assert np.allclose(out[0], f(rows[5, :512]), atol=1e-6)


# --------------------------------------------------------------------- whole step

def small_workload(D=2, H=3, ctx=300, k=24, S=None, B=2, steps=12):
    S = S or D * k + 8
    return synth.Workload("pin", layers=1, batch=B, context=ctx, steps=steps, top_k=k,
                          hot_slots=S, positions=D, heads=H, seed=77)


def run_oracle(w, want_pool=False, queries=None):
    o = oracle.Oracle(w.layers, w.batch, w.capacity, w.top_k, w.hot_slots, w.positions,
                      w.heads, 1.0 / 24.0)
    for b in range(w.batch):
        o.append(0, b, w.index_rows(0, b, 0, w.context), w.kv_rows(0, b, 0, w.context))
    qs = [w.index_queries(0, b) for b in range(w.batch)] if queries is None else queries
    results = []
    for t in range(w.steps):
        before = [o.state(0, b) for b in range(w.batch)]
        for b in range(w.batch):
            o.append(0, b, w.index_rows(0, b, w.context + t, 1), w.kv_rows(0, b, w.context + t, 1))
        qi = np.stack([qs[b][t] for b in range(w.batch)])
        qa = np.stack([w.attn_queries(0, b, t) for b in range(w.batch)])
        r = o.decode_step(0, qi, qa, want_pool_out=want_pool)
        after = [o.state(0, b) for b in range(w.batch)]
        results.append((before, r, after))
    return o, results


def pin_step_invariants():
    w = small_workload()
    o, results = run_oracle(w, want_pool=True)
    pool = {b: w.kv_rows(0, b, 0, w.capacity) for b in range(w.batch)}
    for before, r, after in results:
        # offload changes where rows live, not the result
        assert np.array_equal(r["out"], r["out_pool"])
        for b in range(w.batch):
            cn = r["counts"][b]
            nU, nH, nM, nEv, kk = cn[:5]
            assert nU == nH + nM and nM <= w.positions * kk and nU >= kk
            cs0, cs1 = before[b]["cache_slots"], after[b]["cache_slots"]
            st1 = after[b]["slot_token"]
            for p in range(w.positions):
                W = r["topk"][b, p, :kk]
                tok = W & 0x7FFFFFFF
                assert len(set(tok.tolist())) == kk
                # packed flag says miss exactly when the token was absent
                assert np.array_equal(W < 0, cs0[tok] == -1)
                # remap after the update; every winner is resident
                assert np.array_equal(r["phys"][b, p, :kk], cs1[tok])
                assert np.all(cs1[tok] >= 0)
            # only misses move; their count equals the unique misses
            moved = r["misses"][b, :nM]
            assert np.all(cs0[moved] == -1) and len(set(moved.tolist())) == nM
            # hits need no fetch: their slots' rows are unchanged
            hit_slots = [cs0[t_] for t_ in np.unique(r["topk"][b, :, :kk] & 0x7FFFFFFF) if cs0[t_] >= 0]
            assert np.array_equal(before[b]["hot"][hit_slots], after[b]["hot"][hit_slots])
            # resident rows equal the pool rows; tables are mutual inverses
            res = np.nonzero(cs1 >= 0)[0]
            assert np.array_equal(after[b]["hot"][cs1[res]], pool[b][res])
            assert np.all(st1[cs1[res]] == res)
            assert int(np.sum(st1 >= 0)) == len(res) <= w.hot_slots
            assert nEv == int(np.sum(r["evict_old"][b, :nM] >= 0))


def pin_dedupe():
    """Identical queries at every position: the merged list equals one
    position's winners and the misses equal the single-position run."""
    w2 = small_workload(D=3, H=1, B=1, steps=6)
    w1 = w2.replace(positions=1)
    q1 = [w1.index_queries(0, 0)]
    q3 = [np.repeat(q1[0], 3, axis=1)]
    _, r3 = run_oracle(w2, queries=q3)
    _, r1 = run_oracle(w1.replace(hot_slots=w2.hot_slots), queries=q1)
    for (_, a, _), (_, b, _) in zip(r3, r1):
        assert a["counts"][0, 0] == w2.top_k
        assert a["counts"][0, 2] == b["counts"][0, 2]
        assert np.array_equal(a["misses"][0, :a["counts"][0, 2]], b["misses"][0, :b["counts"][0, 2]])


def replay_decode_steps(c8):
    """The whole decode step, replayed step by step from the pinned parts:
    every token's key is the ordered key of the per-row score (score_one, or
    the int8 pipeline of quantize_row / hadamard_rotate / c8_score) of the
    synthetic rows regenerated on their own, the winners are a full sort on
    (key desc, index asc), the flags are residency at step start, misses /
    victims / evicted owners / hits and the whole tables come from the
    recency-list formulation fed with that step's winners, the remap is its
    slot map, and the attention of every (seq, position) is the textbook
    softmax (numpy, fp64) over the pool rows of those winners."""
    w = small_workload(D=2, H=2, B=2, steps=10, ctx=180, k=20)
    o = oracle.Oracle(w.layers, w.batch, w.capacity, w.top_k, w.hot_slots, w.positions, w.heads,
                      1.0 / 24.0, indexer_c8=c8)
    lrus = [ListLRU(w.hot_slots) for _ in range(w.batch)]
    # sequence 0: i.i.d. rows; sequence 1 repeats its first 40 indexer rows,
    # so every step has tied scores across the top-k boundary
    idx = [w.index_rows(0, b, 0, w.capacity) for b in range(w.batch)]
    idx[1][40:] = idx[1][np.arange(40, w.capacity) % 40]
    kv = [w.kv_rows(0, b, 0, w.capacity) for b in range(w.batch)]
    for b in range(w.batch):
        o.append(0, b, idx[b][:w.context], kv[b][:w.context])
    qs = [w.index_queries(0, b) for b in range(w.batch)]
    scale = np.float64(np.float32(1.0 / 24.0))
    for t in range(w.steps):
        for b in range(w.batch):
            o.append(0, b, idx[b][w.context + t:w.context + t + 1], kv[b][w.context + t:w.context + t + 1])
        qi = np.stack([qs[b][t] for b in range(w.batch)])
        qa = np.stack([w.attn_queries(0, b, t) for b in range(w.batch)])
        r = o.decode_step(0, qi, qa, want_keys=True)
        for b in range(w.batch):
            n = w.context + t + 1
            kk = min(w.top_k, n)
            rows, pool = idx[b][:n], kv[b][:n]
            if c8:
                kq = [oracle.quantize_row(oracle.hadamard_rotate(rows[i])) for i in range(n)]
            sel_all, lru = [], lrus[b]
            for p in range(w.positions):
                if c8:
                    q8, sq = oracle.quantize_row(oracle.hadamard_rotate(qi[b, p]))
                    sc = [oracle.c8_score(q8, sq, kq[i][0], kq[i][1]) for i in range(n)]
                else:
                    sc = [oracle.score_one(qi[b, p], rows[i]) for i in range(n)]
                keys = np.array([oracle.ordered_key(v) for v in sc], np.uint32)
                assert np.array_equal(r["keys"][b, p, :n], keys), (t, b, p)
                order = sorted(range(n), key=lambda i: (-int(keys[i]), i))[:kk]
                W = r["topk"][b, p, :kk]
                assert (W & 0x7FFFFFFF).tolist() == order, (t, b, p)
                assert [bool(x < 0) for x in W] == [i not in lru.slot_of for i in order], (t, b, p)
                sel_all += order
            nU = len(set(sel_all))
            m, v, old, nh = lru.apply(sel_all)
            nM = len(m)
            assert r["counts"][b, :5].tolist() == [nU, nh, nM, sum(x >= 0 for x in old), kk], (t, b)
            assert r["misses"][b, :nM].tolist() == m and r["victims"][b, :nM].tolist() == v
            assert r["evict_old"][b, :nM].tolist() == old
            st = o.state(0, b)
            cs = np.full(w.capacity, -1, np.int32)
            for tok, slot in lru.slot_of.items():
                cs[tok] = slot
            assert np.array_equal(st["cache_slots"], cs) and st["slot_token"].tolist() == lru.owner
            assert st["last_use"].tolist() == lru.stamp
            for p in range(w.positions):
                toks = (r["topk"][b, p, :kk] & 0x7FFFFFFF)
                assert r["phys"][b, p, :kk].tolist() == [lru.slot_of[int(x)] for x in toks]
                z = (f(qa[b, p]) @ f(pool[toks]).T) * scale
                want = softmax(z, axis=1) @ f(pool[toks, :512])
                assert np.allclose(r["out"][b, p], want, rtol=1e-11, atol=1e-13), (t, b, p)
    o.close()


def pin_bf16_decode_replay():
    replay_decode_steps(False)


def pin_c8_decode_replay():
    replay_decode_steps(True)


# ------------------------------------------------- int8 indexer (LIM C8)

def sylvester(n):
    """Sylvester's construction: H_1 = [1], H_2m = [[H, H], [H, -H]]."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def pin_f16_conversion():
    """binary32 -> binary16 round-to-nearest-even and back, against numpy's
    IEEE half conversion, over random magnitudes and the edge cases
    (largest finite, overflow to inf, subnormals, ties)."""
    rng = np.random.default_rng(21)
    xs = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 6, 3000),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 7e4, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 5 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2048.0 + 1.0, 2048.0 + 3.0])])
    for x in xs.astype(np.float32):
        with np.errstate(over="ignore"):  # overflow to inf is one of the cases
            want = int(np.array([x], dtype=np.float32).astype(np.float16).view(np.uint16)[0])
        assert oracle.f32_to_f16(float(x)) == want, (float(x), hex(want))
    for h in range(0, 0x10000, 7):
        v = np.array([h], dtype=np.uint16).view(np.float16).astype(np.float32)[0]
        if np.isnan(v):
            continue
        assert oracle.f16_to_f32(h) == v, hex(h)


def pin_hadamard_closed_form():
    """Unit vectors give the columns of H/8 (H from Sylvester's recursion),
    and the rotation is an involution on exactly representable rows
    ((H/8)^2 = I)."""
    H = sylvester(64)
    for j in (0, 1, 5, 33, 63):
        e = np.zeros(64, dtype=np.uint16)
        e[j] = bf([1.0])[0]
        assert np.array_equal(oracle.hadamard_rotate(e).astype(np.float64), H[:, j] / 8.0), j
    rng = np.random.default_rng(22)
    for _ in range(20):
        x = rng.integers(-4, 5, 64).astype(np.float64)
        y = oracle.hadamard_rotate(bf(x)).astype(np.float64)
        assert np.array_equal(y, H @ x / 8.0)
        assert np.array_equal(oracle.hadamard_rotate(bf(y)).astype(np.float64), x)


def pin_hadamard_error_bound():
    """Random rows: within the recursive-summation bound of (H/8) x in fp64
    (64 exact terms), and the norm is kept (orthonormal rotation)."""
    H = sylvester(64)
    rng = np.random.default_rng(23)
    g = 63 * U32 / (1 - 63 * U32)
    for _ in range(200):
        x = rand_bf16(rng, 64)
        y = oracle.hadamard_rotate(x).astype(np.float64)
        exact = H @ f(x) / 8.0
        assert np.all(np.abs(y - exact) <= g * np.sum(np.abs(f(x))) / 8.0 + 1e-300)
        assert abs(np.linalg.norm(y) - np.linalg.norm(f(x))) <= 1e-5 * np.linalg.norm(f(x)) + 1e-30


def pin_quantize_row():
    """Codes are round-to-nearest-even of x / s with s = max|x| / 127: the
    largest entry maps to +-127, every code is within half a step, ties go to
    the even code, the stored scale is s in binary16, a zero row gives zeros."""
    rng = np.random.default_rng(24)
    for _ in range(300):
        x = (rng.standard_normal(64) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
        codes, sc = oracle.quantize_row(x)
        a = np.float32(np.max(np.abs(x)))
        s = np.float32(a / np.float32(127.0))
        assert np.all(np.abs(codes.astype(np.int32)) <= 127)
        assert abs(int(codes[np.argmax(np.abs(x))])) == 127
        err = np.abs(x.astype(np.float64) / float(s) - codes.astype(np.float64))
        assert np.all(err <= 0.5 + 1e-6), err.max()
        assert sc == int(np.array([s], np.float32).astype(np.float16).view(np.uint16)[0])
    codes, sc = oracle.quantize_row(np.zeros(64, np.float32))
    assert np.all(codes == 0) and sc == 0
    # exact ties: a = 127 gives s = 1
    x = np.zeros(64, np.float32)
    x[:6] = [127.0, 2.5, 3.5, -2.5, -3.5, 0.5]
    codes, sc = oracle.quantize_row(x)
    assert codes[:6].tolist() == [127, 2, 4, -2, -4, 0] and sc == 0x3C00


def c8_pipeline(q, k):
    q8, sq = oracle.quantize_row(oracle.hadamard_rotate(q))
    k8, sk = oracle.quantize_row(oracle.hadamard_rotate(k))
    return q8, sq, k8, sk


def pin_c8_score_bound():
    """The int8 score approximates q . k (the rotation is orthonormal), with
    error at most the dequantization error of both rows: per element at most
    s / 2 plus 127 |s - fp16(s)|, summed against the other row's entries."""
    rng = np.random.default_rng(25)
    H = sylvester(64)
    for _ in range(300):
        q, k = rand_bf16(rng, 64), rand_bf16(rng, 64)
        q8, sq, k8, sk = c8_pipeline(q, k)
        score = oracle.c8_score(q8, sq, k8, sk)
        exact = float(np.dot(f(q), f(k)))
        qr, kr = H @ f(q) / 8.0, H @ f(k) / 8.0
        sq32 = float(np.max(np.abs(qr))) / 127.0
        sk32 = float(np.max(np.abs(kr))) / 127.0
        eq = sq32 / 2 + 127 * sq32 * 2.0 ** -11 + 1e-6 * sq32
        ek = sk32 / 2 + 127 * sk32 * 2.0 ** -11 + 1e-6 * sk32
        bound = np.sum(np.abs(qr) * ek + np.abs(kr) * eq + eq * ek)
        assert abs(score - exact) <= bound + 1e-6 * abs(exact), (score, exact, bound)
    # the integer dot is exact: a zero key scores +0, a scaled copy scales
    z = np.zeros(64, np.int8)
    s0 = oracle.c8_score(np.full(64, 3, np.int8), 0x3C00, z, 0x3C00)
    assert s0 == 0.0 and not np.signbit(np.float32(s0))
    assert oracle.c8_score(np.full(64, 127, np.int8), 0x3C00, np.full(64, -127, np.int8), 0x3800) == \
        np.float32(-64 * 127 * 127 * 0.5)


def pin_c8_decode_consistent():
    """The oracle's int8 decode stores the rotated, quantized rows on append,
    quantizes the rotated query, and ranks by the int8 score of the pinned
    functions (keys compared for every token, winners by brute force)."""
    w = small_workload(D=2, B=2, steps=3)
    o = oracle.Oracle(w.layers, w.batch, w.capacity, w.top_k, w.hot_slots, w.positions, w.heads,
                      1.0 / 24.0, indexer_c8=True)
    for b in range(w.batch):
        o.append(0, b, w.index_rows(0, b, 0, w.context), w.kv_rows(0, b, 0, w.context))
    for t in range(3):
        for b in range(w.batch):
            o.append(0, b, w.index_rows(0, b, w.context + t, 1), w.kv_rows(0, b, w.context + t, 1))
        qi = np.stack([w.index_queries(0, b)[t] for b in range(w.batch)])
        qa = np.stack([w.attn_queries(0, b, t) for b in range(w.batch)])
        r = o.decode_step(0, qi, qa, want_keys=True, want_out=False)
        for b in range(w.batch):
            codes, scales = o.indexer_c8(0, b)
            n = w.context + t + 1
            rows = w.index_rows(0, b, 0, n)
            for i in range(0, n, 37):
                c_i, s_i = oracle.quantize_row(oracle.hadamard_rotate(rows[i]))
                assert np.array_equal(codes[i], c_i) and scales[i] == s_i
            for p in range(w.positions):
                q8, sq = oracle.quantize_row(oracle.hadamard_rotate(qi[b, p]))
                sc = np.array([oracle.c8_score(q8, sq, codes[i], scales[i]) for i in range(n)], np.float32)
                keys = np.array([oracle.ordered_key(v) for v in sc], np.uint32)
                assert np.array_equal(r["keys"][b, p, :n], keys)
                order = sorted(range(n), key=lambda i: (-int(keys[i]), i))[:min(w.top_k, n)]
                assert (r["topk"][b, p, :len(order)] & 0x7FFFFFFF).tolist() == order
    o.close()


PINS = [pin_score_error_bound, pin_score_special_cases, pin_score_order, pin_ordered_key_monotone,
        pin_topk_bruteforce, pin_topk_all_equal, pin_lru_golden_trace,
        pin_lru_matches_list_formulation, pin_attention_single_row, pin_attention_uniform_mean,
        pin_attention_textbook, pin_attention_peaked, pin_step_invariants, pin_dedupe,
        pin_f16_conversion, pin_hadamard_closed_form, pin_hadamard_error_bound, pin_quantize_row,
        pin_c8_score_bound, pin_c8_decode_consistent, pin_bf16_decode_replay, pin_c8_decode_replay]

# Slips that the whole-step replay must reject by itself.  It recomputes the
# step from the part functions (score, ordered key, the int8 pipeline), so
# slips inside those are left to their own pins; everything the step adds on
# top (which rows it scores, the order of winners, dedupe, flags, victim
# order, the miss <-> victim pairing, stamps, evictions, remap, attention
# wiring) is covered here.
MUST_CATCH = {
    "append_offset": "pin_bf16_decode_replay",
    "step_victim_slot_desc": "pin_bf16_decode_replay",
    "step_miss_desc": "pin_bf16_decode_replay",
    "victim_slot_desc": "pin_bf16_decode_replay",
    "victim_ignore_stamp": "pin_bf16_decode_replay",
    "hits_not_stamped": "pin_bf16_decode_replay",
    "evict_keeps_old": "pin_bf16_decode_replay",
    "no_dedupe": "pin_bf16_decode_replay",
    "flag_inverted": "pin_bf16_decode_replay",
    "tie_larger_index": "pin_bf16_decode_replay",
    "scale_512": "pin_bf16_decode_replay",
    "v_wrong_slice": "pin_bf16_decode_replay",
    "c8_query_not_rotated": "pin_c8_decode_replay",
}


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    oracle.set_mutation(0)
    pin()


@pytest.mark.parametrize("mutation", sorted(oracle.MUTATIONS))
def test_planted_mistakes(mutation):
    """Every planted slip in the oracle must be rejected by at least one pin."""
    oracle.set_mutation(mutation)
    try:
        caught = []
        for pin in PINS:
            try:
                pin()
            except (AssertionError, RuntimeError):
                caught.append(pin.__name__)
        assert caught, f"no pin rejects mutation {mutation}"
        if mutation in MUST_CATCH:
            assert MUST_CATCH[mutation] in caught, (mutation, caught)
    finally:
        oracle.set_mutation(0)
