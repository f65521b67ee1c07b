"""GPU checks of the HBM row cache over K/V rows in pinned host memory
(qsa_row_cache_step + qsa_sparse_decode_cached; "125B MoE を 3090 3 枚で運用する vLLM 最適化編",
section 5).

A hit reads the same bytes the host holds and the arithmetic is unchanged,
so the cached decode must equal qsa_sparse_decode on the same inputs bit for
bit. Checked over several steps whose selections overlap (as consecutive
decode steps do), with rows appended, rows rewritten in place and dropped,
slot collisions in a tiny cache, several queries of one sequence in one
launch, and split counts 1..8. With a cache of one slot per row (no
collisions) every miss is kept, so the hits are exactly the list positions
whose row was read in an earlier step and not dropped since: that set is
computed on the host and compared. Every plan entry is checked for validity
(a miss names its token, a hit names the row's slot), one step is compared
with the oracle, and a row rewritten without being dropped is shown to come
from the cache (the pages' consistency rule made visible). The cache step and
the cached decode are also replayed from a HIP graph, each replay equal to the
uncached decode while the cache fills.
"""
import numpy as np
import pytest
import torch

import qsa_inputs as qi
from oracle import qsa_oracle as orc
from tests import qsa_cases as qc

pytestmark = pytest.mark.gpu

BLOCK, TOPK, HKV, D = 4, 512, 2, 256


@pytest.fixture(scope="module")
def pkg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import indexer_selected_sparse_pooled_amd as p
    p.qsa.lib()  # fails loudly if the library is missing
    return p


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


def _pinned(bits_arr):
    t = torch.empty(bits_arr.shape, dtype=torch.bfloat16, pin_memory=True)
    t.view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(bits_arr).view(np.int16)))
    return t


def _set_row(host, arr, s, pos, bits_row):
    """Write one token's [hkv, d] row into the pinned tensor and its numpy copy."""
    arr[s, pos] = bits_row
    host[s, pos].view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(bits_row).view(np.int16)))


def _next_sel(rng, prev, nblk, keep):
    """A selection of min(topk, nblk) blocks that keeps about `keep` of prev."""
    n = min(TOPK, nblk)
    if n == nblk:
        return np.arange(nblk, dtype=np.int64)
    kept = np.empty(0, dtype=np.int64) if prev is None else prev[(rng.random(prev.size) < keep) & (prev < nblk)]
    kept = kept[:n]
    pool = np.setdiff1d(np.arange(nblk), kept)
    new = rng.choice(pool, n - kept.size, replace=False)
    return np.sort(np.concatenate([kept, new])).astype(np.int64)


class Stepper:
    """nseq sequences in pinned host memory, nq decode queries (q_seq) per
    step, one row cache; each step runs the uncached and the cached decode."""

    def __init__(self, pkg, seed, ctxs, q_seq, n_slots, n_split, steps):
        self.pkg, self.seed = pkg, seed
        self.ctxs = list(ctxs)
        self.nseq = len(ctxs)
        self.q_seq = list(q_seq)
        self.nq = len(q_seq)
        self.cap = (max(ctxs) + steps + 8 + 7) // 8 * 8
        case = qc.DecodeCase(seed, ctxs, cap=self.cap)
        self.k, self.v = case.k.copy(), case.v.copy()
        self.q = case.q[self.q_seq]
        self.k_host, self.v_host = _pinned(self.k), _pinned(self.v)
        self.kv = pkg.make_kv(self.k_host, self.v_host)
        self.n_slots, self.n_split = n_slots, n_split
        self.cache = pkg.row_cache_empty(pkg.ATTN_A, n_slots)
        self.src_ld = TOPK * BLOCK + BLOCK - 1
        assert pkg.qsa_decode_cached_plan_bytes(pkg.SEL_A, self.nq) == self.nq * self.src_ld * 4
        self.plan = torch.empty(self.nq, self.src_ld, dtype=torch.int32, device="cuda")
        self.q_dev = qc.to_dev(self.q)
        self.rng = np.random.default_rng(seed)
        self.sels = [None] * self.nq
        self.cached = set()  # keys held by a collision-free cache
        self.t = 0

    def fresh_row(self, tag):
        S = qi.stream_id(0, 1000 + self.t, "k", salt=7)
        return qc.bits(self.seed + tag, S, (HKV, D))

    def store(self, s, pos):
        """Store a new row at (s, pos) (K and V new bytes)."""
        _set_row(self.k_host, self.k, s, pos, self.fresh_row(2 * (s * 100003 + pos)))
        _set_row(self.v_host, self.v, s, pos, self.fresh_row(2 * (s * 100003 + pos) + 1))

    def step(self, dropped, keep=0.72, same=False):
        """dropped: (seq, pos) pairs passed to qsa_row_cache_step. Returns
        (o_uncached, lse_uncached, o_cached, lse_cached, plan, token lists)."""
        pkg = self.pkg
        torch.cuda.synchronize()
        rs = qc.i32([s for s, _ in dropped]) if dropped else None
        rp = qc.i32([p for _, p in dropped]) if dropped else None
        pkg.qsa_row_cache_step(pkg.ATTN_A, self.cache, self.n_slots, rp, self.kv, row_seq=rs)
        for s, p in dropped:
            self.cached.discard(s * self.cap + p)
        ctxs = [self.ctxs[s] for s in self.q_seq]
        if not same:
            self.sels = [_next_sel(self.rng, self.sels[i], ctxs[i] // BLOCK, keep) for i in range(self.nq)]
        sel = torch.full((self.nq, TOPK), -1, dtype=torch.int32, device="cuda")
        n_sel = torch.zeros(self.nq, dtype=torch.int32, device="cuda")
        for i, s in enumerate(self.sels):
            sel[i, :len(s)] = torch.tensor(s.astype(np.int32))
            n_sel[i] = len(s)
        q_ctx, q_seq = qc.i32(ctxs), qc.i32(self.q_seq)
        max_ctx = self.cap
        outs = []
        for cached in (False, True):
            o = torch.full((self.n_split, self.nq, 16, D), float("nan"), device="cuda")
            lse = torch.full((self.n_split, self.nq, 16), float("nan"), device="cuda")
            if cached:
                self.plan.fill_(0x7FFF0000)
                pkg.qsa_sparse_decode_cached(pkg.SEL_A, pkg.ATTN_A, q_ctx, max_ctx, self.q_dev, self.kv, sel, n_sel,
                                             self.n_split, o, lse, self.cache, self.n_slots, self.plan, q_seq=q_seq)
            else:
                pkg.qsa_sparse_decode(pkg.SEL_A, pkg.ATTN_A, q_ctx, max_ctx, self.q_dev, self.kv, sel, n_sel,
                                      self.n_split, o, lse, q_seq=q_seq)
            outs += [o, lse]
        torch.cuda.synchronize()
        lists = [orc.selected_tokens(self.sels[i], ctxs[i], BLOCK) for i in range(self.nq)]
        self.t += 1
        return (*outs, self.plan.cpu().numpy(), lists)

    def check_plan(self, plan, lists, exact_hits):
        """Every entry valid; with a collision-free cache the hits exactly
        those predicted. Returns (hits, positions)."""
        hits = tot = 0
        for i, toks in enumerate(lists):
            s = self.q_seq[i]
            e = plan[i, :len(toks)]
            keys = s * self.cap + toks
            miss = e >= 0
            assert np.array_equal(e[miss], toks[miss]), f"query {i}: a miss must name its token"
            assert np.array_equal(-e[~miss] - 1, keys[~miss] % self.n_slots), f"query {i}: a hit must name its slot"
            if exact_hits:
                want = np.array([int(k) in self.cached for k in keys], dtype=bool)
                assert np.array_equal(~miss, want), f"query {i}: hit set"
            hits += int((~miss).sum())
            tot += len(toks)
        if exact_hits:
            for i, toks in enumerate(lists):
                self.cached.update(int(k) for k in self.q_seq[i] * self.cap + toks)
        return hits, tot


def _equal(a, b):
    return torch.equal(a, b)


@pytest.mark.parametrize("n_slots_kind,n_split", [("one_per_row", 1), ("one_per_row", 8), ("tiny", 3), ("tiny", 1)])
def test_cached_decode_bit_identical_over_steps(pkg, n_slots_kind, n_split):
    ctxs = [9000, 12003, 2051, 0]
    steps = 6
    cap = (max(ctxs) + steps + 8 + 7) // 8 * 8
    n_slots = len(ctxs) * cap if n_slots_kind == "one_per_row" else 37
    _print_case("row_cache_steps", ctxs=ctxs, n_slots=n_slots, n_split=n_split)
    st = Stepper(pkg, 41, ctxs, range(len(ctxs)), n_slots, n_split, steps)
    exact = n_slots_kind == "one_per_row"
    rates = []
    for t in range(steps):
        dropped = []
        if t > 0:  # one appended row per sequence
            for s in range(st.nseq):
                st.store(s, st.ctxs[s])
                dropped.append((s, st.ctxs[s]))
                st.ctxs[s] += 1
        if t == 3:  # rows read earlier, rewritten in place
            for s, p in ((0, int(st.sels[0][0]) * BLOCK + 1), (1, int(st.sels[1][-1]) * BLOCK), (2, 7)):
                st.store(s, p)
                dropped.append((s, p))
        ou, lu, oc, lc, plan, lists = st.step(dropped)
        assert _equal(ou, oc) and _equal(lu, lc), f"step {t}: cached output differs"
        hits, tot = st.check_plan(plan, lists, exact)
        rates.append(hits / max(tot, 1))
    if exact:
        assert rates[0] == 0.0
        assert min(rates[1:]) > 0.6, rates  # about keep + the full-attention sequence
    print(f"[hit rates] {[round(r, 3) for r in rates]}", flush=True)


@pytest.mark.parametrize("n_slots", [None, 53])
def test_several_queries_of_one_sequence(pkg, n_slots):
    """Queries of one sequence in one launch read (and claim) the same rows."""
    ctxs = [7001, 4100]
    q_seq = [0, 1, 0, 0, 1]
    cap = (max(ctxs) + 4 + 8 + 7) // 8 * 8
    ns = n_slots or len(ctxs) * cap
    _print_case("row_cache_shared_rows", ctxs=ctxs, q_seq=q_seq, n_slots=ns)
    st = Stepper(pkg, 42, ctxs, q_seq, ns, 2, 4)
    for t in range(4):
        ou, lu, oc, lc, plan, lists = st.step([], keep=0.8)
        assert _equal(ou, oc) and _equal(lu, lc), f"step {t}"
        st.check_plan(plan, lists, n_slots is None)


def test_cached_step_matches_oracle(pkg):
    ctxs = [6003, 2051, 3]
    _print_case("row_cache_oracle", ctxs=ctxs)
    cap = (max(ctxs) + 2 + 8 + 7) // 8 * 8
    st = Stepper(pkg, 43, ctxs, range(3), 3 * cap, 1, 2)
    st.step([])
    _, _, oc, lc, plan, lists = st.step([], keep=0.5)
    assert (plan[0, :len(lists[0])] < 0).any()
    for i, toks in enumerate(lists):
        o_ref, lse_ref = orc.attend(st.q[i], st.k[i], st.v[i], toks, 1.0 / 16)
        qc.check_attention(oc[0, i].cpu().numpy(), lc[0, i].cpu().numpy(), o_ref, lse_ref)


def test_rewritten_row_not_dropped_is_served_from_cache(pkg):
    """A cached row rewritten on the host without being dropped keeps its old
    bytes in the cache (so the cached decode repeats the earlier result);
    once dropped, the cached decode sees the new bytes."""
    ctxs = [8000]
    _print_case("row_cache_stale_rule", ctxs=ctxs)
    cap = (max(ctxs) + 3 + 8 + 7) // 8 * 8
    st = Stepper(pkg, 44, ctxs, [0], cap, 1, 3)
    ou0, lu0, oc0, lc0, _, lists = st.step([])
    assert _equal(ou0, oc0)
    p = int(lists[0][100])
    st.store(0, p)
    ou1, lu1, oc1, lc1, plan, _ = st.step([], same=True)
    assert plan[0, 100] < 0, "the row must be a hit"
    assert not _equal(ou1, ou0), "the rewrite must change the uncached result"
    assert _equal(oc1, ou0) and _equal(lc1, lu0), "the cache must serve the bytes it holds"
    ou2, lu2, oc2, lc2, plan, _ = st.step([(0, p)], same=True)
    assert plan[0, 100] >= 0
    assert _equal(oc2, ou2) and _equal(lc2, lu2) and _equal(ou2, ou1)


def test_cache_reset_by_zero_fill(pkg):
    """Zero-filling the buffer drops every row (and restarts the epochs)."""
    ctxs = [5000, 3000]
    _print_case("row_cache_reset", ctxs=ctxs)
    cap = (max(ctxs) + 4 + 8 + 7) // 8 * 8
    st = Stepper(pkg, 45, ctxs, range(2), 2 * cap, 2, 4)
    st.step([])
    st.step([])
    st.cache.zero_()
    st.cached.clear()
    ou, lu, oc, lc, plan, lists = st.step([])
    assert _equal(ou, oc) and _equal(lu, lc)
    assert st.check_plan(plan, lists, True)[0] == 0
    ou, lu, oc, lc, plan, lists = st.step([])
    assert _equal(ou, oc) and _equal(lu, lc)
    assert st.check_plan(plan, lists, True)[0] > 0


def test_cached_decode_argument_errors(pkg):
    st_cap = 4096
    k = torch.zeros(1, st_cap, HKV, D, dtype=torch.bfloat16, device="cuda")
    kv = pkg.make_kv(k, k)
    cache = pkg.row_cache_empty(pkg.ATTN_A, 100)
    plan = torch.empty(1, TOPK * BLOCK + 3, dtype=torch.int32, device="cuda")
    q = torch.zeros(1, 16, D, dtype=torch.bfloat16, device="cuda")
    sel = torch.zeros(1, TOPK, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros(1, dtype=torch.int32, device="cuda")
    o = torch.empty(1, 1, 16, D, device="cuda")
    lse = torch.empty(1, 1, 16, device="cuda")
    args = (pkg.SEL_A, pkg.ATTN_A, qc.i32([100]), st_cap, q, kv, sel, n_sel, 1, o, lse)
    with pytest.raises(pkg.QsaError):  # cache smaller than its slot count needs
        pkg.qsa_sparse_decode_cached(*args, cache[:-1], 100, plan)
    with pytest.raises(pkg.QsaError):  # plan workspace too small
        pkg.qsa_sparse_decode_cached(*args, cache, 100, plan[:, :-1].contiguous())
    with pytest.raises(pkg.QsaError):
        pkg.qsa_row_cache_step(pkg.ATTN_A, cache, 0, qc.i32([1]), kv)
    torch.cuda.synchronize()


def test_cached_decode_graph_replays(pkg):
    """The cache step and the cached decode captured in one HIP graph and
    replayed (with eager work between replays): every replay equals the
    uncached decode, while the cache fills and then serves hits."""
    ctxs = [9000, 5003]
    _print_case("row_cache_graph", ctxs=ctxs)
    cap = (max(ctxs) + 8 + 7) // 8 * 8
    st = Stepper(pkg, 46, ctxs, range(2), 2 * cap, 4, 1)
    ou, lu, oc, lc, _, _ = st.step([])  # selections fixed from here on
    sel = torch.full((2, TOPK), -1, dtype=torch.int32, device="cuda")
    n_sel = torch.zeros(2, dtype=torch.int32, device="cuda")
    for i, s in enumerate(st.sels):
        sel[i, :len(s)] = torch.tensor(s.astype(np.int32))
        n_sel[i] = len(s)
    q_ctx, q_seq = qc.i32(ctxs), qc.i32([0, 1])
    stored = qc.i32([c - 1 for c in ctxs])
    o = torch.empty(4, 2, 16, D, device="cuda")
    lse = torch.empty(4, 2, 16, device="cuda")
    st.cache.zero_()
    torch.cuda.synchronize()

    def call():
        pkg.qsa_row_cache_step(pkg.ATTN_A, st.cache, st.n_slots, stored, st.kv, row_seq=q_seq)
        pkg.qsa_sparse_decode_cached(pkg.SEL_A, pkg.ATTN_A, q_ctx, st.cap, st.q_dev, st.kv, sel, n_sel, 4, o, lse,
                                     st.cache, st.n_slots, st.plan, q_seq=q_seq)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    hits = []
    for _ in range(4):
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ou) and torch.equal(lse, lu), "replay differs from the uncached decode"
        hits.append(int((st.plan[:, :TOPK * BLOCK] < 0).sum().item()))
    assert hits[0] == 0 and hits[1] > 0, hits
    del g
