"""Parity of the HIP path with the CPU oracle (MI355X).

Every comparison is bit-exact after canonical ordering by position: the set of
selected positions, their slots, and the -1 padding. The five workloads run at
full size under the planner's choice and under each forced path; seeded fuzz
cases cover ragged and empty rows, heavy ties, +-0 and -inf, page sizes,
shared and per-row tables, the candidate-overflow fallback, slot-only output
and unaligned score rows.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.fixture(scope="module")
def workloads():
    return {i: synth.make_config(i) for i in range(1, 6)}


CONFIG_CASES = [
    (1, "auto", {}), (1, "register", {}), (1, "single", {}), (1, "multi", {}), (1, "multi", {"wg_per_row": 4}),
    (2, "auto", {}), (2, "single", {}), (2, "multi", {"wg_per_row": 8}), (2, "multi", {"wg_per_row": 36}),
    # minimum chunks above half a tile: the chunks then exceed one tile
    (2, "auto", {"min_chunk": 32768}), (2, "auto", {"min_chunk": 20000}), (4, "auto", {"min_chunk": 30000}),
    (3, "auto", {}), (3, "single", {}), (3, "multi", {"cand_capacity": 64}),
    (4, "auto", {}), (4, "single", {}), (4, "multi", {}),
    (5, "auto", {}), (5, "single", {}),
]


@pytest.mark.parametrize("i,path,kw", CONFIG_CASES,
                         ids=[f"c{i}-{p}-{'-'.join(f'{k}{v}' for k, v in kw.items())}" for i, p, kw in CONFIG_CASES])
def test_config_parity(workloads, i, path, kw):
    w = workloads[i]
    _gpu.say(f"[parity] config {i} {w.name} path={path} {kw}")
    got = _gpu.run_gpu(w, path, **kw)
    _gpu.assert_matches_oracle(w, got, f"c{i} {path} {kw}")


def c5_half(w):
    """32 rows of each of C5's four tie groups (128 rows): the most rows a
    forced split can serve when the grid holds 256 workgroups."""
    rows = np.concatenate([np.arange(g * 64, g * 64 + 32) for g in range(4)])
    return synth.Workload(w.name + "_half", np.ascontiguousarray(w.scores[rows]), w.lengths[rows].copy(),
                          np.ascontiguousarray(w.block_table[rows]), w.bt_row_stride, w.page_size, w.k, w.seed)


@pytest.mark.parametrize("kw", [{}, {"cand_capacity": 512}], ids=["default", "cap512"])
def test_c5_forced_split(workloads, kw):
    w = c5_half(workloads[5])
    _gpu.say(f"[parity] c5 half forced multi {kw}")
    _gpu.assert_matches_oracle(w, _gpu.run_gpu(w, "multi", **kw), f"c5 half multi {kw}")


def test_forced_split_too_many_rows_is_unsupported():
    from sparse_attention_indexer_amd import topk
    with pytest.raises(topk.TopKError) as e:
        topk.TopK(2048, 4096, 100_000, force_path="multi")
    assert e.value.status == topk.TOPK_ERR_UNSUPPORTED


def test_config_invariants_independent_of_oracle(workloads):
    for i in (1, 2, 4):
        w = workloads[i]
        got = _gpu.run_gpu(w, "auto")
        _gpu.assert_invariants(w, got, label=f"c{i}")


FUZZ = []
for s in range(24):
    FUZZ.append(dict(seed=100 + s, rows=1 + (s * 7) % 13, max_len=[300, 2100, 5000, 17000, 40000][s % 5],
                     alphabet=[0, 3, 40, 0][s % 4], special=bool(s % 3 == 0), page_size=[64, 1, 16, 128, 48][s % 5],
                     shared_table=bool(s % 2), stride_pad=[0, 3, 8][s % 3],
                     path=["auto", "single", "multi", "auto"][s % 4]))


@pytest.mark.parametrize("case", FUZZ, ids=[f"fuzz{c['seed']}" for c in FUZZ])
def test_fuzz_parity(case):
    c = dict(case)
    path = c.pop("path")
    seed = c.pop("seed")
    w = synth.random_case(seed, **c)
    if path == "register" and w.max_len > 32768:
        path = "single"
    _gpu.say(f"[fuzz] seed {seed} rows {w.rows} max_len {w.max_len} k {w.k} ps {w.page_size} path {path}")
    got = _gpu.run_gpu(w, path, max_len=w.stride)
    _gpu.assert_matches_oracle(w, got, f"fuzz {seed}")
    _gpu.assert_invariants(w, got, label=f"fuzz {seed}")


@pytest.mark.parametrize("k", [1, 2, 63, 64, 65, 1000, 2047, 2048])
@pytest.mark.parametrize("path", ["auto", "multi"])
def test_k_values(k, path):
    w = synth.random_case(7 + k, rows=5, max_len=30000, alphabet=50, k=k, exact_len=True)
    _gpu.say(f"[k] k {k} path {path}")
    got = _gpu.run_gpu(w, path)
    _gpu.assert_matches_oracle(w, got, f"k {k}")


def test_register_path_exact_tile():
    w = synth.random_case(5, rows=3, max_len=32768, alphabet=9, k=2048, exact_len=True)
    _gpu.assert_matches_oracle(w, _gpu.run_gpu(w, "register"), "register 32768")


@pytest.mark.parametrize("cap", [1, 8, 300])
def test_candidate_overflow_fallback(cap):
    w = synth.random_case(31, rows=4, max_len=60000, alphabet=5, k=1500, exact_len=True)
    _gpu.say(f"[overflow] cap {cap}")
    got = _gpu.run_gpu(w, "multi", cand_capacity=cap)
    _gpu.assert_matches_oracle(w, got, f"cap {cap}")


def test_slots_only_output(workloads):
    w = workloads[2]
    got = _gpu.run_gpu(w, "auto", with_idx=False)
    _gpu.assert_matches_oracle(w, got, "slots only")


def test_unaligned_scores():
    w = synth.random_case(41, rows=6, max_len=25000, stride_pad=1, alphabet=30, k=900)
    got = _gpu.run_gpu(w, "multi", scores_offset=1, max_len=w.stride)
    _gpu.assert_matches_oracle(w, got, "unaligned")
    got = _gpu.run_gpu(w, "single", scores_offset=1, max_len=w.stride)
    _gpu.assert_matches_oracle(w, got, "unaligned single")


def test_repeated_calls_reuse_plan_and_workspace(workloads):
    w = workloads[3]
    outs = _gpu.run_gpu(w, "auto", repeat=3)
    for got in outs:
        _gpu.assert_matches_oracle(w, got, "repeat")


def test_empty_and_tiny_rows():
    st = synth.Stream(77)
    lengths = np.array([0, 1, 2, 2048, 2049, 0, 5000], np.int32)
    stride = 5000
    scores = synth._f32(st.normal(7 * stride)).reshape(7, stride)
    bt = synth.page_permutation_tables(st, 7, (stride + 63) // 64)
    w = synth.Workload("tiny", scores, lengths, bt, bt.shape[1], 64, 2048, 77)
    for path in ("auto", "single", "multi"):
        _gpu.assert_matches_oracle(w, _gpu.run_gpu(w, path), f"tiny {path}")


def test_debug_keys_match_fp16_definition():
    """Device bins equal the top 10 bits of the ordered key of numpy's FP16
    rounding (RNE) of each score, with -0 folded into +0; device FP32 keys
    order like the scores."""
    from sparse_attention_indexer_amd import topk
    st = synth.Stream(5)
    x = np.concatenate([
        synth._f32(st.normal(200_000) * np.exp(st.normal(200_000) * 4)),
        np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65520, -65520, 1e-8, -1e-8, 6e-8, 2.98e-8,
                  np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny, 1e-45, -1e-45], np.float32),
        np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32),
    ]).astype(np.float32)
    x = x[~np.isnan(x)]
    bins, keys = topk.topk_debug_keys(torch.from_numpy(x).cuda())
    bins = bins.cpu().numpy().view(np.uint32)
    keys = keys.cpu().numpy().view(np.uint32)
    h = x.astype(np.float16)
    h[h == 0] = np.float16(0.0)
    hb = h.view(np.uint16).astype(np.uint32)
    key16 = np.where(hb & 0x8000, (~hb) & 0xFFFF, hb | 0x8000)
    np.testing.assert_array_equal(bins, key16 >> 6)
    order = np.argsort(x, kind="stable")
    xs, ks = x[order], keys[order]
    assert (np.diff(ks.astype(np.int64))[np.diff(xs) > 0] > 0).all()
    assert (ks[1:][np.diff(xs) == 0] == ks[:-1][np.diff(xs) == 0]).all()


@pytest.mark.parametrize("rows,prefix,k", [(1500, 1800, 2048), (600, 20000, 1024)])
def test_many_ragged_rows(rows, prefix, k):
    """Prefill-like batches: row t of a causal block sees prefix + t positions.
    More rows than one planning pass handles (1,024) and than the grid holds."""
    st = synth.Stream(rows + prefix)
    lengths = (prefix + np.arange(rows)).astype(np.int32)
    stride = int(lengths.max()) + 4 - int(lengths.max()) % 4
    vals = synth._f32(st.normal(64))
    scores = vals[st.below(rows * stride, 64)].reshape(rows, stride)   # heavy ties
    pages = (stride + 63) // 64
    bt = synth.page_permutation_tables(st, 1, pages)
    w = synth.Workload(f"ragged{rows}", np.ascontiguousarray(scores), lengths, bt, 0, 64, k, 1)
    _gpu.say(f"[ragged] rows {rows} prefix {prefix} k {k}")
    _gpu.assert_matches_oracle(w, _gpu.run_gpu(w, "auto"), f"ragged {rows}")


def test_timed_entry_matches_and_times_the_kernel(workloads):
    """topk_select_paged_timed gives the untimed call's result, and its kernel
    events bracket a positive interval no longer than the stream's view."""
    from sparse_attention_indexer_amd import topk
    w = workloads[2]
    dev = torch.device("cuda:0")
    tk = topk.TopK(w.k, w.rows, w.max_len, device=dev)
    sc = torch.from_numpy(w.scores).to(dev)
    ln = torch.from_numpy(w.lengths).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    tk.plan(ln)
    s0, i0 = tk.select(sc, ln, bt, w.bt_row_stride, w.page_size)
    ks, ke, ss, se = (torch.cuda.Event(enable_timing=True) for _ in range(4))
    ss.record()
    s1, i1 = tk.select(sc, ln, bt, w.bt_row_stride, w.page_size, events=(ks, ke))
    se.record()
    torch.cuda.synchronize()
    assert tk.status() == 0
    # the order within a row is unspecified: compare each row's sorted entries
    assert torch.equal(s0.sort(dim=1).values, s1.sort(dim=1).values)
    assert torch.equal(i0.sort(dim=1).values, i1.sort(dim=1).values)
    _gpu.assert_matches_oracle(w, (i1.cpu().numpy(), s1.cpu().numpy()), "timed")
    kernel_ms, stream_ms = ks.elapsed_time(ke), ss.elapsed_time(se)
    _gpu.say(f"[timed] kernel {kernel_ms * 1e3:.1f} us, stream {stream_ms * 1e3:.1f} us")
    assert 0 < kernel_ms <= stream_ms * 1.01


def test_mixed_long_rows_stay_register_resident():
    """A batch whose row tile counts fit the grid: every chunk must fit one
    register tile (the library then leaves the streamed-item code out), with
    rows of very different lengths sharing the grid."""
    st = synth.Stream(91)
    lengths = np.array([1_000_000, 1_000_000, 40_000, 33_000, 2049, 0, 500_000], np.int32)
    stride = 1_000_000
    vals = synth._f32(st.normal(4096))
    scores = vals[st.below(7 * stride, 4096)].reshape(7, stride)   # ties everywhere
    bt = synth.page_permutation_tables(st, 1, stride // 64)
    w = synth.Workload("mixed_long", np.ascontiguousarray(scores), lengths, bt, 0, 64, 2048, 91)
    _gpu.say("[mixed] 7 rows up to 1M, lengths very uneven")
    _gpu.assert_matches_oracle(w, _gpu.run_gpu(w, "auto", max_len=stride), "mixed long rows")


@pytest.mark.parametrize("kind", ["sorted", "all_equal", "random"])
def test_split_rows_extreme_distributions(kind):
    """Rows split across workgroups whose chunks fit the register tile, under
    three score shapes: descending order (one chunk holds the whole top k),
    all-equal scores (every element sits in the threshold bin, resolved only
    by position) and random scores. Three calls in a row check that the
    per-row cross-workgroup state is reset after each call."""
    st = synth.Stream(300 + len(kind))
    rows, n = 5, 100_000
    if kind == "sorted":
        scores = -np.sort(-synth._f32(st.normal(rows * n)).reshape(rows, n), axis=1)
    elif kind == "all_equal":
        scores = np.repeat(synth._f32(st.normal(rows))[:, None], n, axis=1)
    else:
        scores = synth._f32(st.normal(rows * n)).reshape(rows, n)
    lengths = np.full(rows, n, np.int32)
    bt = synth.page_permutation_tables(st, rows, (n + 63) // 64)
    w = synth.Workload(f"split_{kind}", np.ascontiguousarray(scores, dtype=np.float32), lengths, bt,
                       bt.shape[1], 64, 2048, 300)
    _gpu.say(f"[split extreme] {kind}")
    for got in _gpu.run_gpu(w, "auto", repeat=3):
        _gpu.assert_matches_oracle(w, got, f"split {kind}")


@pytest.mark.parametrize("max_len,exact,alphabet", [
    (16_384, True, 0), (20_000, True, 0), (32_768, True, 97), (30_000, False, 0),   # whole rows
    (70_000, True, 0), (140_000, True, 11), (100_000, False, 0),                    # split rows
], ids=["16k", "20k", "32k-ties", "30k-ragged", "70k", "140k-ties", "100k-ragged"])
def test_guessed_tile_paths(max_len, exact, alphabet):
    """Batches planned in the kernel whose guessed first tile is at least half
    a tile long (its loads then overlap the planning) or shorter, whole and
    split rows, equal lengths (the guess holds) and ragged ones (it mostly
    does not), with junk past every valid prefix."""
    w = synth.random_case(700 + max_len % 997, 9, max_len, exact_len=exact, alphabet=alphabet)
    _gpu.say(f"[guess] 9 rows, max_len {max_len}, exact {exact}, alphabet {alphabet}")
    for got in _gpu.run_gpu(w, "auto", repeat=2):
        _gpu.assert_matches_oracle(w, got, f"guessed tile {max_len}")


@pytest.mark.parametrize("rows,max_len,exact", [
    (1, 90_000, True), (63, 40_000, False), (64, 40_000, True), (65, 40_000, True), (65, 40_000, False),
    (130, 12_000, False),
], ids=["1-row", "63-ragged", "64", "65", "65-ragged", "130-ragged"])
def test_in_kernel_plan_across_the_one_wave_boundary(rows, max_len, exact):
    """In-kernel planning reduces and scans the row lengths inside each wave
    while the batch has at most 64 rows, and across the workgroup's waves
    above that: both sides of the switch, with split rows (lengths beyond one
    register tile) and ragged lengths, must give the oracle's result."""
    w = synth.random_case(900 + rows, rows, max_len, exact_len=exact, alphabet=0)
    _gpu.say(f"[plan boundary] {rows} rows, max_len {max_len}, exact {exact}")
    for got in _gpu.run_gpu(w, "auto", repeat=2):
        _gpu.assert_matches_oracle(w, got, f"plan boundary {rows}")


@pytest.mark.parametrize("n", [0, 3, 4, 1_000_003, 7_000_000])
def test_stream_read_hook_reads_every_vector(n):
    """The read-ceiling hook reads each 16-byte vector of x exactly once: its
    partial sums add up to the sum of x's whole vectors (a tail of fewer than
    4 floats is not read)."""
    from sparse_attention_indexer_amd import topk
    g = torch.Generator(device="cuda:0").manual_seed(n)
    x = torch.rand(max(n, 1), generator=g, device="cuda:0")[:n]
    out = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    topk.topk_debug_stream_read(x, out)
    torch.cuda.synchronize()
    want = x[: n // 4 * 4].double().sum().item()
    assert abs(out.double().sum().item() - want) <= 1e-4 * max(1.0, want)


@pytest.mark.parametrize("rows,max_len", [(7, 80_000), (600, 6_000)], ids=["7x80k-in-kernel-plan", "600-rows-plan-kernel"])
def test_plan_and_select_replay_from_a_hip_graph(rows, max_len):
    """topk_plan + topk_select_paged captured once into a HIP graph and
    replayed four times, with new scores and lengths copied in eagerly (and a
    synchronisation) before each replay; every replay must match the oracle
    for its own inputs. 600 rows take the planning kernel, 7 rows plan inside
    the selection kernel (the split rows' per-row state must be left reset
    after each replay)."""
    from sparse_attention_indexer_amd import topk
    dev = torch.device("cuda:0")
    cases = [synth.random_case(900 + rows + i, rows, max_len, k=2048, exact_len=(i % 2 == 0)) for i in range(2)]
    tk = topk.TopK(2048, rows, max_len, device=dev)
    sc = torch.from_numpy(np.ascontiguousarray(cases[0].scores)).to(dev)
    ln = torch.from_numpy(cases[0].lengths).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(cases[0].block_table)).to(dev)
    slots = torch.empty((rows, 2048), dtype=torch.int32, device=dev)
    idx = torch.empty_like(slots)
    assert cases[0].bt_row_stride == cases[1].bt_row_stride and cases[0].block_table.shape == cases[1].block_table.shape
    # eager warm-up on the capture's buffers, then the capture
    tk.plan(ln)
    tk.select(sc, ln, bt, cases[0].bt_row_stride, cases[0].page_size, out_slots=slots, out_indices=idx)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tk.plan(ln)
        tk.select(sc, ln, bt, cases[0].bt_row_stride, cases[0].page_size, out_slots=slots, out_indices=idx)
    torch.cuda.synchronize()
    for rep in range(4):
        w = cases[rep % 2]
        sc.copy_(torch.from_numpy(np.ascontiguousarray(w.scores)))
        ln.copy_(torch.from_numpy(w.lengths))
        bt.copy_(torch.from_numpy(np.ascontiguousarray(w.block_table)))
        slots.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _gpu.say(f"[graph] rows {rows} replay {rep}")
        _gpu.assert_matches_oracle(w, (idx.cpu().numpy(), slots.cpu().numpy()), f"graph replay {rep}")
    assert tk.status() == 0


@pytest.fixture(scope="module")
def plan_split():
    return synth.make_plan_split()


def _plan_header_items(tk):
    """(num_items, num_multi_items, num_groups) from the plan the planning
    kernel wrote (64-byte header: magic, rows, items, split items, grid, k,
    groups, ...)."""
    h = tk.plan_buf[:16].cpu().numpy()
    assert h[0] == 0x31504B54, "the planning kernel wrote no plan"
    return int(h[2]), int(h[3]), int(h[6])


@pytest.mark.parametrize("kw", [{}, {"min_chunk": 8192}], ids=["default", "min_chunk8192"])
def test_plan_kernel_emits_split_rows(plan_split, kw):
    """600 rows, four of 300,000 positions: more rows than the selection
    kernel plans itself, so topk_plan's kernel writes the work list, and the
    long rows are split across workgroups by it (its split-row branch)."""
    from sparse_attention_indexer_amd import topk
    w = plan_split
    dev = torch.device("cuda:0")
    _gpu.say(f"[plan split] 600 rows, 4 x 300,000, {kw}")
    tk = topk.TopK(w.k, w.rows, w.max_len, device=dev, **kw)
    sc = torch.from_numpy(w.scores).to(dev)
    ln = torch.from_numpy(w.lengths).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    tk.plan(ln)
    slots, idx = tk.select(sc, ln, bt, w.bt_row_stride, w.page_size)
    torch.cuda.synchronize()
    assert tk.status() == 0
    n_items, n_multi, n_groups = _plan_header_items(tk)
    _gpu.say(f"[plan split] items {n_items}, split items {n_multi}, split rows {n_groups}")
    assert n_groups == 4 and n_multi >= 8 and n_items == n_multi + (w.rows - 4)
    _gpu.assert_matches_oracle(w, (idx.cpu().numpy(), slots.cpu().numpy()), f"plan split {kw}")


def test_plan_kernel_split_rows_replay_from_a_hip_graph():
    """topk_plan (planning kernel, split rows) + topk_select_paged captured
    into a HIP graph and replayed with two batches of different lengths copied
    in eagerly before each replay; every replay must match the oracle."""
    from sparse_attention_indexer_amd import topk
    dev = torch.device("cuda:0")
    cases = [synth.make_plan_split(seed=8 + i) for i in range(2)]
    w0 = cases[0]
    tk = topk.TopK(w0.k, w0.rows, w0.stride, device=dev)
    sc = torch.from_numpy(w0.scores).to(dev)
    ln = torch.from_numpy(w0.lengths).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(w0.block_table)).to(dev)
    slots = torch.empty((w0.rows, w0.k), dtype=torch.int32, device=dev)
    idx = torch.empty_like(slots)
    tk.plan(ln)
    tk.select(sc, ln, bt, w0.bt_row_stride, w0.page_size, out_slots=slots, out_indices=idx)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tk.plan(ln)
        tk.select(sc, ln, bt, w0.bt_row_stride, w0.page_size, out_slots=slots, out_indices=idx)
    torch.cuda.synchronize()
    for rep in range(4):
        w = cases[rep % 2]
        sc.copy_(torch.from_numpy(w.scores))
        ln.copy_(torch.from_numpy(w.lengths))
        bt.copy_(torch.from_numpy(np.ascontiguousarray(w.block_table)))
        slots.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _gpu.say(f"[graph plan split] replay {rep}")
        _gpu.assert_matches_oracle(w, (idx.cpu().numpy(), slots.cpu().numpy()), f"split graph replay {rep}")
    assert tk.status() == 0


def test_split_row_wait_gives_up_and_workspace_recovers():
    """The split-row wait's time-out path, forced from the host: with
    spin_limit -1 every workgroup of a split row gives up before its first
    poll. The kernel must end, report TOPK_DEVICE_SPIN_TIMEOUT, and after
    topk_workspace_init the same workspace must give the oracle's result."""
    from sparse_attention_indexer_amd import topk
    w = synth.random_case(61, rows=7, max_len=100_000, alphabet=0, k=2048, exact_len=True)
    dev = torch.device("cuda:0")
    tk = topk.TopK(w.k, w.rows, w.max_len, device=dev, spin_limit=-1)
    sc = torch.from_numpy(np.ascontiguousarray(w.scores)).to(dev)
    ln = torch.from_numpy(w.lengths).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    _gpu.say("[timeout] 7 x 100,000 split rows, spin_limit -1")
    tk.plan(ln)
    tk.select(sc, ln, bt, w.bt_row_stride, w.page_size)
    torch.cuda.synchronize()   # the kernel ended
    st = tk.status()
    assert st & topk.DEVICE_SPIN_TIMEOUT, f"status {st}: the forced time-out was not reported"
    assert st & ~topk.DEVICE_SPIN_TIMEOUT == 0, f"status {st}"
    # one poll at most: either every row's merge was complete at its first
    # poll or the time-out is reported; the kernel ends either way
    tk.cfg.spin_limit = 1
    topk.topk_workspace_init(tk.workspace)
    tk.select(sc, ln, bt, w.bt_row_stride, w.page_size)
    torch.cuda.synchronize()
    st = tk.status()
    assert st in (0, topk.DEVICE_SPIN_TIMEOUT), f"status {st}"
    _gpu.say(f"[timeout] spin_limit 1 -> status {st}")
    tk.cfg.spin_limit = 0
    topk.topk_workspace_init(tk.workspace)
    for rep in range(2):
        got = tk.select(sc, ln, bt, w.bt_row_stride, w.page_size)
        torch.cuda.synchronize()
        assert tk.status() == 0
        _gpu.assert_matches_oracle(w, (got[1].cpu().numpy(), got[0].cpu().numpy()), f"after re-init {rep}")


def test_prefill_4096_rows_full_size():
    """Ragged prefill top-k at full size: 4,096 causal rows of 80,000 + t
    positions (the planning kernel's regime), bit-exact against the oracle."""
    w = synth.make_prefill()
    _gpu.say(f"[prefill] {w.rows} rows x up to {w.max_len}")
    got = _gpu.run_gpu(w, "auto")
    _gpu.assert_matches_oracle(w, got, "prefill 4096x80k")


def _key16_bins(x: np.ndarray) -> np.ndarray:
    """Ordered 1,024-bin index of each score: numpy's FP16 rounding (RNE),
    -0 folded into +0, sign-magnitude bits flipped into unsigned order, top
    10 bits (the Figure 3 caption's key), written out here from the
    definition, independently of the kernel."""
    h = x.astype(np.float16)
    h[h == 0] = np.float16(0.0)
    hb = h.view(np.uint16).astype(np.uint32)
    key = np.where(hb & 0x8000, (~hb) & 0xFFFF, hb | 0x8000)
    return key >> 6


@pytest.mark.parametrize("case", ["c1", "c2", "c3", "c5_rows", "fuzz_special", "short_rows"])
def test_device_histogram_and_threshold_bin(workloads, case):
    """The kernel's coarse histogram equals a CPU histogram of the same keys
    (exact counts, summing to the row length), and its threshold bin is the
    bin of the oracle's k-th score, with above(b*) < k <= above(b*) + h[b*]."""
    from sparse_attention_indexer_amd import topk
    if case.startswith("c") and case != "c5_rows":
        w = workloads[int(case[1])]
    elif case == "c5_rows":
        w = c5_half(workloads[5])
    elif case == "fuzz_special":
        w = synth.random_case(505, rows=9, max_len=70_000, alphabet=0, special=True, k=1500)
    else:
        w = synth.random_case(506, rows=6, max_len=3000, alphabet=7, special=True, k=2048)
    _gpu.say(f"[hist] {case}: {w.rows} x {w.stride}")
    dev = torch.device("cuda:0")
    hist, thr = topk.topk_debug_histogram(torch.from_numpy(np.ascontiguousarray(w.scores)).to(dev),
                                          torch.from_numpy(w.lengths).to(dev), w.k)
    hist = hist.cpu().numpy().view(np.uint32).astype(np.int64)
    thr = thr.cpu().numpy().view(np.uint32).astype(np.int64)
    ref_idx, _ = oracle_sorted(w)
    # Ordered bins 15 (-inf) .. 1008 (+inf) hold every non-NaN score; the
    # others hold only NaN codes. The kernel counts a tile's NaN padding past
    # the row's end there and never scans them.
    lo, hi = 15, 1009
    for r in range(w.rows):
        n = int(w.lengths[r])
        want = np.bincount(_key16_bins(w.scores[r, :n]), minlength=1024)
        assert want[:lo].sum() == 0 and want[hi:].sum() == 0
        np.testing.assert_array_equal(hist[r, lo:hi], want[lo:hi], err_msg=f"{case} row {r}")
        assert hist[r, lo:hi].sum() == n
        if n <= w.k:
            assert thr[r, 0] == 0xFFFFFFFF
            continue
        b, above, cnt = thr[r]
        vk = w.scores[r, ref_idx[r, w.k - 1]]
        assert b == _key16_bins(np.array([vk], np.float32))[0], f"{case} row {r}"
        assert above == hist[r, b + 1:hi].sum() and cnt == hist[r, b]
        assert above < w.k <= above + cnt


def oracle_sorted(w):
    """The oracle's output in its own (score desc, position asc) order."""
    import oracle
    return oracle.topk_workload(w, threads=8)


def _large_bin_rows(kind: str, seed: int):
    """5 split rows of 40,000 scores whose threshold bin (k = 2048) holds
    between 4,097 and 12,288 candidates: the rows whose boundary is first
    narrowed by the fine FP32-key digit. Kinds place that bin where the
    digit frame is narrow (a cluster at 3.0), where one key repeats, and
    where it is widest: the -inf bin (finite values below -65520 round to
    -inf in FP16), the zero bin (+-0 and FP32 denormals) and the +inf bin."""
    st = synth.Stream(seed, 17)
    rows, n, k = 5, 40_000, 2048
    # The -inf bin is the lowest: only the 9,000 scores at and above it are valid there.
    valid = 9_000 if kind == "neg_inf_bin" else n
    scores = np.empty((rows, n), np.float32)
    for r in range(rows):
        row = synth._f32(st.normal(n) - 20.0)               # far below the boundary
        pos = st.permutation(valid)
        top, mid = pos[:1000], pos[1000:1000 + 8000]
        row[top] = synth._f32(st.normal(1000) + 50.0)        # above the boundary bin
        if kind == "cluster":
            row[mid] = synth._f32(3.0 + st.below(8000, 600) * 2.0 ** -22)
        elif kind == "big_tie_front":
            # as big_tie, all inside the first 16,384 positions: split over two
            # workgroups, one holds every candidate and more survivors than
            # its LDS staging takes
            front = pos[pos < 16_384]
            top, tie, rest = front[:500], front[500:5500], front[5500:12500]
            row[top] = synth._f32(st.normal(500) + 50.0)
            row[tie] = np.float32(7.375)
            row[rest] = synth._f32(7.375 - (1 + st.below(rest.size, 100_000)) * 2.0 ** -21)
        elif kind == "big_tie":
            # 12,000 in the bin [7.25, 7.5): 5,000 copies of the cut value
            # 7.375 (one fine digit holding the cut, too many to compact past
            # the list) and 7,000 distinct values just below it in the bin
            top = pos[:500]
            row[top] = synth._f32(st.normal(500) + 50.0)
            tie, rest = pos[500:5500], pos[5500:12500]
            row[tie] = np.float32(7.375)
            row[rest] = synth._f32(7.375 - (1 + st.below(7000, 100_000)) * 2.0 ** -21)
        elif kind == "split_vote":
            # The first quarter holds ten private bins of 200 scores each
            # (20 + 4 b), 2,000 in all; the rest holds 5,000 cluster scores at
            # 3.0, where the row's threshold lies. Chunks of the first quarter
            # may predict a private bin and the others the cluster bin: either
            # vote may decide the row, and a wrong one must fall back.
            row[top] = synth._f32(st.normal(1000) - 20.0)   # (no scores above the private bins)
            for b in range(10):
                blk = 1000 * b + st.permutation(1000)[:200]
                row[blk] = synth._f32(20.0 + 4.0 * b + st.uniform(200) * 0.01)
            zpos = 10_000 + st.permutation(n - 10_000)[:5000]
            row[zpos] = synth._f32(3.0 + st.below(5000, 600) * 2.0 ** -22)
        elif kind == "one_key":
            row[mid] = np.float32(7.25)
        elif kind == "neg_inf_bin":
            v = synth._f32(-1e30 * (1.0 + st.uniform(8000)))
            v[st.below(8000, 4) == 0] = -np.inf
            row[mid] = v
            row[valid:] = np.float32(1e30)                  # junk past the valid length
        elif kind == "zero_bin":
            v = synth._f32(st.uniform(8000) * 3.7e-6)
            sel = st.below(8000, 5)
            v[sel == 0] = np.float32(0.0)
            v[sel == 1] = np.float32(-0.0)
            v[sel == 2] = synth._f32(st.uniform(int((sel == 2).sum())) * 1e-39)   # FP32 denormals
            row[mid] = v
        elif kind == "pos_inf_bin":
            row[top] = synth._f32(st.normal(1000) + 30.0)
            v = synth._f32(65520.0 * (1.0 + st.uniform(8000)))
            v[st.below(8000, 8) == 0] = np.inf
            row[mid] = v
            row[top] = np.inf if r % 2 else row[top]
        scores[r] = row
    lengths = np.full(rows, valid, np.int32)
    bt = synth.page_permutation_tables(st, rows, (n + 63) // 64)
    return synth.Workload(f"large_bin_{kind}", scores, lengths, bt, bt.shape[1], 64, k, seed)


@pytest.mark.parametrize("kind", ["cluster", "one_key", "big_tie", "big_tie_front", "neg_inf_bin", "zero_bin",
                                  "pos_inf_bin", "split_vote"])
@pytest.mark.parametrize("path,kw", [("multi", {"wg_per_row": 2}), ("multi", {"wg_per_row": 8}),
                                     ("multi", {"wg_per_row": 36})], ids=["wg2", "wg8", "wg36"])
def test_split_row_large_threshold_bin(kind, path, kw):
    w = _large_bin_rows(kind, 440 + len(kind))
    _gpu.say(f"[large bin] {kind} {kw}")
    for got in _gpu.run_gpu(w, path, repeat=2, **kw):
        _gpu.assert_matches_oracle(w, got, f"large bin {kind} {kw}")


def _owned_large_bin_rows(kind: str, seed: int):
    """4 rows of 140,000 scores (250,000 for "sparse_extract") selected by one
    streamed workgroup each, whose threshold bin holds more candidates than
    the LDS list (16,384): counted by fine digit while classified, or, when
    they all hold one key, taken in position order."""
    st = synth.Stream(seed, 23)
    rows, k = 4, 2048
    n = 250_000 if kind == "sparse_extract" else 140_000
    scores = np.empty((rows, n), np.float32)
    for r in range(rows):
        row = synth._f32(st.normal(n) - 10.0)                 # far below the boundary
        pos = st.permutation(n)
        n_top = [0, 500, 1000, 2047][r]                      # row 3: one candidate needed
        row[pos[:n_top]] = synth._f32(st.normal(n_top) + 100.0)
        rest = pos[n_top:]
        if kind == "one_key_scattered":                      # 30,000 copies anywhere
            row[rest[:30_000]] = np.float32(5.0)
        elif kind == "one_key_late":                         # 20,000 copies, all past position 90,000
            late = rest[rest >= 90_000][:20_000]
            row[late] = np.float32(5.0)
        elif kind == "one_key_whole_row":                    # every other score is the key
            row[rest] = np.float32(5.0)
        elif kind == "hot_digit":                            # 18,000 copies of 5.0 and 1,500 just above
            row[rest[:18_000]] = np.float32(5.0)
            row[rest[18_000:19_500]] = synth._f32(5.0 + (1 + st.below(1500, 3000)) * 2.0 ** -20)
        elif kind == "one_bin_distinct":                     # 8,192 values of one FP16 bin, ~17 copies each
            row[rest] = synth._f32(1.0 + st.below(rest.size, 8192) * 2.0 ** -23)
        elif kind == "sparse_extract":                       # 20,000 of 250,000: re-binned, not re-read whole
            row[rest[:20_000]] = synth._f32(3.0 + st.below(20_000, 2000) * 2.0 ** -22)
        scores[r] = row
    lengths = np.full(rows, n, np.int32)
    bt = synth.page_permutation_tables(st, rows, (n + 63) // 64)
    return synth.Workload(f"owned_large_bin_{kind}", scores, lengths, bt, bt.shape[1], 64, k, seed)


@pytest.mark.parametrize("kind", ["one_key_scattered", "one_key_late", "one_key_whole_row", "hot_digit",
                                  "one_bin_distinct", "sparse_extract"])
@pytest.mark.parametrize("offset", [0, 1], ids=["aligned", "unaligned"])
def test_owned_row_large_threshold_bin(kind, offset):
    w = _owned_large_bin_rows(kind, 610 + len(kind))
    _gpu.say(f"[owned large bin] {kind} offset {offset}")
    for got in _gpu.run_gpu(w, "single", scores_offset=offset, repeat=2):
        _gpu.assert_matches_oracle(w, got, f"owned large bin {kind} offset {offset}")
