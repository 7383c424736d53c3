"""GPU parity of the indexer's score producer (query prologue and MQA
logits on the matrix cores) against the oracle (oracle/indexer_logits.py),
through the C ABI.

Tolerance of a score (derived from the FP32 arithmetic): the 128 products of
a dot are exact in FP32 (E4M3 x E4M3 needs 8 significant bits) and their sum
is rounded at most 127 times, the 32 or more head terms at most H - 1 times,
each rounding at most 2^-24 of a partial sum bounded by the sum of the terms'
magnitudes; with H <= 128 that is below 256 * 2^-24 = 1.6e-5 of
bound = k_scale * sum_h |w| * sum_d |q * k|. The test allows 2e-5 * bound.
The query prologue's codes follow the key path's tie rule and its weights
a relative 1e-5 (see test_prologue_gpu.py).
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from oracle import indexer_logits as L
from tests import _gpu
from tests.test_prologue_gpu import assert_codes_match

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    HAVE_GPU = False

pytestmark = pytest.mark.gpu
if not HAVE_GPU:
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_indexer_amd import logits as G  # noqa: E402
from sparse_attention_indexer_amd import prologue as K  # noqa: E402

SENT = -12345.0


def run_logits(w: synth.LogitsInputs, max_len: int | None = None):
    dev = torch.device("cuda:0")
    ml = int(w.lengths.max()) if max_len is None else max_len
    out = torch.full((w.tokens, ml + 5), SENT, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    G.indexer_mqa_logits(torch.from_numpy(w.q_codes).to(dev), torch.from_numpy(w.w).to(dev),
                         torch.from_numpy(w.k_fp8).to(dev), torch.from_numpy(w.k_scale).to(dev),
                         torch.from_numpy(np.ascontiguousarray(w.block_table[0])).to(dev), w.page_size,
                         torch.from_numpy(w.lengths).to(dev), ml, out, status)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(status.item())


def check_logits(w: synth.LogitsInputs, label: str, sample: int | None = None):
    got, st = run_logits(w)
    assert st == 0, f"{label}: status {st:#x}"
    L_ = int(w.lengths.max())
    assert (got[:, L_:] == SENT).all(), f"{label}: wrote past max_len"
    rng = np.random.default_rng(0)
    for t in range(w.tokens):
        n = int(w.lengths[t])
        assert (got[t, n:L_] == SENT).all(), f"{label}: token {t} wrote past its length"
        pos = np.arange(n) if sample is None or n <= sample else np.unique(np.concatenate(
            [np.arange(64), np.arange(n - 64, n), rng.integers(0, n, sample)]))
        ref, bound = L.mqa_logits_at(w.q_codes, w.w, w.k_fp8, w.k_scale, w.block_table, 0, w.page_size, t, pos)
        err = np.abs(got[t, pos].astype(np.float64) - ref)
        bad = err > 2e-5 * bound + 1e-30
        assert not bad.any(), f"{label}: token {t}: {int(bad.sum())} scores off, e.g. pos {pos[bad][:3]} " \
                              f"got {got[t, pos][bad][:3]} want {ref[bad][:3]} bound {bound[bad][:3]}"


CASES = [
    dict(tokens=1, keys=32, heads=32),        # one MFMA block: the operand layout
    dict(tokens=3, keys=77, heads=32, page_size=16),
    dict(tokens=7, keys=1000, heads=64),
    dict(tokens=8, keys=5000, heads=64, page_size=1),
    dict(tokens=16, keys=700, heads=32),      # tokens x heads = 512, the maximum
    dict(tokens=2, keys=40_000, heads=128),
    dict(tokens=1, keys=3000, heads=64),
    dict(tokens=2, keys=2100, heads=64, page_size=16),
    dict(tokens=3, keys=1500, heads=64, page_size=48),   # a page size that is not a power of two
    dict(tokens=5, keys=2000, heads=32),
]


@pytest.mark.parametrize("case", CASES, ids=[",".join(f"{k}={v}" for k, v in c.items()) for c in CASES])
def test_mqa_logits_parity(case):
    w = synth.make_logits(seed=70 + case["keys"] % 97, with_table=False, **case)
    _gpu.say(f"[logits] {case}")
    check_logits(w, str(case))


def test_mqa_logits_full_size_sampled():
    """The benchmarked shape: 7 verify tokens x 64 heads over 1,000,000 keys,
    every score of the first and last 64 positions and 20,000 random ones per token."""
    w = synth.make_logits(7, 1_000_000, seed=22, with_table=False)
    _gpu.say("[logits] 7 x 1,000,000 sampled")
    check_logits(w, "7x1M", sample=20_000)


def test_mqa_logits_many_tiles_sampled():
    """Many key steps per wave of the persistent grid, 32 heads, a page size
    other than the default."""
    w = synth.make_logits(6, 150_000, heads=32, page_size=32, seed=23, with_table=False)
    _gpu.say("[logits] 6 x 150,000 x 32 heads sampled")
    check_logits(w, "6x150K", sample=5000)


def test_mqa_logits_limits_and_flags():
    w = synth.make_logits(17, 100, heads=32, seed=5, with_table=False)     # 544 query rows
    dev = torch.device("cuda:0")
    out = torch.zeros((17, 100), dtype=torch.float32, device=dev)
    with pytest.raises(Exception):
        G.indexer_mqa_logits(torch.from_numpy(w.q_codes).to(dev), torch.from_numpy(w.w).to(dev),
                             torch.from_numpy(w.k_fp8).to(dev), torch.from_numpy(w.k_scale).to(dev),
                             torch.from_numpy(np.ascontiguousarray(w.block_table[0])).to(dev), w.page_size,
                             torch.from_numpy(w.lengths).to(dev), 100, out)
    w = synth.make_logits(2, 300, heads=32, seed=6, with_table=False)
    w.block_table = w.block_table.copy()
    w.block_table[0, 2] = 10_000                                            # a page past the cache
    got, st = run_logits(w)
    assert st & K.DEVICE_BAD_SLOT
    assert (got[:, 128:192] == SENT).all()                                  # that page's keys skipped


@pytest.mark.parametrize("tokens,heads,rope_dim", [(7, 64, 64), (1, 32, 0), (5, 96, 128)])
def test_query_prologue_parity(tokens, heads, rope_dim):
    w = synth.make_logits(tokens, 3000, heads=heads, rope_dim=rope_dim, seed=tokens + heads)
    dev = torch.device("cuda:0")
    cs = torch.from_numpy(w.cos_sin).to(dev) if rope_dim else None
    codes, wq = K.indexer_query_prologue(torch.from_numpy(w.q_bf16.view(np.int16)).to(dev),
                                         torch.from_numpy(w.w_raw).to(dev), 0.01, cs, rope_dim,
                                         torch.from_numpy(w.positions).to(dev))
    torch.cuda.synchronize()
    rc, rw, scaled = L.query_prologue(w.q_bf16, w.w_raw, 0.01, w.cos_sin, rope_dim, w.positions)
    assert_codes_match(codes.cpu().numpy().reshape(-1, 128), rc.reshape(-1, 128), scaled.reshape(-1, 128),
                       f"query {tokens}x{heads}")
    rel = np.abs(wq.cpu().numpy().astype(np.float64) - rw) / np.maximum(np.abs(rw), 1e-30)
    assert rel.max() <= 1e-5


def test_indexer_pipeline_feeds_the_top_k():
    """Query prologue -> logits -> top-k on the GPU: the top-k of the GPU's own
    scores equals the oracle top-k of those scores, and the scores match the
    oracle's within the tolerance."""
    import oracle
    from sparse_attention_indexer_amd import topk
    w = synth.make_logits(7, 60_000, seed=9, rope_dim=64)
    dev = torch.device("cuda:0")
    codes, wq = K.indexer_query_prologue(torch.from_numpy(w.q_bf16.view(np.int16)).to(dev),
                                         torch.from_numpy(w.w_raw).to(dev), 0.01,
                                         torch.from_numpy(w.cos_sin).to(dev), 64,
                                         torch.from_numpy(w.positions).to(dev))
    L_ = int(w.lengths.max())
    scores = torch.full((7, L_), float("-inf"), dtype=torch.float32, device=dev)
    lengths = torch.from_numpy(w.lengths).to(dev)
    table = torch.from_numpy(np.ascontiguousarray(w.block_table[0])).to(dev)
    G.indexer_mqa_logits(codes, wq, torch.from_numpy(w.k_fp8).to(dev), torch.from_numpy(w.k_scale).to(dev),
                         table, w.page_size, lengths, L_, scores)
    tk = topk.TopK(2048, 7, L_, device=dev)
    tk.plan(lengths)
    slots, idx = tk.select(scores, lengths, table[None, :].contiguous(), 0, w.page_size)
    torch.cuda.synchronize()
    s_host = scores.cpu().numpy()
    ref_idx, ref_slots = oracle.topk_paged(s_host, w.lengths, w.block_table, 0, w.page_size, 2048)
    gi, gs = oracle.canonical(idx.cpu().numpy(), slots.cpu().numpy())
    ri, rs = oracle.canonical(ref_idx, ref_slots)
    assert np.array_equal(gi, ri) and np.array_equal(gs, rs)
    # and the scores themselves (spot check) against the oracle chain
    rc, rw, _ = L.query_prologue(w.q_bf16, w.w_raw, 0.01, w.cos_sin, 64, w.positions)
    ref, bound = L.mqa_logits_at(codes.cpu().numpy(), wq.cpu().numpy(), w.k_fp8, w.k_scale, w.block_table, 0,
                                 w.page_size, 3, np.arange(0, int(w.lengths[3]), 7))
    assert np.all(np.abs(s_host[3, 0:int(w.lengths[3]):7] - ref) <= 2e-5 * bound + 1e-30)
