"""Helpers that run the HIP path on a synth.Workload and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from tests import _checks

_oracle_cache: dict = {}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_result(w, key=None):
    key = key or (w.name, w.digest())
    if key not in _oracle_cache:
        _oracle_cache[key] = oracle.canonical(*oracle.topk_workload(w, threads=8))
    return _oracle_cache[key]


def run_gpu(w, path="auto", *, wg_per_row=0, cand_capacity=0, min_chunk=0, with_idx=True,
            scores_offset=0, repeat=1, max_len=None):
    """Plan + select on the GPU; returns numpy (idx or None, slots) per call."""
    import torch
    from sparse_attention_indexer_amd import topk
    dev = torch.device("cuda:0")
    ml = w.max_len if max_len is None else max_len
    tk = topk.TopK(w.k, max(1, w.rows), ml, force_path=path, wg_per_row=wg_per_row,
                   cand_capacity=cand_capacity, min_chunk=min_chunk, device=dev)
    if scores_offset:
        big = torch.zeros((w.rows, w.stride + scores_offset), dtype=torch.float32, device=dev)
        big[:, scores_offset:] = torch.from_numpy(w.scores).to(dev)
        scores = big[:, scores_offset:]
    else:
        scores = torch.from_numpy(np.ascontiguousarray(w.scores)).to(dev)
    lengths = torch.from_numpy(w.lengths).to(dev)
    table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    tk.plan(lengths)
    outs = []
    for _ in range(repeat):
        slots, idx = tk.select(scores, lengths, table, w.bt_row_stride, w.page_size, with_indices=with_idx)
        torch.cuda.synchronize()
        outs.append((None if idx is None else idx.cpu().numpy(), slots.cpu().numpy()))
    st = tk.status()
    assert st == 0, f"device status {st}"
    return outs if repeat > 1 else outs[0]


def assert_matches_oracle(w, got, label=""):
    idx, slots = got
    ref_idx, ref_slots = oracle_result(w)
    if idx is not None:
        ci, cs = oracle.canonical(idx, slots)
        bad = np.flatnonzero((ci != ref_idx).any(axis=1) | (cs != ref_slots).any(axis=1))
        assert bad.size == 0, f"{label}: rows {bad[:10]} differ from the oracle"
    else:
        cs = oracle.canonical_slots(slots)
        rs = oracle.canonical_slots(ref_slots)
        bad = np.flatnonzero((cs != rs).any(axis=1))
        assert bad.size == 0, f"{label}: rows {bad[:10]} (slots only) differ from the oracle"


def assert_invariants(w, got, rows=None, label=""):
    idx, slots = got
    inv = _checks.invert_tables(w.block_table, w.bt_row_stride, w.rows, w.page_size)
    for r in (range(w.rows) if rows is None else rows):
        _checks.check_row(w.scores[r], int(w.lengths[r]), w.k, None if idx is None else idx[r],
                          slots[r], inv[r], w.page_size, f"{label} row {r}")
