"""topk_select_paged_noalloc: the entry point that allocates nothing.

It must give exactly what topk_select_paged gives on the same inputs (which
the parity tests tie to the oracle), on consecutive calls that share the
library's device array, the second with a smaller batch; a timed-out call
must not leave state that spoils the next one; sizes beyond the array are
refused before anything is enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests import _gpu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _tensors(w, dev):
    return (torch.from_numpy(np.ascontiguousarray(w.scores)).to(dev), torch.from_numpy(w.lengths).to(dev),
            torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev))


def _with_workspace(w, dev):
    from sparse_attention_indexer_amd import topk
    tk = topk.TopK(w.k, w.rows, w.max_len, device=dev)
    sc, ln, bt = _tensors(w, dev)
    tk.plan(ln)
    slots, idx = tk.select(sc, ln, bt, w.bt_row_stride, w.page_size)
    torch.cuda.synchronize()
    assert tk.status() == 0
    return oracle.canonical(idx.cpu().numpy(), slots.cpu().numpy())


def _no_alloc(w, dev, cfg=None, status=None):
    from sparse_attention_indexer_amd import topk
    cfg = cfg or topk.make_config(w.k, w.rows, w.max_len)
    sc, ln, bt = _tensors(w, dev)
    slots = torch.full((w.rows, w.k), -7, dtype=torch.int32, device=dev)
    idx = torch.full_like(slots, -7)
    topk.topk_select_paged_noalloc(cfg, sc, ln, bt, w.bt_row_stride, w.page_size, slots, idx, status)
    torch.cuda.synchronize()
    return oracle.canonical(idx.cpu().numpy(), slots.cpu().numpy())


def test_no_alloc_matches_workspace_entry_on_two_calls():
    dev = torch.device("cuda:0")
    big = synth.make_config(3)                                                   # 7 x 1M, split rows
    small = synth.random_case(77, rows=5, max_len=50_000, alphabet=40, k=1500)   # smaller, ragged
    for label, w in (("7x1M", big), ("5x50K", small)):
        _gpu.say(f"[no-alloc] {label}")
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        got = _no_alloc(w, dev, status=status)
        assert int(status.item()) == 0
        want = _with_workspace(w, dev)
        np.testing.assert_array_equal(got[0], want[0], err_msg=f"{label} positions")
        np.testing.assert_array_equal(got[1], want[1], err_msg=f"{label} slots")
        _gpu.assert_matches_oracle(w, got, f"no-alloc {label}")


def test_no_alloc_recovers_after_a_timed_out_call():
    """A call whose split rows give up (spin_limit -1) reports the time-out in
    device_status and leaves the shared array dirty; the next call clears it
    and is exact."""
    from sparse_attention_indexer_amd import topk
    dev = torch.device("cuda:0")
    w = synth.random_case(62, rows=7, max_len=100_000, alphabet=0, k=2048, exact_len=True)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    _no_alloc(w, dev, cfg=topk.make_config(w.k, w.rows, w.max_len, spin_limit=-1), status=status)
    assert int(status.item()) == topk.DEVICE_SPIN_TIMEOUT
    status.zero_()
    got = _no_alloc(w, dev, status=status)
    assert int(status.item()) == 0
    _gpu.assert_matches_oracle(w, got, "no-alloc after time-out")


def test_no_alloc_refuses_what_does_not_fit():
    from sparse_attention_indexer_amd import topk
    dev = torch.device("cuda:0")
    sc = torch.zeros((1, 8), dtype=torch.float32, device=dev)
    ln = torch.zeros(1, dtype=torch.int32, device=dev)
    bt = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    out = torch.empty((1, 2048), dtype=torch.int32, device=dev)
    too_big = topk.make_config(2048, 512, 1_000_000)   # 128 split rows x 16K candidates > the array
    with pytest.raises(topk.TopKError) as e:
        topk.topk_select_paged_noalloc(too_big, torch.zeros((1, 1_000_000), device=dev), ln, bt, 0, 64, out, None)
    assert e.value.status == topk.TOPK_ERR_BUFFER_TOO_SMALL
    many = topk.make_config(2048, 600, 8)
    lens = torch.zeros(600, dtype=torch.int32, device=dev)
    with pytest.raises(topk.TopKError) as e:
        topk.topk_select_paged_noalloc(many, torch.zeros((600, 8), device=dev), lens, bt, 0, 64,
                                       torch.empty((600, 2048), dtype=torch.int32, device=dev), None)
    assert e.value.status == topk.TOPK_ERR_UNSUPPORTED
    del sc, out
