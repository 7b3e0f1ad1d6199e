"""nabla_check_lists on the GPU: the lists every mask builder writes pass, and each
kind of malformed row is counted exactly once (a count outside [0, n], an entry
outside [0, n), a repeated or descending entry), including faults past the first
64 entries of a row and in the last row."""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _nb():
    import block_sparse_attention_nabla_amd as nb
    nb.load_library()
    return nb


def test_builder_lists_pass_and_faults_are_counted():
    nb = _nb()
    w = synth.get_workload("dit_small")
    x = synth.make_inputs(w, device="cuda")
    lists = nb.nabla_build_mask(x["q"], x["k"], w.thresholds()[0], transpose=True)
    n = w.n
    assert nb.nabla_check_lists(lists["kv_count"], lists["kv_idx"]) == 0
    assert nb.nabla_check_lists(lists["q_count"], lists["q_idx"]) == 0
    full = nb.nabla_build_mask(x["q"], x["k"], 1.0)
    assert nb.nabla_check_lists(full["kv_count"], full["kv_idx"]) == 0  # n = 176 > 64: several chunks

    cnt = full["kv_count"].clone()
    idx = full["kv_idx"].clone()
    B, H = cnt.shape[:2]
    bad = set()
    cnt[0, 0, 0] = n + 1; bad.add((0, 0, 0))                  # count above n
    cnt[0, 0, 1] = -1; bad.add((0, 0, 1))                     # negative count
    idx[0, 1, 2, 5] = n; bad.add((0, 1, 2))                   # entry out of range
    idx[0, 1, 3, 0] = -7; bad.add((0, 1, 3))                  # negative entry
    idx[0, 2, 4, 70] = idx[0, 2, 4, 69]; bad.add((0, 2, 4))   # repeat, second chunk
    idx[0, 2, 5, 64] = 3; bad.add((0, 2, 5))                  # descending across a chunk edge
    idx[0, H - 1, n - 1, n - 1] = 0; bad.add((0, H - 1, n - 1))  # last row, last entry
    # Entries past the count are never read: garbage there is fine.
    cnt[0, 3, 6] = 10
    idx[0, 3, 6, 10:] = -5
    assert nb.nabla_check_lists(cnt, idx) == len(bad)
    # An empty list and a full list are well formed.
    cnt2 = full["kv_count"].clone()
    cnt2[0, 0, 0] = 0
    assert nb.nabla_check_lists(cnt2, full["kv_idx"]) == 0
