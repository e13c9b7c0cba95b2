"""Device-data checks: mp_check_indices counts out-of-range labels / ids
exactly, and with MP_DEBUG_CHECKS set the calls that read labels, token ids or
expert ids refuse a negative one with MP_ERR_DATA before launching anything
(without it they run, as documented: the fast path does not check)."""

import numpy as np
import pytest
import torch

from gpu_util import say, sync
from megatron_tensor_transformer_02_amd import mp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [0, 1, 1000, 300001])
def test_check_indices_counts_out_of_range(n):
    say("check indices", n)
    rng = np.random.default_rng(n)
    v = rng.integers(-5, 51205, size=n).astype(np.int32)
    idx = torch.from_numpy(v).cuda()
    cnt = torch.full((1,), 12345, dtype=torch.int64, device="cuda")
    mp.mp_check_indices(idx, 0, 51200, cnt)
    sync()
    assert int(cnt.item()) == int(((v < 0) | (v >= 51200)).sum())


def test_debug_checks_reject_negative_labels_and_ids(monkeypatch):
    say("debug checks")
    T, Vi, K = 64, 128, 64
    labels = torch.arange(T, dtype=torch.int32, device="cuda")
    labels[17] = -3
    z = torch.randn(T, Vi, device="cuda")
    tr = torch.empty(T, 3, device="cuda")
    monkeypatch.setenv("MP_DEBUG_CHECKS", "0")
    mp.mp_vocab_parallel_xent(z, labels, 0, tr)  # fast path: not checked
    sync()
    monkeypatch.setenv("MP_DEBUG_CHECKS", "1")
    with pytest.raises(mp.MPError) as e:
        mp.mp_vocab_parallel_xent(z, labels, 0, tr)
    assert e.value.code == -9 and "labels[17] = -3" in str(e.value)
    emb = torch.randn(Vi, K, device="cuda").to(torch.bfloat16)
    out = torch.empty(T, K, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mp.MPError) as e:
        mp.mp_vocab_parallel_embedding(labels, emb, 0, out)
    assert e.value.code == -9
    ids = torch.zeros(T, 2, dtype=torch.int32, device="cuda")
    ids[:, 1] = 1
    ids[5, 0] = -1
    w = torch.full((T, 2), 0.5, device="cuda")
    wgu = torch.zeros(2, 128, K, dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros(2, K, 64, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(T, K, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mp.MPError) as e:
        mp.mp_grouped_expert_gemm(x, ids, w, wgu, wd, 0, out)
    assert e.value.code == -9 and "topk_ids[10] = -1" in str(e.value)
    ids[5, 0] = 0
    mp.mp_grouped_expert_gemm(x, ids, w, wgu, wd, 0, out)  # valid data passes the check
    sync()
