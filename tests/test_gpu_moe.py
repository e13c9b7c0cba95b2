"""GPU parity: the MoE expert shard (permutation, grouped gate/up GEMM with
SwiGLU, grouped down GEMM, weighted unpermute) against the oracle, in both
the weighted-unpermute form and the memory-efficient form (routing weight on
the activation).  The permutation and expert offsets are compared bit for
bit."""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import TOL, cu, f64, rel_frobenius, say, sync
from megatron_tensor_transformer_02_amd import mp, synthetic as S

pytestmark = pytest.mark.gpu


def routing(seed, T, experts, topk):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(experts)[:topk] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, topk)).astype(np.float32)
    return torch.from_numpy(ids), torch.from_numpy(w / w.sum(axis=1, keepdims=True))


def run(x, ids, w, wgu, wd, e_start, fn=None):
    fn = fn or mp.mp_grouped_expert_gemm
    T, Hd = x.shape
    topk = ids.shape[1]
    e_local = wgu.shape[0]
    out = torch.empty((T, Hd), dtype=torch.bfloat16, device="cuda")
    perm = torch.full((T * topk,), -7, dtype=torch.int32, device="cuda")
    offs = torch.empty(e_local + 1, dtype=torch.int32, device="cuda")
    fn(cu(x), cu(ids), cu(w), cu(wgu), cu(wd), e_start, out, perm, offs)
    sync()
    return out, perm.cpu().numpy(), offs.cpu().numpy()


CASES = [
    (50, 64, 40, 16, 4, 4, 4),      # ragged Fe against the 128-column act tile
    (300, 256, 136, 32, 8, 0, 8),
    (77, 128, 64, 8, 1, 5, 2),      # a single local expert
    (40, 64, 64, 16, 16, 0, 3),     # every expert local
    (33, 64, 64, 16, 4, 12, 1),     # top-1
    (700, 200, 264, 4, 2, 1, 2),    # >256 rows per expert, ragged k-tiles in both GEMMs
    (513, 72, 520, 8, 3, 2, 4),     # K = 72 (one full and one 8-wide k-tile), 5 act tiles
    (300, 1096, 1032, 32, 8, 0, 2), # sparse experts with both GEMMs split over k (ragged last k-tiles)
    (8500, 64, 64, 16, 4, 2, 8),    # 34 blocks of 256 tokens in the two-kernel routing
    (200, 64, 64, 80, 70, 3, 4),    # 70 local experts: more than the two-kernel routing takes (four kernels)
    (200, 64, 64, 80, 64, 3, 4),    # 64 local experts: the most the two-kernel routing takes
    (65536, 64, 64, 8, 4, 2, 2),    # 65536 tokens: the most the two-kernel routing takes (256 blocks)
    (65537, 64, 64, 8, 4, 2, 2),    # one token more: the four-kernel routing
]
FORMS = {"weighted_unpermute": (lambda: mp.mp_grouped_expert_gemm, O.moe_forward),
         "weighted_act": (lambda: mp.mp_grouped_expert_gemm_weighted_act, O.moe_forward_weighted_act)}


@pytest.mark.parametrize("form", list(FORMS))
@pytest.mark.parametrize("T,Hd,Fe,experts,e_local,e_start,topk", CASES)
def test_grouped_expert_gemm(T, Hd, Fe, experts, e_local, e_start, topk, form):
    say("moe", form, T, Hd, Fe, experts, e_local, e_start, topk)
    fn, oracle_fn = FORMS[form]
    ids, w = routing(T + Hd, T, experts, topk)
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((T, Hd), dtype=np.float32)).to(torch.bfloat16)
    wgu = torch.from_numpy((rng.standard_normal((e_local, 2 * Fe, Hd), dtype=np.float32) * 0.1)).to(torch.bfloat16)
    wd = torch.from_numpy((rng.standard_normal((e_local, Hd, Fe), dtype=np.float32) * 0.1)).to(torch.bfloat16)
    out, perm, offs = run(x, ids, w, wgu, wd, e_start, fn())
    want, counts, woffs, picks, _ = oracle_fn(f64(x), ids.numpy(), w.numpy(), f64(wgu), f64(wd), e_start)
    r = picks.size
    assert np.array_equal(offs, woffs)
    assert np.array_equal(perm[:r], picks)
    assert np.all(perm[r:] == -7)  # entries past R untouched
    assert rel_frobenius(f64(out), want) <= TOL["bf16"]


@pytest.mark.parametrize("form", list(FORMS))
def test_no_local_picks_gives_zeros(form):
    say("moe empty shard", form)
    T, Hd, Fe = 20, 64, 64
    ids, w = routing(1, T, 8, 2)
    x = torch.ones((T, Hd), dtype=torch.bfloat16)
    wgu = torch.ones((2, 2 * Fe, Hd), dtype=torch.bfloat16)
    wd = torch.ones((2, Hd, Fe), dtype=torch.bfloat16)
    out, perm, offs = run(x, ids, w, wgu, wd, 100, FORMS[form][0]())  # experts 100, 101 are never picked
    assert np.all(offs == 0)
    assert np.all(f64(out) == 0)


@pytest.mark.slow
@pytest.mark.parametrize("form", list(FORMS))
def test_moe_shard_full_size(form):
    # The hot expert-parallel shard (experts 0-7 of 256, Zipf(1.1) routing):
    # permutation in full, outputs for 48 sampled tokens through the oracle.
    say("moe full size", form)
    fn, oracle_fn = FORMS[form]
    wl = S.WORKLOADS["moe"]
    inp = S.moe_inputs(wl)
    out, perm, offs = run(inp["x"], inp["topk_ids"], inp["topk_w"], inp["w_gu"], inp["w_d"], 0, fn())
    counts, woffs, picks = O.moe_permutation(inp["topk_ids"].numpy(), 0, wl.e_local)
    assert np.array_equal(offs, woffs)
    assert np.array_equal(perm[:picks.size], picks)
    toks = np.random.default_rng(3).choice(wl.T, 48, replace=False)
    sub_out = oracle_fn(f64(inp["x"])[toks], inp["topk_ids"].numpy()[toks], inp["topk_w"].numpy()[toks],
                        f64(inp["w_gu"]), f64(inp["w_d"]), 0)[0]
    assert rel_frobenius(f64(out)[toks], sub_out) <= TOL["bf16"]


@pytest.mark.parametrize("form", list(FORMS))
def test_split_sparse_experts_beside_dense(form):
    """One dense expert (300 rows: a full and a partial 256-row tile) beside
    sparse ones (about 60 rows) whose 64-row launches are split over k; the
    two kinds of launch write disjoint rows."""
    say("moe dense + split sparse", form)
    T, Hd, Fe, experts, e_local, topk = 600, 1024, 1024, 16, 4, 2
    rng = np.random.default_rng(11)
    ids = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        first = 0 if t < 300 else int(rng.integers(1, experts))
        rest = rng.permutation([e for e in range(experts) if e != first])[: topk - 1]
        ids[t] = [first, *rest]
    wts = rng.random((T, topk)).astype(np.float32)
    w = torch.from_numpy(wts / wts.sum(axis=1, keepdims=True))
    ids = torch.from_numpy(ids)
    x = torch.from_numpy(rng.standard_normal((T, Hd), dtype=np.float32)).to(torch.bfloat16)
    wgu = torch.from_numpy(rng.standard_normal((e_local, 2 * Fe, Hd), dtype=np.float32) * 0.05).to(torch.bfloat16)
    wd = torch.from_numpy(rng.standard_normal((e_local, Hd, Fe), dtype=np.float32) * 0.05).to(torch.bfloat16)
    fn, oracle_fn = FORMS[form]
    out, perm, offs = run(x, ids, w, wgu, wd, 0, fn())
    want, counts, woffs, picks, _ = oracle_fn(f64(x), ids.numpy(), w.numpy(), f64(wgu), f64(wd), 0)
    assert counts[0] >= 256 and 0 < counts[1:].max() < 192  # one dense expert, the rest sparse
    assert np.array_equal(offs, woffs) and np.array_equal(perm[:picks.size], picks)
    assert rel_frobenius(f64(out), want) <= TOL["bf16"]
    # Rows of each expert separately: a wrong sparse slot would misplace whole rows.
    for e in range(e_local):
        toks = np.nonzero((ids.numpy() == e).any(axis=1))[0]
        if toks.size:
            assert rel_frobenius(f64(out)[toks], want[toks]) <= TOL["bf16"], e


@pytest.mark.slow
@pytest.mark.parametrize("form", list(FORMS))
def test_moe_median_shard_full_size(form):
    """The median expert-parallel shard of the full-size routing (experts
    128-135 of 256: a few hundred rows, every expert sparse, both GEMMs split
    over k) with the timed configuration's weights; outputs of 48 sampled
    tokens that have a pick in the shard, through the oracle."""
    say("moe median shard full size", form)
    fn, oracle_fn = FORMS[form]
    wl = S.WORKLOADS["moe"]
    inp = S.moe_inputs(wl)
    e_med = wl.experts // 2
    out, perm, offs = run(inp["x"], inp["topk_ids"], inp["topk_w"], inp["w_gu"], inp["w_d"], e_med, fn())
    ids = inp["topk_ids"].numpy()
    counts, woffs, picks = O.moe_permutation(ids, e_med, wl.e_local)
    assert 0 < counts.max() < 192
    assert np.array_equal(offs, woffs) and np.array_equal(perm[:picks.size], picks)
    hit = np.nonzero(((ids >= e_med) & (ids < e_med + wl.e_local)).any(axis=1))[0]
    toks = np.random.default_rng(4).choice(hit, min(48, hit.size), replace=False)
    sub_out = oracle_fn(f64(inp["x"])[toks], ids[toks], inp["topk_w"].numpy()[toks],
                        f64(inp["w_gu"]), f64(inp["w_d"]), e_med)[0]
    assert rel_frobenius(f64(out)[toks], sub_out) <= TOL["bf16"]
    miss = np.setdiff1d(np.arange(wl.T), hit)
    assert torch.all(out.float()[torch.from_numpy(miss)] == 0)
