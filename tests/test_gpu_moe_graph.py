"""The MoE shard's training forward and backward captured once in a HIP graph
and replayed (MOE-core, technical summary 2.4: the dynamic shapes stay on the
device, so the whole shard can be captured).  Between replays the routing is
rewritten in place on the device (a different number of routed rows per
expert each time) and eager work runs; every replay must equal a fresh eager
run of the same inputs bit for bit."""

import numpy as np
import pytest
import torch

from gpu_util import say, sync
from megatron_tensor_transformer_02_amd import mp

pytestmark = pytest.mark.gpu


def routing(seed, T, experts, topk):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(experts)[:topk] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, topk)).astype(np.float32)
    return torch.from_numpy(ids), torch.from_numpy(w / w.sum(axis=1, keepdims=True))


@pytest.mark.parametrize("Hd,Fe", [(256, 136), (1096, 1032)])  # the second splits the sparse launches over k
def test_moe_train_step_graph_replay(Hd, Fe):
    say("moe graph capture", Hd, Fe)
    T, experts, e_local, topk = 300, 32, 8, 8
    rng = np.random.default_rng(9)
    dev = "cuda"
    x = torch.from_numpy(rng.standard_normal((T, Hd), dtype=np.float32)).to(dev, torch.bfloat16)
    wgu = torch.from_numpy(rng.standard_normal((e_local, 2 * Fe, Hd), dtype=np.float32) * 0.1).to(dev, torch.bfloat16)
    wd = torch.from_numpy(rng.standard_normal((e_local, Hd, Fe), dtype=np.float32) * 0.1).to(dev, torch.bfloat16)
    dout = torch.from_numpy(rng.standard_normal((T, Hd), dtype=np.float32)).to(dev, torch.bfloat16)
    ids0, w0 = routing(1, T, experts, topk)
    ids, w = ids0.to(dev), w0.to(dev)
    out = torch.empty((T, Hd), dtype=torch.bfloat16, device=dev)
    gu = torch.empty((T * topk, 2 * Fe), dtype=torch.bfloat16, device=dev)
    fws = torch.empty(mp.lib().mp_grouped_expert_gemm_workspace(T, Hd, Fe, topk, e_local), dtype=torch.uint8,
                      device=dev)
    bws = torch.empty(mp.lib().mp_grouped_expert_gemm_bwd_workspace(T, Hd, Fe, topk, e_local), dtype=torch.uint8,
                      device=dev)
    dx = torch.empty((T, Hd), dtype=torch.bfloat16, device=dev)
    dwgu = torch.empty((e_local, 2 * Fe, Hd), dtype=torch.float32, device=dev)
    dwd = torch.empty((e_local, Hd, Fe), dtype=torch.float32, device=dev)
    dtw = torch.empty((T, topk), dtype=torch.float32, device=dev)

    def step(stream=None):
        mp.mp_grouped_expert_gemm_fwd_train(x, ids, w, wgu, wd, 0, out, gu, fws, stream=stream)
        mp.mp_grouped_expert_gemm_bwd(x, w, wgu, wd, dout, gu, fws, dx, dwgu, dwd, dtw, bws, stream=stream)

    def snapshot():
        return [t.clone() for t in (out, dx, dwgu, dwd, dtw)]

    # Warm up on a side stream, as capture requires, then capture.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    sync()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    sync()

    rows = []
    for rep, seed in enumerate((1, 2, 3, 2)):
        ids_r, w_r = routing(seed, T, experts, topk)
        ids.copy_(ids_r.to(dev))
        w.copy_(w_r.to(dev))
        rows.append(int(((ids_r >= 0) & (ids_r < e_local)).sum()))
        torch.cuda.synchronize()
        step()                      # eager reference for these inputs
        sync()
        want = snapshot()
        for t in (out, dx, dwgu, dwd, dtw):
            t.fill_(7.0)            # eager work between replays; stale values must be overwritten
        sync()
        graph.replay()
        sync()
        got = snapshot()
        names = ("out", "dx", "dW_gu", "dW_d", "dtopk_w")
        for name, a, b in zip(names, got, want):
            assert torch.equal(a, b), (rep, name)
    assert len(set(rows[:3])) > 1  # the replays routed different numbers of rows
