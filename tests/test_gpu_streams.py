"""Calls on two streams at once, each with the binding's default scratch
workspace: the cached workspace is kept per (device, stream), so two
weight-gradient GEMMs whose split-K partials use it can run concurrently and
give exactly what they give one after the other."""

import numpy as np
import pytest
import torch

from gpu_util import say, sync
from megatron_tensor_transformer_02_amd import mp

pytestmark = pytest.mark.gpu


def test_concurrent_streams_use_separate_workspaces():
    say("two streams, default workspaces")
    T, Fi, K = 8192, 384, 3072  # the out-projection's backward (split-K weight gradient)
    g = torch.Generator().manual_seed(3)
    mk = lambda *s, sc=1.0: (torch.randn(*s, generator=g) * sc).to("cuda", torch.bfloat16)  # noqa: E731
    jobs = []
    for _ in range(2):
        jobs.append(dict(Y=mk(T, Fi), B=mk(K, Fi, sc=0.02), dO=mk(T, K),
                         dY=torch.empty(T, Fi, dtype=torch.bfloat16, device="cuda"),
                         dB=torch.empty(K, Fi, dtype=torch.float32, device="cuda")))
    assert mp.lib().mp_row_linear_partial_bwd_workspace(mp.MP_BF16, T, Fi, K) > 0  # scratch is used

    def run(j, stream=None):
        mp.mp_row_linear_partial_bwd(j["Y"], j["B"], j["dO"], j["dY"], j["dB"], stream=stream)

    want = []
    for j in jobs:
        run(j)
        sync()
        want.append((j["dY"].clone(), j["dB"].clone()))
        j["dY"].fill_(0)
        j["dB"].fill_(0)
    sync()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        run(jobs[0], s1)
        run(jobs[1], s2)
        torch.cuda.current_stream().wait_stream(s1)
        torch.cuda.current_stream().wait_stream(s2)
        sync()
        for j, (dy, db) in zip(jobs, want):
            assert torch.equal(j["dY"], dy) and torch.equal(j["dB"], db)


def test_workspace_growth_while_another_stream_is_busy():
    """The cached workspace of stream s1 grows (a bigger call replaces it)
    while s1 still has queued work that writes the old buffer, and s2 works
    on its own buffer meanwhile: the old block is allocated under s1, so it
    goes back to s1's pool and no other stream's allocation can take it
    while s1's kernels use it.  Every result equals its sequential value."""
    say("workspace growth under load")
    g = torch.Generator().manual_seed(4)
    mk = lambda *s, sc=1.0: (torch.randn(*s, generator=g) * sc).to("cuda", torch.bfloat16)  # noqa: E731
    shapes = [(2048, 384, 3072), (8192, 384, 3072), (8192, 1536, 3072)]  # growing split-K workspaces
    jobs = [dict(Y=mk(T, Fi), B=mk(K, Fi, sc=0.02), dO=mk(T, K),
                 dY=torch.empty(T, Fi, dtype=torch.bfloat16, device="cuda"),
                 dB=torch.empty(K, Fi, dtype=torch.float32, device="cuda")) for T, Fi, K in shapes]
    need = [mp.lib().mp_row_linear_partial_bwd_workspace(mp.MP_BF16, T, Fi, K) for T, Fi, K in shapes]
    assert need[0] < need[1] < need[2]

    def run(j, stream=None):
        mp.mp_row_linear_partial_bwd(j["Y"], j["B"], j["dO"], j["dY"], j["dB"], stream=stream)

    want = []
    for j in jobs:
        run(j)
        sync()
        want.append((j["dY"].clone(), j["dB"].clone()))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(2):
        mp._ws_cache.clear()
        for j in jobs:
            j["dY"].fill_(0)
            j["dB"].fill_(0)
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        run(jobs[0], s1)  # small workspace on s1
        run(jobs[2], s1)  # grows s1's workspace while the first call may still run
        junk = [torch.empty(n, dtype=torch.uint8, device="cuda") for n in need]  # allocations elsewhere
        with torch.cuda.stream(s2):
            for t in junk:
                t.fill_(0xFF)
        run(jobs[1], s2)
        torch.cuda.current_stream().wait_stream(s1)
        torch.cuda.current_stream().wait_stream(s2)
        sync()
        del junk
        for j, (dy, db) in zip(jobs, want):
            assert torch.equal(j["dY"], dy) and torch.equal(j["dB"], db)
