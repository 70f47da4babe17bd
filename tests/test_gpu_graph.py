"""A whole step (subspace, centroid build, quantize-append, attention with a
self segment) captured once in a HIP graph on the cache's stream and replayed
several times, with eager work and synchronizations between the replays:
every replay must leave the same cache bytes and write the same output bits
as the eager calls."""

import numpy as np
import pytest

import workloads as W
from tests.gpu_helpers import log, small, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("objective,rank", [("qsac", 8), ("nearest", 0)])
def test_graph_replays_equal_eager(objective, rank):
    from video_world_model_amd import Cache
    w = small(W.workload("video_chunk"), heads=2, n_kv=1000, n_q=100, n_self=100)
    log(f"[graph] objective={objective} rank={rank}")
    gens = [W.HeadGen(w, h) for h in range(2)]
    keys = to_dev([g.keys(0, 1000) for g in gens], w.dtype)
    vals = to_dev([g.values(0, 1000) for g in gens], w.dtype)
    qh = to_dev([g.hist_queries() for g in gens], w.dtype)
    q = to_dev([g.current_queries()[:100] for g in gens], w.dtype)
    ks = to_dev([g.keys(1000, 1100) for g in gens], w.dtype)
    vs = to_dev([g.values(1000, 1100) for g in gens], w.dtype)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        cache = Cache(2, w.head_dim, w.n_centroids, rank, 1000, dtype=torch_dtype(w.dtype), max_query_tokens=100,
                      max_build_tokens=1000, objective=objective)
        out = torch.empty((2, 100, w.head_dim), dtype=torch.float32, device="cuda")

    def step():
        cache.truncate(0)
        if objective == "qsac" or rank > 0:
            cache.build_subspace(qh)
        cache.build_centroids(keys, 4)
        cache.quantize_append(keys, vals)
        cache.attend(q, ks, vs, mask="full", out=out)

    with torch.cuda.stream(stream):
        step()
        ref_cache = cache.export().clone()
        ref_out = out.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        with torch.cuda.stream(stream):
            out.zero_()
            g.replay()
            got_cache = cache.export().clone()
            got_out = out.clone()
        torch.cuda.synchronize()
        assert torch.equal(got_cache, ref_cache), f"replay {rep}: cache bytes differ"
        assert torch.equal(got_out.view(torch.int32), ref_out.view(torch.int32)), f"replay {rep}: output differs"
        # eager work between replays: an eager attend into another buffer
        with torch.cuda.stream(stream):
            other = cache.attend(q, ks, vs, mask="full")
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int32), ref_out.view(torch.int32))
    log("  4 replays equal the eager step")
