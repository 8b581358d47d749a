"""The 8k-token Hash-sparse forward step (LSH + sort of Q and K, exact lists, forward through the sort
permutations) captured once as a HIP graph, as ``bench.py --workload 2 --graph`` times it: every replay
gives the eager step's outputs bit for bit, with eager steps run on the same buffers between replays.
The library enqueues kernels only (no memset, copy or synchronisation), so the whole step is capturable."""

import pytest

from helpers import note

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_workload2_graph_replays_equal_eager():
    import bench
    import sparse_causal_attention_amd as scfa

    note("[graph] hash_fwd_bf16_T8192_nb16: eager step")
    w, step, _, _ = bench.workload_setup(scfa, torch, 2)
    _, ref = step(None)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(None)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, outs = step(None)
    for rep in range(4):
        note(f"[graph] replay {rep}")
        _, eager = step(None)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(outs[k], ref[k]), (rep, k)
            assert torch.equal(eager[k], ref[k]), (rep, k)
