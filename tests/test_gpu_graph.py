"""HIP graph capture of the calls (as bench.py times them): every replay equals
the eager call bit for bit.

The library records no memset and allocates no memory, so a captured call is a
fixed set of kernel nodes.  Each test captures a call, then replays the graph
several times with eager calls and synchronisations in between, and checks the
outputs (and, for the fused step, the cache words) of every replay against an
eager run of the same call on identical inputs."""
import numpy as np
import pytest
import torch

import decode_attention_group_amd as kvq
from synth import small_q_bits, small_randn
from test_gpu_attention import make_pair, q_dev

pytestmark = pytest.mark.gpu


def clone(g):
    c = kvq.KVCache(g.batch, g.n_kv_heads, g.head_dim, g.k_bits, g.v_bits, g.capacity, window=g.window)
    for a, b in ((c.k_codes, g.k_codes), (c.v_codes, g.v_codes), (c.k_sb, g.k_sb), (c.v_sb, g.v_sb)):
        if a is not None:
            a.copy_(b)
    return c


@pytest.mark.parametrize("bits", [(4, 8), (8, 8), (16, 16)])
def test_graph_replays_of_decode_step(bits):
    kb, vb = bits
    B, Hq, Hkv, D, R, W, L = 4, 8, 2, 256, 512, 512, 1000
    print(f"graph decode step bits={bits}", flush=True)
    g0, _ = make_pair(B, Hkv, D, kb, vb, R, W, L - 1, seed=601 + kb)
    k = torch.from_numpy(small_randn(602, (B, Hkv, D), D ** -0.25)).cuda()
    v = torch.from_numpy(small_randn(603, (B, Hkv, D), D ** -0.25)).cuda()
    q = q_dev(small_q_bits(604, (B, Hq, D), D ** -0.25))
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(kvq.kvq_decode_step_workspace_bytes(g0, Hq, L), 256), dtype=torch.uint8, device="cuda")
    # eager reference on a copy of the cache
    ge = clone(g0)
    ref = kvq.kvq_decode_step(ge, k, v, q, lens, L, workspace=ws)
    torch.cuda.synchronize()
    gg = clone(g0)
    out = torch.empty_like(q)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kvq.kvq_decode_step(gg, k, v, q, lens, L, out=out, workspace=ws)      # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        kvq.kvq_decode_step(gg, k, v, q, lens, L, out=out, workspace=ws)
    for rep in range(4):
        out.fill_(float("nan"))
        gg.k_codes.copy_(g0.k_codes)              # the step rewrites the token's slot: start each replay equal
        gg.v_codes.copy_(g0.v_codes)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}: output"
        assert torch.equal(gg.k_codes, ge.k_codes) and torch.equal(gg.v_codes, ge.v_codes), f"replay {rep}: cache"
        # eager work between replays, on another cache and the same workspace
        other = clone(g0)
        kvq.kvq_decode_step(other, k, v, q, lens, L, workspace=ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("bits", [(4, 4), (16, 16)])
def test_graph_replays_of_prefill(bits):
    kb, vb = bits
    B, Hq, Hkv, D, R, W, L, C = 2, 8, 2, 256, 1024, 512, 1500, 128
    print(f"graph prefill bits={bits}", flush=True)
    g, _ = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=611 + kb)
    q = q_dev(small_q_bits(612, (B, Hq, C, D), D ** -0.25))
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    nbytes = kvq.kvq_prefill_workspace_bytes(g, Hq, C, L)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    ref = kvq.kvq_attn_prefill_chunk(g, q, lens, L, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kvq.kvq_attn_prefill_chunk(g, q, lens, L, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kvq.kvq_attn_prefill_chunk(g, q, lens, L, out=out, workspace=ws)
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xA5)                            # stale workspace bytes between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        kvq.kvq_attn_prefill_chunk(g, q, lens, L, workspace=ws)             # eager work in between
        torch.cuda.synchronize()


def test_graph_replays_of_mixed_read():
    """A mixed read whose verify chunk runs in a launch of its own (three kernel
    launches: the decode reads, the short-chunk kernel, the combine)."""
    B, L = 2, 3000
    lens = torch.tensor([L, L - 7], dtype=torch.int32, device="cuda")
    specs = [(2, 256, 4, 8, 520, 512, 3, 8, 1), (1, 512, 8, 8, 4096, 0, 1, 8, 5)]
    reads = []
    for i, (Hkv, D, kb, vb, R, W, layers, Hq, C) in enumerate(specs):
        g, _ = make_pair(B, Hkv, D, kb, vb, R, W, L, seed=621 + i)
        qs = [q_dev(small_q_bits(622 + 10 * i + l, (B, Hq, C, D), D ** -0.25)) for l in range(layers)]
        reads.append(kvq.Read(g, qs, lens, L))
    print("graph mixed read", flush=True)
    ws = torch.empty(max(kvq.kvq_mixed_workspace_bytes(reads), 256), dtype=torch.uint8, device="cuda")
    refs = [[x.clone() for x in o] for o in kvq.kvq_attn_mixed(reads, workspace=ws)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kvq.kvq_attn_mixed(reads, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kvq.kvq_attn_mixed(reads, workspace=ws)
    for rep in range(4):
        for r in reads:
            for o in r.out:
                o.fill_(float("nan"))
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, r in enumerate(reads):
            for l, o in enumerate(r.out):
                assert torch.equal(o.view(torch.int16), refs[i][l].view(torch.int16)), f"replay {rep} read {i}.{l}"
        kvq.kvq_attn_mixed(reads, workspace=ws)                             # eager work in between
        torch.cuda.synchronize()
