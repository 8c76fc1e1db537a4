"""The forward, decode and backward entry points can be captured in a HIP graph
(through torch.cuda.CUDAGraph) when the caller provides outputs and workspaces:
nothing on the path allocates or clears memory once the RoPE table exists (the
first eager call creates it).  Each replay is compared bit for bit with the
eager results, with eager work on the same buffers between the replays."""

import math

import numpy as np
import pytest

import workloads as W
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def test_fwd_decode_bwd_replay_in_a_graph():
    import torch
    B, Hq, Hkv, N, d = 1, 8, 2, 300, 128
    q = dev(W.normal((B, Hq, N, d), 13001, 1.0, "bf16"))
    k = dev(W.normal((B, Hkv, N, d), 13002, 1.0, "bf16"))
    v = dev(W.normal((B, Hkv, N, d), 13003, 1.0, "bf16"))
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(esd.fwd_workspace_bytes(B, Hkv, N, d, 1e4, esd.ATTN_BF16), dtype=torch.uint8,
                     device="cuda")
    w4 = W.WORKLOADS["decode_b32"]
    lens = np.array([5, 700, 2100, 4097], dtype=np.int32)
    qd, kc, vc = W.decode_inputs(w4, lens, Hq=8, Hkv=2, max_len=4100, d=d, seed_base=13100)
    qd, kc, vc, dl = dev(qd), dev(kc), dev(vc), dev(lens)
    od = torch.empty((len(lens), 8, d), dtype=torch.float32, device="cuda")
    ld = torch.empty((len(lens), 8), dtype=torch.float32, device="cuda")
    wsd = torch.empty(esd.decode_workspace_bytes(len(lens), 8, 2, 4100, d), dtype=torch.uint8,
                      device="cuda")

    do = dev(W.normal((B, Hq, N, d), 13004, 1.0, "f32"))
    gq = torch.empty((B, Hq, N, d), dtype=torch.float32, device="cuda")
    gk = torch.empty((B, Hkv, N, d), dtype=torch.float32, device="cuda")
    gv = torch.empty((B, Hkv, N, d), dtype=torch.float32, device="cuda")
    wsb = torch.empty(esd.bwd_workspace_bytes(B, Hq, Hkv, N, N, d, 1e4, esd.ATTN_BF16),
                      dtype=torch.uint8, device="cuda")
    outs = (o, lse, od, ld, gq, gk, gv)

    def work():
        esd.fwd(q, k, v, True, 1 / math.sqrt(d), 1e4, out=o, lse=lse, workspace=ws)
        esd.decode(qd, kc, vc, dl, scale=1 / math.sqrt(d), out=od, lse=ld, workspace=wsd)
        esd.bwd(q, k, v, o, lse, do, True, 1 / math.sqrt(d), 1e4, dq=gq, dk=gk, dv=gv,
                workspace=wsb)

    # eager reference (also creates the RoPE table outside the capture)
    work()
    torch.cuda.synchronize()
    ref = [host(x).copy() for x in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))  # eager work on the same buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(x) for x in outs]
        same = all(np.array_equal(a, b) for a, b in zip(got, ref))
        say(f"graph replay {rep}: {'identical to eager' if same else 'DIFFERENT'}")
        assert same


def test_concurrent_calls_from_threads():
    """Four host threads call attn_fwd at once, each on its own stream with its
    own buffers and a RoPE base no call has used yet (so the fp64 tables are
    created concurrently, under the library's lock); each result equals the same
    call made alone."""
    import threading
    import torch
    B, Hq, Hkv, N, d = 1, 4, 2, 200, 64
    bases = [1111.0, 2222.0, 3333.0, 4444.0]
    ins = [tuple(dev(W.normal(s, 13200 + 10 * i + t, 1.0, "bf16"))
                 for t, s in enumerate([(B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)]))
           for i in range(len(bases))]
    results = [None] * len(bases)
    errors = []

    def run(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                o, l = esd.fwd(*ins[i], True, 1 / math.sqrt(d), bases[i])
            s.synchronize()
            results[i] = (host(o), host(l))
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(bases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, base in enumerate(bases):
        o, l = esd.fwd(*ins[i], True, 1 / math.sqrt(d), base)
        torch.cuda.synchronize()
        assert np.array_equal(results[i][0], host(o)) and np.array_equal(results[i][1], host(l))
    say("concurrent calls from 4 threads: identical to serial calls")


def test_rope_table_not_built_inside_a_capture():
    """A RoPE call whose table does not exist yet, made while its stream is being
    captured, returns an error (the table would need blocking copies) and leaves
    the capture intact: the rest of the graph replays like the eager calls."""
    import torch
    B, Hq, Hkv, N, d = 1, 4, 2, 150, 128
    q = dev(W.normal((B, Hq, N, d), 13301, 1.0, "bf16"))
    k = dev(W.normal((B, Hkv, N, d), 13302, 1.0, "bf16"))
    v = dev(W.normal((B, Hkv, N, d), 13303, 1.0, "bf16"))
    o = torch.empty((B, Hq, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o)
    ws = torch.empty(esd.fwd_workspace_bytes(B, Hkv, N, d, 9876.5, esd.ATTN_BF16),
                     dtype=torch.uint8, device="cuda")
    esd.fwd(q, k, v, True, 1 / math.sqrt(d), 0.0, out=o, lse=lse)
    torch.cuda.synchronize()
    ref = (host(o).copy(), host(lse).copy())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        with pytest.raises(esd.AttnError):
            # base 9876.5 has no table yet
            esd.fwd(q, k, v, True, 1 / math.sqrt(d), 9876.5, out=o2, workspace=ws)
        esd.fwd(q, k, v, True, 1 / math.sqrt(d), 0.0, out=o, lse=lse)
    o.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(host(o), ref[0]) and np.array_equal(host(lse), ref[1])
    # outside the capture the same call builds the table and runs
    esd.fwd(q, k, v, True, 1 / math.sqrt(d), 9876.5, out=o2, workspace=ws)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(o2)))
    say("RoPE table refused inside a capture; the graph replays; built afterwards")
