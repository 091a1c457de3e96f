"""The library's calls inside a HIP graph (torch.cuda.CUDAGraph on the calls' stream): the streaming
kernel's in-kernel split sum (arrival counters left at zero by every replay), the fragment pass with the
512-, 256- (split, with the reduce kernel) and 128-row tile kernels, the forward streaming kernel and a
split forward on 256-row tiles, the grouped backward and forward launches at M <= 16, and a grouped forward
at M > 16 with a shared conversion of the activations.  Each replay, with new input values copied in and eager calls
on the same workspace between replays, is compared bitwise with an eager call on the same inputs.  The
workspace is allocated by an eager call before capture, so nothing is allocated inside the graph."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(M, N, K, seed):
    b = synth.random_code_bytes(N, K, seed)
    s = synth.random_scales_uniform(N, K, seed + 1)
    g = synth.grad_out_normal(M, N, seed + 2)
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in (g, s, b)]


def test_calls_in_a_graph_match_eager(lib):
    st = torch.cuda.Stream()
    cases = [("stream", 16, 3000, 512, 4), ("wide16", 600, 1024, 384, 1), ("mid", 300, 2048, 384, 2),
             ("small", 200, 1024, 256, 1)]
    with torch.cuda.stream(st):
        ins = [_inputs(M, N, K, seed=600 + i) for i, (_, M, N, K, _) in enumerate(cases)]
        outs = [torch.empty((M, K), device="cuda") for (_, M, N, K, _) in cases]
        a_fwd = torch.randn((8, 1024), device="cuda")
        w_fwd = _inputs(8, 2048, 1024, seed=650)[1:]
        c_fwd = torch.empty((8, 2048), device="cuda")
        # tile-kernel forward (256-row tiles, K split in 2: partials and reduce) and, at M > 16, a grouped
        # forward whose first two problems share one conversion of their activations
        a_tile = torch.randn((300, 1024), device="cuda")
        w_tile = _inputs(300, 512, 1024, seed=655)[1:]
        c_tile = torch.empty((300, 512), device="cuda")
        a_shared = torch.randn((200, 448), device="cuda")
        tgrp = [(a_shared,) + tuple(_inputs(8, N, 448, seed=690 + i)[1:]) for i, N in enumerate([512, 128])]
        tgrp.append((torch.randn((200, 320), device="cuda"),) + tuple(_inputs(8, 264, 320, seed=695)[1:]))
        tgrp_out = [torch.empty((200, s.shape[0]), device="cuda") for (a, s, b) in tgrp]

        grp = [_inputs(16, N, K, seed=660 + i) for i, (N, K) in enumerate([(3000, 512), (700, 1344), (9000, 128)])]
        grp_out = [torch.empty((16, b.shape[1] * 2), device="cuda") for (g, s, b) in grp]
        fgrp = [(torch.randn((8, K), device="cuda"),) + tuple(_inputs(8, N, K, seed=680 + i)[1:])
                for i, (N, K) in enumerate([(2048, 1536), (520, 1344)])]
        fgrp_out = [torch.empty((8, s.shape[0]), device="cuda") for (a, s, b) in fgrp]

        def run():
            for (kern, M, N, K, sp), (g, s, b), o in zip(cases, ins, outs):
                lib.grad_a_forced(g, s, b, kern, rb=0 if kern == "stream" else 1, splits=sp, out=o)
            lib.forward(a_fwd, *w_fwd, out=c_fwd, splits=3, kernel="stream")
            lib.forward(a_tile, *w_tile, out=c_tile, splits=2, kernel="mid")
            lib.grad_a_grouped(grp, outs=grp_out)
            lib.forward_grouped(fgrp, outs=fgrp_out)
            lib.forward_grouped(tgrp, outs=tgrp_out)

        run()  # eager: allocates the stream's workspace before capture
    st.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        run()
    for rep in range(4):
        with torch.cuda.stream(st):
            for i, (_, M, N, K, _) in enumerate(cases):
                fresh = _inputs(M, N, K, seed=700 + 10 * rep + i)
                for dst, src in zip(ins[i], fresh):
                    dst.copy_(src)
            a_fwd.copy_(torch.randn((8, 1024), device="cuda"))
            a_tile.copy_(torch.randn((300, 1024), device="cuda"))
            a_shared.copy_(torch.randn((200, 448), device="cuda"))
        st.synchronize()
        # the replay, the copies of its results and the eager calls all on the capture stream: a replay
        # uses that stream's workspace, so it must not overlap the eager calls
        with torch.cuda.stream(st):
            graph.replay()
        st.synchronize()
        with torch.cuda.stream(st):
            got = [o.clone() for o in outs + [c_fwd, c_tile] + grp_out + fgrp_out + tgrp_out]
            run()  # eager on the same inputs and workspace
        st.synchronize()
        want = outs + [c_fwd, c_tile] + grp_out + fgrp_out + tgrp_out
        for k, (x, y) in enumerate(zip(got, want)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (rep, k)


def test_capture_that_would_grow_the_workspace_is_refused(lib):
    """A call whose stream is capturing and whose workspace would have to grow returns NF4_ERR_CAPTURE and
    enqueues nothing (the graph stays valid); once an eager call has sized the workspace, the same call can be
    captured and its replay matches eager."""
    lib.release_workspaces()  # every stream starts without a workspace
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        g, s, b = _inputs(16, 3000, 512, seed=900)
        o = torch.empty((16, 512), device="cuda")
        x = torch.zeros(4, device="cuda")
    st.synchronize()
    graph = torch.cuda.CUDAGraph()
    raised = None
    with torch.cuda.graph(graph, stream=st):
        try:
            lib.grad_a_forced(g, s, b, "stream", rb=0, splits=4, out=o)
        except lib.Nf4Error as e:
            raised = e
        x.add_(1.0)
    assert raised is not None and raised.status == lib.NF4_ERR_CAPTURE, raised
    with torch.cuda.stream(st):
        graph.replay()
    st.synchronize()
    assert torch.equal(x, torch.ones(4, device="cuda"))
    with torch.cuda.stream(st):
        lib.grad_a_forced(g, s, b, "stream", rb=0, splits=4, out=o)  # eager: sizes the workspace
    st.synchronize()
    want = o.clone()
    o.fill_(float("nan"))
    torch.cuda.synchronize()
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2, stream=st):
        lib.grad_a_forced(g, s, b, "stream", rb=0, splits=4, out=o)
    with torch.cuda.stream(st):
        graph2.replay()
    st.synchronize()
    assert torch.equal(o.view(torch.int32), want.view(torch.int32))
