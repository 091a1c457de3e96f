"""The library's calls inside a HIP graph (torch.cuda.CUDAGraph on the calls' stream): the streaming
kernel's in-kernel split sum (arrival counters left at zero by every replay), the fragment pass and wide
kernel, the forward streaming kernel, and the grouped backward and forward launches at M <= 16.  Each replay, with new input values copied in and eager calls
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
    cases = [("stream", 16, 3000, 512, 4), ("wide16", 600, 1024, 384, 1)]
    with torch.cuda.stream(st):
        ins = [_inputs(M, N, K, seed=600 + i) for i, (_, M, N, K, _) in enumerate(cases)]
        outs = [torch.empty((M, K), device="cuda") for (_, M, N, K, _) in cases]
        a_fwd = torch.randn((8, 1024), device="cuda")
        w_fwd = _inputs(8, 2048, 1024, seed=650)[1:]
        c_fwd = torch.empty((8, 2048), device="cuda")

        grp = [_inputs(16, N, K, seed=660 + i) for i, (N, K) in enumerate([(3000, 512), (700, 1344), (9000, 128)])]
        grp_out = [torch.empty((16, b.shape[1] * 2), device="cuda") for (g, s, b) in grp]
        fgrp = [(torch.randn((8, K), device="cuda"),) + tuple(_inputs(8, N, K, seed=680 + i)[1:])
                for i, (N, K) in enumerate([(2048, 1536), (520, 1344)])]
        fgrp_out = [torch.empty((8, s.shape[0]), device="cuda") for (a, s, b) in fgrp]

        def run():
            for (kern, M, N, K, sp), (g, s, b), o in zip(cases, ins, outs):
                lib.grad_a_forced(g, s, b, kern, rb=1 if kern == "wide16" else 0, splits=sp, out=o)
            lib.forward(a_fwd, *w_fwd, out=c_fwd, splits=3, kernel="stream")
            lib.grad_a_grouped(grp, outs=grp_out)
            lib.forward_grouped(fgrp, outs=fgrp_out)

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
        st.synchronize()
        graph.replay()
        st.synchronize()
        got = [o.clone() for o in outs + [c_fwd] + grp_out + fgrp_out]
        with torch.cuda.stream(st):
            run()  # eager on the same inputs and workspace
        st.synchronize()
        want = outs + [c_fwd] + grp_out + fgrp_out
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
    graph2.replay()
    st.synchronize()
    assert torch.equal(o.view(torch.int32), want.view(torch.int32))
