"""The entry points under HIP graph capture (torch.cuda.graph): they
allocate nothing, synchronize nothing and record no memset, so a captured
forward+backward replays with the eager results.  Each replay is checked bit
for bit against the eager run, with eager work and synchronizations between
replays."""
import pytest

from bwd_bn_stats_amd import workloads as wl

from helpers import dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nh():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bwd_bn_stats_amd import normhip
    return normhip


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_graph_replays_match_eager(nh):
    c = wl.bn_ragged()
    x, dy, g, b = dev(c.x), dev(c.dy), dev(c.gamma), dev(c.beta)
    r = wl.ln_bwd(rows=1024)
    lx, ldy, lw, lb = dev(r.x), dev(r.dy), dev(r.w), dev(r.b)
    m = wl.rms_bwd(wl.BF16, rows=256)
    mx, mdy, mw = dev(m.x), dev(m.dy), dev(m.w)
    ws_bn = torch.empty(nh.bn_forward_train_workspace(c.N, c.C, c.hw), dtype=torch.uint8, device="cuda")
    ws_ln = torch.empty(nh.layernorm_backward_workspace(r.rows, r.cols), dtype=torch.uint8, device="cuda")
    ws_rms = torch.empty(nh.rmsnorm_backward_workspace(m.rows, m.cols), dtype=torch.uint8, device="cuda")
    outs = {}

    def work():
        y, stats = nh.bn_forward_train(x, g, b, act="relu", workspace=ws_bn)
        dx, grads = nh.bn_backward(dy, x, stats, beta=b, act="relu", workspace=ws_bn)
        ly, mean, rstd = nh.layernorm_forward(lx, lw, lb, 1e-5)
        ldx, ldw, ldb = nh.layernorm_backward(ldy, lx, mean, rstd, lw, dx_dtype=torch.float32,
                                              workspace=ws_ln)
        my, rms = nh.rmsnorm_forward(mx, mw, 1e-5)
        mdx, mdw = nh.rmsnorm_backward(mdy, mx, rms, mw, 1e-5, workspace=ws_rms)
        return dict(y=y, stats=stats, dx=dx, grads=grads, ly=ly, mean=mean, rstd=rstd, ldx=ldx,
                    ldw=ldw, ldb=ldb, my=my, rms=rms, mdx=mdx, mdw=mdw)

    eager = work()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in eager.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()   # warm the caching allocator outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = work()
    print("[graph] captured BN+ReLU fwd/bwd, LN fwd/bwd, RMS fwd/bwd", flush=True)
    for rep in range(3):
        # unrelated eager work between replays overwrites the inputs' neighbours
        scratch = torch.randn(1 << 20, device="cuda") * rep
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert torch.equal(_bits(outs[k]), _bits(v)), f"replay {rep}: {k} differs from eager"
        del scratch
    print("[graph] 3 replays bit-identical to eager", flush=True)


def test_graph_generic_rows(nh):
    """The generic row kernels under capture: misaligned rows (coefficient
    and strip kernels), short odd rows (narrow kernels) and rows wider than
    the vector path, forward and backward, replayed against eager bits."""
    from helpers import place
    wide = wl.rows_case(64, 20000, x_t=wl.BF16, dy_t=wl.BF16, w_t=wl.BF16, seed=31, with_bias=True)
    odd = wl.rows_case(3000, 1601, x_t=wl.F32, dy_t=wl.F32, w_t=wl.F32, seed=32, with_bias=True)
    short = wl.rows_case(5000, 7, x_t=wl.F32, dy_t=wl.F32, w_t=wl.F32, seed=33, with_bias=True)
    sets = []
    for c, off in ((wide, 0), (odd, 1), (short, 1)):
        sets.append(dict(x=place(c.x, off), dy=place(c.dy, off), w=place(c.w, off), b=place(c.b, off),
                         ws=torch.empty(nh.layernorm_backward_workspace(c.rows, c.cols), dtype=torch.uint8,
                                        device="cuda"),
                         wsr=torch.empty(nh.rmsnorm_backward_workspace(c.rows, c.cols), dtype=torch.uint8,
                                         device="cuda")))

    def work():
        out = {}
        for i, t in enumerate(sets):
            y, mean, rstd = nh.layernorm_forward(t["x"], t["w"], t["b"], 1e-5)
            dx, dw, db = nh.layernorm_backward(t["dy"], t["x"], mean, rstd, t["w"], dx_dtype=torch.float32,
                                               workspace=t["ws"])
            ry, rms = nh.rmsnorm_forward(t["x"], t["w"], 1e-5)
            rdx, rdw = nh.rmsnorm_backward(t["dy"], t["x"], None, t["w"], 1e-5, workspace=t["wsr"])
            out.update({f"{k}{i}": v for k, v in dict(y=y, mean=mean, rstd=rstd, dx=dx, dw=dw, db=db, ry=ry,
                                                      rms=rms, rdx=rdx, rdw=rdw).items()})
        return out

    eager = {k: v.clone() for k, v in work().items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = work()
    for rep in range(3):
        scratch = torch.randn(1 << 20, device="cuda") * rep
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert torch.equal(_bits(outs[k]), _bits(v)), f"replay {rep}: {k} differs from eager"
        del scratch
    print("[graph] generic row kernels: 3 replays bit-identical to eager", flush=True)


@pytest.mark.parametrize("shape,io", [((20000, 64, 1, 1), wl.F32),    # many row chunks: XCD-ordered blocks
                                      ((64, 100, 7, 7), wl.BF16)])   # 7x7 planes: a wave per channel finalizes
def test_graph_bn_row_layout(nh, shape, io):
    """The BatchNorm row layout (small planes, the tensor as [N, C*HW] rows)
    under capture: forward, backward and inference replay bit for bit."""
    N, C, H, W = shape
    c = wl.bn_case(N, C, H, W, io, seed=N + C, x_mean=1.0)
    x, dy, g, b = dev(c.x), dev(c.dy), dev(c.gamma), dev(c.beta)
    # fixed running statistics for inference; training runs without the
    # running update, so every replay repeats the same work
    rm = torch.full((C,), 0.5, device="cuda")
    rv = torch.full((C,), 1.5, device="cuda")
    ws = torch.empty(nh.bn_forward_train_workspace(N, C, H * W), dtype=torch.uint8, device="cuda")

    def work():
        y, stats = nh.bn_forward_train(x, g, b, act="relu", workspace=ws)
        dx, grads = nh.bn_backward(dy, x, stats, beta=b, act="relu", workspace=ws)
        yi = nh.bn_forward_infer(x, rm, rv, g, b, act="relu")
        return dict(y=y, stats=stats, dx=dx, grads=grads, yi=yi)

    eager = {k: v.clone() for k, v in work().items()}
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = work()
    print(f"[graph] captured BN row layout {shape} {io}", flush=True)
    for rep in range(3):
        scratch = torch.randn(1 << 20, device="cuda") * rep
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert torch.equal(_bits(outs[k]), _bits(v)), f"replay {rep}: {k} differs from eager"
        del scratch
