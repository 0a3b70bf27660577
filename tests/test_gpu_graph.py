"""The layer's calls captured in a HIP graph: every replay must reproduce the eager
result bit for bit (the kernels are deterministic), with eager work and host
synchronisation between replays."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    lay = synth.make_layer(w, seed=3, device="cuda", bias="zipf")
    xs = synth.make_tokens(w, T=4, seed=3, device="cuda")
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, 4)
    print("case graph decode T=1..4", flush=True)
    eager = []
    for T in (1, 4):
        eager.append(layer.forward(xs[:T]).clone())
    torch.cuda.synchronize()

    x_in = torch.empty_like(xs)
    x_in.copy_(xs)
    outs = [torch.empty((1, w.d), dtype=torch.bfloat16, device="cuda"),
            torch.empty((4, w.d), dtype=torch.bfloat16, device="cuda")]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x_in[:1], out=outs[0])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x_in[:1], out=outs[0])
        layer.forward(x_in[:4], out=outs[1])
    for rep in range(4):
        outs[0].zero_()
        outs[1].zero_()
        _ = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[0], eager[0]), rep
        assert torch.equal(outs[1], eager[1]), rep
    moe.moe_check_device_error()


@pytest.mark.parametrize("T", [300, 600])
def test_graph_replays_match_eager_prefill_path(T):
    # 300 tokens x top-10: the split router, the chunked grouping (3000 pairs), the GEMV for
    # the experts with few pairs and the grouped MFMA GEMM for the rest, and the combine;
    # 600 tokens: the bounded router (planes, MFMA logits, selection) and the GEMM alone
    # (6000 pairs); each inside one graph
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    lay = synth.make_layer(w, seed=5, device="cuda", bias="zipf")
    x = synth.make_tokens(w, T=T, seed=5, device="cuda")
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, T)
    print("case graph prefill T=%d" % T, flush=True)
    eager = layer.forward(x).clone()
    eager_ids = layer.ids[:T].clone()
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, out=out)
    for rep in range(4):
        out.zero_()
        layer.ids.zero_()
        _ = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        assert torch.equal(layer.ids[:T], eager_ids), rep
    moe.moe_check_device_error()


def test_graph_replays_match_eager_batched_decode():
    # 32 and 64 tokens x top-10 (320 / 640 pairs): the split router GEMV and its selection
    # kernel, the one-block grouping, the chunk list and the GEMV in sorted mode, and the
    # combine, all inside one graph; then the decode layer at 6 tokens
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_sparse_moe_router_amd as moe
    w = synth.WORKLOADS["decode_d2048_e512_top10_t1"]
    lay = synth.make_layer(w, seed=6, device="cuda", bias="zipf")
    xs = synth.make_tokens(w, T=64, seed=6, device="cuda")
    layer = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, 64)
    small = moe.MoeLayer(lay.router, lay.routed, lay.shared, w.k, 6)
    assert small.can_decode and not layer.can_decode
    print("case graph batched decode T=32, 64, 6", flush=True)
    eager = [layer.forward(xs[:32]).clone(), layer.forward(xs).clone(),
             small.decode(xs[:6]).clone()]
    torch.cuda.synchronize()
    moe.moe_check_device_error()
    outs = [torch.empty((T, w.d), dtype=torch.bfloat16, device="cuda") for T in (32, 64, 6)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(xs[:32], out=outs[0])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(xs[:32], out=outs[0])
        layer.forward(xs, out=outs[1])
        small.decode(xs[:6], out=outs[2])
    for rep in range(4):
        for o in outs:
            o.zero_()
        _ = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(outs[i], eager[i]), (rep, i)
    moe.moe_check_device_error()
