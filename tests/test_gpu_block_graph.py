"""A transformer block's sequence of library calls (the AWQ modulation
projection, the QKV and output projections, the fused MLP pair) captured in
a HIP graph and replayed: every replay, with the program's own eager work
and synchronisations between replays, gives the eager result bit for bit
(the kernels sum in a fixed order, so a replay is exactly reproducible).
Small shapes with ragged tails."""
import numpy as np
import pytest
import torch

import synth
from tests.conftest import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import w4a4_rank_corrected_smooth_amd as lib
    lib.device_check()
    return lib


def layer(S, seed, N, K, rank, ax=None):
    c = synth.linear_case(f"blk{seed}", seed, 8, N, K, rank)
    return S.Linear(S.prepare_weights(c.W, ax, c.bias, rank))


def test_block_sequence_replays_exactly(S):
    M, D, F = 300, 320, 640
    dev = torch.device("cuda")
    announce(f"block graph M={M} d={D} ff={F}: preparing layers")
    a = synth.awq_case(m_max=1, N=6 * D, K=D, seed=41)
    q, s, z = S.awq_quantize_weights(a.W)
    awq = S.AwqLinear(q, s, z, dev)
    qkv, out = layer(S, 42, 3 * D, D, 16), layer(S, 43, D, D, 16)
    fc1, fc2 = layer(S, 44, F, D, 16), layer(S, 45, D, F, 16)
    x = torch.from_numpy(np.ascontiguousarray(a.x[:1])).to(dev)
    X = torch.randn(M, D, device=dev).to(torch.bfloat16)
    H = torch.randn(M, D, device=dev).to(torch.bfloat16)
    mod = torch.empty(1, 6 * D, dtype=torch.float16, device=dev)
    Yq = torch.empty(M, 3 * D, dtype=torch.bfloat16, device=dev)
    Yo = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    Ym = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    wq, wo = qkv.new_workspace(M), out.new_workspace(M)
    w1, w2 = fc1.new_workspace(M), fc2.new_workspace(M)

    def block():
        S.awq_forward(awq, x, out=mod)
        S.linear_forward(qkv, X, out=Yq, workspace=wq)
        S.linear_forward(out, H, out=Yo, workspace=wo)
        S.mlp_forward(fc1, fc2, X, out=Ym, ws1=w1, ws2=w2)

    announce("block graph: eager reference")
    block()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (mod, Yq, Yo, Ym)]
    announce("block graph: capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        block()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        block()
    torch.cuda.synchronize()
    for rep in range(4):
        announce(f"block graph: replay {rep}")
        for t in (mod, Yq, Yo, Ym):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((mod, Yq, Yo, Ym), ref):
            assert torch.equal(got, want), f"replay {rep} differs from the eager result"
        # eager work of the program's own between replays
        S.linear_forward(qkv, H, out=Yq, workspace=wq)
        torch.cuda.synchronize()
