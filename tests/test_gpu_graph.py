"""Calls captured in a HIP graph stay correct on every replay: the quantiser's
call counter lives in the workspace (device memory), not in the captured
launch arguments.  Each replay runs on a new input copied in eagerly between
replays and is checked against the oracle (quantiser) or the eager call."""

import numpy as np
import pytest
import torch

import bit_block_scaled_amd as nv
import oracle
import workloads
from gpu_helpers import announce, bf16_to_dev, to_np

pytestmark = pytest.mark.gpu


def _inputs(n, M, K):
    return [workloads.random_matrix(60 + i, M, K, sigma=0.5 + i, outliers=(i % 2 == 0)) for i in range(n)]


@pytest.mark.parametrize("M,K", [(1024, 3072), (24 * 100, 128)])
def test_quantize_graph_replays(M, K):
    announce(f"graph replay of quantize {M}x{K}")
    xs = _inputs(4, M, K)
    x = bf16_to_dev(xs[0])
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty((1,), dtype=torch.float32, device=x.device)
    ws = nv.workspace(nv.quantize_workspace_bytes(M, K), x.device)
    nv.quantize_into(x, codes, scales, g, ws)                 # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.quantize_into(x, codes, scales, g, ws)
    torch.cuda.synchronize()
    for r, xb in enumerate(xs + xs[:1]):
        x.copy_(bf16_to_dev(xb))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        rc, rs, rg = oracle.quantize(xb)
        assert to_np(g)[0] == rg, r
        assert np.array_equal(to_np(scales), rs) and np.array_equal(to_np(codes), rc), r


def test_linear_and_linear_q_graph_replays():
    M, N, K = 512, 1024, 768
    announce(f"graph replay of linear / linear_q {M}x{N}x{K}")
    xs = _inputs(3, M, K)
    wq = nv.quantize(bf16_to_dev(workloads.random_matrix(70, N, K, 0.02)))
    x = bf16_to_dev(xs[0])
    out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    lws = nv.workspace(nv.linear_workspace_bytes(M, K), x.device)
    hq = (torch.empty((M, N // 2), dtype=torch.uint8, device=x.device),
          torch.empty((M, N // 16), dtype=torch.uint8, device=x.device),
          torch.empty((1,), dtype=torch.float32, device=x.device))
    qws = nv.workspace(nv.linear_q_workspace_bytes(M, N, K), x.device)
    nv.linear(x, *wq, gelu=True, out=out, ws=lws)
    nv.linear_q(x, *wq, gelu=True, out=hq, ws=qws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nv.linear(x, *wq, gelu=True, out=out, ws=lws)
        nv.linear_q(x, *wq, gelu=True, out=hq, ws=qws)
    torch.cuda.synchronize()
    for r, xb in enumerate(xs + xs[:1]):
        x.copy_(bf16_to_dev(xb))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = nv.linear(x, *wq, gelu=True)                     # eager, fresh workspace
        wq_h = nv.quantize(want)
        torch.cuda.synchronize()
        assert torch.equal(out, want), r
        for a, b in zip(hq, wq_h):
            assert torch.equal(a, b), r


def test_kv_append_and_dequant_graph_replays():
    # a captured append writes the token range current at capture time on
    # every replay; its tensor scales and codes must follow each replay's input
    H, D, T = 24, 128, 64
    announce("graph replay of kv append + dequant")
    rng = np.random.default_rng(80)
    ks = [workloads.to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32) * (1 + 3 * i))
          for i in range(3)]
    vs = [workloads.to_bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32) / (1 + i))
          for i in range(3)]
    kd, vd = bf16_to_dev(ks[0]), bf16_to_dev(vs[0])
    kv = nv.KVCache(T, H, D, max_chunks=1)
    ko = torch.empty((T, H, D), dtype=torch.bfloat16, device=kd.device)
    vo = torch.empty_like(ko)
    kv.append(kd, vd)
    kv.dequant(0, T, ko, vo)
    torch.cuda.synchronize()
    kv.reset()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kv.append(kd, vd)
        kv.dequant(0, T, ko, vo)
    torch.cuda.synchronize()
    for r in range(4):
        kd.copy_(bf16_to_dev(ks[r % 3]))
        vd.copy_(bf16_to_dev(vs[r % 3]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.KVCacheRef(T, H, D)
        ref.append(ks[r % 3], vs[r % 3])
        assert np.array_equal(to_np(kv.k_codes), ref.k_codes) and np.array_equal(to_np(kv.v_scales), ref.v_scales), r
        rk, rv = ref.dequant(0, T)
        assert np.array_equal(to_np(ko.view(torch.int16)).view(np.uint16), rk), r
        assert np.array_equal(to_np(vo.view(torch.int16)).view(np.uint16), rv), r
