"""The library's calls captured into HIP graphs (torch.cuda.CUDAGraph on ROCm),
as the benchmark replays them.

Each call is captured once with static buffers and replayed several times,
with eager work of the program's own and a synchronization between replays.
Every replay must equal the eager result bit for bit, also after the input
changes between replays (a graph reads its inputs when it runs). The paths
covered: the one-token and few-token decode kernels, the prefill kernel with
split-K partial sums and their finishing kernel, the gated gate|up kernel, the
decoder chain at one token (the fused projections) and at 64 tokens (the
quantize -> contract chain with split partials), and the cached decoder with
RoPE, the cache append and attention.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from ternary_weight_bitlinear_w1_amd import bitlinear as bl
from ternary_weight_bitlinear_w1_amd import synth

from _cases import EPS, Matrix, assert_equal, note, seed

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
REPLAYS = 3


def gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _stream():
    return torch.cuda.current_stream(DEV).cuda_stream


def _capture(call):
    call()  # first launch outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def _check_replays(graph, call, inputs, outputs, fresh):
    """Replays against eager runs: before replay i the inputs get new values
    (fresh(i)), the eager call computes the expected outputs, the outputs are
    overwritten with garbage by eager work, then the graph runs."""
    for i in range(REPLAYS):
        for t, v in zip(inputs, fresh(i)):
            t.copy_(v)
        call()
        expect = [host(o).copy() for o in outputs]
        for o in outputs:
            o.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        for o, e in zip(outputs, expect):
            assert_equal(host(o), e, f"replay {i}")


def _forward_call(packed, k, gammas, ends, x, y, path, m):
    L = bl.lib()
    n = packed.shape[0]
    g = (ctypes.c_float * len(gammas))(*gammas)
    se = (ctypes.c_int64 * len(ends))(*ends)
    nb = L.bitlinear_forward_workspace_bytes(m, n, k, 1)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)

    def call():
        st = L.bitlinear_forward(x.data_ptr(), None, None, None, m, k, packed.data_ptr(), n, g, se, len(gammas),
                                 y.data_ptr(), None, path, ws.data_ptr(), nb, _stream())
        assert st == 0, L.bitlinear_last_error()
    return call, ws


# 1, 4 and 16 tokens on the decode kernels; 64 tokens with few tiles (split K
# and the finishing kernel); 300 tokens on the pipelined tile
@pytest.mark.parametrize("m,n,k,path", [(1, 1024, 2560, bl.PATH_DECODE), (4, 1024, 2560, bl.PATH_DECODE),
                                        (16, 768, 1024, bl.PATH_DECODE), (64, 512, 2560, bl.PATH_PREFILL),
                                        (300, 768, 512, bl.PATH_PREFILL)])
def test_graph_forward(m, n, k, path):
    note(f"graph forward m={m} n={n} k={k} path={path}")
    mats = [Matrix(n // 2, k, seed(40, n, 1)), Matrix(n - n // 2, k, seed(40, n, 2))]
    packed = torch.cat([gpu(oracle.pack(mt.codes)) for mt in mats])
    gammas = [float(np.float32(mt.gamma)) for mt in mats]
    ends = [n // 2, n]
    x = torch.empty((m, k), dtype=torch.float32, device=DEV)
    y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    x.copy_(gpu(synth.activations(seed(40, m, 0), m, k, 2)))
    call, _ws = _forward_call(packed, k, gammas, ends, x, y, path, m)
    graph = _capture(call)
    fresh = lambda i: [gpu(synth.activations(seed(40, m, 1 + i), m, k, 2))]
    _check_replays(graph, call, [x], [y], fresh)
    # the last replay also against the oracle
    ref = oracle.forward(host(x), np.concatenate([mt.codes for mt in mats]), [mt.gamma for mt in mats], ends)
    assert_equal(host(y), ref["y"], "last replay against the oracle")


def test_graph_forward_relu2_glu():
    m, inter, k = 256, 512, 1024
    note(f"graph gated gate|up m={m} inter={inter} k={k}")
    mats = [Matrix(inter, k, seed(41, 0, 1)), Matrix(inter, k, seed(41, 0, 2))]
    packed = torch.cat([gpu(oracle.pack(mt.codes)) for mt in mats])
    g = (ctypes.c_float * 2)(*[float(np.float32(mt.gamma)) for mt in mats])
    x = gpu(synth.activations(seed(41, m, 0), m, k, 2))
    y = torch.empty((m, inter), dtype=torch.float32, device=DEV)
    L = bl.lib()
    nb = L.bitlinear_forward_relu2_glu_workspace_bytes(m, inter, k, 1, bl.PATH_PREFILL)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)

    def call():
        st = L.bitlinear_forward_relu2_glu(x.data_ptr(), None, None, None, m, k, packed.data_ptr(), inter, g,
                                           y.data_ptr(), bl.PATH_PREFILL, ws.data_ptr(), nb, _stream())
        assert st == 0, L.bitlinear_last_error()
    graph = _capture(call)
    _check_replays(graph, call, [x], [y], lambda i: [gpu(synth.activations(seed(41, m, 1 + i), m, k, 2))])


def _decoder_spec(kind, hdim, inter, nh, nkv, hd, layers, **kw):
    kvd = nkv * hd
    lws = []
    for l in range(layers):
        mt = [Matrix(n, kk, seed(42, l, i)) for i, (n, kk) in enumerate(
            ((hdim, hdim), (kvd, hdim), (kvd, hdim), (hdim, hdim), (inter, hdim), (inter, hdim), (hdim, inter)))]
        pk = lambda ms: torch.cat([gpu(oracle.pack(a.codes)) for a in ms])
        f = lambda a: float(np.float32(a.gamma))
        lws.append(bl.LayerWeights(qkv=pk(mt[0:3]), qkv_gamma=[f(a) for a in mt[0:3]], o=pk(mt[3:4]),
                                   o_gamma=f(mt[3]), gate_up=pk(mt[4:6]), gate_up_gamma=[f(a) for a in mt[4:6]],
                                   down=pk(mt[6:7]), down_gamma=f(mt[6])))
    return lws, (lambda: bl.BlockSpec(kind, hdim, inter, lws, nh, nkv, hd, EPS, **kw))


@pytest.mark.parametrize("m", [1, 64])
def test_graph_decoder_stack(m):
    hdim, inter, nh, nkv, hd, layers = 512, 1024, 4, 1, 128, 2
    note(f"graph decoder stack m={m}")
    _lws, make = _decoder_spec(bl.BLOCK_DECODER, hdim, inter, nh, nkv, hd, layers)
    spec = make()
    x = gpu(synth.activations(seed(43, m, 0), m, hdim, 1))
    y = torch.empty_like(x)
    blk, _keep = spec.to_c()
    nb = int(bl.lib().bitlinear_block_workspace_bytes(ctypes.byref(blk), m))
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)
    call = lambda: bl.block_forward(spec, x, out=y, workspace=ws)
    graph = _capture(call)
    _check_replays(graph, call, [x], [y], lambda i: [gpu(synth.activations(seed(43, m, 1 + i), m, hdim, 1))])


@pytest.mark.parametrize("m", [1, 4])
def test_graph_cached_decoder_step(m):
    """One decode step of the cached decoder (RoPE, the cache append, attention)
    at position p: replaying it appends the same rows again, so the caches after
    every replay equal those after the eager step."""
    hdim, inter, nh, nkv, hd, layers, tmax = 512, 768, 4, 1, 128, 2, 256
    note(f"graph cached decoder m={m}")
    r = np.random.default_rng(44 + m)
    slot = gpu(np.arange(m, dtype=np.int64))
    pos = gpu(np.array([37 + 50 * i for i in range(m)], dtype=np.int64))
    table = bl.rope_table(5e5, hd, 4096, DEV)
    lws, make = _decoder_spec(bl.BLOCK_DECODER_CACHED, hdim, inter, nh, nkv, hd, layers, slot=slot, pos=pos,
                              rope_table=table)
    caches0 = []
    for lw in lws:
        kc = gpu(oracle.round_bf16(r.normal(size=(m, nkv, tmax, hd)).astype(np.float32)).view(np.uint16))
        vc = gpu(oracle.round_bf16(r.normal(size=(m, nkv, tmax, hd)).astype(np.float32)).view(np.uint16))
        lw.k_cache, lw.v_cache = kc, vc
        caches0.append((kc.clone(), vc.clone()))
    spec = make()
    x = gpu(synth.activations(seed(44, m, 0), m, hdim, 1))
    y = torch.empty_like(x)
    blk, _keep = spec.to_c()
    nb = int(bl.lib().bitlinear_block_workspace_bytes(ctypes.byref(blk), m))
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=DEV)

    def reset_caches():
        for lw, (kc, vc) in zip(lws, caches0):
            lw.k_cache.copy_(kc)
            lw.v_cache.copy_(vc)

    call = lambda: bl.block_forward(spec, x, out=y, workspace=ws)
    graph = _capture(call)
    for i in range(REPLAYS):
        x.copy_(gpu(synth.activations(seed(44, m, 1 + i), m, hdim, 1)))
        reset_caches()
        call()
        expect = [host(y).copy()] + [host(t).copy() for lw in lws for t in (lw.k_cache, lw.v_cache)]
        reset_caches()
        y.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        got = [host(y)] + [host(t) for lw in lws for t in (lw.k_cache, lw.v_cache)]
        for j, (a, b) in enumerate(zip(got, expect)):
            assert_equal(a, b, f"replay {i}, output {j}")
