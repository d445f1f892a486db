"""GPU parity of the gated-MLP step and of a decoder block's seven projections on packed weights.

Each step of the block is checked against the oracle on the GPU's own inputs to that step
(sampled rows), so rounding of intermediates does not accumulate into the comparison.
"""
import numpy as np
import pytest
import torch

import oracle
import tile_gemm_amd as hts
import tile_gemm_amd.block as block
import workloads as wl
from helpers import DEV, activations, oracle_map, say, weight

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,pad", [(1, 8, 0), (37, 11008, 0), (256, 4096, 24)])
def test_silu_mul(dtype, M, N, pad):
    g = np.random.default_rng(M * 7 + N)
    G = wl.gaussian_bits((M, N + pad), 4.0, dtype, g)
    U = wl.gaussian_bits((M, N + pad), 1.0, dtype, g)
    G[:, :4] = wl.to_bits(np.array([0.0, -0.0, 30.0, -30.0], np.float32), dtype)   # zeros and saturation
    say(f"[silu_mul] {dtype} M={M} N={N} pad={pad}")
    Gt = hts.tensor_from_bits(G, dtype, DEV)[:, :N]
    Ut = hts.tensor_from_bits(U, dtype, DEV)[:, :N]
    Hbig = torch.full((M, N + 8), 3.0, dtype=Gt.dtype, device=DEV)
    H = Hbig[:, :N]
    hts.silu_mul(Gt, Ut, out=H)
    torch.cuda.synchronize()
    ref = oracle.silu_mul_ref(np.ascontiguousarray(G[:, :N]), np.ascontiguousarray(U[:, :N]), dtype)
    got = oracle.widen_f64(hts.bits_from_tensor(H), dtype)
    # one rounding of an fp32 result to the 16-bit type: 2^-8 relative (bf16) bounds both types,
    # plus the smallest f16 subnormal step for results near zero
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -24)
    assert torch.all(Hbig[:, N:] == 3.0)


def _weights(c, M, hybrid):
    out = {}
    for L in c.layers:
        W = weight(c.cfg_id, L.name)
        Wt = hts.tensor_from_bits(W, L.dtype, DEV)
        out[L.name] = hts.pack(Wt, oracle_map(c.cfg_id, L.name), L.bn, L.bk) if hybrid else Wt
    return out


def _masked(c, name):
    L = next(x for x in c.layers if x.name == name)
    return oracle.masked_weights(weight(c.cfg_id, name), L.dtype, oracle_map(c.cfg_id, name), L.bn, L.bk)


@pytest.mark.parametrize("hybrid", [True, False])
def test_block_step_parity(hybrid):
    # the block at its workload's M = 2048, every element of every output
    c = wl.config("7b_block")
    M = 2048
    say(f"[block] hybrid={hybrid} M={M}")
    W = _weights(c, M, hybrid)
    X = activations(c.cfg_id, "q")[:M]
    Xt = hts.tensor_from_bits(np.ascontiguousarray(X), "bf16", DEV)
    bufs = block.buffers(M, W, Xt.dtype, DEV)
    block.forward(Xt, W, bufs)
    torch.cuda.synchronize()
    rows = np.arange(M)
    bits = {k: hts.bits_from_tensor(v) for k, v in bufs.items()}
    weights_m = {L.name: (_masked(c, L.name) if hybrid else weight(c.cfg_id, L.name)) for L in c.layers}
    inputs = {"q": X, "k": X, "v": X, "gate": X, "up": X, "o": bits["q"], "down": bits["h"]}
    for name in block.PROJECTIONS:
        ref = oracle.gemm_ref(inputs[name][rows], weights_m[name], "bf16")
        got = oracle.widen_f64(bits[name][rows], "bf16")
        ok, rel = oracle.within_tolerance(got, ref, TOL)
        assert ok, f"{name}: {rel:.3e}"
    h_ref = oracle.silu_mul_ref(bits["gate"][rows], bits["up"][rows], "bf16")
    got = oracle.widen_f64(bits["h"][rows], "bf16")
    assert np.all(np.abs(got - h_ref) <= 2.0 ** -8 * np.abs(h_ref) + 2.0 ** -24)


def test_block_step_fused_gate_parity():
    # the up product writes silu(gate) * up in its output stage: h against the oracle's gated step
    # on the unrounded up product, and the down projection against h
    c = wl.config("7b_block")
    M = 2048
    say(f"[block-fused] M={M}")
    W = _weights(c, M, True)
    X = activations(c.cfg_id, "q")[:M]
    Xt = hts.tensor_from_bits(np.ascontiguousarray(X), "bf16", DEV)
    bufs = block.buffers(M, W, Xt.dtype, DEV)
    block.forward(Xt, W, bufs, fused=True)
    torch.cuda.synchronize()
    rows = np.arange(M)
    bits = {k: hts.bits_from_tensor(v) for k, v in bufs.items()}
    up_ref = oracle.gemm_ref(X[rows], _masked(c, "up"), "bf16")
    h_ref = oracle.gated_ref(bits["gate"][rows], up_ref, "bf16")
    ok, rel = oracle.within_tolerance(oracle.widen_f64(bits["h"][rows], "bf16"), h_ref, TOL)
    assert ok, f"h: {rel:.3e}"
    d_ref = oracle.gemm_ref(bits["h"][rows], _masked(c, "down"), "bf16")
    ok, rel = oracle.within_tolerance(oracle.widen_f64(bits["down"][rows], "bf16"), d_ref, TOL)
    assert ok, f"down: {rel:.3e}"


@pytest.mark.parametrize("fused", [False, True])
def test_block_step_in_a_graph(fused):
    # captured once, replayed with eager work in between: every replay equals the eager step
    c = wl.config("7b_block")
    M = 128
    W = _weights(c, M, True)
    X = hts.tensor_from_bits(np.ascontiguousarray(activations(c.cfg_id, "q")[:M]), "bf16", DEV)
    bufs = block.buffers(M, W, X.dtype, DEV)
    eager = block.forward(X, W, bufs, fused).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        block.forward(X, W, bufs, fused)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        block.forward(X, W, bufs, fused)
    for rep in range(3):
        for v in bufs.values():
            v.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs["down"], eager), f"replay {rep}"
