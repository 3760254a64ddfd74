"""Whole MoE layers byte for byte against the oracle, no sampling.

* A Qwen3-235B-A22B-shaped layer (128 experts of gate_up bf16 [3072,4096]
  and 128 of down bf16 [4096,1536], layer 0 of the 5000 + l seeds): MXFP8
  and NVFP4, linear and swizzled scales, each projection in the benchmark's
  launch configuration (16 experts per launch, 8 launches).
* The Qwen3-30B-A3B-shaped layer (gate_up [1536,2048], down [2048,768]),
  MXFP8 with swizzled scales, 16 experts per launch, at two layer seeds
  (2000 + l, l = 0, 1).
* The NVFP4 auto-scaled launch of 16 gate_up experts [3072,4096]: every
  expert's payload and scales, every encode scale and amax.

Every payload and scale byte of every expert is compared; the oracle runs on
the host threads of the machine's CPU share (its C calls release the GIL).
NVFP4 encode scales come from the oracle's encode-scale rule on each
expert's amax, computed on the host.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantization_moe_amd as mxq
from nvfp4_quantization_moe_amd import workloads
from gpu_common import HOST_THREADS, par_map, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
E, G = workloads.N_EXPERTS, workloads.GROUP


def _host_bits(stack):
    return stack.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _encode_scales(orc, stack):
    amax = stack.float().abs().amax(dim=(1, 2)).cpu().numpy()
    return np.array([orc.nvfp4_encode_scale(float(a)) for a in amax], np.float32)


def _quantize_layer(fmt, layout, stack, g):
    """Quantize all experts of one projection as the benchmark does: 16 per
    launch through prepacked calls.  Returns host payload [E, rows, pw] and
    scales [E, nsc]."""
    n, rows, cols = stack.shape
    pw = cols if fmt == mxq.MXFP8 else cols // 2
    nsc = mxq.scale_bytes(rows, cols, fmt, layout)
    pay = torch.empty(n, rows, pw, dtype=torch.uint8, device=DEV)
    sc = torch.empty(n, nsc, dtype=torch.uint8, device=DEV)
    pay.fill_(0xA5)
    sc.fill_(0xA5)
    gs = None if g is None else torch.from_numpy(g).to(DEV)
    for b in range(0, n, G):
        call = mxq.GroupedCall(fmt, layout, [stack[b + i] for i in range(G)],
                               [pay[b + i] for i in range(G)], [sc[b + i] for i in range(G)],
                               None if gs is None else gs[b:b + G])
        call()
    torch.cuda.synchronize()
    return pay.cpu().numpy(), sc.cpu().numpy()


def _compare_all(orc, fmt, layout, host, pay, sc, g, what):
    def one(i):
        p, s = orc.quantize(fmt, layout, host[i], g=1.0 if g is None else float(g[i]))
        return np.array_equal(pay[i], p) and np.array_equal(sc[i], s)
    ok = par_map(one, range(len(host)))
    bad = [i for i, v in enumerate(ok) if not v]
    assert not bad, (what, "experts differing from the oracle", bad[:16])


@pytest.fixture(scope="module")
def layer_235b():
    say("generating the Qwen3-235B-A22B layer 0 (seed 5000)")
    lay = workloads.moe_layer(workloads.QWEN3_235B_A22B, 0, 5000, 0.015, device=DEV)
    torch.cuda.synchronize()
    host = {p: _host_bits(t) for p, t in lay.items()}
    yield lay, host
    del lay, host
    torch.cuda.empty_cache()


@pytest.mark.parametrize("proj", ["gate_up", "down"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("fmt", [0, 1])
def test_qwen3_235b_full_layer(orc, layer_235b, fmt, layout, proj):
    lay, host = layer_235b
    stack = lay[proj]
    g = _encode_scales(orc, stack) if fmt == mxq.NVFP4 else None
    say("qwen3-235b layer 0", proj, "fmt", fmt, "layout", layout, "threads", HOST_THREADS)
    pay, sc = _quantize_layer(fmt, layout, stack, g)
    _compare_all(orc, fmt, layout, host[proj], pay, sc, g, (proj, fmt, layout))


@pytest.mark.parametrize("layer", [0, 1])
def test_qwen3_30b_full_layer_mxfp8_swizzled(orc, layer):
    say("qwen3-30b-a3b layer", layer, "(seed", 2000 + layer, ")")
    lay = workloads.moe_layer(workloads.QWEN3_30B_A3B, layer, 2000, 0.02, device=DEV)
    for proj, stack in lay.items():
        host = _host_bits(stack)
        pay, sc = _quantize_layer(mxq.MXFP8, mxq.SWIZZLED, stack, None)
        _compare_all(orc, mxq.MXFP8, mxq.SWIZZLED, host, pay, sc, None, (layer, proj))


def test_auto_qwen3_235b_gate_up_launch_full(orc):
    """One auto-scaled launch of 16 gate_up experts: every byte of every
    expert, every encode scale and amax."""
    r, c = workloads.QWEN3_235B_A22B["gate_up"]
    stack = workloads.expert_stack(G, r, c, std=0.015, seed=5000, device=DEV)
    say("auto-scaled Qwen3-235B gate_up launch, full compare")
    call = mxq.GroupedAutoCall(mxq.SWIZZLED, [stack[i] for i in range(G)])
    pays, scs, g, am = call()
    torch.cuda.synchronize()
    host = _host_bits(stack)
    want_am = np.array([orc.tensor_amax(host[i]) for i in range(G)], np.float32)
    want_g = np.array([orc.nvfp4_encode_scale(a) for a in want_am], np.float32)
    assert np.array_equal(am.cpu().numpy(), want_am)
    assert np.array_equal(g.cpu().numpy(), want_g)
    pay = np.stack([p.cpu().numpy() for p in pays])
    sc = np.stack([s.cpu().numpy() for s in scs])
    _compare_all(orc, mxq.NVFP4, mxq.SWIZZLED, host, pay, sc, want_g, "auto")
