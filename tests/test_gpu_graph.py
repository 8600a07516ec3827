"""GPU tier: the forward captured into a HIP graph and replayed.

moe_w4a4_forward only enqueues kernels on the caller's stream (no allocation,
no synchronization, no memset), so a serving loop can capture it.  For the
streaming path (DeepSeek-V4-Flash shape at 64 tokens) and the LDS-staged path
(a prefill shape), a graph captured on one input set is replayed three times
with new inputs copied into the captured buffers, and with eager forwards of
other inputs on the same workspace and synchronizations between the replays;
every replay must equal the eager forward of its inputs bit for bit."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests.gpu_support import dev, dev_bf16, host_bits, layer_for, log, synth_layer

pytestmark = pytest.mark.gpu

CASES = [
    synth.CONFIGS[1],
    synth.LayerConfig(130, "graph_prefill_h512_i512_e16_k2_t1000", 1000, 512, 512, 16, 2, "uniform", 130),
]


def inputs(cfg):
    x = synth.make_tokens(cfg)
    ids, w = synth.make_routing(cfg)
    return dev_bf16(x), dev(ids), dev(w)


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_forward_graph_replays_equal_eager(cfg):
    log(f"[test] graph capture and replay, {cfg.name}")
    if cfg.name.startswith("dsv4"):
        layer = synth_layer(1, cfg.tokens)
    else:
        layer = layer_for(cfg.hidden, cfg.inter, cfg.experts, cfg.topk, cfg.tokens)
        layer.load_fp32(lambda e: synth.expert_weights_f32(cfg, e), threads=4)
    sets = [inputs(cfg), inputs(dataclasses.replace(cfg, index=cfg.index + 500))]
    eager = []
    for x, ids, w in sets:
        eager.append(host_bits(layer.forward(x, ids, w)))
        torch.cuda.synchronize()
    assert not np.array_equal(eager[0], eager[1])

    x_s, ids_s, w_s = (t.clone() for t in sets[0])
    out_s = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                       # one eager call on the capture stream first
        layer.forward(x_s, ids_s, w_s, out=out_s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x_s, ids_s, w_s, out=out_s)
    torch.cuda.synchronize()

    for i, which in enumerate((1, 0, 1)):
        for dst, src in zip((x_s, ids_s, w_s), sets[which]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = host_bits(out_s)
        log(f"    replay {i} on input set {which}: bit-identical {np.array_equal(got, eager[which])}")
        assert np.array_equal(got, eager[which])
        other = sets[1 - which]                         # eager work on the same workspace in between
        assert np.array_equal(host_bits(layer.forward(*other)), eager[1 - which])
        torch.cuda.synchronize()
