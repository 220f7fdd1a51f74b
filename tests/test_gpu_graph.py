"""The fake-quant step captured as a HIP graph (as the benchmark times it)
replays to exactly the results of eager launches: outputs are cleared
eagerly before every replay, other eager GPU work and synchronizations run
between replays, and every replay is compared with the eager result."""
import numpy as np
import pytest
import torch

import fp4_block_quantization_fq_amd as fq
import workloads as wl
from gpu_util import make_desc, to_bits, to_dev

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    R, C = 512, 1024
    x = to_dev(wl.nv_activation(R, C, seed=3))
    dy = to_dev(wl.grad_output(R, C, seed=4))
    descs = [make_desc("mx"), make_desc("nv_tensor"), make_desc("nv_128"),
             make_desc("nv_128", "sr", "row", 1234), make_desc("nv_128", "sr", "col", 1234),
             make_desc("mx", "sr", "col", 1235)]
    outs = [fq.alloc_outputs(d, R, C, x.device) for d in descs]
    ys = [torch.empty_like(x) for _ in descs]
    ws = torch.empty((4096,), dtype=torch.uint8, device=x.device)
    dx = torch.empty_like(x)
    yd = torch.empty_like(x)
    d128 = descs[2]

    def step():
        for d, o, y in zip(descs, outs, ys):
            fq.fq_fake_quant(d, x, y=y, out=o, ws=ws)
        fq.fq_ste_backward(d128, x, outs[2], dy, dx=dx)
        fq.fq_dequantize(d128, outs[2], R, C, y=yd)

    def snapshot():
        res = [to_bits(y) for y in ys] + [to_bits(dx), to_bits(yd)]
        for o in outs:
            res += [o.codes.cpu().numpy(), o.scales.cpu().numpy()]
            if o.outer is not None:
                res.append(o.outer.cpu().numpy().view(np.uint32))
        return res

    def clear():
        for t in ys + [dx, yd]:
            t.zero_()
        for o in outs:
            o.codes.zero_()
            o.scales.zero_()
            if o.outer is not None:
                o.outer.zero_()

    step()
    torch.cuda.synchronize()
    want = snapshot()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step()
    other = to_dev(wl.nv_activation(R, C, seed=9))
    for rep in range(4):
        clear()
        fq.fq_fake_quant(descs[1], other, ws=ws)       # unrelated eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), (rep, k)
