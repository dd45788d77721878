"""The library under HIP graph capture: the grouped paths (device offsets,
group tables rebuilt on the device), the fused casts, the tensor-wise cast's
three launches and the grouped GEMM captured once with torch.cuda.graph and
replayed several times, with eager work and synchronisations between the
replays.  Every replay must reproduce the eager outputs byte for byte, which
also fails if the library synchronised, read device memory on the host or
recorded a memset (nothing of the kind is captured), and shows any run-to-run
difference (a race) as a mismatch.  The eager outputs themselves are checked
against the oracle by the other GPU tests."""
import numpy as np
import pytest
import torch

import fp8_precision_quantization_amd as mx
from fp8_precision_quantization_amd import workloads
from tests.gpu_util import device, to_dev_bf16

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _calls(dev):
    """The captured work and its preallocated outputs: (fn, outputs)."""
    bits, ends = workloads.moe_activations(rows=1024, cols=512, groups=4, seed=31)
    x = to_dev_bf16(bits, dev)
    offs = torch.from_numpy(ends).to(dev)
    rows, cols = x.shape
    g = offs.numel()
    u8 = dict(dtype=torch.uint8, device=dev)
    outs = {
        "mg": (torch.empty(rows, cols, **u8), torch.empty(rows + 128 * g, cols // 32, **u8),
               torch.empty(g + 1, dtype=torch.int64, device=dev), torch.empty(cols, rows, **u8),
               torch.empty(cols, rows // 32, **u8)),
        "plain": (torch.empty(rows, cols, **u8), torch.empty(rows, cols // 32, **u8),
                  torch.empty(cols, rows, **u8), torch.empty(cols, rows // 32, **u8)),
        "blk": (torch.empty(rows, cols, **u8), torch.empty(rows, cols // 32, **u8),   # 1024 and 512: no padding
                torch.empty(cols, rows, **u8), torch.empty(cols, rows // 32, **u8)),
        "gb": (torch.empty(rows, cols, **u8), torch.empty(rows + 128 * g, cols // 32, **u8),
               torch.empty(cols, rows, **u8), torch.empty(cols, rows // 32 + 4 * g, **u8),
               torch.empty(g + 1, dtype=torch.int64, device=dev), torch.empty(g + 1, dtype=torch.int64, device=dev)),
        "kg": (torch.empty(cols, rows // 32 + 4 * g, **u8),   # (ceil128(512), ceil4(32) + 4 G)
               torch.empty(g + 1, dtype=torch.int64, device=dev)),
        "tw": (torch.empty(rows, cols, **u8), torch.empty(1, dtype=torch.int16, device=dev),
               torch.empty(mx.mx_tensorwise_workspace_bytes(rows * cols), **u8)),
    }
    # weights for the grouped GEMM: one (192, 512) matrix per group, cast once
    ws = [mx.mx_cast_dim0_dim1_blocked(to_dev_bf16(workloads.heavy_tailed_rows(192, cols, seed=40 + i), dev),
                                       dim1=False, raw=True) for i in range(g)]
    qb = torch.stack([w[0] for w in ws])
    sb = torch.cat([w[1].reshape(-1) for w in ws])
    outs["gemm"] = (torch.empty(rows, 192, dtype=torch.float32, device=dev),)
    # K-grouped layout input: the dim1 scales of the M-grouped cast, grouped
    # along their columns with the same ends in scale columns
    kends = torch.from_numpy(np.asarray(ends, np.int32) // 32).to(dev)

    def run():
        mg = outs["mg"]
        mx.mx_cast_dim0_dim1_mgrouped(x, offs, out=mg[:2] + mg[3:], out_group_starts=mg[2], raw=True)
        mx.mx_cast_dim0_dim1(x, out=outs["plain"], raw=True)
        gb = outs["gb"]
        mx.mx_cast_dim0_dim1_grouped_blocked(x, offs, out=gb[:4], out_row_starts=gb[4], out_col_starts=gb[5],
                                             raw=True)
        mx.mx_cast_dim0_dim1_blocked(x, out=outs["blk"], raw=True)
        kg = outs["kg"]
        mx.mx_scales_to_blocked_grouped(mg[4], kends, 1, out=kg[0], out_group_starts=kg[1], raw=True)
        tw = outs["tw"]
        mx.mx_quantize_fp8_tensorwise(x, out=tw[:2], workspace=tw[2], raw=True)
        mx.mx_grouped_gemm_mxfp8(mg[0], mg[1], qb, sb, offs, out_dtype=torch.float32, out=outs["gemm"][0])

    # every output byte is written by the library (the workspace is scratch)
    flat = [t for v in outs.values() for t in v if t is not outs["tw"][2]]
    return run, flat


def test_graph_replays_match_eager():
    dev = device()
    run, outs = _calls(dev)
    run()
    torch.cuda.synchronize(dev)
    eager = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize(dev)
    noise = torch.empty(1 << 22, device=dev)
    for rep in range(REPLAYS):
        for t in outs:
            t.view(torch.uint8).fill_(0xCD)
        noise.normal_()           # eager work between replays
        torch.cuda.synchronize(dev)
        graph.replay()
        torch.cuda.synchronize(dev)
        for i, (t, e) in enumerate(zip(outs, eager)):
            assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), "replay %d, output %d differs" % (rep, i)
