"""Merged launches: layers that read the same input (q/k/v, gate/up) run as one
fp8w_linear call over their weights stacked along n.

Per-row scales make the merge exact at build time: each row's scale and codes
depend on that row alone ("FP8 weight-only (precision: fp8_weights)", section
"The contract": one scale per output channel), so the merged codes must equal
the separately quantised layers' codes, bit for bit. The merged outputs are
held to the same oracle gate as any call; which kernel plan runs may differ
from the separate calls', so the columns agree with the separate outputs only
to within fp32 summation order, which the gate covers.
"""
import numpy as np
import pytest
import torch

import fp8_weight_only_amd as fw
import oracle
import workloads
from parity_util import assert_gate, assert_same_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _merged_case(sizes, k, m, seed, dtype, with_bias):
    cases = [workloads.random_case(seed + i, m, n, k, dtype, with_bias) for i, n in enumerate(sizes)]
    x = cases[0].x
    ws = [torch.from_numpy(c.layer.w).to(DEV) for c in cases]
    bs = [c.layer.bias.to(DEV) for c in cases] if with_bias else None
    return cases, x, ws, bs


@pytest.mark.parametrize("sizes,k,m,dtype,with_bias", [
    ((48, 80, 16), 512, 1, torch.bfloat16, True),
    ((48, 80, 16), 512, 5, torch.float16, False),
    ((64, 64, 64), 1024, 16, torch.bfloat16, True),
    ((256, 512), 768, 32, torch.bfloat16, False),
    ((100, 36), 300, 7, torch.float16, True),     # k % 256 != 0: the merged call takes the fallback
])
def test_merged_codes_and_outputs(sizes, k, m, dtype, with_bias):
    cases, x, ws, bs = _merged_case(sizes, k, m, 40, dtype, with_bias)
    print(f"merged {sizes} k={k} m={m}", flush=True)
    merged = fw.QuantizedLinear.build_merged(ws, bs)
    assert merged.split_sizes == list(sizes)
    parts = [fw.QuantizedLinear.build(w, None if bs is None else bs[i]) for i, w in enumerate(ws)]
    assert_same_bits(merged.q.cpu().numpy(), torch.cat([p.q for p in parts]).cpu().numpy(), "merged codes")
    assert_same_bits(merged.scale.cpu().numpy(), torch.cat([p.scale for p in parts]).cpu().numpy(),
                     "merged scales")

    xd = x.to(DEV)
    y = merged(xd)
    torch.cuda.synchronize()
    w_all = np.concatenate([c.layer.w for c in cases])
    q_ref, s_ref, st = oracle.quantize_rows(w_all)
    assert st == 0
    assert_same_bits(merged.q.cpu().numpy(), q_ref, "merged codes vs oracle")
    x64 = x.double().numpy()
    b64 = None if bs is None else torch.cat([c.layer.bias for c in cases]).double().numpy()
    y_ref = oracle.linear_f64(x64, q_ref, s_ref, b64)
    amax = oracle.row_amax(w_all)
    yv = y.double().cpu().numpy()
    assert_gate(yv, y_ref, x64, amax, "merged call")
    # each layer's own call lands in the same gate on its columns
    c0 = 0
    for p, n in zip(parts, sizes):
        yp = p(xd).double().cpu().numpy()
        assert_gate(yp, y_ref[:, c0:c0 + n], x64, amax[c0:c0 + n], f"separate call, columns {c0}..")
        c0 += n


@pytest.mark.parametrize("group", [(0, 1, 2), (4, 5)])
def test_merged_block_layers(group):
    """The decoder block's q/k/v ([12288, 4096]) and gate/up ([28672, 4096])
    merged, at M = 16, bf16, against the oracle on every output."""
    lws = [workloads.block_layer(i) for i in group]
    print("merged " + "+".join(lw.name for lw in lws), flush=True)
    merged = fw.QuantizedLinear.build_merged([torch.from_numpy(lw.w).to(DEV) for lw in lws])
    w_all = np.concatenate([lw.w for lw in lws])
    q_ref, s_ref, st = oracle.quantize_rows(w_all)
    assert st == 0
    assert_same_bits(merged.scale.cpu().numpy(), s_ref, "merged scales")
    assert_same_bits(merged.q.cpu().numpy(), q_ref, "merged codes")
    x = workloads.block_x(group[0])
    y = merged(x.to(DEV))
    torch.cuda.synchronize()
    x64 = x.double().numpy()
    assert_gate(y.double().cpu().numpy(), oracle.linear_f64(x64, q_ref, s_ref, None), x64,
                oracle.row_amax(w_all), "merged block layer")
