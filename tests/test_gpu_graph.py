"""Decode launches captured in a HIP graph (GPU): one launch per layer, as a
model calls the library, with sub-page partitions and the fold in each
launch. Every replay must give the eager launches' bits and match the
oracle; replays are interleaved with eager work and synchronisations, and
the outputs are cleared by a kernel before each replay."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_182_amd as pkv
import synth
from synth.device import to_device
from synth.layout import FP8, FP16, INT4, INT8
from gpu_util import compare

pytestmark = pytest.mark.gpu


def per_layer_params(w, rows, partition_tokens):
    return pkv.make_params(rows=rows, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                           head_dim=w.head_dim, page_size=w.page_size, num_pages=w.num_pages,
                           max_pages_per_row=w.max_pages, pool_bytes=w.pool.nbytes, max_sel_pages=w.max_sel,
                           partition_tokens=partition_tokens, k_codec=pkv.CODEC_MIXED, v_codec=pkv.CODEC_MIXED,
                           softmax_scale=w.softmax_scale)


@pytest.mark.parametrize("partition_tokens", [0, 48])
def test_per_layer_launches_in_a_graph(partition_tokens):
    print(f"case graph per-layer T={partition_tokens}", flush=True)
    cyc = [(FP16, FP16), (FP8, FP8), (INT8, INT4)]
    layers, per = 4, 2
    w = synth.build_workload("graph_layers", rows=layers * per, hq=8, hkv=2, dim=64, page=64,
                             seq_lens=[900, 130, 1024, 64, 1, 700, 513, 333],
                             codec_of=lambda r, lp: cyc[(r + lp) % 3], seed=21)
    dw = to_device(w)
    p = per_layer_params(w, per, partition_tokens)
    q, pool, koff, voff, codec, scale, bt, lens, _, _ = dw.args()
    out = torch.empty((w.rows, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.rows, w.num_q_heads), dtype=torch.float32, device="cuda")
    ws = torch.zeros(max(pkv.workspace_bytes(p), 16), dtype=torch.uint8, device="cuda")

    def step():
        for layer in range(layers):
            r = slice(layer * per, (layer + 1) * per)
            pkv.decode_attention(p, q[r], pool, koff, voff, codec, scale, bt[r], lens[r],
                                 out=out[r], lse=lse[r], workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    compare(ref[0].cpu().numpy().astype(np.float64), ref[1].cpu().numpy().astype(np.float64),
            *oracle.decode_attention(w), f"eager per-layer T={partition_tokens}")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), f"replay {rep} differs from eager"
        step()                      # eager work between replays
        torch.cuda.synchronize()
