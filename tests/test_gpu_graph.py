"""The library's calls under HIP graph capture (torch.cuda.graph): a decode
step and a RoPE + prefill pass captured once and replayed with new inputs
copied into the captured buffers, eager work and synchronizations between
the replays; every replay must equal the eager call on the same inputs bit
for bit.  The library allocates nothing and sets no memory on the stream, so
the captured graph holds only its kernel launches."""
import numpy as np
import pytest
import torch

import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
from gpu_util import bits_to_dev, dev, say

pytestmark = pytest.mark.gpu


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_graph_replays():
    B, L, Hq, Hkv, d, G, theta = 4, 3000, 16, 4, 128, 16, 1e4
    say("decode graph: B=%d L=%d Hq=%d Hkv=%d" % (B, L, Hq, Hkv))
    kt = bits_to_dev(synth.normal_bits(61, 1, B * L, (Hkv, d)), (B, L, Hkv, d))
    vt = bits_to_dev(synth.normal_bits(61, 2, B * L, (Hkv, d)), (B, L, Hkv, d))
    cut = W.group_cutoffs(theta, d, G)
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device=dev())
    cl = torch.tensor([3000, 2500, 1, 1234], dtype=torch.int32, device=dev())
    qp = cl.clone()
    out = torch.empty_like(q)
    ws = torch.empty(W.decode_workspace_size(B, L, Hq, Hkv, d), dtype=torch.uint8, device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                        # warm-up off the capture
        W.decode(q, kt, vt, cl, qp, cut, G, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        W.decode(q, kt, vt, cl, qp, cut, G, workspace=ws, out=out)
    for r in range(4):
        qr = bits_to_dev(synth.normal_bits(62 + r, 0, B, (Hq, d)), (B, Hq, d))
        q.copy_(qr)
        cl.copy_(torch.tensor([3000 - r, 2500 + r, 1 + r, 1234], dtype=torch.int32))
        qp.copy_(cl + r)
        g.replay()
        torch.cuda.synchronize()
        ref = W.decode(qr, kt, vt, cl.clone(), qp.clone(), cut, G)
        torch.cuda.synchronize()
        assert _same(out, ref), r


def test_prefill_graph_replays():
    B, n, Hq, Hkv, d, G, theta = 1, 700, 8, 2, 128, 16, 300.0
    say("prefill graph: n=%d Hq=%d Hkv=%d" % (n, Hq, Hkv))
    cut = W.group_cutoffs(theta, d, G)
    qraw = torch.zeros((B, n, Hq, d), dtype=torch.bfloat16, device=dev())
    kraw = torch.zeros((B, n, Hkv, d), dtype=torch.bfloat16, device=dev())
    v = torch.zeros((B, n, Hkv, d), dtype=torch.bfloat16, device=dev())
    qr = torch.empty_like(qraw)
    kr = torch.empty_like(kraw)
    o = torch.empty_like(qraw)
    lse = torch.empty((B, Hq, n), dtype=torch.float32, device=dev())

    def path():
        W.rope_apply(qraw, theta, out=qr)
        W.rope_apply(kraw, theta, out=kr)
        W.prefill(qr, kr, v, cut, G, out=o, lse=lse, return_lse=True)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        path()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    for r in range(3):
        x = [bits_to_dev(synth.normal_bits(70 + r, t, B * n, (h, d)), (B, n, h, d))
             for t, h in ((0, Hq), (1, Hkv), (2, Hkv))]
        qraw.copy_(x[0])
        kraw.copy_(x[1])
        v.copy_(x[2])
        g.replay()
        torch.cuda.synchronize()
        q2 = W.rope_apply(x[0], theta)
        k2 = W.rope_apply(x[1], theta)
        o2, l2 = W.prefill(q2, k2, x[2], cut, G, return_lse=True)
        torch.cuda.synchronize()
        assert _same(o, o2), r
        assert torch.equal(lse, l2), r
