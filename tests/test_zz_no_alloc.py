"""wp_decode_noalloc (the decode entry point that allocates nothing, its
partial results in the library's fixed device scratch) against wp_decode
with a caller workspace, through the C ABI: bit-identical outputs and
counters on two calls in a row, the second with a smaller input, and the
size limit rejected before any launch."""
import numpy as np
import pytest
import torch

import oracle as O
import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
from gpu_util import bits_to_dev, dev, say

pytestmark = pytest.mark.gpu


def _case(B, L, Hq, Hkv, d, seed, q_pos=None):
    q = bits_to_dev(synth.normal_bits(seed, 0, B, (Hq, d)), (B, Hq, d))
    kc = bits_to_dev(synth.normal_bits(seed, 1, B * L, (Hkv, d)), (B, L, Hkv, d))
    vc = bits_to_dev(synth.normal_bits(seed, 2, B * L, (Hkv, d)), (B, L, Hkv, d))
    lens = np.random.default_rng(seed).integers(1, L + 1, size=B)
    lens[0] = L
    cl = torch.from_numpy(lens.astype(np.int32)).to(dev())
    qp = torch.from_numpy((lens + (0 if q_pos is None else q_pos)).astype(np.int32)).to(dev())
    return q, kc, vc, cl, qp


@pytest.mark.parametrize("dense", [False, True])
def test_noalloc_matches_workspace_decode(dense):
    # two calls in a row on the shared scratch, the second smaller, each
    # against wp_decode with its own workspace on the same inputs
    for B, L, Hq, Hkv, d, G, theta, seed in ((16, 3000, 32, 8, 128, 16, 1e4, 61),
                                             (3, 700, 8, 2, 64, 32, 300.0, 62)):
        say("noalloc decode B=%d L=%d Hq=%d Hkv=%d d=%d G=%d dense=%s" % (B, L, Hq, Hkv, d, G, dense))
        q, kc, vc, cl, qp = _case(B, L, Hq, Hkv, d, seed)
        cut = W.group_cutoffs(theta, d, G)
        ng = d // G
        c1 = torch.zeros(3 * ng + 1, dtype=torch.int64, device=dev())
        c2 = torch.zeros_like(c1)
        o_ref = W.decode(q, kc, vc, cl, qp, None if dense else cut, G, dense=dense, counters=c1)
        o_na = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device=dev())
        W.decode_noalloc(q, kc, vc, cl, qp, None if dense else cut, G, dense=dense, counters=c2, out=o_na)
        torch.cuda.synchronize()
        assert torch.equal(o_ref.view(torch.int16), o_na.view(torch.int16))
        assert torch.equal(c1, c2)


def test_noalloc_split_counts_and_oracle():
    # explicit split counts, including the largest the scratch holds at this
    # shape, against the oracle
    B, L, Hq, Hkv, d, G, theta = 4, 1500, 16, 4, 128, 16, 1e3
    q, kc, vc, cl, qp = _case(B, L, Hq, Hkv, d, 63)
    cut = W.group_cutoffs(theta, d, G)
    dc = O.dim_cutoffs_grouped(np.array(cut), G)
    for S in (1, 5, 47):
        assert W.decode_workspace_size(B, L, Hq, Hkv, d, S) <= 8 << 20
        o = W.decode_noalloc(q, kc, vc, cl, qp, cut, G, num_splits=S)
        o_ref = W.decode(q, kc, vc, cl, qp, cut, G, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), S
    got = o.float().cpu().numpy().astype(np.float64)
    qn = q.float().cpu().numpy().astype(np.float64)
    kn = kc.float().cpu().numpy().astype(np.float64)
    vn = vc.float().cpu().numpy().astype(np.float64)
    for b in range(B):
        L_b, p_b = int(cl[b]), int(qp[b])
        ref = O.decode(qn[b], kn[b], vn[b], p_b, L_b, dc)
        err = np.abs(got[b] - ref)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (b, err.max(), err.mean())


def test_noalloc_rejects_sizes_beyond_the_scratch():
    B, L, Hq, Hkv, d = 64, 4096, 64, 8, 128
    S = 200
    assert W.decode_workspace_size(B, L, Hq, Hkv, d, S) > 8 << 20
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device=dev())
    # the size check comes before any launch: a broadcast view stands in for the cache
    kc = torch.zeros((1, 1, 1, d), dtype=torch.bfloat16, device=dev()).expand(B, L, Hkv, d)
    cl = torch.full((B,), L, dtype=torch.int32, device=dev())
    with pytest.raises(W.WPError) as ei:
        W.decode_noalloc(q, kc, kc, cl, cl, None, 16, dense=True, num_splits=S)
    assert ei.value.status == -5 and "scratch" in str(ei.value)
