"""GPU parity of wp_rope_apply against the oracle's float64 RoPE."""
import numpy as np
import pytest
import torch

import oracle as O
import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
from gpu_util import bf16_to_np, bits_to_dev, dev, say

pytestmark = pytest.mark.gpu


def _check(got, ref, label):
    # output is bf16 (nearest even) of a float32 rotation: |err| <= 2^-9|ref| + fp32 error
    err = np.abs(got - ref)
    bound = np.abs(ref) * 2.0 ** -8 + 2e-6
    say("%-36s max_abs=%.3e worst ratio=%.3f" % (label, err.max(), (err / bound).max()))
    assert np.all(err <= bound), label


@pytest.mark.parametrize("B,n,H,d,theta,s,p0", [
    (1, 256, 1, 64, 1e4, 1.0, None),          # the tiny fp32 case shape
    (3, 77, 5, 128, 1e6, 4.0, [0, 1000, 131000]),
    (2, 33, 8, 128, 1e6, 1.0, [32768, 5]),
    (1, 1, 3, 64, 500.0, 2.0, [123456789]),
])
@pytest.mark.parametrize("fp32", [False, True])
def test_rope_matches_oracle(B, n, H, d, theta, s, p0, fp32):
    say("rope B=%d n=%d H=%d d=%d theta=%g s=%g fp32=%s" % (B, n, H, d, theta, s, fp32))
    rng_seed = 100 + n
    x = synth.normal_rows(rng_seed, 0, B * n, (H, d), round_bf16=not fp32)
    if fp32:
        xt = torch.from_numpy(x).reshape(B, n, H, d).to(dev())
    else:
        xt = bits_to_dev(synth.bf16_bits(x), (B, n, H, d))
    ps = None if p0 is None else torch.tensor(p0, dtype=torch.int64, device=dev())
    y = W.rope_apply(xt, theta, s, pos_start=ps)
    torch.cuda.synchronize()
    got = bf16_to_np(y).reshape(B, n, H, d)
    for b in range(B):
        pos = np.arange(n) + (0 if p0 is None else p0[b])
        ref = O.rope(x.reshape(B, n, H, d)[b].astype(np.float64), pos, theta, s)
        _check(got[b], ref, "rope b=%d" % b)


def test_rope_in_place_and_strided():
    B, n, H, d = 2, 50, 4, 128
    x = synth.normal_rows(7, 0, B * n, (H, d))
    xt = bits_to_dev(synth.bf16_bits(x), (B, n, H, d))
    ref = bf16_to_np(W.rope_apply(xt, 1e6, 1.0))
    W.rope_apply(xt, 1e6, 1.0, out=xt)           # in place
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_np(xt), ref)
    # a head-strided view (every other head of a wider tensor)
    wide = torch.zeros((B, n, 2 * H, d), dtype=torch.bfloat16, device=dev())
    src = bits_to_dev(synth.bf16_bits(x), (B, n, H, d))
    wide[:, :, ::2] = src
    view = wide[:, :, ::2]
    y = W.rope_apply(view, 1e6, 1.0)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_np(y), ref)
