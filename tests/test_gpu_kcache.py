"""GPU tests of the group-major compact K store.

* wp_kcache_append: byte-exact against the ring built here on the host from
  its definition (group g keeps key j in slot j % cap[g], later keys
  replace earlier ones), for one large append and for a prefill followed by
  single-token appends that wrap every small ring several times.  Slots no
  key reached keep their sentinel.
* wp_decode_kcache: identical bits to wp_decode on the full cache (same
  arithmetic, same order) and the tile counters, and within 2e-2 / 2e-3 of
  the oracle; with small thetas the rings are shorter than the cache, so
  evicted slots sit under partial groups and must be masked."""
import numpy as np
import pytest
import torch

import oracle as O
import rope_positional_encoding_amd as W
from rope_positional_encoding_amd import synth
from gpu_util import bf16_to_np, bits_to_dev, compare, dev, say, to_f64

pytestmark = pytest.mark.gpu

SENTINEL = 0x7F7F   # a bf16 bit pattern no normal(0,1) draw produces here


def _ring_reference(kbits, pos0, T, Hkv, d, G, caps, offs, store_init):
    """kbits [B*T, Hkv, d] bf16 bits (int16) in token order of each row; the
    store [B, Hkv, elements] after appending row b's tokens at positions
    pos0[b] + t in order: group g, slot s, element e of kv head h sits at
    [b, h, offs[g] + s * G + e]."""
    B = len(pos0)
    st = store_init.copy()
    for b in range(B):
        for t in range(T):
            p = pos0[b] + t
            for g in range(d // G):
                slot = p % caps[g]
                st[b, :, offs[g] + slot * G: offs[g] + (slot + 1) * G] = kbits[b * T + t, :, g * G:(g + 1) * G]
    return st


def _store_with_sentinel(B, Hkv, total):
    return np.full((B, Hkv, total), SENTINEL, dtype=np.int16)


def _to_dev_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev()).view(torch.bfloat16)


def _from_dev_bits(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("B,T,Hkv,d,G,theta,pos0", [
    (2, 300, 2, 128, 16, 30.0, [0, 0]),
    (3, 257, 1, 64, 32, 100.0, [0, 5, 40]),
    (1, 1000, 4, 128, 16, 1e3, [17]),
])
def test_append_bulk_matches_ring_definition(B, T, Hkv, d, G, theta, pos0):
    say("kcache append B=%d T=%d Hkv=%d d=%d G=%d theta=%g pos0=%s" % (B, T, Hkv, d, G, theta, pos0))
    Lmax = max(pos0) + T
    cut = W.group_cutoffs(theta, d, G)
    caps, offs = W.kcache_layout(Lmax, d, G, cut)
    kb = synth.normal_bits(61, 1, B * T, (Hkv, d))
    k = bits_to_dev(kb, (B, T, Hkv, d))
    init = _store_with_sentinel(B, Hkv, offs[-1])
    store = _to_dev_bits(init)
    W.kcache_append(k, torch.tensor(pos0, dtype=torch.int32, device=dev()), store, Lmax, cut, G)
    torch.cuda.synchronize()
    ref = _ring_reference(kb, pos0, T, Hkv, d, G, caps, offs, init)
    assert np.array_equal(_from_dev_bits(store), ref)


def test_append_stepwise_wraps_rings():
    B, Hkv, d, G, theta = 2, 2, 64, 16, 30.0
    Lp, steps = 50, 140
    Lmax = Lp + steps
    cut = W.group_cutoffs(theta, d, G)
    caps, offs = W.kcache_layout(Lmax, d, G, cut)
    say("kcache stepwise caps=%s" % caps)
    assert min(caps) < 20            # the small rings wrap many times
    kb = synth.normal_bits(62, 1, B * Lmax, (Hkv, d)).reshape(B, Lmax, Hkv, d)
    init = _store_with_sentinel(B, Hkv, offs[-1])
    store = _to_dev_bits(init)
    kdev = bits_to_dev(kb.reshape(B * Lmax, Hkv, d), (B, Lmax, Hkv, d))
    W.kcache_append(kdev[:, :Lp].contiguous(), torch.zeros(B, dtype=torch.int32, device=dev()), store,
                    Lmax, cut, G)
    for t in range(Lp, Lmax):
        W.kcache_append(kdev[:, t:t + 1], torch.full((B,), t, dtype=torch.int32, device=dev()), store,
                        Lmax, cut, G)
    torch.cuda.synchronize()
    ref = _ring_reference(kb.reshape(B * Lmax, Hkv, d), [0] * B, Lmax, Hkv, d, G, caps, offs, init)
    assert np.array_equal(_from_dev_bits(store), ref)


# B, Lmax, Hq, Hkv, d, G, theta, cache lengths, q_pos offset, splits
CASES = [
    (2, 700, 8, 2, 128, 16, 30.0, [700, 333], 0, 0),
    (3, 1200, 16, 4, 64, 32, 100.0, [1200, 64, 1], 1, 3),
    (2, 3000, 32, 8, 128, 16, 1e3, [3000, 2047], -1, 0),
    (1, 4096, 8, 1, 128, 32, 300.0, [4096], 0, 5),
    (2, 900, 32, 1, 128, 16, 100.0, [900, 17], 0, 0),    # 32 query heads on one kv head: two head sets
]


@pytest.mark.parametrize("B,Lmax,Hq,Hkv,d,G,theta,lens,qoff,splits", CASES)
def test_decode_kcache_equals_decode_and_oracle(B, Lmax, Hq, Hkv, d, G, theta, lens, qoff, splits):
    say("decode_kcache B=%d Lmax=%d Hq=%d Hkv=%d d=%d G=%d theta=%g lens=%s qoff=%d splits=%d"
        % (B, Lmax, Hq, Hkv, d, G, theta, lens, qoff, splits))
    cut = W.group_cutoffs(theta, d, G)
    caps, offs = W.kcache_layout(Lmax, d, G, cut)
    seed = 63 + Lmax
    q = synth.normal_bits(seed, 0, B, (Hq, d))
    kc = synth.normal_bits(seed, 1, B * Lmax, (Hkv, d))
    vc = synth.normal_bits(seed, 2, B * Lmax, (Hkv, d))
    q_pos = [L + qoff if L + qoff >= L - 1 else L - 1 for L in lens]
    qt = bits_to_dev(q, (B, Hq, d))
    kt = bits_to_dev(kc, (B, Lmax, Hkv, d))
    vt = bits_to_dev(vc, (B, Lmax, Hkv, d))
    cl = torch.tensor(lens, dtype=torch.int32, device=dev())
    qp = torch.tensor(q_pos, dtype=torch.int32, device=dev())
    # the store holds positions 0 .. cache_len-1 of each sequence: append
    # each sequence's prefix on its own
    store = _to_dev_bits(_store_with_sentinel(B, Hkv, offs[-1]))
    for b in range(B):
        W.kcache_append(kt[b:b + 1, :lens[b]], torch.zeros(1, dtype=torch.int32, device=dev()),
                        store[b:b + 1], Lmax, cut, G)
    cnt_a = torch.zeros(3 * (d // G) + 1, dtype=torch.int64, device=dev())
    cnt_b = torch.zeros_like(cnt_a)
    ref_dev = W.decode(qt, kt, vt, cl, qp, cut, G, num_splits=splits, counters=cnt_a)
    got_dev = W.decode_kcache(qt, store, vt, cl, qp, cut, G, num_splits=splits, counters=cnt_b)
    torch.cuda.synchronize()
    assert torch.equal(got_dev.view(torch.int16), ref_dev.view(torch.int16))
    assert torch.equal(cnt_a, cnt_b)
    got = bf16_to_np(got_dev)
    dim_cut = O.dim_cutoffs_grouped(np.array(cut), G)
    for b in range(B):
        sl = slice(b * Lmax, (b + 1) * Lmax)
        ref = O.decode(to_f64(q[b]), to_f64(kc[sl]), to_f64(vc[sl]), q_pos[b], lens[b], dim_cut)
        compare(got[b], ref, "decode_kcache b=%d L=%d" % (b, lens[b]))
    kept = offs[-1] / float(Lmax * d)
    say("K store %.3f of the full K cache" % kept)
