"""The seeded input generator: SplitMix64 against its published outputs, and
the workload table against the five decode workloads."""
import math

import numpy as np
import pytest
import torch

import lrgen


def test_splitmix64_published_sequence():
    # First outputs of the SplitMix64 reference generator seeded with 1234567.
    s = 1234567
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    got = []
    for _ in range(5):
        s = (s + lrgen.GAMMA) & ((1 << 64) - 1)
        got.append(lrgen.mix64_int(s))
    assert got == want


def test_tensor_mix64_matches_integer_definition():
    key = lrgen.stream_key(99, 1, 2, 3)
    z = lrgen.raw_draws(key, 1000, 257)
    ref = [lrgen.mix64_int(key + (i + 1) * lrgen.GAMMA) for i in range(1000, 1257)]
    assert [(int(v) & ((1 << 64) - 1)) for v in z.tolist()] == ref


def test_normal_stream_is_chunk_invariant_and_standard():
    key = lrgen.stream_key(5, 7)
    full = lrgen.normal(key, 0, 1 << 20)
    part = lrgen.normal(key, 12345, 1000)
    assert torch.equal(full[12345:13345], part)
    x = full.double()
    assert abs(x.mean().item()) < 5e-3 and abs(x.var().item() - 1) < 5e-3
    # fourth moment of a standard normal is 3
    assert abs((x ** 4).mean().item() - 3) < 3e-2


def test_workload_table():
    w = lrgen.WORKLOADS
    assert [x.index for x in w] == [0, 1, 2, 3, 4]
    c0, c1, c2, c3, c4 = w
    assert (c0.batch, c0.n_heads, c0.embed, c0.context, c0.steps, c0.qfmt) == (1, 8, 1024, 512, 1, 0)
    assert (c1.batch, c1.n_heads, c1.embed, c1.context, c1.prefix, c1.steps) == (16, 32, 4096, 4096, 576, 128)
    assert c1.ranks_k[0] == [32] * 32 and c1.qfmt == lrgen.QFMT_INT8
    assert (c2.batch, c2.context, c2.qfmt, c2.n_outliers) == (64, 8192, lrgen.QFMT_INT4, 4)
    assert c2.ranks_v[0] == [64] * 32
    assert (c3.n_layers, c3.batch, c3.context, c3.steps) == (32, 32, 2048, 1)
    flat = sum(c3.ranks_k, []) + sum(c3.ranks_v, [])
    assert set(flat) == set(range(8, 97, 8))
    assert c3.ranks_k != c3.ranks_v
    assert (c4.batch, c4.context, c4.prefix, c4.steps, c4.qfmt) == (8, 32768, 2304, 64, lrgen.QFMT_INT4)
    assert c4.ranks_k[0] == [48] * 32
    assert all(x.head_dim == 128 for x in w)


def test_activation_variances_and_outliers():
    w = lrgen.workload(2)
    x = lrgen.activations(w, 0, 3, 560, 600).double()
    oc = lrgen.outlier_channels(w, 0)
    assert len(set(oc)) == 4
    normal_cols = [c for c in range(w.embed) if c not in oc]
    pre = x[:16][:, normal_cols]     # tokens 560..575 are image-prefix tokens
    txt = x[16:][:, normal_cols]
    assert abs(pre.var().item() - 1.5) < 0.05 and abs(txt.var().item() - 1.0) < 0.05
    assert x[:, oc].abs().mean().item() > 10 * x[:, normal_cols].abs().mean().item()


def test_factor_shapes_and_scales():
    w = lrgen.workload(3)
    ak = lrgen.down_factors(w, 5, 0)
    bv = lrgen.up_factors(w, 5, 1, dtype=torch.float32)
    assert ak.shape == (4096, sum(w.ranks_k[5])) and bv.shape == (sum(w.ranks_v[5]), 128)
    assert abs(ak.double().var().item() * 4096 - 1) < 0.02
    off = lrgen.head_offsets(w.ranks_v[5])
    h = 0
    r = w.ranks_v[5][h]
    blk = bv[off[h]:off[h] + r].double()
    assert abs(blk.var().item() * r - 1) < 0.25


def test_vectorised_draws_equal_the_per_stream_definitions():
    """normal_keyed draws element idx of stream key exactly as normal() does;
    the factors and the batched activations built from it equal the same
    tensors drawn one stream (head, batch row) at a time."""
    import math
    w = lrgen.workload(3)
    l = 4
    for kv, tag in ((0, lrgen.TAG_AK), (1, lrgen.TAG_AV)):
        a = lrgen.down_factors(w, l, kv)
        ranks = w.ranks_k[l] if kv == 0 else w.ranks_v[l]
        off = 0
        for h in (0, 7, 31):
            off = sum(ranks[:h])
            want = lrgen.normal(lrgen.stream_key(w.seed, tag, l, h), 0, w.embed * ranks[h],
                                1.0 / math.sqrt(w.embed)).view(w.embed, ranks[h])
            assert torch.equal(a[:, off:off + ranks[h]], want)
    b = lrgen.up_factors(w, l, 1, dtype=torch.float32)
    for h in (0, 13, 31):
        off, r = sum(w.ranks_v[l][:h]), w.ranks_v[l][h]
        want = lrgen.normal(lrgen.stream_key(w.seed, lrgen.TAG_BV, l, h), 0, r * w.head_dim,
                            1.0 / math.sqrt(r)).view(r, w.head_dim)
        assert torch.equal(b[off:off + r], want)
    w2 = lrgen.workload(2)   # outlier channels and the image prefix boundary
    x = lrgen.activations_rows(w2, 0, 3, 6, 570, 580)
    for i, bb in enumerate(range(3, 6)):
        assert torch.equal(x[i], lrgen.activations(w2, 0, bb, 570, 580))
