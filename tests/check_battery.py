"""Child process of tests/test_checked_build.py, run with LR_ATTN_LIB naming
the checked library (liblr_attn_check.so: every cache access of the kernels
tested against the cache buffer).  Runs the seeded random plans of
test_gpu_random_shapes and the decode cases of test_gpu_parity that reach the
edges of the layout (ragged and empty contexts, every row tail width, small
heads in the paired buckets, context splits, the fused append, 128 heads, a
2^24-token context with offsets past 4 GiB) -- each still checked against the
oracle -- the hybrid FFN's fixed, full-size, multi-pass and seeded random
shapes, and latent generation's random shapes and entry points; then one
decode, one FFN call and one projection with the tested extents shrunk by
4 KiB, and prints one JSON line: the accesses found outside their
buffers in the first parts (must be 0) and in the second (must not be: the
check fires)."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np   # noqa: E402
import torch         # noqa: E402

import latent_kv_attention_lr_amd as lr                     # noqa: E402
from latent_kv_attention_lr_amd.session import DecodeSession   # noqa: E402
import test_ffn as tf                                       # noqa: E402
import test_gpu_project as tp                               # noqa: E402
import test_gpu_parity as gp                                # noqa: E402
import test_gpu_random_shapes as rs                         # noqa: E402


def main():
    assert os.path.basename(lr.LIB_PATH) == "liblr_attn_check.so", lr.LIB_PATH
    lr.lr_attn_check_count()                     # start from 0
    for seed in range(rs.N_CASES):
        rs.test_random_shape_decode_matches_oracle(seed)
    I8, I4, BF, F32 = lr.LR_Q_INT8_TOKEN, lr.LR_Q_INT4_G32, lr.LR_DT_BF16, lr.LR_DT_F32
    for qfmt in (I8, I4):
        for io in (BF, F32):
            for max_splits in (0, 1):
                gp.test_decode_ragged_and_degenerate_lengths(qfmt, io, max_splits)
            for bucket in (32, 96, 128):
                gp.test_decode_every_row_tail_width(qfmt, io, bucket)
            gp.test_decode_context_split_path(qfmt, io)
            gp.test_append_decode_fused_equals_separate(qfmt, io)
        gp.test_decode_all_128_heads(qfmt)
        gp.test_decode_at_maximum_capacity(qfmt)
    for io in (BF, F32):
        for bucket in (96, 128):
            gp.test_decode_small_heads_in_paired_buckets(io, bucket)
    torch.cuda.synchronize()
    outside = lr.lr_attn_check_count()

    # the hybrid FFN: its fixed shapes, the full workload, the seeded random shapes
    shapes = [m for m in tf.test_ffn_decode_matches_oracle.pytestmark if m.name == "parametrize"][0].args[1]
    for shape in shapes:
        tf.test_ffn_decode_matches_oracle(*shape)
    tf.test_ffn_decode_full_size_and_deterministic()
    tf.test_ffn_decode_in_several_passes()
    for seed in range(16):
        tf.test_ffn_decode_random_shapes(seed)
    torch.cuda.synchronize()
    outside_ffn = lr.lr_attn_check_count()

    # latent generation: packing, the product (unsplit and in parts), the
    # generate-then-append and one-step-from-activations entry points
    for seed in range(16):
        tp.test_project_random_shapes(seed)
    for qfmt in (I8, I4):
        tp.test_project_append_equals_project_then_append(qfmt)
    shapes = [m for m in tp.test_project_append_decode_integer_inputs_equal_two_calls.pytestmark
              if m.name == "parametrize"][0].args[1]
    for shape in shapes:
        tp.test_project_append_decode_integer_inputs_equal_two_calls(*shape)
    tp.test_project_append_decode_full_layer_shape_matches_oracle_chain()
    torch.cuda.synchronize()
    outside_proj = lr.lr_attn_check_count()

    # the check fires: a cache whose last tiles lie past the tested extent
    rng = np.random.default_rng(5)
    B, H, cap, rk, rv = 2, 4, 300, [32, 8, 64, 16], [16, 40, 8, 32]
    s = DecodeSession(1, B, H, cap, lr.LR_Q_INT8_TOKEN, lr.LR_DT_BF16, [rk], [rv], device="cuda:0")
    ck = torch.from_numpy(rng.standard_normal((B, cap, sum(rk))).astype(np.float32)).cuda()
    cv = torch.from_numpy(rng.standard_normal((B, cap, sum(rv))).astype(np.float32)).cuda()
    s.append(0, ck, cv, torch.zeros(B, dtype=torch.int32, device="cuda:0"))
    s.set_factors(0, torch.zeros(sum(rk), 128, dtype=torch.bfloat16, device="cuda:0"),
                  torch.zeros(sum(rv), 128, dtype=torch.bfloat16, device="cuda:0"))
    s.lengths.fill_(cap)
    q = torch.zeros(B, H, 128, dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty_like(q)
    lr.lr_attn_check_shrink(4096)
    s.decode(0, q, out, max_len=cap)
    torch.cuda.synchronize()
    lr.lr_attn_check_shrink(0)
    fired = lr.lr_attn_check_count()
    s.close()
    from latent_kv_attention_lr_amd.ffn import FfnLayer
    f, w, x = tf._case(256, 160, 64, 128, 17, seed=3)
    layer = FfnLayer(256, 160, 64, 128, device="cuda:0")
    layer.set_weights(*w)
    lr.lr_attn_check_shrink(4096)
    layer(x.to("cuda:0"))
    torch.cuda.synchronize()
    lr.lr_attn_check_shrink(0)
    fired_ffn = lr.lr_attn_check_count()
    ps = tp._session([8, 32], [16, 24], batch=1, cap=64)
    ak = torch.from_numpy(rng.standard_normal((512, 40)).astype(np.float32))
    av = torch.from_numpy(rng.standard_normal((512, 40)).astype(np.float32))
    tp._set_factors(ps, ak, av)
    lr.lr_attn_check_shrink(4096)
    ps.project(0, torch.zeros(20, 512, dtype=torch.bfloat16, device="cuda:0"))
    torch.cuda.synchronize()
    lr.lr_attn_check_shrink(0)
    fired_proj = lr.lr_attn_check_count()
    ps.close()
    print(json.dumps({"random_plans": rs.N_CASES, "outside": outside, "outside_with_shrink": fired,
                      "ffn_outside": outside_ffn, "ffn_outside_with_shrink": fired_ffn,
                      "project_outside": outside_proj, "project_outside_with_shrink": fired_proj}), flush=True)


if __name__ == "__main__":
    main()
