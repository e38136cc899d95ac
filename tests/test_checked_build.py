"""The checked build (liblr_attn_check.so, kernels built with LR_ATTN_CHECK=1):
every cache access of the append, decode and explicit kernels, and every
weight, workspace, input and output access of the FFN and latent-generation
kernels, is tested
against the extent of its buffer; one outside is counted and redirected
instead of faulting.  On the GPU, in a child process that loads that library,
the seeded random plans of test_gpu_random_shapes, the layout-edge decode
cases of test_gpu_parity, the FFN cases of test_ffn and the latent-generation
cases of test_gpu_project (tests/check_battery.py)
make no access outside their buffers, and shrinking the tested extents makes
the check fire.  On the CPU, the
release library answers the check calls with LR_EUNSUPPORTED."""
import json
import os
import subprocess
import sys

import pytest

import latent_kv_attention_lr_amd as lr

HERE = os.path.dirname(os.path.abspath(__file__))
CHECK_LIB = os.path.join(os.path.dirname(HERE), "latent_kv_attention_lr_amd", "liblr_attn_check.so")


def test_release_library_has_no_check():
    if os.path.basename(lr.LIB_PATH) == "liblr_attn_check.so":
        pytest.skip("this process loaded the checked library")
    for call in (lambda: lr.lr_attn_check_count(), lambda: lr.lr_attn_check_shrink(0)):
        with pytest.raises(lr.LrAttnError) as e:
            call()
        assert e.value.status == lr.LR_EUNSUPPORTED


@pytest.mark.gpu
def test_checked_kernels_stay_inside_their_caches():
    assert os.path.exists(CHECK_LIB), "build the library first (latent_kv_attention_lr_amd/build.py)"
    print("checked build: random plans in a child process", flush=True)
    env = dict(os.environ, LR_ATTN_LIB=CHECK_LIB)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "check_battery.py")], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    print(d, flush=True)
    assert d["outside"] == 0 and d["ffn_outside"] == 0 and d["project_outside"] == 0, d
    assert d["outside_with_shrink"] > 0 and d["ffn_outside_with_shrink"] > 0, d
    assert d["project_outside_with_shrink"] > 0, d
