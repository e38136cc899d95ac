"""The compiler's resource report of the last in-tree build
(``_build/kernel_resources.json``, written by ``build.py``): no kernel of
the library spills registers to scratch memory, and every absorbed decode
kernel runs at the wavefronts per SIMD its register budget was compiled for.
A spill to memory inside a streaming loop adds a scratch load, and the wait
for it, to every step.  (A spill into the accumulation registers, as the
int4 explicit kernels of the largest buckets have, is a register copy.)"""
import json
import os
import re

import pytest

RES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "latent_kv_attention_lr_amd", "_build", "kernel_resources.json")


def _report():
    if not os.path.exists(RES):
        pytest.skip("library not built in-tree (run latent_kv_attention_lr_amd/build.py)")
    with open(RES) as f:
        return json.load(f)


def test_every_kernel_is_reported():
    r = _report()
    for name in ("k_decode", "k_decode_explicit", "k_merge", "k_append", "k_project", "k_pack",
                 "k_ffn_quant", "k_ffn_in", "k_ffn_mid", "k_ffn_out"):
        assert any(f"{len(name)}{name}I" in k or f"{len(name)}{name}E" in k for k in r), name


def test_no_kernel_uses_scratch_memory():
    bad = {k: v for k, v in _report().items()
           if v.get("ScratchSize [bytes/lane]") != "0" or v.get("Dynamic Stack") != "False"}
    assert not bad, sorted(bad)


def test_absorbed_decode_kernels_do_not_spill():
    bad = {k: v for k, v in _report().items() if "8k_decodeILi" in k and v.get("VGPRs Spill") != "0"}
    assert not bad, sorted(bad)


def test_decode_kernels_keep_their_occupancy():
    # k_decode<QF, IOT, R, NW, LPT>: waves per SIMD of each (format, bucket)
    want = {(0, 32): 5, (0, 64): 3, (0, 96): 4, (0, 128): 3, (1, 32): 5, (1, 64): 4, (1, 96): 2, (1, 128): 2}
    seen = 0
    for k, v in _report().items():
        if "8k_decodeILi" not in k:
            continue
        # mangled template arguments: ILi<QF>E<IOT>Li<R>ELi<NW>ELi<LPT>E
        m = re.search(r"8k_decodeILi(\d)E[a-z]Li(\d+)ELi(\d+)ELi(\d)E", k)
        qf, r = int(m.group(1)), int(m.group(2))
        assert int(v["Occupancy [waves/SIMD]"]) == want[(qf, r)], (k, v)
        seen += 1
    assert seen >= 40
