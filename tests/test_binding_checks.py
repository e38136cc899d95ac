"""Argument checks of the Python layer (session.py, ffn.py) that must raise
before anything is launched; the objects live on the CPU here, so a check
that let a bad argument through would reach the library with host pointers
and fail differently."""
import numpy as np
import pytest
import torch

import lrgen
import latent_kv_attention_lr_amd as lr
from latent_kv_attention_lr_amd.ffn import FfnLayer
from latent_kv_attention_lr_amd.session import DecodeSession


def _layer():
    layer = FfnLayer(128, 96, 32, 64, device="cpu")
    layer.set_weights(*lrgen.ffn_weights(lrgen.FfnWorkload("t", 128, 96, 32, 64, 2, 5)))
    return layer


@pytest.mark.parametrize("x", [torch.zeros(2, 128, dtype=torch.float32),      # dtype
                               torch.zeros(2, 64, dtype=torch.bfloat16),       # embed
                               torch.zeros(128, 4, dtype=torch.bfloat16).t(),  # not contiguous
                               torch.zeros(2, 2, 128, dtype=torch.bfloat16)])  # rank
def test_ffn_layer_rejects_bad_inputs(x):
    with pytest.raises(ValueError):
        _layer()(x)


@pytest.mark.parametrize("y", [torch.zeros(2, 128, dtype=torch.bfloat16), torch.zeros(3, 128),
                               torch.zeros(2, 64), torch.zeros(256, 2).t()])
def test_ffn_layer_rejects_bad_outputs(y):
    with pytest.raises(ValueError):
        _layer()(torch.zeros(2, 128, dtype=torch.bfloat16), y)


def test_ffn_layer_needs_weights_and_a_supported_shape():
    with pytest.raises(ValueError):
        FfnLayer(128, 96, 32, 64, device="cpu")(torch.zeros(1, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        FfnLayer(100, 96, 32, 64, device="cpu")


def _session():
    return DecodeSession(1, 2, 4, 64, lr.LR_Q_INT8_TOKEN, lr.LR_DT_BF16, [[32, 16, 8, 128]],
                         [[40, 96, 64, 8]], device="cpu")


@pytest.mark.parametrize("pos", [torch.zeros(2, dtype=torch.int64), torch.zeros(3, dtype=torch.int32),
                                 torch.zeros(4, dtype=torch.int32)[::2]])
def test_session_append_rejects_bad_pos(pos):
    s = _session()
    ck = torch.zeros(2, 1, s.latent_elems(0, 0))
    cv = torch.zeros(2, 1, s.latent_elems(0, 1))
    with pytest.raises(ValueError):
        s.append(0, ck, cv, pos)


def test_session_append_rejects_bad_latents():
    s = _session()
    pos = torch.zeros(2, dtype=torch.int32)
    good_k, good_v = torch.zeros(2, 1, s.latent_elems(0, 0)), torch.zeros(2, 1, s.latent_elems(0, 1))
    for ck, cv in [(good_k.double(), good_v), (good_k, torch.zeros(2, 1, 3)),
                   (torch.zeros(2, 2, s.latent_elems(0, 0))[:, :1], good_v)]:   # strided
        with pytest.raises(ValueError):
            s.append(0, ck, cv, pos)
