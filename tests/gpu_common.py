"""Helpers shared by the GPU test modules: the library fixture and device transfers."""
import pytest
import torch

import synth

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def bsa():
    import block_sparse_attention_top_amd as m

    m.load()
    assert torch.cuda.is_available()
    return m


def to_dev(x, layout="bhnd"):
    """Copy a CPU tensor to the GPU, as [B,H,N,D] ("bhnd") or [B,N,H,D] storage ("bnhd")."""
    if layout == "bnhd":
        x = x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    t = x.to(DEV)
    assert t.stride() == x.stride()
    return t


def f64(t):
    return synth.to_f64(t.cpu())
