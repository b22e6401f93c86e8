"""CPU checks of the torch binding (no GPU): every entry point that takes a `stream` runs its
body with that stream current, so the buffers it allocates belong to that stream's pool."""
import contextlib
import inspect

import torch

from block_sparse_attention_top_amd import ops


def test_every_stream_entry_point_allocates_on_its_stream():
    names = [n for n, f in inspect.getmembers(ops, inspect.isfunction)
             if (n.startswith("recap_") or n == "sparse_step") and f.__module__ == ops.__name__
             and "stream" in inspect.signature(f).parameters]
    assert len(names) >= 15, names
    for n in names:
        assert getattr(getattr(ops, n), "on_stream", False), n


def test_on_stream_enters_the_given_stream(monkeypatch):
    entered = []

    @contextlib.contextmanager
    def fake_stream(s):
        entered.append(s)
        yield

    monkeypatch.setattr(torch.cuda, "stream", fake_stream)

    @ops._on_stream
    def f(a, b=None, stream=None):
        return (a, b, len(entered))

    assert f(1) == (1, None, 0) and entered == []
    assert f(1, 2, "side") == (1, 2, 1) and entered == ["side"]
    assert f(1, stream="other") == (1, None, 2) and entered == ["side", "other"]
