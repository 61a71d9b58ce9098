"""Saving and loading int8 weight states (codes + row absmax): host-side round
trips and the checks on read-back.  The GPU round trip through the library's
weight quantization is in test_gpu_parity.py."""

import numpy as np
import pytest
import torch

from int8_mixed_precision_vectorwise_amd.serialize import FORMAT, load_int8_weights, save_int8_weights


def _pair(n, k, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randint(-127, 128, (n, k), generator=g, dtype=torch.int64).to(torch.int8)
    s = torch.rand(n, generator=g, dtype=torch.float32) * 3.0
    return q, s


def test_round_trip_exact(tmp_path):
    w = {"model.layers.0.mlp.up": _pair(33, 70, 1), "model.layers.0.mlp.down": _pair(70, 33, 2),
         "tiny": _pair(1, 1, 3)}
    p = str(tmp_path / "w.safetensors")
    save_int8_weights(p, w, metadata={"source": "unit test"})
    back = load_int8_weights(p)
    assert set(back) == set(w)
    for name, (q, s) in w.items():
        assert torch.equal(back[name][0], q) and back[name][0].dtype == torch.int8
        assert torch.equal(back[name][1], s) and back[name][1].dtype == torch.float32


def test_bad_pairs_rejected(tmp_path):
    p = str(tmp_path / "w.safetensors")
    q, s = _pair(4, 8, 4)
    with pytest.raises(ValueError):
        save_int8_weights(p, {"w": (q.to(torch.int16), s)})
    with pytest.raises(ValueError):
        save_int8_weights(p, {"w": (q, s[:3])})
    with pytest.raises(ValueError):
        save_int8_weights(p, {"w": (q, s.double())})


def test_foreign_or_incomplete_files_rejected(tmp_path):
    from safetensors.torch import save_file
    q, s = _pair(4, 8, 5)
    p = str(tmp_path / "a.safetensors")
    save_file({"w.weight_int8": q, "w.row_absmax": s}, p, metadata={"format": "something else"})
    with pytest.raises(ValueError):
        load_int8_weights(p)
    save_file({"w.weight_int8": q}, p, metadata={"format": FORMAT})
    with pytest.raises(ValueError):
        load_int8_weights(p)
    save_file({"w.row_absmax": s}, p, metadata={"format": FORMAT})
    with pytest.raises(ValueError):
        load_int8_weights(p)
    save_file({"w.weight_int8": q, "w.row_absmax": s, "w.bias": s.clone()}, p, metadata={"format": FORMAT})
    with pytest.raises(ValueError):
        load_int8_weights(p)
