"""Saving and loading row-wise int8 weight states: the codes with their row absmax.

A quantized weight is usable only together with its quantization statistics;
the transformers integration page ("`bitsandbytes` - `Linear8bitLt`
integration into `transformers` models") records that saved int8 checkpoints
could not be reloaded while those statistics were missing from the saved
state.  Here both are written side by side into one safetensors file (plain
tensors, nothing pickled), with the format recorded in the file's metadata,
and both are checked when read back.

Layout of one weight `name`:
  `name.weight_int8`  int8 [out_features, in_features], row-major
  `name.row_absmax`   float32 [out_features]
and the weight they stand for is weight_int8 * row_absmax / 127 row by row
(the codes of the library's weight quantization, `quantize_weight`).
"""

from __future__ import annotations

from typing import Dict, Mapping, Optional, Tuple

import torch

FORMAT = "i8mp-int8-rowwise-absmax-v1"
_Q, _S = "weight_int8", "row_absmax"


def _check_pair(name: str, q: torch.Tensor, s: torch.Tensor) -> None:
    if q.dtype != torch.int8 or q.dim() != 2:
        raise ValueError(f"{name}: codes must be a 2-D int8 tensor, got {q.dtype} {tuple(q.shape)}")
    if s.dtype != torch.float32 or s.dim() != 1 or s.shape[0] != q.shape[0]:
        raise ValueError(f"{name}: row absmax must be float32 [{q.shape[0]}], got {s.dtype} {tuple(s.shape)}")


def save_int8_weights(path: str, weights: Mapping[str, Tuple[torch.Tensor, torch.Tensor]],
                      metadata: Optional[Mapping[str, str]] = None) -> None:
    """Write {name: (codes int8 [n, k], row absmax float32 [n])} to a safetensors file."""
    from safetensors.torch import save_file

    tensors: Dict[str, torch.Tensor] = {}
    for name, (q, s) in weights.items():
        _check_pair(name, q, s)
        tensors[f"{name}.{_Q}"] = q.detach().contiguous().cpu()
        tensors[f"{name}.{_S}"] = s.detach().contiguous().cpu()
    meta = {str(k): str(v) for k, v in (metadata or {}).items()}
    meta.update({"format": FORMAT, "scale": "weight = weight_int8 * row_absmax / 127, per row",
                 "layout": "row-major [out_features, in_features]"})
    save_file(tensors, path, metadata=meta)


def load_int8_weights(path: str, device: Optional[torch.device | str] = None
                      ) -> Dict[str, Tuple[torch.Tensor, torch.Tensor]]:
    """Read a file written by save_int8_weights; tensors go to `device` (host if None)."""
    from safetensors import safe_open

    out: Dict[str, Tuple[torch.Tensor, torch.Tensor]] = {}
    with safe_open(path, framework="pt", device="cpu") as f:
        meta = f.metadata() or {}
        if meta.get("format") != FORMAT:
            raise ValueError(f"{path}: not an int8 weight file of format {FORMAT} (found {meta.get('format')!r})")
        keys = set(f.keys())
        names = {k[: -len(_Q) - 1] for k in keys if k.endswith("." + _Q)}
        for k in keys:
            if not (k.endswith("." + _Q) or k.endswith("." + _S)):
                raise ValueError(f"{path}: unexpected tensor {k!r}")
            base = k.rsplit(".", 1)[0]
            if base not in names:
                raise ValueError(f"{path}: {base!r} has row absmax but no codes")
        for name in sorted(names):
            if f"{name}.{_S}" not in keys:
                raise ValueError(f"{path}: {name!r} has codes but no row absmax")
            q = f.get_tensor(f"{name}.{_Q}")
            s = f.get_tensor(f"{name}.{_S}")
            _check_pair(name, q, s)
            if device is not None:
                q, s = q.to(device), s.to(device)
            out[name] = (q, s)
    return out
