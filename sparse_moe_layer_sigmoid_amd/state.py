"""Checkpoint / resume of the layer's training-mode state.

The only state the forward changes is the per-expert routing bias b [N] (float32), moved by
+/- gamma after every step from that step's expert loads ("DeepSeek-V3 Technical Report",
"DeepSeekMoE と補助損失なしの負荷分散": the bias is adjusted from the load observed over
the batch).  A checkpoint therefore holds the bias bit pattern and the index of the next
step; the inputs of a step are regenerated from their seed and step index.

The file is safetensors (no code is executed when it is read).
"""
from __future__ import annotations

import torch
from safetensors.torch import load_file, save_file


def save_bias_state(path: str, layer, step: int) -> None:
    """Write ``layer.bias`` (its exact float32 values) and ``step`` (the next step to run)."""
    bias = layer.bias.detach().to("cpu", torch.float32).contiguous()
    save_file({"bias": bias, "step": torch.tensor([int(step)], dtype=torch.int64)}, path)


def load_bias_state(path: str, layer) -> int:
    """Restore ``layer.bias`` in place from a file written by ``save_bias_state`` and return
    the step index to resume from.  The bias shape must match the layer's."""
    st = load_file(path)
    bias, step = st["bias"], st["step"]
    if bias.dtype != torch.float32 or bias.shape != layer.bias.shape:
        raise ValueError(f"bias state {tuple(bias.shape)} {bias.dtype} does not fit the layer's "
                         f"{tuple(layer.bias.shape)} float32 bias")
    layer.bias.copy_(bias.to(layer.bias.device))
    return int(step[0])
