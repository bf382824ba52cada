"""Device-memory plumbing for the C ABI: uploads host arrays with torch and
fills the ABI's weight/config structs. Marshalling only; no arithmetic."""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import binding as B


def to_device(a, device="cuda"):
    """Copy a numpy array to the device byte for byte (uint16 is carried as
    int16, since both are raw bf16 bits here); device tensors pass through."""
    import torch
    if isinstance(a, torch.Tensor):
        return a.to(device).contiguous()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def model_config(shape, max_anchor_len: int, max_suffix_len: int) -> B.ModelConfig:
    return B.ModelConfig(
        n_layers=shape.n_layers, hidden=shape.hidden, n_q_heads=shape.n_q_heads,
        n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim, intermediate=shape.intermediate,
        vocab=shape.vocab, rope_theta=shape.rope_theta, rms_eps=shape.rms_eps,
        kv_dtype=B.DTYPE_FP8_E4M3 if shape.kv_fp8 else B.DTYPE_BF16,
        k_scale=shape.k_scale, v_scale=shape.v_scale,
        max_anchor_len=max_anchor_len, max_suffix_len=max_suffix_len,
        act_dtype=B.DTYPE_FP8_E4M3 if getattr(shape, "act_fp8", False) else B.DTYPE_BF16)


class DeviceModel:
    """Weights resident in HBM plus the ABI structs that point at them."""

    _LAYER_KEYS = ("attn_norm", "mlp_norm", "w_qkv", "w_o", "w_gate_up", "w_down",
                   "s_qkv", "s_o", "s_gate_up", "s_down")

    def __init__(self, shape, weights: dict, max_anchor_len: int, max_suffix_len: int,
                 device="cuda"):
        self.shape = shape
        self.cfg = model_config(shape, max_anchor_len, max_suffix_len)
        self.t = {k: to_device(weights[k], device) for k in ("embed", "final_norm", "head8")}
        self.layers = [{k: to_device(lw[k], device) for k in self._LAYER_KEYS}
                       for lw in weights["layers"]]
        arr = (B.LayerWeights * shape.n_layers)()
        for i, lw in enumerate(self.layers):
            for k in self._LAYER_KEYS:
                setattr(arr[i], k, lw[k].data_ptr())
        self._layer_arr = arr
        self.weights = B.Weights(embed=self.t["embed"].data_ptr(),
                                 layers=C.cast(arr, C.POINTER(B.LayerWeights)),
                                 final_norm=self.t["final_norm"].data_ptr(),
                                 head8=self.t["head8"].data_ptr())

    def context(self, pool_bytes: int, max_batch_tokens: int, device="cuda") -> B.Context:
        import torch
        ws_bytes = B.quail_workspace_bytes(self.cfg, max_batch_tokens)
        pool = torch.empty(max(pool_bytes, 256), dtype=torch.uint8, device=device)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        return B.Context(self.cfg, self.weights, pool, ws, max_batch_tokens)
