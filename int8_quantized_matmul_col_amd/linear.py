"""An 8-bit linear layer (forward only) over the library's C ABI.

"PyTorch 2.9 supports LLM.int8()" swaps the ``nn.Linear`` layers of a model
for an 8-bit layer that keeps no fp16 copy of its weight
(``has_fp16_weights=False`` in its ``Linear8bitLt`` example), quantizes the
weight once, on first use (its notes put the cost of that one-time step on
the first inference), and leaves small layers in fp16 (a size threshold on
``in_features``).  "8-bit quantization in practice" (section 5.2) also skips
chosen modules by name, typically ``lm_head``.

``Int8Linear`` is that layer on this library: the weight is prepared with
``int8_prepare_weight`` the first time the layer runs on a GPU (or when
``quantize_()`` is called), after which the layer holds only the int8 weight,
its per-channel scales and the fp16 bias (its state dict then carries ``Wq``
and ``w_scale``, and loads back without re-quantizing); ``forward`` is one
``int8_linear`` call.  No arithmetic of the method runs here: inputs are
reshaped to 2-D and handed to the HIP kernels as they are.
"""

from __future__ import annotations

from typing import Iterable, Optional

import torch

from . import binding


class Int8Linear(torch.nn.Module):
    """y = x W^T + b with W held as int8 (per-channel absmax scales) and the
    input split into outlier and regular columns on every call.

    x must be float16 on the layer's GPU, shape [..., in_features]; the
    result is float16 [..., out_features].
    """

    def __init__(self, in_features: int, out_features: int, bias: bool = True,
                 threshold: float = binding.DEFAULT_THRESHOLD, device=None):
        super().__init__()
        if threshold != threshold or threshold < 0:
            raise ValueError("threshold must be a non-negative number")
        self.in_features = int(in_features)
        self.out_features = int(out_features)
        self.threshold = float(threshold)
        # fp16 weight until the first forward on a GPU (or quantize_())
        self.weight = torch.nn.Parameter(
            torch.empty((self.out_features, self.in_features), dtype=torch.float16,
                        device=device), requires_grad=False)
        self.register_buffer("Wq", None)
        self.register_buffer("w_scale", None)
        if bias:
            self.bias = torch.nn.Parameter(
                torch.zeros((self.out_features,), dtype=torch.float16, device=device),
                requires_grad=False)
        else:
            self.register_parameter("bias", None)

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear,
                    threshold: float = binding.DEFAULT_THRESHOLD) -> "Int8Linear":
        """The 8-bit layer of a float16 nn.Linear (weight and bias copied;
        quantized on first use)."""
        if linear.weight.dtype != torch.float16:
            raise TypeError(f"expected a float16 nn.Linear, got {linear.weight.dtype}")
        m = cls(linear.in_features, linear.out_features, linear.bias is not None, threshold,
                device=linear.weight.device)
        with torch.no_grad():
            m.weight.copy_(linear.weight)
            if linear.bias is not None:
                m.bias.copy_(linear.bias)
        return m

    @property
    def quantized(self) -> bool:
        return self.Wq is not None

    @torch.no_grad()
    def quantize_(self) -> "Int8Linear":
        """One-time per-channel quantization of the fp16 weight (on its GPU);
        the fp16 weight is dropped afterwards."""
        if self.quantized:
            return self
        w = self.weight
        if not w.is_cuda:
            raise RuntimeError("Int8Linear quantizes on a GPU: move the layer there first")
        Wq, ws = binding.int8_prepare_weight(w.detach().contiguous())
        self.Wq = Wq
        self.w_scale = ws
        self.weight = None
        return self

    def _load_from_state_dict(self, state_dict, prefix, local_metadata, strict, missing_keys,
                              unexpected_keys, error_msgs):
        # a saved 8-bit layer carries Wq and w_scale instead of the fp16
        # weight: take them as they are (no re-quantization)
        kq, ks, kw = prefix + "Wq", prefix + "w_scale", prefix + "weight"
        if kq in state_dict and ks in state_dict:
            Wq, ws = state_dict[kq], state_dict[ks]
            ldk = (self.in_features + 63) // 64 * 64
            Np = (self.out_features + 255) // 256 * 256
            if tuple(Wq.shape) != (Np, ldk) or Wq.dtype != torch.int8:
                error_msgs.append(f"{kq}: expected int8 {(Np, ldk)}, got {Wq.dtype} "
                                  f"{tuple(Wq.shape)}")
                return
            if tuple(ws.shape) != (self.out_features,) or ws.dtype != torch.float32:
                error_msgs.append(f"{ks}: expected float32 ({self.out_features},), got "
                                  f"{ws.dtype} {tuple(ws.shape)}")
                return
            dev = self.bias.device if self.bias is not None else (
                self.weight.device if self.weight is not None else Wq.device)
            self.Wq = Wq.detach().to(dev).clone()
            self.w_scale = ws.detach().to(dev).clone()
            self.weight = None
            if self.bias is not None:
                kb = prefix + "bias"
                if kb in state_dict:
                    with torch.no_grad():
                        self.bias.copy_(state_dict[kb])
                elif strict:
                    missing_keys.append(kb)
            if kw in state_dict:
                unexpected_keys.append(kw)
            return
        if self.weight is None:
            # a quantized layer loading an fp16 weight: back to the fp16 form
            if kw in state_dict:
                self.weight = torch.nn.Parameter(torch.empty(
                    (self.out_features, self.in_features), dtype=torch.float16,
                    device=self.Wq.device), requires_grad=False)
                self.Wq = None
                self.w_scale = None
        super()._load_from_state_dict(state_dict, prefix, local_metadata, strict, missing_keys,
                                      unexpected_keys, error_msgs)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.dtype != torch.float16:
            raise TypeError(f"Int8Linear takes float16 inputs, got {x.dtype}")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"last dimension {x.shape[-1]} != in_features {self.in_features}")
        if not self.quantized:
            self.quantize_()
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        y = binding.int8_linear(x2, self.Wq, self.w_scale, self.bias, self.threshold)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, threshold={self.threshold}, "
                f"quantized={self.quantized}")


def replace_linear_with_int8(module: torch.nn.Module,
                             threshold: float = binding.DEFAULT_THRESHOLD,
                             min_in_features: int = 0,
                             skip_modules: Iterable[str] = ("lm_head",),
                             _prefix: str = "") -> torch.nn.Module:
    """Replaces, in place, every float16 nn.Linear of ``module`` by an
    Int8Linear, except layers with fewer than ``min_in_features`` inputs and
    layers whose own name or qualified name (``block.q_proj``) is in
    ``skip_modules``.
    Returns ``module``."""
    skip = set(skip_modules or ())
    for name, child in list(module.named_children()):
        qual = f"{_prefix}.{name}" if _prefix else name
        if qual in skip or name in skip:
            continue
        if isinstance(child, torch.nn.Linear) and not isinstance(child, Int8Linear):
            if child.weight.dtype == torch.float16 and child.in_features >= min_in_features:
                setattr(module, name, Int8Linear.from_linear(child, threshold))
        else:
            replace_linear_with_int8(child, threshold, min_in_features, skip, qual)
    return module


__all__ = ["Int8Linear", "replace_linear_with_int8"]
