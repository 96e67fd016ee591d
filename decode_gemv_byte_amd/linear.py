"""A torch module over the C ABI: a BF16 linear layer whose weight stays
compressed in GPU memory.

NWC converts a model's ``nn.Linear`` layers into compressed ones that run the
fused decode-GEMV ("NWC -- Neural Weight Compression", How it works, and its
usage section on fusing and converting a model); this module is the same
idea over this library's entry points.  ``forward`` picks the path by the
number of input rows:

* 1 row: ``nwc_gemv`` (fused decode-GEMV),
* 2..16 rows (up to 32 with 8-row tiles): ``nwc_gemm_skinny`` (fused skinny
  decode-GEMM, from 5 rows on the matrix cores),
* more: ``nwc_gemm_prefill`` (decode into a scratch buffer + hipBLASLt GEMM).

All arithmetic runs in the library's kernels (and hipBLASLt for prefill);
the bias, if any, is added by torch.  The module owns its workspaces, so
calls on one module must be ordered on one stream (the current stream is
used).  Quality and perplexity on trained weights are outside this
package: the tests check the products against the dense BF16 layer.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import (Blas, nwc_decode, nwc_encode, nwc_gemm_prefill, nwc_gemm_skinny, nwc_gemv, nwc_inspect,
               nwc_prefill_workspace_size, nwc_workspace_size)

SKINNY_MAX = 16      # any tile height
SKINNY_MAX_MC = 32   # 8-row tiles (the matrix-core skinny GEMM)


class NWCLinear(torch.nn.Module):
    """y = x W^T (+ b) with W [out, in] held as a compressed blob on the GPU."""

    def __init__(self, blob: np.ndarray, bias: Optional[torch.Tensor] = None, device=None):
        super().__init__()
        device = torch.device(device or "cuda")
        self.info = nwc_inspect(blob)
        self.in_features = int(self.info.cols)
        self.out_features = int(self.info.rows)
        self.register_buffer("blob", torch.from_numpy(np.ascontiguousarray(blob)).to(device), persistent=True)
        self.bias = None if bias is None else torch.nn.Parameter(
            bias.detach().to(device=device, dtype=torch.bfloat16), requires_grad=False)
        # the batch-1 workspace must start zero-filled; the library leaves it so
        self._ws1 = torch.zeros(max(1, nwc_workspace_size(self.info, 1)), dtype=torch.uint8, device=device)
        self._ws = {}        # batch -> skinny workspace
        self._prefill = None  # (Blas, workspace), made on first use

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, params=None, device=None) -> "NWCLinear":
        """Compress a linear layer's weight (rounded to BF16 if it is not) on the host."""
        w = linear.weight.detach().to(torch.bfloat16).cpu().contiguous()
        bits = w.view(torch.int16).numpy().view(np.uint16)
        blob = nwc_encode(bits, params)
        dev = device or (linear.weight.device if linear.weight.is_cuda else "cuda")
        return cls(blob, linear.bias, dev)

    def compressed_bytes(self) -> int:
        return int(self.blob.numel())

    def dense_weight(self) -> torch.Tensor:
        """The exact BF16 weight, decoded into a new [out, in] tensor."""
        ld = (self.in_features + 7) // 8 * 8
        out = torch.empty((self.out_features, ld), dtype=torch.int16, device=self.blob.device)
        nwc_decode(self.info, self.blob, out, ld)
        return out[:, :self.in_features].contiguous().view(torch.bfloat16)

    def _workspace(self, batch: int):
        if batch not in self._ws:
            n = nwc_workspace_size(self.info, batch)
            self._ws[batch] = torch.zeros(n, dtype=torch.uint8, device=self.blob.device) if n else None
        return self._ws[batch]

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError("expected %d input features, got %d" % (self.in_features, x.shape[-1]))
        lead = x.shape[:-1]
        X = x.reshape(-1, self.in_features).to(torch.bfloat16).contiguous()
        B = X.shape[0]
        Xb = X.view(torch.int16)
        if B == 1:
            y = torch.empty(self.out_features, dtype=torch.bfloat16, device=x.device)
            nwc_gemv(self.info, self.blob, Xb[0], y, self._ws1)
            Y = y.view(1, -1)
        elif B <= (SKINNY_MAX_MC if self.info.tile_rows == 8 else SKINNY_MAX):
            Y = torch.empty((B, self.out_features), dtype=torch.bfloat16, device=x.device)
            nwc_gemm_skinny(self.info, self.blob, Xb, Y, self._workspace(B))
        else:
            if self._prefill is None:
                ws = torch.empty(nwc_prefill_workspace_size(self.info), dtype=torch.uint8, device=self.blob.device)
                self._prefill = (Blas(), ws)
            blas, ws = self._prefill
            # the GEMM takes rows 16 bytes apart: pad odd feature counts
            ldx, ldy = (self.in_features + 7) // 8 * 8, (self.out_features + 7) // 8 * 8
            if ldx != self.in_features:
                Xp = torch.zeros((B, ldx), dtype=torch.int16, device=x.device)
                Xp[:, :self.in_features] = Xb
                Xb = Xp[:, :self.in_features]
            Y = torch.empty((B, ldy), dtype=torch.bfloat16, device=x.device)[:, :self.out_features]
            nwc_gemm_prefill(blas, self.info, self.blob, Xb, Y, ws)
        if self.bias is not None:
            Y = Y + self.bias
        return Y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return "in_features=%d, out_features=%d, compressed=%.4f B/weight, bias=%s" % (
            self.in_features, self.out_features, self.compressed_bytes() / (self.in_features * self.out_features),
            self.bias is not None)


def convert(module: torch.nn.Module, params=None, device=None) -> torch.nn.Module:
    """Replace every nn.Linear inside `module` (in place) with an NWCLinear."""
    for name, child in list(module.named_children()):
        if isinstance(child, torch.nn.Linear):
            setattr(module, name, NWCLinear.from_linear(child, params, device))
        else:
            convert(child, params, device)
    return module
