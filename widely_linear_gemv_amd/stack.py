"""One decode step over a stack of widely-linear layers, as grouped launches.

Sources: ModelScope card "Fairy2i-W2", "Method" (every linear layer of the model becomes a
widely-linear layer y = U x + W conj(x)); 36Kr article, parallel stages (the stage terms, and
the projections that read the same input, are independent).

Per transformer layer the seven projections form four groups by their input: q, k and v share x;
o reads its own; gate and up share x; down reads its own.  A group is one grouped GEMV launch, so
a 32-layer stack is 128 launches, captured once in a HIP graph and replayed.  By default (AUTO)
the launches take the bf16 x as it is: at batch 1 the fp4 kernel digitizes x on chip, each wave
the chunks it multiplies (these launches are small, 4-23 MB, and a separate digit-form launch per
group would cost more than it saves), at larger batches the bf16 kernel runs.  With algo=GEMV_MFMA_F4
or GEMV_MFMA_I8 each group first makes the digit form of its x in a launch of its own; with
digits_given=True the digit forms are made once when the step is built and the step runs the
GEMVs alone (for inputs that arrive in digit form, from a producer that writes it).  This module only sequences
calls of the C ABI (through the binding); all arithmetic runs in the library's kernels.
"""
from __future__ import annotations

import torch

from . import (GEMV_AUTO, GEMV_MFMA_F4, GEMV_MFMA_I8, X_DIGITS, X_DIGITS_F6, XDigits,
               fairy2i_gemv_grouped, fairy2i_x_digits, fairy2i_x_digits_bytes, fairy2i_x_digits_f6,
               fairy2i_x_digits_f6_bytes)

# the digit form each digit-form kernel takes: (size in bytes, converter, dtype code)
_DIGIT_FORMS = {GEMV_MFMA_F4: (fairy2i_x_digits_f6_bytes, fairy2i_x_digits_f6, X_DIGITS_F6),
                GEMV_MFMA_I8: (fairy2i_x_digits_bytes, fairy2i_x_digits, X_DIGITS)}

# LLaMA-2 7B projections of one layer: name, real rows (2n), real columns (2m), input group
PROJECTIONS = (("q", 4096, 4096, 0), ("k", 4096, 4096, 0), ("v", 4096, 4096, 0), ("o", 4096, 4096, 1),
               ("gate", 11008, 4096, 2), ("up", 11008, 4096, 2), ("down", 4096, 11008, 3))
GROUPS = 4


class DecodeStep:
    """layers[L][p] = (packed, scales) for projection p of layer L (shapes as PROJECTIONS);
    xs[L][g] = bf16 input [B][2m] of group g of layer L.  Outputs: self.ys[L][p] fp32 [B][2n].
    digits_given (digit-form algos only): make each x's digit form once, here, instead of in
    every run()."""

    def __init__(self, layers, xs, *, algo: int | None = None, digits_given: bool = False):
        self.layers, self.xs = layers, xs
        B = xs[0][0].shape[0]
        self.B = B
        self.algo = algo if algo is not None else GEMV_AUTO
        dev = xs[0][0].device
        self.ys = [[torch.empty((B, rows), dtype=torch.float32, device=dev)
                    for (_, rows, _, _) in PROJECTIONS] for _ in layers]
        self.digits = None
        if digits_given and self.algo not in _DIGIT_FORMS:
            raise ValueError("digits_given needs a digit-form algo (GEMV_MFMA_F4 or GEMV_MFMA_I8)")
        self.digits_given = digits_given
        if self.algo in _DIGIT_FORMS:
            nbytes, self._convert, code = _DIGIT_FORMS[self.algo]
            self.digits = [[XDigits(torch.empty((nbytes(x.shape[1] // 2, B),), dtype=torch.uint8, device=dev),
                                    B, x.shape[1] // 2, code)
                            for x in layer_xs] for layer_xs in xs]
            if digits_given:
                for layer_xs, layer_digits in zip(xs, self.digits):
                    for x, d in zip(layer_xs, layer_digits):
                        self._convert(x, out=d)

    def run(self, stream=None):
        for L, projs in enumerate(self.layers):
            for g in range(GROUPS):
                x = self.xs[L][g]
                if self.digits_given:
                    x = self.digits[L][g]
                elif self.digits is not None:
                    x = self._convert(x, out=self.digits[L][g], stream=stream)
                items = [(projs[p][0], projs[p][1], x, self.ys[L][p])
                         for p, (_, _, _, grp) in enumerate(PROJECTIONS) if grp == g]
                fairy2i_gemv_grouped(items, algo=self.algo, stream=stream)
        return self.ys

    def capture(self):
        """Capture one step into a HIP graph (on a side stream); returns the graph."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream()):
            self.run()
        return g
