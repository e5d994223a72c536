"""Seeded inputs of the indexer prolog: the hidden rows x, the two projection
weights, each row's new index key before normalisation and the norm's weight,
all bf16, on any torch device.  Random draws only, none of the prolog's
arithmetic.

Shapes: x [rows, D_x], w_q [H_I * D_I, D_x], w_g [H_I, D_x], k_new
[rows, D_I], k_gamma [D_I].  The input width defaults to 4096, the input
dimension THInfer fixes for its Linear-operator measurements (experiments,
part D); the pages give no model width for the indexer.

Modes:
* "int": x in {-2..2}, both weights in {-1, 0, 1}, k_new in {-3..3},
  k_gamma in {1, 2} -- every projection sum is an integer below 2**24, exact
  in float32 in any order;
* "gauss": x and k_new N(0, 1), weights N(0, 1) / sqrt(D_x) (so q and g are
  of order 1), k_gamma 1 + N(0, 0.1^2); all rounded to bf16 by torch.
"""

from dataclasses import dataclass

import torch

#: input width of the prolog's projections
PROLOG_D_X = 4096


@dataclass
class PrologInputs:
    x: torch.Tensor        # bf16 [rows, D_x]
    w_q: torch.Tensor      # bf16 [H_I * D_I, D_x]
    w_g: torch.Tensor      # bf16 [H_I, D_x]
    k_new: torch.Tensor    # bf16 [rows, D_I]
    k_gamma: torch.Tensor  # bf16 [D_I]

    @property
    def rows(self) -> int:
        return self.x.shape[0]

    @property
    def D_x(self) -> int:
        return self.x.shape[1]


def make_prolog_inputs(rows, H_I, D_I, D_x=PROLOG_D_X, mode="gauss", seed=0, device="cpu",
                       key_pm4=False):
    """Draw the prolog's inputs for ``rows`` rows from ``seed``.  ``key_pm4``:
    every new-key element is +4 or -4 (random signs), a key whose RMS is
    exactly 4."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed * 104729 + 31)
    bf = torch.bfloat16

    def ints(shape, lo, hi):
        return torch.randint(lo, hi + 1, shape, generator=g, device=device).to(bf)

    def normal(shape, std=1.0):
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std).to(bf)

    if mode == "int":
        x = ints((rows, D_x), -2, 2)
        w_q = ints((H_I * D_I, D_x), -1, 1)
        w_g = ints((H_I, D_x), -1, 1)
        k_new = ints((rows, D_I), -3, 3)
        k_gamma = ints((D_I,), 1, 2)
    elif mode == "gauss":
        x = normal((rows, D_x))
        w_q = normal((H_I * D_I, D_x), D_x ** -0.5)
        w_g = normal((H_I, D_x), D_x ** -0.5)
        k_new = normal((rows, D_I))
        k_gamma = (1.0 + 0.1 * torch.randn((D_I,), generator=g, device=device)).to(bf)
    else:
        raise ValueError(f"mode {mode!r}")
    if key_pm4:
        signs = torch.randint(0, 2, (rows, D_I), generator=g, device=device)
        k_new = (signs * 8 - 4).to(bf)
    return PrologInputs(x=x, w_q=w_q, w_g=w_g, k_new=k_new, k_gamma=k_gamma)


def prolog_arrays(inp: PrologInputs) -> dict:
    """The inputs as numpy uint16 bf16 bit patterns, for the oracle."""
    def bits(t):
        return t.detach().cpu().view(torch.int16).numpy().view("uint16")
    return {"x": bits(inp.x), "w_q": bits(inp.w_q), "w_g": bits(inp.w_g),
            "k_new": bits(inp.k_new), "k_gamma": bits(inp.k_gamma)}
