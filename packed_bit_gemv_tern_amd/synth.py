"""Seeded synthetic inputs for the ternary linear layer.

This module only draws inputs: int8 ternary weight matrices, per-row scales,
int8 activations and per-token scale / zero point.  It holds none of the
method's arithmetic (no packing, no sums, no scaling), so the HIP library's
tests and the CPU oracle can both take their inputs from it.

Shapes and value distributions follow the Neutrino-1 pages:
  * 8B geometry: 36 decoder layers, hidden 4,096, 32 query / 8 key-value heads
    of width 128, SwiGLU feed-forward 12,288, seven linears per layer
    (Neutrino-1 8B model card, "Architecture"; article "Neutrino-1:
    quantization is a training decision ...", "What's actually ternary");
  * 0.6B geometry: 28 layers, hidden 1,024, 16 query / 8 key-value heads of
    width 128, 196 transformer linears (Fermion Research models page,
    "The family" and "Neutrino-1 0.6B");
  * state mix: 62.63 % zero, 18.68 % plus, 18.69 % minus over the 8B; the
    attention projections sit near 62 % zero at every depth while gate and
    down rise to about 70-72.5 % zero in the earliest feed-forward blocks
    (article, "Sparsity is learned, not imposed"; model card, "Inside the
    coded lane").  Layer numbers below are 0-based, the reading under which
    the article's 1-based "down 72.47 % at layer 3, gate 70.48 % at layer 4"
    and the wiki's "down 72.5 % at layer 2, gate 70.5 % at layer 3" agree.

Recipe (numpy PCG64 ``default_rng``).  Linear ``idx`` (0..6 in the order q,
k, v, o, gate, up, down) of layer ``layer`` draws its weights from
``default_rng([seed, layer, idx])``:
  1. W: one float32 uniform u per weight in row-major order; w = -1 if
     u < p_minus, 0 if u < p_minus + p_zero, else +1, with
     p_minus = p_plus = (1 - p_zero) / 2;
  2. s_row: ``uniform(0.01, 0.1, N)`` rounded to float32;
and its M tokens of activations from ``default_rng([seed, layer, idx, M])``:
  3. q: ``integers(-128, 127, (M, K), int8, endpoint=True)``;
  4. per-token parameters: for M = 1, s_act = 0.02 and z = 3; for M > 1,
     s_act = ``uniform(0.01, 0.03, M)`` (float32) then z = ``integers(-8, 9, M)``.
The same weights therefore serve every M.  Block-wise scales (one per block
of B columns) come from ``default_rng([seed, layer, idx, 2**20, B])``:
``uniform(0.01, 0.1, (N, ceil(K / B)))`` rounded to float32.
"""
from __future__ import annotations

import concurrent.futures as _cf
from dataclasses import dataclass

import numpy as np

# (name, N rows = output features, K = input features), in layer order.
LAYER_8B = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 12288, 4096),
    ("up", 12288, 4096),
    ("down", 4096, 12288),
)
LAYERS_8B = 36

LAYER_06B = (
    ("q", 2048, 1024),
    ("k", 1024, 1024),
    ("v", 1024, 1024),
    ("o", 1024, 2048),
    ("gate", 3072, 1024),
    ("up", 3072, 1024),
    ("down", 1024, 3072),
)
LAYERS_06B = 28

P_ZERO_DEFAULT = 0.626
P_ZERO_ATTENTION = 0.62

# Linears of a decoder layer that read the same input (both tables above use
# the order q, k, v, o, gate, up, down): the query, key and value projections
# all take the layer's normalised hidden state, and the gate and up
# projections of the gated feed-forward block take the same input (model
# card "Architecture": grouped-query attention, SwiGLU).  Entry idx is the
# linear whose activations linear idx reads.
INPUT_LEADER = (0, 0, 0, 3, 4, 4, 6)

# 0-based layer -> zero share, for the feed-forward spike.
_DOWN_SPIKE = {0: 0.6059, 1: 0.70, 2: 0.7247, 3: 0.70}
_GATE_SPIKE = {1: 0.70, 2: 0.70, 3: 0.7048}


def zero_rate_8b(layer: int, name: str) -> float:
    """Zero share for one linear of the 8B-shaped stack."""
    if name in ("q", "k", "v", "o"):
        return P_ZERO_ATTENTION
    if name == "down":
        return _DOWN_SPIKE.get(layer, P_ZERO_DEFAULT)
    if name == "gate":
        return _GATE_SPIKE.get(layer, P_ZERO_DEFAULT)
    return P_ZERO_DEFAULT


def ternary(rng: np.random.Generator, N: int, K: int, p_zero: float) -> np.ndarray:
    """(N, K) int8 matrix with entries -1 / 0 / +1 (step 1 of the recipe)."""
    u = rng.random((N, K), dtype=np.float32)
    p_minus = np.float32((1.0 - p_zero) / 2.0)
    upper = np.float32(p_minus + np.float32(p_zero))
    # (u >= p_minus) + (u >= upper) - 1 is -1, 0 or +1
    w = (u >= p_minus).view(np.int8) + (u >= upper).view(np.int8)
    w -= np.int8(1)
    return w


def token_params(rng: np.random.Generator, M: int):
    """(s_act float32 (M,), z int32 (M,)) -- step 4 of the recipe."""
    if M == 1:
        return np.array([0.02], np.float32), np.array([3], np.int32)
    s_act = rng.uniform(0.01, 0.03, M).astype(np.float32)
    z = rng.integers(-8, 9, M).astype(np.int32)
    return s_act, z


def activations(rng: np.random.Generator, M: int, K: int) -> np.ndarray:
    return rng.integers(-128, 127, (M, K), dtype=np.int8, endpoint=True)


@dataclass
class Linear:
    """Inputs of one linear: W (N, K) int8, s_row (N,), q (M, K), s_act / z (M,)."""
    name: str
    w: np.ndarray
    s_row: np.ndarray
    q: np.ndarray
    s_act: np.ndarray
    z: np.ndarray

    @property
    def N(self) -> int:
        return self.w.shape[0]

    @property
    def K(self) -> int:
        return self.w.shape[1]

    @property
    def M(self) -> int:
        return self.q.shape[0]


def make_weights(seed, layer: int, idx: int, N: int, K: int, p_zero: float):
    """(W int8 (N, K), s_row float32 (N,)) -- steps 1-2 of the recipe."""
    rng = np.random.default_rng([seed, layer, idx])
    w = ternary(rng, N, K, p_zero)
    s_row = rng.uniform(0.01, 0.1, N).astype(np.float32)
    return w, s_row


def make_activations(seed, layer: int, idx: int, K: int, M: int):
    """(q int8 (M, K), s_act float32 (M,), z int32 (M,)) -- steps 3-4."""
    rng = np.random.default_rng([seed, layer, idx, M])
    q = activations(rng, M, K)
    s_act, z = token_params(rng, M)
    return q, s_act, z


def make_hidden(seed, layer: int, idx: int, K: int, M: int) -> np.ndarray:
    """float32 (M, K) token rows before quantisation, the input of a linear
    that quantises its own activations: standard normal values with one
    column in 256 (the same columns for every token) twenty times larger,
    the outlier channels of a normalised hidden state."""
    rng = np.random.default_rng([seed, layer, idx, 2 << 20, M])
    x = rng.normal(0.0, 1.0, (M, K))
    x[:, rng.permutation(K)[: max(1, K // 256)]] *= 20.0
    return x.astype(np.float32)


def make_linear(seed, layer: int, idx: int, N: int, K: int, p_zero: float, M: int,
                name: str = "") -> Linear:
    w, s_row = make_weights(seed, layer, idx, N, K, p_zero)
    q, s_act, z = make_activations(seed, layer, idx, K, M)
    return Linear(name, w, s_row, q, s_act, z)


def make_block_scales(seed, layer: int, idx: int, N: int, K: int, B: int) -> np.ndarray:
    """float32 (N, ceil(K / B)) block scales of one linear."""
    rng = np.random.default_rng([seed, layer, idx, 1 << 20, B])
    return rng.uniform(0.01, 0.1, (N, -(-K // B))).astype(np.float32)


def single_gemv_case() -> Linear:
    """One 256 x 512 GEMV, seed 0: P(0) = 0.626, P(+1) = P(-1) = 0.187,
    s_row ~ U(0.01, 0.1), q uniform int8, s_act = 0.02, z = 3."""
    rng = np.random.default_rng(0)
    w = rng.choice(np.array([-1, 0, 1], np.int8), p=[0.187, 0.626, 0.187], size=(256, 512))
    s_row = rng.uniform(0.01, 0.1, 256).astype(np.float32)
    q = rng.integers(-128, 128, 512).astype(np.int8).reshape(1, 512)
    return Linear("gemv256x512", w.astype(np.int8), s_row, q,
                  np.array([0.02], np.float32), np.array([3], np.int32))


def stack_specs(model: str = "8b", layers: int | None = None):
    """[(layer, idx, name, N, K, p_zero)] for the 8B- or 0.6B-shaped stack."""
    if model == "8b":
        table, nl = LAYER_8B, LAYERS_8B
    elif model == "0.6b":
        table, nl = LAYER_06B, LAYERS_06B
    else:
        raise ValueError(model)
    nl = nl if layers is None else layers
    out = []
    for layer in range(nl):
        for idx, (name, N, K) in enumerate(table):
            p0 = zero_rate_8b(layer, name) if model == "8b" else P_ZERO_DEFAULT
            out.append((layer, idx, name, N, K, p0))
    return out


def make_stack(seed, M: int, model: str = "8b", layers: int | None = None,
               threads: int = 8, consume=None):
    """Draw every linear of a stack.  With ``consume`` (a callable taking
    (position, Linear)) each linear is handed over as soon as it is drawn and
    not kept, so the whole int8 stack never sits in host memory at once."""
    specs = stack_specs(model, layers)

    def one(spec):
        layer, idx, name, N, K, p0 = spec
        return make_linear(seed, layer, idx, N, K, p0, M, "L%d.%s" % (layer, name))

    out = [] if consume is None else None
    with _cf.ThreadPoolExecutor(max(1, threads)) as ex:
        # keep a bounded window of draws in flight
        window = max(1, threads) * 2
        futs = {}
        for pos, spec in enumerate(specs):
            futs[pos] = ex.submit(one, spec)
            if pos - window in futs:
                _take(futs, pos - window, out, consume)
        for pos in sorted(futs):
            _take(futs, pos, out, consume)
    return out


def _take(futs, pos, out, consume):
    lin = futs.pop(pos).result()
    if consume is None:
        out.append(lin)
    else:
        consume(pos, lin)


# The 8B's output head: vocabulary x hidden width (model card "Architecture":
# vocabulary 151,936, hidden 4,096), int8 with one scale per row ("Where the
# bytes live").  Trained values are not available: entries are uniform int8
# in [-127, 127] and row scales U(1e-3, 1e-2).
HEAD_8B = (151936, 4096)


def make_head(seed, N: int = HEAD_8B[0], K: int = HEAD_8B[1]):
    """(W int8 (N, K), s_row float32 (N,)) of a synthetic int8 output head."""
    rng = np.random.default_rng([seed, 151936])
    W = rng.integers(-127, 128, (N, K), dtype=np.int8)
    s_row = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    return W, s_row
