"""A whole stack of ternary linears resident in device memory.

Plumbing around the C ABI: draws the seeded synthetic weights on the host
(``synth``), packs each linear on the device with ``tern_pack`` (the int8
matrix is dropped right after), then binds activation / output buffers for a
token count M and prepares the persistent ``tern_linear_stack`` launch.
torch only allocates memory; every step of the computation is a HIP kernel.
"""
from __future__ import annotations

import concurrent.futures as cf
from dataclasses import dataclass, field

import numpy as np
import torch

from . import synth, tern


@dataclass
class PackedLinear:
    layer: int
    idx: int
    name: str
    N: int
    K: int
    packed: torch.Tensor
    rowsum: torch.Tensor
    s_row: torch.Tensor
    # block-wise scales (block > 0): N x ceil(K / block) scales and row sums
    block: int = 0
    s_block: torch.Tensor | None = None
    rowsum_block: torch.Tensor | None = None
    # host copies of a few rows, for sampled checks (row index -> weights)
    sample_rows: np.ndarray | None = None
    sample_w: np.ndarray | None = None
    sample_s_row: np.ndarray | None = None


def _pad16(n: int) -> int:
    return (n + 15) // 16 * 16


class DeviceStack:
    """Packed weights and metadata of every linear of a synthetic stack."""

    def __init__(self, model: str = "8b", layers: int | None = None, seed: int = 0,
                 threads: int = 8, device: str = "cuda:0", sample_rows: int = 0, block: int = 0):
        """block > 0: every linear also gets block-wise scales along K (one per
        `block` columns, ``synth.make_block_scales``) and their block row
        sums (``tern_block_rowsum`` on the packed weights)."""
        self.model, self.seed, self.device, self.block = model, seed, device, block
        self.specs = synth.stack_specs(model, layers)
        self.linears: list[PackedLinear] = []
        bad_total = torch.zeros(1, dtype=torch.int32, device=device)
        bad = torch.empty(1, dtype=torch.int32, device=device)
        rng = np.random.default_rng([seed, 99991])

        def draw(spec):
            layer, idx, name, N, K, p0 = spec
            return spec, synth.make_weights(seed, layer, idx, N, K, p0)

        with cf.ThreadPoolExecutor(max(1, threads)) as ex:
            futs = [ex.submit(draw, sp) for sp in self.specs[: 2 * threads]]
            nxt = len(futs)
            for i in range(len(self.specs)):
                (layer, idx, name, N, K, _), (w, s_row) = futs[i].result()
                futs[i] = None
                if nxt < len(self.specs):
                    futs.append(ex.submit(draw, self.specs[nxt]))
                    nxt += 1
                wd = torch.from_numpy(w).to(device)
                packed = torch.empty((N, tern.tern_row_bytes(K)), dtype=torch.uint8, device=device)
                rowsum = torch.empty(N, dtype=torch.int32, device=device)
                tern.tern_pack(wd, N, K, K, packed, rowsum, bad)
                bad_total += bad
                del wd
                pl = PackedLinear(layer, idx, "L%d.%s" % (layer, name), N, K, packed, rowsum,
                                  torch.from_numpy(s_row).to(device))
                if block:
                    nb = -(-K // block)
                    pl.block = block
                    pl.s_block = torch.from_numpy(synth.make_block_scales(seed, layer, idx, N, K, block)).to(device)
                    pl.rowsum_block = torch.empty((N, nb), dtype=torch.int32, device=device)
                    tern.tern_block_rowsum(packed, N, K, block, pl.rowsum_block)
                if sample_rows:
                    rows = np.unique(np.concatenate([
                        [0, N - 1], rng.choice(N, min(N, sample_rows), replace=False)]))
                    pl.sample_rows, pl.sample_w, pl.sample_s_row = rows, w[rows].copy(), s_row[rows].copy()
                self.linears.append(pl)
        torch.cuda.synchronize()
        if int(bad_total.item()) != 0:
            raise RuntimeError("synthetic weights held values outside {-1, 0, +1}")

    @property
    def weights(self) -> int:
        return sum(pl.N * pl.K for pl in self.linears)

    def bind(self, M: int, path: int = tern.TERN_PATH_AUTO, with_acc: bool = False,
             act_seed: int | None = None, share_inputs: bool = False,
             quantise: str = "none") -> "StackBinding":
        """Buffers and a prepared launch for M tokens.  With ``share_inputs``
        the linears of a layer that read one input (``synth.INPUT_LEADER``:
        q/k/v, gate/up) are given one activation buffer, drawn for the
        group's first linear; otherwise every linear has its own.
        ``quantise``: "none" (int8 activations drawn directly), "first" (the
        first input is fp32, ``synth.make_hidden``, quantised by the launch
        itself) or "all" (every input is)."""
        assert quantise in ("none", "first", "all")
        return StackBinding(self, M, path, with_acc, self.seed if act_seed is None else act_seed,
                            share_inputs, quantise)


@dataclass
class StackBinding:
    """Activations, outputs and a prepared launch for M tokens."""
    stack: DeviceStack
    M: int
    path: int
    with_acc: bool
    act_seed: int
    share_inputs: bool = False
    quantise: str = "none"
    q: list = field(default_factory=list)
    s_act: list = field(default_factory=list)
    z: list = field(default_factory=list)
    y: list = field(default_factory=list)
    acc: list = field(default_factory=list)
    host_act: list = field(default_factory=list)
    x: list = field(default_factory=list)       # fp32 inputs (device) or None
    host_x: list = field(default_factory=list)  # their host copies or None

    def __post_init__(self):
        dev, M = self.stack.device, self.M
        descs = []
        shared = {}  # (layer, leader idx) -> (q, s_act, z) host arrays and device tensors
        for pl in self.stack.linears:
            src = synth.INPUT_LEADER[pl.idx] if self.share_inputs else pl.idx
            key = (pl.layer, src)
            if key not in shared:
                ldq = _pad16(pl.K)
                if self.quantise == "all" or (self.quantise == "first" and not shared):
                    # an fp32 input: q, s_act and z are written by the launch
                    x = synth.make_hidden(self.act_seed, pl.layer, src, pl.K, M)
                    shared[key] = (None, torch.zeros((M, ldq), dtype=torch.int8, device=dev),
                                   torch.zeros(M, dtype=torch.float32, device=dev),
                                   torch.zeros(M, dtype=torch.int32, device=dev), x, torch.from_numpy(x).to(dev))
                else:
                    q, s_act, z = synth.make_activations(self.act_seed, pl.layer, src, pl.K, M)
                    qp = np.zeros((M, ldq), np.int8)
                    qp[:, : pl.K] = q
                    shared[key] = ((q, s_act, z), torch.from_numpy(qp).to(dev), torch.from_numpy(s_act).to(dev),
                                   torch.from_numpy(z).to(dev), None, None)
            host, qd, sd, zd, hx, xd = shared[key]
            ldq = qd.shape[1]
            self.x.append(xd)
            self.host_x.append(hx)
            # (an fp32 input has no host int8 activations: its q, s_act and z
            # exist only once the launch has run)
            q, s_act, z = host if host is not None else (None, None, None)
            yd = torch.empty((M, pl.N), dtype=torch.float32, device=dev)
            ad = torch.empty((M, pl.N), dtype=torch.int32, device=dev) if self.with_acc else None
            self.q.append(qd)
            self.s_act.append(sd)
            self.z.append(zd)
            self.y.append(yd)
            self.acc.append(ad)
            if pl.sample_rows is not None:
                self.host_act.append((q, s_act, z))
            descs.append(tern.make_desc(pl.packed, pl.s_row, pl.rowsum, pl.N, pl.K, qd, ldq, sd,
                                        zd, yd, pl.N, ad, pl.block, pl.s_block, pl.rowsum_block,
                                        x=xd, ldx=pl.K))
        self.descs = descs
        L = len(descs)
        self.workspace = torch.empty(tern.tern_linear_stack_workspace_bytes(L, M),
                                     dtype=torch.uint8, device=dev)
        self.plan = tern.tern_linear_stack_prepare(descs, M, self.workspace, self.path)

    @property
    def bytes(self) -> int:
        """Algorithmic bytes of one pass: packed weights, 8 B of row metadata
        per row, int8 activations, 8 B per token and fp32 outputs."""
        return int(self.plan.bytes)

    def run(self, stream=None):
        tern.tern_linear_stack(self.plan, stream)
