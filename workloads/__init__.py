"""Seeded synthetic inputs for the indexer -> top-k -> sparse-attention path.

This module draws random tensors and fixes shapes; it holds none of the method's
arithmetic (no scoring, no selection, no softmax). Both the CPU oracle's tests and
the HIP path's tests and benchmark take their inputs from here, so the two sides
see the same bytes.

Five workloads, named by what they are:

* ``tiny_fp32``      T=S=256 fp32, indexer 4x64, top-k 64, sparse MLA 8 heads x 576.
* ``nope_unaligned`` T=S=1024 bf16, indexer 16x128 with 30% of key rows forced
                     negative (many zero scores), top-k 65/127, sparse MLA 16 heads,
                     q/kv built 512 wide then zero-padded to 576, one all-invalid row.
* ``block_gqa``      T=S=8192 bf16, indexer 16x128 scoring 64-key blocks, top-16 blocks
                     including the query's own, sparse GQA 32 q heads / 4 kv heads x 128.
* ``long_dsa``       T=S=32768 bf16 one sequence, indexer 64x128, top-k 2048, sparse
                     MLA 128 heads, q [T,128,576], latent kv [T,576], d_v 512.
* ``thd_varlen``     16 packed sequences, total 65536, lengths log-uniform in
                     [512, 16384], indexer 64x128, top-k 2048, sparse MLA 64 heads.

Random draws use ``torch.Generator`` seeded per workload and per tensor (the
tensor's position in a fixed list is added to the seed), so a tensor does not
depend on which other tensors were drawn. Small workloads are drawn on the CPU
(identical on every machine); the two large ones are drawn on the device they
will run on. bf16 tensors are drawn in fp32 and rounded to bf16 (round to nearest
even) by ``Tensor.to``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str                      # "f32" or "bf16"
    lengths: tuple                  # sequence lengths; sum = T
    # indexer
    H_I: int
    D_I: int
    w_dist: str                     # "uniform01" | "normal" | "normal_over_8"
    topk: tuple                     # top-k values exercised (tokens, or blocks)
    block_size: int = 1             # 1 = token routing, B = block routing
    # sparse MLA
    H: int = 0
    d_qk: int = 576
    d_v: int = 512
    nope: bool = False              # q/kv drawn 512 wide, zero-padded to 576
    # sparse GQA
    Hq: int = 0
    Hkv: int = 0
    D: int = 0
    Dv: int = 0
    # extras
    grid: float = 0.0               # >0: indexer and MLA inputs rounded to this grid
    neg_key_frac: float = 0.0       # fraction of indexer key rows forced <= 0
    invalid_rows: tuple = ()        # rows whose index row is overwritten with -1
    gen_on_device: bool = False     # large: draw on the run device

    @property
    def T(self) -> int:
        return int(sum(self.lengths))

    @property
    def scale(self) -> float:
        if self.Hq:
            return 1.0 / math.sqrt(self.D)
        # NoPE: the unpadded width sets the scale; zero padding must not change it
        return 1.0 / math.sqrt(512 if self.nope else self.d_qk)


def thd_lengths(seed: int = 4, n: int = 16, total: int = 65536,
                lo: int = 512, hi: int = 16384) -> tuple:
    """Log-uniform sequence lengths in [lo, hi] summing to ``total``.

    u_i ~ U(ln lo, ln hi); L_i = round(e^{u_i} / sum e^u * total); clip to
    [lo, hi]; the rounding remainder goes to the longest sequence.
    """
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(lo), math.log(hi), n)
    e = np.exp(u)
    L = np.round(e / e.sum() * total).astype(np.int64)
    L = np.clip(L, lo, hi)
    L[int(np.argmax(L))] += total - int(L.sum())
    assert L.sum() == total and L.min() >= lo and L.max() <= hi, L
    return tuple(int(x) for x in L)


WORKLOADS = {
    "tiny_fp32": Workload(
        name="tiny_fp32", seed=0, dtype="f32", lengths=(256,),
        H_I=4, D_I=64, w_dist="uniform01", topk=(64,),
        H=8, d_qk=576, d_v=512, grid=0.25),
    "nope_unaligned": Workload(
        name="nope_unaligned", seed=1, dtype="bf16", lengths=(1024,),
        H_I=16, D_I=128, w_dist="uniform01", topk=(65, 127),
        H=16, d_qk=576, d_v=512, nope=True, neg_key_frac=0.3,
        invalid_rows=(511,)),
    "block_gqa": Workload(
        name="block_gqa", seed=2, dtype="bf16", lengths=(8192,),
        H_I=16, D_I=128, w_dist="normal", topk=(16,), block_size=64,
        Hq=32, Hkv=4, D=128, Dv=128),
    "long_dsa": Workload(
        name="long_dsa", seed=3, dtype="bf16", lengths=(32768,),
        H_I=64, D_I=128, w_dist="normal_over_8", topk=(2048,),
        H=128, d_qk=576, d_v=512, gen_on_device=True),
    "thd_varlen": Workload(
        name="thd_varlen", seed=4, dtype="bf16", lengths=thd_lengths(4),
        H_I=64, D_I=128, w_dist="normal_over_8", topk=(2048,),
        H=64, d_qk=576, d_v=512, gen_on_device=True),
}


def cu_seqlens(lengths) -> np.ndarray:
    """Prefix offsets [0, L0, L0+L1, ...] as int32."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


# ----------------------------------------------------------------------------- draws

def _gen(seed: int, slot: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(slot))
    return g


def _normal(shape, seed, slot, device, chunk_rows=4096):
    """N(0,1) fp32 of ``shape``, drawn row-chunk by row-chunk (bounded peak memory)."""
    g = _gen(seed, slot, device)
    out = torch.empty(shape, dtype=torch.float32, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=g,
                                  dtype=torch.float32, device=device)
    return out


def _uniform(shape, seed, slot, device):
    g = _gen(seed, slot, device)
    return torch.rand(shape, generator=g, dtype=torch.float32, device=device)


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x.contiguous()


def _on_grid(x: torch.Tensor, step: float, lim: float | None = None) -> torch.Tensor:
    y = torch.round(x / step) * step
    if lim is not None:
        y = y.clamp(-lim, lim)
    return y


def _device_for(wl: Workload, device):
    return device if wl.gen_on_device else "cpu"


def indexer_inputs(wl: Workload, device="cpu", integer: bool = False, T: int | None = None):
    """Indexer operands: q_I [T,H_I,D_I], k_I [T,D_I] (wl.dtype), w [T,H_I] fp32.

    ``integer=True`` draws the integer-valued variant used for bit-exact index
    comparisons: q_I and k_I on a 0.5 grid clamped to [-2, 2] (the tiny workload
    keeps its 0.25 grid, clamped to [-4, 4]), and w on a 2^-6 grid, so every
    partial sum of the score is exactly representable in fp32.
    """
    T = wl.T if T is None else T
    gd = _device_for(wl, device)
    q = _normal((T, wl.H_I, wl.D_I), wl.seed, 0, gd)
    k = _normal((T, wl.D_I), wl.seed, 1, gd)
    if wl.neg_key_frac > 0:
        q = q.abs()
        sel = _uniform((T,), wl.seed, 2, gd) < wl.neg_key_frac
        k = torch.where(sel[:, None], -k.abs(), k)
    if wl.w_dist == "uniform01":
        w = _uniform((T, wl.H_I), wl.seed, 3, gd)
    elif wl.w_dist == "normal":
        w = _normal((T, wl.H_I), wl.seed, 3, gd)
    else:
        w = _normal((T, wl.H_I), wl.seed, 3, gd) / 8.0
    if wl.grid > 0:
        q = _on_grid(q, wl.grid)
        k = _on_grid(k, wl.grid)
    if integer:
        if wl.grid > 0:
            q = _on_grid(q, wl.grid, 4.0)
            k = _on_grid(k, wl.grid, 4.0)
        else:
            q = _on_grid(q, 0.5, 2.0)
            k = _on_grid(k, 0.5, 2.0)
        w = _on_grid(w, 2.0 ** -6)
    out = dict(q_I=_cast(q, wl.dtype), k_I=_cast(k, wl.dtype), w=w.contiguous())
    return {n: t.to(device) for n, t in out.items()}


def exact_sum_bound(q_I: torch.Tensor, k_I: torch.Tensor, w: torch.Tensor) -> float:
    """Largest |partial sum| of a score over its grid unit (must stay below 2^24).

    Bound per row t: sum_h |w[t,h]| * sum_d |q[t,h,d]| * max_s |k[s,d]|, divided by
    the product of the three grids' finest units. Used by tests to check that the
    integer variant is exact in fp32 in any summation order.
    """
    qa = q_I.float().abs()
    kmax = k_I.float().abs().amax(dim=0)
    per = (qa * kmax).sum(-1)
    b = (w.abs() * per).sum(-1).max().item()

    def unit(x):
        # finest power of two 2^-p that divides every value of x
        x = x.float().flatten()
        for p in range(0, 40):
            if torch.all(torch.frac(x * (2.0 ** p)) == 0):
                return 2.0 ** -p
        raise ValueError("values are not on a power-of-two grid")

    return b / (unit(q_I) * unit(k_I) * unit(w))


def mla_inputs(wl: Workload, device="cpu", T: int | None = None):
    """Sparse-MLA operands: q [T,H,d_qk], kv [T,d_qk] (wl.dtype).

    For the NoPE workload, q and kv are drawn 512 wide; ``q512``/``kv512`` hold
    those and ``q``/``kv`` their zero-padded 576-wide copies.
    """
    T = wl.T if T is None else T
    gd = _device_for(wl, device)
    width = 512 if wl.nope else wl.d_qk
    q = _normal((T, wl.H, width), wl.seed, 10, gd)
    kv = _normal((T, width), wl.seed, 11, gd)
    if wl.grid > 0:
        q = _on_grid(q, wl.grid)
        kv = _on_grid(kv, wl.grid)
    q = _cast(q, wl.dtype)
    kv = _cast(kv, wl.dtype)
    out = {}
    if wl.nope:
        out["q512"], out["kv512"] = q, kv
        q = torch.nn.functional.pad(q, (0, 576 - 512))
        kv = torch.nn.functional.pad(kv, (0, 576 - 512))
    out["q"], out["kv"] = q.contiguous(), kv.contiguous()
    return {n: t.to(device) for n, t in out.items()}


def gqa_inputs(wl: Workload, device="cpu", T: int | None = None):
    """Sparse-GQA operands: q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,Dv] (wl.dtype)."""
    T = wl.T if T is None else T
    gd = _device_for(wl, device)
    q = _normal((T, wl.Hq, wl.D), wl.seed, 20, gd)
    k = _normal((T, wl.Hkv, wl.D), wl.seed, 21, gd)
    v = _normal((T, wl.Hkv, wl.Dv), wl.seed, 22, gd)
    out = dict(q=_cast(q, wl.dtype), k=_cast(k, wl.dtype), v=_cast(v, wl.dtype))
    return {n: t.to(device) for n, t in out.items()}


def random_index_rows(T, S, k, seed, lengths=None, device="cpu", frac_invalid=0.0):
    """Random causal token indices [T,k] int32 (global rows), -1 padded.

    Row t of sequence [c, c+L) draws min(k, t-c+1) distinct keys from [c, t] and
    places them in random slots; a seeded fraction of the remaining valid slots is
    also turned into -1. Used to feed attention kernels index rows that do not come
    from any selection code.
    """
    g = _gen(seed, 30, "cpu")
    lengths = lengths or (S,)
    starts = cu_seqlens(lengths)
    idx = torch.full((T, k), -1, dtype=torch.int32)
    for j in range(len(lengths)):
        c0, c1 = int(starts[j]), int(starts[j + 1])
        for t in range(c0, c1):
            n = t - c0 + 1
            m = min(k, n)
            pick = torch.randperm(n, generator=g)[:m] + c0
            slots = torch.randperm(k, generator=g)[:m]
            idx[t, slots] = pick.to(torch.int32)
    if frac_invalid > 0:
        drop = torch.rand((T, k), generator=g) < frac_invalid
        idx[drop] = -1
    return idx.to(device)


def random_causal_index(T, k, seed, lengths=None, device="cpu", frac_invalid=0.05):
    """Random causal token indices [T,k] int32, vectorised (duplicates allowed).

    Slot j of row t (sequence [c, c+L)) holds c + floor(u * (t - c + 1)), u ~ U(0,1),
    i.e. a uniformly drawn causal key; a seeded fraction of slots is -1. Used to feed
    attention kernels index rows at full size without any selection code.
    """
    lengths = lengths or (T,)
    starts = torch.from_numpy(cu_seqlens(lengths)[:-1].astype(np.int64))
    lens = torch.tensor(lengths, dtype=torch.int64)
    seq_of = torch.repeat_interleave(torch.arange(len(lengths)), lens)
    start = starts[seq_of].to(device)
    t = torch.arange(T, device=device, dtype=torch.int64)
    g = _gen(seed, 31, device)
    u = torch.rand((T, k), generator=g, device=device, dtype=torch.float64)
    idx = start[:, None] + torch.floor(u * (t - start + 1)[:, None].double()).long()
    drop = torch.rand((T, k), generator=g, device=device) < frac_invalid
    idx = torch.where(drop, torch.full_like(idx, -1), idx)
    return idx.to(torch.int32).contiguous()


def random_block_index(T, nblk, block_size, seed, lengths=None, device="cpu"):
    """Random block routes [T,nblk] int32: the query's own block plus distinct earlier
    blocks drawn at random, -1 padded when the row has fewer blocks. Local block ids."""
    lengths = lengths or (T,)
    g = _gen(seed, 32, "cpu")
    out = torch.full((T, nblk), -1, dtype=torch.int32)
    starts = cu_seqlens(lengths)
    for j in range(len(lengths)):
        c0, c1 = int(starts[j]), int(starts[j + 1])
        for t in range(c0, c1):
            own = (t - c0) // block_size
            others = torch.randperm(own, generator=g)[:nblk - 1] if own > 0 else torch.empty(0, dtype=torch.long)
            row = torch.cat([others, torch.tensor([own])]).sort().values
            out[t, :row.numel()] = row.to(torch.int32)
    return out.to(device)
