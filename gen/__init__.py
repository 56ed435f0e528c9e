"""Seeded synthetic inputs for the MoE expert combine.

This module only *builds inputs*: routing (top-k expert choice), router
weights, slot drops, the dispatch-order slot map, and the bf16 tensors
(expert-output payload, shared-expert output, residual, RMSNorm gamma). It
holds none of the combine's arithmetic: no weighted sum, no output rounding,
no normalisation, no quantisation. Both the CPU oracle and the HIP path
consume what it returns, and neither imports the other.

Layouts follow the pages:
  * payload  [ep_size, max_tokens_per_rank, hidden] bf16, per-expert-rank rows
    in dispatch order (flashinfer ``moe_a2a_combine``, Parameters: payload;
    ``runtime_max_tokens_per_rank``);
  * src_info [num_tokens, top_k, 2] int32 = (rank, row) per (token, slot);
    (-1, -1) marks a dropped slot (MAX ``ep.combine`` Args: src_info records
    the source of each row; flashinfer ``nvfp4_mega_moe`` Parameters:
    num_tokens, rows routed to -1 contribute nothing). The map is the inverse
    (gather) form of the dispatch scatter;
  * router_weights [num_tokens, top_k] fp32 (MAX ``ep.combine`` Args:
    router_weights).

Random streams. Small draws (routing keys, router logits, slot drops, hot
rows) come from one PCG64 generator seeded with ``seed``, in that order.
Large normal tensors are split into fixed blocks of ``_BLOCK`` elements; block
``b`` of stream ``s`` is drawn from ``SeedSequence(seed, spawn_key=(s, b))``,
so values do not depend on the number of threads. Normals are drawn in fp32,
scaled as ``mean + sd * z`` in fp32 and rounded to bf16 (round to nearest
even) by torch's CPU cast.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import torch

__all__ = ["CONFIGS", "Inputs", "make_inputs", "dispatch_slots",
           "scatter_rows", "normal_bf16", "algorithmic_bytes", "DenseInputs",
           "make_dense_inputs", "DENSE_CONFIGS"]

_BLOCK = 1 << 22  # elements per independently seeded block of a normal tensor

# Stream ids of the large normal tensors (the spawn_key's first element).
_S_PAYLOAD, _S_SHARED, _S_RESIDUAL, _S_GAMMA, _S_DENSE = 1, 2, 3, 4, 5

# The five synthetic workloads (sizes of the combine; see the DESIGN notes on
# the input recipe for every choice the workload text leaves open).
CONFIGS = {
    # T=64, H=1024, 8 experts on one rank, top-2 uniform: payload [1,128,1024].
    "tiny": dict(T=64, H=1024, E=8, ep=1, k=2, routing="uniform",
                 capacity="fit"),
    # DeepSeek-V3 shape: 256 experts over 8 simulated ranks, top-8 uniform.
    "dsv3": dict(T=4096, H=7168, E=256, ep=8, k=8, routing="uniform",
                 capacity="fit"),
    # Zipf(1.2) routing, 10% dropped slots, capped per-rank capacity,
    # fused shared-expert output N(0, 0.5).
    "skewed": dict(T=8192, H=4096, E=128, ep=8, k=8, routing="zipf",
                   zipf_s=1.2, drop_frac=0.1, capacity="cap", shared_sd=0.5),
    # Residual N(0,1), gamma N(1, 0.1), eps 1e-6 (run with weight_bias 0 and 1).
    "rmsnorm": dict(T=2048, H=7168, E=256, ep=8, k=8, routing="uniform",
                    capacity="fit", residual_sd=1.0, gamma_mean=1.0,
                    gamma_sd=0.1, eps=1e-6),
    # MXFP8 output; 1% of occupied payload rows scaled by 64.
    "mxfp8": dict(T=16384, H=7168, E=256, ep=8, k=8, routing="uniform",
                  capacity="fit", hot_row_frac=0.01, hot_scale=64.0),
}


@dataclasses.dataclass
class Inputs:
    """Host-side inputs of one combine call (numpy arrays, C-contiguous).

    bf16 tensors are carried as their raw ``uint16`` bit patterns.
    """
    payload: np.ndarray          # uint16 [ep, mtpr, H]
    src_info: np.ndarray         # int32  [T, k, 2]
    weights: np.ndarray          # float32 [T, k]
    topk_ids: np.ndarray         # int32  [T, k] (expert chosen by the router)
    shared: np.ndarray | None    # uint16 [T, H]
    residual: np.ndarray | None  # uint16 [T, H]
    gamma: np.ndarray | None     # uint16 [H]
    eps: float
    meta: dict

    @property
    def T(self):
        return self.src_info.shape[0]

    @property
    def k(self):
        return self.src_info.shape[1]

    @property
    def H(self):
        return self.payload.shape[2]

    @property
    def ep(self):
        return self.payload.shape[0]

    @property
    def mtpr(self):
        return self.payload.shape[1]


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 draws -> uint16 bf16 bit patterns, rounded by torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(shape, seed: int, stream: int, mean: float = 0.0,
                sd: float = 1.0) -> np.ndarray:
    """bf16 bits of N(mean, sd) draws, block-seeded (thread-count independent)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    nblk = (n + _BLOCK - 1) // _BLOCK

    def fill(b):
        lo = b * _BLOCK
        hi = min(n, lo + _BLOCK)
        ss = np.random.SeedSequence(seed, spawn_key=(stream, b))
        z = np.random.default_rng(ss).standard_normal(hi - lo, dtype=np.float32)
        if sd != 1.0:
            z *= np.float32(sd)
        if mean != 0.0:
            z += np.float32(mean)
        out[lo:hi] = _to_bf16_bits(z)

    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# Routing and dispatch
# ----------------------------------------------------------------------------

def _route_uniform(rng, T, E, k):
    """k distinct experts per token, uniform without replacement, random order."""
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def _route_zipf(rng, T, E, k, s):
    """k distinct experts per token drawn from p(e) ~ (e+1)^-s without
    replacement (Gumbel top-k on log p, which equals sequential sampling
    without replacement); experts keep identity order, so low ids are hot."""
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    g = rng.gumbel(size=(T, E))
    return np.argsort(-(logp[None, :] + g), axis=1, kind="stable")[:, :k].astype(np.int32)


def _softmax_weights(rng, T, k):
    """Router logits N(0,1) in fp32, softmaxed over the chosen k in float64,
    stored as fp32 (the router is upstream of the combine)."""
    logits = rng.standard_normal((T, k), dtype=np.float32).astype(np.float64)
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def dispatch_slots(topk_ids: np.ndarray, dropped: np.ndarray, E: int, ep: int,
                   capacity: int | None):
    """Dispatch-order slot map (the scatter the combine inverts).

    Kept (token, slot) pairs are enumerated token-major, slot-minor and
    stably sorted by expert id; expert ``e`` lives on rank ``e // (E/ep)``;
    a pair's row is its position among its rank's pairs in that order, so a
    rank's rows are ordered by (expert, token, slot). With ``capacity`` set,
    rows at or past it are dropped too. Returns (src_info [T,k,2] int32,
    loads per rank before the capacity cut).
    """
    T, k = topk_ids.shape
    if E % ep:
        raise ValueError("E must be a multiple of ep")
    epr = E // ep
    flat_e = topk_ids.reshape(-1).astype(np.int64)
    keep = ~dropped.reshape(-1)
    idx = np.nonzero(keep)[0]                     # token-major order
    order = idx[np.argsort(flat_e[idx], kind="stable")]
    rank_sorted = flat_e[order] // epr
    loads = np.bincount(rank_sorted, minlength=ep)
    starts = np.concatenate([[0], np.cumsum(loads)[:-1]])
    row_sorted = np.arange(order.size) - starts[rank_sorted]
    src = np.full((T * k, 2), -1, dtype=np.int32)
    ok = np.ones(order.size, dtype=bool) if capacity is None else row_sorted < capacity
    src[order[ok], 0] = rank_sorted[ok]
    src[order[ok], 1] = row_sorted[ok]
    return src.reshape(T, k, 2), loads


def scatter_rows(src_info: np.ndarray, rows: np.ndarray, ep: int, mtpr: int,
                 fill: np.ndarray | None = None) -> np.ndarray:
    """Place per-(token, slot) rows into a payload (dispatch of given rows).

    ``rows`` is [T, k, H] (bf16 bits); valid slots are written to
    ``payload[rank, row]``; unoccupied rows keep ``fill`` (default zero bits).
    """
    T, k, H = rows.shape
    payload = (np.zeros((ep, mtpr, H), dtype=rows.dtype) if fill is None
               else np.array(fill, dtype=rows.dtype, copy=True))
    r = src_info[..., 0].reshape(-1)
    w = src_info[..., 1].reshape(-1)
    v = r >= 0
    payload[r[v], w[v]] = rows.reshape(T * k, H)[v]
    return payload


def _round_up(x, m):
    return (x + m - 1) // m * m


def make_inputs(cfg: str | dict, seed: int = 0, **override) -> Inputs:
    """Build one synthetic combine workload.

    ``cfg`` is a name in ``CONFIGS`` or a dict with the same keys; keyword
    overrides replace single keys. Extra keys used by tests:
      weights (bool, default True): False -> router_weights omitted (None);
      unoccupied ("normal" | "nan"): fill of payload rows no slot points at;
      mtpr (int): force max_tokens_per_rank (must hold every kept row);
      row_shuffle (bool): permute each rank's rows (a different dispatch order
        holding the same (token, slot) values).
    """
    c = dict(CONFIGS[cfg]) if isinstance(cfg, str) else dict(cfg)
    c.update(override)
    T, H, E, ep, k = c["T"], c["H"], c["E"], c["ep"], c["k"]
    if k > E:
        raise ValueError("top_k exceeds expert count")
    rng = np.random.default_rng(np.random.SeedSequence(seed))

    # 1. routing
    if c.get("routing", "uniform") == "zipf":
        topk = _route_zipf(rng, T, E, k, c.get("zipf_s", 1.2))
    else:
        topk = _route_uniform(rng, T, E, k)
    # 2. router weights
    weights = _softmax_weights(rng, T, k)
    # 3. slot drops: exactly floor(frac * T * k) slots, uniform w/o replacement
    dropped = np.zeros(T * k, dtype=bool)
    nd = int(math.floor(c.get("drop_frac", 0.0) * T * k))
    if nd:
        dropped[rng.choice(T * k, size=nd, replace=False)] = True
    dropped = dropped.reshape(T, k)

    # 4. dispatch order and capacity
    base_cap = _round_up(-(-T * k // ep), 128) if T else 128
    policy = c.get("capacity", "fit")
    if policy == "cap":
        src, loads = dispatch_slots(topk, dropped, E, ep, base_cap)
        mtpr = base_cap
    else:
        src, loads = dispatch_slots(topk, dropped, E, ep, None)
        mtpr = max(base_cap, _round_up(int(loads.max()) if loads.size else 0, 128))
    if c.get("mtpr") is not None:
        used = src[..., 1][src[..., 0] >= 0]
        if used.size and int(used.max()) >= int(c["mtpr"]):
            raise ValueError("forced mtpr too small for the kept rows")
        mtpr = int(c["mtpr"])
    if c.get("row_shuffle"):
        # new row numbers inside each rank, same (token, slot) -> data relation
        perm = np.stack([rng.permutation(mtpr) for _ in range(ep)])
        v = src[..., 0] >= 0
        src = src.copy()
        src[..., 1][v] = perm[src[..., 0][v], src[..., 1][v]]

    # 5. payload (all rows, then optional NaN fill of unoccupied rows)
    payload = normal_bf16((ep, mtpr, H), seed, _S_PAYLOAD)
    occ = np.zeros((ep, mtpr), dtype=bool)
    vv = src[..., 0] >= 0
    occ[src[..., 0][vv], src[..., 1][vv]] = True
    if c.get("unoccupied", "normal") == "nan":
        payload[~occ] = np.uint16(0x7FC0)
    # 6. hot rows (x64, exact in bf16): round(frac * T * k) occupied rows
    nh = int(round(c.get("hot_row_frac", 0.0) * T * k))
    hot = None
    if nh:
        occ_idx = np.flatnonzero(occ.reshape(-1))
        hot = np.sort(rng.choice(occ_idx, size=min(nh, occ_idx.size), replace=False))
        flat = payload.reshape(ep * mtpr, H)
        rows = torch.from_numpy(flat[hot].view(np.int16)).view(torch.bfloat16)
        rows = rows * float(c.get("hot_scale", 64.0))
        flat[hot] = rows.view(torch.int16).numpy().view(np.uint16)
    # 7-9. shared expert output, residual, gamma
    shared = (normal_bf16((T, H), seed, _S_SHARED, 0.0, c["shared_sd"])
              if c.get("shared_sd") is not None else None)
    residual = (normal_bf16((T, H), seed, _S_RESIDUAL, 0.0, c["residual_sd"])
                if c.get("residual_sd") is not None else None)
    gamma = (normal_bf16((H,), seed, _S_GAMMA, c.get("gamma_mean", 1.0),
                         c.get("gamma_sd", 0.1))
             if c.get("gamma_sd") is not None else None)

    kept = int((src[..., 0] >= 0).sum())
    meta = dict(T=T, H=H, E=E, ep=ep, k=k, mtpr=int(mtpr), seed=seed,
                loads=[int(x) for x in loads], kept_slots=kept,
                dropped_slots=int(T * k - kept), hot_rows=0 if hot is None else int(hot.size),
                capacity_policy=policy)
    return Inputs(payload=payload, src_info=np.ascontiguousarray(src),
                  weights=weights if c.get("weights", True) else None,
                  topk_ids=topk, shared=shared, residual=residual, gamma=gamma,
                  eps=float(c.get("eps", 1e-6)), meta=meta)


def algorithmic_bytes(inp: Inputs, kind: str = "bf16") -> int:
    """Bytes the combine must move (no padding, no dropped rows): gathered
    valid rows, 12 B of slot map + weight per (token, slot), optional shared,
    residual and gamma reads, and the outputs of ``kind``
    ("bf16" | "rmsnorm" | "mxfp8" | "rmsnorm_mxfp8" | "mxfp4")."""
    T, H, k = inp.T, inp.H, inp.k
    b = inp.meta["kept_slots"] * 2 * H + T * k * (8 + (4 if inp.weights is not None else 0))
    if inp.shared is not None:
        b += T * H * 2
    if kind == "bf16":
        b += T * H * 2
    elif kind == "rmsnorm":
        b += T * H * 2 + H * 2 + 2 * T * H * 2
    elif kind == "mxfp8":
        b += T * H + T * (H // 32)
    elif kind == "mxfp4":
        b += T * H // 2 + T * (H // 32)
    elif kind == "rmsnorm_mxfp8":
        # residual in, gamma, residual_out, e4m3 codes and scales of the norm
        b += T * H * 2 + H * 2 + T * H * 2 + T * H + T * (H // 32)
    else:
        raise ValueError(kind)
    return int(b)



# Dense (expert-major) inputs of the local reduce: n_in buffers [T, H].
DENSE_CONFIGS = {
    # 8 partial sums of [4096, 7168] (one per simulated rank), unit scales
    "dense8": dict(n_in=8, T=4096, H=7168, scales=False),
}


@dataclasses.dataclass
class DenseInputs:
    x: np.ndarray                  # uint16 [n_in, T, H]
    scales: np.ndarray | None      # float32 [T, n_in]
    tok: np.ndarray | None         # uint16 [T, H]
    residual: np.ndarray | None    # uint16 [T, H]
    gamma: np.ndarray | None       # uint16 [H]
    eps: float

    @property
    def n_in(self):
        return self.x.shape[0]

    @property
    def T(self):
        return self.x.shape[1]

    @property
    def H(self):
        return self.x.shape[2]


def make_dense_inputs(cfg, seed: int = 0, **override) -> DenseInputs:
    """Expert-major inputs x [n_in, T, H] bf16 N(0,1); scales [T, n_in] as a
    softmax of N(0,1) logits (if ``scales``); optional token input N(0, sd),
    residual N(0, sd) and gamma N(1, sd)."""
    c = dict(DENSE_CONFIGS[cfg]) if isinstance(cfg, str) else dict(cfg)
    c.update(override)
    n_in, T, H = c["n_in"], c["T"], c["H"]
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    scales = _softmax_weights(rng, T, n_in) if c.get("scales", True) else None
    x = normal_bf16((n_in, T, H), seed, _S_DENSE)
    tok = (normal_bf16((T, H), seed, _S_SHARED, 0.0, c["token_sd"])
           if c.get("token_sd") is not None else None)
    res = (normal_bf16((T, H), seed, _S_RESIDUAL, 0.0, c["residual_sd"])
           if c.get("residual_sd") is not None else None)
    gam = (normal_bf16((H,), seed, _S_GAMMA, 1.0, c.get("gamma_sd", 0.1))
           if c.get("residual_sd") is not None else None)
    return DenseInputs(x=x, scales=scales, tok=tok, residual=res, gamma=gam,
                       eps=float(c.get("eps", 1e-6)))


def dense_algorithmic_bytes(d: DenseInputs, rmsnorm: bool = False) -> int:
    """n_in rows per token + scales + token input (+ residual, gamma) + outputs."""
    T, H, n = d.T, d.H, d.n_in
    b = n * T * H * 2 + (T * n * 4 if d.scales is not None else 0)
    if d.tok is not None:
        b += T * H * 2
    b += T * H * 2
    if rmsnorm:
        b += T * H * 2 + H * 2 + T * H * 2
    return int(b)


__all__.append("dense_algorithmic_bytes")
