"""CPU baseline: the fp64 oracle, as it stands, timed on a bounded sample of a workload.

TEST INFRASTRUCTURE (used only by the benchmark's cpu_baseline leg). Work is spread over a pool of
worker processes (one per core, BLAS pinned to one thread each); the sample is stated in the
returned record and scaled to the whole step:
  * prefill: the pooling of every block (all blocks are pooled once per step), plus index, top-k
    and attention (or dense HCA attention) for a random sample of the step's queries, scaled by
    the number of queries;
  * decode: every query of the step (index over all entries, top-k, attention; the HCA layer too
    for the hybrid workload).
Storage decoding of the rows a query touches is part of the timed work.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import time

import numpy as np

from . import csa_oracle as orc
from .numerics import bf16_decode, e4m3_decode

_G: dict = {}


def _dec(a, dtype):
    if dtype == "bf16":
        return bf16_decode(a.view(np.uint16))
    if dtype == "e4m3":
        return e4m3_decode(a.view(np.uint8))
    return np.asarray(a, np.float64)


def _init_worker():
    # numpy's BLAS is already loaded in the forked worker: limit its pool through threadpoolctl.
    from threadpoolctl import threadpool_limits
    _G["limits"] = threadpool_limits(1)


def _compress_chunk(args):
    b, j0, j1 = args
    wl, h = _G["wl"], _G["host"]
    m = wl.m
    x = _dec(h["x"][b, j0 * m:j1 * m], wl.kv_dtype)
    g = _dec(h["g"][b, j0 * m:j1 * m], wl.kv_dtype)
    e = orc.store_bf16(orc.compress(x, g, h["bias"], m)) if wl.kv_dtype == "bf16" else \
        orc.compress(x, g, h["bias"], m)
    return b, j0, e


def _indexer_row(wl, h, qi, b):
    if wl.idx_dtype == "e4m3":
        q = _dec(h["q_i"][qi], "e4m3") * h["q_i_scale"][qi][:, None].astype(np.float64)
        k = _dec(h["k_i"][b], "e4m3") * h["k_i_scale"][b][:, None].astype(np.float64)
    else:
        q, k = _dec(h["q_i"][qi], wl.idx_dtype), _dec(h["k_i"][b], wl.idx_dtype)
    return q, k, h["w_i"][qi].astype(np.float64)


def _query(qi):
    wl, h = _G["wl"], _G["host"]
    b, pos = int(_G["seq"][qi]), int(_G["pos"][qi])
    if wl.kind == "hca_prefill":
        e = _G["entries"][b]
        q = _dec(h["q"][qi], wl.q_dtype)
        orc.hca_attend_one(q, (e[:, :wl.d_c], e[:, wl.d_c:], None, 0), pos, wl.m, wl.sm_scale)
        return qi
    nv = orc.n_visible(pos, wl.m, wl.n_entries)
    qi_, ki_, wi_ = _indexer_row(wl, h, qi, b)
    s = orc.index_scores(qi_, wi_, ki_, nv)
    idx, _ = orc.topk(s, nv, wl.k)
    sel = idx[idx >= 0]
    q = _dec(h["q"][qi], wl.q_dtype)
    if wl.kind == "csa_prefill":
        e = _G["entries"][b]
        ent = (e[:, :wl.d_c], e[:, wl.d_c:], None, 0)
        x = _dec(h["x"][b, max(0, pos - wl.window + 1):pos + 1], wl.kv_dtype)
        raw = (x[:, :wl.d_c], x[:, wl.d_c:], None, max(0, pos - wl.window + 1))
        orc.csa_attend_one(q, ent, idx, raw, pos, wl.window, wl.sm_scale)
    else:
        # Decode only the selected rows (compact store, remapped indices).
        ent = (_dec(h["ent_c"][b][sel], "e4m3"), _dec(h["ent_r"][b][sel], "bf16"),
               h["ent_scale"][b][sel].astype(np.float64), 0)
        raw = (_dec(h["raw_c"][b], "e4m3"), _dec(h["raw_r"][b], "bf16"),
               h["raw_scale"][b].astype(np.float64), wl.T - wl.window)
        orc.csa_attend_one(q, ent, np.arange(sel.size), raw, pos, wl.window, wl.sm_scale)
        if wl.kind == "hybrid_decode":
            hca = (_dec(h["hca_c"][b], "e4m3"), _dec(h["hca_r"][b], "bf16"),
                   h["hca_scale"][b].astype(np.float64), 0)
            orc.hca_attend_one(_dec(h["q_hca"][qi], wl.q_dtype), hca, pos, wl.m_hca,
                               wl.sm_scale)
    return qi


def _noop(i):
    return i


def _c1_step():
    wl, h = _G["wl"], _G["host"]
    x, g = orc.project(h["hidden"][0], h["w_x"], h["w_g"])
    e = orc.compress(x, g, h["bias"], wl.m)
    pos = int(_G["pos"][0])
    nv = orc.n_visible(pos, wl.m, wl.n_entries)
    s = orc.index_scores(h["q_i"][0], h["w_i"][0], h["k_i"][0], nv)
    idx, _ = orc.topk(s, nv, wl.k)
    orc.csa_attend_one(h["q"][0], (e, None, None, 0), idx, (x, None, None, 0), pos, wl.window,
                       wl.sm_scale)


def run(wl, host: dict, cores: int, budget_s: float, seed: int = 0) -> dict:
    """Time the oracle on a bounded sample of one step of `wl`; return the baseline record."""
    seq = np.repeat(np.arange(wl.B, dtype=np.int64), wl.nq)
    pos = np.tile(np.arange(wl.T - wl.nq, wl.T, dtype=np.int64), wl.B)
    _G.update(wl=wl, host=host, seq=seq, pos=pos, entries={})
    nq = seq.size
    rng = np.random.default_rng(seed)
    if wl.d_model:                                   # fp32 workload: the whole step, one core
        t = time.perf_counter()
        _c1_step()
        dt = time.perf_counter() - t
        return {"value": nq / dt, "unit": "queries/s", "cores": 1, "kind": "oracle",
                "sample": "the whole step (projection, pooling, index, top-k, attention)"}
    ctx = mp.get_context("fork")
    with cf.ProcessPoolExecutor(cores, mp_context=ctx, initializer=_init_worker) as ex:
        list(ex.map(_noop, range(4 * cores)))          # start the workers outside the timing
        t_comp = 0.0
        if wl.kind in ("csa_prefill", "hca_prefill"):
            nb = wl.n_entries
            chunk = max(1, nb // (4 * cores))
            jobs = [(b, j, min(nb, j + chunk)) for b in range(wl.B) for j in range(0, nb, chunk)]
            t = time.perf_counter()
            parts = list(ex.map(_compress_chunk, jobs))
            t_comp = time.perf_counter() - t
            for b in range(wl.B):
                _G["entries"][b] = np.concatenate([e for bb, j, e in sorted(parts, key=lambda z: z[1])
                                                   if bb == b], axis=0)
    # Re-fork so the workers see the pooled entries.
    with cf.ProcessPoolExecutor(cores, mp_context=ctx, initializer=_init_worker) as ex:
        list(ex.map(_noop, range(4 * cores)))
        decode = wl.kind in ("csa_decode", "hybrid_decode")
        if decode:
            sample = np.arange(nq)
        else:
            # Probe the per-query cost (after one untimed round), then size the sample to the
            # time budget.
            list(ex.map(_query, rng.choice(nq, size=min(nq, cores), replace=False)))
            probe = rng.choice(nq, size=min(nq, 4 * cores), replace=False)
            t = time.perf_counter()
            list(ex.map(_query, probe))
            t_probe = (time.perf_counter() - t) / len(probe) * cores
            n = int(max(cores, min(nq, 0.8 * budget_s * cores / max(t_probe, 1e-6))))
            sample = rng.choice(nq, size=n, replace=False)
        t = time.perf_counter()
        list(ex.map(_query, sample, chunksize=max(1, len(sample) // (8 * cores))))
        t_q = time.perf_counter() - t
    t_step = t_comp + t_q * nq / len(sample)
    what = (f"{len(sample)} of {nq} queries" + (" (all)" if len(sample) == nq else
                                                 ", uniform random positions, scaled by count"))
    if t_comp:
        what = f"pooling of all {wl.B * wl.n_entries} blocks + " + what
    return {"value": nq / t_step, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": what, "seconds": round(t_comp + t_q, 2)}
