"""Test infrastructure: stage-wise and end-to-end comparison of one GPU step with the fp64 oracle.

Stage-wise checks feed each oracle stage the GPU's own upstream outputs (stored entries, scores,
selected indices), so a mismatch is attributed to the stage that produced it. The end-to-end check
compares the GPU's selection with the oracle's own (fp64 scores) wherever the selection is unique
by more than the 1e-4 relative gap.
"""
from __future__ import annotations

import numpy as np
import torch

from long_context_compressed_07_amd.configs import Workload
from long_context_compressed_07_amd.inputs import query_positions
from oracle import csa_oracle as orc
from oracle.numerics import E4M3_MAX, bf16_round, f32_round

from oracle_io import (ATT_TOL, GAP_EXACT, check_topk_valid, dec, rel_err, rel_err_per_query,
                       to_np)

BF16_ULP_REL = 2.0 ** -8


def _blocks_sample(n_blocks: int, limit: int | None, rng) -> np.ndarray:
    if limit is None or n_blocks <= limit:
        return np.arange(n_blocks)
    return np.unique(np.concatenate([[0, n_blocks - 1], rng.choice(n_blocks, limit, False)]))


def check_compress(wl: Workload, host: dict, step, sample_blocks: int | None = None, seed=0):
    """GPU entries vs oracle pooling (on every block, or a sample of blocks per sequence)."""
    rng = np.random.default_rng(seed)
    m, d, d_c = wl.m, wl.d, wl.d_c
    gpu = to_np(step.entries.c)                      # [B, N, d] (f32 or bf16 codes)
    for b in range(wl.B):
        blocks = _blocks_sample(wl.n_entries, sample_blocks, rng)
        if wl.d_model:
            hid = host["hidden"][b].astype(np.float64)
            x, g = orc.project(hid, host["w_x"], host["w_g"])
            raw_gpu = to_np(step.raw_x)[b].astype(np.float64)
            assert rel_err(raw_gpu, x) <= 1e-5, "projected raw rows"
            # fp32 projection error (recursive summation over d_model terms: n 2^-24 sum |h w|)
            # of the pooling's inputs x and g; an error dg in a gate logit moves the entry by at
            # most max|x| |dg| (the softmax weights' derivative is below 1).
            un = wl.d_model * 2.0 ** -24
            dx = un * (np.abs(hid) @ np.abs(host["w_x"].astype(np.float64)))
            dg = un * (np.abs(hid) @ np.abs(host["w_g"].astype(np.float64)))
        for j0 in range(0, len(blocks), 256):
            bl = blocks[j0:j0 + 256]
            rows = (bl[:, None] * m + np.arange(m)[None, :]).reshape(-1)
            if wl.d_model:
                xs, gs = x[rows], g[rows]
            else:
                xs = dec(host["x"][b][rows], wl.kv_dtype)
                gs = dec(host["g"][b][rows], wl.kv_dtype)
            e = np.stack([orc.compress(xs[i * m:(i + 1) * m], gs[i * m:(i + 1) * m],
                                       host["bias"], m)[0] for i in range(len(bl))])
            ge = dec(gpu[b][bl], wl.kv_dtype)
            # fp32 pooling error: a few fp32 ulps of the block's largest input per channel
            # (covers cancellation when the pooled value is far smaller than its inputs).
            xmax = np.abs(xs).reshape(len(bl), m, -1).max(axis=1)
            fp32_abs = 8.0 * m * 2.0 ** -24 * xmax
            if wl.d_model:
                fp32_abs = fp32_abs + dx[rows].reshape(len(bl), m, -1).max(axis=1) + \
                    2.0 * xmax * dg[rows].reshape(len(bl), m, -1).max(axis=1)
            if wl.kv_dtype == "bf16":
                # Half a bf16 ulp of the exact value (RNE of the fp32 result) plus fp32 error.
                bound = BF16_ULP_REL * np.abs(e) + fp32_abs
                assert (np.abs(ge - e) <= bound).all(), "bf16 entries beyond rounding bound"
            else:
                assert (np.abs(ge - e) <= 1e-6 * np.abs(e) + fp32_abs).all(), "fp32 entries"


def _entry_store(wl: Workload, host: dict, step, b: int):
    """Oracle view (float64) of sequence b's compressed entries as the GPU holds them."""
    if wl.compress_on_path or wl.d_model:
        e = dec(to_np(step.entries.c)[b], wl.kv_dtype)
        return (e[:, :wl.d_c], e[:, wl.d_c:] if wl.d_r else None, None, 0)
    return (dec(host["ent_c"][b], "e4m3"), dec(host["ent_r"][b], "bf16"),
            host["ent_scale"][b].astype(np.float64), 0)


def _raw_store(wl: Workload, host: dict, step, b: int):
    if wl.d_model:
        x = to_np(step.raw_x)[b].astype(np.float64)
        return (x[:, :wl.d_c], x[:, wl.d_c:] if wl.d_r else None, None, 0)
    if wl.kind == "csa_prefill":
        x = dec(host["x"][b], wl.kv_dtype)
        return (x[:, :wl.d_c], x[:, wl.d_c:], None, 0)
    return (dec(host["raw_c"][b], "e4m3"), dec(host["raw_r"][b], "bf16"),
            host["raw_scale"][b].astype(np.float64), wl.T - wl.window)


def _indexer(wl: Workload, host: dict):
    if wl.idx_dtype == "e4m3":
        qi = dec(host["q_i"], "e4m3") * host["q_i_scale"][..., None].astype(np.float64)
        ki = dec(host["k_i"], "e4m3") * host["k_i_scale"][..., None].astype(np.float64)
    else:
        qi, ki = dec(host["q_i"], wl.idx_dtype), dec(host["k_i"], wl.idx_dtype)
    return qi, ki, host["w_i"].astype(np.float64)


def _lse_err(got: np.ndarray, ref: np.ndarray) -> float:
    fin = np.isfinite(ref)
    assert (np.isfinite(got) == fin).all(), "lse finiteness differs"
    assert (got[~fin] == ref[~fin]).all(), "empty key sets must give lse = -inf"
    return float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0


def _subset(store, rows: np.ndarray):
    """(store restricted to the given rows, as float64, with the same tuple form)."""
    c, r, sc, pos0 = store
    rows = np.asarray(rows, np.int64)
    return (np.asarray(c)[rows], None if r is None else np.asarray(r)[rows],
            None if sc is None else np.asarray(sc)[rows], pos0)


def _entry_rows(wl: Workload, host: dict, step, b: int, rows: np.ndarray):
    """Oracle view (float64) of the given rows of sequence b's entry store as the GPU holds it."""
    if wl.compress_on_path or wl.d_model:
        e = dec(to_np(step.entries.c)[b][rows], wl.kv_dtype)
        return (e[:, :wl.d_c], e[:, wl.d_c:] if wl.d_r else None, None, 0)
    return (dec(host["ent_c"][b][rows], "e4m3"), dec(host["ent_r"][b][rows], "bf16"),
            host["ent_scale"][b][rows].astype(np.float64), 0)


def _attend_selected(q, store_rows_fn, idx_row, raw, pos, window, sm_scale):
    """csa_attend_one over only the rows an index row selects (decoded on demand): the store is
    restricted to the selected rows and the slots renumbered, which leaves the key list (and its
    order) unchanged."""
    idx_row = np.asarray(idx_row, np.int64)
    valid = idx_row >= 0
    sub = store_rows_fn(idx_row[valid])
    local = np.full(idx_row.shape, -1, np.int64)
    local[valid] = np.arange(int(valid.sum()))
    return orc.csa_attend_one(q, sub, local, raw, pos, window, sm_scale)


def check_csa(wl: Workload, host: dict, step, qsel=None, stats: dict | None = None):
    """Index, top-k and attention of the CSA layer for the queries in qsel (default: all)."""
    seq, pos = query_positions(wl)
    qsel = np.arange(seq.size) if qsel is None else np.asarray(qsel)
    qi_all, ki_all, wi_all = _indexer(wl, host)
    scores = step.scores.detach().cpu().numpy()
    idx = step.idx.detach().cpu().numpy()
    out = step.out.detach().cpu().numpy()
    lse = step.lse.detach().cpu().numpy()
    q_all = host["q"]
    raws = {}
    ref_o, ref_lse, got_o, got_lse = [], [], [], []
    n_exact = n_tie = 0
    for qi in qsel:
        b, p = int(seq[qi]), int(pos[qi])
        nv = orc.n_visible(p, wl.m, wl.n_entries)
        s_ref = orc.index_scores(qi_all[qi], wi_all[qi], ki_all[b], nv)
        s_gpu = scores[qi, :nv].astype(np.float64)
        if nv:
            assert rel_err(s_gpu, s_ref[:nv]) <= 1e-5, f"index scores, query {qi}"
        # Top-k on the GPU's own scores is integer work: bit-exact.
        sel_o, _ = orc.topk(s_gpu, nv, wl.k)
        assert (sel_o == idx[qi]).all(), f"top-k of identical scores differs, query {qi}"
        # End to end against the oracle's fp64 scores.
        sel_ref, gap = orc.topk(s_ref, nv, wl.k)
        if gap > GAP_EXACT:
            assert (sel_ref == idx[qi]).all(), f"selection differs at gap {gap}, query {qi}"
            n_exact += 1
        else:
            check_topk_valid(idx[qi], s_ref, nv, wl.k)
            n_tie += 1
        if b not in raws:
            raws.clear()
            raws[b] = _raw_store(wl, host, step, b)
        q = dec(q_all[qi], wl.q_dtype)
        o, l = _attend_selected(q, lambda rows: _entry_rows(wl, host, step, b, rows), idx[qi],
                                raws[b], p, wl.window, step.sm_scale)
        ref_o.append(o); ref_lse.append(l); got_o.append(out[qi]); got_lse.append(lse[qi])
    per_q = rel_err_per_query(np.stack(got_o), np.stack(ref_o))
    err = float(per_q.max()) if per_q.size else 0.0
    lse_err = _lse_err(np.stack(got_lse), np.stack(ref_lse))
    if stats is not None:
        stats.update(attend_rel_err=err, attend_rel_err_call=rel_err(np.stack(got_o),
                                                                      np.stack(ref_o)),
                     worst_query=int(np.asarray(qsel)[int(np.argmax(per_q))]) if per_q.size else -1,
                     lse_abs_err=lse_err, exact_sets=n_exact, tie_sets=n_tie)
    assert err <= ATT_TOL[wl.kv_dtype], \
        f"attention rel err {err} at query {np.asarray(qsel)[int(np.argmax(per_q))]}"
    assert lse_err <= 1e-3, f"lse abs err {lse_err}"


def check_hca(wl: Workload, host: dict, step, qsel=None, stats: dict | None = None):
    seq, pos = query_positions(wl)
    qsel = np.arange(seq.size) if qsel is None else np.asarray(qsel)
    if wl.kind == "hca_prefill":
        out, lse, qs, m_h = step.out, step.lse, host["q"], wl.m
    else:
        out, lse, qs, m_h = step.hca_out, step.hca_lse, host["q_hca"], wl.m_hca
    out = out.detach().cpu().numpy()
    lse = lse.detach().cpu().numpy()
    ents = {}
    ref_o, ref_l, got_o, got_l = [], [], [], []
    for qi in qsel:
        b, p = int(seq[qi]), int(pos[qi])
        if b not in ents:
            if wl.kind == "hca_prefill":
                ents[b] = _entry_store(wl, host, step, b)
            else:
                ents[b] = (dec(host["hca_c"][b], "e4m3"), dec(host["hca_r"][b], "bf16"),
                           host["hca_scale"][b].astype(np.float64), 0)
        o, l = orc.hca_attend_one(dec(qs[qi], wl.q_dtype), ents[b], p, m_h, step.sm_scale)
        ref_o.append(o); ref_l.append(l); got_o.append(out[qi]); got_l.append(lse[qi])
    per_q = rel_err_per_query(np.stack(got_o), np.stack(ref_o))
    err = float(per_q.max()) if per_q.size else 0.0
    lse_err = _lse_err(np.stack(got_l), np.stack(ref_l))
    if stats is not None:
        stats.update(hca_rel_err=err, hca_rel_err_call=rel_err(np.stack(got_o), np.stack(ref_o)),
                     hca_lse_abs_err=lse_err)
    assert err <= ATT_TOL[wl.kv_dtype], f"HCA rel err {err}"
    assert lse_err <= 1e-3, f"HCA lse abs err {lse_err}"


def oracle_entry_store(wl: Workload, host: dict, b: int, chunk: int = 256):
    """The oracle's own compressed entries of sequence b, from the raw inputs: projection (fp32
    workload), pooling in fp64, then the storage step of the workload's entry dtype."""
    m, N, d_c = wl.m, wl.n_entries, wl.d_c
    if wl.d_model:
        x, g = orc.project(host["hidden"][b].astype(np.float64), host["w_x"], host["w_g"])
    parts = []
    for j0 in range(0, N, chunk):
        j1 = min(N, j0 + chunk)
        if wl.d_model:
            xs, gs = x[j0 * m:j1 * m], g[j0 * m:j1 * m]
        else:
            xs = dec(host["x"][b, j0 * m:j1 * m], wl.kv_dtype)
            gs = dec(host["g"][b, j0 * m:j1 * m], wl.kv_dtype)
        parts.append(orc.compress(xs, gs, host["bias"], m))
    e = np.concatenate(parts) if parts else np.zeros((0, wl.d))
    e = orc.store_bf16(e) if wl.kv_dtype == "bf16" else f32_round(e)
    return (e[:, :d_c], e[:, d_c:] if wl.d_r else None, None, 0)


def oracle_raw_store(wl: Workload, host: dict, b: int):
    """The raw window rows as the oracle forms them (prefill workloads): the stored x rows, or
    for the fp32 workload the oracle's own projection rounded to the fp32 store."""
    if wl.d_model:
        x, _ = orc.project(host["hidden"][b].astype(np.float64), host["w_x"], host["w_g"])
        x = f32_round(x)
        return (x[:, :wl.d_c], x[:, wl.d_c:] if wl.d_r else None, None, 0)
    x = dec(host["x"][b], wl.kv_dtype)
    return (x[:, :wl.d_c], x[:, wl.d_c:], None, 0)


def check_end_to_end(wl: Workload, host: dict, step, qsel=None, stats: dict | None = None):
    """The GPU's final outputs against the oracle run from the raw inputs alone: the oracle's own
    pooled and stored entries (prefill workloads), its own fp64 index scores and its own
    selection. Queries whose selection is not unique by more than the 1e-4 relative gap are
    skipped (several sets are correct there) and counted."""
    seq, pos = query_positions(wl)
    qsel = np.arange(seq.size) if qsel is None else np.asarray(qsel)
    hca = wl.kind == "hca_prefill"
    out = step.out.detach().cpu().numpy()
    if not hca:
        qi_all, ki_all, wi_all = _indexer(wl, host)
    ents, raws = {}, {}
    got, ref, n_skip = [], [], 0
    for qi in qsel:
        b, p = int(seq[qi]), int(pos[qi])
        if b not in ents:
            ents.clear(); raws.clear()
            if wl.compress_on_path or wl.d_model:
                ents[b] = oracle_entry_store(wl, host, b)
                raws[b] = None if hca else oracle_raw_store(wl, host, b)
            else:
                ents[b] = None
                raws[b] = _raw_store(wl, host, step, b)
        q = dec(host["q"][qi], wl.q_dtype)
        if hca:
            o, _ = orc.hca_attend_one(q, ents[b], p, wl.m, step.sm_scale)
        else:
            nv = orc.n_visible(p, wl.m, wl.n_entries)
            s_ref = orc.index_scores(qi_all[qi], wi_all[qi], ki_all[b], nv)
            sel, gap = orc.topk(s_ref, nv, wl.k)
            if gap <= GAP_EXACT:
                n_skip += 1
                continue
            if ents[b] is None:
                o, _ = _attend_selected(q, lambda rows: _entry_rows(wl, host, step, b, rows), sel,
                                        raws[b], p, wl.window, step.sm_scale)
            else:
                o, _ = orc.csa_attend_one(q, ents[b], sel, raws[b], p, wl.window, step.sm_scale)
        got.append(out[qi]); ref.append(o)
    per_q = rel_err_per_query(np.stack(got), np.stack(ref)) if got else np.zeros(0)
    err = float(per_q.max()) if per_q.size else 0.0
    if stats is not None:
        stats.update(e2e_rel_err=err, e2e_queries=len(got), e2e_skipped_ties=n_skip)
    assert err <= ATT_TOL[wl.kv_dtype], f"end-to-end rel err {err}"


def check_compress_e4m3(wl: Workload, host: dict, ent_c: np.ndarray, ent_r: np.ndarray,
                        ent_scale: np.ndarray, sample_blocks: int | None = None, seed: int = 0):
    """GPU entries stored as e4m3 rows (codes, row scale, bf16 RoPE part) against the oracle's
    pooling and its e4m3 storage step (store_e4m3_rows): the scale within the fp32 pooling error
    of the oracle's, each code within one e4m3 step of the oracle's, and the dequantised value
    within half an e4m3 step (relative 2^-4, or the subnormal step) plus that error."""
    rng = np.random.default_rng(seed)
    m, d_c = wl.m, wl.d_c
    for b in range(wl.B):
        blocks = _blocks_sample(wl.n_entries, sample_blocks, rng)
        rows = (blocks[:, None] * m + np.arange(m)[None, :]).reshape(-1)
        xs = dec(host["x"][b][rows], wl.kv_dtype)
        gs = dec(host["g"][b][rows], wl.kv_dtype)
        e = np.stack([orc.compress(xs[i * m:(i + 1) * m], gs[i * m:(i + 1) * m], host["bias"],
                                   m)[0] for i in range(len(blocks))])
        q_ref, sig_ref = orc.store_e4m3_rows(e[:, :d_c])
        xmax = np.abs(xs).reshape(len(blocks), m, -1).max(axis=1)
        fp32_abs = 8.0 * m * 2.0 ** -24 * xmax                  # per channel
        amax_err = fp32_abs[:, :d_c].max(axis=1)
        sig = ent_scale[b][blocks].astype(np.float64)
        assert (np.abs(sig - sig_ref) * E4M3_MAX <= amax_err + 2.0 ** -23 * sig_ref * E4M3_MAX).all(), \
            "e4m3 row scale"
        codes = dec(ent_c[b][blocks], "e4m3")
        # one e4m3 step at the code's magnitude: 2^(floor(log2 |q|) - 3), at least 2^-9
        mag = np.maximum(np.abs(q_ref), 2.0 ** -6)
        step = np.ldexp(1.0, np.floor(np.log2(mag)).astype(np.int64) - 3)
        assert (np.abs(codes - q_ref) <= step + 1e-12).all(), "e4m3 codes beyond one step"
        deq = codes * sig[:, None]
        bound = 2.0 ** -4 * np.abs(e[:, :d_c]) + 2.0 ** -10 * sig[:, None] + \
            2.0 * fp32_abs[:, :d_c] + 2.0 ** -23 * np.abs(e[:, :d_c])
        assert (np.abs(deq - e[:, :d_c]) <= bound).all(), "dequantised e4m3 entries"
        r = dec(ent_r[b][blocks], "bf16")
        assert (np.abs(r - e[:, d_c:]) <= BF16_ULP_REL * np.abs(e[:, d_c:]) +
                fp32_abs[:, d_c:]).all(), "bf16 RoPE part of e4m3 entries"


def outputs(step) -> list[torch.Tensor]:
    names = ["entries", "scores", "idx", "out", "lse", "hca_out", "hca_lse", "raw_x"]
    res = []
    for n in names:
        v = getattr(step, n, None)
        if v is None:
            continue
        res.append(v.c if n == "entries" else v)
    return res
