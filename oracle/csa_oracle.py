"""Plain fp64 CPU oracle of the hybrid compressed attention layer (CSA + HCA).

TEST INFRASTRUCTURE. This module is the correctness reference for the HIP library. Only tests/,
the smoke check and the CPU-baseline leg of the benchmark may import it. It imports nothing from
the GPU path and shares no code with it; inputs reach it as float64 arrays decoded from the same
storage bytes the GPU reads.

Sources (page title / section, cited per function below):
  [csdn]    deepseek.csdn.net "一文搞懂 DeepSeek：从 V3 的 KV 压缩与 MoE，到 V4 的百万 token 上下文",
            sections "V3 看家本领一：MLA" and "V4 改进一：CSA 与 HCA".
  [yudong]  yudonglee.me "DeepSeek-V4 详解", section 2.2 (CSA Steps 1-4) and 2.3 (HCA Steps 1-2).
  [hongke]  hongke120.com/20112.html, sections 2.2-2.3 and 4.1 (heterogeneous KV cache).
  [jaylab]  jaylab-temp.pages.dev "DeepSeek-V4 — 百万 Token 上下文的高效 MoE 模型",
            section 三大架构创新 1 (混合注意力) and 其他技术细节 (KV cache 混合精度).

The pages print no formulas for the compressor, the indexer or the attention; every formula below
is the plainest reading consistent with their prose, and each reading is named where it is used.

Every function is pinned in tests/test_oracle_*.py by closed forms, invariants, textbook special
cases or brute force on tiny inputs. Readings whose agreement with DeepSeek-V4 itself cannot be
checked (no weights, code or worked example on the pages): the pooling form, the indexer formula
and the provenance of indexer keys -- "parity unpinned" against the model, pinned only for
internal consistency.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_round, e4m3_round, f32_round, E4M3_MAX

NEG_INF = -np.inf


# --------------------------------------------------------------------------------------------
# a1. Projection (fp32 workload only)
# --------------------------------------------------------------------------------------------
def project(hidden: np.ndarray, w_x: np.ndarray, w_g: np.ndarray):
    """Latent KV x and gate logits g as linear maps of the hidden state.

    [csdn] "V3 看家本领一：MLA": the cached latent is a down-projection of the token's input.
    Reading: the gate logits come from a second projection of the same hidden state.
    hidden [T, d_model], w_x and w_g [d_model, d] -> x, g [T, d] (float64 matmul).
    """
    hidden = np.asarray(hidden, dtype=np.float64)
    return hidden @ np.asarray(w_x, np.float64), hidden @ np.asarray(w_g, np.float64)


# --------------------------------------------------------------------------------------------
# a2. Compression: softmax-gated pooling with a learned position bias
# --------------------------------------------------------------------------------------------
def pool_weights(g_block: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Per-channel softmax over the m positions of one block.

    [csdn] V4 改进一 (CSA step one) and [yudong] 2.2 Step 1: m adjacent tokens' KV are merged
    into one row with softmax weights that carry a position bias. Reading: the logit of position i
    in channel c is g[i, c] + bias[i]; the softmax runs over i separately for every channel.
    g_block [m, d], bias [m] -> weights [m, d], each column summing to 1.
    """
    a = np.asarray(g_block, np.float64) + np.asarray(bias, np.float64)[:, None]
    a = a - a.max(axis=0, keepdims=True)
    ea = np.exp(a)
    return ea / ea.sum(axis=0, keepdims=True)


def compress(x: np.ndarray, g: np.ndarray, bias: np.ndarray, m: int) -> np.ndarray:
    """Pool every m consecutive rows of x into one entry: e[j] = sum_i w[i] * x[j*m + i].

    CSA uses m = 4 ([csdn] V4 改进一; [yudong] 2.2 Step 1); HCA uses the same pooling with
    m' = 128 ([yudong] 2.3 Step 1; [hongke] 2.3). A trailing partial block is not emitted
    (reading: only complete blocks become entries).
    x, g [T, d] -> e [T // m, d].
    """
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    n = x.shape[0] // m
    out = np.empty((n, x.shape[1]), dtype=np.float64)
    for j in range(n):
        w = pool_weights(g[j * m:(j + 1) * m], bias)
        out[j] = (w * x[j * m:(j + 1) * m]).sum(axis=0)
    return out


def store_bf16(e: np.ndarray) -> np.ndarray:
    """Storage step of a bf16 entry store: round each value to bf16 (RNE). Returns float64."""
    return bf16_round(e)


def store_e4m3_rows(e_c: np.ndarray):
    """Storage step of an fp8 entry row: one fp32 scale per row and E4M3 codes.

    [jaylab] 其他技术细节: cache rows keep the RoPE dims in bf16 and the rest in FP8. Reading: the
    row scale is sigma = fp32(max_c |e_c| / 448), each value is stored as RNE-satfinite e4m3 of
    e_c / sigma; an all-zero row stores sigma = 0 and zero codes.
    e_c [n, d_c] -> (values of the codes as float64 [n, d_c], sigma float64 [n]).
    """
    e_c = np.asarray(e_c, np.float64)
    amax = np.abs(e_c).max(axis=1)
    sigma = f32_round(amax / E4M3_MAX)
    safe = np.where(sigma > 0, sigma, 1.0)
    q = e4m3_round(e_c / safe[:, None])
    q = np.where(sigma[:, None] > 0, q, 0.0)
    return q, sigma


# --------------------------------------------------------------------------------------------
# a3. Visibility
# --------------------------------------------------------------------------------------------
def n_visible(pos: int, m: int, n_entries: int) -> int:
    """Number of entries a query at absolute position pos may see.

    Reading (the pages are silent on causality over compressed rows): entry j summarises tokens
    [j*m, (j+1)*m - 1] and is visible iff its last token is at or before pos; so
    n_vis = min(N, floor((pos + 1) / m)).
    """
    return int(min(n_entries, (int(pos) + 1) // int(m)))


# --------------------------------------------------------------------------------------------
# a4. Lightning indexer
# --------------------------------------------------------------------------------------------
def index_scores(q_i: np.ndarray, w: np.ndarray, k_i: np.ndarray, n_vis: int) -> np.ndarray:
    """Indexer score of every entry for one query.

    [csdn] V4 改进一 and [yudong] 2.2 Step 2: a light indexer scores each compressed row against
    the query, in the manner of the V3.2 lightning indexer. Reading: per indexer head h a dot
    product, passed through ReLU and weighted by the query's head weight w[h], summed over heads:
        s[j] = sum_h w[h] * max(0, q_i[h] . k_i[j])   for j < n_vis,   -inf otherwise.
    q_i [H_I, d_I] (dequantised), w [H_I], k_i [N, d_I] (dequantised) -> s [N].
    """
    q_i = np.asarray(q_i, np.float64)
    k_i = np.asarray(k_i, np.float64)
    w = np.asarray(w, np.float64)
    n = k_i.shape[0]
    s = np.full(n, NEG_INF)
    if n_vis > 0:
        dots = k_i[:n_vis] @ q_i.T                       # [n_vis, H_I]
        s[:n_vis] = (np.maximum(dots, 0.0) * w[None, :]).sum(axis=1)
    return s


def store_scores_bf16(s: np.ndarray) -> np.ndarray:
    """Storage step of the low-precision indexer's scores: round each visible score to bf16
    (nearest, ties to even); invisible entries stay -inf.

    [csdn] V4 的其他升级 (FP4 paragraph): with the indexer's QK path in FP4, the index scores drop
    to BF16. The scores themselves are index_scores() of the dequantised MXFP4 vectors (an E2M1
    value times its block's power-of-two scale is exact in float64).
    """
    s = np.asarray(s, np.float64)
    out = s.copy()
    fin = np.isfinite(s)
    out[fin] = bf16_round(s[fin])
    return out


def recall(sel: np.ndarray, ref: np.ndarray) -> float:
    """Fraction of the reference selection's entries (-1 slots ignored) that a selection keeps:
    the "KV recall" by which [csdn] V4 的其他升级 rates the low-precision indexer (99.7%)."""
    ref = np.asarray(ref)
    ref = ref[ref >= 0]
    if ref.size == 0:
        return 1.0
    sel = np.asarray(sel)
    return float(np.isin(ref, sel[sel >= 0]).mean())


# --------------------------------------------------------------------------------------------
# a5. Per-query top-k
# --------------------------------------------------------------------------------------------
def topk(s: np.ndarray, n_vis: int, k: int):
    """The k visible entries with the largest score.

    [csdn] V4 改进一 and [yudong] 2.2 Step 3: only the highest-scoring k compressed rows enter
    attention. Readings: ties go to the lower index; the result is listed in ascending index
    order; when fewer than k entries are visible all of them are taken and the rest is -1.
    Also returns the relative gap between the k-th and (k+1)-th largest visible scores
    (+inf when n_vis <= k): the selected set is unique iff the gap is nonzero.
    """
    s = np.asarray(s, np.float64)
    out = np.full(k, -1, dtype=np.int64)
    if n_vis <= 0 or k <= 0:
        return out, np.inf
    j = np.arange(n_vis)
    order = np.lexsort((j, -s[:n_vis]))                  # primary: -s, secondary: j
    take = min(k, n_vis)
    out[:take] = np.sort(order[:take])
    if n_vis <= k:
        return out, np.inf
    a, b = s[order[k - 1]], s[order[k]]
    gap = (a - b) / max(abs(a), abs(b), 1e-300)
    return out, gap


# --------------------------------------------------------------------------------------------
# a6/a7. Attention core
# --------------------------------------------------------------------------------------------
def softmax_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray, sm_scale: float):
    """Softmax attention of several heads against one shared key/value set (MQA).

    [csdn] V4 改进一: CSA attends in MQA form with one KV shared by all heads; [csdn] MLA: scores
    and outputs work directly on the cached latent (up-projections absorbed), so the key row is
    the latent followed by the decoupled RoPE key and the value row is the latent itself.
    q [H, d_k], keys [n, d_k], values [n, d_v] ->
        o [H, d_v] = sum_j p[h, j] values[j],  p = softmax_j(sm_scale * q[h] . keys[j]),
        lse [H]    = log sum_j exp(sm_scale * q[h] . keys[j]).
    An empty key set gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.float64)
    values = np.asarray(values, np.float64)
    h = q.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((h, values.shape[1])), np.full(h, NEG_INF)
    logits = sm_scale * (q @ keys.T)                      # [H, n]
    mx = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - mx)
    den = ex.sum(axis=1, keepdims=True)
    o = (ex / den) @ values
    lse = (mx + np.log(den))[:, 0]
    return o, lse


def kv_rows(c: np.ndarray, r: np.ndarray | None, scale: np.ndarray | None, rows: np.ndarray):
    """Key and value rows of a cache store at the given row numbers.

    A cache row is c[d_c] followed by r[d_r] ([csdn] MLA: latent plus decoupled RoPE key). An fp8
    store carries one scale per row that multiplies the c part ([jaylab] KV cache 混合精度).
    Returns (keys [n, d_c + d_r], values [n, d_c]) in float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cv = np.asarray(c, np.float64)[rows]
    if scale is not None:
        cv = cv * np.asarray(scale, np.float64)[rows][:, None]
    if r is not None and np.asarray(r).shape[-1] > 0:
        keys = np.concatenate([cv, np.asarray(r, np.float64)[rows]], axis=1)
    else:
        keys = cv
    return keys, cv


def window_rows(pos: int, window: int, pos0: int, n_rows: int) -> np.ndarray:
    """Row numbers, in a raw-row store, of the sliding window of a query at position pos.

    [csdn] V4 改进一: besides the selected rows, CSA keeps a short stretch of the most recent raw
    KV uncompressed. Reading: the window is positions [max(0, pos - window + 1), pos], the query's
    own token included. The store is a ring of n_rows rows: position p sits in row
    (p - pos0) mod n_rows (a store holding every position from pos0 on is the case without wrap;
    a window store rolls by overwriting its oldest row). The window must fit in the ring.
    """
    lo = max(0, int(pos) - int(window) + 1)
    p = np.arange(lo, int(pos) + 1) if window > 0 else np.arange(0)
    if p.size > n_rows:
        raise ValueError("the window is longer than the raw store's ring")
    return np.mod(p - int(pos0), int(n_rows)) if p.size else p

def csa_attend_one(q, entries, idx_row, raw, pos: int, window: int, sm_scale: float):
    """CSA attention of one query: selected entries plus the raw sliding window, one softmax.

    [csdn] V4 改进一 and [yudong] 2.2 Step 4. entries and raw are (c, r, scale, pos0) tuples of
    float64 arrays (scale None unless fp8; pos0 the position of raw row 0). idx_row [k] from
    topk() (-1 = empty slot). Readings: the key set is the selected entries followed by the window
    rows, with no de-duplication and no masking beyond the entries' own visibility (already
    enforced by top-k); K = [c; r] and V = c.
    """
    ec, er, es, _ = entries
    rc, rr, rs, rpos0 = raw
    sel = np.asarray(idx_row, dtype=np.int64)
    sel = sel[sel >= 0]
    k1, v1 = kv_rows(ec, er, es, sel)
    wr = window_rows(pos, window, rpos0, np.asarray(rc).shape[0])
    k2, v2 = kv_rows(rc, rr, rs, wr)
    keys = np.concatenate([k1, k2], axis=0)
    vals = np.concatenate([v1, v2], axis=0)
    return softmax_attention(q, keys, vals, sm_scale)


def csa_attend_tokens_one(q, raw, idx_row, m: int, pos: int, window: int, sm_scale: float):
    """Token-selection CSA attention of one query: the original tokens of the selected blocks plus
    the raw sliding window, one softmax.

    [hongke] 2.2 (item 3): after retrieval, attention runs at token granularity over the original
    tokens of each selected block; [yudong] 2.2 Steps 3-4: the top 1024 blocks stand for 4096
    original tokens, attended in full. Readings: block j (a slot of idx_row, -1 = empty) covers
    positions j*m .. j*m + m - 1, taken in that order; the window follows as in csa_attend_one,
    with no de-duplication; keys [c; r], values c. raw is a (c, r, scale, pos0) store holding
    every position it is asked for at row p - pos0.
    """
    rc, rr, rs, rpos0 = raw
    n_rows = np.asarray(rc).shape[0]
    sel = np.asarray(idx_row, dtype=np.int64)
    sel = sel[sel >= 0]
    tok = (sel[:, None] * int(m) + np.arange(int(m))[None, :]).reshape(-1) - int(rpos0)
    if tok.size and (tok.min() < 0 or tok.max() >= n_rows):
        raise ValueError("a selected token is not held by the raw store")
    k1, v1 = kv_rows(rc, rr, rs, tok)
    wr = window_rows(pos, window, rpos0, n_rows)
    k2, v2 = kv_rows(rc, rr, rs, wr)
    return softmax_attention(q, np.concatenate([k1, k2], axis=0),
                             np.concatenate([v1, v2], axis=0), sm_scale)


def hca_attend_one(q, entries, pos: int, m_prime: int, sm_scale: float):
    """HCA attention of one query: dense attention over every visible heavily-compressed entry.

    [csdn] V4 改进一 (HCA) and [yudong] 2.3 Step 2: after m'-fold compression the sequence is short
    enough that no selection is made; attention is dense. Readings: no sliding window; causal
    visibility as in n_visible().
    """
    ec, er, es, _ = entries
    n_vis = n_visible(pos, m_prime, np.asarray(ec).shape[0])
    keys, vals = kv_rows(ec, er, es, np.arange(n_vis))
    return softmax_attention(q, keys, vals, sm_scale)


def lse_merge(parts):
    """Merge attention partials (o_i, lse_i) over disjoint key sets into the result over their
    union: lse = log sum_i exp(lse_i), o = sum_i exp(lse_i - lse) o_i."""
    lses = np.stack([p[1] for p in parts], axis=0)            # [P, H]
    mx = np.max(lses, axis=0)
    mx_safe = np.where(np.isfinite(mx), mx, 0.0)
    wts = np.exp(lses - mx_safe[None, :])                     # exp(-inf) = 0 for empty parts
    tot = wts.sum(axis=0)
    lse = np.where(tot > 0, mx_safe + np.log(np.where(tot > 0, tot, 1.0)), NEG_INF)
    o = sum(wts[i][:, None] * parts[i][0] for i in range(len(parts)))
    o = o / np.where(tot > 0, tot, 1.0)[:, None]
    return o, lse
