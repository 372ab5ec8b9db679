"""CPU checks of the GPU-parity harness itself (tests/parity.py, tests/oracle_io.py).

A stand-in for a GPU step is filled with the oracle's own results on a tiny workload; every check
must accept it, and must reject it once a plausible mistake is planted in it (a dropped top entry
at a near-tie, a wrong key in the attention, a mis-rounded fp8 code, a wrong row scale).
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from long_context_compressed_07_amd.configs import SMALL
from long_context_compressed_07_amd.inputs import make_inputs, query_positions, to_bf16_bits
from oracle import csa_oracle as orc
from oracle.numerics import E4M3_MAX

import parity
from oracle_io import check_topk_valid, dec, rel_err_per_query


def _fake_step(wl, host):
    """Oracle results in the layout a GPU step exposes (torch CPU tensors)."""
    seq, pos = query_positions(wl)
    ent = parity.oracle_entry_store(wl, host, 0)
    e = np.concatenate([ent[0], ent[1]], axis=1)
    codes = to_bf16_bits(e.astype(np.float32))[None]
    qi, ki, wi = parity._indexer(wl, host)
    N = wl.n_entries
    scores = np.full((seq.size, N), -np.inf, np.float32)
    idx = np.full((seq.size, wl.k), -1, np.int32)
    out = np.zeros((seq.size, wl.H, wl.d_c), np.float32)
    lse = np.zeros((seq.size, wl.H), np.float32)
    raw = parity.oracle_raw_store(wl, host, 0)
    for i in range(seq.size):
        nv = orc.n_visible(int(pos[i]), wl.m, N)
        s = orc.index_scores(qi[i], wi[i], ki[0], nv).astype(np.float32)
        scores[i] = s
        sel, _ = orc.topk(s.astype(np.float64), nv, wl.k)
        idx[i] = sel
        o, l = orc.csa_attend_one(dec(host["q"][i], "bf16"), ent, sel, raw, int(pos[i]),
                                  wl.window, wl.sm_scale)
        out[i], lse[i] = o, l
    return SimpleNamespace(entries=SimpleNamespace(c=torch.from_numpy(codes.view(np.int16))),
                           scores=torch.from_numpy(scores), idx=torch.from_numpy(idx),
                           out=torch.from_numpy(out), lse=torch.from_numpy(lse),
                           sm_scale=wl.sm_scale)


@pytest.fixture(scope="module")
def tiny():
    wl = SMALL["C2"].replace(T=4 * 30 + 3, nq=4 * 30 + 3, k=8, window=6, H=4)
    host = make_inputs(wl, 99)
    return wl, host, _fake_step(wl, host)


def test_harness_accepts_oracle_results(tiny):
    wl, host, step = tiny
    stats = {}
    parity.check_compress(wl, host, step)
    parity.check_csa(wl, host, step, stats=stats)
    parity.check_end_to_end(wl, host, step, stats=stats)
    assert stats["attend_rel_err"] < 1e-6 and stats["e2e_rel_err"] < 1e-6
    assert stats["e2e_queries"] > 0


def test_harness_rejects_a_wrong_output(tiny):
    wl, host, step = tiny
    bad = SimpleNamespace(**vars(step))
    o = step.out.clone()
    o[wl.nq - 1, 2, 7] += 0.01 * float(o[wl.nq - 1].abs().max())   # 1% of one late query
    bad.out = o
    with pytest.raises(AssertionError):
        parity.check_end_to_end(wl, host, bad)
    with pytest.raises(AssertionError):
        parity.check_csa(wl, host, bad)


def test_per_query_error_is_not_masked_by_a_large_query():
    ref = np.zeros((2, 3))
    ref[0] = 100.0          # a query with large outputs
    ref[1] = 1.0
    got = ref.copy()
    got[1, 0] += 0.01       # 1% error on the small query: 1e-4 of the call-wide maximum
    per_q = rel_err_per_query(got, ref)
    assert per_q[0] == 0.0 and abs(per_q[1] - 0.01) < 1e-12


def test_topk_validity_rejects_a_dropped_maximum():
    s = np.array([5.0, 1.0, 3.0, 3.0 * (1 + 1e-6), 0.5])
    check_topk_valid(np.array([0, 2, -1])[:2], s, 5, 2)        # {0, 2}: near-tie at 3, valid
    check_topk_valid(np.array([0, 3]), s, 5, 2)
    with pytest.raises(AssertionError):
        check_topk_valid(np.array([2, 3]), s, 5, 2)             # drops the maximum (index 0)


def test_e4m3_compress_check(tiny):
    wl, host, _ = tiny
    e = parity.oracle_entry_store(wl, host, 0)
    full = np.concatenate([orc.compress(dec(host["x"][0], "bf16"), dec(host["g"][0], "bf16"),
                                        host["bias"], wl.m)], axis=0)
    q, sig = orc.store_e4m3_rows(full[:, :wl.d_c])
    codes = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
    ent_c = codes.numpy()[None]
    ent_r = to_bf16_bits(full[:, wl.d_c:].astype(np.float32))[None]
    ent_s = sig.astype(np.float32)[None]
    parity.check_compress_e4m3(wl, host, ent_c, ent_r, ent_s)
    bad_s = ent_s.copy()
    bad_s[0, 3] *= 1.01
    with pytest.raises(AssertionError):
        parity.check_compress_e4m3(wl, host, ent_c, ent_r, bad_s)
    bad_c = ent_c.copy()
    j = int(np.argmax(np.abs(q[5])))             # the code at +-448: two steps down
    bad_c[0, 5, j] = (bad_c[0, 5, j] & 0x80) | 0x7c
    with pytest.raises(AssertionError):
        parity.check_compress_e4m3(wl, host, bad_c, ent_r, ent_s)
    assert np.abs(q).max() == E4M3_MAX
    del e
