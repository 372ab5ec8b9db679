"""GPU parity of csa_attend_tokens (the token-selection variant) against the oracle.

hongke120.com 2.2 item 3 and yudonglee.me "DeepSeek-V4 详解" 2.2 Steps 3-4: the selected blocks'
original tokens (m per block) are attended instead of their pooled entries, with the raw window in
the same softmax. The selection comes from the layer's own index and top-k; the raw token store is
the prefill's token rows (bf16) or a full fp8 token cache (decode).
"""
import numpy as np
import pytest
import torch

from long_context_compressed_07_amd import lib
from long_context_compressed_07_amd.configs import SMALL
from long_context_compressed_07_amd.inputs import _e4m3_rows, _normal, make_inputs, \
    query_positions, to_bf16_bits
from long_context_compressed_07_amd.layer import Step
from oracle import csa_oracle as orc

from oracle_io import ATT_TOL, dec, rel_err_per_query

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()


def _check(wl, q_host, raw_host, idx, out, lse, sm_scale, qsel):
    seq, pos = query_positions(wl)
    got, ref, got_l, ref_l = [], [], [], []
    for qi in qsel:
        b, p = int(seq[qi]), int(pos[qi])
        o, l = orc.csa_attend_tokens_one(dec(q_host[qi], wl.q_dtype), raw_host(b), idx[qi], wl.m,
                                         p, wl.window, sm_scale)
        got.append(out[qi]); ref.append(o); got_l.append(lse[qi]); ref_l.append(l)
    err = rel_err_per_query(np.stack(got), np.stack(ref)).max()
    lerr = np.abs(np.stack(got_l) - np.stack(ref_l)).max()
    print(f"tokens: max per-query rel err {err:.2e}, lse {lerr:.2e}", flush=True)
    assert err <= ATT_TOL[wl.kv_dtype] and lerr <= 1e-3


@pytest.mark.parametrize("sharp", [False, True])
def test_tokens_prefill_bf16(sharp):
    wl = SMALL["C2"].replace(T=4 * 300 + 3, nq=4 * 300 + 3, k=40, window=24)
    print(f"[tokens] prefill bf16 sharp={sharp}", flush=True)
    host = make_inputs(wl, 5150, sharp=sharp)
    step = Step(wl, host, sm_scale=1.0 if sharp else None)
    step.run()
    out = torch.empty_like(step.out)
    lse = torch.empty_like(step.lse)
    lib.csa_attend_tokens(step.seq, step.pos, step.t["q"], lib.BF16, wl.H, step.raw, wl.m,
                          step.idx, wl.k, wl.window, step.sm_scale, out, lse)
    torch.cuda.synchronize()
    x = dec(host["x"][0], "bf16")
    raw = (x[:, :wl.d_c], x[:, wl.d_c:], None, 0)
    qsel = np.unique(np.concatenate([np.arange(0, wl.nq, 7), np.arange(wl.nq - 6, wl.nq)]))
    _check(wl, host["q"], lambda b: raw, step.idx.cpu().numpy(), out.cpu().numpy(),
           lse.cpu().numpy(), step.sm_scale, qsel)


def test_tokens_decode_fp8_split():
    # fp8 token cache of every position; 520 blocks x 4 tokens + 64 window rows = 2144 keys per
    # query, split over workgroups.
    wl = SMALL["C4"]
    print("[tokens] decode fp8", flush=True)
    host = make_inputs(wl, 5151, sharp=True)
    step = Step(wl, host, sm_scale=1.0)
    step.run()
    rng = np.random.default_rng(5152)
    d = wl.d
    tc, ts = _e4m3_rows(rng, (wl.B, wl.T, wl.d_c), 1.0 / np.sqrt(d))
    tr = to_bf16_bits(_normal(rng, (wl.B, wl.T, wl.d_r), 1.0 / np.sqrt(d)))
    dev = step.dev
    store = lib.Store(torch.from_numpy(tc).to(dev), lib.E4M3, wl.d_c, wl.d_r, wl.T, wl.d_c,
                      r=torch.from_numpy(tr.view(np.int16)).to(dev), ld_r=wl.d_r,
                      scale=torch.from_numpy(ts).to(dev))
    out = torch.empty_like(step.out)
    lse = torch.empty_like(step.lse)
    lib.csa_attend_tokens(step.seq, step.pos, step.t["q"], lib.BF16, wl.H, store, wl.m, step.idx,
                          wl.k, wl.window, 1.0, out, lse)
    torch.cuda.synchronize()

    def raw(b):
        return (dec(tc[b], "e4m3") * ts[b][:, None].astype(np.float64), dec(tr[b], "bf16"),
                None, 0)
    _check(wl, host["q"], raw, step.idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy(), 1.0,
           np.arange(wl.B * wl.nq))
