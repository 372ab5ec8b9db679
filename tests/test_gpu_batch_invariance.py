"""Batch invariance: a query's results are bitwise the same whatever batch it is computed in.

deepseek.csdn.net "一文搞懂 DeepSeek", V4 的其他升级: the kernels are deterministic and
batch-invariant (bitwise-equal outputs whatever a token's position in the batch). The full batch of
a workload runs once; then permuted and resized batches of the same queries (over the same caches)
run through the same C-ABI calls, and every query's scores, selection, outputs and lse must equal
its results in the full batch bit for bit.
"""
import numpy as np
import pytest
import torch

from long_context_compressed_07_amd import lib
from long_context_compressed_07_amd.configs import SMALL
from long_context_compressed_07_amd.inputs import make_inputs
from long_context_compressed_07_amd.layer import Step

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib.load()


def _rerun(step, sel: np.ndarray):
    """Index, top-k, attend (and the HCA layer) for the queries `sel` of the step, in that order,
    as a batch of their own. Returns the per-query outputs."""
    wl, t = step.wl, step.t
    dev = step.dev
    si = torch.from_numpy(sel.astype(np.int64)).to(dev)
    seq, pos = step.seq[si].contiguous(), step.pos[si].contiguous()
    n = sel.size
    N = wl.n_entries
    res = {}
    if wl.kind != "hca_prefill":
        scores = torch.empty((n, N), dtype=torch.float32, device=dev)
        idx = torch.empty((n, wl.k), dtype=torch.int32, device=dev)
        dt = {"f32": lib.F32, "bf16": lib.BF16, "e4m3": lib.E4M3}[wl.idx_dtype]
        lib.csa_index(seq, pos, t["q_i"][si].contiguous(), t["w_i"][si].contiguous(), t["k_i"],
                      scores, dt, wl.H_I, wl.d_I, wl.B, N, wl.m,
                      q_i_scale=t["q_i_scale"][si].contiguous() if "q_i_scale" in t else None,
                      k_i_scale=t.get("k_i_scale"))
        lib.csa_topk(seq, pos, scores, idx, N, wl.m, wl.k)
        out = torch.empty((n, wl.H, wl.d_c), dtype=torch.float32, device=dev)
        lse = torch.empty((n, wl.H), dtype=torch.float32, device=dev)
        lib.csa_attend(seq, pos, t["q"][si].contiguous(), lib.BF16, wl.H, step.entries, wl.m, idx,
                       wl.k, step.raw, wl.window, step.sm_scale, out, lse)
        res.update(scores=scores, idx=idx, out=out, lse=lse)
    if wl.kind == "hybrid_decode":
        ho = torch.empty((n, wl.H, wl.d_c), dtype=torch.float32, device=dev)
        hl = torch.empty((n, wl.H), dtype=torch.float32, device=dev)
        lib.hca_attend(seq, pos, t["q_hca"][si].contiguous(), lib.BF16, wl.H, step.hca_entries,
                       wl.m_hca, step.sm_scale, ho, hl)
        res.update(hca_out=ho, hca_lse=hl)
    if wl.kind == "hca_prefill":
        ho = torch.empty((n, wl.H, wl.d_c), dtype=torch.float32, device=dev)
        hl = torch.empty((n, wl.H), dtype=torch.float32, device=dev)
        lib.hca_attend(seq, pos, t["q"][si].contiguous(), lib.BF16, wl.H, step.entries, wl.m,
                       step.sm_scale, ho, hl)
        res.update(out=ho, lse=hl)
    torch.cuda.synchronize()
    return res


def _full(step):
    names = ("scores", "idx", "out", "lse", "hca_out", "hca_lse")
    return {n: getattr(step, n) for n in names if getattr(step, n, None) is not None}


@pytest.mark.parametrize("cfg,sharp", [("C4", False), ("C5", True), ("C2", False), ("C3", True)])
def test_outputs_independent_of_batch(cfg, sharp):
    # The fp8 decode variants' key lists are split over workgroups (2 splits each).
    wl = SMALL[cfg]
    host = make_inputs(wl, 3100 + int(cfg[1]), sharp=sharp)
    step = Step(wl, host, sm_scale=1.0 if sharp else None)
    step.run()
    torch.cuda.synchronize()
    full = _full(step)
    nq = step.nq
    rng = np.random.default_rng(5)
    batches = [np.arange(nq)[::-1].copy(),                      # reversed
               rng.permutation(nq),                              # shuffled
               np.array([nq - 1]),                               # one query alone
               np.sort(rng.choice(nq, size=max(1, nq // 3), replace=False)),   # a third
               np.concatenate([np.arange(nq), np.arange(nq)[:5]])]          # with repeats
    print(f"[batch] {cfg} nq={nq}: {len(batches)} batches", flush=True)
    for sel in batches:
        got = _rerun(step, sel)
        for name, ref in full.items():
            g = got[name]
            r = ref[torch.from_numpy(sel.astype(np.int64)).to(ref.device)]
            if name == "scores":   # only the visible columns are defined
                continue
            assert torch.equal(g.view(torch.int32) if g.dtype == torch.float32 else g,
                               r.view(torch.int32) if r.dtype == torch.float32 else r), \
                (cfg, name, sel[:8])
        if "scores" in got:
            from long_context_compressed_07_amd.inputs import query_positions
            _, pos = query_positions(wl)
            gs, fs = got["scores"].cpu().numpy(), full["scores"].cpu().numpy()
            for i, q in enumerate(sel):
                nv = min(wl.n_entries, (int(pos[q]) + 1) // wl.m)
                assert (gs[i, :nv].view(np.int32) == fs[q, :nv].view(np.int32)).all(), (cfg, q)
