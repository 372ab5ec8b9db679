"""One step of the hybrid compressed attention layer through libcsa, for a given workload.

`Step(wl, host_inputs)` uploads the storage-format inputs (from `inputs.make_inputs`) to the GPU,
allocates every output and workspace once, and `run()` enqueues the whole hot path on the current
stream: compress (when it is part of the workload) -> index -> top-k -> attend for CSA, compress ->
dense attend for HCA, both layers for the hybrid decode (the HCA layer on a second stream, since
it depends on none of the CSA layer's results). Only marshalling and stream ordering happen here;
every step runs in the library's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import lib
from .configs import Workload
from .inputs import query_positions

_DT = {"f32": lib.F32, "bf16": lib.BF16, "e4m3": lib.E4M3}


def _dev(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.to(device)


class Step:
    def __init__(self, wl: Workload, host: dict, device="cuda", sm_scale: float | None = None):
        self.wl = wl
        self.dev = torch.device(device)
        self.sm_scale = wl.sm_scale if sm_scale is None else sm_scale
        self.t = {k: _dev(v, self.dev) for k, v in host.items()}
        seq, pos = query_positions(wl)
        self.seq = _dev(seq, self.dev)
        self.pos = _dev(pos, self.dev)
        self.nq = seq.size
        B, T, N, d, d_c, d_r = wl.B, wl.T, wl.n_entries, wl.d, wl.d_c, wl.d_r
        f32 = dict(dtype=torch.float32, device=self.dev)
        kv_dt = _DT[wl.kv_dtype]
        kind = wl.kind
        self.ws = {}
        if kind in ("csa_decode", "hybrid_decode") and not wl.d_model:
            self.entries = self._given_store("ent", N)
            pos0 = torch.full((B,), T - wl.window, dtype=torch.int64, device=self.dev)
            self.raw = self._given_store("raw", wl.window, pos0=pos0)
        else:
            # Compressed entries are produced by csa_compress inside the step.
            if kv_dt == lib.F32:
                ent_c = torch.empty((B, N, d), **f32)
                self.entries = lib.Store(ent_c, lib.F32, d_c, d_r, N, d, r_offset=d_c)
            else:
                ent_c = torch.empty((B, N, d), dtype=torch.int16, device=self.dev)
                self.entries = lib.Store(ent_c, lib.BF16, d_c, d_r, N, d, r_offset=d_c)
            if wl.d_model:
                self.raw_x = torch.empty((B, T, d), **f32)
                self.raw = lib.Store(self.raw_x, lib.F32, d_c, d_r, T, d, r_offset=d_c)
            else:
                self.raw = lib.Store(self.t["x"], kv_dt, d_c, d_r, T, d, r_offset=d_c)
        if kind == "hca_prefill":
            self.out = torch.empty((self.nq, wl.H, d_c), **f32)
            self.lse = torch.empty((self.nq, wl.H), **f32)
            need = lib.hca_attend_workspace_bytes(self.nq, wl.H, d_c, N)
            self.ws["hca"] = torch.empty(max(need, 1), dtype=torch.uint8, device=self.dev)
            self._bind()
            return
        self.scores = torch.empty((self.nq, N), **f32)
        self.idx = torch.empty((self.nq, wl.k), dtype=torch.int32, device=self.dev)
        self.out = torch.empty((self.nq, wl.H, d_c), **f32)
        self.lse = torch.empty((self.nq, wl.H), **f32)
        need = lib.csa_topk_workspace_bytes(self.nq, N, wl.k)
        self.ws["topk"] = torch.empty(max(need, 1), dtype=torch.uint8, device=self.dev)
        need = lib.csa_attend_workspace_bytes(self.nq, wl.H, d_c, wl.k + wl.window)
        self.ws["attend"] = torch.empty(max(need, 1), dtype=torch.uint8, device=self.dev)
        if kind == "hybrid_decode":
            nh = wl.n_hca
            self.hca_entries = lib.Store(self.t["hca_c"], lib.E4M3, d_c, d_r, nh, d_c,
                                         r=self.t["hca_r"], ld_r=d_r,
                                         scale=self.t["hca_scale"])
            self.hca_out = torch.empty((self.nq, wl.H, d_c), **f32)
            self.hca_lse = torch.empty((self.nq, wl.H), **f32)
            need = lib.hca_attend_workspace_bytes(self.nq, wl.H, d_c, nh)
            self.ws["hca"] = torch.empty(max(need, 1), dtype=torch.uint8, device=self.dev)
            # The HCA layer reads nothing the CSA layer writes: it runs on a second stream (default
            # priority, like every stream here) beside the CSA attention.
            self._side = torch.cuda.Stream(device=self.dev)
            self._side_h = self._side.cuda_stream
            self._fork = torch.cuda.Event()
            self._join = torch.cuda.Event()
        self._bind()

    def _given_store(self, pfx: str, rows: int, pos0=None) -> lib.Store:
        wl = self.wl
        return lib.Store(self.t[f"{pfx}_c"], lib.E4M3, wl.d_c, wl.d_r, rows, wl.d_c,
                         r=self.t[f"{pfx}_r"], ld_r=wl.d_r, scale=self.t[f"{pfx}_scale"],
                         pos0=pos0)

    # ---- the individual calls ------------------------------------------------------------
    # Each call's arguments are marshalled once (lib's bind=True form); a call then costs the host
    # one foreign call, on the stream current when it is made.
    def _bind(self):
        wl, t = self.wl, self.t
        b = {}
        if wl.kind == "hca_prefill" or wl.compress_on_path:
            if wl.d_model:
                b["compress"] = lib.csa_compress(
                    None, None, lib.F32, t["bias"], wl.m, wl.B, wl.T, wl.d_c, wl.d_r,
                    self.entries, hidden=t["hidden"], w_x=t["w_x"], w_g=t["w_g"],
                    d_model=wl.d_model, raw_x_out=self.raw_x, bind=True)
            else:
                b["compress"] = lib.csa_compress(t["x"], t["g"], _DT[wl.kv_dtype], t["bias"], wl.m,
                                                 wl.B, wl.T, wl.d_c, wl.d_r, self.entries,
                                                 bind=True)
        if wl.kind == "hca_prefill":
            b["hca"] = lib.hca_attend(self.seq, self.pos, t["q"], _DT[wl.q_dtype], wl.H,
                                      self.entries, wl.m, self.sm_scale, self.out, self.lse,
                                      ws=self.ws["hca"], bind=True)
            self._b = b
            return
        b["index"] = lib.csa_index(self.seq, self.pos, t["q_i"], t["w_i"], t["k_i"], self.scores,
                                   _DT[wl.idx_dtype], wl.H_I, wl.d_I, wl.B, wl.n_entries, wl.m,
                                   q_i_scale=t.get("q_i_scale"), k_i_scale=t.get("k_i_scale"),
                                   bind=True)
        b["topk"] = lib.csa_topk(self.seq, self.pos, self.scores, self.idx, wl.n_entries, wl.m,
                                 wl.k, ws=self.ws["topk"], bind=True)
        b["attend"] = lib.csa_attend(self.seq, self.pos, t["q"], _DT[wl.q_dtype], wl.H,
                                     self.entries, wl.m, self.idx, wl.k, self.raw, wl.window,
                                     self.sm_scale, self.out, self.lse, ws=self.ws["attend"],
                                     bind=True)
        if wl.kind == "hybrid_decode":
            b["hca"] = lib.hca_attend(self.seq, self.pos, t["q_hca"], _DT[wl.q_dtype], wl.H,
                                      self.hca_entries, wl.m_hca, self.sm_scale, self.hca_out,
                                      self.hca_lse, ws=self.ws["hca"], bind=True)
        self._b = b

    def _h(self) -> int:
        return torch.cuda.current_stream(self.dev).cuda_stream

    def compress(self):
        self._b["compress"](self._h())

    def index(self):
        self._b["index"](self._h())

    def topk(self):
        self._b["topk"](self._h())

    def attend(self, idx=None):
        if idx is None:
            self._b["attend"](self._h())
            return
        wl = self.wl
        lib.csa_attend(self.seq, self.pos, self.t["q"], _DT[wl.q_dtype], wl.H, self.entries,
                       wl.m, idx, wl.k, self.raw, wl.window, self.sm_scale, self.out, self.lse,
                       ws=self.ws["attend"])

    def hca(self):
        self._b["hca"](self._h())

    def run(self):
        """Enqueue one whole step of the workload's hot path on the current stream (the hybrid
        decode's HCA layer on a second stream that the current one waits for at the end)."""
        wl, b = self.wl, self._b
        main = torch.cuda.current_stream(self.dev)
        h = main.cuda_stream
        if wl.kind == "hca_prefill":
            b["compress"](h)
            b["hca"](h)
            return
        if wl.compress_on_path:
            b["compress"](h)
        b["index"](h)
        if wl.kind == "hybrid_decode":
            # The HCA layer needs nothing the CSA layer computes. It starts once the CSA index,
            # which streams at the memory's rate on every CU, is done, and runs beside the CSA
            # top-k and attention, whose few workgroups leave most CUs free (measured per hybrid
            # step: 110.1 us, against 111.0 us forked before the index; forked after the top-k,
            # with earlier kernels, it measured 150 against 128 us).
            self._fork.record(main)
            self._side.wait_event(self._fork)
            b["hca"](self._side_h)
            self._join.record(self._side)
        b["topk"](h)
        b["attend"](h)
        if wl.kind == "hybrid_decode":
            main.wait_event(self._join)
