"""Generates the QK instruction blocks of attend_tile.h (between the GENERATED markers).

The blocks are long, regular instruction sequences (36 MFMAs, or 18 pairs of 16x16 MFMAs, with
K-fragment reads kept four ahead and the next tile's DMA interleaved between the MFMAs);
writing them by hand would be error-prone, so they are produced here and committed. Run
`python gen_qk_asm.py` from this directory after changing the sequences below.
"""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
TARGET = os.path.join(HERE, "attend_tile.h")
NL = "\\n"
N = 36      # k-steps of a 576-dim row (16 dims each)
D = 4       # K-fragment reads in flight
C_QK = 1         # independent accumulation chains per QK block (summed on return)
ST_PAIR = 1040   # fp8 staging: bytes between latent row pairs (kStPair in attend_fp8.hip)


def _statement(lines, outs, ins):
    """The asm statement. M0 is a reserved register: each block saves it into an SGPR operand
    (m0s) before its first DMA and restores it after the last one, so the compiler's view of M0
    is intact and it need not (and cannot) be declared clobbered. The s_add_u32 forming the DMA
    bases writes SCC, and the block reads LDS and writes it by DMA: both are declared."""
    out_s = ", ".join('"=&%s"(%s)' % ("s" if o == "m0s" else "v", o) for o in outs)
    in_s = ", ".join('"%s"(%s)' % (c, n) for n, c in ins)
    return "    asm volatile(\n      " + "\n      ".join(lines) + "\n      : " + out_s + \
        "\n      : " + in_s + "\n      : \"scc\", \"memory\");"


def block(mnemonic, q_lat_cons, nv, dmas, tk_rows_v, D=D, C=1):
    """Returns (asm text lines, outputs, inputs) for one QK block.

    dmas: list of DMA ops, each (m0_operand, m0_imm, load_mnemonic, addr_operands) where operands
    are symbolic names resolved below."""
    T = D + 1   # rotating K-fragment registers
    accs = ["acc"] if C == 1 else ["acc", "acc2"]   # C independent accumulation chains
    outs = accs + ["t%d" % i for i in range(T)] + ["vr[%d]" % i for i in range(2 * nv)] + ["m0s"]
    ins = [("q[%d]" % i, q_lat_cons if i < 32 else "v") for i in range(36)]
    ins += [("lb[%d]" % i, "v") for i in range(4)] + [("rb[%d]" % i, "v") for i in range(4)]
    if nv:
        ins += [("ve", "v"), ("vo", "v")]
    dma_names = []
    for d in dmas:
        for name, cons in d[3]:
            if (name, cons) not in dma_names:
                dma_names.append((name, cons))
        if (d[0], "s") not in dma_names:
            dma_names.append((d[0], "s"))
    ins += dma_names
    num = {}
    for i, o in enumerate(outs):
        num[o] = i
    for j, (name, _) in enumerate(ins):
        num[name] = len(outs) + j

    def op(x):
        return "%%%d" % num[x]

    L = []

    def emit(x):
        L.append('"%s%s"' % (x, NL))

    t = ["t%d" % i for i in range(T)]
    emit("s_mov_b32 %s, m0" % op("m0s"))
    for j in range(D):
        emit("ds_read_b128 %s, %s%s" % (op(t[j]), op("lb[%d]" % (j & 3)),
                                        "" if j < 4 else " offset:%d" % (128 * (j >> 2))))
    vreads = []
    for f in range(nv):
        ks, mt = f // 4, f % 4
        koff = (ks >> 1) * 32 * 1024 + (ks & 1) * 16384
        base = "vo" if (mt & 1) else "ve"
        off = 64 * mt + koff
        vreads.append("ds_read_b64_tr_b16 %s, %s offset:%d" % (op("vr[%d]" % (2 * f)), op(base), off))
        vreads.append("ds_read_b64_tr_b16 %s, %s offset:%d"
                      % (op("vr[%d]" % (2 * f + 1)), op(base), off + 8192))
    plan = {32: 6, 33: 6, 34: 2}   # V^T reads after these MFMAs (lgkmcnt stays <= 15)
    nd = len(dmas)
    place = [min(N - 1, (i * N) // nd) for i in range(nd)]
    issued_tr = 0
    di = 0
    for st in range(N):
        kissued = min(N, st + D)
        allowed = (kissued - st - 1) + issued_tr
        assert allowed <= 15
        emit("s_waitcnt lgkmcnt(%d)" % allowed)
        a = accs[st % C]
        src = "0" if st < C else op(a)
        emit("%s %s, %s, %s, %s" % (mnemonic, op(a), op(t[st % T]), op("q[%d]" % st), src))
        nx = st + D
        if nx < N:
            if nx < 32:
                emit("ds_read_b128 %s, %s offset:%d" % (op(t[nx % T]), op("lb[%d]" % (nx & 3)),
                                                        128 * (nx >> 2)))
            else:
                emit("ds_read_b128 %s, %s" % (op(t[nx % T]), op("rb[%d]" % (nx & 3))))
        while di < nd and place[di] == st:
            m0, imm, ld, addr = dmas[di]
            if imm:
                emit("s_add_u32 m0, %s, %d" % (op(m0), imm))
            else:
                emit("s_mov_b32 m0, %s" % op(m0))
            emit("s_nop 0")
            emit("%s %s" % (ld, ", ".join(op(a) if not a.startswith("off") else a
                                          for a in [x[0] for x in addr] + (["off"] if len(addr) == 1 else []))))
            di += 1
        k = plan.get(st, 0) if nv else 0
        if st == N - 1 and nv:
            k = len(vreads) - issued_tr
        for _ in range(min(k, len(vreads) - issued_tr)):
            emit(vreads[issued_tr])
            issued_tr += 1
    assert di == nd
    if nv:
        emit("s_waitcnt lgkmcnt(0)")
    emit("s_mov_b32 m0, %s" % op("m0s"))
    emit("s_nop 7")
    emit("s_nop 7")
    emit("s_nop 4")
    return _statement(L, outs, ins)


def block16(dmas, D=4):
    """S^T for 16 keys x 32 heads with v_mfma_f32_16x16x32_bf16: 18 k-steps of 32 dims, two
    accumulators (heads 0-15, 16-31 of the row group) sharing each K fragment. K-step s reads the
    lane's 16 bytes at (s & 1 ? lbo : lbe) + 128 (s >> 1) for the latent steps 0-15 and at
    (s & 1 ? rbo : rbe) for the RoPE steps 16, 17; Q^T fragment of step s and head half h is
    q[2 s + h] (latent ones from accumulation registers)."""
    NS = 18
    T = D + 1
    outs = ["acc0", "acc1"] + ["t%d" % i for i in range(T)] + ["m0s"]
    ins = [("q[%d]" % i, "a" if i < 32 else "v") for i in range(36)]
    ins += [("lbe", "v"), ("lbo", "v"), ("rbe", "v"), ("rbo", "v")]
    dma_names = []
    for d in dmas:
        for name, cons in d[3]:
            if (name, cons) not in dma_names:
                dma_names.append((name, cons))
        if (d[0], "s") not in dma_names:
            dma_names.append((d[0], "s"))
    ins += dma_names
    num = {}
    for i, o in enumerate(outs):
        num[o] = i
    for j, (name, _) in enumerate(ins):
        num[name] = len(outs) + j

    def op(x):
        return "%%%d" % num[x]

    L = []

    def emit(x):
        L.append('"%s%s"' % (x, NL))

    def kread(st):
        if st < 16:
            base = op("lbo" if st & 1 else "lbe")
            off = 128 * (st >> 1)
        else:
            base = op("rbo" if st & 1 else "rbe")
            off = 0
        return "%s%s" % (base, "" if off == 0 else " offset:%d" % off)

    t = ["t%d" % i for i in range(T)]
    emit("s_mov_b32 %s, m0" % op("m0s"))
    for j in range(D):
        emit("ds_read_b128 %s, %s" % (op(t[j]), kread(j)))
    nd = len(dmas)
    place = [min(NS - 1, (i * NS) // nd) for i in range(nd)]
    di = 0
    for st in range(NS):
        allowed = min(NS, st + D) - st - 1
        assert allowed <= 15
        emit("s_waitcnt lgkmcnt(%d)" % allowed)
        for h in range(2):
            a = "acc%d" % h
            src = "0" if st == 0 else op(a)
            emit("v_mfma_f32_16x16x32_bf16 %s, %s, %s, %s" % (op(a), op(t[st % T]),
                                                              op("q[%d]" % (2 * st + h)), src))
        nx = st + D
        if nx < NS:
            emit("ds_read_b128 %s, %s" % (op(t[nx % T]), kread(nx)))
        while di < nd and place[di] == st:
            m0, imm, ld, addr = dmas[di]
            if imm:
                emit("s_add_u32 m0, %s, %d" % (op(m0), imm))
            else:
                emit("s_mov_b32 m0, %s" % op(m0))
            emit("s_nop 0")
            emit("%s %s" % (ld, ", ".join(op(a) if not a.startswith("off") else a
                                          for a in [x[0] for x in addr] + (["off"] if len(addr) == 1 else []))))
            di += 1
    assert di == nd
    emit("s_mov_b32 m0, %s" % op("m0s"))
    emit("s_nop 7")
    emit("s_nop 7")
    emit("s_nop 4")
    return _statement(L, outs, ins)


def bf16_dmas(nlat, nrope, tk):
    d = [("dma.m0_sel", 0, "global_load_lds_dword", [("dma.sel", "v")])]
    for j in range(nlat):
        d.append(("dma.m0_rows", 4096 * j, "global_load_lds_dwordx4",
                  [("dma.off[%d]" % (j & 1), "v"), ("dma.lat[%d]" % j, "s")]))
    for jj in range(nrope):
        d.append(("dma.m0_rows", tk * 1024 + 4096 * jj, "global_load_lds_dwordx4",
                  [("dma.rope[%d]" % jj, "v")]))
    return d


def f8_dmas():
    d = [("dma.m0_sel", 0, "global_load_lds_dword", [("dma.sel", "v")])]
    for i in range(4):
        d.append(("dma.m0_lat", 4 * ST_PAIR * i, "global_load_lds_dwordx4",
                  [("dma.lat[%d]" % i, "v")]))
    d.append(("dma.m0_rope", 0, "global_load_lds_dwordx4", [("dma.rope", "v")]))
    d.append(("dma.m0_scl", 0, "global_load_lds_dword", [("dma.scl", "v")]))
    return d


def main():
    src = open(TARGET).read()
    b0 = src.index("// ---- BEGIN GENERATED QK BLOCKS ----")
    b1 = src.index("// ---- END GENERATED QK BLOCKS ----")
    gen = ["// ---- BEGIN GENERATED QK BLOCKS ----",
           "// (written by gen_qk_asm.py; edit the generator, not these lines)",
           "__device__ __forceinline__ void qk16_chain(const v4i (&q)[36], int lbe, int lbo, int rbe,",
           "                                           int rbo, const TileDma<8, 1>& dma,",
           "                                           floatx4& acc0, floatx4& acc1) {",
           "  v4i t0, t1, t2, t3, t4;",
           "  int m0s;",
           block16(bf16_dmas(8, 1, 32)),
           "}",
           "",
           "__device__ __forceinline__ floatx16 qk_chain_f16(const v4i (&q)[kKSteps], const int (&lb)[4],",
           "                                                 const int (&rb)[4], const TileDmaF8& dma) {",
           "  floatx16 acc" + (", acc2" if C_QK == 2 else "") + ";",
           "  v4i t0, t1, t2, t3, t4;",
           "  int m0s;",
           block("v_mfma_f32_32x32x16_f16", "v", 0, f8_dmas(), 32, C=C_QK),
           "  return acc" + (" + acc2" if C_QK == 2 else "") + ";",
           "}",
           ""]
    src = src[:b0] + "\n".join(gen) + src[b1:]
    open(TARGET, "w").write(src)
    print("regenerated", TARGET)


if __name__ == "__main__":
    main()
