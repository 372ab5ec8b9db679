// MFMA attention for bf16 caches (csa_attend / hca_attend; 512 latent + 64 RoPE dims per row,
// bf16 queries, heads in groups of 64 or 128 per workgroup): the prefill path.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA: selected compressed rows plus the
// raw window, MQA with one KV shared by every head; HCA: dense over the m'-compressed rows) and the
// MLA section (key row = [latent; RoPE key], value row = latent); yudonglee.me "DeepSeek-V4 详解"
// 2.2 Step 4 and 2.3 Step 2.
//
// A workgroup is 4 waves and serves R = 32 RG heads of one query (RG = 2 or 4 row groups of 32
// heads). Key rows reach LDS by DMA (global_load_lds, 16 bytes per lane, no registers) in tiles of
// TK = 128 / RG rows, double-buffered: tile t + 1 streams in while tile t is computed. Each tile is
// computed in two phases split differently over the waves:
//   QK   wave w takes row group w % RG and key block w / RG (32 keys):
//        S^T[32 keys x 32 heads] = K . Q^T, 36 x mfma_f32_32x32x16_bf16 with Q^T held in
//        registers; each lane owns one head's column, so the softmax is lane-local. P (fp16) goes
//        to LDS in exactly the register layout the PV phase reads back.
//   PV   wave w owns the value dims [128 w, 128 w + 128) of all R heads:
//        O^T[128 dims x R heads] += V^T . P^T, 32 x mfma_f32_32x32x16_f16 per tile; V^T fragments
//        come from transposed LDS reads (ds_read_b64_tr_b16) and each feeds RG MFMAs.
// Splitting the output dims keeps O^T at 64 RG accumulator registers per lane and leaves the
// vector registers for loads in flight. Nothing has to be merged across waves at the end.
//
// Numerics. Keys and queries stay bf16 (products exact in fp32). V converts to fp16 in registers
// (exact in fp16's normal range) and P is fp16 (relative rounding 2^-11). The softmax takes a fixed
// per-head reference: the maximum logit of the first tile that has a key, so no running rescale is
// needed. A later logit about 16 (log2 units) above it overflows P's fp16, and a value outside
// fp16's range overflows V; either turns the output non-finite, which flags the workgroup, and the
// fixup pass then recomputes that query in fp32.
//
// LDS tile layout: rows stay unpadded, split into a latent region ([rows][1024 B]) and a RoPE
// region ([rows][128 B]), so one DMA instruction moves one row's latent (a wave-uniform row
// address). 16-byte chunk c of row r sits at chunk position c ^ f(r), f(r) = 2 (r & 3) + (r >> 2 & 1),
// which keeps the K-fragment reads (8 consecutive rows, one chunk) and the transposed V reads
// (4 consecutive rows, 2 adjacent chunks) free of bank conflicts.
#include "attend_generic.h"
#include "attend_plan.h"
#include "attend_tile.h"

namespace csa {
namespace {

template <int RG, int NBUF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attend_bf16_kernel(AttendArgs a, AttnPlan plan) {
  constexpr int KB = 4 / RG;            // 32-key blocks per tile
  constexpr int TK = 32 * KB;           // keys per tile
  constexpr int kAhead = NBUF - 1;      // tiles in flight ahead of the one being computed
  constexpr int kSlots = NBUF + 1;      // key-code slots: tiles t .. t + NBUF
  constexpr int kDmaOps = TK / 4 + TK / 32;   // tile DMA instructions per wave and tile
  constexpr int R = 32 * RG;            // heads per workgroup
  constexpr int kBufB = TK * kRowB;
  constexpr int kPSteps = TK / 16;      // PV k-steps per tile
  // Two distinct arrays (not halves of one): every access below names its buffer statically, so
  // the compiler can tell that reading one buffer does not wait for the DMA into the other.
  // NBUF tile buffers: the DMA of tile t + NBUF - 1 is issued while tile t is computed.
  __shared__ __attribute__((aligned(1024))) char kv[NBUF][kBufB];
  __shared__ __attribute__((aligned(16))) char s_p[kPSteps * RG * 1024];
  __shared__ int s_code[kSlots][TK];
  __shared__ KeyAddr s_addr[kSlots][TK];   // global addresses of each key's row parts
  __shared__ int s_has_key[kSlots];     // per code slot: the tile holds at least one key
  __shared__ int s_full[kSlots];        // per code slot: every key of the tile is present
  __shared__ int s_sel[2][64];          // selection slots of tiles t + kAhead + 1, t + kAhead + 2
  __shared__ float s_ref[KB][R];
  __shared__ float s_l[KB][R];
  __shared__ int s_flag;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rg = w % RG;                // QK: row group
  const int kb = w / RG;                // QK: key block of the tile
  const int hi = lane >> 5;
  const int per_q = plan.head_groups * plan.n_split;
  const int item = xcd_item();
  const int qi = item / per_q;
  const int rem = item - qi * per_q;
  const int hgrp = rem / plan.n_split;
  const int split = rem - hgrp * plan.n_split;
  const int hbase = hgrp * R;
  const int qrow_i = 32 * rg + (lane & 31);           // QK: this lane's head within the group
  if (threadIdx.x == 0) s_flag = 0;

  const KeyList kl = make_key_list(a, qi);
  const int64_t per_split = (kl.total + plan.n_split - 1) / plan.n_split;
  const int64_t k0 = (int64_t)split * per_split;
  const int64_t ke = k0 + per_split < kl.total ? k0 + per_split : kl.total;
  const RowBases rbases = row_bases(a, kl.b);

  // Q^T fragments (bf16, as stored): head hbase + qrow_i, dims 16 s + 8 hi + [0, 8).
  // Q^T of this lane's head; with two row groups its latent part lives in accumulation registers
  // (O takes the other half), which leaves the vector registers to the loop's loads in flight.
  constexpr bool kQA = RG == 2;
  // With the vector registers freed, the QK block also fetches the tile's V^T fragments.
  constexpr int kNV = RG == 2 ? 4 * kPSteps : 0;
  v4i qb[kKSteps];
  load_q<kQA>(static_cast<const uint16_t*>(a.q) + ((int64_t)qi * a.H + hbase + qrow_i) * kD, hi,
              qb);
  floatx16 o[4][RG];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < RG; ++r) o[mt][r] = floatx16{};
  float m_ref = -INFINITY, l_run = 0.f;
  bool have_ref = false;
  bool overflow = false;
  const float cscale = a.sm_scale * kLog2e;

  // Prologue: key codes of tiles 0 .. NBUF - 1; tiles 0 .. NBUF - 2 in flight, tile 0 landed.
  // Codes are written by wave 0 (TK <= 64 lanes), which also records whether each tile has a key
  // and whether it is full.
  if (threadIdx.x < 64) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      const int c = threadIdx.x < TK ? key_code(a, kl, k0 + j * TK + threadIdx.x, ke) : -1;
      if (threadIdx.x < TK) {
        s_code[j][threadIdx.x] = c;
        s_addr[j][threadIdx.x] = key_addr(rbases, c);
      }
      const bool h = __any(c >= 0);
      const bool f = __all(c >= 0 || threadIdx.x >= TK);
      if (threadIdx.x == 0) {
        s_has_key[j] = h;
        s_full[j] = f;
      }
    }
  }
  __syncthreads();
  const bool sel_dma = kl.sel != nullptr;   // CSA: selection slots come from idx
  const KeyCodes32 kc = key_codes32(kl, ke);
  if (sel_dma && threadIdx.x < 64) dma_sel<TK>(kl, k0 + (kAhead + 1) * TK, ke, s_sel[(kAhead + 1) & 1]);
  // Every tile issues exactly kDmaOps DMA instructions per wave (tiles past the end copy the zero
  // row), so the count of outstanding loads is the same on every path and the waits below stay
  // exact.
#pragma unroll
  for (int j = 0; j < kAhead; ++j) dma_tile<TK>(s_addr[j], kv[j]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // PV addressing. V^T fragment of dim tile mt (32 dims) and k-step s (16 keys): lane (group g,
  // la) reads rows r0 = 16 s + 4 hi + la / 4 (and r0 + 8), dims d = 32 mt + 16 (g & 1) + 4 (la & 3).
  // f(r0) = 2 (la / 4) + hi for every s, and chunk (4 mt + c0) ^ f = 4 (mt ^ f2) + (c0 ^ (f & 3)),
  // so the address is a per-lane base (one for even, one for odd mt) plus compile-time offsets.
  // The key order inside a k-step matches the S^T accumulator layout of the QK phase.
  int v_even, v_odd;
  {
    const int g = lane >> 4, la = lane & 15;
    const int f = 2 * (la >> 2) + hi;
    const int c0 = 2 * (g & 1) + ((la & 3) >> 1);
    const int f2 = f >> 2;
    const int base = (4 * hi + (la >> 2)) * 1024 + 16 * (c0 ^ (f & 3)) + 8 * (la & 1) + 256 * w;
    v_even = base + 64 * f2;
    v_odd = base - 64 * f2;
  }

  // One tile: compute from `cbuf` while the next tile streams into `nbuf`.
  // One tile: compute from `cbuf` while tile t + kAhead streams into `nbuf`.
  // The buffers are restrict-qualified so that the compiler knows that reading the current tile or
  // the P exchange never has to wait for the DMA into `nbuf`.
  auto tile = [&](const char* __restrict__ cbuf, char* __restrict__ nbuf, char* __restrict__ pbuf,
                  int64_t t0, int it) {
    const int slot = it % kSlots;
    const int* codes = s_code[slot];
    // DMA issued from inside the QK block: the selection slots of tile t + kAhead + 2 (every wave
    // copies the same values), then this wave's rows of tile t + kAhead. Per wave and tile that is
    // 1 + kDmaOps instructions, in this order.
    TileDma<TK / 4, TK / 32> dma;
    {
      const int64_t kk = t0 + (kAhead + 2) * TK + lane;
      dma.sel = (sel_dma && lane < TK && kk < ke && kk < kl.n_sel)
                    ? reinterpret_cast<const char*>(kl.sel + kk)
                    : reinterpret_cast<const char*>(kZeroRow);
      const KeyAddr* ad = s_addr[(it + kAhead) % kSlots];
      const char* mine = lane < TK / 4 ? ad[4 * lane + w].lat : nullptr;
      dma.off[0] = 16 * (lane ^ swz(w));
      dma.off[1] = 16 * (lane ^ swz(w + 4));
#pragma unroll
      for (int j = 0; j < TK / 4; ++j) {
        const uint64_t base =
            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(uintptr_t)mine, j)) |
            ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uintptr_t)mine >> 32), j)
             << 32);
        dma.lat[j] = reinterpret_cast<const char*>(base);
      }
#pragma unroll
      for (int jj = 0; jj < TK / 32; ++jj) {
        const int r = 8 * (w + 4 * jj) + (lane >> 3);
        dma.rope[jj] = ad[r].rope + 16 * ((lane & 7) ^ swz(r));
      }
      // Wave-uniform LDS targets, made scalar for the block's M0 writes.
      dma.m0_rows = __builtin_amdgcn_readfirstlane(lds_addr(nbuf) + 1024 * w);
      dma.m0_sel = __builtin_amdgcn_readfirstlane(
          lds_addr(reinterpret_cast<const char*>(s_sel[(it + kAhead + 2) & 1])));
    }

    v2i vraw[kNV > 0 ? 2 * kNV : 1];   // the tile's V^T fragments, fetched by the QK block
    // ---- QK: S^T = K . Q^T for key block kb; latent k-steps 0..31 (chunk 2 s + hi), RoPE 32..35.
    floatx16 acc;
    {
      // Chunk 2 s + hi of row r sits at (2 s + hi) ^ f = 2 (s ^ f1) + (hi ^ f0): for s = 4 q + t
      // that is byte 128 q + 32 (t ^ f1) + 16 (hi ^ f0): four per-lane bases (one per t) plus
      // compile-time offsets.
      const int r = lane & 31;
      const int f = swz(r);
      const int h16 = 16 * (hi ^ (f & 1));
      const int lat = lds_addr(cbuf) + (32 * kb + r) * 1024 + h16;
      const int rope = lds_addr(cbuf) + TK * 1024 + (32 * kb + r) * 128 + h16;
      int lb[4], rb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lb[t] = lat + 32 * (t ^ (f >> 1));
        rb[t] = rope + 32 * (t ^ (f >> 1));
      }
      acc = qk_chain<kQA, kNV, TK / 4, TK / 32, TK>(qb, lb, rb, lds_addr(cbuf) + v_even,
                                                    lds_addr(cbuf) + v_odd, vraw, dma);
    }

    if (!s_full[slot]) {            // empty slots (a partial tile, -1 selections): no logit
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
        acc[i] = codes[key] >= 0 ? acc[i] : -INFINITY;
      }
    }
    // Reference maximum (scaled logits, log2 units), set at the first tile that holds a key. Every
    // head of the query sees the same keys, so the condition is uniform across the workgroup.
    if (!have_ref && s_has_key[slot]) {
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, acc[i] * cscale);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      if (KB > 1) {
        if (hi == 0) s_ref[kb][qrow_i] = tmax;
        lds_barrier();
        float mx = s_ref[0][qrow_i];
#pragma unroll
        for (int j = 1; j < KB; ++j) mx = fmaxf(mx, s_ref[j][qrow_i]);
        tmax = mx;
      }
      m_ref = tmax;
      have_ref = true;
    }
    // Logits more than 2^16 above the reference overflow P's fp16 and reach O as inf/NaN, which
    // the final check flags; no per-tile test is needed.
    const float nm = have_ref ? -m_ref : 0.f;   // no reference yet: the tile is empty, P = 0
    // P^T in the B-operand layout of the PV MFMA: k-step s of lane half hi holds keys
    // 16 s + 4 hi + [0,4) and 16 s + 8 + 4 hi + [0,4) of this key block.
    {
      f16x8 ph[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], cscale, nm));   // exp2(-inf) = 0
        l_run += p;
        ph[i >> 3][i & 7] = (_Float16)p;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s)
        *reinterpret_cast<f16x8*>(pbuf + (((2 * kb + s) * RG + rg) * 64 + lane) * 16) = ph[s];
    }
    lds_barrier();   // P of the whole tile is in LDS

    // ---- PV: O^T[dims 128 w + 32 mt, heads 32 r] += V^T . P^T over the tile's k-steps.
    static_assert(kPSteps * RG == 8, "eight P fragments per tile");
    // 64-head groups read all eight P^T fragments at once; 128-head groups (short of vector
    // registers) read the four of each k-step.
    v4i pall[RG == 2 ? 8 : 4];
    if constexpr (RG == 2) load_p8(lds_addr(pbuf) + lane * 16, pall);
#pragma unroll
    for (int ks = 0; ks < kPSteps; ++ks) {
      if constexpr (RG == 4) load_p4(lds_addr(pbuf) + lane * 16 + 4096 * ks, pall);
      f16x8 pf[RG];
#pragma unroll
      for (int r = 0; r < RG; ++r)
        pf[r] = __builtin_bit_cast(f16x8, pall[(RG == 2 ? ks * RG : 0) + r]);
      const int koff = (ks >> 1) * 32 * 1024 + (ks & 1) * 16384;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        uint2 x0, x1;
        if constexpr (kNV > 0) {
          x0 = __builtin_bit_cast(uint2, vraw[2 * (4 * ks + mt)]);
          x1 = __builtin_bit_cast(uint2, vraw[2 * (4 * ks + mt) + 1]);
        } else {
          const char* b0 = cbuf + ((mt & 1) ? v_odd : v_even) + 64 * mt + koff;
          x0 = __builtin_bit_cast(
              uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(const lds_char*)b0));
          x1 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                             (lds_short4*)(const lds_char*)(b0 + 8 * 1024)));
        }
        const f16x8 vf = bf16x8_to_f16(x0.x, x0.y, x1.x, x1.y);
#pragma unroll
        for (int r = 0; r < RG; ++r)
          o[mt][r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[r], o[mt][r], 0, 0, 0);
      }
    }
    // The selection slots read below were copied during the previous tile; at most the DMA
    // instructions issued after them (that tile's rows, then this tile's slots and rows) may
    // still be outstanding.
    __builtin_amdgcn_s_waitcnt(kVmcntDma<2 * kDmaOps + 1>);
    if (threadIdx.x < 64) {
      // Codes of tile t + kAhead + 1, from the selection slots copied during the previous tile.
      const int kk2 = (int)t0 + (kAhead + 1) * TK + (int)threadIdx.x;
      const int raw2 = sel_dma ? s_sel[(it + kAhead + 1) & 1][threadIdx.x] : 0;
      const int c2 = threadIdx.x < TK ? key_code32(kc, kk2, raw2) : -1;
      const int slot2 = (it + kAhead + 1) % kSlots;
      if (threadIdx.x < TK) {
        s_code[slot2][threadIdx.x] = c2;
        s_addr[slot2][threadIdx.x] = key_addr(rbases, c2);
      }
      const bool h2 = __any(c2 >= 0);
      const bool f2 = __all(c2 >= 0 || threadIdx.x >= TK);
      if (threadIdx.x == 0) {
        s_has_key[slot2] = h2;
        s_full[slot2] = f2;
      }
    }
    // This wave's DMA of tile t + 1 (and the selection slots issued with it) has landed once at most
    // the DMA instructions issued in the last kAhead - 1 tiles are outstanding (vector memory
    // operations complete in order).
    __builtin_amdgcn_s_waitcnt(kVmcntDma<(kAhead - 1) * (kDmaOps + 1)>);
    lds_barrier();                   // every wave is done with this tile and with s_p
  };
  int it = 0;
  for (int64_t t0 = k0; t0 < ke; t0 += TK, ++it)
    tile(kv[it % NBUF], kv[(it + kAhead) % NBUF], s_p, t0, it);
  __builtin_amdgcn_s_waitcnt(0);   // no DMA may land in LDS after the workgroup has finished

  // Row sums of each key block and the reference maxima go through LDS to the PV layout.
  l_run += __shfl_xor(l_run, 32);
  if (hi == 0) {
    s_l[kb][qrow_i] = l_run;
    if (kb == 0) s_ref[0][qrow_i] = m_ref;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) overflow |= !__builtin_isfinite(o[mt][r][i]);
  if (__any(overflow)) atomicOr(&s_flag, 1);
  __syncthreads();
  if (threadIdx.x == 0) plan.flags[item] = s_flag;

  // Outputs (n_split == 1: o / l in fp32) or partials (o / l in fp16, and (m, l)), one 32-head
  // row group at a time, staged in the (now idle) tile buffers.
  char* stage = &kv[0][0];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int hrow = 32 * r + (lane & 31);
    float l = s_l[0][hrow];
#pragma unroll
    for (int j = 1; j < KB; ++j) l += s_l[j][hrow];
    const float m = s_ref[0][hrow];
    const int head = hbase + hrow;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int64_t row0 = plan.n_split == 1 ? (int64_t)qi * a.H + hbase + 32 * r
                                           : ((int64_t)qi * plan.n_split + split) * a.H + hbase + 32 * r;
    if (plan.n_split == 1) {
      stage_rows<float>(o, r, inv, stage);
      if (a.lse != nullptr && w == 0 && hi == 0)
        a.lse[(int64_t)qi * a.H + head] =
            l > 0.f ? (m + __log2f(l)) * 0.6931471805599453f : -INFINITY;
      __syncthreads();
      flush_rows<float>(stage, a.out + row0 * kDC);
    } else {
      stage_rows<_Float16>(o, r, inv, stage);
      if (w == 0 && hi == 0) {
        const int64_t pidx = row0 + (lane & 31);
        plan.ws_ml[pidx * 2] = m;
        plan.ws_ml[pidx * 2 + 1] = l;
      }
      __syncthreads();
      flush_rows<_Float16>(stage, plan.ws_o + row0 * kDC);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_attend_bf16(const AttendArgs& a, const AttnPlan& p, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.Q.nq * p.head_groups * p.n_split);
  if (p.rg == 4)
    attend_bf16_kernel<4, 3><<<grid, 256, 0, s>>>(a, p);
  else
    attend_bf16_kernel<2, 2><<<grid, 256, 0, s>>>(a, p);
  return hipGetLastError();
}

}  // namespace csa
