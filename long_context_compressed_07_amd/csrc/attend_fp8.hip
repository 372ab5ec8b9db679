// MFMA attention for fp8 caches (csa_attend / hca_attend; e4m3 latent rows of 512 dims with one fp32
// scale per row, bf16 RoPE rows of 64 dims, bf16 queries, heads in groups of 128 per workgroup):
// the decode path.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA: selected compressed rows plus the
// raw window, MQA with one KV shared by every head; HCA: dense over the m'-compressed rows) and the
// MLA section (key row = [latent; RoPE key], value row = latent); yudonglee.me "DeepSeek-V4 详解"
// 2.2 Step 4 and 2.3 Step 2; jaylab-temp.pages.dev "DeepSeek-V4 — 百万 Token 上下文的高效 MoE 模型"
// 其他技术细节 (fp8 latent with bf16 RoPE dims in the KV cache).
//
// A workgroup of 4 waves serves 128 heads (four 32-head row groups) of one query (and one key
// range when a query's keys are split over workgroups); in tiles of 32 keys, wave w computes S^T for row group w (QK) and then O^T for the value dims
// [128 w, 128 w + 128) of all 128 heads (PV), with P exchanged through LDS. What differs is the
// staging: rows arrive by DMA in their compact cache format (512 B fp8 latent, 128 B bf16 RoPE,
// 4 B scale) into one of three staging slots, three tiles ahead of use. While tile t's PV runs,
// the waves convert tile t + 1 from its staging slot into an fp16 tile in the shared layout
// (attend_tile.h): latent = e4m3 value x row scale, RoPE = the bf16 value, both rounded to fp16.
// QK and PV then run as fp16 MFMAs with no per-fragment conversion.
//
// Numerics. The scale is applied in two exact-or-rounded-once steps: its power of two inside the
// fp8 conversion (exact), its mantissa as an fp16 multiply (one rounding, relative 2^-11). Queries
// are rounded bf16 -> fp16 (exact in fp16's normal range), P is fp16, accumulation is fp32. As in
// the bf16 kernel (attend_pp.hip), the softmax uses a fixed per-head reference and a non-finite output (overflow of
// fp16 P or of a converted value) flags the workgroup for the fp32 fixup pass.
#include "attend_generic.h"
#include "attend_plan.h"
#include "attend_tile.h"

namespace csa {
namespace {

constexpr int kTK = 32;                      // keys per tile
// Staging: fp8 latent rows in 16 pairs (rows j and j + 16, 512 B apart, one DMA instruction
// each); pair j starts at kStPair j, 16 bytes past a multiple of 1 KB per pair, so that the
// conversion's reads of one part of 8 consecutive rows fall in 8 different LDS bank groups.
constexpr int kStPair = 1024 + 16;
constexpr int kStLat = 16 * kStPair;         // staging: fp8 latent rows
constexpr int kStRope = kTK * 128;           // staging: bf16 RoPE rows
constexpr int kStB = kStLat + kStRope + 1024;   // + row scales (64 x 4 B written), rounded to 1 KB
constexpr int kNst = 3;                      // staging slots (tiles t + 1 .. t + 3)
constexpr int kAheadF8 = 3;                  // DMA issued three tiles ahead of use
constexpr int kSlotsF8 = kAheadF8 + 2;       // key-code slots: tiles t .. t + 4
constexpr int kDmaOpsF8 = 6;                 // per wave and tile: 4 latent pairs, RoPE, scales

// Row addressing of the two stores of one sequence (entries, raw window rows).
struct RowBases8 {
  const char* c0;          // fp8 latent rows
  const char* c1;
  const char* r0;          // bf16 RoPE rows
  const char* r1;
  const char* s0;          // fp32 row scales
  const char* s1;
  uint32_t ldc0, ldc1, ldr0, ldr1;   // row strides in bytes
};

__device__ __forceinline__ RowBases8 row_bases8(const AttendArgs& a, int64_t b) {
  RowBases8 rb;
  rb.c0 = static_cast<const char*>(a.ent.c) + b * a.ent.rows * a.ent.ld_c;
  rb.r0 = static_cast<const char*>(a.ent.r) + b * a.ent.rows * a.ent.ld_r * 2;
  rb.s0 = reinterpret_cast<const char*>(a.ent.scale + b * a.ent.rows);
  rb.ldc0 = (uint32_t)a.ent.ld_c;
  rb.ldr0 = (uint32_t)(a.ent.ld_r * 2);
  const bool win = a.raw.c != nullptr;
  rb.c1 = win ? static_cast<const char*>(a.raw.c) + b * a.raw.rows * a.raw.ld_c : rb.c0;
  rb.r1 = win ? static_cast<const char*>(a.raw.r) + b * a.raw.rows * a.raw.ld_r * 2 : rb.r0;
  rb.s1 = win ? reinterpret_cast<const char*>(a.raw.scale + b * a.raw.rows) : rb.s0;
  rb.ldc1 = win ? (uint32_t)a.raw.ld_c : rb.ldc0;
  rb.ldr1 = win ? (uint32_t)(a.raw.ld_r * 2) : rb.ldr0;
  return rb;
}

struct KeyAddr8 {
  const char* lat;
  const char* rope;
  const char* scl;
};

__device__ __forceinline__ KeyAddr8 key_addr8(const RowBases8& rb, int code) {
  KeyAddr8 k;
  if (code < 0) {
    k.lat = k.rope = k.scl = reinterpret_cast<const char*>(kZeroRow);
  } else {
    const bool raw = code >> 30;
    const uint64_t row = (uint32_t)(code & 0x3fffffff);
    k.lat = (raw ? rb.c1 : rb.c0) + row * (raw ? rb.ldc1 : rb.ldc0);
    k.rope = (raw ? rb.r1 : rb.r0) + row * (raw ? rb.ldr1 : rb.ldr0);
    k.scl = (raw ? rb.s1 : rb.s0) + row * 4;
  }
  return k;
}

// This wave's share of the DMA of one tile into staging slot `st` (the prologue's form of what the
// QK block issues): latent row pairs j = w + 4 i (lanes 0-31 row j, 32-63 row j + 16), RoPE rows
// 8 w .. 8 w + 7, and the 32 row scales (every wave copies the same values).
__device__ __forceinline__ void dma_stage(const KeyAddr8* ad, char* st) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = w + 4 * i;
    const char* src = ad[j + 16 * (lane >> 5)].lat + 16 * (lane & 31);
    __builtin_amdgcn_global_load_lds(src, (lds_char*)(st + kStPair * j), 16, 0, 0);
  }
  {
    const char* src = ad[8 * w + (lane >> 3)].rope + 16 * (lane & 7);
    __builtin_amdgcn_global_load_lds(src, (lds_char*)(st + kStLat + 1024 * w), 16, 0, 0);
  }
  {
    const char* src = lane < kTK ? ad[lane].scl : reinterpret_cast<const char*>(kZeroRow);
    __builtin_amdgcn_global_load_lds(src, (lds_char*)(st + kStLat + kStRope), 4, 0, 0);
  }
}

// Converts staging slot `st` into the fp16 tile `kvb` (layout of attend_tile.h). Latent: wave w
// converts rows 8 w .. 8 w + 7, lane l row 8 w + (l & 7) and its 64-dim part p = l >> 3 (so the
// 8 lanes of one part write 8 different 16-byte bank groups). RoPE: lane l row 8 w + (l >> 3),
// dims 8 (l & 7) .. + 7.
__device__ __forceinline__ void convert_stage(const char* st, char* kvb) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = 8 * w + (lane & 7), p = lane >> 3;
  const int f = swz(r);
  const int rr = 8 * w + (lane >> 3), pr = lane & 7;
  // All six LDS reads in flight at once (one instruction block, so the waits cannot split them).
  // They read only the staging slot, which nothing but DMA writes; the waits and barriers around
  // the call order them, so no memory clobber constrains the interleave with the PV MFMAs.
  v4i lv[4], rv;
  int sb;
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:16\n\t"
      "ds_read_b128 %2, %6 offset:32\n\t"
      "ds_read_b128 %3, %6 offset:48\n\t"
      "ds_read_b128 %4, %7\n\t"
      "ds_read_b32 %5, %8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lv[0]), "=&v"(lv[1]), "=&v"(lv[2]), "=&v"(lv[3]), "=&v"(rv), "=&v"(sb)
      : "v"(lds_addr(st + kStPair * (r & 15) + 512 * (r >> 4) + 64 * p)),
        "v"(lds_addr(st + kStLat + rr * 128 + 16 * pr)),
        "v"(lds_addr(st + kStLat + kStRope + 4 * r)));
  const uint32_t sbits = (uint32_t)sb;
  const float pow2 = __uint_as_float(sbits & 0x7f800000u);                  // 2^e (0 for 0)
  const _Float16 mant = (_Float16)__uint_as_float((sbits & 0x007fffffu) | 0x3f800000u);
  const h2 mm = {mant, mant};
  char* row = kvb + r * 1024;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t wd = (uint32_t)lv[k][j];
      const h2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd, pow2, false) * mm;
      const h2 hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd, pow2, true) * mm;
      o[2 * j] = __builtin_bit_cast(uint32_t, lo);
      o[2 * j + 1] = __builtin_bit_cast(uint32_t, hi2);
    }
    const int c = 8 * p + 2 * k;   // 16-byte chunk of the fp16 row
    *reinterpret_cast<uint4*>(row + 16 * (c ^ f)) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(row + 16 * ((c + 1) ^ f)) = make_uint4(o[4], o[5], o[6], o[7]);
  }
  const f16x8 rh = bf16x8_to_f16((uint32_t)rv[0], (uint32_t)rv[1], (uint32_t)rv[2], (uint32_t)rv[3]);
  *reinterpret_cast<f16x8*>(kvb + kTK * 1024 + rr * 128 + 16 * (pr ^ swz(rr))) = rh;
}

// TOK: token selection (a.tok_m > 0). The entry form is compiled with the token fields known to
// be zero, so its per-tile key arithmetic has no branches. DENSE: hca_attend, whose keys are the
// visible entries in order (key kk is entry row kk): the rows' addresses and the tile masks follow
// from the key index, so the loop has no per-tile key codes and reads no row addresses from LDS.
template <bool TOK, bool DENSE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attend_fp8_kernel(AttendArgs a, AttnPlan plan) {
  constexpr int RG = 4;
  constexpr int R = 128;
  constexpr int kBufB = kTK * kRowB;
  constexpr int kPSteps = kTK / 16;
  // Two fp16 tiles, then the staging slots of cache rows; after the tile loop the whole region
  // stages the outputs.
  __shared__ __attribute__((aligned(1024))) char smem[2 * kBufB + kNst * kStB];
  char (*const kv)[kBufB] = reinterpret_cast<char (*)[kBufB]>(smem);
  char (*const stg)[kStB] = reinterpret_cast<char (*)[kStB]>(smem + 2 * kBufB);
  static_assert(4 * 32 * kStageLd<_Float16> <= 2 * kBufB + kNst * kStB, "fp16 output staging");
  static_assert(2 * 32 * kStageLd<float> <= 2 * kBufB + kNst * kStB, "fp32 output staging");
  __shared__ __attribute__((aligned(16))) char s_p[kPSteps * RG * 1024];
  __shared__ int s_code[kSlotsF8][kTK];
  __shared__ KeyAddr8 s_addr[kSlotsF8][kTK];
  __shared__ int s_has_key[kSlotsF8];
  __shared__ int s_full[kSlotsF8];
  __shared__ int s_sel[3][64];          // selection slots, copied three tiles before their codes
  __shared__ float s_ref[R];
  __shared__ float s_l[R];
  __shared__ int s_flag;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rg = w;                     // QK: row group
  const int hi = lane >> 5;
  const int per_q = plan.head_groups * plan.n_split;
  const int item = xcd_item();
  const int qi = item / per_q;
  const int rem = item - qi * per_q;
  const int hgrp = rem / plan.n_split;
  const int split = rem - hgrp * plan.n_split;
  const int hbase = hgrp * R;
  const int qrow_i = 32 * rg + (lane & 31);
  if (threadIdx.x == 0) s_flag = 0;

  // Prologue loads that wait for nothing. The selection slot of this lane's key in tiles
  // 0 .. kAheadF8 (tile w in wave w) is loaded at the key range a query with a full window
  // has, before the query's position is known (it is a dependent load); a query whose range
  // turns out different (an early position, in a key split past the first) loads it again below.
  // The queries' loads follow: issued before anything waits, and not waited for by the codes.
  const int64_t n_sel0 = TOK ? (int64_t)a.k * a.tok_m : (int64_t)a.k;
  int64_t k0_spec = 0;
  int raw_spec = 0;
  if (!a.dense) {
    const bool win = a.window > 0 && a.raw.c != nullptr && a.raw.rows > 0;
    const int64_t tot = n_sel0 + (win ? a.window : 0);
    k0_spec = (int64_t)split * ((tot + plan.n_split - 1) / plan.n_split);
    const int64_t kk = k0_spec + w * kTK + lane;
    if (lane < kTK && kk < n_sel0)
      raw_spec = a.idx[(int64_t)qi * a.k + (TOK ? kk / a.tok_m : kk)];
  }
  // Q^T fragments of this lane's head (dims 16 s + 8 hi + [0, 8)), loaded as bf16 now and
  // rounded to fp16 once the rows' DMA is out.
  uint4 qraw[kKSteps];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((int64_t)qi * a.H + hbase + qrow_i) * kD + 8 * hi;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qraw[s] = *reinterpret_cast<const uint4*>(qrow + 16 * s);
  }

  KeyList kl = make_key_list(a, qi);
  if constexpr (!TOK) kl.tok_m = 0;
  const int64_t per_split = (kl.total + plan.n_split - 1) / plan.n_split;
  const int64_t k0 = (int64_t)split * per_split;
  const int64_t ke = k0 + per_split < kl.total ? k0 + per_split : kl.total;
  const RowBases8 rbases = row_bases8(a, kl.b);

  const bool sel_dma = kl.sel != nullptr;
  const KeyCodes32 kc = key_codes32(kl, ke);

  // Codes of tiles 0 .. kAheadF8, so that the rows' DMA is issued while the queries are still in
  // flight. No LDS DMA goes out between the loads above and this use of the selection slot: the
  // compiler would then wait for every load outstanding, the queries included.
  int raw0 = raw_spec;
  if (sel_dma && k0 != k0_spec) {
    const int64_t kk = k0 + w * kTK + lane;
    raw0 = (lane < kTK && kk < kl.n_sel && kk < ke) ? kl.sel[sel_index(kl, kk)] : 0;
    asm volatile("" ::"v"(raw0));   // waited for here, so that only the early loads stay pending
  }
  const int c_pro = lane < kTK ? key_code32(kc, (int)(k0 + w * kTK + lane), raw0) : -1;
  if (lane < kTK) {
    s_code[w][lane] = c_pro;
    s_addr[w][lane] = key_addr8(rbases, c_pro);
  }
  if (w == 0 && sel_dma) {   // selection slots of tiles kAheadF8 + 1 and + 2
    dma_sel<kTK>(kl, k0 + (kAheadF8 + 1) * kTK, ke, s_sel[(kAheadF8 + 1) % 3]);
    dma_sel<kTK>(kl, k0 + (kAheadF8 + 2) * kTK, ke, s_sel[(kAheadF8 + 2) % 3]);
  }
  {
    const bool h = __any(c_pro >= 0);
    const bool f = __all(c_pro >= 0 || lane >= kTK);
    if (lane == 0) {
      s_has_key[w] = h;
      s_full[w] = f;
    }
  }
  lds_barrier();   // codes and row addresses of tiles 0 .. kAheadF8 (LDS only)
#pragma unroll
  for (int j = 0; j < kAheadF8; ++j) dma_stage(s_addr[j], stg[j]);
  v4i qb[kKSteps];
#pragma unroll
  for (int s = 0; s < kKSteps; ++s)
    qb[s] = __builtin_bit_cast(v4i, bf16x8_to_f16(qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w));
  floatx16 o[4][RG];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < RG; ++r) o[mt][r] = floatx16{};
  float m_ref = -INFINITY, l_run = 0.f;
  bool have_ref = false;
  const float cscale = a.sm_scale * kLog2e;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  convert_stage(stg[0], kv[0]);
  __syncthreads();

  int v_even, v_odd;   // PV addressing (as in the bf16 kernel)
  {
    const int g = lane >> 4, la = lane & 15;
    const int f = 2 * (la >> 2) + hi;
    const int c0 = 2 * (g & 1) + ((la & 3) >> 1);
    const int f2 = f >> 2;
    const int base = (4 * hi + (la >> 2)) * 1024 + 16 * (c0 ^ (f & 3)) + 8 * (la & 1) + 256 * w;
    v_even = base + 64 * f2;
    v_odd = base - 64 * f2;
  }

  // One tile: compute from `cbuf`, convert staging `cnext` into `nbuf` (the next tile), and stage
  // tile t + 3 into `sdst`. Restrict-qualified: none of these regions alias.
  auto tile = [&](const char* __restrict__ cbuf, char* __restrict__ nbuf,
                  const char* __restrict__ cnext, char* __restrict__ sdst,
                  char* __restrict__ pbuf, int64_t t0, int it) {
    const int slot = it % kSlotsF8;
    const int* codes = s_code[slot];
    TileDmaF8 dma;
    {
      const int64_t kk = t0 + (kAheadF8 + 3) * kTK + lane;
      dma.sel = (sel_dma && lane < kTK && kk < ke && kk < kl.n_sel)
                    ? reinterpret_cast<const char*>(kl.sel + sel_index(kl, kk))
                    : reinterpret_cast<const char*>(kZeroRow);
      if constexpr (DENSE) {
        // Entry rows of tile it + kAheadF8. A key past the list reads the list's last row instead
        // (finite values; its logit is masked to -inf, so it adds 0 to every sum).
        const int tb = (int)(t0 + kAheadF8 * kTK), last = (int)ke - 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = min(tb + (w + 4 * i) + 16 * (lane >> 5), last);
          dma.lat[i] = rbases.c0 + (uint64_t)(uint32_t)row * rbases.ldc0 + 16 * (lane & 31);
        }
        const int rrow = min(tb + 8 * w + (lane >> 3), last);
        dma.rope = rbases.r0 + (uint64_t)(uint32_t)rrow * rbases.ldr0 + 16 * (lane & 7);
        dma.scl = rbases.s0 + 4 * (uint64_t)(uint32_t)min(tb + (lane & (kTK - 1)), last);
      } else {
        const KeyAddr8* ad = s_addr[(it + kAheadF8) % kSlotsF8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dma.lat[i] = ad[(w + 4 * i) + 16 * (lane >> 5)].lat + 16 * (lane & 31);
        dma.rope = ad[8 * w + (lane >> 3)].rope + 16 * (lane & 7);
        dma.scl = lane < kTK ? ad[lane].scl : reinterpret_cast<const char*>(kZeroRow);
      }
      dma.m0_sel = __builtin_amdgcn_readfirstlane(
          lds_addr(reinterpret_cast<const char*>(s_sel[(it + kAheadF8 + 3) % 3])));
      dma.m0_lat = __builtin_amdgcn_readfirstlane(lds_addr(sdst) + kStPair * w);
      dma.m0_rope = __builtin_amdgcn_readfirstlane(lds_addr(sdst) + kStLat + 1024 * w);
      dma.m0_scl = __builtin_amdgcn_readfirstlane(lds_addr(sdst) + kStLat + kStRope);
    }

    // ---- QK (fp16): S^T = K . Q^T for row group rg over the tile's 32 keys.
    floatx16 acc;
    {
      const int r = lane & 31;
      const int f = swz(r);
      const int h16 = 16 * (hi ^ (f & 1));
      const int lat = lds_addr(cbuf) + r * 1024 + h16;
      const int rope = lds_addr(cbuf) + kTK * 1024 + r * 128 + h16;
      int lb[4], rb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lb[t] = lat + 32 * (t ^ (f >> 1));
        rb[t] = rope + 32 * (t ^ (f >> 1));
      }
      acc = qk_chain_f16(qb, lb, rb, dma);
    }

    if (DENSE ? t0 + kTK > ke : !s_full[slot]) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hi + (i & 3);
        const bool ok = DENSE ? t0 + key < ke : codes[key] >= 0;
        acc[i] = ok ? acc[i] : -INFINITY;
      }
    }
    // (A dense tile always holds a key: t0 < ke.)
    if (!have_ref && (DENSE || s_has_key[slot])) {   // uniform: every head sees the same keys
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, acc[i] * cscale);
      m_ref = fmaxf(tmax, __shfl_xor(tmax, 32));
      have_ref = true;
    }
    const float nm = have_ref ? -m_ref : 0.f;
    {
      f16x8 ph[2];
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], cscale, nm));
        ph[i >> 3][i & 7] = (_Float16)pv[i];
      }
      // The tile's 16 values summed as a tree (depth 4, not a chain of 16 dependent adds).
#pragma unroll
      for (int w2 = 8; w2 >= 1; w2 >>= 1)
#pragma unroll
        for (int i = 0; i < w2; ++i) pv[i] += pv[i + w2];
      l_run += pv[0];
#pragma unroll
      for (int s = 0; s < 2; ++s)
        *reinterpret_cast<f16x8*>(pbuf + ((s * RG + rg) * 64 + lane) * 16) = ph[s];
    }
    lds_barrier();   // P of the whole tile is in LDS

    // ---- PV (fp16) for the value dims [128 w, 128 w + 128) of all 128 heads, and the conversion
    // of the next tile (independent work the compiler can interleave with the MFMAs).
#pragma unroll
    for (int ks = 0; ks < kPSteps; ++ks) {
      v4i pall[4];
      load_p4(lds_addr(pbuf) + lane * 16 + 4096 * ks, pall);
      const int koff = ks * 16384;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const char* b0 = cbuf + ((mt & 1) ? v_odd : v_even) + 64 * mt + koff;
        const uint2 x0 = __builtin_bit_cast(
            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(const lds_char*)b0));
        const uint2 x1 = __builtin_bit_cast(
            uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                       (lds_short4*)(const lds_char*)(b0 + 8 * 1024)));
        const f16x8 vf = __builtin_bit_cast(f16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
#pragma unroll
        for (int r = 0; r < RG; ++r)
          o[mt][r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, __builtin_bit_cast(f16x8, pall[r]),
                                                            o[mt][r], 0, 0, 0);
      }
    }
    convert_stage(cnext, nbuf);

    // Selection slots for the codes below were copied two tiles ago; at most the DMA instructions
    // issued since (two tiles' worth) may still be outstanding.
    if (!DENSE) __builtin_amdgcn_s_waitcnt(kVmcntDma<2 * (kDmaOpsF8 + 1)>);
    if (!DENSE && threadIdx.x < 64) {
      const int kk2 = (int)t0 + (kAheadF8 + 1) * kTK + (int)threadIdx.x;
      const int raw2 = sel_dma ? s_sel[(it + kAheadF8 + 1) % 3][threadIdx.x] : 0;
      const int c2 = threadIdx.x < kTK ? key_code32(kc, kk2, raw2) : -1;
      const int slot2 = (it + kAheadF8 + 1) % kSlotsF8;
      if (threadIdx.x < kTK) {
        s_code[slot2][threadIdx.x] = c2;
        s_addr[slot2][threadIdx.x] = key_addr8(rbases, c2);
      }
      const bool h2 = __any(c2 >= 0);
      const bool f2 = __all(c2 >= 0 || threadIdx.x >= kTK);
      if (threadIdx.x == 0) {
        s_has_key[slot2] = h2;
        s_full[slot2] = f2;
      }
    }
    // The staging of tile t + 2 (issued in the previous tile) has landed once at most this tile's
    // DMA instructions are outstanding.
    __builtin_amdgcn_s_waitcnt(kVmcntDma<kDmaOpsF8 + 1>);
    lds_barrier();   // tile done, next tile converted, P buffer free
  };
  int it = 0;
  for (int64_t t0 = k0; t0 < ke; t0 += kTK, ++it)
    tile(kv[it & 1], kv[(it + 1) & 1], stg[(it + 1) % kNst], stg[(it + kAheadF8) % kNst], s_p, t0,
         it);
  __builtin_amdgcn_s_waitcnt(0);   // no DMA may land in LDS after the workgroup has finished

  l_run += __shfl_xor(l_run, 32);
  if (hi == 0) {
    s_l[qrow_i] = l_run;
    s_ref[qrow_i] = m_ref;
  }
  __syncthreads();   // (m, l) of every head; the tile and staging buffers are idle

  // Outputs (n_split == 1: o / l in fp32, two 32-head row groups per pass) or partials (o / l in
  // fp16, all 128 heads in one pass, and (m, l)), staged through LDS and written as whole rows.
  // A staged value that is not finite in its type (fp16 P overflowed, or a converted value did)
  // flags the workgroup for the fp32 recompute.
  bool bad = false;
  if (plan.n_split == 1) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int r = 2 * half + rr;
        const int hrow = 32 * r + (lane & 31);
        const float l = s_l[hrow];
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        stage_rows_checked<float>(o, r, inv, smem + rr * 32 * kStageLd<float>, bad);
        if (a.lse != nullptr && w == 0 && hi == 0)
          a.lse[(int64_t)qi * a.H + hbase + hrow] =
              l > 0.f ? (s_ref[hrow] + __log2f(l)) * 0.6931471805599453f : -INFINITY;
      }
      __syncthreads();
      flush_rows<float, 64>(smem, a.out + ((int64_t)qi * a.H + hbase + 64 * half) * kDC);
      __syncthreads();
    }
  } else {
    const int64_t row0 = ((int64_t)qi * plan.n_split + split) * a.H + hbase;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int hrow = 32 * r + (lane & 31);
      const float l = s_l[hrow];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      stage_rows_checked<_Float16>(o, r, inv, smem + r * 32 * kStageLd<_Float16>, bad);
      if (w == 0 && hi == 0) {
        plan.ws_ml[(row0 + hrow) * 2] = s_ref[hrow];
        plan.ws_ml[(row0 + hrow) * 2 + 1] = l;
      }
    }
    __syncthreads();
    flush_rows<_Float16, 128>(smem, plan.ws_o + row0 * kDC);
  }
  if (__any(bad)) atomicOr(&s_flag, 1);
  __syncthreads();
  if (threadIdx.x == 0) plan.flags[item] = s_flag;
}

}  // namespace

hipError_t launch_attend_fp8(const AttendArgs& a, const AttnPlan& p, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.Q.nq * p.head_groups * p.n_split);
  if (a.tok_m > 0)
    attend_fp8_kernel<true, false><<<grid, 256, 0, s>>>(a, p);
  else if (a.dense)
    attend_fp8_kernel<false, true><<<grid, 256, 0, s>>>(a, p);
  else
    attend_fp8_kernel<false, false><<<grid, 256, 0, s>>>(a, p);
  return hipGetLastError();
}

}  // namespace csa
