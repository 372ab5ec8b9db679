// MFMA attention for bf16 caches with 64 heads per workgroup (csa_attend / hca_attend; 512
// latent + 64 RoPE dims per row, bf16 queries, H a multiple of 64), with the work of each key
// tile split between two wave roles that share every SIMD.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA: selected compressed rows plus the
// raw window, MQA with one KV shared by every head; HCA: dense over the m'-compressed rows) and the
// MLA section (key row = [latent; RoPE key], value row = latent); yudonglee.me "DeepSeek-V4 详解"
// 2.2 Step 4 and 2.3 Step 2.
//
// A workgroup is 8 waves, 2 per SIMD, serving the 64 heads (two row groups of 32) of one query.
// Key rows reach LDS by DMA in tiles of 32 rows (the layout of attend_tile.h), four buffers deep.
// In iteration i:
//   QK waves 0-3 (row group w & 1, key half w >> 1) compute S^T[16 keys x 32 heads] = K . Q^T
//     for tile i with 36 mfma_f32_16x16x32_bf16 (Q^T of the row group in registers, its latent
//     part in accumulation registers), issue the DMA of tile i + 2 and the selection indices of
//     tile i + 5 from inside that instruction block, apply the softmax with the fixed per-head
//     reference, and write P (fp16) for the PV waves;
//   PV waves 4-7 (value dims [128 p, 128 p + 128), p = w - 4) accumulate
//     O^T[128 dims x 64 heads] += V^T . P^T for tile i - 1 with 16 mfma_f32_32x32x16_f16, the
//     P^T and the transposed V^T (ds_read_b64_tr_b16) of the next step read ahead of those
//     MFMAs, V^T converted to fp16 in registers; every PV wave also computes the key codes and
//     row addresses of tile i + 3 (the same values), in between.
// One barrier closes each iteration. Each SIMD holds one wave of each role, so while one runs its
// softmax, conversions or LDS traffic the other keeps the matrix unit busy. The prologue copies
// the 64 heads' queries once (loads written into the two buffers idle until the first tile) and
// the QK waves read their fragments from there.
//
// Numerics: bf16 products exact in fp32, V converted to fp16 (exact in fp16's normal range), P
// fp16, fixed reference maximum from the first tile that holds a key, and a non-finite output
// flags the workgroup for the fp32 fixup pass.
#include "attend_generic.h"
#include "attend_plan.h"
#include "attend_tile.h"

namespace csa {
namespace {

constexpr int kPpTK = 32;                   // keys per tile
constexpr int kPpBuf = 4;                   // tile buffers: PV (i-1), QK (i), DMA (i+1, i+2)
constexpr int kPpTileB = kPpTK * kRowB;     // 32 x (1024 + 128) bytes
constexpr int kPpRowOps = kPpTK / 4 + 1;    // row DMA instructions per QK wave and tile
constexpr int kPpR = 64;                    // heads per workgroup

// Transposed 64-bit LDS read (ds_read_b64_tr_b16) from a pointer into shared memory.
typedef short v4s16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s16 lds_v4s16;
__device__ __forceinline__ v2i lds_tr16(const char* p) {
  return __builtin_bit_cast(
      v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(lds_char*)const_cast<char*>(p)));
}

// key_code32 and key_addr as selects (no branches), so that the PV waves' code arithmetic can
// be scheduled among their MFMAs.
__device__ __forceinline__ int key_code_sel(const KeyCodes32& c, int kk, int raw) {
  if (c.tok_m > 0) return key_code32(c, kk, raw);   // token selection: the general form
  const int r = kk + c.woff;
  const int v = kk < c.n_sel ? (c.has_sel ? raw : kk) : ((r < c.wrap ? r : r - c.wrap) | (1 << 30));
  const bool empty = kk >= c.ke || raw < 0 || (kk < c.n_sel && c.has_sel && raw >= c.ent_rows);
  return empty ? -1 : v;
}

__device__ __forceinline__ KeyAddr key_addr_sel(const RowBases& rb, int code) {
  const bool raw = (code >> 30) & 1;
  const uint64_t row = (uint32_t)(code & 0x3fffffff);
  const char* lat = (raw ? rb.c1 : rb.c0) + row * (raw ? rb.ldc1 : rb.ldc0);
  const char* rope = (raw ? rb.r1 : rb.r0) + row * (raw ? rb.ldr1 : rb.ldr0);
  const char* z = reinterpret_cast<const char*>(kZeroRow);
  return KeyAddr{code < 0 ? z : lat, code < 0 ? z : rope};
}

// The DMA of one tile's rows (the layout of dma_tile in attend_tile.h), share wv of 4, from
// row addresses held in registers: lane l (and l + 32) holds those of key l.
__device__ __forceinline__ void dma_tile_regs(const KeyAddr& ka, char* buf, int wv) {
  const int lane = threadIdx.x & 63;
  const uint32_t off0 = 16 * (lane ^ swz(wv)), off1 = 16 * (lane ^ swz(wv + 4));
  const uint32_t lat_lo = (uint32_t)(uintptr_t)ka.lat, lat_hi = (uint32_t)((uintptr_t)ka.lat >> 32);
#pragma unroll
  for (int j = 0; j < kPpTK / 4; ++j) {
    const int r = 4 * j + wv;
    const uint64_t base = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lat_lo, r) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lat_hi, r) << 32);
    const char* src = reinterpret_cast<const char*>(base) + ((j & 1) ? off1 : off0);
    __builtin_amdgcn_global_load_lds(src, (lds_char*)(buf + 1024 * r), 16, 0, 0);
  }
  // RoPE rows 8 wv .. 8 wv + 7, eight lanes per row.
  const int r = 8 * wv + (lane >> 3);
  const uint32_t rp_lo = (uint32_t)__shfl((int)(uint32_t)(uintptr_t)ka.rope, r);
  const uint32_t rp_hi = (uint32_t)__shfl((int)(uint32_t)((uintptr_t)ka.rope >> 32), r);
  const char* src = reinterpret_cast<const char*>((uint64_t)rp_lo | ((uint64_t)rp_hi << 32)) +
                    16 * ((lane & 7) ^ swz(r));
  __builtin_amdgcn_global_load_lds(src, (lds_char*)(buf + kPpTK * 1024 + 1024 * wv), 16, 0, 0);
}

// Q^T fragments of a QK wave for mfma_f32_16x16x32_bf16 from LDS: q[2 s + h] = Q[head
// 16 h + (lane & 15)][dims 32 s + 8 (lane >> 4) + (0..7)] of the row group, where the
// workgroup's DMA has put fragment f of this row group at base + 1 KB f (lane l's 16 bytes at
// 16 l). One block that waits for its reads, the 32 latent fragments into accumulation registers
// (at most 15 reads outstanding).
__device__ __forceinline__ void load_q16_lds(int base, v4i (&q)[36]) {
  asm volatile(
      "ds_read_b128 %0, %32 offset:0\n"
      "ds_read_b128 %1, %32 offset:1024\n"
      "ds_read_b128 %2, %32 offset:2048\n"
      "ds_read_b128 %3, %32 offset:3072\n"
      "ds_read_b128 %4, %32 offset:4096\n"
      "ds_read_b128 %5, %32 offset:5120\n"
      "ds_read_b128 %6, %32 offset:6144\n"
      "ds_read_b128 %7, %32 offset:7168\n"
      "ds_read_b128 %8, %32 offset:8192\n"
      "ds_read_b128 %9, %32 offset:9216\n"
      "ds_read_b128 %10, %32 offset:10240\n"
      "ds_read_b128 %11, %32 offset:11264\n"
      "ds_read_b128 %12, %32 offset:12288\n"
      "ds_read_b128 %13, %32 offset:13312\n"
      "ds_read_b128 %14, %32 offset:14336\n"
      "s_waitcnt lgkmcnt(0)\n"
      "ds_read_b128 %15, %32 offset:15360\n"
      "ds_read_b128 %16, %32 offset:16384\n"
      "ds_read_b128 %17, %32 offset:17408\n"
      "ds_read_b128 %18, %32 offset:18432\n"
      "ds_read_b128 %19, %32 offset:19456\n"
      "ds_read_b128 %20, %32 offset:20480\n"
      "ds_read_b128 %21, %32 offset:21504\n"
      "ds_read_b128 %22, %32 offset:22528\n"
      "ds_read_b128 %23, %32 offset:23552\n"
      "ds_read_b128 %24, %32 offset:24576\n"
      "ds_read_b128 %25, %32 offset:25600\n"
      "ds_read_b128 %26, %32 offset:26624\n"
      "ds_read_b128 %27, %32 offset:27648\n"
      "ds_read_b128 %28, %32 offset:28672\n"
      "ds_read_b128 %29, %32 offset:29696\n"
      "s_waitcnt lgkmcnt(0)\n"
      "ds_read_b128 %30, %32 offset:30720\n"
      "ds_read_b128 %31, %32 offset:31744\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=a"(q[0]), "=a"(q[1]), "=a"(q[2]), "=a"(q[3]), "=a"(q[4]), "=a"(q[5]), "=a"(q[6]),
        "=a"(q[7]), "=a"(q[8]), "=a"(q[9]), "=a"(q[10]), "=a"(q[11]), "=a"(q[12]), "=a"(q[13]),
        "=a"(q[14]), "=a"(q[15]), "=a"(q[16]), "=a"(q[17]), "=a"(q[18]), "=a"(q[19]), "=a"(q[20]),
        "=a"(q[21]), "=a"(q[22]), "=a"(q[23]), "=a"(q[24]), "=a"(q[25]), "=a"(q[26]), "=a"(q[27]),
        "=a"(q[28]), "=a"(q[29]), "=a"(q[30]), "=a"(q[31])
      : "v"(base)
      : "memory");
}

// TOK: token selection (a.tok_m > 0). The entry form is compiled with the token fields known to
// be zero, so its per-tile key arithmetic has no branches and the compiler can place it among
// the MFMAs.
// DENSE: hca_attend, whose keys are the visible entries in order (key kk is entry row kk): the
// QK waves take the rows' addresses and the tile masks from the key index, and the PV waves compute
// no key codes after the prologue.
template <bool TOK, bool DENSE>
__global__ void __launch_bounds__(512) attend_pp_kernel(AttendArgs a, AttnPlan plan) {
  constexpr int TK = kPpTK;
  constexpr int R = kPpR;
  __shared__ __attribute__((aligned(1024))) char kv[kPpBuf][kPpTileB];
  __shared__ __attribute__((aligned(16))) char s_p[2][4 * 1024];   // P^T of tiles i, i + 1
  __shared__ int s_code[kPpBuf][TK];
  __shared__ KeyAddr s_addr[kPpBuf][TK];
  __shared__ int s_sel[3][64];          // selection slots of tiles i + 3 (read), i + 4, i + 5
  __shared__ float s_ref[2][R];         // per key half: maxima of the reference tile
  __shared__ float s_l[2][R];           // per key half: softmax sums
  __shared__ float s_m[R];              // reference maxima
  __shared__ int s_flag;
  __shared__ int s_last_sel;            // last selection slot that names an entry

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hi = lane >> 5;
  const int per_q = plan.head_groups * plan.n_split;
  const int item = xcd_item();
  const int qi = item / per_q;
  const int rem = item - qi * per_q;
  const int hgrp = rem / plan.n_split;
  const int split = rem - hgrp * plan.n_split;
  const int hbase = hgrp * R;
  if (threadIdx.x == 0) {
    s_flag = 0;
    s_last_sel = -1;
  }

  KeyList kl = make_key_list(a, qi);
  if constexpr (!TOK) kl.tok_m = 0;
  // Trailing selection slots that name no entry (-1, or a row past the entry store: a query that
  // sees fewer than k entries) contribute nothing; the key list ends after the last slot that
  // names one, so such queries skip those tiles. The slots are loaded (coalesced) before the
  // queries' DMA and reduced after it, so waiting for them does not wait for the queries.
  const bool trim = !TOK && kl.sel != nullptr;
  constexpr int kTrimPer = 4;   // slots per thread held in registers; more are read in a loop
  int sv[kTrimPer];
  if (trim) {
#pragma unroll
    for (int u = 0; u < kTrimPer; ++u) {
      const int j = (int)threadIdx.x + 512 * u;
      sv[u] = j < kl.n_sel ? kl.sel[j] : -1;
    }
  }
  // The PV waves' selection slots of tiles 0-2 (the first workgroup of a query, whose key range
  // starts at 0 whatever the trim finds), also loaded ahead of the queries' DMA: loads return in
  // order, so loaded after it they would wait for the whole 72 KB of queries before the codes and
  // the first rows' DMA could go out. Slots past the trimmed range are loaded but never used.
  const bool early_sel = trim && split == 0 && w >= 4;
  int raw_pre[3] = {0, 0, 0};
  if (early_sel) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int kk = j * TK + (lane & (TK - 1));
      raw_pre[j] = kk < kl.n_sel ? kl.sel[kk] : 0;
    }
  }
  asm volatile("" ::: "memory");   // keep those loads ahead of the DMA below

  // Prologue, in parallel: every wave copies its share of the queries (non-temporal loads: read
  // once, so that they do not displace key rows from the caches), while the PV
  // waves compute the codes of tiles 0-2, copy the selection slots of tiles 3 and 4 and issue the
  // DMA of tiles 0 and 1. The queries of the 64 heads go to tile buffers 2 and 3 (idle until the
  // first tile's block) in the QK waves' fragment order: fragment f of row group rg at
  // (36 rg + f) KB, lane l's 16 bytes at 16 l; each of the 8 waves copies 9 of the 72 fragments.
  // The copy is made of ordinary loads into registers, written to LDS once they land: the
  // compiler counts those loads exactly when it waits for the selection slots above, whereas any
  // LDS DMA issued after a load makes its wait for that load a wait for everything outstanding.
  v4i qld[9];
  {
    const int c = lane & 15, g = lane >> 4;
    const char* qblk = static_cast<const char*>(a.q) + ((int64_t)qi * a.H + hbase) * kD * 2;
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int F = 9 * w + i;
      const int rgF = F / 36, f = F - 36 * rgF;
      const char* src = qblk + ((32 * rgF + 16 * (f & 1) + c) * kD + 32 * (f >> 1) + 8 * g) * 2;
      qld[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src));
    }
  }
  auto store_queries = [&]() {
#pragma unroll
    for (int i = 0; i < 9; ++i)
      *reinterpret_cast<v4i*>(&kv[2][0] + 1024 * (9 * w + i) + 16 * lane) = qld[i];
  };

  if (trim) {
    int last = -1;
#pragma unroll
    for (int u = 0; u < kTrimPer; ++u) {
      const int j = (int)threadIdx.x + 512 * u;
      last = sv[u] >= 0 && sv[u] < kl.ent_rows ? j : last;
    }
    for (int j = (int)threadIdx.x + 512 * kTrimPer; j < kl.n_sel; j += 512) {
      const int v = kl.sel[j];
      last = v >= 0 && v < kl.ent_rows ? j : last;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
    lds_barrier();   // s_last_sel initialised
    if (lane == 0) atomicMax(&s_last_sel, last);
    lds_barrier();
    kl.n_sel = s_last_sel + 1;
    kl.total = kl.n_sel + kl.n_win;
  }
  const int64_t per_split = (kl.total + plan.n_split - 1) / plan.n_split;
  const int64_t k0 = (int64_t)split * per_split;
  const int64_t ke = k0 + per_split < kl.total ? k0 + per_split : kl.total;
  const RowBases rbases = row_bases(a, kl.b);
  const bool sel_dma = kl.sel != nullptr;   // CSA: selection slots come from idx
  const KeyCodes32 kc = key_codes32(kl, ke);
  const int nt = ke > k0 ? (int)((ke - k0 + TK - 1) / TK) : 0;
  const float cscale = a.sm_scale * kLog2e;

  if (w < 4) {
    // ================================ QK waves ================================
    const int rg = w & 1, kh = w >> 1;
    const int c = lane & 15, g = lane >> 4;
    v4i qb[36];
    store_queries();                  // this wave's share of the queries
    __syncthreads();                  // all queries and the prologue's tiles in LDS
    {
      const char* qf = &kv[2][0] + 36 * 1024 * rg + 16 * lane;
      load_q16_lds(lds_addr(qf), qb);
#pragma unroll
      for (int f = 32; f < 36; ++f) qb[f] = *reinterpret_cast<const v4i*>(qf + 1024 * f);
    }
    __syncthreads();                  // queries read: buffers 2 and 3 free for the tile DMA
    float m_ref[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};
    bool have_ref = false;
    // K fragment of key row 16 kh + c: chunk 4 s + g (latent k-step s) sits at (4 s + g) ^ f.
    const int r = 16 * kh + c;
    const int f = swz(r);
    const int oe = 16 * (g ^ f), oo = 16 * ((4 | g) ^ f);
    const int lat_off = r * 1024, rope_off = TK * 1024 + r * 128;

    auto tile = [&](const char* __restrict__ cbuf, char* __restrict__ nbuf,
                    char* __restrict__ pbuf, int i) {
      const int64_t t0 = k0 + (int64_t)i * TK;
      const int slot = i % kPpBuf;
      TileDma<TK / 4, TK / 32> dma;
      {
        const int64_t kk = t0 + 5 * TK + lane;
        dma.sel = (sel_dma && lane < TK && kk < ke && kk < kl.n_sel)
                      ? reinterpret_cast<const char*>(kl.sel + sel_index(kl, kk))
                      : reinterpret_cast<const char*>(kZeroRow);
        dma.off[0] = 16 * (lane ^ swz(w));
        dma.off[1] = 16 * (lane ^ swz(w + 4));
        const int rr = 8 * w + (lane >> 3);
        if constexpr (DENSE) {
          // Entry rows of tile i + 2. A key past the list reads the list's last row instead
          // (finite values; its logit is masked to -inf, so it adds 0 to every sum).
          const int tb = (int)(t0 + 2 * TK), last = (int)ke - 1;
          const int wu = __builtin_amdgcn_readfirstlane(w);   // wave-uniform: scalar addresses
#pragma unroll
          for (int j = 0; j < TK / 4; ++j)
            dma.lat[j] = rbases.c0 + (uint64_t)(uint32_t)min(tb + 4 * j + wu, last) * rbases.ldc0;
          dma.rope[0] = rbases.r0 + (uint64_t)(uint32_t)min(tb + rr, last) * rbases.ldr0 +
                        16 * ((lane & 7) ^ swz(rr));
        } else {
          const KeyAddr* ad = s_addr[(i + 2) % kPpBuf];
          const char* mine = lane < TK / 4 ? ad[4 * lane + w].lat : nullptr;
#pragma unroll
          for (int j = 0; j < TK / 4; ++j) {
            const uint64_t base =
                ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(uintptr_t)mine, j)) |
                ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                     (int)(uint32_t)((uintptr_t)mine >> 32), j)
                 << 32);
            dma.lat[j] = reinterpret_cast<const char*>(base);
          }
          dma.rope[0] = ad[rr].rope + 16 * ((lane & 7) ^ swz(rr));
        }
        dma.m0_rows = __builtin_amdgcn_readfirstlane(lds_addr(nbuf) + 1024 * w);
        dma.m0_sel = __builtin_amdgcn_readfirstlane(
            lds_addr(reinterpret_cast<const char*>(s_sel[(i + 5) % 3])));
      }
      // Whether the tile holds a key / only keys (uniform), from its 32 codes.
      const int code_l = DENSE ? (t0 + (lane & (TK - 1)) < ke ? 0 : -1) : s_code[slot][lane & (TK - 1)];
      floatx4 acc[2];
      const int cb = lds_addr(cbuf);
      qk16_chain(qb, cb + lat_off + oe, cb + lat_off + oo, cb + rope_off + oe, cb + rope_off + oo,
                 dma, acc[0], acc[1]);
      // acc[h][j]: key 16 kh + 4 g + j, head 32 rg + 16 h + c.
      const bool has_key = __any(code_l >= 0);
      if (!__all(code_l >= 0)) {
        const int* codes = s_code[slot];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = DENSE ? t0 + 16 * kh + 4 * g + j < ke : codes[16 * kh + 4 * g + j] >= 0;
          acc[0][j] = ok ? acc[0][j] : -INFINITY;
          acc[1][j] = ok ? acc[1][j] : -INFINITY;
        }
      }
      if (!have_ref && has_key) {   // uniform over the workgroup (the PV waves match it)
        float tm[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float t = fmaxf(fmaxf(acc[h][0], acc[h][1]), fmaxf(acc[h][2], acc[h][3])) * cscale;
          t = fmaxf(t, __shfl_xor(t, 16));
          t = fmaxf(t, __shfl_xor(t, 32));
          tm[h] = t;
        }
        if (g == 0) {
          s_ref[kh][32 * rg + c] = tm[0];
          s_ref[kh][32 * rg + 16 + c] = tm[1];
        }
        lds_barrier();
#pragma unroll
        for (int h = 0; h < 2; ++h)
          m_ref[h] = fmaxf(s_ref[0][32 * rg + 16 * h + c], s_ref[1][32 * rg + 16 * h + c]);
        have_ref = true;
      }
      // Logits more than 2^16 above the reference overflow P's fp16 and reach O as inf/NaN, which
      // the final check flags. Before the reference (empty tiles) every logit is -inf: P = 0.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float nm = have_ref ? -m_ref[h] : 0.f;
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        h4 ph;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[h][j], cscale, nm));
          l_run[h] += p;
          ph[j] = (_Float16)p;
        }
        // P^T fragment (row group rg, k-step kh) of the PV MFMA: lane L = head (16 h + c) +
        // 32 (g & 1) holds keys 4 (g & 1) + (0..3) then 8 + 4 (g & 1) + (0..3).
        const int L = 16 * h + c + 32 * (g & 1);
        *reinterpret_cast<h4*>(pbuf + ((2 * kh + rg) * 64 + L) * 16 + 8 * (g >> 1)) = ph;
      }
      // Everything this wave issued before this tile's block (tile i + 1, the selection slots of
      // tile i + 4) has landed once at most the block's own DMA is outstanding.
      __builtin_amdgcn_s_waitcnt(kVmcntDma<kPpRowOps + 1>);
    };
    for (int i = 0; i <= nt; ++i) {
      if (i < nt) tile(kv[i % kPpBuf], kv[(i + 2) % kPpBuf], s_p[i & 1], i);
      lds_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);   // no DMA may land in LDS after the workgroup has finished
    // Softmax sums of this wave's keys per head (lanes 16 g + c share head c).
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float l = l_run[h];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      if (g == 0) {
        s_l[kh][32 * rg + 16 * h + c] = l;
        if (kh == 0) s_m[32 * rg + 16 * h + c] = m_ref[h];
      }
    }
    lds_barrier();                    // sums and maxima in LDS (epilogue barrier 1)
    // The PV waves stage and write the outputs in two row groups, two barriers each.
#pragma unroll
    for (int j = 0; j < 4; ++j) lds_barrier();
  } else {
    // ================================ PV waves ================================
    // Prologue, PV side: every PV wave computes the codes and row addresses of tiles 0-2 (the
    // three selection loads issued together) and stores them (the same values from every wave),
    // then issues its quarter of the DMA of tiles 0 and 1 from those registers; wave 4 also copies
    // the selection slots of tiles 3 and 4.
    {
      const int kl32 = lane & (TK - 1);
      int raw[3];
      if (early_sel) {   // as below: a key past the (trimmed) selection reads a zero
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int kk = (int)k0 + j * TK + kl32;
          raw[j] = kk < kc.ke && kk < kc.n_sel ? raw_pre[j] : 0;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int kk = (int)k0 + j * TK + kl32;
          const int32_t* src = (sel_dma && kk < kc.ke && kk < kc.n_sel)
                                   ? kl.sel + sel_index(kl, kk)
                                   : reinterpret_cast<const int32_t*>(kZeroRow);
          raw[j] = *src;
        }
        // Waited for here, inside this branch, so that after it only the early loads are
        // pending and the wait for them need not include the queries' loads.
        asm volatile("" ::"v"(raw[0]), "v"(raw[1]), "v"(raw[2]));
      }
      KeyAddr ad[2];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int c = key_code_sel(kc, (int)k0 + j * TK + kl32, raw[j]);
        const KeyAddr ka = key_addr_sel(rbases, c);
        s_code[j][kl32] = c;
        s_addr[j][kl32] = ka;
        if (j < 2) ad[j] = ka;
      }
      if (w == 4 && sel_dma) {
        dma_sel<TK>(kl, k0 + 3 * TK, ke, s_sel[0]);
        dma_sel<TK>(kl, k0 + 4 * TK, ke, s_sel[1]);
      }
      dma_tile_regs(ad[0], kv[0], w - 4);
      dma_tile_regs(ad[1], kv[1], w - 4);
      store_queries();
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    __syncthreads();                  // the QK waves have read their queries
    const int p = w - 4;
    floatx16 o[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt][0] = o[mt][1] = floatx16{};
    bool have_ref = false;
    int v_even, v_odd;   // V^T fragment addressing in the swizzled tile layout (attend_tile.h)
    {
      const int g = lane >> 4, la = lane & 15;
      const int f = 2 * (la >> 2) + hi;
      const int c0 = 2 * (g & 1) + ((la & 3) >> 1);
      const int f2 = f >> 2;
      const int base = (4 * hi + (la >> 2)) * 1024 + 16 * (c0 ^ (f & 3)) + 8 * (la & 1) + 256 * p;
      v_even = base + 64 * f2;
      v_odd = base - 64 * f2;
    }
    // V^T of a tile (16 half-fragments: k-step ks, dim tile mt, rows +0 / +8) and the P^T
    // fragments of the tile before it are read at the start of an iteration, ahead of that
    // iteration's MFMAs (which use the V^T read one iteration earlier), so the reads overlap the
    // matrix work.
    auto read_v = [&](const char* buf, v2i (&vr)[16]) {
      const char* be = buf + v_even;
      const char* bo = buf + v_odd;
      vr[0] = lds_tr16(be);
      vr[1] = lds_tr16(be + 8192);
      vr[2] = lds_tr16(bo + 64);
      vr[3] = lds_tr16(bo + 8256);
      vr[4] = lds_tr16(be + 128);
      vr[5] = lds_tr16(be + 8320);
      vr[6] = lds_tr16(bo + 192);
      vr[7] = lds_tr16(bo + 8384);
      vr[8] = lds_tr16(be + 16384);
      vr[9] = lds_tr16(be + 24576);
      vr[10] = lds_tr16(bo + 16448);
      vr[11] = lds_tr16(bo + 24640);
      vr[12] = lds_tr16(be + 16512);
      vr[13] = lds_tr16(be + 24704);
      vr[14] = lds_tr16(bo + 16576);
      vr[15] = lds_tr16(bo + 24768);
    };
    auto read_p = [&](const char* pbuf, v4i (&pf)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j) pf[j] = *reinterpret_cast<const v4i*>(pbuf + 1024 * j + 16 * lane);
    };
    // O^T += V^T . P^T for one tile: V^T already in fp16 (vh), P^T fragments in pf.
    auto pv = [&](const f16x8 (&vh)[8], const v4i (&pf)[4]) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int rg = 0; rg < 2; ++rg)
            o[mt][rg] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                vh[4 * ks + mt], __builtin_bit_cast(f16x8, pf[2 * ks + rg]), o[mt][rg], 0, 0, 0);
    };
    // Codes and row addresses of tile i + 3 from its selection slots (copied during iteration
    // i - 2). Every PV wave computes them (lanes l and l + 32 alike) and stores the same values,
    // so the stores need no branch and the arithmetic can interleave with the MFMAs.
    const int kl32 = lane & (TK - 1);
    auto codes = [&](int i, int raw) {
      const int kk = (int)k0 + (i + 3) * TK + kl32;
      const int c2 = key_code_sel(kc, kk, sel_dma ? raw : 0);
      const int slot2 = (i + 3) % kPpBuf;
      s_code[slot2][kl32] = c2;
      s_addr[slot2][kl32] = key_addr_sel(rbases, c2);
    };
    // Iteration i: PV of tile i - 1 (its V^T converted at the end of iteration i - 1), while the
    // V^T of tile i and the codes of tile i + 3 are fetched. The first iteration's PV adds zero;
    // the last iteration's reads and codes (of tiles past the end) go unused.
    f16x8 vh[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vh[j] = f16x8{};
    for (int i = 0; i <= nt; ++i) {
      if (i < nt && !have_ref) {   // the QK waves' reference barrier, at the first tile with a key
        if (DENSE || __any(s_code[i % kPpBuf][kl32] >= 0)) {
          lds_barrier();
          have_ref = true;
        }
      }
      const int raw = DENSE ? 0 : s_sel[(i + 3) % 3][kl32];   // issued first: waited for by count
      v4i pf[4];
      read_p(s_p[(i + 1) & 1], pf);
      v2i vr[16];
      read_v(kv[i % kPpBuf], vr);
      if (!DENSE) codes(i, raw);
      const bool first = i == 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) pf[j] = first ? v4i{} : pf[j];
      pv(vh, pf);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const v2i* x = &vr[2 * j];
        vh[j] = bf16x8_to_f16((uint32_t)x[0][0], (uint32_t)x[0][1], (uint32_t)x[1][0],
                              (uint32_t)x[1][1]);
      }
      lds_barrier();
    }
    lds_barrier();                    // epilogue barrier 1: sums and maxima complete
    // Outputs (n_split == 1: o / l in fp32) or partials (o / l in fp16, and (m, l)), one 32-head
    // row group at a time, staged in the (idle) tile buffers by the PV waves, written as rows. A
    // staged value that is not finite in its type (fp16 P overflowed) flags the workgroup for the
    // fp32 recompute; the flag is complete after the last barrier.
    bool bad = false;
    char* stage = &kv[0][0];
    const int pt = threadIdx.x - 256;   // 0 .. 255 over the PV waves
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int hrow = 32 * rg + (lane & 31);
      const float l = s_l[0][hrow] + s_l[1][hrow];
      const float m = s_m[hrow];
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      const int head = hbase + hrow;
      const int64_t row0 = plan.n_split == 1
                               ? (int64_t)qi * a.H + hbase + 32 * rg
                               : ((int64_t)qi * plan.n_split + split) * a.H + hbase + 32 * rg;
      if (plan.n_split == 1) {
        char* row = stage + (lane & 31) * kStageLd<float> + (128 * p + 4 * hi) * 4;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              x[u] = o[mt][rg][4 * j + u] * inv;
              bad |= !(__builtin_fabsf(x[u]) <= 3.4028235e38f);
            }
            *reinterpret_cast<float4*>(row + (32 * mt + 8 * j) * 4) =
                make_float4(x[0], x[1], x[2], x[3]);
          }
        if (a.lse != nullptr && p == 0 && hi == 0)
          a.lse[(int64_t)qi * a.H + head] =
              l > 0.f ? (m + __log2f(l)) * 0.6931471805599453f : -INFINITY;
      } else {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        char* row = stage + (lane & 31) * kStageLd<_Float16> + (128 * p + 4 * hi) * 2;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              x[u] = o[mt][rg][4 * j + u] * inv;
              bad |= !(__builtin_fabsf(x[u]) <= 65504.f);
            }
            *reinterpret_cast<h4*>(row + (32 * mt + 8 * j) * 2) =
                h4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
          }
        if (p == 0 && hi == 0) {
          const int64_t pidx = row0 + (lane & 31);
          plan.ws_ml[pidx * 2] = m;
          plan.ws_ml[pidx * 2 + 1] = l;
        }
      }
      if (rg == 1 && __any(bad)) atomicOr(&s_flag, 1);
      lds_barrier();                  // rows staged (the QK waves take part in every barrier)
      if (plan.n_split == 1) {
        // 16-byte chunk k of head row h: thread pt takes k = pt & 127 of rows pt / 128 + 2 u.
        constexpr int kCh = 512 * 4 / 16;
        constexpr int kU = 32 * kCh / 256;
        const int k = pt & (kCh - 1), h0 = pt / kCh;
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
          v[u] = *reinterpret_cast<const uint4*>(stage + (h0 + 2 * u) * kStageLd<float> + 16 * k);
#pragma unroll
        for (int u = 0; u < kU; ++u)   // final outputs: non-temporal stores
          store_nt(reinterpret_cast<char*>(a.out + (row0 + h0 + 2 * u) * kDC) + 16 * k, v[u]);
      } else {
        constexpr int kCh = 512 * 2 / 16;
        constexpr int kU = 32 * kCh / 256;
        const int k = pt & (kCh - 1), h0 = pt / kCh;
        uint4 v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
          v[u] = *reinterpret_cast<const uint4*>(stage + (h0 + 4 * u) * kStageLd<_Float16> + 16 * k);
#pragma unroll
        for (int u = 0; u < kU; ++u)
          *reinterpret_cast<uint4*>(reinterpret_cast<char*>(plan.ws_o + (row0 + h0 + 4 * u) * kDC) +
                                    16 * k) = v[u];
      }
      lds_barrier();                  // rows written, staging area free
    }
    if (threadIdx.x == 256) plan.flags[item] = s_flag;
  }
}

}  // namespace

hipError_t launch_attend_pp(const AttendArgs& a, const AttnPlan& p, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.Q.nq * p.head_groups * p.n_split);
  if (a.tok_m > 0)
    attend_pp_kernel<true, false><<<grid, 512, 0, s>>>(a, p);
  else if (a.dense)
    attend_pp_kernel<false, true><<<grid, 512, 0, s>>>(a, p);
  else
    attend_pp_kernel<false, false><<<grid, 512, 0, s>>>(a, p);
  return hipGetLastError();
}

}  // namespace csa
