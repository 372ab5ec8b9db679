// Building blocks shared by the MFMA attention kernels that stage key tiles in LDS by DMA
// (attend_pp.hip, attend_fp8.hip): tile layout helpers, key codes, the barrier and wait
// encodings, P^T exchange reads and the generated QK instruction blocks.
//
// LDS tile layout: rows stay unpadded, split into a latent region ([rows][1024 B]) and a RoPE
// region ([rows][128 B]) of 16-bit values. 16-byte chunk c of row r sits at chunk position
// c ^ f(r), f(r) = 2 (r & 3) + (r >> 2 & 1), which keeps the K-fragment reads (8 consecutive rows,
// one chunk) and the transposed V reads (4 consecutive rows, 2 adjacent chunks) free of bank
// conflicts.
#pragma once

#include "attend_keys.h"
#include "csa_internal.h"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kD = kDC + kDR;
constexpr int kRowB = kD * 2;            // 1152 bytes per staged row
constexpr int kKSteps = kD / 16;         // QK k-steps
constexpr float kLog2e = 1.4426950408889634f;

// Source of empty key slots: one zero row, so any lane offset within a row stays inside it.
__device__ const uint4 kZeroRow[kRowB / 16] = {};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding global loads (a __syncthreads() fence would also wait for the DMA of the next
// tile, which must stay in flight across the barrier).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt immediate that waits until at most N vector memory operations are outstanding and
// leaves the other counters unconstrained (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8).
template <int N>
constexpr int kVmcntDma = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);

// Byte address in LDS of a pointer into a __shared__ array.
__device__ __forceinline__ int lds_addr(const char* p) {
  return (int)(uintptr_t)(const lds_char*)p;
}

// 8 bf16 values (4 words, low half first) -> 8 fp16 values, round to nearest even (exact for
// values in fp16's normal range; larger magnitudes become infinite and are caught downstream).
__device__ __forceinline__ f16x8 bf16x8_to_f16(uint32_t w0, uint32_t w1, uint32_t w2,
                                               uint32_t w3) {
  const uint32_t w[4] = {w0, w1, w2, w3};
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = (_Float16)__uint_as_float(w[j] << 16);
    r[2 * j + 1] = (_Float16)__uint_as_float(w[j] & 0xffff0000u);
  }
  return r;
}

__device__ __forceinline__ int key_code(const AttendArgs& a, const KeyList& kl, int64_t kk,
                                        int64_t ke) {
  if (kk >= ke) return -1;
  int src;
  const int64_t row = key_row(a, kl, kk, src);
  return row >= 0 ? (int)row | (src << 30) : -1;
}

// Selection slots of one tile (TK keys from kk0) copied by DMA into LDS (wave 0, lane j ->
// dst[j]); keys outside the selection read a zero instead. Copying by DMA keeps the loop free of
// register loads, so its waits can be exact counts of DMA instructions.
template <int TK>
__device__ __forceinline__ void dma_sel(const KeyList& kl, int64_t kk0, int64_t ke, int* dst) {
  const int lane = threadIdx.x & 63;
  const int64_t kk = kk0 + lane;
  const void* src = (lane < TK && kk < ke && kk < kl.n_sel) ? (const void*)(kl.sel + sel_index(kl, kk))
                                                           : (const void*)kZeroRow;
  __builtin_amdgcn_global_load_lds(src, (lds_char*)dst, 4, 0, 0);
}

// Output rows through LDS. The accumulators hold O^T in the MFMA layout (lane: one head, 4-dim
// pieces of 32 rows at once), so stores straight from registers would write 32 rows x 16 bytes per
// instruction. Instead each wave stages its 128 dims of 32 heads (row group r of o[mt][r], scaled
// by the lane's inv) as rows of 512 values of T, and the workgroup then writes whole rows, 16
// bytes per lane. kStageLd: LDS row stride (16 bytes of padding spread the staging writes over the banks).
template <typename T>
constexpr int kStageLd = 512 * (int)sizeof(T) + 16;

template <typename T, int RG>
__device__ __forceinline__ void stage_rows(const floatx16 (&o)[4][RG], int r, float inv, char* buf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hi = lane >> 5;
  char* row = buf + (lane & 31) * kStageLd<T> + (128 * w + 4 * hi) * (int)sizeof(T);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      typedef T t4 __attribute__((ext_vector_type(4)));
      const t4 v = {(T)(o[mt][r][4 * j] * inv), (T)(o[mt][r][4 * j + 1] * inv),
                    (T)(o[mt][r][4 * j + 2] * inv), (T)(o[mt][r][4 * j + 3] * inv)};
      *reinterpret_cast<t4*>(row + (32 * mt + 8 * j) * (int)sizeof(T)) = v;
    }
}

// stage_rows that also tells whether any staged value is not a finite value of T: each scaled
// value is compared with T's largest finite magnitude (a NaN fails the comparison), so an
// accumulator that overflowed, and a finite value that T cannot hold, both set `bad`.
template <typename T, int RG>
__device__ __forceinline__ void stage_rows_checked(const floatx16 (&o)[4][RG], int r, float inv,
                                                   char* buf, bool& bad) {
  constexpr float kMax = sizeof(T) == 2 ? 65504.f : 3.4028235e38f;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, hi = lane >> 5;
  char* row = buf + (lane & 31) * kStageLd<T> + (128 * w + 4 * hi) * (int)sizeof(T);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      typedef T t4 __attribute__((ext_vector_type(4)));
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        x[u] = o[mt][r][4 * j + u] * inv;
        bad |= !(__builtin_fabsf(x[u]) <= kMax);
      }
      const t4 v = {(T)x[0], (T)x[1], (T)x[2], (T)x[3]};
      *reinterpret_cast<t4*>(row + (32 * mt + 8 * j) * (int)sizeof(T)) = v;
    }
}

// Cache policy of a DMA (global_load_lds) whose rows are read once: non-temporal.
constexpr int kNonTemporal = 2;

// 16-byte store of data written once (final outputs): non-temporal, so that it does not displace
// the key rows that later workgroups read from the caches.
__device__ __forceinline__ void store_nt(char* dst, uint4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
}

// Writes ROWS staged rows: row h to dst + h * 512 (consecutive heads are consecutive rows).
template <typename T, int ROWS = 32>
__device__ __forceinline__ void flush_rows(const char* buf, T* dst) {
  constexpr int kChunksRow = 512 * (int)sizeof(T) / 16;
  static_assert(ROWS * kChunksRow % 256 == 0, "whole passes of 256 threads");
#pragma unroll
  for (int i = 0; i < ROWS * kChunksRow / 256; ++i) {
    const int c = (int)threadIdx.x + 256 * i;
    const int h = c / kChunksRow, k = c - h * kChunksRow;
    const uint4 v = *reinterpret_cast<const uint4*>(buf + h * kStageLd<T> + 16 * k);
    char* d = reinterpret_cast<char*>(dst + (int64_t)h * 512) + 16 * k;
    if constexpr (sizeof(T) == 4)
      store_nt(d, v);   // fp32: final outputs, written once
    else
      *reinterpret_cast<uint4*>(d) = v;   // fp16 partials: read back by the merge
  }
}

// ---- bf16 caches: row addressing and the prologue's tile DMA ----------------------------------

// Row addressing of the two stores for one sequence, computed once per workgroup (kept as plain
// scalars: a runtime-indexed array would live in scratch memory).
struct RowBases {
  const char* c0;          // latent rows of sequence b in the entry store
  const char* c1;          // ... in the raw window store
  const char* r0;          // RoPE rows, entry store
  const char* r1;          // RoPE rows, raw window store
  uint32_t ldc0, ldc1, ldr0, ldr1;   // row strides in bytes
};

__device__ __forceinline__ RowBases row_bases(const AttendArgs& a, int64_t b) {
  RowBases rb;
  rb.c0 = static_cast<const char*>(a.ent.c) + b * a.ent.rows * a.ent.ld_c * 2;
  rb.r0 = static_cast<const char*>(a.ent.r) + b * a.ent.rows * a.ent.ld_r * 2;
  rb.ldc0 = (uint32_t)(a.ent.ld_c * 2);
  rb.ldr0 = (uint32_t)(a.ent.ld_r * 2);
  const bool win = a.raw.c != nullptr;
  rb.c1 = win ? static_cast<const char*>(a.raw.c) + b * a.raw.rows * a.raw.ld_c * 2 : rb.c0;
  rb.r1 = win ? static_cast<const char*>(a.raw.r) + b * a.raw.rows * a.raw.ld_r * 2 : rb.r0;
  rb.ldc1 = win ? (uint32_t)(a.raw.ld_c * 2) : rb.ldc0;
  rb.ldr1 = win ? (uint32_t)(a.raw.ld_r * 2) : rb.ldr0;
  return rb;
}

// Global addresses of one key's latent and RoPE parts (a zero row for an empty slot).
struct KeyAddr {
  const char* lat;
  const char* rope;
};

__device__ __forceinline__ KeyAddr key_addr(const RowBases& rb, int code) {
  KeyAddr k;
  if (code < 0) {
    k.lat = k.rope = reinterpret_cast<const char*>(kZeroRow);
  } else {
    const bool raw = code >> 30;
    const uint64_t row = (uint32_t)(code & 0x3fffffff);
    k.lat = (raw ? rb.c1 : rb.c0) + row * (raw ? rb.ldc1 : rb.ldc0);
    k.rope = (raw ? rb.r1 : rb.r0) + row * (raw ? rb.ldr1 : rb.ldr0);
  }
  return k;
}

// Issue the DMA of one tile (TK rows) into buf = [latent region TK x 1024 B][RoPE region TK x 128 B].
// addr[r] holds the global addresses of row r. Latent: one instruction per row (wave w takes rows
// w, w + 4, ...): the row address is a scalar base and lane l adds 16 (l ^ f(row)). RoPE: one
// instruction per 8 rows, lane l fetching row 8 j + l / 8, chunk (l & 7) ^ f(row).
template <int TK>
__device__ __forceinline__ void dma_tile(const KeyAddr* addr, char* buf, int w = threadIdx.x >> 6) {
  const int lane = threadIdx.x & 63;
  // Lane j holds the latent address of row 4 j + w; rows of one wave have f(row) in {f(w), f(w + 4)}.
  const char* mine = lane < TK / 4 ? addr[4 * lane + w].lat : nullptr;
  const uint32_t off0 = 16 * (lane ^ swz(w)), off1 = 16 * (lane ^ swz(w + 4));
#pragma unroll
  for (int j = 0; j < TK / 4; ++j) {
    const int r = 4 * j + w;
    const uint64_t base = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                               (int)(uint32_t)(uintptr_t)mine, j)) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(
                               (int)(uint32_t)((uintptr_t)mine >> 32), j) << 32);
    const char* src = reinterpret_cast<const char*>(base) + ((j & 1) ? off1 : off0);
    __builtin_amdgcn_global_load_lds(src, (lds_char*)(buf + 1024 * r), 16, 0, 0);
  }
  char* rbuf = buf + TK * 1024;
#pragma unroll
  for (int j = w; j < TK / 8; j += 4) {
    const int r = 8 * j + (lane >> 3);
    const char* src = addr[r].rope + 16 * ((lane & 7) ^ swz(r));
    __builtin_amdgcn_global_load_lds(src, (lds_char*)(rbuf + 1024 * j), 16, 0, 0);
  }
}

// Key codes in 32-bit arithmetic, for the tile loops (key indices and rows fit in 31 bits): the
// row of key kk in its store, with bit 30 set for the raw (window) store, or -1 for an empty slot.
struct KeyCodes32 {
  int ke;        // end of this workgroup's key range
  int n_sel;     // entry slots before the window rows
  int woff;      // ring row of window key kk: kk + woff, less wrap when that reaches wrap
  int wrap;      // raw-store rows (the ring length)
  int ent_rows;  // entry-store rows: selected slots at or past it are empty
  int has_sel;   // 1: entry slots map through the selection
  int tok_m;     // token selection: tokens per selected block (0: the slots are entries)
  int tok_base;  // token selection: raw row of position p is p + tok_base
};

__device__ __forceinline__ KeyCodes32 key_codes32(const KeyList& kl, int64_t ke) {
  return {(int)ke, (int)kl.n_sel, (int)(kl.w_row0 - kl.n_sel), (int)kl.raw_rows,
          (int)(kl.ent_rows < 0x40000000 ? kl.ent_rows : 0x40000000), kl.sel != nullptr,
          (int)kl.tok_m, (int)kl.tok_base};
}

// Raw row of token kk (kk < n_sel) of selected block `blk` in token selection, or -1.
__device__ __forceinline__ int token_row32(const KeyCodes32& c, int kk, int blk) {
  const int64_t r = (int64_t)blk * c.tok_m + kk % c.tok_m + c.tok_base;
  return r >= 0 && r < c.wrap ? (int)r : -1;
}

__device__ __forceinline__ int key_code32(const KeyCodes32& c, int kk, int raw) {
  if (kk >= c.ke || raw < 0) return -1;
  if (kk < c.n_sel && c.tok_m > 0) {
    const int r = token_row32(c, kk, raw);
    return r < 0 ? -1 : r | (1 << 30);
  }
  if (kk < c.n_sel) return c.has_sel ? (raw < c.ent_rows ? raw : -1) : kk;
  const int r = kk + c.woff;
  return (r < c.wrap ? r : r - c.wrap) | (1 << 30);
}

// S^T[32 keys x 32 heads] = K . Q^T over the 36 k-steps of a 576-dim row, as one instruction
// block: 4 K-fragment reads stay in flight ahead of the MFMA chain (5 rotating register quads, so a
// quad is rewritten only after the MFMA that read it and one more have issued). lb[t]: LDS address
// of latent k-step t (k-step s reads lb[s & 3] + 128 (s >> 2)); rb[t]: LDS address of RoPE k-step
// 32 + t. With QA the 32 latent Q^T fragments are read from accumulation registers (MFMA takes its
// B operand from either register file). With NV > 0 the block also fetches the tile's NV
// transposed V^T fragments for the PV phase (two ds_read_b64_tr_b16 each, from the per-lane bases
// ve / vo for even / odd dim tiles), issued under the last MFMAs. Every LDS read is waited for
// inside the block (lgkmcnt never exceeds 15 outstanding), and the trailing s_nop covers the wait
// states before VALU code may read the accumulator.
//
// The DMA of a later tile is issued between the MFMAs (so the wave never stalls on the load path
// while the matrix unit idles): the selection slots (4 bytes per lane), then this wave's latent
// rows (scalar row base + per-lane offset) and RoPE row groups (TileDma). These write LDS only;
// the caller waits for them by count.
// The block sets M0; no M0 value of the compiler's is live across it (the loop issues no other
// DMA).
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

template <int NLAT, int NROPE>
struct TileDma {
  const char* sel;          // per-lane source of the selection slots
  const char* lat[NLAT];    // wave-uniform row addresses of this wave's latent rows
  uint32_t off[2];          // per-lane byte offsets within a row: rows 4 j + w for even / odd j
  const char* rope[NROPE];  // per-lane sources of this wave's RoPE row groups
  int m0_rows;              // LDS address of this wave's first latent row in the target buffer
  int m0_sel;               // LDS address of the selection slot
};

// DMA of a later tile issued from inside the fp16 QK block (fp8 caches): the selection slots,
// this wave's four latent row pairs (lanes 0-31 one row, 32-63 the next), one RoPE row group and
// the tile's row scales, each into its staging region (M0 = the region's LDS address).
struct TileDmaF8 {
  const char* sel;          // per-lane source of the selection slots
  const char* lat[4];       // per-lane sources of this wave's latent row pairs
  const char* rope;         // per-lane source of this wave's RoPE row group
  const char* scl;          // per-lane source of the row scales
  int m0_sel, m0_lat, m0_rope, m0_scl;
};

// ---- BEGIN GENERATED QK BLOCKS ----
// (written by gen_qk_asm.py; edit the generator, not these lines)
__device__ __forceinline__ void qk16_chain(const v4i (&q)[36], int lbe, int lbo, int rbe,
                                           int rbo, const TileDma<8, 1>& dma,
                                           floatx4& acc0, floatx4& acc1) {
  v4i t0, t1, t2, t3, t4;
  int m0s;
    asm volatile(
      "s_mov_b32 %7, m0\n"
      "ds_read_b128 %2, %44\n"
      "ds_read_b128 %3, %45\n"
      "ds_read_b128 %4, %44 offset:128\n"
      "ds_read_b128 %5, %45 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %8, 0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %9, 0\n"
      "ds_read_b128 %6, %44 offset:256\n"
      "s_mov_b32 m0, %49\n"
      "s_nop 0\n"
      "global_load_lds_dword %48, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %10, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %11, %1\n"
      "ds_read_b128 %2, %45 offset:256\n"
      "s_mov_b32 m0, %52\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %50, %51\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %12, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %13, %1\n"
      "ds_read_b128 %3, %44 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %14, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %15, %1\n"
      "ds_read_b128 %4, %45 offset:384\n"
      "s_add_u32 m0, %52, 4096\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %53, %54\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %16, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %17, %1\n"
      "ds_read_b128 %5, %44 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %18, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %19, %1\n"
      "ds_read_b128 %6, %45 offset:512\n"
      "s_add_u32 m0, %52, 8192\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %50, %55\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %20, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %21, %1\n"
      "ds_read_b128 %2, %44 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %22, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %23, %1\n"
      "ds_read_b128 %3, %45 offset:640\n"
      "s_add_u32 m0, %52, 12288\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %53, %56\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %24, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %25, %1\n"
      "ds_read_b128 %4, %44 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %26, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %27, %1\n"
      "ds_read_b128 %5, %45 offset:768\n"
      "s_add_u32 m0, %52, 16384\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %50, %57\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %28, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %29, %1\n"
      "ds_read_b128 %6, %44 offset:896\n"
      "s_add_u32 m0, %52, 20480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %53, %58\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %30, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %31, %1\n"
      "ds_read_b128 %2, %45 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %32, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %33, %1\n"
      "ds_read_b128 %3, %46\n"
      "s_add_u32 m0, %52, 24576\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %50, %59\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %34, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %35, %1\n"
      "ds_read_b128 %4, %47\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %36, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %37, %1\n"
      "s_add_u32 m0, %52, 28672\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %53, %60\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %38, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %39, %1\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %40, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %41, %1\n"
      "s_add_u32 m0, %52, 32768\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %61, off\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %42, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %43, %1\n"
      "s_mov_b32 m0, %7\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : "=&v"(acc0), "=&v"(acc1), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&s"(m0s)
      : "a"(q[0]), "a"(q[1]), "a"(q[2]), "a"(q[3]), "a"(q[4]), "a"(q[5]), "a"(q[6]), "a"(q[7]), "a"(q[8]), "a"(q[9]), "a"(q[10]), "a"(q[11]), "a"(q[12]), "a"(q[13]), "a"(q[14]), "a"(q[15]), "a"(q[16]), "a"(q[17]), "a"(q[18]), "a"(q[19]), "a"(q[20]), "a"(q[21]), "a"(q[22]), "a"(q[23]), "a"(q[24]), "a"(q[25]), "a"(q[26]), "a"(q[27]), "a"(q[28]), "a"(q[29]), "a"(q[30]), "a"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35]), "v"(lbe), "v"(lbo), "v"(rbe), "v"(rbo), "v"(dma.sel), "s"(dma.m0_sel), "v"(dma.off[0]), "s"(dma.lat[0]), "s"(dma.m0_rows), "v"(dma.off[1]), "s"(dma.lat[1]), "s"(dma.lat[2]), "s"(dma.lat[3]), "s"(dma.lat[4]), "s"(dma.lat[5]), "s"(dma.lat[6]), "s"(dma.lat[7]), "v"(dma.rope[0])
      : "scc", "memory");
}

__device__ __forceinline__ floatx16 qk_chain_f16(const v4i (&q)[kKSteps], const int (&lb)[4],
                                                 const int (&rb)[4], const TileDmaF8& dma) {
  floatx16 acc;
  v4i t0, t1, t2, t3, t4;
  int m0s;
    asm volatile(
      "s_mov_b32 %6, m0\n"
      "ds_read_b128 %1, %43\n"
      "ds_read_b128 %2, %44\n"
      "ds_read_b128 %3, %45\n"
      "ds_read_b128 %4, %46\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %7, 0\n"
      "ds_read_b128 %5, %43 offset:128\n"
      "s_mov_b32 m0, %52\n"
      "s_nop 0\n"
      "global_load_lds_dword %51, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %8, %0\n"
      "ds_read_b128 %1, %44 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %9, %0\n"
      "ds_read_b128 %2, %45 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %10, %0\n"
      "ds_read_b128 %3, %46 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %11, %0\n"
      "ds_read_b128 %4, %43 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %12, %0\n"
      "ds_read_b128 %5, %44 offset:256\n"
      "s_mov_b32 m0, %54\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %53, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %13, %0\n"
      "ds_read_b128 %1, %45 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %14, %0\n"
      "ds_read_b128 %2, %46 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %15, %0\n"
      "ds_read_b128 %3, %43 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %16, %0\n"
      "ds_read_b128 %4, %44 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %17, %0\n"
      "ds_read_b128 %5, %45 offset:384\n"
      "s_add_u32 m0, %54, 4160\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %55, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %18, %0\n"
      "ds_read_b128 %1, %46 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %19, %0\n"
      "ds_read_b128 %2, %43 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %20, %0\n"
      "ds_read_b128 %3, %44 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %21, %0\n"
      "ds_read_b128 %4, %45 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %22, %0\n"
      "ds_read_b128 %5, %46 offset:512\n"
      "s_add_u32 m0, %54, 8320\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %56, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %23, %0\n"
      "ds_read_b128 %1, %43 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %24, %0\n"
      "ds_read_b128 %2, %44 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %25, %0\n"
      "ds_read_b128 %3, %45 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %26, %0\n"
      "ds_read_b128 %4, %46 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %27, %0\n"
      "ds_read_b128 %5, %43 offset:768\n"
      "s_add_u32 m0, %54, 12480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %57, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %28, %0\n"
      "ds_read_b128 %1, %44 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %29, %0\n"
      "ds_read_b128 %2, %45 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %30, %0\n"
      "ds_read_b128 %3, %46 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %31, %0\n"
      "ds_read_b128 %4, %43 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %32, %0\n"
      "ds_read_b128 %5, %44 offset:896\n"
      "s_mov_b32 m0, %59\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %58, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %33, %0\n"
      "ds_read_b128 %1, %45 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %34, %0\n"
      "ds_read_b128 %2, %46 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %35, %0\n"
      "ds_read_b128 %3, %47\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %36, %0\n"
      "ds_read_b128 %4, %48\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %37, %0\n"
      "ds_read_b128 %5, %49\n"
      "s_mov_b32 m0, %61\n"
      "s_nop 0\n"
      "global_load_lds_dword %60, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %38, %0\n"
      "ds_read_b128 %1, %50\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %39, %0\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %40, %0\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %41, %0\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %42, %0\n"
      "s_mov_b32 m0, %6\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : "=&v"(acc), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&s"(m0s)
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]), "v"(q[8]), "v"(q[9]), "v"(q[10]), "v"(q[11]), "v"(q[12]), "v"(q[13]), "v"(q[14]), "v"(q[15]), "v"(q[16]), "v"(q[17]), "v"(q[18]), "v"(q[19]), "v"(q[20]), "v"(q[21]), "v"(q[22]), "v"(q[23]), "v"(q[24]), "v"(q[25]), "v"(q[26]), "v"(q[27]), "v"(q[28]), "v"(q[29]), "v"(q[30]), "v"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35]), "v"(lb[0]), "v"(lb[1]), "v"(lb[2]), "v"(lb[3]), "v"(rb[0]), "v"(rb[1]), "v"(rb[2]), "v"(rb[3]), "v"(dma.sel), "s"(dma.m0_sel), "v"(dma.lat[0]), "s"(dma.m0_lat), "v"(dma.lat[1]), "v"(dma.lat[2]), "v"(dma.lat[3]), "v"(dma.rope), "s"(dma.m0_rope), "v"(dma.scl), "s"(dma.m0_scl)
      : "scc", "memory");
  return acc;
}
// ---- END GENERATED QK BLOCKS ----

// Four P^T fragments (consecutive 1 KB slots from addr), read in one block that waits for them.
__device__ __forceinline__ void load_p4(int addr, v4i (&p)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:0\n"
      "ds_read_b128 %1, %4 offset:1024\n"
      "ds_read_b128 %2, %4 offset:2048\n"
      "ds_read_b128 %3, %4 offset:3072\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=v"(p[0]), "=v"(p[1]), "=v"(p[2]), "=v"(p[3])
      : "v"(addr)
      : "memory");
}

}  // namespace
}  // namespace csa
