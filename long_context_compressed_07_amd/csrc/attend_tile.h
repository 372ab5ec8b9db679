// Building blocks shared by the MFMA attention kernels that stage key tiles in LDS by DMA
// (attend_bf16.hip, attend_fp8.hip): tile layout helpers, key codes, the barrier and wait
// encodings, P^T exchange reads and the QK instruction block.
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
  const void* src = (lane < TK && kk < ke && kk < kl.n_sel) ? (const void*)(kl.sel + kk)
                                                           : (const void*)kZeroRow;
  __builtin_amdgcn_global_load_lds(src, (lds_char*)dst, 4, 0, 0);
}

__device__ __forceinline__ int key_code_of(const KeyList& kl, int64_t kk, int raw, int64_t ke) {
  if (kk >= ke || raw < 0) return -1;
  if (kk < kl.n_sel) return kl.sel != nullptr ? raw : (int)kk;          // entry row (store 0)
  return (int)(kl.wlo + (kk - kl.n_sel) - kl.raw_base) | (1 << 30);   // raw-window row
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

// Writes the 32 staged rows: row h to dst + h * 512 (consecutive heads are consecutive rows).
template <typename T>
__device__ __forceinline__ void flush_rows(const char* buf, T* dst) {
  constexpr int kChunksRow = 512 * (int)sizeof(T) / 16;
#pragma unroll
  for (int c = threadIdx.x; c < 32 * kChunksRow; c += 256) {
    const int h = c / kChunksRow, k = c - h * kChunksRow;
    const uint4 v = *reinterpret_cast<const uint4*>(buf + h * kStageLd<T> + 16 * k);
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(dst + (int64_t)h * 512) + 16 * k) = v;
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

// key_code_of in 32-bit arithmetic, for the tile loops (key indices and rows fit in 31 bits).
struct KeyCodes32 {
  int ke;        // end of this workgroup's key range
  int n_sel;     // entry slots before the window rows
  int woff;      // raw row of window key kk: kk + woff
  int has_sel;   // 1: entry slots map through the selection
};

__device__ __forceinline__ KeyCodes32 key_codes32(const KeyList& kl, int64_t ke) {
  return {(int)ke, (int)kl.n_sel, (int)(kl.wlo - kl.n_sel - kl.raw_base), kl.sel != nullptr};
}

__device__ __forceinline__ int key_code32(const KeyCodes32& c, int kk, int raw) {
  if (kk >= c.ke || raw < 0) return -1;
  if (kk < c.n_sel) return c.has_sel ? raw : kk;
  return (kk + c.woff) | (1 << 30);
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
template <bool QA, int NV, int NLAT, int NROPE, int TK>
__device__ __forceinline__ floatx16 qk_chain(const v4i (&q)[kKSteps], const int (&lb)[4],
                                             const int (&rb)[4], int ve, int vo,
                                             v2i (&vr)[NV > 0 ? 2 * NV : 1],
                                             const TileDma<NLAT, NROPE>& dma) {
  floatx16 acc;
  v4i t0, t1, t2, t3, t4;
  if constexpr (QA && NV == 16 && NLAT == 16 && NROPE == 2 && TK == 64) {
    asm volatile(
      "ds_read_b128 %1, %74\n"
      "ds_read_b128 %2, %75\n"
      "ds_read_b128 %3, %76\n"
      "ds_read_b128 %4, %77\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %38, 0\n"
      "ds_read_b128 %5, %74 offset:128\n"
      "s_mov_b32 m0, %85\n"
      "s_nop 0\n"
      "global_load_lds_dword %84, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %39, %0\n"
      "ds_read_b128 %1, %75 offset:128\n"
      "s_mov_b32 m0, %88\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %86, %87\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %40, %0\n"
      "ds_read_b128 %2, %76 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %41, %0\n"
      "ds_read_b128 %3, %77 offset:128\n"
      "s_add_u32 m0, %88, 4096\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %89, %90\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %42, %0\n"
      "ds_read_b128 %4, %74 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %43, %0\n"
      "ds_read_b128 %5, %75 offset:256\n"
      "s_add_u32 m0, %88, 8192\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %86, %91\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %44, %0\n"
      "ds_read_b128 %1, %76 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %45, %0\n"
      "ds_read_b128 %2, %77 offset:256\n"
      "s_add_u32 m0, %88, 12288\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %89, %92\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %46, %0\n"
      "ds_read_b128 %3, %74 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %47, %0\n"
      "ds_read_b128 %4, %75 offset:384\n"
      "s_add_u32 m0, %88, 16384\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %86, %93\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %48, %0\n"
      "ds_read_b128 %5, %76 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %49, %0\n"
      "ds_read_b128 %1, %77 offset:384\n"
      "s_add_u32 m0, %88, 20480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %89, %94\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %50, %0\n"
      "ds_read_b128 %2, %74 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %51, %0\n"
      "ds_read_b128 %3, %75 offset:512\n"
      "s_add_u32 m0, %88, 24576\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %86, %95\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %52, %0\n"
      "ds_read_b128 %4, %76 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %53, %0\n"
      "ds_read_b128 %5, %77 offset:512\n"
      "s_add_u32 m0, %88, 28672\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %89, %96\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %54, %0\n"
      "ds_read_b128 %1, %74 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %55, %0\n"
      "ds_read_b128 %2, %75 offset:640\n"
      "s_add_u32 m0, %88, 32768\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %86, %97\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %56, %0\n"
      "ds_read_b128 %3, %76 offset:640\n"
      "s_add_u32 m0, %88, 36864\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %89, %98\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %57, %0\n"
      "ds_read_b128 %4, %77 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %58, %0\n"
      "ds_read_b128 %5, %74 offset:768\n"
      "s_add_u32 m0, %88, 40960\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %86, %99\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %59, %0\n"
      "ds_read_b128 %1, %75 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %60, %0\n"
      "ds_read_b128 %2, %76 offset:768\n"
      "s_add_u32 m0, %88, 45056\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %89, %100\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %61, %0\n"
      "ds_read_b128 %3, %77 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %62, %0\n"
      "ds_read_b128 %4, %74 offset:896\n"
      "s_add_u32 m0, %88, 49152\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %86, %101\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %63, %0\n"
      "ds_read_b128 %5, %75 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %64, %0\n"
      "ds_read_b128 %1, %76 offset:896\n"
      "s_add_u32 m0, %88, 53248\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %89, %102\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %65, %0\n"
      "ds_read_b128 %2, %77 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %66, %0\n"
      "ds_read_b128 %3, %78\n"
      "s_add_u32 m0, %88, 57344\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %86, %103\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %67, %0\n"
      "ds_read_b128 %4, %79\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %68, %0\n"
      "ds_read_b128 %5, %80\n"
      "s_add_u32 m0, %88, 61440\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %89, %104\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %69, %0\n"
      "ds_read_b128 %1, %81\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %70, %0\n"
      "s_add_u32 m0, %88, 65536\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %105, off\n"
      "ds_read_b64_tr_b16 %6, %82 offset:0\n"
      "ds_read_b64_tr_b16 %7, %82 offset:8192\n"
      "ds_read_b64_tr_b16 %8, %83 offset:64\n"
      "ds_read_b64_tr_b16 %9, %83 offset:8256\n"
      "ds_read_b64_tr_b16 %10, %82 offset:128\n"
      "ds_read_b64_tr_b16 %11, %82 offset:8320\n"
      "s_waitcnt lgkmcnt(8)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %71, %0\n"
      "ds_read_b64_tr_b16 %12, %83 offset:192\n"
      "ds_read_b64_tr_b16 %13, %83 offset:8384\n"
      "ds_read_b64_tr_b16 %14, %82 offset:16384\n"
      "ds_read_b64_tr_b16 %15, %82 offset:24576\n"
      "ds_read_b64_tr_b16 %16, %83 offset:16448\n"
      "ds_read_b64_tr_b16 %17, %83 offset:24640\n"
      "s_waitcnt lgkmcnt(13)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %72, %0\n"
      "s_add_u32 m0, %88, 69632\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %106, off\n"
      "ds_read_b64_tr_b16 %18, %82 offset:16512\n"
      "ds_read_b64_tr_b16 %19, %82 offset:24704\n"
      "s_waitcnt lgkmcnt(14)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %73, %0\n"
      "ds_read_b64_tr_b16 %20, %83 offset:16576\n"
      "ds_read_b64_tr_b16 %21, %83 offset:24768\n"
      "ds_read_b64_tr_b16 %22, %82 offset:32768\n"
      "ds_read_b64_tr_b16 %23, %82 offset:40960\n"
      "ds_read_b64_tr_b16 %24, %83 offset:32832\n"
      "ds_read_b64_tr_b16 %25, %83 offset:41024\n"
      "ds_read_b64_tr_b16 %26, %82 offset:32896\n"
      "ds_read_b64_tr_b16 %27, %82 offset:41088\n"
      "ds_read_b64_tr_b16 %28, %83 offset:32960\n"
      "ds_read_b64_tr_b16 %29, %83 offset:41152\n"
      "ds_read_b64_tr_b16 %30, %82 offset:49152\n"
      "ds_read_b64_tr_b16 %31, %82 offset:57344\n"
      "ds_read_b64_tr_b16 %32, %83 offset:49216\n"
      "ds_read_b64_tr_b16 %33, %83 offset:57408\n"
      "ds_read_b64_tr_b16 %34, %82 offset:49280\n"
      "ds_read_b64_tr_b16 %35, %82 offset:57472\n"
      "ds_read_b64_tr_b16 %36, %83 offset:49344\n"
      "ds_read_b64_tr_b16 %37, %83 offset:57536\n"
      "s_waitcnt lgkmcnt(0)\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : "=&v"(acc), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4), "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]), "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]), "=&v"(vr[12]), "=&v"(vr[13]), "=&v"(vr[14]), "=&v"(vr[15]), "=&v"(vr[16]), "=&v"(vr[17]), "=&v"(vr[18]), "=&v"(vr[19]), "=&v"(vr[20]), "=&v"(vr[21]), "=&v"(vr[22]), "=&v"(vr[23]), "=&v"(vr[24]), "=&v"(vr[25]), "=&v"(vr[26]), "=&v"(vr[27]), "=&v"(vr[28]), "=&v"(vr[29]), "=&v"(vr[30]), "=&v"(vr[31])
      : "a"(q[0]), "a"(q[1]), "a"(q[2]), "a"(q[3]), "a"(q[4]), "a"(q[5]), "a"(q[6]), "a"(q[7]), "a"(q[8]), "a"(q[9]), "a"(q[10]), "a"(q[11]), "a"(q[12]), "a"(q[13]), "a"(q[14]), "a"(q[15]), "a"(q[16]), "a"(q[17]), "a"(q[18]), "a"(q[19]), "a"(q[20]), "a"(q[21]), "a"(q[22]), "a"(q[23]), "a"(q[24]), "a"(q[25]), "a"(q[26]), "a"(q[27]), "a"(q[28]), "a"(q[29]), "a"(q[30]), "a"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35]), "v"(lb[0]), "v"(lb[1]), "v"(lb[2]), "v"(lb[3]), "v"(rb[0]), "v"(rb[1]), "v"(rb[2]), "v"(rb[3]), "v"(ve), "v"(vo), "v"(dma.sel), "s"(dma.m0_sel), "v"(dma.off[0]), "s"(dma.lat[0]), "s"(dma.m0_rows), "v"(dma.off[1]), "s"(dma.lat[1]), "s"(dma.lat[2]), "s"(dma.lat[3]), "s"(dma.lat[4]), "s"(dma.lat[5]), "s"(dma.lat[6]), "s"(dma.lat[7]), "s"(dma.lat[8]), "s"(dma.lat[9]), "s"(dma.lat[10]), "s"(dma.lat[11]), "s"(dma.lat[12]), "s"(dma.lat[13]), "s"(dma.lat[14]), "s"(dma.lat[15]), "v"(dma.rope[0]), "v"(dma.rope[1])
      : "m0");
  } else if constexpr (!QA && NV == 0 && NLAT == 8 && NROPE == 1 && TK == 32) {
    asm volatile(
      "ds_read_b128 %1, %42\n"
      "ds_read_b128 %2, %43\n"
      "ds_read_b128 %3, %44\n"
      "ds_read_b128 %4, %45\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %6, 0\n"
      "ds_read_b128 %5, %42 offset:128\n"
      "s_mov_b32 m0, %51\n"
      "s_nop 0\n"
      "global_load_lds_dword %50, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %7, %0\n"
      "ds_read_b128 %1, %43 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %8, %0\n"
      "ds_read_b128 %2, %44 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %9, %0\n"
      "ds_read_b128 %3, %45 offset:128\n"
      "s_mov_b32 m0, %54\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, %53\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %10, %0\n"
      "ds_read_b128 %4, %42 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %11, %0\n"
      "ds_read_b128 %5, %43 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %12, %0\n"
      "ds_read_b128 %1, %44 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %13, %0\n"
      "ds_read_b128 %2, %45 offset:256\n"
      "s_add_u32 m0, %54, 4096\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %55, %56\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %14, %0\n"
      "ds_read_b128 %3, %42 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %15, %0\n"
      "ds_read_b128 %4, %43 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %16, %0\n"
      "ds_read_b128 %5, %44 offset:384\n"
      "s_add_u32 m0, %54, 8192\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, %57\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %17, %0\n"
      "ds_read_b128 %1, %45 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %18, %0\n"
      "ds_read_b128 %2, %42 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %19, %0\n"
      "ds_read_b128 %3, %43 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %20, %0\n"
      "ds_read_b128 %4, %44 offset:512\n"
      "s_add_u32 m0, %54, 12288\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %55, %58\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %21, %0\n"
      "ds_read_b128 %5, %45 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %22, %0\n"
      "ds_read_b128 %1, %42 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %23, %0\n"
      "ds_read_b128 %2, %43 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %24, %0\n"
      "ds_read_b128 %3, %44 offset:640\n"
      "s_add_u32 m0, %54, 16384\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, %59\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %25, %0\n"
      "ds_read_b128 %4, %45 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %26, %0\n"
      "ds_read_b128 %5, %42 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %27, %0\n"
      "ds_read_b128 %1, %43 offset:768\n"
      "s_add_u32 m0, %54, 20480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %55, %60\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %28, %0\n"
      "ds_read_b128 %2, %44 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %29, %0\n"
      "ds_read_b128 %3, %45 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %30, %0\n"
      "ds_read_b128 %4, %42 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %31, %0\n"
      "ds_read_b128 %5, %43 offset:896\n"
      "s_add_u32 m0, %54, 24576\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, %61\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %32, %0\n"
      "ds_read_b128 %1, %44 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %33, %0\n"
      "ds_read_b128 %2, %45 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %34, %0\n"
      "ds_read_b128 %3, %46\n"
      "s_add_u32 m0, %54, 28672\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %55, %62\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %35, %0\n"
      "ds_read_b128 %4, %47\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %36, %0\n"
      "ds_read_b128 %5, %48\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %37, %0\n"
      "ds_read_b128 %1, %49\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %38, %0\n"
      "s_add_u32 m0, %54, 32768\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %63, off\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %39, %0\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %40, %0\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %41, %0\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : "=&v"(acc), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4)
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]), "v"(q[8]), "v"(q[9]), "v"(q[10]), "v"(q[11]), "v"(q[12]), "v"(q[13]), "v"(q[14]), "v"(q[15]), "v"(q[16]), "v"(q[17]), "v"(q[18]), "v"(q[19]), "v"(q[20]), "v"(q[21]), "v"(q[22]), "v"(q[23]), "v"(q[24]), "v"(q[25]), "v"(q[26]), "v"(q[27]), "v"(q[28]), "v"(q[29]), "v"(q[30]), "v"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35]), "v"(lb[0]), "v"(lb[1]), "v"(lb[2]), "v"(lb[3]), "v"(rb[0]), "v"(rb[1]), "v"(rb[2]), "v"(rb[3]), "v"(dma.sel), "s"(dma.m0_sel), "v"(dma.off[0]), "s"(dma.lat[0]), "s"(dma.m0_rows), "v"(dma.off[1]), "s"(dma.lat[1]), "s"(dma.lat[2]), "s"(dma.lat[3]), "s"(dma.lat[4]), "s"(dma.lat[5]), "s"(dma.lat[6]), "s"(dma.lat[7]), "v"(dma.rope[0])
      : "m0");
  } else {
    static_assert(QA && NV == 16, "unsupported configuration");
  }
  return acc;
}

__device__ __forceinline__ void qk16_chain(const v4i (&q)[36], int lbe, int lbo, int rbe,
                                           int rbo, const TileDma<8, 1>& dma,
                                           floatx4& acc0, floatx4& acc1) {
  v4i t0, t1, t2, t3, t4;
    asm volatile(
      "ds_read_b128 %2, %43\n"
      "ds_read_b128 %3, %44\n"
      "ds_read_b128 %4, %43 offset:128\n"
      "ds_read_b128 %5, %44 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %7, 0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %8, 0\n"
      "ds_read_b128 %6, %43 offset:256\n"
      "s_mov_b32 m0, %48\n"
      "s_nop 0\n"
      "global_load_lds_dword %47, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %9, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %10, %1\n"
      "ds_read_b128 %2, %44 offset:256\n"
      "s_mov_b32 m0, %51\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %49, %50\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %11, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %12, %1\n"
      "ds_read_b128 %3, %43 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %13, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %14, %1\n"
      "ds_read_b128 %4, %44 offset:384\n"
      "s_add_u32 m0, %51, 4096\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, %53\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %15, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %16, %1\n"
      "ds_read_b128 %5, %43 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %17, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %18, %1\n"
      "ds_read_b128 %6, %44 offset:512\n"
      "s_add_u32 m0, %51, 8192\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %49, %54\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %19, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %20, %1\n"
      "ds_read_b128 %2, %43 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %21, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %22, %1\n"
      "ds_read_b128 %3, %44 offset:640\n"
      "s_add_u32 m0, %51, 12288\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, %55\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %23, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %24, %1\n"
      "ds_read_b128 %4, %43 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %25, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %26, %1\n"
      "ds_read_b128 %5, %44 offset:768\n"
      "s_add_u32 m0, %51, 16384\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %49, %56\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %27, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %28, %1\n"
      "ds_read_b128 %6, %43 offset:896\n"
      "s_add_u32 m0, %51, 20480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, %57\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %29, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %30, %1\n"
      "ds_read_b128 %2, %44 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %31, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %32, %1\n"
      "ds_read_b128 %3, %45\n"
      "s_add_u32 m0, %51, 24576\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %49, %58\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %33, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %34, %1\n"
      "ds_read_b128 %4, %46\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %35, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %36, %1\n"
      "s_add_u32 m0, %51, 28672\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, %59\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %37, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %2, %38, %1\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %39, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %40, %1\n"
      "s_add_u32 m0, %51, 32768\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %60, off\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %41, %0\n"
      "v_mfma_f32_16x16x32_bf16 %1, %4, %42, %1\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : "=&v"(acc0), "=&v"(acc1), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4)
      : "a"(q[0]), "a"(q[1]), "a"(q[2]), "a"(q[3]), "a"(q[4]), "a"(q[5]), "a"(q[6]), "a"(q[7]), "a"(q[8]), "a"(q[9]), "a"(q[10]), "a"(q[11]), "a"(q[12]), "a"(q[13]), "a"(q[14]), "a"(q[15]), "a"(q[16]), "a"(q[17]), "a"(q[18]), "a"(q[19]), "a"(q[20]), "a"(q[21]), "a"(q[22]), "a"(q[23]), "a"(q[24]), "a"(q[25]), "a"(q[26]), "a"(q[27]), "a"(q[28]), "a"(q[29]), "a"(q[30]), "a"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35]), "v"(lbe), "v"(lbo), "v"(rbe), "v"(rbo), "v"(dma.sel), "s"(dma.m0_sel), "v"(dma.off[0]), "s"(dma.lat[0]), "s"(dma.m0_rows), "v"(dma.off[1]), "s"(dma.lat[1]), "s"(dma.lat[2]), "s"(dma.lat[3]), "s"(dma.lat[4]), "s"(dma.lat[5]), "s"(dma.lat[6]), "s"(dma.lat[7]), "v"(dma.rope[0])
      : "m0");
}

__device__ __forceinline__ floatx16 qk_chain_f16(const v4i (&q)[kKSteps], const int (&lb)[4],
                                                 const int (&rb)[4], const TileDmaF8& dma) {
  floatx16 acc;
  v4i t0, t1, t2, t3, t4;
    asm volatile(
      "ds_read_b128 %1, %42\n"
      "ds_read_b128 %2, %43\n"
      "ds_read_b128 %3, %44\n"
      "ds_read_b128 %4, %45\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %6, 0\n"
      "ds_read_b128 %5, %42 offset:128\n"
      "s_mov_b32 m0, %51\n"
      "s_nop 0\n"
      "global_load_lds_dword %50, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %7, %0\n"
      "ds_read_b128 %1, %43 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %8, %0\n"
      "ds_read_b128 %2, %44 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %9, %0\n"
      "ds_read_b128 %3, %45 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %10, %0\n"
      "ds_read_b128 %4, %42 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %11, %0\n"
      "ds_read_b128 %5, %43 offset:256\n"
      "s_mov_b32 m0, %53\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %52, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %12, %0\n"
      "ds_read_b128 %1, %44 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %13, %0\n"
      "ds_read_b128 %2, %45 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %14, %0\n"
      "ds_read_b128 %3, %42 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %15, %0\n"
      "ds_read_b128 %4, %43 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %16, %0\n"
      "ds_read_b128 %5, %44 offset:384\n"
      "s_add_u32 m0, %53, 4160\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %54, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %17, %0\n"
      "ds_read_b128 %1, %45 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %18, %0\n"
      "ds_read_b128 %2, %42 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %19, %0\n"
      "ds_read_b128 %3, %43 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %20, %0\n"
      "ds_read_b128 %4, %44 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %21, %0\n"
      "ds_read_b128 %5, %45 offset:512\n"
      "s_add_u32 m0, %53, 8320\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %55, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %22, %0\n"
      "ds_read_b128 %1, %42 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %23, %0\n"
      "ds_read_b128 %2, %43 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %24, %0\n"
      "ds_read_b128 %3, %44 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %25, %0\n"
      "ds_read_b128 %4, %45 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %26, %0\n"
      "ds_read_b128 %5, %42 offset:768\n"
      "s_add_u32 m0, %53, 12480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %56, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %27, %0\n"
      "ds_read_b128 %1, %43 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %28, %0\n"
      "ds_read_b128 %2, %44 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %29, %0\n"
      "ds_read_b128 %3, %45 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %30, %0\n"
      "ds_read_b128 %4, %42 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %31, %0\n"
      "ds_read_b128 %5, %43 offset:896\n"
      "s_mov_b32 m0, %58\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %57, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %32, %0\n"
      "ds_read_b128 %1, %44 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %33, %0\n"
      "ds_read_b128 %2, %45 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %34, %0\n"
      "ds_read_b128 %3, %46\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %35, %0\n"
      "ds_read_b128 %4, %47\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %36, %0\n"
      "ds_read_b128 %5, %48\n"
      "s_mov_b32 m0, %60\n"
      "s_nop 0\n"
      "global_load_lds_dword %59, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %2, %37, %0\n"
      "ds_read_b128 %1, %49\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_f16 %0, %3, %38, %0\n"
      "s_waitcnt lgkmcnt(2)\n"
      "v_mfma_f32_32x32x16_f16 %0, %4, %39, %0\n"
      "s_waitcnt lgkmcnt(1)\n"
      "v_mfma_f32_32x32x16_f16 %0, %5, %40, %0\n"
      "s_waitcnt lgkmcnt(0)\n"
      "v_mfma_f32_32x32x16_f16 %0, %1, %41, %0\n"
      "s_nop 7\n"
      "s_nop 7\n"
      "s_nop 4\n"
      : "=&v"(acc), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3), "=&v"(t4)
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]), "v"(q[8]), "v"(q[9]), "v"(q[10]), "v"(q[11]), "v"(q[12]), "v"(q[13]), "v"(q[14]), "v"(q[15]), "v"(q[16]), "v"(q[17]), "v"(q[18]), "v"(q[19]), "v"(q[20]), "v"(q[21]), "v"(q[22]), "v"(q[23]), "v"(q[24]), "v"(q[25]), "v"(q[26]), "v"(q[27]), "v"(q[28]), "v"(q[29]), "v"(q[30]), "v"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35]), "v"(lb[0]), "v"(lb[1]), "v"(lb[2]), "v"(lb[3]), "v"(rb[0]), "v"(rb[1]), "v"(rb[2]), "v"(rb[3]), "v"(dma.sel), "s"(dma.m0_sel), "v"(dma.lat[0]), "s"(dma.m0_lat), "v"(dma.lat[1]), "v"(dma.lat[2]), "v"(dma.lat[3]), "v"(dma.rope), "s"(dma.m0_rope), "v"(dma.scl), "s"(dma.m0_scl)
      : "m0");
  return acc;
}
// ---- END GENERATED QK BLOCKS ----

// Q^T fragments of one head (bf16, as stored): fragment s holds dims 16 s + 8 hi + [0, 8). With QA
// the 32 latent fragments are loaded straight into accumulation registers, in one block that
// waits for its loads.
template <bool QA>
__device__ __forceinline__ void load_q(const uint16_t* qrow, int hi, v4i (&q)[kKSteps]) {
  const uint16_t* p = qrow + 8 * hi;
  if constexpr (QA) {
    asm volatile(
        "global_load_dwordx4 %0, %32, off offset:0\n"
        "global_load_dwordx4 %1, %32, off offset:32\n"
        "global_load_dwordx4 %2, %32, off offset:64\n"
        "global_load_dwordx4 %3, %32, off offset:96\n"
        "global_load_dwordx4 %4, %32, off offset:128\n"
        "global_load_dwordx4 %5, %32, off offset:160\n"
        "global_load_dwordx4 %6, %32, off offset:192\n"
        "global_load_dwordx4 %7, %32, off offset:224\n"
        "global_load_dwordx4 %8, %32, off offset:256\n"
        "global_load_dwordx4 %9, %32, off offset:288\n"
        "global_load_dwordx4 %10, %32, off offset:320\n"
        "global_load_dwordx4 %11, %32, off offset:352\n"
        "global_load_dwordx4 %12, %32, off offset:384\n"
        "global_load_dwordx4 %13, %32, off offset:416\n"
        "global_load_dwordx4 %14, %32, off offset:448\n"
        "global_load_dwordx4 %15, %32, off offset:480\n"
        "global_load_dwordx4 %16, %32, off offset:512\n"
        "global_load_dwordx4 %17, %32, off offset:544\n"
        "global_load_dwordx4 %18, %32, off offset:576\n"
        "global_load_dwordx4 %19, %32, off offset:608\n"
        "global_load_dwordx4 %20, %32, off offset:640\n"
        "global_load_dwordx4 %21, %32, off offset:672\n"
        "global_load_dwordx4 %22, %32, off offset:704\n"
        "global_load_dwordx4 %23, %32, off offset:736\n"
        "global_load_dwordx4 %24, %32, off offset:768\n"
        "global_load_dwordx4 %25, %32, off offset:800\n"
        "global_load_dwordx4 %26, %32, off offset:832\n"
        "global_load_dwordx4 %27, %32, off offset:864\n"
        "global_load_dwordx4 %28, %32, off offset:896\n"
        "global_load_dwordx4 %29, %32, off offset:928\n"
        "global_load_dwordx4 %30, %32, off offset:960\n"
        "global_load_dwordx4 %31, %32, off offset:992\n"
        "s_waitcnt vmcnt(0)\n"
        : "=a"(q[0]), "=a"(q[1]), "=a"(q[2]), "=a"(q[3]), "=a"(q[4]), "=a"(q[5]), "=a"(q[6]), "=a"(q[7]), "=a"(q[8]), "=a"(q[9]), "=a"(q[10]), "=a"(q[11]), "=a"(q[12]), "=a"(q[13]), "=a"(q[14]), "=a"(q[15]), "=a"(q[16]), "=a"(q[17]), "=a"(q[18]), "=a"(q[19]), "=a"(q[20]), "=a"(q[21]), "=a"(q[22]), "=a"(q[23]), "=a"(q[24]), "=a"(q[25]), "=a"(q[26]), "=a"(q[27]), "=a"(q[28]), "=a"(q[29]), "=a"(q[30]), "=a"(q[31])
        : "v"(p));
  } else {
#pragma unroll
    for (int s = 0; s < 32; ++s) q[s] = *reinterpret_cast<const v4i*>(p + 16 * s);
  }
#pragma unroll
  for (int s = 32; s < kKSteps; ++s) q[s] = *reinterpret_cast<const v4i*>(p + 16 * s);
}

// The P^T fragments of one tile (8 of them: k-step ks and row group r at index ks * RG + r), read
// from the exchange buffer in one block that waits for its reads.
__device__ __forceinline__ void load_p8(int addr, v4i (&p)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:0\n"
      "ds_read_b128 %1, %8 offset:1024\n"
      "ds_read_b128 %2, %8 offset:2048\n"
      "ds_read_b128 %3, %8 offset:3072\n"
      "ds_read_b128 %4, %8 offset:4096\n"
      "ds_read_b128 %5, %8 offset:5120\n"
      "ds_read_b128 %6, %8 offset:6144\n"
      "ds_read_b128 %7, %8 offset:7168\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=v"(p[0]), "=v"(p[1]), "=v"(p[2]), "=v"(p[3]), "=v"(p[4]), "=v"(p[5]), "=v"(p[6]), "=v"(p[7])
      : "v"(addr));
}

// Four P^T fragments (consecutive 1 KB slots from addr), read in one block that waits for them.
__device__ __forceinline__ void load_p4(int addr, v4i (&p)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:0\n"
      "ds_read_b128 %1, %4 offset:1024\n"
      "ds_read_b128 %2, %4 offset:2048\n"
      "ds_read_b128 %3, %4 offset:3072\n"
      "s_waitcnt lgkmcnt(0)\n"
      : "=v"(p[0]), "=v"(p[1]), "=v"(p[2]), "=v"(p[3])
      : "v"(addr));
}

}  // namespace
}  // namespace csa
