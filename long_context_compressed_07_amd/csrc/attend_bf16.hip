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

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
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
__device__ __forceinline__ void dma_tile(const KeyAddr* addr, char* buf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
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
      "s_mov_b32 m0, %106\n"
      "s_nop 0\n"
      "global_load_lds_dword %84, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %39, %0\n"
      "ds_read_b128 %1, %75 offset:128\n"
      "s_add_u32 m0, %105, 0\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %101, %85\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %40, %0\n"
      "ds_read_b128 %2, %76 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %41, %0\n"
      "ds_read_b128 %3, %77 offset:128\n"
      "s_add_u32 m0, %105, 4096\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %102, %86\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %42, %0\n"
      "ds_read_b128 %4, %74 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %43, %0\n"
      "ds_read_b128 %5, %75 offset:256\n"
      "s_add_u32 m0, %105, 8192\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %101, %87\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %44, %0\n"
      "ds_read_b128 %1, %76 offset:256\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %45, %0\n"
      "ds_read_b128 %2, %77 offset:256\n"
      "s_add_u32 m0, %105, 12288\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %102, %88\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %46, %0\n"
      "ds_read_b128 %3, %74 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %47, %0\n"
      "ds_read_b128 %4, %75 offset:384\n"
      "s_add_u32 m0, %105, 16384\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %101, %89\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %48, %0\n"
      "ds_read_b128 %5, %76 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %49, %0\n"
      "ds_read_b128 %1, %77 offset:384\n"
      "s_add_u32 m0, %105, 20480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %102, %90\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %50, %0\n"
      "ds_read_b128 %2, %74 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %51, %0\n"
      "ds_read_b128 %3, %75 offset:512\n"
      "s_add_u32 m0, %105, 24576\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %101, %91\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %52, %0\n"
      "ds_read_b128 %4, %76 offset:512\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %53, %0\n"
      "ds_read_b128 %5, %77 offset:512\n"
      "s_add_u32 m0, %105, 28672\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %102, %92\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %54, %0\n"
      "ds_read_b128 %1, %74 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %55, %0\n"
      "ds_read_b128 %2, %75 offset:640\n"
      "s_add_u32 m0, %105, 32768\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %101, %93\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %56, %0\n"
      "ds_read_b128 %3, %76 offset:640\n"
      "s_add_u32 m0, %105, 36864\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %102, %94\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %57, %0\n"
      "ds_read_b128 %4, %77 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %58, %0\n"
      "ds_read_b128 %5, %74 offset:768\n"
      "s_add_u32 m0, %105, 40960\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %101, %95\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %59, %0\n"
      "ds_read_b128 %1, %75 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %60, %0\n"
      "ds_read_b128 %2, %76 offset:768\n"
      "s_add_u32 m0, %105, 45056\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %102, %96\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %61, %0\n"
      "ds_read_b128 %3, %77 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %62, %0\n"
      "ds_read_b128 %4, %74 offset:896\n"
      "s_add_u32 m0, %105, 49152\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %101, %97\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %63, %0\n"
      "ds_read_b128 %5, %75 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %64, %0\n"
      "ds_read_b128 %1, %76 offset:896\n"
      "s_add_u32 m0, %105, 53248\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %102, %98\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %65, %0\n"
      "ds_read_b128 %2, %77 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %66, %0\n"
      "ds_read_b128 %3, %78\n"
      "s_add_u32 m0, %105, 57344\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %101, %99\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %67, %0\n"
      "ds_read_b128 %4, %79\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %68, %0\n"
      "ds_read_b128 %5, %80\n"
      "s_add_u32 m0, %105, 61440\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %102, %100\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %69, %0\n"
      "ds_read_b128 %1, %81\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %70, %0\n"
      "s_add_u32 m0, %105, 65536\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %103, off\n"
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
      "s_add_u32 m0, %105, 69632\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %104, off\n"
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
                 : "a"(q[0]), "a"(q[1]), "a"(q[2]), "a"(q[3]), "a"(q[4]), "a"(q[5]), "a"(q[6]), "a"(q[7]), "a"(q[8]), "a"(q[9]), "a"(q[10]), "a"(q[11]), "a"(q[12]), "a"(q[13]), "a"(q[14]), "a"(q[15]), "a"(q[16]), "a"(q[17]), "a"(q[18]), "a"(q[19]), "a"(q[20]), "a"(q[21]), "a"(q[22]), "a"(q[23]), "a"(q[24]), "a"(q[25]), "a"(q[26]), "a"(q[27]), "a"(q[28]), "a"(q[29]), "a"(q[30]), "a"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35]),
                   "v"(lb[0]), "v"(lb[1]), "v"(lb[2]), "v"(lb[3]), "v"(rb[0]), "v"(rb[1]),
                   "v"(rb[2]), "v"(rb[3]), "v"(ve), "v"(vo), "v"(dma.sel), "s"(dma.lat[0]), "s"(dma.lat[1]), "s"(dma.lat[2]), "s"(dma.lat[3]), "s"(dma.lat[4]), "s"(dma.lat[5]), "s"(dma.lat[6]), "s"(dma.lat[7]), "s"(dma.lat[8]), "s"(dma.lat[9]), "s"(dma.lat[10]), "s"(dma.lat[11]), "s"(dma.lat[12]), "s"(dma.lat[13]), "s"(dma.lat[14]), "s"(dma.lat[15]), "v"(dma.off[0]), "v"(dma.off[1]), "v"(dma.rope[0]), "v"(dma.rope[1]), "s"(dma.m0_rows), "s"(dma.m0_sel)
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
      "s_mov_b32 m0, %65\n"
      "s_nop 0\n"
      "global_load_lds_dword %52, off\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %7, %0\n"
      "ds_read_b128 %1, %43 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %8, %0\n"
      "ds_read_b128 %2, %44 offset:128\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %9, %0\n"
      "ds_read_b128 %3, %45 offset:128\n"
      "s_add_u32 m0, %64, 0\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %61, %53\n"
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
      "s_add_u32 m0, %64, 4096\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %62, %54\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %14, %0\n"
      "ds_read_b128 %3, %42 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %15, %0\n"
      "ds_read_b128 %4, %43 offset:384\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %16, %0\n"
      "ds_read_b128 %5, %44 offset:384\n"
      "s_add_u32 m0, %64, 8192\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %61, %55\n"
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
      "s_add_u32 m0, %64, 12288\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %62, %56\n"
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
      "s_add_u32 m0, %64, 16384\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %61, %57\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %5, %25, %0\n"
      "ds_read_b128 %4, %45 offset:640\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %1, %26, %0\n"
      "ds_read_b128 %5, %42 offset:768\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %27, %0\n"
      "ds_read_b128 %1, %43 offset:768\n"
      "s_add_u32 m0, %64, 20480\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %62, %58\n"
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
      "s_add_u32 m0, %64, 24576\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %61, %59\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %32, %0\n"
      "ds_read_b128 %1, %44 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %3, %33, %0\n"
      "ds_read_b128 %2, %45 offset:896\n"
      "s_waitcnt lgkmcnt(3)\n"
      "v_mfma_f32_32x32x16_bf16 %0, %4, %34, %0\n"
      "ds_read_b128 %3, %46\n"
      "s_add_u32 m0, %64, 28672\n"
      "s_nop 0\n"
      "global_load_lds_dwordx4 %62, %60\n"
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
      "s_add_u32 m0, %64, 32768\n"
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
                 : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "v"(q[4]), "v"(q[5]), "v"(q[6]), "v"(q[7]), "v"(q[8]), "v"(q[9]), "v"(q[10]), "v"(q[11]), "v"(q[12]), "v"(q[13]), "v"(q[14]), "v"(q[15]), "v"(q[16]), "v"(q[17]), "v"(q[18]), "v"(q[19]), "v"(q[20]), "v"(q[21]), "v"(q[22]), "v"(q[23]), "v"(q[24]), "v"(q[25]), "v"(q[26]), "v"(q[27]), "v"(q[28]), "v"(q[29]), "v"(q[30]), "v"(q[31]), "v"(q[32]), "v"(q[33]), "v"(q[34]), "v"(q[35]),
                   "v"(lb[0]), "v"(lb[1]), "v"(lb[2]), "v"(lb[3]), "v"(rb[0]), "v"(rb[1]),
                   "v"(rb[2]), "v"(rb[3]), "v"(ve), "v"(vo), "v"(dma.sel), "s"(dma.lat[0]), "s"(dma.lat[1]), "s"(dma.lat[2]), "s"(dma.lat[3]), "s"(dma.lat[4]), "s"(dma.lat[5]), "s"(dma.lat[6]), "s"(dma.lat[7]), "v"(dma.off[0]), "v"(dma.off[1]), "v"(dma.rope[0]), "s"(dma.m0_rows), "s"(dma.m0_sel)
                 : "m0");
  } else {
    static_assert(QA && NV == 16, "unsupported configuration");
  }
  return acc;
}

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
  const int qi = blockIdx.x / per_q;
  const int rem = blockIdx.x - qi * per_q;
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
    if (threadIdx.x < 64) {
      // Codes of tile t + kAhead + 1 (its selection slots landed with the DMA of tile t + kAhead - 1,
      // which this wave has waited for).
      const int64_t kk2 = t0 + (kAhead + 1) * TK + threadIdx.x;
      const int raw2 = sel_dma ? s_sel[(it + kAhead + 1) & 1][threadIdx.x] : 0;
      const int c2 = threadIdx.x < TK ? key_code_of(kl, kk2, raw2, ke) : -1;
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
  if (threadIdx.x == 0) plan.flags[blockIdx.x] = s_flag;

#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int hrow = 32 * r + (lane & 31);
    float l = s_l[0][hrow];
#pragma unroll
    for (int j = 1; j < KB; ++j) l += s_l[j][hrow];
    const float m = s_ref[0][hrow];
    const int head = hbase + hrow;
    if (plan.n_split == 1) {
      const float inv = l > 0.f ? 1.0f / l : 0.f;
      float* orow = a.out + ((int64_t)qi * a.H + head) * kDC + 128 * w;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(orow + 32 * mt + 8 * j + 4 * hi) =
              make_float4(o[mt][r][4 * j] * inv, o[mt][r][4 * j + 1] * inv,
                          o[mt][r][4 * j + 2] * inv, o[mt][r][4 * j + 3] * inv);
      if (a.lse != nullptr && w == 0 && hi == 0)
        a.lse[(int64_t)qi * a.H + head] =
            l > 0.f ? (m + __log2f(l)) * 0.6931471805599453f : -INFINITY;
    } else {
      const int64_t pidx = ((int64_t)qi * plan.n_split + split) * a.H + head;
      float* orow = plan.ws_o + pidx * kDC + 128 * w;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<float4*>(orow + 32 * mt + 8 * j + 4 * hi) =
              make_float4(o[mt][r][4 * j], o[mt][r][4 * j + 1], o[mt][r][4 * j + 2],
                          o[mt][r][4 * j + 3]);
      if (w == 0 && hi == 0) {
        plan.ws_ml[pidx * 2] = m;
        plan.ws_ml[pidx * 2 + 1] = l;
      }
    }
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
