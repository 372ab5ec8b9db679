// MFMA attention for bf16 caches (csa_attend / hca_attend; 512 latent + 64 RoPE dims per row,
// bf16 queries, heads in groups of 32): the prefill path.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA: selected compressed rows plus the
// raw window, MQA with one KV shared by every head; HCA: dense over the m'-compressed rows) and the
// MLA section (key row = [latent; RoPE key], value row = latent); yudonglee.me "DeepSeek-V4 详解"
// 2.2 Step 4 and 2.3 Step 2.
//
// A workgroup is 4 waves and serves one query: HGW groups of 32 heads x KSW splits of its key list
// (HGW * KSW = 4). Key rows reach LDS by DMA (global_load_lds, 16 bytes per lane, no registers):
// tile t + 1 streams into the second buffer while tile t is computed, so each tile costs one
// barrier. Rows stay bf16 and unpadded, split into a latent region ([rows][1024 B]) and a RoPE
// region ([rows][128 B]) so that one DMA instruction moves one row's latent (a wave-uniform row
// address). 16-byte chunk c of row r sits at chunk position c ^ f(r), f(r) = 2 (r & 3) + (r >> 2 & 1),
// which keeps the K-fragment reads (8 consecutive rows, one chunk) and the transposed V reads
// (4 consecutive rows, 2 adjacent chunks) free of bank conflicts. Per wave and 32-key tile:
//   S^T[32 keys x 32 heads] = K . Q^T      36 x mfma_f32_32x32x16_bf16 (Q^T in registers)
//   softmax per head                        lane-local (each lane owns one head's column); the
//                                           reference max is fixed at the first non-empty tile
//   O^T[512 x 32 heads] += V^T . P^T        P = P_hi + P_lo, both bf16 (P_lo = bf16(p - P_hi)):
//                                           2 x 32 mfma, relative error of P about 2^-16
// Products of bf16 values are exact in the fp32 accumulators, so only P is rounded.
#include "attend_generic.h"
#include "attend_plan.h"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kDC = 512;
constexpr int kDR = 64;
constexpr int kD = kDC + kDR;
constexpr int kChunks = kD / 8;          // 72 chunks of 16 bytes per row
constexpr int kRowB = kD * 2;            // 1152 bytes per staged row
constexpr int kKSteps = kD / 16;
constexpr int kMT = kDC / 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRange = 60.0f;          // log2 headroom of P above the reference max (bf16 range)

__device__ const uint4 kZeroChunk = {0u, 0u, 0u, 0u};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ int key_code(const AttendArgs& a, const KeyList& kl, int64_t kk,
                                        int64_t ke) {
  if (kk >= ke) return -1;
  int src;
  const int64_t row = key_row(a, kl, kk, src);
  return row >= 0 ? (int)row | (src << 30) : -1;
}

// Issue the DMA of one tile (TK rows) into buf = [latent region TK x 1024 B][RoPE region TK x 128 B].
// Latent: one instruction per row (wave w takes rows w, w + 4, ...), lane l fetching chunk
// l ^ f(row). RoPE: one instruction per 8 rows, lane l fetching row 8 j + l / 8, chunk
// (l & 7) ^ f(row). Empty slots read a zero chunk.
template <int TK>
__device__ __forceinline__ void dma_tile(const AttendArgs& a, int64_t b, const int* codes,
                                         char* buf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int code[TK / 4];
#pragma unroll
  for (int j = 0; j < TK / 4; ++j) code[j] = codes[4 * j + w];
#pragma unroll
  for (int j = 0; j < TK / 4; ++j) {
    const int r = 4 * j + w;
    const int cd = __builtin_amdgcn_readfirstlane(code[j]);
    const void* src = &kZeroChunk;
    if (cd >= 0) {
      const Store& st = (cd >> 30) ? a.raw : a.ent;
      const uint16_t* crow = static_cast<const uint16_t*>(st.c) +
                             (b * st.rows + (cd & 0x3fffffff)) * st.ld_c;
      src = crow + 8 * (lane ^ swz(r));
    }
    __builtin_amdgcn_global_load_lds(src, (lds_char*)(buf + 1024 * r), 16, 0, 0);
  }
  char* rbuf = buf + TK * 1024;
#pragma unroll
  for (int j = w; j < TK / 8; j += 4) {
    const int r = 8 * j + (lane >> 3);
    const int cd = codes[r];
    const void* src = &kZeroChunk;
    if (cd >= 0) {
      const Store& st = (cd >> 30) ? a.raw : a.ent;
      const uint16_t* rrow = static_cast<const uint16_t*>(st.r) +
                             (b * st.rows + (cd & 0x3fffffff)) * st.ld_r;
      src = rrow + 8 * ((lane & 7) ^ swz(r));
    }
    __builtin_amdgcn_global_load_lds(src, (lds_char*)(rbuf + 1024 * j), 16, 0, 0);
  }
}

// Raw list entry for key kk (the selection slot, or the row for window / dense keys), fetched
// early; key_code_of() turns it into a code later, so the load's latency overlaps a whole tile.
__device__ __forceinline__ int64_t key_prefetch(const AttendArgs& a, const KeyList& kl,
                                                int64_t kk, int64_t ke) {
  if (kk >= ke) return -1;
  if (kk < kl.n_sel && kl.sel != nullptr) return (int64_t)kl.sel[kk];
  return kk;
}

__device__ __forceinline__ int key_code_of(const KeyList& kl, int64_t kk, int64_t raw,
                                           int64_t ke) {
  if (kk >= ke || raw < 0) return -1;
  if (kk < kl.n_sel) return (int)raw;                            // entry row (store 0)
  return (int)(kl.wlo + (kk - kl.n_sel) - kl.raw_base) | (1 << 30);   // raw-window row
}

template <int KSW>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attend_bf16_kernel(AttendArgs a, AttnPlan plan) {
  constexpr int HGW = 4 / KSW;
  constexpr int TK = 32 * KSW;
  constexpr int kBufB = TK * kRowB;
  constexpr int kMergeB = KSW > 1 ? (KSW / 2) * HGW * (kMT * 16 + 2) * 64 * 4 : 0;
  constexpr int kLdsB = 2 * kBufB > kMergeB ? 2 * kBufB : kMergeB;
  __shared__ __attribute__((aligned(1024))) char lds[kLdsB];
  __shared__ int s_code[3][TK];
  __shared__ int s_flag;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hgw = w % HGW;
  const int ks = w / HGW;
  const int hi = lane >> 5;
  const int per_q = plan.head_groups * plan.n_split;
  const int qi = blockIdx.x / per_q;
  const int rem = blockIdx.x - qi * per_q;
  const int hgrp = rem / plan.n_split;
  const int split = rem - hgrp * plan.n_split;
  const int head = (hgrp * HGW + hgw) * 32 + (lane & 31);
  if (threadIdx.x == 0) s_flag = 0;

  const KeyList kl = make_key_list(a, qi);
  const int64_t per_split = (kl.total + plan.n_split - 1) / plan.n_split;
  const int64_t kb = (int64_t)split * per_split;
  const int64_t ke = kb + per_split < kl.total ? kb + per_split : kl.total;

  // Q^T fragments (bf16, as stored): head `head`, dims 16 s + 8 hi + [0, 8).
  bf16x8 qb[kKSteps];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)qi * a.H + head) * kD;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
      qb[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * hi));
  }
  floatx16 o[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) o[mt] = floatx16{};
  float m_run = -INFINITY, l_run = 0.f;
  bool overflow = false;
  const float cscale = a.sm_scale * kLog2e;

  // Prologue: codes of tiles 0 and 1; tile 0 in flight.
  if (threadIdx.x < TK) {
    s_code[0][threadIdx.x] = key_code(a, kl, kb + threadIdx.x, ke);
    s_code[1][threadIdx.x] = key_code(a, kl, kb + TK + threadIdx.x, ke);
  }
  __syncthreads();
  if (kb < ke) dma_tile<TK>(a, kl.b, s_code[0], lds);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  int it = 0;
  for (int64_t t0 = kb; t0 < ke; t0 += TK, ++it) {
    const int cb = it & 1;
    const int* codes = s_code[it % 3];
    // The list entries of the tile after next are fetched first (their wait comes at the end of
    // the iteration), then the next tile's rows stream into the other buffer.
    const int64_t kk2 = t0 + 2 * TK + threadIdx.x;
    int64_t raw2 = -1;
    if (threadIdx.x < TK) raw2 = key_prefetch(a, kl, kk2, ke);
    if (t0 + TK < ke) dma_tile<TK>(a, kl.b, s_code[(it + 1) % 3], lds + (cb ^ 1) * kBufB);

    const char* cbuf = lds + cb * kBufB;                 // latent region of this tile
    const char* wlat = cbuf + (32 * ks) * 1024;          // this wave's 32 rows
    const char* wrope = cbuf + TK * 1024 + (32 * ks) * 128;
    // S^T = K . Q^T: latent k-steps 0..31 (chunk 2 s + hi), RoPE k-steps 32..35.
    floatx16 acc = floatx16{};
    {
      // Chunk 2 s + hi of row r sits at (2 s + hi) ^ f = 2 (s ^ f1) + (hi ^ f0): for s = 4 q + t
      // that is byte 128 q + 32 (t ^ f1) + 16 (hi ^ f0), i.e. four per-lane bases (one per t)
      // plus compile-time offsets.
      const int r = lane & 31;
      const int f = swz(r);
      const int h16 = 16 * (hi ^ (f & 1));
      const char* lb[4];
      const char* rb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lb[t] = wlat + r * 1024 + 32 * (t ^ (f >> 1)) + h16;
        rb[t] = wrope + r * 128 + 32 * (t ^ (f >> 1)) + h16;
      }
      // Four K fragments in flight ahead of the MFMA that consumes them.
      constexpr int kAhead = 4;
      bf16x8 kf[kAhead];
#pragma unroll
      for (int s = 0; s < kAhead; ++s)
        kf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(lb[s & 3] + 128 * (s >> 2)));
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const bf16x8 av = kf[s % kAhead];
        const int sn = s + kAhead;
        if (sn < kKSteps) {
          const char* src = sn < kDC / 16 ? lb[sn & 3] + 128 * (sn >> 2) : rb[sn & 3];
          kf[s % kAhead] = as_bf16x8(*reinterpret_cast<const uint4*>(src));
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qb[s], acc, 0, 0, 0);
      }
    }

    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 32 * ks + 8 * (i >> 2) + 4 * hi + (i & 3);
      acc[i] = codes[key] >= 0 ? acc[i] * cscale : -INFINITY;
      tmax = fmaxf(tmax, acc[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    m_run = m_run == -INFINITY ? tmax : m_run;
    overflow |= tmax > m_run + kRange;
    // P^T = P_hi + P_lo in bf16, in the B-operand layout: k-step s of lane half hi covers keys
    // 16 s + 4 hi + [0,4) and 16 s + 8 + 4 hi + [0,4).
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = acc[i] == -INFINITY ? 0.f : exp2f(fminf(acc[i] - m_run, kRange));
      l_run += p;
      const __bf16 h = (__bf16)p;
      ph[i >> 3][i & 7] = h;
      pl[i >> 3][i & 7] = (__bf16)(p - (float)h);
    }
    // O^T += V^T . P^T; V^T fragments read transposed from the bf16 rows. Lane (group g, la)
    // reads rows r0 = 16 s + 4 hi + la / 4 (and r0 + 8), dims d = 32 mt + 16 (g & 1) + 4 (la & 3):
    // f(r0) = 2 (la / 4) + hi for every s, and chunk (4 mt + c0) ^ f = 4 (mt ^ f2) + (c0 ^ (f & 3)),
    // so the address is a per-lane base (one for even, one for odd mt) plus compile-time offsets.
    {
      const int g = lane >> 4, la = lane & 15;
      const int f = 2 * (la >> 2) + hi;
      const int c0 = 2 * (g & 1) + ((la & 3) >> 1);
      const int within = 8 * (la & 1);
      const int f2 = f >> 2;
      const char* base = wlat + (4 * hi + (la >> 2)) * 1024 + 16 * (c0 ^ (f & 3)) + within;
      const char* be = base + 64 * f2;          // even mt: 4 mt ^ 4 f2 = 4 mt + 4 f2
      const char* bo = base - 64 * f2;          // odd mt: 4 mt - 4 f2
#pragma unroll
      for (int mt = 0; mt < kMT; mt += 4) {
        bf16x8 av[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const char* b0 = ((mt + u) & 1 ? bo : be) + 64 * (mt + u) + 16384 * s;
            const uint2 v0 = __builtin_bit_cast(
                uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(const lds_char*)b0));
            const uint2 v1 = __builtin_bit_cast(
                uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (lds_short4*)(const lds_char*)(b0 + 8 * 1024)));
            av[u][s] = as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y));
          }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            o[mt + u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[u][s], ph[s], o[mt + u], 0, 0, 0);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            o[mt + u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[u][s], pl[s], o[mt + u], 0, 0, 0);
        }
      }
    }
    if (threadIdx.x < TK) s_code[(it + 2) % 3][threadIdx.x] = key_code_of(kl, kk2, raw2, ke);
    __builtin_amdgcn_s_waitcnt(0);   // this thread's DMA of the next tile has landed
    __syncthreads();                 // every wave is done with this tile; next tile complete
  }

  l_run += __shfl_xor(l_run, 32);
  if (__any(overflow)) atomicOr(&s_flag, 1);

  // Merge the KSW key splits of each head group through LDS (lane-local log-sum-exp merge).
  if (KSW > 1) {
    float* xo = reinterpret_cast<float*>(lds);
    for (int span = KSW / 2; span >= 1; span >>= 1) {
      const bool sender = ks >= span && ks < 2 * span;
      const bool receiver = ks < span;
      float* slot = xo + (size_t)((ks % span) * HGW + hgw) * (kMT * 16 + 2) * 64;
      if (sender) {
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) slot[(mt * 16 + i) * 64 + lane] = o[mt][i];
        slot[(kMT * 16) * 64 + lane] = m_run;
        slot[(kMT * 16 + 1) * 64 + lane] = l_run;
      }
      __syncthreads();
      if (receiver) {
        const float m2 = slot[(kMT * 16) * 64 + lane];
        const float l2 = slot[(kMT * 16 + 1) * 64 + lane];
        const float mm = fmaxf(m_run, m2);
        const float a1 = m_run == -INFINITY ? 0.f : exp2f(m_run - mm);
        const float a2 = m2 == -INFINITY ? 0.f : exp2f(m2 - mm);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          floatx16 other;
#pragma unroll
          for (int i = 0; i < 16; ++i) other[i] = slot[(mt * 16 + i) * 64 + lane];
          o[mt] = o[mt] * a1 + other * a2;
        }
        l_run = l_run * a1 + l2 * a2;
        m_run = mm;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) plan.flags[blockIdx.x] = s_flag;
  if (ks != 0) return;

  if (plan.n_split == 1) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* orow = a.out + ((int64_t)qi * a.H + head) * kDC;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(orow + 32 * mt + 8 * j + 4 * hi) =
            make_float4(o[mt][4 * j] * inv, o[mt][4 * j + 1] * inv, o[mt][4 * j + 2] * inv,
                        o[mt][4 * j + 3] * inv);
    if (a.lse != nullptr && hi == 0)
      a.lse[(int64_t)qi * a.H + head] =
          l_run > 0.f ? (m_run + __log2f(l_run)) * 0.6931471805599453f : -INFINITY;
  } else {
    const int64_t pidx = ((int64_t)qi * plan.n_split + split) * a.H + head;
    float* orow = plan.ws_o + pidx * kDC;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4*>(orow + 32 * mt + 8 * j + 4 * hi) =
            make_float4(o[mt][4 * j], o[mt][4 * j + 1], o[mt][4 * j + 2], o[mt][4 * j + 3]);
    if (hi == 0) {
      plan.ws_ml[pidx * 2] = m_run;
      plan.ws_ml[pidx * 2 + 1] = l_run;
    }
  }
}

}  // namespace

hipError_t launch_attend_bf16(const AttendArgs& a, const AttnPlan& p, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)a.Q.nq * p.head_groups * p.n_split);
  if (p.ksw == 1)
    attend_bf16_kernel<1><<<grid, 256, 0, s>>>(a, p);
  else
    attend_bf16_kernel<2><<<grid, 256, 0, s>>>(a, p);
  return hipGetLastError();
}

}  // namespace csa
