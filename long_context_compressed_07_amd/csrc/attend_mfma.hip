// MFMA attention kernel for csa_attend / hca_attend on gfx950 (bf16 or fp8 cache rows of
// d_c = 512 latent + d_r = 64 RoPE dims, bf16 queries, heads in groups of 32).
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA: selected compressed rows plus the
// raw window, MQA with one KV shared by every head; HCA: dense over the m'-compressed rows) and the
// MLA section (key row = [latent; RoPE key], value row = latent); yudonglee.me "DeepSeek-V4 详解"
// 2.2 Step 4 and 2.3 Step 2. The jaylab-temp.pages.dev report (其他技术细节) gives the fp8 latent +
// bf16 RoPE cache row.
//
// Layout of the work. A workgroup is 4 wavefronts and serves one query: HGW groups of 32 heads x
// KSW splits of that query's key list (HGW * KSW = 4). Keys are staged tile by tile (32 * KSW
// keys) into LDS as fp16 rows [key][576 + 16 pad], converted exactly from bf16 or from
// (fp8 code x row scale); every wave then works on its own 32 keys of the tile:
//   S^T[32 keys x 32 heads] = K_tile . Q^T       36 x mfma_f32_32x32x16_f16, K from LDS
//                                                 (ds_read_b128), Q^T held in registers
//   softmax per head                              each lane owns one head (column of S^T), so
//                                                 the row max / sum are lane-local plus one
//                                                 exchange with lane ^ 32. The reference max of
//                                                 a head is fixed at its first non-empty tile;
//                                                 later tiles may reach 2^15 above it (fp16 P
//                                                 range), so the accumulators are never rescaled
//                                                 inside the loop. A head that would exceed the
//                                                 range flags its workgroup, and the heads it
//                                                 computed are recomputed with the fp32
//                                                 reference code (combine_kernel for key-split
//                                                 plans, fixup_kernel: the whole query).
//   O^T[512 x 32 heads] += V^T . P^T              32 x mfma, V^T fragments read transposed from
//                                                 the same LDS rows (ds_read_tr16_b64), P^T is
//                                                 the softmax output already in registers
// The KSW key splits of a head group are merged through LDS at the end (log-sum-exp merge); with
// n_split > 1 workgroups per query, partial outputs (normalised, fp16) and (m, l) go to the
// workspace and combine_kernel merges them.
//
// Precision: products in fp16 are exact for these inputs (bf16 and scaled fp8 values lie inside
// fp16's range; values below 2^-17 keep <= 2^-25 absolute error), accumulation is fp32; P is
// rounded to fp16 (relative error 2^-11) and the softmax denominator sums the rounded values.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "attend_generic.h"
#include "attend_plan.h"

namespace csa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) _Float16 lds_half;

// Transposed LDS read (gfx950 ds_read_tr16_b64): within each group of 16 lanes, lane i receives
// element i % 4 of the 8-byte chunks addressed by lanes 4 j + i / 4, j = 0..3.
__device__ __forceinline__ half4 read_tr16(const lds_half* p) {
  const short4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
  return __builtin_bit_cast(half4, v);
}

constexpr int kDC = 512;                 // latent (value) dims
constexpr int kDR = 64;                  // RoPE dims
constexpr int kD = kDC + kDR;            // key dims
constexpr int kChunks = kD / 8;          // 16-byte fp16 chunks per key row
constexpr int kRowH = kD + 16;           // LDS row stride in halfs (pad keeps reads conflict-free)
constexpr int kKSteps = kD / 16;         // k-steps of the S^T contraction
constexpr int kMT = kDC / 32;            // 32-dim output tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRange = 15.0f;          // log2 headroom of P above the reference max (fp16)

using MfmaPlan = AttnPlan;

__device__ __forceinline__ half8 cvt8_bf16(uint4 v) {
  half8 h;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[2 * i] = (_Float16)__uint_as_float(w[i] << 16);
    h[2 * i + 1] = (_Float16)__uint_as_float(w[i] & 0xffff0000u);
  }
  return h;
}

__device__ __forceinline__ half8 cvt8_e4m3(uint2 v, float s) {
  half8 h;
  const int w0 = (int)v.x, w1 = (int)v.y;
  h[0] = (_Float16)(__builtin_amdgcn_cvt_f32_fp8(w0, 0) * s);
  h[1] = (_Float16)(__builtin_amdgcn_cvt_f32_fp8(w0, 1) * s);
  h[2] = (_Float16)(__builtin_amdgcn_cvt_f32_fp8(w0, 2) * s);
  h[3] = (_Float16)(__builtin_amdgcn_cvt_f32_fp8(w0, 3) * s);
  h[4] = (_Float16)(__builtin_amdgcn_cvt_f32_fp8(w1, 0) * s);
  h[5] = (_Float16)(__builtin_amdgcn_cvt_f32_fp8(w1, 1) * s);
  h[6] = (_Float16)(__builtin_amdgcn_cvt_f32_fp8(w1, 2) * s);
  h[7] = (_Float16)(__builtin_amdgcn_cvt_f32_fp8(w1, 3) * s);
  return h;
}

// Staging of a key tile (32 * KSW keys) into LDS as fp16, in batches of 32 keys. In a batch,
// thread t owns key row t / 8 and its 16-byte chunks 9 (t % 8) .. 9 (t % 8) + 8 (of the 72 chunks
// of a 576-dim row: 64 latent chunks, then 8 RoPE chunks), so it needs one row address and nine
// loads, all in flight at once. batch_load only issues the loads; batch_store converts and writes.
// s_key holds, per tile key, the store (bit 30) and row, or -1 for an empty slot (zeros).
constexpr int kBatch = kChunks / 8;   // 9 chunks per thread

struct Batch {
  uint4 v[kBatch];
  float sc;
};

template <int KVT>
__device__ __forceinline__ void batch_load(const AttendArgs& a, int64_t b, const int* s_key,
                                           int bi, Batch& B) {
  const int r = 32 * bi + (threadIdx.x >> 3);
  const int c0 = kBatch * (threadIdx.x & 7);
  const int code = s_key[r];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) B.v[j] = make_uint4(0u, 0u, 0u, 0u);
  B.sc = 0.f;
  if (code < 0) return;
  const Store& st = (code >> 30) ? a.raw : a.ent;
  const int64_t row = b * st.rows + (code & 0x3fffffff);
  const char* crow = static_cast<const char*>(st.c) + row * st.ld_c * (KVT == CSA_BF16 ? 2 : 1);
  const char* rrow = static_cast<const char*>(st.r) + row * st.ld_r * 2;
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int c = c0 + j;
    if (c < kDC / 8) {
      if (KVT == CSA_BF16) {
        B.v[j] = *reinterpret_cast<const uint4*>(crow + c * 16);
      } else {
        const uint2 u = *reinterpret_cast<const uint2*>(crow + c * 8);
        B.v[j].x = u.x;
        B.v[j].y = u.y;
      }
    } else {
      B.v[j] = *reinterpret_cast<const uint4*>(rrow + (c - kDC / 8) * 16);
    }
  }
  if (KVT == CSA_E4M3) B.sc = st.scale[row];
}

template <int KVT>
__device__ __forceinline__ void batch_store(const Batch& B, int bi, _Float16* tile) {
  const int r = 32 * bi + (threadIdx.x >> 3);
  const int c0 = kBatch * (threadIdx.x & 7);
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int c = c0 + j;
    const half8 h = (KVT == CSA_E4M3 && c < kDC / 8)
                        ? cvt8_e4m3(make_uint2(B.v[j].x, B.v[j].y), B.sc)
                        : cvt8_bf16(B.v[j]);
    *reinterpret_cast<half8*>(tile + r * kRowH + c * 8) = h;
  }
}

// Code of key kk of the query's key list for s_key: row | store << 30, or -1.
__device__ __forceinline__ int key_code(const AttendArgs& a, const KeyList& kl, int64_t kk,
                                        int64_t ke) {
  if (kk >= ke) return -1;
  int src;
  const int64_t row = key_row(a, kl, kk, src);
  return row >= 0 ? (int)row | (src << 30) : -1;
}

template <int KVT, int KSW>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attend_mfma_kernel(AttendArgs a, MfmaPlan plan) {
  constexpr int HGW = 4 / KSW;
  constexpr int kTileBytes = 32 * KSW * kRowH * 2;
  constexpr int kMergeBytes = KSW > 1 ? (KSW / 2) * HGW * (kMT * 16 + 2) * 64 * 4 : 0;
  __shared__ __attribute__((aligned(16))) char lds[kTileBytes > kMergeBytes ? kTileBytes
                                                                             : kMergeBytes];
  __shared__ int s_key[2][32 * KSW];
  __shared__ int s_flag;
  _Float16* tile = reinterpret_cast<_Float16*>(lds);
  if (threadIdx.x == 0) s_flag = 0;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hgw = w % HGW;
  const int ks = w / HGW;
  const int hi = lane >> 5;                       // lane half
  const int per_q = plan.head_groups * plan.n_split;
  const int item = xcd_item();
  const int qi = item / per_q;
  const int rem = item - qi * per_q;
  const int hgrp = rem / plan.n_split;
  const int split = rem - hgrp * plan.n_split;
  const int h0 = (hgrp * HGW + hgw) * 32;
  const int head = h0 + (lane & 31);

  const KeyList kl = make_key_list(a, qi);
  const int64_t per_split = (kl.total + plan.n_split - 1) / plan.n_split;
  const int64_t kb = (int64_t)split * per_split;
  const int64_t ke = kb + per_split < kl.total ? kb + per_split : kl.total;

  // Q^T operand fragments: head `head`, dims 16 s + 8 hi + [0, 8).
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)qi * a.H + head) * kD;
  half8 qb[kKSteps];
#pragma unroll
  for (int s = 0; s < kKSteps; ++s)
    qb[s] = cvt8_bf16(*reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * hi));

  floatx16 o[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) o[mt] = floatx16{};
  float m_run = -INFINITY;   // reference max of the scaled logits (log2 units), per head
  float l_run = 0.f;         // running sum of this lane's half of the keys
  bool overflow = false;
  const float cscale = a.sm_scale * kLog2e;

  const _Float16* wtile = tile + (32 * ks) * kRowH;        // this wave's 32 keys
  constexpr int TK = 32 * KSW;                              // keys per tile
  // Prologue: codes of tiles 0 and 1, tile 0 staged.
  if (threadIdx.x < TK) {
    s_key[0][threadIdx.x] = key_code(a, kl, kb + threadIdx.x, ke);
    s_key[1][threadIdx.x] = key_code(a, kl, kb + TK + threadIdx.x, ke);
  }
  __syncthreads();
  if (kb < ke) {
#pragma unroll
    for (int bi = 0; bi < KSW; ++bi) {
      Batch B;
      batch_load<KVT>(a, kl.b, s_key[0], bi, B);
      batch_store<KVT>(B, bi, tile);
    }
  }
  __syncthreads();
  int cur = 0;
  for (int64_t t0 = kb; t0 < ke; t0 += TK) {
    const bool has_next = t0 + TK < ke;
    // Prefetch: the first 32 keys of the next tile (registers) and the codes of the tile after.
    Batch pre;
    if (has_next) batch_load<KVT>(a, kl.b, s_key[cur ^ 1], 0, pre);
    int code2 = -1;
    if (threadIdx.x < TK) code2 = key_code(a, kl, t0 + 2 * TK + threadIdx.x, ke);
    const int* keys = s_key[cur];

    // S^T = K . Q^T for this wave's 32 keys.
    floatx16 acc = floatx16{};
    const _Float16* arow = wtile + (lane & 31) * kRowH + 8 * hi;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const half8 av = *reinterpret_cast<const half8*>(arow + 16 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qb[s], acc, 0, 0, 0);
    }
    // Scale, mask empty slots, tile max per head (lane-local over 16 keys, then lane ^ 32).
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 32 * ks + 8 * (i >> 2) + 4 * hi + (i & 3);
      acc[i] = keys[key] >= 0 ? acc[i] * cscale : -INFINITY;
      tmax = fmaxf(tmax, acc[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // The reference max is set by the first non-empty tile (the accumulators are still zero
    // then); afterwards it never moves and P may reach 2^kRange. A head that would exceed that
    // marks the workgroup for the fp32 fixup pass.
    m_run = m_run == -INFINITY ? tmax : m_run;
    overflow |= tmax > m_run + kRange;
    // P^T in fp16, already in the B-operand layout of the next contraction: k-step s of lane
    // half hi covers keys 16 s + 4 hi + [0,4) and 16 s + 8 + 4 hi + [0,4).
    half8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = acc[i] == -INFINITY ? 0.f : exp2f(fminf(acc[i] - m_run, kRange));
      const _Float16 ph = (_Float16)p;
      l_run += (float)ph;
      pb[i >> 3][i & 7] = ph;
    }
    // O^T += V^T . P^T; V^T fragments come transposed from the fp16 rows.
    const int g = lane >> 4;
    const int la = lane & 15;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const int col = 32 * mt + 16 * (g & 1) + 4 * (la & 3);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int r0 = 16 * s + 4 * hi + (la >> 2);
        const lds_half* base = (const lds_half*)wtile;
        const half4 v0 = read_tr16(base + r0 * kRowH + col);
        const half4 v1 = read_tr16(base + (r0 + 8) * kRowH + col);
        const half8 av = half8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, pb[s], o[mt], 0, 0, 0);
      }
    }
    __syncthreads();   // every wave is done with this tile and its codes
    if (has_next) {
      batch_store<KVT>(pre, 0, tile);
#pragma unroll
      for (int bi = 1; bi < KSW; ++bi) {
        Batch B;
        batch_load<KVT>(a, kl.b, s_key[cur ^ 1], bi, B);
        batch_store<KVT>(B, bi, tile);
      }
    }
    if (threadIdx.x < TK) s_key[cur][threadIdx.x] = code2;
    __syncthreads();
    cur ^= 1;
  }

  // Both lane halves hold the same head; their sums cover different keys.
  l_run += __shfl_xor(l_run, 32);
  if (__any(overflow)) atomicOr(&s_flag, 1);

  // Merge the KSW key splits of each head group through LDS (lane-local log-sum-exp merge).
  if (KSW > 1) {
    float* xo = reinterpret_cast<float*>(lds);      // per slot: [kMT*16 + 2][64] floats
    for (int span = KSW / 2; span >= 1; span >>= 1) {
      // waves with ks in [span, 2 span) send to ks - span.
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
  if (threadIdx.x == 0) plan.flags[item] = s_flag;
  if (ks != 0) return;

  // Output rows: lane owns head `head`, dims 32 mt + 8 j + 4 hi + [0, 4).
  if (plan.n_split == 1) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* orow = a.out + ((int64_t)qi * a.H + head) * kDC;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float4 v = make_float4(o[mt][4 * j] * inv, o[mt][4 * j + 1] * inv,
                               o[mt][4 * j + 2] * inv, o[mt][4 * j + 3] * inv);
        *reinterpret_cast<float4*>(orow + 32 * mt + 8 * j + 4 * hi) = v;
      }
    if (a.lse != nullptr && hi == 0)
      a.lse[(int64_t)qi * a.H + head] =
          l_run > 0.f ? (m_run + __log2f(l_run)) * 0.6931471805599453f : -INFINITY;
  } else {
    const int64_t pidx = ((int64_t)qi * plan.n_split + split) * a.H + head;
    _Float16* orow = plan.ws_o + pidx * kDC;
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_partial4(orow + 32 * mt + 8 * j + 4 * hi, o[mt][4 * j], o[mt][4 * j + 1],
                       o[mt][4 * j + 2], o[mt][4 * j + 3], inv);
    if (hi == 0) {
      plan.ws_ml[pidx * 2] = m_run;
      plan.ws_ml[pidx * 2 + 1] = l_run;
    }
  }
}

// Log-sum-exp merge of n_split partials, fused with the overflow fixup of split plans: one block of
// four waves per (query, four heads), wave w merging head h0 + w with one lane per 8 dims. Partial
// s holds o_s / l_s: out = sum_s (l_s 2^(m_s - mx)) (o_s / l_s) / sum_s l_s 2^(m_s - mx), taken in
// batches of 8 splits whose loads are all issued before use, with a running maximum. When a
// workgroup that computed these heads (their head group, any key split) flagged a head whose
// logits left the fp16 range of P, the block recomputes the four heads with the fp32 reference
// code instead.
constexpr int kCombHeads = kGenThreads / kWave;

__global__ void __launch_bounds__(kGenThreads) combine_kernel(AttendArgs a, MfmaPlan plan) {
  __shared__ float smem[generic_smem_bytes(kD) / sizeof(float)];
  const int per_q = a.H / kCombHeads;
  const int qi = blockIdx.x / per_q;
  const int h0 = (blockIdx.x - qi * per_q) * kCombHeads;
  const int hgrp = h0 / (a.H / plan.head_groups);
  const int t = threadIdx.x;
  int flag = 0;
  for (int s = t; s < plan.n_split; s += kGenThreads)
    flag |= plan.flags[((int64_t)qi * plan.head_groups + hgrp) * plan.n_split + s];
  if (__syncthreads_or(flag)) {
    for (int h = h0; h < h0 + kCombHeads; ++h) attend_generic_one(a, qi, h, smem);
    return;
  }
  merge_partials8(a, plan, qi, h0 + t / kWave, (t & (kWave - 1)) * 8);
}

// Plans without key splits: recompute, with the fp32 reference code, every query one of whose
// workgroups flagged a head whose logits left the fp16 range of P. Nearly always a no-op: block b
// owns queries b + gridDim.x j, each thread checks one of them at a time, and the block recomputes
// the flagged ones.
__global__ void __launch_bounds__(kGenThreads) fixup_kernel(AttendArgs a, MfmaPlan plan) {
  __shared__ float smem[generic_smem_bytes(kD) / sizeof(float)];
  __shared__ int s_q[kGenThreads];
  __shared__ int s_n;
  const int per_q = plan.head_groups * plan.n_split;
  const int64_t stride = (int64_t)gridDim.x * kGenThreads;
  for (int64_t q0 = blockIdx.x; q0 < a.Q.nq; q0 += stride) {
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    const int64_t qi = q0 + (int64_t)threadIdx.x * gridDim.x;
    if (qi < a.Q.nq) {
      int any = 0;
      for (int i = 0; i < per_q; ++i) any |= plan.flags[qi * per_q + i];
      if (any) s_q[atomicAdd(&s_n, 1)] = (int)qi;
    }
    __syncthreads();
    const int n = s_n;
    for (int j = 0; j < n; ++j)
      for (int h = 0; h < a.H; ++h) attend_generic_one(a, s_q[j], h, smem);
    __syncthreads();
  }
}

// Work decomposition (the split rule is make_plan's). bf16 caches with a multiple of 64 heads
// take the two-role DMA kernel (attend_pp.hip): one workgroup per query and group of 64 heads.
// fp8 caches with a multiple of 128 heads take the fp8 DMA kernel (attend_fp8.hip): one workgroup
// per query and group of 128 heads. Everything else takes the fp16-staging kernel here: 4 head
// groups sharing each staged tile (ksw 1), 2 head groups x 2 key halves (ksw 2) or one 32-head
// group x 4 key quarters (ksw 4), by the head count. Each query's keys may also be split over
// workgroups (n_split), merged by combine_kernel in split order.
enum PlanKind { kPlanStaging = 0, kPlanBf16 = 1, kPlanF8 = 2 };

// Split rule. The number of key splits per query depends only on the call's longest key list
// (max_keys: k + window for CSA, the entry rows for HCA), the call (CSA or HCA) and the kernel,
// never on the number of queries, and the merge takes the splits in a fixed order: a query's outputs are bitwise the same
// whatever batch it is in and wherever in the batch it sits (deepseek.csdn.net "一文搞懂
// DeepSeek", V4 的其他升级: deterministic, batch-invariant kernels). keys_per_split is the
// kernel's granularity. fp8 (the decode cache): 288 keys for csa_attend, so that a 1152-key list
// takes 4 splits (64 sequences: one workgroup per CU; 3, 5, 6 and 8 splits measured 2-25% slower
// per decode step), and 512 keys for hca_attend, whose dense lists are long: 16 splits for 8192
// entries, so that the hybrid decode's HCA layer (8 queries, 128 workgroups) leaves CUs for the
// CSA layer it runs beside (28 splits took every CU: 150 against 128 us per hybrid step; 13-20
// splits measured alike). bf16 (the prefill path, many queries per call): 8192, so that the
// prefill workloads run unsplit. At most 64 splits.
int splits_by_keys(int64_t max_keys, int64_t keys_per_split) {
  const int64_t ns = max_keys / keys_per_split;
  return (int)(ns < 1 ? 1 : (ns > 64 ? 64 : ns));
}

MfmaPlan make_plan(int H, int64_t max_keys, int kind, bool dense) {
  MfmaPlan p{};
  const int groups32 = H / 32;
  if (kind == kPlanBf16 && groups32 % 2 == 0) {
    // 64-head workgroups with the two wave roles (attend_pp.hip) for every even number of 32-head
    // groups (measured on 128 heads: 8.3 vs 9.2 ms for the HCA prefill against a 4-wave kernel
    // with 128 heads per workgroup, although each key tile is loaded once per 64 heads).
    p.pp = 1;
    p.rg = 2;
    p.head_groups = groups32 / p.rg;
    p.n_split = splits_by_keys(max_keys, 8192);
    return p;
  }
  if (kind == kPlanF8 && groups32 % 4 == 0) {
    p.f8_dma = 1;
    p.rg = 4;
    p.head_groups = groups32 / 4;
    p.n_split = splits_by_keys(max_keys, dense ? 512 : 288);
    return p;
  }
  // fp16-staging kernel: as many 32-head groups per staged tile as the head count allows.
  p.ksw = groups32 % 4 == 0 ? 1 : (groups32 % 2 == 0 ? 2 : 4);
  p.head_groups = groups32 / (4 / p.ksw);
  p.n_split = splits_by_keys(max_keys, 1024);
  return p;
}

// Which kernel a call takes.
int plan_kind(const AttendArgs& a) {
  const bool win = !a.dense && a.window > 0 && a.raw.c != nullptr;
  if (a.ent.dtype == CSA_BF16 && (!win || a.raw.dtype == CSA_BF16)) return kPlanBf16;
  if (a.ent.dtype == CSA_E4M3 && (!win || a.raw.dtype == CSA_E4M3) && a.ent.ld_c % 16 == 0 &&
      (!win || a.raw.ld_c % 16 == 0) &&
      (reinterpret_cast<uintptr_t>(a.ent.c) & 15) == 0 &&
      (!win || (reinterpret_cast<uintptr_t>(a.raw.c) & 15) == 0))
    return kPlanF8;
  return kPlanStaging;
}

}  // namespace

bool attend_mfma_supported(const AttendArgs& a) {
  return a.q_dtype == CSA_BF16 && (a.ent.dtype == CSA_BF16 || a.ent.dtype == CSA_E4M3) &&
         a.ent.d_c == kDC && a.ent.d_r == kDR && a.H % 32 == 0 &&
         (a.ent.ld_c % 8 == 0) && (a.ent.ld_r % 8 == 0) &&
         (a.dense || a.window == 0 || (a.raw.ld_c % 8 == 0 && a.raw.ld_r % 8 == 0)) &&
         a.ent.rows < (1 << 30) && (a.dense || a.raw.rows < (1 << 30));
}

// Workspace: partial outputs when a query spans several workgroups, then one flag per workgroup.
// The dtype is not part of the workspace query, so this covers both plans.
static size_t plan_partial_bytes(const MfmaPlan& p, int nq, int H) {
  return p.n_split > 1 ? (size_t)nq * p.n_split * H * (kDC * sizeof(_Float16) + 2 * sizeof(float))
                       : 0;
}
static size_t plan_flag_bytes(const MfmaPlan& p, int nq) {
  return (size_t)nq * p.head_groups * p.n_split * sizeof(int);
}
size_t attend_mfma_workspace(int nq, int H, int64_t max_keys, bool dense) {
  // The dtypes are not part of the workspace query: cover every plan kind.
  size_t part = 0, flags = 0;
  for (int kind = 0; kind < 3; ++kind) {
    const MfmaPlan p = make_plan(H, max_keys, kind, dense);
    part = std::max(part, plan_partial_bytes(p, nq, H));
    flags = std::max(flags, plan_flag_bytes(p, nq));
  }
  return part + flags;
}

// Optional timing of the main attention kernel alone (slot 0: CSA, slot 1: HCA): a HIP event
// pair recorded on the launch stream around it. The state is guarded by a mutex; while timing is
// off (the normal case) an attention call reads one atomic flag and touches nothing else.
namespace {
struct KernelTiming {
  int cap = 0;
  int n[2] = {0, 0};
  hipEvent_t ev[2][2][kTimingCap];   // [slot][start / end][launch]
};
KernelTiming g_timing;
std::mutex g_timing_mu;
std::atomic<int> g_timing_on{0};
}  // namespace

hipError_t kernel_timing_enable(int cap) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on.store(0, std::memory_order_release);
  for (int slot = 0; slot < 2; ++slot)
    for (int j = 0; j < 2; ++j)
      for (int i = 0; i < g_timing.cap; ++i) (void)hipEventDestroy(g_timing.ev[slot][j][i]);
  g_timing.cap = 0;
  g_timing.n[0] = g_timing.n[1] = 0;
  if (cap < 0 || cap > kTimingCap) return hipErrorInvalidValue;
  for (int i = 0; i < cap; ++i) {
    for (int slot = 0; slot < 2; ++slot)
      for (int j = 0; j < 2; ++j) {
        hipError_t e = hipEventCreate(&g_timing.ev[slot][j][i]);
        if (e != hipSuccess) return e;
      }
    g_timing.cap = i + 1;
  }
  g_timing_on.store(cap > 0 ? 1 : 0, std::memory_order_release);
  return hipSuccess;
}

hipError_t kernel_timing_read(int slot, double* ms, int* n) {
  *ms = 0.0;
  *n = 0;
  if (slot < 0 || slot > 1) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (int i = 0; i < g_timing.n[slot]; ++i) {
    hipError_t e = hipEventSynchronize(g_timing.ev[slot][1][i]);
    if (e != hipSuccess) return e;
    float t = 0.f;
    e = hipEventElapsedTime(&t, g_timing.ev[slot][0][i], g_timing.ev[slot][1][i]);
    if (e != hipSuccess) return e;
    *ms += t;
  }
  *n = g_timing.n[slot];
  g_timing.n[slot] = 0;
  return hipSuccess;
}

int timing_start(int slot, hipStream_t s) {
  if (!g_timing_on.load(std::memory_order_acquire)) return -1;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (g_timing.n[slot] >= g_timing.cap) return -1;
  const int i = g_timing.n[slot]++;
  (void)hipEventRecord(g_timing.ev[slot][0][i], s);
  return i;
}

void timing_stop(int slot, int i, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (i < g_timing.cap) (void)hipEventRecord(g_timing.ev[slot][1][i], s);
}

hipError_t launch_attend_mfma(const AttendArgs& a, int64_t max_keys, hipStream_t s) {
  MfmaPlan p = make_plan(a.H, max_keys, plan_kind(a), a.dense);
  if (p.n_split > 1) {
    p.ws_o = static_cast<_Float16*>(a.ws);
    p.ws_ml = reinterpret_cast<float*>(p.ws_o + (size_t)a.Q.nq * p.n_split * a.H * kDC);
  }
  p.flags = reinterpret_cast<int*>(static_cast<char*>(a.ws) + plan_partial_bytes(p, a.Q.nq, a.H));
  const unsigned grid = (unsigned)((int64_t)a.Q.nq * p.head_groups * p.n_split);
  const bool fp8 = a.ent.dtype == CSA_E4M3;
  const int tslot = a.dense ? 1 : 0;
  const int timed = timing_start(tslot, s);
  if (p.pp) {
    (void)launch_attend_pp(a, p, s);
  } else if (p.f8_dma) {
    (void)launch_attend_fp8(a, p, s);
  } else switch (p.ksw * 2 + (fp8 ? 1 : 0)) {
    case 2: attend_mfma_kernel<CSA_BF16, 1><<<grid, 256, 0, s>>>(a, p); break;
    case 3: attend_mfma_kernel<CSA_E4M3, 1><<<grid, 256, 0, s>>>(a, p); break;
    case 4: attend_mfma_kernel<CSA_BF16, 2><<<grid, 256, 0, s>>>(a, p); break;
    case 5: attend_mfma_kernel<CSA_E4M3, 2><<<grid, 256, 0, s>>>(a, p); break;
    case 8: attend_mfma_kernel<CSA_BF16, 4><<<grid, 256, 0, s>>>(a, p); break;
    default: attend_mfma_kernel<CSA_E4M3, 4><<<grid, 256, 0, s>>>(a, p); break;
  }
  hipError_t e = hipGetLastError();
  if (timed >= 0) timing_stop(tslot, timed, s);   // closes the pair even after a failed launch
  if (e != hipSuccess) return e;
  if (p.n_split > 1) {
    combine_kernel<<<(unsigned)((int64_t)a.Q.nq * (a.H / kCombHeads)), kGenThreads, 0, s>>>(a, p);
  } else {
    fixup_kernel<<<(unsigned)(a.Q.nq < 1024 ? a.Q.nq : 1024), kGenThreads, 0, s>>>(a, p);
  }
  return hipGetLastError();
}

}  // namespace csa
