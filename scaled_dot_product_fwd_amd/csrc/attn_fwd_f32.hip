// fp32 forward of the fused attention for CDNA4 (gfx950), behind attn_fwd / attn_fwd_strided
// with dtype ATTN_F32.
//
// The article on masked multi-head attention in CUDA works in fp32 throughout (its naive and
// tiled kernels, §3-§4); this path keeps fp32 end to end: Q, K, V, the products, the softmax
// state and O are fp32, the products on v_mfma_f32_32x32x2_f32 (no rounding to 16 bits anywhere).
// The algorithm is the 16-bit kernel's (online softmax over key tiles, "Triton Cuda Attention",
// online softmax section; implicit causal / valid_len masks, GQA kv = hq / group, empty rows
// 0 / -inf), with a simpler schedule: the fp32 MFMA takes 64 cycles for 4096 flops, so the
// loop is bound by the MFMA pipe and needs no software pipelining of its own.
//
// Decomposition: one workgroup per (batch, query head, 128-query tile), 4 waves x 32 queries,
// the 16-bit kernel's XCD-aware order; 32-key K / V tiles, double-buffered in LDS by buffer DMA.
//
//   * S^T = K Q^T in k-steps of 2 head elements: lane l supplies K[key l%32][d(s, l/32)] and
//     Q[query l%32][d(s, l/32)] with d(4t + e, h) = 8t + 4h + e, so one 16-byte LDS read gives a
//     lane the K values of four k-steps, and its Q values stay in registers (D / 2 VGPRs).
//   * O^T += V^T P^T in k-steps of 2 keys: key(s, h) = 8(s/4) + 4h + s%4 is exactly the key of
//     the lane's score register s, so P enters the MFMA as the fp32 scores' exponentials
//     themselves; lane l reads V[key(s, l/32)][32u + l%32] (4 bytes).
//   * LDS rows are XOR-swizzled by 16-byte chunk: K by (row & 15) (16 rows of one read phase on
//     distinct bank slots), V by 8 * ((row >> 2) & 1) (the rows key and key + 4 that one V read
//     touches land in opposite halves of the 256-byte bank window).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "attn_common.h"

namespace attn_detail {
namespace {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kKT = 32;   // keys per tile

template <int D>
struct G32 {
  static constexpr int ROW = 4 * D;                    // bytes per row
  static constexpr int CH = D / 4;                     // 16-byte chunks per row
  static constexpr int TILE = kKT * ROW;               // bytes per K or V tile
  static constexpr int LOADS = TILE / 1024 / kWaves;   // 1 KiB DMA blocks per wave per tile
  static constexpr int RPB = 1024 / ROW;               // rows per block
  static constexpr int QT = D / 8;                     // 16-byte Q fragments per lane
  static constexpr int OT = D / 32;                    // 32-row tiles of O^T
  static constexpr int K0 = 0, K1 = TILE, V0 = 2 * TILE, V1 = 3 * TILE;
  static constexpr int LDS = 4 * TILE;
  static_assert(LOADS >= 1 && OT >= 1, "tile geometry");
  __device__ static constexpr int kswz(int r) { return r & (CH < 16 ? CH - 1 : 15); }
  // 128-byte rows (D = 32) have a single 8-chunk half: no V swizzle there.
  __device__ static constexpr int vswz(int r) { return CH >= 16 ? 8 * ((r >> 2) & 1) : 0; }
};

__device__ inline f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// DH is the tensors' head dimension; DH = 16 runs the D = 32 geometry with the missing 16-byte
// chunks of every row zero-filled (their DMA lanes fetch out of range) and never stored.
// MK: kMaskNone, or an explicit uint8 keep / fp32 additive mask (attn_fwd_masked).
template <int DH, bool CAUSAL, int MK>
__device__ __forceinline__ void fwd_f32_body(const F32Params& p) {
  constexpr int D = DH < 32 ? 32 : DH;   // geometry
  constexpr int DCH = DH / 4;            // 16-byte chunks of a row that exist
  using G = G32<D>;
  constexpr int QT = G::QT;
  constexpr int OT = G::OT;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[G::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int ql = lane & 31;

  int qt, b, hq;
  {
    const int wid = blockIdx.x;
    if (p.xcd_order) {
      const int xcd = wid & 7, local = wid >> 3;
      const int per_head = p.group * p.nqt;
      const int head_local = local / per_head;
      const int r = local - head_local * per_head;
      const int kv_head = head_local * 8 + xcd;
      const int qi = r / p.group;
      qt = CAUSAL ? p.nqt - 1 - qi : qi;
      b = kv_head / p.Hkv;
      hq = (kv_head - b * p.Hkv) * p.group + (r - qi * p.group);
    } else {
      const int BH = p.B * p.Hq;
      const int qi = wid / BH, bh = wid - qi * BH;
      qt = CAUSAL ? p.nqt - 1 - qi : qi;
      b = bh / p.Hq;
      hq = bh - b * p.Hq;
    }
  }
  const int kvh = hq / p.group;
  const int q0 = qt * kBM;
  int kv_end = p.N;
  if (p.valid_len) kv_end = min(max(p.valid_len[b], 0), p.N);
  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, q0 + kBM);
  const int ntiles = (kv_stop + kKT - 1) / kKT;
  const int qa = q0 + wave * 32;
  const int qrow = qa + ql;

  // K and V of this (batch, KV head) as buffers spanning its N rows (rows past N read as 0).
  const uint32_t krow = (uint32_t)p.ks_n * 4, vrow = (uint32_t)p.vs_n * 4;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k + b * p.ks_b + kvh * p.ks_h), (short)0, (p.N - 1) * krow + 4 * DH,
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.v + b * p.vs_b + kvh * p.vs_h), (short)0, (p.N - 1) * vrow + 4 * DH,
      kBufferFlags);
  constexpr uint32_t kNoChunk = 0x80000000u;   // past every buffer (spans stay below 2^31)
  // Block (wave * LOADS + i) of a tile holds rows [blk * RPB, +RPB); the lane writes LDS chunk
  // (lane % CH) of row (lane / CH) and fetches the global chunk its row's swizzle maps there.
  uint32_t koff[G::LOADS], voff[G::LOADS];
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const int row = (wave * G::LOADS + i) * G::RPB + lane / G::CH;
    const int kc = (lane % G::CH) ^ G::kswz(row), vc = (lane % G::CH) ^ G::vswz(row);
    koff[i] = (DCH < G::CH && kc >= DCH) ? kNoChunk : row * krow + kc * 16;
    voff[i] = (DCH < G::CH && vc >= DCH) ? kNoChunk : row * vrow + vc * 16;
  }
  auto dma = [&](int tile, int kdst, int vdst) {
    const uint32_t row0 = (uint32_t)tile * kKT;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int blk = (wave * G::LOADS + i) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(smem + kdst + blk), 16, koff[i],
                                               row0 * krow, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(smem + vdst + blk), 16, voff[i],
                                               row0 * vrow, 0, 0);
    }
  };
  if (ntiles > 0) dma(0, G::K0, G::V0);

  // Q: lane holds Q[qrow][8t + 4h .. +3] for t < QT (rows past N read row N-1, never stored),
  // times the sign of the scale (0 when the scale is 0).
  const float* qsrc = p.q + b * p.qs_b + hq * p.qs_h + min(qrow, p.N - 1) * p.qs_n + 4 * h;
  f32x4 qf[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const f32x4 x = (DCH < G::CH && 2 * t + h >= DCH) ? f32x4{} : *(const f32x4*)(qsrc + 8 * t);
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[t][e] = x[e] * p.qmul;
  }
  // LDS offsets: K fragment t of this lane (row ql, logical chunk 2t + h); V value of k-step s
  // and d-tile u: row key(s, h), column 32u + ql = chunk 8u + ql / 4 (swizzled), word ql % 4.
  uint32_t kaddr[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) kaddr[t] = ql * G::ROW + 16 * ((2 * t + h) ^ G::kswz(ql));
  auto vaddr = [&](int s, int u) -> uint32_t {
    const int key = 8 * (s >> 2) + 4 * h + (s & 3);
    return key * G::ROW + 16 * ((8 * u + (ql >> 2)) ^ G::vswz(key)) + 4 * (ql & 3);
  };

  // Explicit mask: the lane reads its query's row of the (batch, query head) plane (rows past N
  // read row N - 1, never stored) as a range-checked buffer that ends at the last row's 16-byte
  // boundary (a dword or 16-byte load that crosses the end reads as 0, which would hide keys
  // below N), for the keys of its score registers:
  // kb0 + 8g + 4h + e is byte e of word g (keep) or word 4g + e (additive). A tile's words are
  // loaded at the top of its step, before the next tile's DMA, so that their wait (after the
  // score MFMAs) leaves that DMA in flight.
  constexpr int MES = MK == kMaskKeep ? 1 : 4;        // bytes per mask element
  constexpr int MW = MK == kMaskAdd ? 16 : 4;         // mask words per lane and tile
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      MK != kMaskNone ? (void*)((const unsigned char*)p.mask + (b * p.ms_b + hq * p.ms_h) * MES)
                      : (void*)p.q,
      (short)0,
      MK != kMaskNone ? (uint32_t)((int64_t)(p.N - 1) * p.ms_n * MES + ((p.N * MES + 15) & ~15))
                      : 0u,
      kBufferFlags);
  const uint32_t moff =
      MK != kMaskNone ? (uint32_t)(min(qrow, p.N - 1) * p.ms_n + 4 * h) * MES : 0u;
  auto mask_load = [&](int tile, uint32_t (&w)[MW]) {
    const uint32_t base = moff + (uint32_t)tile * kKT * MES;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (MK == kMaskKeep) {
        w[g] = __builtin_amdgcn_raw_buffer_load_b32(mrs, base + 8 * g, 0, 0);
      } else {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(mrs, base + 32 * g, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * g + e] = x[e];
      }
    }
  };

  f32x16 acc[OT];
#pragma unroll
  for (int u = 0; u < OT; ++u) acc[u] = f32x16{};
  float m = -INFINITY;   // running maximum, log2 units
  float l = 0.f;         // this lane's part of the denominator
  const float c = p.c;

  for (int j = 0; j < ntiles; ++j) {
    const int P = j & 1;
    wait_loads_and_lds();
    __syncthreads();
    uint32_t mw[MW];
    if constexpr (MK != kMaskNone) {
      mask_load(j, mw);
      // Issued after the mask words (the scheduler may not swap them) and on every step (the
      // last one reloads its own tile into the idle buffer), so that the wait for the mask words
      // counts the same loads on every step and leaves the DMA in flight.
      __builtin_amdgcn_sched_barrier(0);
      dma(min(j + 1, ntiles - 1), P ? G::K0 : G::K1, P ? G::V0 : G::V1);
    } else if (j + 1 < ntiles) {
      dma(j + 1, P ? G::K0 : G::K1, P ? G::V0 : G::V1);
    }
    const unsigned char* kb = smem + (P ? G::K1 : G::K0);
    const unsigned char* vb = smem + (P ? G::V1 : G::V0);
    // scores of keys kb0 + 8(r/4) + 4h + r%4 for this lane's query
    f32x16 sc = f32x16{};
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const f32x4 kf = *(const f32x4*)(kb + kaddr[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sc = mfma_f32(kf[e], qf[t][e], sc);
    }
    const int kb0 = j * kKT;
    const bool full = (!CAUSAL || kb0 + kKT - 1 <= qa) && kb0 + kKT <= kv_end;
    if constexpr (MK != kMaskNone) {
      // Every tile: the additive value is folded into the raw score first, then keys hidden by
      // the mask, causality or valid_len become -inf (a non-finite value on a hidden key never
      // reaches the softmax).
      int lim = kv_end - 1 - kb0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow - kb0 - 4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int g = r >> 2, e = r & 3;
        bool vis = 8 * g + e <= lim;
        float x = sc[r];
        if constexpr (MK == kMaskKeep)
          vis = vis && ((mw[g] >> (8 * e)) & 0xffu) != 0;
        else
          x = __builtin_fmaf(__uint_as_float(mw[r]), p.mscale, x);
        sc[r] = vis ? x : -INFINITY;
      }
    } else if (!full) {
      int lim = kv_end - 1 - kb0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow - kb0 - 4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sc[r] = (8 * (r >> 2) + (r & 3) <= lim) ? sc[r] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = pair_max(mx);
    const float mn = fmaxf(m, mx * c);
    const float alpha = mn == m ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    const float mneg = m == -INFINITY ? 0.f : -m;
    float lsum = 0.f;
    float pr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c, mneg));
      lsum += pr[r];
    }
    l = l * alpha + lsum;
#pragma unroll
    for (int u = 0; u < OT; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][r] *= alpha;
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int u = 0; u < OT; ++u)
        acc[u] = mfma_f32(*(const float*)(vb + vaddr(s, u)), pr[s], acc[u]);
  }

  // The last step's reload lands before the workgroup's LDS can be handed to another.
  if constexpr (MK != kMaskNone) wait_loads_and_lds();

  // O = acc / l (0 for a row with no visible key); lane holds O[qrow][32u + 8 r4 + 4h .. +3].
  const float lt = pair_sum(l);
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.0f / lt;
  if (qrow < p.N) {
    float* orow = p.o + b * p.os_b + hq * p.os_h + qrow * p.os_n;
#pragma unroll
    for (int u = 0; u < OT; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        if (32 * u + 8 * r4 + 4 * h >= DH) continue;   // chunks past DH do not exist
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = acc[u][4 * r4 + e] * inv;
        *(f32x4*)(orow + 32 * u + 8 * r4 + 4 * h) = w;
      }
    if (p.lse && h == 0)
      p.lse[((size_t)b * p.Hq + hq) * p.N + qrow] = empty ? -INFINITY : m * kLn2 + logf(lt);
  }
}

// D = 256 holds 128 KiB of tiles in LDS (one workgroup per CU): one wave per SIMD, with the
// whole register file for its 128 Q and 128 accumulator registers.
template <int D, bool CAUSAL, int MK>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2, D > 128 ? 1 : 2)))
void attn_fwd_f32_kernel(F32Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
  fwd_f32_body<D, CAUSAL, MK>(p);
#endif
}

template <int D, bool CAUSAL, int MK>
hipError_t launch_d(const F32Params& p, hipStream_t s) {
  const int64_t nwg = (int64_t)p.B * p.Hq * p.nqt;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL, MK>), dim3((unsigned)nwg), dim3(kThreads),
                     0, s, p);
  return hipGetLastError();
}

template <int MK>
hipError_t launch_m(const F32Params& p, int D, bool causal, hipStream_t s) {
  switch (D) {
    case 16: return causal ? launch_d<16, true, MK>(p, s) : launch_d<16, false, MK>(p, s);
    case 32: return causal ? launch_d<32, true, MK>(p, s) : launch_d<32, false, MK>(p, s);
    case 256: return causal ? launch_d<256, true, MK>(p, s) : launch_d<256, false, MK>(p, s);
    case 64: return causal ? launch_d<64, true, MK>(p, s) : launch_d<64, false, MK>(p, s);
    default: return causal ? launch_d<128, true, MK>(p, s) : launch_d<128, false, MK>(p, s);
  }
}

}  // namespace

hipError_t launch_fwd_f32(const F32Params& p, int D, bool causal, int mask_type, hipStream_t s) {
  if (mask_type == ATTN_MASK_KEEP_U8) return launch_m<kMaskKeep>(p, D, causal, s);
  if (mask_type == ATTN_MASK_ADD) return launch_m<kMaskAdd>(p, D, causal, s);
  return launch_m<kMaskNone>(p, D, causal, s);
}

}  // namespace attn_detail
