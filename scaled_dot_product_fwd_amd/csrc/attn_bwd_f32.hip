// fp32 backward of the fused attention for CDNA4 (gfx950), behind attn_bwd / attn_bwd_strided
// with dtype ATTN_F32.
//
// Same gradients and the same two-kernel, atomic-free split as the 16-bit backward (attn_bwd.hip;
// tiny_flash_attn_triton.py keeps the forward's L for its backward pass): with
// P = exp(scale * q.k - L) on the visible keys and D_i = sum_d dO[i,d] O[i,d],
//
//   dP = dO V^T,  dS = P o (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO,
//
// dK and dV summed over the query heads of each KV head. Everything stays fp32 (the article on
// masked multi-head attention in CUDA works in fp32 throughout): the products run on
// v_mfma_f32_32x32x2_f32 (64 cycles for 4096 flops), so both loops are bound by the MFMA pipe
// and are written for clarity rather than software-pipelined.
//
//   * dQ kernel: one workgroup per (batch, query head, 128-query tile), 4 waves x 32 queries, the
//     forward's order. Q and dO rows of the wave's queries stay in registers; D and L * log2(e)
//     go to the workspace for the second kernel. Per 32-key tile (K and V double-buffered in LDS
//     by buffer DMA): S^T = K Q^T and dP^T = V dO^T (lane = query, k-steps of 2 head elements
//     d(4t + e, h) = 8t + 4h + e, so one 16-byte LDS read feeds four k-steps), P and dS on the
//     VALU, dQ^T += K^T dS^T in k-steps of 2 keys: key(s, h) = 8(s/4) + 4h + s%4 is the key of
//     the lane's score register s, so dS enters the MFMA as it is, and the lane reads the single
//     K element [key(s, h)][32u + lane % 32].
//   * dK/dV kernel: one workgroup per (batch, KV head, 128-key tile), 4 waves x 32 keys. K and V
//     rows of the wave's keys stay in registers; 32-query tiles of Q, dO, L2 and D of every query
//     head of the group stream through LDS: S = Q K^T and dP = dO V^T (lane = key), P and dS,
//     dV^T += dO^T P and dK^T += Q^T dS with single-element reads of dO and Q.
//   * Tiles read both as 16-byte row fragments and as single elements use one XOR swizzle of
//     their 16-byte chunks, swz(r) = (r & 15) ^ (8 * ((r >> 2) & 1)) for rows of 256 bytes or
//     more: the 16 rows of a row-fragment read phase land on 16 distinct bank slots, and the
//     two rows key and key + 4 of an element read on opposite halves of the 256-byte bank
//     window. (128-byte rows, D = 32, keep a 2-way conflict on the element reads.)
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "attn.h"
#include "attn_common.h"

namespace attn_detail {
namespace {

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kT = 32;   // keys per tile (dQ kernel), queries per iteration (dK/dV kernel)
constexpr uint32_t kNoChunk = 0x80000000u;   // DMA voffset past every buffer: zero-fill

template <int D>
struct B32 {
  static constexpr int ROW = 4 * D;                    // bytes per row
  static constexpr int CH = D / 4;                     // 16-byte chunks per row
  static constexpr int TILE = kT * ROW;                // bytes per 32-row tile
  static constexpr int LOADS = TILE / 1024 / kWaves;   // 1 KiB DMA blocks per wave per tile
  static constexpr int RPB = 1024 / ROW;               // rows per block
  static constexpr int QT = D / 8;                     // 16-byte row fragments per lane
  static constexpr int RA = QT < 8 ? QT : 8;           // distinct row-fragment base offsets
  static constexpr int OT = D / 32;                    // 32-row output tiles
  static_assert(LOADS >= 1 && OT >= 1, "tile geometry");
  __device__ static constexpr int swz(int r) {
    return D >= 64 ? ((r & 15) ^ (((r >> 2) & 1) << 3)) : ((r >> 1) & 7);
  }
};

__device__ inline f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ inline float lse_log2_f32(float L) { return L == -INFINITY ? 0.f : L * kLog2e; }

// Per-lane LDS offsets of a 32-row tile stored with B32<D>::swz.
//   * Row fragment t (row lane % 32, logical chunk 2t + h): ra[t & 7] + 256 * (t >> 3).
//   * Element (row 8 sq + 4h + e, column 32u + lane % 32):
//       (8 sq + e) * ROW + 128 * (u & ~1) + eb[(u ^ sq) & 1][e]
//     (for rows of 256 bytes or more the chunk is 8 (u ^ (sq & 1) ^ h) + ((lane % 32) / 4 ^
//     (4h + e)); for 128-byte rows u = 0 and the chunk is (lane % 32) / 4 ^ (4 (sq & 1) + 2h +
//     e / 2)).
template <int D>
struct Offsets {
  uint32_t ra[B32<D>::RA];
  uint32_t eb[2][4];
  __device__ void init(int lane) {
    using G = B32<D>;
    const int h = lane >> 5, ql = lane & 31, a = ql >> 2;
#pragma unroll
    for (int t = 0; t < G::RA; ++t) ra[t] = ql * G::ROW + 16 * ((2 * t + h) ^ G::swz(ql));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (D >= 64) {
        const uint32_t pe = 4 * h * G::ROW + 16 * (a ^ (4 * h + e)) + 4 * (ql & 3);
        eb[0][e] = pe + 128 * h;
        eb[1][e] = pe + 128 * (1 - h);
      } else {
#pragma unroll
        for (int x = 0; x < 2; ++x)
          eb[x][e] = 4 * h * G::ROW + 16 * (a ^ ((4 * x + 2 * h + (e >> 1)) & 7)) + 4 * (ql & 3);
      }
    }
  }
  __device__ uint32_t row(int t) const { return ra[t & 7] + 256 * (t >> 3); }
  __device__ uint32_t elem(int s, int u) const {
    const int sq = s >> 2, e = s & 3;
    return (8 * sq + e) * B32<D>::ROW + 128 * (u & ~1) + eb[(u ^ sq) & 1][e];
  }
};

// 16-byte DMA lane offsets of a 32-row tile: block (wave * LOADS + i) holds rows
// [blk * RPB, +RPB); the lane writes LDS chunk (lane % CH) of row (lane / CH) and fetches the
// global chunk that the row's swizzle maps there. Chunks past the head dimension DH fetch
// nothing (zeros).
template <int D, int DH>
__device__ inline uint32_t dma_lane(int wave, int i, int lane, uint32_t rowbytes, bool rel) {
  using G = B32<D>;
  const int r = (wave * G::LOADS + i) * G::RPB + lane / G::CH;
  const int c = (lane % G::CH) ^ G::swz(r);
  if (DH / 4 < G::CH && c >= DH / 4) return kNoChunk;
  // rel: row offset relative to the block's first row (the block's rows go in the scalar offset)
  return (uint32_t)(rel ? lane / G::CH : r) * rowbytes + c * 16;
}

// Store a wave's 32 x DH block held transposed (acc[u][4 r4 + e] is element
// 32 (U0 + u) + 8 r4 + 4h + e of row `row`, for the UN 32-column tiles from U0), times `mul`.
template <int D, int DH, int U0 = 0, int UN = B32<D>::OT>
__device__ inline void store_row(const f32x16 (&acc)[UN], float mul, float* dst, int h) {
#pragma unroll
  for (int u = 0; u < UN; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int col = 32 * (U0 + u) + 8 * r4 + 4 * h;
      if (col >= DH) continue;
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = acc[u][4 * r4 + e] * mul;
      *(f32x4*)(dst + col) = w;
    }
}

// D = 256 does not fit its row fragments and accumulators in the register file: each kernel
// runs as NP launches (PART 0 .. NP-1), each recomputing the scores and accumulating, then
// storing, 1/NP of the output columns. PART -1: one launch, all columns.
template <int D, int PART, int NP>
struct Cols {
  static constexpr int UN = PART < 0 ? B32<D>::OT : B32<D>::OT / NP;   // 32-column tiles held
  static constexpr int U0 = PART < 0 ? 0 : PART * UN;                 // first of them
};
constexpr int kPartsDq = 2;     // dQ kernel at D = 256: Q, dO rows + half of dQ
constexpr int kPartsDkdv = 4;   // dK/dV kernel at D = 256: K, V rows + a quarter of dK, dV

// The forward's explicit mask (MK: kMaskKeep uint8, kMaskAdd fp32; kMaskNone for none): the
// (batch, query head) plane as a range-checked buffer ending at its last row's 16-byte boundary
// (a load that crosses a buffer's end reads as 0, which would hide keys below N).
template <int MK>
__device__ inline __amdgpu_buffer_rsrc_t mask_plane(const F32BwdParams& p, int b, int hq) {
  constexpr int MES = MK == kMaskKeep ? 1 : 4;
  return __builtin_amdgcn_make_buffer_rsrc(
      MK != kMaskNone ? (void*)((const unsigned char*)p.mask + (b * p.ms_b + hq * p.ms_h) * MES)
                      : (void*)p.q,
      (short)0,
      MK != kMaskNone ? (uint32_t)((int64_t)(p.N - 1) * p.ms_n * MES + ((p.N * MES + 15) & ~15))
                      : 0u,
      kBufferFlags);
}

// ------------------------------------------------------------------------------------------
// dQ (and D, L2)
// ------------------------------------------------------------------------------------------
template <int DH, bool CAUSAL, int MK, int PART>
__device__ __forceinline__ void dq_f32_body(const F32BwdParams& p) {
  constexpr int D = DH < 32 ? 32 : DH;   // geometry; DH = 16 zero-fills half of every row
  constexpr int DCH = DH / 4;
  using G = B32<D>;
  constexpr int QT = G::QT, OT = G::OT;
  constexpr int K0 = 0, K1 = G::TILE, V0 = 2 * G::TILE, V1 = 3 * G::TILE;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[4 * G::TILE];

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
  const int bh = b * p.Hq + hq;
  const int kvh = hq / p.group;
  const int q0 = qt * kBM;
  int kv_end = p.N;
  if (p.valid_len) kv_end = min(max(p.valid_len[b], 0), p.N);
  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, q0 + kBM);
  const int ntiles = (kv_stop + kT - 1) / kT;
  const int qa = q0 + wave * 32;
  const int qrow = qa + ql;
  const int qr = min(qrow, p.N - 1);

  const uint32_t krow = (uint32_t)p.ks_n * 4, vrow = (uint32_t)p.vs_n * 4;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k + b * p.ks_b + kvh * p.ks_h), (short)0, (p.N - 1) * krow + 4 * DH,
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.v + b * p.vs_b + kvh * p.vs_h), (short)0, (p.N - 1) * vrow + 4 * DH,
      kBufferFlags);
  uint32_t kdma[G::LOADS], vdma[G::LOADS];
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    kdma[i] = dma_lane<D, DH>(wave, i, lane, krow, false);
    vdma[i] = dma_lane<D, DH>(wave, i, lane, vrow, false);
  }
  auto dma = [&](int tile, int kdst, int vdst) {
    const uint32_t row0 = (uint32_t)tile * kT;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int blk = (wave * G::LOADS + i) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(smem + kdst + blk), 16, kdma[i],
                                               row0 * krow, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(smem + vdst + blk), 16, vdma[i],
                                               row0 * vrow, 0, 0);
    }
  };
  if (ntiles > 0) dma(0, K0, V0);

  // Q and dO of this lane's row: element 8t + 4h + e in register qf[t][e] (the B operand of
  // k-step 4t + e); D = rowsum(dO o O) from the same layout of O.
  const float* qsrc = p.q + b * p.qs_b + hq * p.qs_h + qr * p.qs_n + 4 * h;
  const float* gsrc = p.dout + b * p.gs_b + hq * p.gs_h + qr * p.gs_n + 4 * h;
  const float* osrc = p.o + b * p.os_b + hq * p.os_h + qr * p.os_n + 4 * h;
  f32x4 qf[QT], gf[QT];
  float dsum = 0.f;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const bool ok = DCH == G::CH || 2 * t + h < DCH;
    qf[t] = ok ? *(const f32x4*)(qsrc + 8 * t) : f32x4{};
    gf[t] = ok ? *(const f32x4*)(gsrc + 8 * t) : f32x4{};
    const f32x4 ov = ok ? *(const f32x4*)(osrc + 8 * t) : f32x4{};
#pragma unroll
    for (int e = 0; e < 4; ++e) dsum = __builtin_fmaf(gf[t][e], ov[e], dsum);
  }
  const float delta = pair_sum(dsum);
  const float L2 = lse_log2_f32(p.lse[(size_t)bh * p.N + qr]);
  if (h == 0 && qrow < p.N) {
    p.delta[(size_t)bh * p.N + qrow] = delta;
    p.lse2[(size_t)bh * p.N + qrow] = L2;
  }
#pragma unroll
  for (int t = 0; t < QT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[t][e] *= p.qmul;

  Offsets<D> off;
  off.init(lane);
  constexpr int UN = Cols<D, PART, kPartsDq>::UN, U0 = Cols<D, PART, kPartsDq>::U0;
  f32x16 acc[UN];
#pragma unroll
  for (int u = 0; u < UN; ++u) acc[u] = f32x16{};
  const float c = p.c;
  // Explicit mask: the words of this lane's query row for the keys of its score registers,
  // kb0 + 8g + 4h + e = byte e of word g (keep) or word 4g + e (additive).
  constexpr int MES = MK == kMaskKeep ? 1 : 4;
  constexpr int MW = MK == kMaskAdd ? 16 : 4;
  const __amdgpu_buffer_rsrc_t mrs = mask_plane<MK>(p, b, hq);
  const uint32_t moff = MK != kMaskNone ? (uint32_t)(qr * p.ms_n + 4 * h) * MES : 0u;

  auto step = [&](auto bufc, int j) {
    constexpr int P = decltype(bufc)::value;
    wait_loads_and_lds();
    __syncthreads();
    uint32_t mw[MW];
    if constexpr (MK != kMaskNone) {
      const uint32_t base = moff + (uint32_t)j * kT * MES;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if constexpr (MK == kMaskKeep) {
          mw[g] = __builtin_amdgcn_raw_buffer_load_b32(mrs, base + 8 * g, 0, 0);
        } else {
          const auto x = __builtin_amdgcn_raw_buffer_load_b128(mrs, base + 32 * g, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) mw[4 * g + e] = x[e];
        }
      }
      // The DMA goes out after the mask words (no reordering) and on every step (the last one
      // reloads its own tile into the idle buffer), so that the wait for the words leaves it in
      // flight.
      __builtin_amdgcn_sched_barrier(0);
      dma(min(j + 1, ntiles - 1), P ? K0 : K1, P ? V0 : V1);
    } else if (j + 1 < ntiles) {
      dma(j + 1, P ? K0 : K1, P ? V0 : V1);
    }
    const unsigned char* kb = smem + (P ? K1 : K0);
    const unsigned char* vb = smem + (P ? V1 : V0);
    // S^T and dP^T: lane holds keys kb0 + 8(r/4) + 4h + r%4 of its query
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const f32x4 kf = *(const f32x4*)(kb + off.row(t));
      const f32x4 vf = *(const f32x4*)(vb + off.row(t));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc = mfma_f32(kf[e], qf[t][e], sc);
        dp = mfma_f32(vf[e], gf[t][e], dp);
      }
    }
    // P and dS; per-element tests only on tiles that reach past the wave's causal diagonal or
    // valid_len (a hidden element's P may be inf: the select removes it).
    const int kb0 = j * kT;
    const bool full = (!CAUSAL || kb0 + kT - 1 <= qa) && kb0 + kT <= kv_end;
    float ds[16];
    if constexpr (MK != kMaskNone) {
      // every tile: the additive value enters the score, hidden keys get dS = 0
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
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -L2));
        ds[r] = vis ? pv * (dp[r] - delta) : 0.f;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ds[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], c, -L2)) * (dp[r] - delta);
    }
    if (MK == kMaskNone && !full) {
      int lim = kv_end - 1 - kb0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow - kb0 - 4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r) ds[r] = (8 * (r >> 2) + (r & 3) <= lim) ? ds[r] : 0.f;
    }
    // dQ^T += K^T dS^T over 16 k-steps of 2 keys
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int u = 0; u < UN; ++u)
        acc[u] = mfma_f32(*(const float*)(kb + off.elem(s, U0 + u)), ds[s], acc[u]);
  };
  for (int j = 0; j < ntiles; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) step(std::integral_constant<int, 1>{}, j + 1);
  }
  // the last step's reload lands before the workgroup's LDS can be handed to another
  if constexpr (MK != kMaskNone) wait_loads_and_lds();
  if (qrow < p.N)
    store_row<D, DH, U0, UN>(acc, p.scale, p.dq + b * p.dqs_b + hq * p.dqs_h + qrow * p.dqs_n,
                             h);
}

// ------------------------------------------------------------------------------------------
// dK, dV
// ------------------------------------------------------------------------------------------
template <int DH, bool CAUSAL, int MK, int PART>
__device__ __forceinline__ void dkdv_f32_body(const F32BwdParams& p) {
  constexpr int D = DH < 32 ? 32 : DH;
  constexpr int DCH = DH / 4;
  using G = B32<D>;
  constexpr int QT = G::QT, OT = G::OT;
  constexpr int LD = 2048;                 // 1 KiB slots for L2 and D of one tile
  constexpr int BUF = 2 * G::TILE + LD;    // one buffer: Q, dO, L2, D
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int ql = lane & 31;

  // (batch, KV head, 128-key tile): each XCD owns whole KV heads, in blocks of two, longest key
  // tiles first under causal masking (the 16-bit dK/dV kernel's order).
  int kt, b, kvh, sp;
  {
    // consecutive workgroups of one XCD take the `split` parts of one key tile
    if (p.xcd_order) {
      const int xcd = blockIdx.x & 7, local0 = blockIdx.x >> 3;
      const int local = local0 / p.split;
      sp = local0 - local * p.split;
      const int hpx = (p.B * p.Hkv) >> 3;
      const int blk = (hpx & 1) ? 1 : 2;
      const int pair = local / (blk * p.nkt);
      const int r = local - pair * blk * p.nkt;
      kt = r / blk;
      const int head_local = pair * blk + (r - kt * blk);
      const int kv_head = head_local * 8 + xcd;
      b = kv_head / p.Hkv;
      kvh = kv_head - b * p.Hkv;
    } else {
      const int wid = blockIdx.x / p.split;
      sp = blockIdx.x - wid * p.split;
      const int BK = p.B * p.Hkv;
      kt = wid / BK;
      const int bk = wid - kt * BK;
      b = bk / p.Hkv;
      kvh = bk - b * p.Hkv;
    }
  }
  const int k0 = kt * kBM;
  const int kw = k0 + wave * 32;
  const int key = kw + ql;
  int kv_end = p.N;
  if (p.valid_len) kv_end = min(max(p.valid_len[b], 0), p.N);

  constexpr int UN = Cols<D, PART, kPartsDkdv>::UN, U0 = Cols<D, PART, kPartsDkdv>::U0;
  f32x16 dk[UN], dv[UN];
#pragma unroll
  for (int u = 0; u < UN; ++u) dk[u] = dv[u] = f32x16{};

  const int qstart = CAUSAL ? k0 : 0;
  const int ntq = k0 < kv_end ? (p.N - qstart + kT - 1) / kT : 0;
  // this workgroup's share [it0, it0 + iters) of the key tile's ntq * group iterations
  const int total = ntq * p.group;
  const int it0 = (int)((int64_t)total * sp / p.split);
  const int iters = (int)((int64_t)total * (sp + 1) / p.split) - it0;

  if (iters > 0) {
    // K (times the scale's sign, 0 for scale 0) and V of this lane's key: B operands of S and dP.
    f32x4 kf[QT], vf[QT];
    {
      const int kr = min(key, p.N - 1);
      const float* ksrc = p.k + b * p.ks_b + kvh * p.ks_h + kr * p.ks_n + 4 * h;
      const float* vsrc = p.v + b * p.vs_b + kvh * p.vs_h + kr * p.vs_n + 4 * h;
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const bool ok = DCH == G::CH || 2 * t + h < DCH;
        kf[t] = ok ? *(const f32x4*)(ksrc + 8 * t) : f32x4{};
        vf[t] = ok ? *(const f32x4*)(vsrc + 8 * t) : f32x4{};
#pragma unroll
        for (int e = 0; e < 4; ++e) kf[t][e] *= p.qmul;
      }
    }
    const uint32_t qrowb = (uint32_t)p.qs_n * 4, growb = (uint32_t)p.gs_n * 4;
    uint32_t qoff[G::LOADS], goff[G::LOADS];
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      qoff[i] = dma_lane<D, DH>(wave, i, lane, qrowb, true);
      goff[i] = dma_lane<D, DH>(wave, i, lane, growb, true);
    }
    // DMA of the iteration over query head kvh * group + g, queries q0 .. q0+31, into buffer
    // `buf`: Q and dO tiles, then L2 (wave 0) and D (wave 1), one dword per query row.
    auto dma = [&](int g, int q0, int buf) {
      const int hq = kvh * p.group + g;
      const int bh = b * p.Hq + hq;
      const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.q + b * p.qs_b + hq * p.qs_h), (short)0, (p.N - 1) * qrowb + 4 * DH,
          kBufferFlags);
      const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.dout + b * p.gs_b + hq * p.gs_h), (short)0, (p.N - 1) * growb + 4 * DH,
          kBufferFlags);
      unsigned char* base = smem + buf * BUF;
#pragma unroll
      for (int i = 0; i < G::LOADS; ++i) {
        const int blk = wave * G::LOADS + i;
        const uint32_t r0 = (uint32_t)(q0 + blk * G::RPB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void*)(base + blk * 1024), 16,
                                                 qoff[i], r0 * qrowb, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ors, (lds_void*)(base + G::TILE + blk * 1024),
                                                 16, goff[i], r0 * growb, 0, 0);
      }
      if (wave < 2) {
        const float* src = wave == 0 ? p.lse2 : p.delta;
        const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(src + (size_t)bh * p.N), (short)0, (uint32_t)p.N * 4, kBufferFlags);
        // lanes 32..63 are out of range and write zeros to bytes 128..255 of the 1 KiB slot
        const uint32_t loff = lane < kT ? (uint32_t)(q0 + lane) * 4 : 0x7ffffff0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            lrs, (lds_void*)(base + 2 * G::TILE + wave * 1024), 4, loff, 0, 0, 0);
      }
    };

    Offsets<D> off;
    off.init(lane);
    const float c = p.c;
    // query tile major from the last tile down, query head minor (as the 16-bit kernel: the
    // key-tile workgroups of a KV head read each Q / dO tile at about the same time)
    const int qlast = qstart + (ntq - 1) * kT;
    const int t0 = it0 / p.group;
    const int g0 = it0 - t0 * p.group, qs0 = qlast - t0 * kT;
    int g_cur = g0, q_cur = qs0, g_nxt = g0, q_nxt = qs0;
    auto advance = [&](int& g, int& q0) {
      if (++g == p.group) { g = 0; q0 -= kT; }
    };
    dma(g_nxt, q_nxt, 0);
    advance(g_nxt, q_nxt);

    // Explicit mask: element (query q0 + 8(r/4) + 4h + r%4, this lane's key) per score register.
    constexpr int MES = MK == kMaskKeep ? 1 : 4;
    const uint32_t mrowb = MK != kMaskNone ? (uint32_t)(p.ms_n * MES) : 0u;
    const uint32_t mcol = (uint32_t)key * MES;   // keys past N are hidden below
    auto step = [&](auto bufc, int it) {
      constexpr int buf = decltype(bufc)::value;
      wait_loads_and_lds();
      __syncthreads();
      const int q0 = q_cur;
      uint32_t mw[16];
      if constexpr (MK != kMaskNone) {
        const __amdgpu_buffer_rsrc_t mrs = mask_plane<MK>(p, b, kvh * p.group + g_cur);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t moff = (uint32_t)(q0 + 8 * (r >> 2) + 4 * h + (r & 3)) * mrowb + mcol;
          if constexpr (MK == kMaskKeep)
            mw[r] = __builtin_amdgcn_raw_buffer_load_b8(mrs, moff, 0, 0);
          else
            mw[r] = __builtin_amdgcn_raw_buffer_load_b32(mrs, moff, 0, 0);
        }
        // The DMA goes out after the mask words (no reordering) and on every step (the last one
        // reloads its own tile into the idle buffer), so that the wait for the words leaves it
        // in flight.
        __builtin_amdgcn_sched_barrier(0);
        const bool more = it + 1 < iters;   // one DMA call without a branch around it
        dma(more ? g_nxt : g_cur, more ? q_nxt : q0, buf ^ 1);
        if (more) advance(g_nxt, q_nxt);
      } else if (it + 1 < iters) {
        dma(g_nxt, q_nxt, buf ^ 1);
        advance(g_nxt, q_nxt);
      }
      advance(g_cur, q_cur);
      const unsigned char* qb = smem + buf * BUF;
      const unsigned char* ob = qb + G::TILE;
      const float* lb = (const float*)(qb + 2 * G::TILE);
      const float* db = (const float*)(qb + 2 * G::TILE + 1024);
      // S = Q K^T and dP = dO V^T: lane holds query rows q0 + 8(r/4) + 4h + r%4 of its key
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const f32x4 qv = *(const f32x4*)(qb + off.row(t));
        const f32x4 ov = *(const f32x4*)(ob + off.row(t));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = mfma_f32(qv[e], kf[t][e], s);
          dp = mfma_f32(ov[e], vf[t][e], dp);
        }
      }
      // P and dS: every element is tested only where the tile touches the causal diagonal,
      // valid_len or the end of the sequence (a hidden element's P may be inf; the select
      // removes it).
      const bool full = (!CAUSAL || q0 >= kw + 31) && kw + 32 <= kv_end && q0 + kT <= p.N;
      float pr[16], ds[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int qi0 = 8 * r4 + 4 * h;
        const f32x4 lv = *(const f32x4*)(lb + qi0);
        const f32x4 dv4 = *(const f32x4*)(db + qi0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          float x = s[r];
          if constexpr (MK == kMaskAdd) x = __builtin_fmaf(__uint_as_float(mw[r]), p.mscale, x);
          pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -lv[e]));
          if (MK != kMaskNone || !full) {
            const int qi = q0 + qi0 + e;
            bool vis = (!CAUSAL || key <= qi) && key < kv_end && qi < p.N;
            if constexpr (MK == kMaskKeep) vis = vis && mw[r] != 0;
            pr[r] = vis ? pr[r] : 0.f;
          }
          ds[r] = pr[r] * (dp[r] - dv4[e]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over 16 k-steps of 2 queries
#pragma unroll
      for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          dv[u] = mfma_f32(*(const float*)(ob + off.elem(k, U0 + u)), pr[k], dv[u]);
          dk[u] = mfma_f32(*(const float*)(qb + off.elem(k, U0 + u)), ds[k], dk[u]);
        }
    };
    for (int it = 0; it < iters; it += 2) {
      step(std::integral_constant<int, 0>{}, it);
      if (it + 1 < iters) step(std::integral_constant<int, 1>{}, it + 1);
    }
    wait_loads_and_lds();
  }
  if (key < p.N) {
    if (p.split > 1) {
      // fp32 partial sums of this part, added in part order by the reduction kernel
      const size_t plane = (size_t)p.B * p.Hkv * p.N * DH;
      float* pk = p.part + (size_t)sp * plane + (((size_t)b * p.Hkv + kvh) * p.N + key) * DH;
      store_row<D, DH, U0, UN>(dk, p.scale, pk, h);
      store_row<D, DH, U0, UN>(dv, 1.0f, pk + (size_t)p.split * plane, h);
    } else {
      store_row<D, DH, U0, UN>(dk, p.scale,
                               p.dk + b * p.dks_b + kvh * p.dks_h + key * p.dks_n, h);
      store_row<D, DH, U0, UN>(dv, 1.0f, p.dv + b * p.dvs_b + kvh * p.dvs_h + key * p.dvs_n,
                               h);
    }
  }
}

// D = 128 keeps 192 (dQ) and 256 (dK/dV) registers of row fragments and accumulators per lane:
// one wave per SIMD with the whole register file. Smaller head dims run two.
template <int D, bool CAUSAL, int MK, int PART>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D > 64 ? 1 : 2, D > 64 ? 1 : 2)))
void attn_bwd_f32_dq_kernel(F32BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  dq_f32_body<D, CAUSAL, MK, PART>(p);
#endif
}

template <int D, bool CAUSAL, int MK, int PART>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D > 64 ? 1 : 2, D > 64 ? 1 : 2)))
void attn_bwd_f32_dkdv_kernel(F32BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  dkdv_f32_body<D, CAUSAL, MK, PART>(p);
#endif
}

// The dQ launches (which also write D and L2) precede the dK/dV launches that read them.
template <int D, bool CAUSAL, int MK>
hipError_t launch_d(const F32BwdParams& p, hipStream_t s) {
  const int64_t nq = (int64_t)p.B * p.Hq * p.nqt;
  const int64_t nk = (int64_t)p.B * p.Hkv * p.nkt * p.split;
  if constexpr (D > 128) {
    hipLaunchKernelGGL((attn_bwd_f32_dq_kernel<D, CAUSAL, MK, 0>), dim3((unsigned)nq),
                       dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL((attn_bwd_f32_dq_kernel<D, CAUSAL, MK, 1>), dim3((unsigned)nq),
                       dim3(kThreads), 0, s, p);
    static_assert(kPartsDq == 2 && kPartsDkdv == 4, "launches below");
  } else {
    hipLaunchKernelGGL((attn_bwd_f32_dq_kernel<D, CAUSAL, MK, -1>), dim3((unsigned)nq),
                       dim3(kThreads), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D > 128) {
    hipLaunchKernelGGL((attn_bwd_f32_dkdv_kernel<D, CAUSAL, MK, 0>), dim3((unsigned)nk),
                       dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL((attn_bwd_f32_dkdv_kernel<D, CAUSAL, MK, 1>), dim3((unsigned)nk),
                       dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL((attn_bwd_f32_dkdv_kernel<D, CAUSAL, MK, 2>), dim3((unsigned)nk),
                       dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL((attn_bwd_f32_dkdv_kernel<D, CAUSAL, MK, 3>), dim3((unsigned)nk),
                       dim3(kThreads), 0, s, p);
  } else {
    hipLaunchKernelGGL((attn_bwd_f32_dkdv_kernel<D, CAUSAL, MK, -1>), dim3((unsigned)nk),
                       dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

template <int MK>
hipError_t launch_m(const F32BwdParams& p, int D, bool causal, hipStream_t s) {
  switch (D) {
    case 16: return causal ? launch_d<16, true, MK>(p, s) : launch_d<16, false, MK>(p, s);
    case 32: return causal ? launch_d<32, true, MK>(p, s) : launch_d<32, false, MK>(p, s);
    case 64: return causal ? launch_d<64, true, MK>(p, s) : launch_d<64, false, MK>(p, s);
    case 256: return causal ? launch_d<256, true, MK>(p, s) : launch_d<256, false, MK>(p, s);
    default: return causal ? launch_d<128, true, MK>(p, s) : launch_d<128, false, MK>(p, s);
  }
}

}  // namespace

hipError_t launch_bwd_f32(const F32BwdParams& p, int D, bool causal, int mask_type,
                          hipStream_t s) {
  if (mask_type == ATTN_MASK_KEEP_U8) return launch_m<kMaskKeep>(p, D, causal, s);
  if (mask_type == ATTN_MASK_ADD) return launch_m<kMaskAdd>(p, D, causal, s);
  return launch_m<kMaskNone>(p, D, causal, s);
}

}  // namespace attn_detail
