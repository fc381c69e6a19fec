// Backward of the fused attention forward for CDNA4 (gfx950), behind attn_bwd in attn.h.
//
// What it computes: the gradients of the forward output O with respect to Q, K and V for an
// upstream gradient dO, using the forward's log-sum-exp L (tiny_flash_attn_triton.py keeps L
// for its backward pass; the forward stores it in base e). With the weights recomputed per tile as
// P = exp(scale * q.k - L) on the visible keys (the same causal / valid_len masks as the
// forward), and D_i = sum_d dO[i,d] * O[i,d]:
//
//   dP = dO V^T,   dS = P o (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO,
//
// with dK and dV summed over the query heads of each KV head (grouped-query attention, the
// "Triton Cuda Attention" page's GQA section). Two kernels, launched in this order on the
// caller's stream:
//
//   * bwd_dq: one workgroup per (batch, query head, 128-query tile), 4 waves x 32 queries, the
//     forward's decomposition. Each wave holds its Q and dO fragments in registers, computes
//     D = rowsum(dO o O) and stores it with L * log2(e) in the caller's workspace for the
//     second kernel, then streams
//     64-key K/V tiles through LDS: S^T = K Q^T and dP^T = V dO^T on MFMA (lane = query, as in
//     the forward), P and dS on the VALU, and dQ^T += K^T dS^T with K^T read through
//     ds_read_b64_tr_b16. dQ is written once (no atomics).
//   * bwd_dkdv: one workgroup per (batch, KV head, 128-key tile; under causal masking a pair of
//     tiles of equal total work), 4 waves x 32 keys. Each wave keeps its keys' K fragments in
//     registers and their V rows in LDS, and streams 32-query tiles of Q, dO, L * log2(e) and D
//     of every query head of the group (only queries at or after the tile's first key under
//     causal masking): S = Q K^T and dP = dO V^T (lane = key), P and dS on the VALU,
//     dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read through ds_read_b64_tr_b16. dK
//     and dV are written once.
//
// Inputs are [B, H, N, D] tensors of one 16-bit type given by (batch, head, row) strides with
// contiguous rows (contiguous tensors are the default); dQ, dK, dV are written in that type
// through strides of their own (fp32 accumulation, round to nearest even). P and dS are rounded
// to the input type before they enter an MFMA, as the forward rounds P.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "attn.h"
#include "attn_common.h"

namespace {

using namespace attn_detail;

constexpr int kQT = 32;   // queries per iteration of the dK/dV kernel
// DMA voffset of a lane whose row chunk does not exist (head dims below 64): past every buffer
// (the host keeps each span and scalar row offset below 2^31 bytes), so the range check writes
// zeros to LDS.
constexpr uint32_t kNoChunk = 0x80000000u;

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;    // workspace row 0: D = rowsum(dO o O)
  float* lse2;     // workspace row 1: L * log2(e) (0 for rows with no visible key)
  const int32_t* valid_len;
  int B, Hq, Hkv, N;
  int group;       // Hq / Hkv
  int nqt;         // ceil(N / kBM): query tiles of the dQ kernel
  int nkt;         // ceil(N / kBM): key tiles of the dK/dV kernel
  int xcd_order;   // 1: KV heads divide evenly over the 8 XCDs
  float c;         // |scale| * log2(e)
  float scale;     // the signed scale (dQ and dK carry it)
  uint32_t qsign;  // 0x80008000 when scale < 0: one operand of the scores is negated instead
  uint32_t qmask;  // 0 when scale == 0 (all scores are 0; c is 1)
  // Element strides (batch, head, row) of Q, K, V, O, dO, dQ, dK, dV; rows are contiguous.
  int64_t qs_b, qs_h, qs_n;
  int64_t ks_b, ks_h, ks_n;
  int64_t vs_b, vs_h, vs_n;
  int64_t os_b, os_h, os_n;
  int64_t gs_b, gs_h, gs_n;
  int64_t dqs_b, dqs_h, dqs_n;
  int64_t dks_b, dks_h, dks_n;
  int64_t dvs_b, dvs_h, dvs_n;
  // Explicit mask (kernels with MK != kMaskNone): element strides (batch, query head, query row)
  const void* mask;
  int64_t ms_b, ms_h, ms_n;
  float mscale;    // log2(e) / c: an additive mask value in raw score units
  // Split of each key tile's (query head, query tile) iterations over `split` workgroups
  // (1: none). With split > 1 the dK/dV kernel writes fp32 partial sums (dK already scaled)
  // to part[2][split][B][Hkv][N][DH] and bwd_reduce adds them in split order.
  int split;
  float* part;
  // 1: under causal masking each dK/dV workgroup takes key tiles i and nkt - 1 - i (see
  // bwd_pairs); 0: one key tile each, longest first
  int pair;
};

// The 4 keys 8g + 4h .. +3 of one mask row as read from a slot: uint8 bytes (keep) or 16-bit
// values of the input type (additive), element e of the group.
template <int DT, int MK>
__device__ inline bool mask_keep(const uint32_t (&w)[2], int e) {
  return MK != kMaskKeep || ((w[0] >> (8 * e)) & 0xffu) != 0;
}
template <int DT, int MK>
__device__ inline float mask_add(const uint32_t (&w)[2], int e) {
  if constexpr (MK != kMaskAdd) {
    return 0.f;
  } else {
    const uint32_t bits = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
    return DT == ATTN_BF16 ? __uint_as_float(bits << 16)
                           : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  }
}

// Row value of the log-sum-exp in log2 units; an empty row (L = -inf) has only hidden keys, and
// 0 keeps exp2(-inf - 0) = 0 there instead of NaN.
__device__ inline float lse_log2(float L) { return L == -INFINITY ? 0.f : L * kLog2e; }

// Round 16 products dS (or P) of one lane, in the forward's key order, into the two 16-bit
// operands of an MFMA k-step: block s holds elements 8s .. 8s+7.
template <int DT>
__device__ inline u32x4 pack8(const float (&x)[16], int s) {
  f32x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = x[8 * s + e];
  return Mfma<DT>::pack(v);
}

// Head-dimension parts: at D = 256 the backward's accumulators (dQ, or dK and dV) of a whole
// row do not fit beside the operands, so each kernel runs twice, accumulating the columns
// [128 p, 128 p + 128) of part p and recomputing S and dP; smaller head dims run one part.
template <int D>
struct Parts {
  static constexpr int NP = D > 128 ? 2 : 1;    // parts
  static constexpr int OT = Geo<D>::OT / NP;    // 32-column accumulator tiles per part
};

// Write a wave's 32 x D block, held transposed in acc (acc[u][4 r4 + e] is element
// d = 32 (U0 + u) + 8 r4 + 4h + e of row ql; U0 = PART * Parts<D>::OT), as rows of `dst` (rows
// `rs` elements apart; DH <= D elements each: the 16-byte chunks past DH, and those of other
// parts, are not written) through the wave's LDS staging area `ost` (32 * ROW bytes). Rows at
// or past n are not written.
template <int DT, int D, int DH = D, int PART = 0>
__device__ inline void store_rows(const f32x16 (&acc)[Parts<D>::OT], float mul,
                                  unsigned char* ost, uint16_t* dst, int64_t rs, int row0, int n,
                                  int lane) {
  using G = Geo<D>;
  using M = Mfma<DT>;
  constexpr int NT = Parts<D>::OT, U0 = PART * NT;
  const int h = lane >> 5, ql = lane & 31;
#pragma unroll
  for (int u = 0; u < NT; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int c = 4 * (U0 + u) + r4;
      const uint32_t w0 = (uint32_t)M::round1(acc[u][4 * r4 + 0] * mul) |
                          ((uint32_t)M::round1(acc[u][4 * r4 + 1] * mul) << 16);
      const uint32_t w1 = (uint32_t)M::round1(acc[u][4 * r4 + 2] * mul) |
                          ((uint32_t)M::round1(acc[u][4 * r4 + 3] * mul) << 16);
      *(u32x2*)(ost + ql * G::ROW + 16 * (c ^ (ql & (G::CH - 1))) + 8 * h) = u32x2{w0, w1};
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int RPI = 64 / G::CH;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / G::CH;
    const int cc = lane % G::CH;
    const u32x4 v = *(const u32x4*)(ost + r * G::ROW + 16 * (cc ^ (r & (G::CH - 1))));
    const bool mine = Parts<D>::NP == 1 || (cc >= 4 * U0 && cc < 4 * (U0 + NT));
    if (row0 + r < n && mine && (DH == D || cc < DH / 8))
      *(u32x4*)(dst + (row0 + r) * rs + 8 * cc) = v;
  }
}

// Write one row of a wave's transposed fp32 block (acc[u][4 r4 + e] is element 32 (U0 + u) +
// 8 r4 + 4h + e of the lane's row) times `mul` to `dst` (DH <= D elements; chunks past DH are
// skipped).
template <int D, int DH, int PART = 0>
__device__ inline void store_part(const f32x16 (&acc)[Parts<D>::OT], float mul, float* dst,
                                  int h) {
  constexpr int U0 = PART * Parts<D>::OT;
#pragma unroll
  for (int u = 0; u < Parts<D>::OT; ++u)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * (U0 + u) + 8 * r4 + 4 * h;
      if (d >= DH) continue;
      f32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = acc[u][4 * r4 + e] * mul;
      *(f32x4*)(dst + d) = w;
    }
}

// Sum of the split parts of dK and dV in part order, rounded once to the output type.
struct ReduceParams {
  const float* part;
  void* dk;
  void* dv;
  int B, Hkv, N, DH, split;
  int64_t dks_b, dks_h, dks_n;
  int64_t dvs_b, dvs_h, dvs_n;
};

template <int DT>
__global__ __launch_bounds__(256) void attn_bwd_reduce_kernel(ReduceParams p) {
  const int C = p.DH / 4;   // 4-element chunks per row
  const int64_t rows = (int64_t)p.B * p.Hkv * p.N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * C) return;
  const int64_t row = i / C;
  const int c = (int)(i - row * C);
  const int n = (int)(row % p.N);
  const int64_t bk = row / p.N;
  const int kvh = (int)(bk % p.Hkv), b = (int)(bk / p.Hkv);
  const size_t plane = (size_t)rows * p.DH;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const float* src = p.part + (size_t)which * p.split * plane + (size_t)row * p.DH + 4 * c;
    f32x4 acc = *(const f32x4*)src;
    for (int s = 1; s < p.split; ++s) {
      const f32x4 x = *(const f32x4*)(src + (size_t)s * plane);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += x[e];
    }
    const int64_t off = which == 0 ? b * p.dks_b + kvh * p.dks_h + n * p.dks_n
                                   : b * p.dvs_b + kvh * p.dvs_h + n * p.dvs_n;
    void* dst = which == 0 ? p.dk : p.dv;
    if constexpr (DT == ATTN_F32) {
      *(f32x4*)((float*)dst + off + 4 * c) = acc;
    } else {
      using M = Mfma<DT>;
      const uint32_t w0 = (uint32_t)M::round1(acc[0]) | ((uint32_t)M::round1(acc[1]) << 16);
      const uint32_t w1 = (uint32_t)M::round1(acc[2]) | ((uint32_t)M::round1(acc[3]) << 16);
      *(u32x2*)((uint16_t*)dst + off + 4 * c) = u32x2{w0, w1};
    }
  }
}

// Lane offsets of ds_read_b64_tr_b16 reads of a transposed 32 x 16 operand from a row-major tile
// stored with Geo<D>::bswz: lane 16g + jj reads row 4(g/2) + jj/4 (+16 per k-step, +8 for the
// second 4 rows), columns 32u + 16(g%2) + 4(jj%4) .. +3 (the forward's V^T read).
template <int D>
__device__ inline uint32_t tr_offset(int lane, int u) {
  using G = Geo<D>;
  const int g = lane >> 4, jj = lane & 15;
  const int row = 4 * (g >> 1) + (jj >> 2);
  return row * G::ROW + 16 * ((4 * u + 2 * (g & 1) + ((jj & 3) >> 1)) ^ G::bswz(row)) +
         8 * (jj & 1);
}

// The 8 values of a k-step: rows from `off` (a tr_offset plus whole 16-row steps) and the same
// columns 8 rows further down. bswz(r + 8) = bswz(r) ^ 2, so the second read's chunk is the
// first's with bit 1 flipped: byte offset ^ 32.
__device__ inline u32x4 tr_frag(const unsigned char* tile, uint32_t off, int rows8) {
  const u32x2 lo = lds_read_tr16(tile + off);
  const u32x2 hi = lds_read_tr16(tile + ((off ^ 32u) + rows8));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ------------------------------------------------------------------------------------------
// dQ (and D)
// ------------------------------------------------------------------------------------------
// DH is the tensors' head dimension; DH < 64 runs the D = 64 geometry with the missing 16-byte
// chunks of every row zero (out-of-range DMA lanes, zero registers) and never stored.
template <int DT, int DH, bool CAUSAL, int MK, int PART>
__device__ __forceinline__ void bwd_dq_body(const BwdParams& p) {
  constexpr int D = DH < 64 ? 64 : DH;
  constexpr int DCH = DH / 8;
  using G = Geo<D>;
  using MG = MaskGeo<MK>;
  constexpr int MOFF = G::LDS;   // per-wave mask slots follow the K/V tiles
  using M = Mfma<DT>;
  constexpr int KSTEPS = G::KSTEPS;
  constexpr int OT = Parts<D>::OT;          // dQ^T tiles of this part
  constexpr int U0 = PART * OT;             // its first
  // K0 K1 V0 V1, 64-key tiles. K is stored with bswz (read both as rows and transposed), V
  // with kswz (read as rows).
  __shared__ __attribute__((aligned(1024))) unsigned char smem[G::LDS + kWaves * MG::WB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int ql = lane & 31;

  // Work: (batch, query head, 128-query tile), the forward's order: each XCD owns whole KV heads
  // and takes them one after the other, the query heads of one KV head side by side (they read
  // the same K and V tiles from L2) and the longest tiles first under causal masking.
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
  const int ntiles = (kv_stop + kBN - 1) / kBN;
  const int qa = q0 + wave * 32;
  const int qrow = qa + ql;
  const int qr = min(qrow, p.N - 1);

  // K and V of this (batch, KV head) as buffers spanning its N rows (rows past N read as 0).
  const uint32_t krow = (uint32_t)p.ks_n * 2, vrow = (uint32_t)p.vs_n * 2;   // bytes
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k + b * p.ks_b + kvh * p.ks_h), (short)0, (p.N - 1) * krow + 2 * DH,
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.v + b * p.vs_b + kvh * p.vs_h), (short)0, (p.N - 1) * vrow + 2 * DH,
      kBufferFlags);
  uint32_t kdma[G::LOADS], vdma[G::LOADS];
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const int r = (wave * G::LOADS + i) * G::RPB + lane / G::CH;
    const int kc = (lane % G::CH) ^ G::bswz(r), vc = (lane % G::CH) ^ G::kswz(r);
    kdma[i] = (DCH < G::CH && kc >= DCH) ? kNoChunk : r * krow + kc * 16;
    vdma[i] = (DCH < G::CH && vc >= DCH) ? kNoChunk : r * vrow + vc * 16;
  }
  auto dma = [&](int tile, int kdst, int vdst) {
    const uint32_t row0 = (uint32_t)tile * kBN;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int blk = (wave * G::LOADS + i) * 1024;
      dma16(krs, smem + kdst + blk, kdma[i], row0 * krow);
      dma16(vrs, smem + vdst + blk, vdma[i], row0 * vrow);
    }
  };

  // Explicit mask: this wave's rows qa .. qa+31 of the (batch, query head) mask matrix, the 64
  // keys of a tile per row, in the wave's LDS slot one tile ahead (the forward's scheme: the
  // step's wait covers the DMA, the slot is refilled right after it has been read).
  const uint32_t mrow = MK != kMaskNone ? (uint32_t)(p.ms_n * MG::ES) : 0;
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      MK != kMaskNone ? (void*)((const unsigned char*)p.mask + (b * p.ms_b + hq * p.ms_h) * MG::ES)
                      : (void*)p.q,
      (short)0, MK != kMaskNone ? (p.N - 1) * mrow + ((p.N * MG::ES + 15) & ~15) : 0,
      kBufferFlags);
  uint32_t moff = 0;
  if constexpr (MK != kMaskNone) {
    const int r = lane / MG::CPR;
    moff = (uint32_t)(qa + r) * mrow + 16 * ((lane % MG::CPR) ^ MG::mswz(r));
  }
  auto mask_dma = [&](int tile) {
    if constexpr (MK != kMaskNone) {
#pragma unroll
      for (int i = 0; i < MG::LOADS; ++i)
        dma16(mrs, smem + MOFF + wave * MG::WB + i * 1024, moff,
              (uint32_t)tile * MG::RB + (uint32_t)(i * MG::RPL) * mrow);
    }
  };

  // Fragment offsets: K rows (A of S^T), V rows (A of dP^T), K^T (A of dQ^T).
  uint32_t kaddr[KSTEPS], vaddr[KSTEPS], taddr[OT];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    kaddr[ks] = ql * G::ROW + 16 * ((2 * ks + h) ^ G::bswz(ql));
    vaddr[ks] = ql * G::ROW + 16 * ((2 * ks + h) ^ G::kswz(ql));
  }
#pragma unroll
  for (int u = 0; u < OT; ++u) taddr[u] = tr_offset<D>(lane, U0 + u);

  if (ntiles > 0) {
    dma(0, G::K0, G::V0);
    mask_dma(0);
  }

  // Q, dO and O of this lane's row (B-operand layout: Q[row][16s + 8h .. +7]).
  const uint16_t* qsrc = p.q + b * p.qs_b + hq * p.qs_h + qr * p.qs_n + 8 * h;
  const uint16_t* gsrc = p.dout + b * p.gs_b + hq * p.gs_h + qr * p.gs_n + 8 * h;
  const uint16_t* osrc = p.o + b * p.os_b + hq * p.os_h + qr * p.os_n + 8 * h;
  u32x4 qf[KSTEPS], dof[KSTEPS], of[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const bool ok = DCH == G::CH || 2 * s + h < DCH;
    qf[s] = ok ? *(const u32x4*)(qsrc + 16 * s) : u32x4{};
    dof[s] = ok ? *(const u32x4*)(gsrc + 16 * s) : u32x4{};
    of[s] = ok ? *(const u32x4*)(osrc + 16 * s) : u32x4{};
  }
  const float L = lse_log2(p.lse[(size_t)bh * p.N + qr]);
  // D = rowsum(dO o O): this lane's half of the row, then the lane pair.
  float dsum = 0.f;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = dof[s][w], o = of[s][w];
      if (DT == ATTN_BF16) {
        dsum = __builtin_fmaf(__uint_as_float(a << 16), __uint_as_float(o << 16), dsum);
        dsum = __builtin_fmaf(__uint_as_float(a & 0xffff0000u), __uint_as_float(o & 0xffff0000u),
                              dsum);
      } else {
        dsum = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(a & 0xffff)),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(o & 0xffff)), dsum);
        dsum = __builtin_fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(a >> 16)),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(o >> 16)), dsum);
      }
    }
  const float delta = pair_sum(dsum);
  if (PART == 0 && h == 0 && qrow < p.N) {
    p.delta[(size_t)bh * p.N + qrow] = delta;
    p.lse2[(size_t)bh * p.N + qrow] = L;
  }
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) qf[s] = (qf[s] ^ p.qsign) & p.qmask;

  f32x16 acc[OT];
#pragma unroll
  for (int u = 0; u < OT; ++u) acc[u] = f32x16{};
  const float c = p.c;

  auto step = [&](auto bufc, int j) {
    constexpr int P = decltype(bufc)::value;
    wait_loads_and_lds();
    __syncthreads();
    if (j + 1 < ntiles) dma(j + 1, P ? G::K0 : G::K1, P ? G::V0 : G::V1);
    const unsigned char* kb = smem + (P ? G::K1 : G::K0);
    const unsigned char* vb = smem + (P ? G::V1 : G::V0);
    // this tile's mask slice (keys 8g + 4h .. +3 of the lane's query row), then the next
    // tile's DMA into the same slot
    uint32_t mw[8][2];
    if constexpr (MK != kMaskNone) {
      const unsigned char* mr = smem + MOFF + wave * MG::WB + ql * MG::RB;
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if constexpr (MK == kMaskKeep) {
          mw[g][0] = *(const uint32_t*)(mr + 16 * ((g >> 1) ^ MG::mswz(ql)) + 8 * (g & 1) +
                                        4 * h);
          mw[g][1] = 0;
        } else {
          const u32x2 w = *(const u32x2*)(mr + 16 * (g ^ MG::mswz(ql)) + 8 * h);
          mw[g][0] = w[0];
          mw[g][1] = w[1];
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (j + 1 < ntiles) mask_dma(j + 1);
    }
    // S^T and dP^T for the tile's two 32-key halves. An additive mask is the scores' starting
    // value (raw score units), so that its words are not live across the MFMAs.
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      sc[t] = f32x16{};
      if constexpr (MK == kMaskAdd)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[t][r] = mask_add<DT, MK>(mw[4 * t + (r >> 2)], r & 3) * p.mscale;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      dp[t] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        sc[t] = M::run(*(const u32x4*)(kb + kaddr[ks] + t * 32 * G::ROW), qf[ks], sc[t]);
        dp[t] = M::run(*(const u32x4*)(vb + vaddr[ks] + t * 32 * G::ROW), dof[ks], dp[t]);
      }
    }
    // P and dS; keys kb0 + 32t + 8(r/4) + 4h + r%4 are tested by position only in tiles that
    // reach past this wave's causal diagonal or the padding boundary (a hidden element's P may
    // be inf: the select removes it); a keep mask is tested on every element.
    const int kb0 = j * kBN;
    const bool full = (!CAUSAL || kb0 + kBN - 1 <= qa) && kb0 + kBN <= kv_end;
    float ds[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][r], c, -L));
        ds[t][r] = pr * (dp[t][r] - delta);
        if constexpr (MK == kMaskKeep)
          ds[t][r] = mask_keep<DT, MK>(mw[4 * t + (r >> 2)], r & 3) ? ds[t][r] : 0.f;
      }
    if (!full) {
      int lim = kv_end - 1 - kb0 - 4 * h;
      if (CAUSAL) lim = min(lim, qrow - kb0 - 4 * h);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ds[t][r] = (32 * t + 8 * (r >> 2) + (r & 3) <= lim) ? ds[t][r] : 0.f;
    }
    // dQ^T += K^T dS^T, four 16-key k-steps
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 bsd = pack8<DT>(ds[s >> 1], s & 1);
#pragma unroll
      for (int u = 0; u < OT; ++u)
        acc[u] = M::run(tr_frag(kb, taddr[u] + 16 * s * G::ROW, 8 * G::ROW), bsd, acc[u]);
    }
  };
  // two tiles per trip, one per buffer, so that the buffer offsets are constants
  for (int j = 0; j < ntiles; j += 2) {
    step(std::integral_constant<int, 0>{}, j);
    if (j + 1 < ntiles) step(std::integral_constant<int, 1>{}, j + 1);
  }

  // dQ = scale * (dQ^T)^T, staged through LDS after every wave is done with the tiles.
  wait_loads_and_lds();
  __syncthreads();
  store_rows<DT, D, DH, PART>(acc, p.scale, smem + wave * 32 * G::ROW,
                              p.dq + b * p.dqs_b + hq * p.dqs_h, p.dqs_n, qa, p.N, lane);
}

// ------------------------------------------------------------------------------------------
// dK, dV
// ------------------------------------------------------------------------------------------
template <int D>
struct BwdGeo {
  using G = Geo<D>;
  static constexpr int QTILE = kQT * G::ROW;           // one 32-row Q or dO tile
  static constexpr int LD = 2048;                      // 1 KiB slots for L and D of one tile
  static constexpr int BUF = 2 * QTILE + LD;           // one buffer: Q, dO, L, D
  static constexpr int VREG = 2 * BUF;                 // V rows of the workgroup's 128 keys
  static constexpr int LDS = VREG + 128 * G::ROW;
  static constexpr int QLOADS = QTILE / 1024 / kWaves; // 1 KiB DMA blocks per wave per tile
  static_assert(QLOADS >= 1, "tile geometry");
  // buffers first, so that every Q / dO / L / D read is a fixed offset (16-bit immediate) from
  // a per-lane base once the loop is unrolled over the two buffers
  static_assert(BUF + QTILE + 24 * G::ROW <= 65535, "LDS offsets fit the immediate field");
};

// Mask slot of a dK/dV wave: the 32 query rows x 32 keys of one iteration, row-major (keys of a
// row contiguous), refilled one iteration ahead.
template <int MK>
struct KMaskGeo {
  static constexpr int ES = MaskGeo<MK>::ES;
  static constexpr int RB = 32 * ES;                          // bytes per row slice
  static constexpr int CPR = RB / 16;                         // 16-byte chunks per row slice
  static constexpr int WB = MK == kMaskNone ? 0 : kQT * RB;   // bytes per wave slot
  static constexpr int LOADS = WB / 1024;
  static constexpr int RPL = 1024 / RB;                       // rows per DMA block
};

template <int DT, int DH, bool CAUSAL, int MK, int PART, bool PAIR>
__device__ __forceinline__ void bwd_dkdv_body(const BwdParams& p) {
  constexpr int D = DH < 64 ? 64 : DH;   // geometry (as in the dQ kernel)
  constexpr int DCH = DH / 8;
  using G = Geo<D>;
  using BG = BwdGeo<D>;
  using KM = KMaskGeo<MK>;
  constexpr int MOFF = BG::LDS;   // per-wave mask slots follow the tiles and V rows
  using M = Mfma<DT>;
  constexpr int KSTEPS = G::KSTEPS;
  constexpr int OT = Parts<D>::OT;          // dK^T / dV^T tiles of this part
  constexpr int U0 = PART * OT;             // its first
  __shared__ __attribute__((aligned(1024))) unsigned char smem[BG::LDS + kWaves * KM::WB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int ql = lane & 31;

  // ---- work: (batch, KV head, item). Under causal masking key tile kt sees N - 128 kt queries.
  // Paired (PAIR, causal only): item i is the pair of key tiles i and nkt - 1 - i, the first
  // swept from the last query tile down, the second from its diagonal up, so that every item
  // has the same work and the items of a KV head that start together stay at the same query
  // tile throughout (the second sweep of item i starts at tile 4 (nkt - 1 - i) when the others'
  // first sweeps have reached the same distance from the end): the XCD's L2 then serves each
  // Q / dO tile to all of them. Each XCD runs its KV heads one after another, all items of a
  // head together.
  // Unpaired: an item is one key tile, swept down; each XCD takes its KV heads in blocks of two,
  // longest tiles first within a block (one head after another would leave a tail of long
  // workgroups), both heads' tile 0 first.
  const int nwk = PAIR ? (p.nkt + 1) >> 1 : p.nkt;   // items per KV head
  int pi, b, kvh, sp;
  {
    // consecutive workgroups of one XCD take the `split` parts of one item
    if (p.xcd_order) {
      const int xcd = blockIdx.x & 7, local0 = blockIdx.x >> 3;
      const int local = local0 / p.split;
      sp = local0 - local * p.split;
      int head_local;
      if constexpr (PAIR) {
        head_local = local / nwk;
        pi = local - head_local * nwk;
      } else {
        const int hpx = (p.B * p.Hkv) >> 3;
        const int blk = (hpx & 1) ? 1 : 2;
        const int block = local / (blk * nwk);
        const int r = local - block * blk * nwk;
        pi = r / blk;
        head_local = block * blk + (r - pi * blk);
      }
      const int kv_head = head_local * 8 + xcd;
      b = kv_head / p.Hkv;
      kvh = kv_head - b * p.Hkv;
    } else {
      const int wid = blockIdx.x / p.split;
      sp = blockIdx.x - wid * p.split;
      const int BK = p.B * p.Hkv;
      pi = wid / BK;
      const int bk = wid - pi * BK;
      b = bk / p.Hkv;
      kvh = bk - b * p.Hkv;
    }
  }
  int kv_end = p.N;
  if (p.valid_len) kv_end = min(max(p.valid_len[b], 0), p.N);
  unsigned char* vreg = smem + BG::VREG + wave * 32 * G::ROW;   // this wave's 32 V rows

  // Rows of the group's first query head in Q, dO and (waves 0 and 1) the base-2 LSE or Delta;
  // query head kvh * group + g is g head strides further.
  const uint16_t* const qhead = p.q + b * p.qs_b + (int64_t)kvh * p.group * p.qs_h;
  const uint16_t* const ohead = p.dout + b * p.gs_b + (int64_t)kvh * p.group * p.gs_h;
  const float* const lhead =
      (wave == 0 ? p.lse2 : p.delta) + ((size_t)b * p.Hq + (size_t)kvh * p.group) * p.N;
  const unsigned char* const mhead =
      MK != kMaskNone ? (const unsigned char*)p.mask +
                            (b * p.ms_b + (int64_t)kvh * p.group * p.ms_h) * KM::ES
                      : nullptr;
  // One key tile: its dK and dV, sweeping the query tiles down (first tile of an item) or up.
  auto run_tile = [&](auto upc) {
    constexpr bool up = decltype(upc)::value;
    const int kt = up ? p.nkt - 1 - pi : pi;
    const int k0 = kt * kBM;
    const int kw = k0 + wave * 32;   // this wave's first key
    const int key = kw + ql;         // this lane's key (MFMA output column)

    f32x16 dk[OT], dv[OT];
#pragma unroll
    for (int u = 0; u < OT; ++u) dk[u] = dv[u] = f32x16{};

    const int qstart = CAUSAL ? k0 : 0;
    const int ntq = k0 < kv_end ? (p.N - qstart + kQT - 1) / kQT : 0;   // query tiles per head
    // this workgroup's share [it0, it0 + iters) of the key tile's ntq * group iterations (query
    // tile major, query head minor)
    const int total = ntq * p.group;
    const int it0 = (int)((int64_t)total * sp / p.split);
    const int iters = (int)((int64_t)total * (sp + 1) / p.split) - it0;

    if (iters > 0) {
      // K^T fragments of this lane's key (B operand: K[key][16s + 8h .. +7]), sign/zero applied.
      u32x4 kf[KSTEPS];
      {
        const uint16_t* ksrc =
            p.k + b * p.ks_b + kvh * p.ks_h + min(key, p.N - 1) * p.ks_n + 8 * h;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          kf[s] = (DCH == G::CH || 2 * s + h < DCH)
                      ? (*(const u32x4*)(ksrc + 16 * s) ^ p.qsign) & p.qmask
                      : u32x4{};
      }
      // V rows of this wave's keys into its LDS rows (bswz layout like Q and dO, so that one set
      // of row-fragment offsets serves all three).
      {
        const uint32_t vrow = (uint32_t)p.vs_n * 2;
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.v + b * p.vs_b + kvh * p.vs_h), (short)0, (p.N - 1) * vrow + 2 * DH,
            kBufferFlags);
#pragma unroll
        for (int i = 0; i < 32 / G::RPB; ++i) {
          const int row = i * G::RPB + lane / G::CH;
          const int vc = (lane % G::CH) ^ G::bswz(row);
          const uint32_t off =
              (DCH < G::CH && vc >= DCH) ? kNoChunk : (lane / G::CH) * vrow + vc * 16;
          dma16(vrs, vreg + i * 1024, off, (uint32_t)(kw + i * G::RPB) * vrow);
        }
      }
      // DMA of the iteration over query head kvh * group + g, queries q0 .. q0+31, into buffer
      // `buf`: Q and dO tiles (bswz layout), L and D (wave 0 and 1).
      // Q and dO rows may have different strides: one chunk position per block, the row offsets
      // applied per tensor.
      const uint32_t qrowb = (uint32_t)p.qs_n * 2, growb = (uint32_t)p.gs_n * 2;
      uint32_t qoff[BG::QLOADS], goff[BG::QLOADS];
#pragma unroll
      for (int i = 0; i < BG::QLOADS; ++i) {
        const int row = (wave * BG::QLOADS + i) * G::RPB + lane / G::CH;   // row in the tile
        const int qc = (lane % G::CH) ^ G::bswz(row);
        const bool none = DCH < G::CH && qc >= DCH;
        qoff[i] = none ? kNoChunk : (lane / G::CH) * qrowb + qc * 16;
        goff[i] = none ? kNoChunk : (lane / G::CH) * growb + qc * 16;
      }
      auto dma = [&](int g, int q0, int buf) {
        const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(qhead + g * p.qs_h), (short)0, (p.N - 1) * qrowb + 2 * DH, kBufferFlags);
        const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(ohead + g * p.gs_h), (short)0, (p.N - 1) * growb + 2 * DH, kBufferFlags);
        unsigned char* base = smem + buf * BG::BUF;
#pragma unroll
        for (int i = 0; i < BG::QLOADS; ++i) {
          const int blk = wave * BG::QLOADS + i;
          const uint32_t r0 = (uint32_t)(q0 + blk * G::RPB);
          dma16(qrs, base + blk * 1024, qoff[i], r0 * qrowb);
          dma16(ors, base + BG::QTILE + blk * 1024, goff[i], r0 * growb);
        }
        if (wave < 2) {
          const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(lhead + (size_t)g * p.N), (short)0, (uint32_t)p.N * 4, kBufferFlags);
          // one dword per query row (lanes 0..31); a 16-byte load would straddle the end of the
          // row range when N % 4 != 0. Lanes 32..63 are out of range and write zeros to bytes
          // 128..255 of the wave's 1 KiB slot.
          const uint32_t loff = lane < kQT ? (uint32_t)(q0 + lane) * 4 : 0x7ffffff0u;
          dma4(lrs, base + 2 * BG::QTILE + wave * 1024, loff, 0);
        }
      };

      // Fragment offsets: rows of Q / dO / V (A of S and dP, B of dP), transposed Q / dO.
      uint32_t raddr[KSTEPS], taddr[OT];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        raddr[ks] = ql * G::ROW + 16 * ((2 * ks + h) ^ G::bswz(ql));
#pragma unroll
      for (int u = 0; u < OT; ++u) taddr[u] = tr_offset<D>(lane, U0 + u);
      const float c = p.c;

      // Explicit mask: rows q0 .. q0+31 (query head g) x this wave's keys kw .. kw+31 into the
      // wave's slot; lane L of block i writes row i * RPL + L / CPR, chunk L % CPR.
      const uint32_t mrow = MK != kMaskNone ? (uint32_t)(p.ms_n * KM::ES) : 0;
      const uint32_t mlane = MK != kMaskNone
                                 ? (uint32_t)(lane / KM::CPR) * mrow + (uint32_t)kw * KM::ES +
                                       16 * (lane % KM::CPR)
                                 : 0;
      auto mask_dma = [&](int g, int q0) {
        if constexpr (MK != kMaskNone) {
          const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(mhead + g * p.ms_h * KM::ES), (short)0,
              (p.N - 1) * mrow + ((p.N * KM::ES + 15) & ~15), kBufferFlags);
#pragma unroll
          for (int i = 0; i < KM::LOADS; ++i)
            dma16(mrs, smem + MOFF + wave * KM::WB + i * 1024, mlane,
                  (uint32_t)(q0 + i * KM::RPL) * mrow);
        }
      };

      // Iteration order: query tile major (from the last tile down, or from qstart up in the
      // second sweep of an item), query head minor. The key-tile workgroups of a KV head that run
      // at the same time then read the same Q / dO tile at the same step, and the XCD's L2 serves
      // all but the first (query head major, every workgroup reading a different tile, took 1.8x
      // the HBM bytes). State: (g, q0) of the tile being computed and of the next one to fetch.
      const int qlast = qstart + (ntq - 1) * kQT;
      const int t0 = it0 / p.group;
      const int dstep = up ? kQT : -kQT;
      const int g0 = it0 - t0 * p.group, qs0 = up ? qstart + t0 * kQT : qlast - t0 * kQT;
      int g_cur = g0, q_cur = qs0, g_nxt = g0, q_nxt = qs0;
      auto advance = [&](int& g, int& q0) {
        if (++g == p.group) { g = 0; q0 += dstep; }
      };
      dma(g_nxt, q_nxt, 0);
      mask_dma(g_nxt, q_nxt);
      advance(g_nxt, q_nxt);

      auto step = [&](auto bufc, int it) {
        constexpr int buf = decltype(bufc)::value;
        wait_loads_and_lds();
        __syncthreads();
        const int gn = g_nxt, qn = q_nxt;   // the next iteration's tile
        if (it + 1 < iters) {
          dma(gn, qn, buf ^ 1);
          advance(g_nxt, q_nxt);
        }
        const int q0 = q_cur;
        advance(g_cur, q_cur);
        // this iteration's mask values (query rows 8 (r/4) + 4h + r%4 of the tile, the lane's
        // key), then the next iteration's DMA into the same slot. Keep masks are packed into
        // one bit per element, additive values two per register.
        // An additive mask enters as the starting value of the score accumulator (in raw score
        // units), so that no mask register stays live across the MFMAs.
        uint32_t kbits = 0;
        f32x16 s = f32x16{};
        if constexpr (MK != kMaskNone) {
          const unsigned char* ms = smem + MOFF + wave * KM::WB + KM::ES * ql;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = 8 * (r >> 2) + 4 * h + (r & 3);
            if constexpr (MK == kMaskKeep) {
              // four bytes at a time, packed into bits as they arrive
              kbits |= (ms[qi * KM::RB] != 0 ? 1u : 0u) << r;
              if ((r & 3) == 3) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kbits) :: "memory");
            } else {
              const uint32_t bits = *(const uint16_t*)(ms + qi * KM::RB);
              const float a = DT == ATTN_BF16 ? __uint_as_float(bits << 16)
                                              : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
              s[r] = a * p.mscale;
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          if (it + 1 < iters) mask_dma(gn, qn);
        }
        const unsigned char* qb = smem + buf * BG::BUF;
        const unsigned char* ob = qb + BG::QTILE;
        const float* lb = (const float*)(qb + 2 * BG::QTILE);
        const float* db = (const float*)(qb + 2 * BG::QTILE + 1024);
        // S = Q K^T and dP = dO V^T (rows: queries q0 + 8(r/4) + 4h + r%4; column: key)
        f32x16 dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          s = M::run(*(const u32x4*)(qb + raddr[ks]), kf[ks], s);
          dp = M::run(*(const u32x4*)(ob + raddr[ks]), *(const u32x4*)(vreg + raddr[ks]), dp);
        }
        // P and dS. The wave's 32 keys are all visible to the tile's 32 queries unless the tile
        // touches the causal diagonal, the padding boundary or the end of the sequence; only then
        // is each element tested. A hidden element may have L = -inf (a row with no visible key)
        // and so x = inf: the select, not a product, removes it.
        // (a keep mask is tested on every element; an additive one is already in the scores)
        const bool full = MK != kMaskKeep && (!CAUSAL || q0 >= kw + 31) && kw + 32 <= kv_end &&
                          q0 + kQT <= p.N;
        float pr[16], ds[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int qi0 = 8 * r4 + 4 * h;   // first of this group's 4 query rows in the tile
          const f32x4 lv = *(const f32x4*)(lb + qi0);
          const f32x4 dv4 = *(const f32x4*)(db + qi0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lv[e]));
          }
          if (!full) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int qi = q0 + qi0 + e;
              bool vis = (!CAUSAL || key <= qi) && key < kv_end && qi < p.N;
              if constexpr (MK == kMaskKeep) vis = vis && ((kbits >> (4 * r4 + e)) & 1u);
              pr[4 * r4 + e] = vis ? pr[4 * r4 + e] : 0.f;
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[4 * r4 + e] = pr[4 * r4 + e] * (dp[4 * r4 + e] - dv4[e]);
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the two 16-query k-steps
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const u32x4 bp = pack8<DT>(pr, k2);
          const u32x4 bs = pack8<DT>(ds, k2);
#pragma unroll
          for (int u = 0; u < OT; ++u) {
            dv[u] = M::run(tr_frag(ob, taddr[u] + 16 * k2 * G::ROW, 8 * G::ROW), bp, dv[u]);
            dk[u] = M::run(tr_frag(qb, taddr[u] + 16 * k2 * G::ROW, 8 * G::ROW), bs, dk[u]);
          }
        }
      };
      // two iterations per trip, one per buffer, so that the buffer offsets are constants
      for (int it = 0; it < iters; it += 2) {
        step(std::integral_constant<int, 0>{}, it);
        if (it + 1 < iters) step(std::integral_constant<int, 1>{}, it + 1);
      }
      wait_loads_and_lds();
    }
    if (p.split > 1) {
      // fp32 partial sums of this part; rows past N are not written
      const size_t plane = (size_t)p.B * p.Hkv * p.N * DH;
      float* pk = p.part + (size_t)sp * plane + ((size_t)b * p.Hkv + kvh) * p.N * DH;
      if (key < p.N) {
        store_part<D, DH, PART>(dk, p.scale, pk + (size_t)key * DH, h);
        store_part<D, DH, PART>(dv, 1.0f, pk + (size_t)p.split * plane + (size_t)key * DH, h);
      }
      return;
    }
    __syncthreads();
    // dK = scale * (dK^T)^T, dV = (dV^T)^T; rows past N are not written. Staging reuses the Q/dO
    // buffers (every wave is past its last read).
    unsigned char* ost = smem + wave * 32 * G::ROW;
    store_rows<DT, D, DH, PART>(dk, p.scale, ost, p.dk + b * p.dks_b + kvh * p.dks_h, p.dks_n, kw,
                                p.N,
                          lane);
    store_rows<DT, D, DH, PART>(dv, 1.0f, ost, p.dv + b * p.dvs_b + kvh * p.dvs_h, p.dvs_n, kw,
                                p.N,
                          lane);
  };
  run_tile(std::false_type{});
  if constexpr (PAIR) {
    if (p.nkt - 1 - pi != pi) {
      __syncthreads();   // every wave is done with the first tile's buffers and staging
      run_tile(std::true_type{});
    }
  }
}

// D = 256 holds 128 KiB of tiles in LDS: one workgroup per CU, one wave per SIMD with the
// whole register file. D <= 64 without an explicit mask fits 168 VGPRs: three waves per SIMD.
template <int D, int MK>
constexpr int bwd_waves_per_eu() { return D > 128 ? 1 : (D <= 64 && MK == kMaskNone ? 3 : 2); }

template <int DT, int D, bool CAUSAL, int MK, int PART>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(bwd_waves_per_eu<D, MK>(), bwd_waves_per_eu<D, MK>())))
void attn_bwd_dq_kernel(BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  bwd_dq_body<DT, D, CAUSAL, MK, PART>(p);
#endif
}

template <int DT, int D, bool CAUSAL, int MK, int PART, bool PAIR>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(bwd_waves_per_eu<D, MK>(), bwd_waves_per_eu<D, MK>())))
void attn_bwd_dkdv_kernel(BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  bwd_dkdv_body<DT, D, CAUSAL, MK, PART, PAIR>(p);
#endif
}

// The dK/dV kernel's parts, one workgroup per key tile or (PAIR) per pair of key tiles.
template <int DT, int D, bool CAUSAL, int MK, bool PAIR>
void launch_dkdv(const BwdParams& p, hipStream_t s) {
  const int64_t nk = (int64_t)p.B * p.Hkv * (PAIR ? (p.nkt + 1) / 2 : p.nkt) * p.split;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DT, D, CAUSAL, MK, 0, PAIR>), dim3((unsigned)nk),
                     dim3(kThreads), 0, s, p);
  if constexpr (Parts<D>::NP > 1)
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DT, D, CAUSAL, MK, 1, PAIR>), dim3((unsigned)nk),
                       dim3(kThreads), 0, s, p);
}

// The dQ kernel's parts, then the dK/dV kernel's (it reads the workspace the first dQ part
// writes).
template <int DT, int D, bool CAUSAL, int MK>
hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
  const int64_t nq = (int64_t)p.B * p.Hq * p.nqt;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<DT, D, CAUSAL, MK, 0>), dim3((unsigned)nq),
                     dim3(kThreads), 0, s, p);
  if constexpr (Parts<D>::NP > 1)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<DT, D, CAUSAL, MK, 1>), dim3((unsigned)nq),
                       dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (CAUSAL && D <= 128) {   // (bwd_pairs pairs nothing above D = 128)
    if (p.pair)
      launch_dkdv<DT, D, true, MK, true>(p, s);
    else
      launch_dkdv<DT, D, true, MK, false>(p, s);
  } else {
    launch_dkdv<DT, D, CAUSAL, MK, false>(p, s);
  }
  return hipGetLastError();
}

template <int DT, int MK>
hipError_t dispatch_bwd_d(const BwdParams& p, int D, bool causal, hipStream_t s) {
  switch (D) {
    case 16:
      return causal ? launch_bwd<DT, 16, true, MK>(p, s) : launch_bwd<DT, 16, false, MK>(p, s);
    case 32:
      return causal ? launch_bwd<DT, 32, true, MK>(p, s) : launch_bwd<DT, 32, false, MK>(p, s);
    case 64:
      return causal ? launch_bwd<DT, 64, true, MK>(p, s) : launch_bwd<DT, 64, false, MK>(p, s);
    case 256:
      return causal ? launch_bwd<DT, 256, true, MK>(p, s) : launch_bwd<DT, 256, false, MK>(p, s);
    default:
      return causal ? launch_bwd<DT, 128, true, MK>(p, s) : launch_bwd<DT, 128, false, MK>(p, s);
  }
}

template <int DT>
hipError_t dispatch_bwd(const BwdParams& p, int D, bool causal, int mask_type, hipStream_t s) {
  if (mask_type == ATTN_MASK_KEEP_U8) return dispatch_bwd_d<DT, kMaskKeep>(p, D, causal, s);
  if (mask_type == ATTN_MASK_ADD) return dispatch_bwd_d<DT, kMaskAdd>(p, D, causal, s);
  return dispatch_bwd_d<DT, kMaskNone>(p, D, causal, s);
}

// The eight [B, H, N, D] tensors of a backward call.
struct BwdLayouts {
  Layout q, k, v, o, dout, dq, dk, dv;
};

BwdLayouts bwd_layouts(const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                       const void* v, const int64_t* vs, const void* o, const int64_t* os,
                       const void* dout, const int64_t* gs, const void* dq, const int64_t* dqs,
                       const void* dk, const int64_t* dks, const void* dv, const int64_t* dvs,
                       int Hq, int Hkv, int N, int D) {
  return BwdLayouts{strided(q, qs, Hq, N, D),     strided(k, ks, Hkv, N, D),
                    strided(v, vs, Hkv, N, D),    strided(o, os, Hq, N, D),
                    strided(dout, gs, Hq, N, D),  strided(dq, dqs, Hq, N, D),
                    strided(dk, dks, Hkv, N, D),  strided(dv, dvs, Hkv, N, D)};
}

// Workspace of a backward call: Delta and the base-2 LSE (2 B Hq N floats), then, when the
// dK/dV kernel splits each key tile's iterations over `split` workgroups, the fp32 partial sums
// [2][split][B][Hkv][N][D] from the next 16-byte boundary.
int64_t ws_base_floats(int B, int Hq, int N) { return 2 * (int64_t)B * Hq * N; }

int64_t ws_floats_for(int B, int Hq, int Hkv, int N, int D, int split) {
  const int64_t base = ws_base_floats(B, Hq, N);
  if (split <= 1) return base;
  return base + 4 + 2 * (int64_t)split * B * Hkv * N * D;
}

// Paired dK/dV items under causal masking all take the same time, so they run in whole rounds
// of the device's resident workgroups (its CUs x the kernel's workgroups per CU): pair only
// when the items fill their last round (at least 15/16 of it), and up to D = 128 (measured on
// the headline shape: unmasked the same time with a third of the HBM bytes, keep mask -10 %,
// additive mask the same time, D = 64 with 1.33 rounds +6.5 %, D = 256 in four whole rounds
// +2.7 %).
int bwd_pairs(int B, int Hkv, int N, int D, int split, int mask_type) {
  if (D > 128) return 0;
  const int64_t nkt = (N + kBM - 1) / kBM;
  const int64_t items = (int64_t)B * Hkv * ((nkt + 1) / 2) * split;
  const int per_cu = D <= 64 && mask_type == ATTN_MASK_NONE ? 3 : 2;
  const int64_t slots = (int64_t)device_cus() * per_cu;
  const int64_t rounds = (items + slots - 1) / slots;
  return items * 16 >= rounds * slots * 15 ? 1 : 0;
}

// Parts per key tile: powers of two up to 16 until there are at least four dK/dV workgroups per
// CU (twice the two the device holds at once: 1024 on a whole MI355X), as long as a part keeps
// about 32 iterations of a key tile's average (half of its group * N / 32 query tiles) to pay
// for writing and reading its partial sums, and as far as the workspace holds them.
int bwd_split(int B, int Hq, int Hkv, int N, int D, int64_t ws_floats) {
  const int64_t tiles = (int64_t)B * Hkv * ((N + kBM - 1) / kBM);
  const int64_t avg_iters = (int64_t)(Hq / Hkv) * ((N + kQT - 1) / kQT) / 2;
  int split = 1;
  const int64_t target = 4 * (int64_t)device_cus();
  while (split < 16 && tiles * split < target && avg_iters / (2 * split) >= 32) split *= 2;
  while (split > 1 && ws_floats_for(B, Hq, Hkv, N, D, split) > ws_floats) split /= 2;
  return split;
}

float* part_base(float* ws, int B, int Hq, int N) {
  const uintptr_t a = (uintptr_t)(ws + ws_base_floats(B, Hq, N));
  return (float*)((a + 15) & ~(uintptr_t)15);
}

int bwd_validate(const BwdLayouts& t, const float* lse, const float* ws, int64_t ws_floats, int B,
                 int Hq, int Hkv, int N, int D, float scale, const int32_t* valid_len, int dtype,
                 const MaskArg& mk = no_mask()) {
  const Layout* all[] = {&t.q, &t.k, &t.v, &t.o, &t.dout, &t.dq, &t.dk, &t.dv};
  for (const Layout* l : all)
    if (!l->ptr) return ATTN_ERR_NULL;
  if (!lse || !ws) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (N > ATTN_MAX_N) return ATTN_ERR_SHAPE;
  if ((int64_t)B * Hq * (((int64_t)N + kBM - 1) / kBM) > ATTN_MAX_TILES) return ATTN_ERR_SHAPE;
  if (D != 16 && D != 32 && D != 64 && D != 128 && D != 256) return ATTN_ERR_HEAD_DIM;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  const int es = dtype == ATTN_F32 ? 4 : 2;   // bytes per element
  for (const Layout* l : all)
    if (!layout_ok(*l, D, es)) return ATTN_ERR_LAYOUT;
  if ((uintptr_t)lse % 4 != 0 || (uintptr_t)ws % 4 != 0) return ATTN_ERR_LAYOUT;
  if (ws_floats < ws_base_floats(B, Hq, N)) return ATTN_ERR_WORKSPACE;
  if (!output_disjoint(t.dq, B, Hq, N, D) || !output_disjoint(t.dk, B, Hkv, N, D) ||
      !output_disjoint(t.dv, B, Hkv, N, D))
    return ATTN_ERR_LAYOUT;
  // K, V, Q and dO of one head are read as 32-bit-addressed buffers, with scalar row offsets up
  // to one tile past N.
  int64_t smax = 0;
  for (const Layout* l : {&t.q, &t.k, &t.v, &t.dout}) smax = l->sn > smax ? l->sn : smax;
  if (((int64_t)N + kBM) * smax * es + es * D > INT32_MAX) return ATTN_ERR_SHAPE;
  // Outputs (dq, dk, dv and the part of the workspace this call uses) overlap no input and no
  // other output.
  const int64_t lb = (int64_t)B * Hq * N * 4;
  const int split = bwd_split(B, Hq, Hkv, N, D, ws_floats);
  const void* outs[] = {t.dq.ptr, t.dk.ptr, t.dv.ptr, ws};
  const int64_t osz[] = {t.dq.span(B, N, D, es), t.dk.span(B, N, D, es),
                         t.dv.span(B, N, D, es), ws_floats_for(B, Hq, Hkv, N, D, split) * 4};
  const void* ins[] = {t.q.ptr, t.k.ptr, t.v.ptr, t.o.ptr, t.dout.ptr, lse};
  const int64_t isz[] = {t.q.span(B, N, D, es), t.k.span(B, N, D, es), t.v.span(B, N, D, es),
                         t.o.span(B, N, D, es), t.dout.span(B, N, D, es), lb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], osz[i], outs[j], osz[j])) return ATTN_ERR_ALIAS;
    if (valid_len && overlaps(outs[i], osz[i], valid_len, (int64_t)B * 4)) return ATTN_ERR_ALIAS;
  }
  if (mk.type != ATTN_MASK_NONE) {
    const int ms = mask_status(mk, N, dtype);
    if (ms != ATTN_OK) return ms;
    const int64_t mbytes = mask_span(mk, B, Hq, N, dtype);
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[i], osz[i], mk.ptr, mbytes)) return ATTN_ERR_ALIAS;
  }
  return ATTN_OK;
}

// Queue the sum of the split parts into dk and dv.
hipError_t launch_reduce(const BwdLayouts& t, const float* part, int B, int Hkv, int N, int D,
                         int split, int dtype, hipStream_t s) {
  ReduceParams r;
  r.part = part;
  r.dk = (void*)t.dk.ptr;
  r.dv = (void*)t.dv.ptr;
  r.B = B;
  r.Hkv = Hkv;
  r.N = N;
  r.DH = D;
  r.split = split;
  r.dks_b = t.dk.sb; r.dks_h = t.dk.sh; r.dks_n = t.dk.sn;
  r.dvs_b = t.dv.sb; r.dvs_h = t.dv.sh; r.dvs_n = t.dv.sn;
  const int64_t n = (int64_t)B * Hkv * N * (D / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (dtype == ATTN_F32)
    hipLaunchKernelGGL(attn_bwd_reduce_kernel<ATTN_F32>, grid, dim3(256), 0, s, r);
  else if (dtype == ATTN_BF16)
    hipLaunchKernelGGL(attn_bwd_reduce_kernel<ATTN_BF16>, grid, dim3(256), 0, s, r);
  else
    hipLaunchKernelGGL(attn_bwd_reduce_kernel<ATTN_F16>, grid, dim3(256), 0, s, r);
  return hipGetLastError();
}

int bwd_run(const BwdLayouts& t, const float* lse, float* ws, int64_t ws_floats, int B, int Hq,
            int Hkv, int N, int D, float scale, int causal, const int32_t* valid_len, int dtype,
            void* stream, const MaskArg& mk = no_mask()) {
  const int st =
      bwd_validate(t, lse, ws, ws_floats, B, Hq, Hkv, N, D, scale, valid_len, dtype, mk);
  if (st != ATTN_OK) return st;
  const int split = bwd_split(B, Hq, Hkv, N, D, ws_floats);
  float* const part = split > 1 ? part_base(ws, B, Hq, N) : nullptr;
  const hipStream_t hs = (hipStream_t)stream;
  if (dtype == ATTN_F32) {
    F32BwdParams f;
    f.q = (const float*)t.q.ptr;
    f.k = (const float*)t.k.ptr;
    f.v = (const float*)t.v.ptr;
    f.o = (const float*)t.o.ptr;
    f.dout = (const float*)t.dout.ptr;
    f.lse = lse;
    f.dq = (float*)t.dq.ptr;
    f.dk = (float*)t.dk.ptr;
    f.dv = (float*)t.dv.ptr;
    f.delta = ws;
    f.lse2 = ws + (size_t)B * Hq * N;
    f.valid_len = valid_len;
    f.B = B;
    f.Hq = Hq;
    f.Hkv = Hkv;
    f.N = N;
    f.group = Hq / Hkv;
    f.nqt = (N + kBM - 1) / kBM;
    f.nkt = (N + kBM - 1) / kBM;
    f.xcd_order = ((int64_t)B * Hkv) % 8 == 0 ? 1 : 0;
    f.qs_b = t.q.sb; f.qs_h = t.q.sh; f.qs_n = t.q.sn;
    f.ks_b = t.k.sb; f.ks_h = t.k.sh; f.ks_n = t.k.sn;
    f.vs_b = t.v.sb; f.vs_h = t.v.sh; f.vs_n = t.v.sn;
    f.os_b = t.o.sb; f.os_h = t.o.sh; f.os_n = t.o.sn;
    f.gs_b = t.dout.sb; f.gs_h = t.dout.sh; f.gs_n = t.dout.sn;
    f.dqs_b = t.dq.sb; f.dqs_h = t.dq.sh; f.dqs_n = t.dq.sn;
    f.dks_b = t.dk.sb; f.dks_h = t.dk.sh; f.dks_n = t.dk.sn;
    f.dvs_b = t.dv.sb; f.dvs_h = t.dv.sh; f.dvs_n = t.dv.sn;
    f.c = scale == 0.f ? 1.0f : fabsf(scale) * kLog2e;
    f.qmul = scale < 0.f ? -1.0f : (scale == 0.f ? 0.0f : 1.0f);
    f.scale = scale;
    f.split = split;
    f.part = part;
    f.mask = mk.ptr;
    f.ms_b = mk.sb; f.ms_h = mk.sh; f.ms_n = mk.sn;
    f.mscale = kLog2e / f.c;
    hipError_t e = launch_bwd_f32(f, D, causal != 0, mk.type, hs);
    if (e == hipSuccess && split > 1) e = launch_reduce(t, part, B, Hkv, N, D, split, dtype, hs);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
  }
  BwdParams p;
  p.q = (const uint16_t*)t.q.ptr;
  p.k = (const uint16_t*)t.k.ptr;
  p.v = (const uint16_t*)t.v.ptr;
  p.o = (const uint16_t*)t.o.ptr;
  p.dout = (const uint16_t*)t.dout.ptr;
  p.lse = lse;
  p.dq = (uint16_t*)t.dq.ptr;
  p.dk = (uint16_t*)t.dk.ptr;
  p.dv = (uint16_t*)t.dv.ptr;
  p.delta = ws;
  p.lse2 = ws + (size_t)B * Hq * N;
  p.valid_len = valid_len;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.group = Hq / Hkv;
  p.nqt = (N + kBM - 1) / kBM;
  p.nkt = (N + kBM - 1) / kBM;
  p.xcd_order = ((int64_t)B * Hkv) % 8 == 0 ? 1 : 0;
  p.c = fabsf(scale) * kLog2e;
  p.scale = scale;
  p.qsign = scale < 0.f ? 0x80008000u : 0u;
  p.qmask = scale == 0.f ? 0u : 0xffffffffu;
  if (scale == 0.f) p.c = 1.0f;
  p.qs_b = t.q.sb; p.qs_h = t.q.sh; p.qs_n = t.q.sn;
  p.ks_b = t.k.sb; p.ks_h = t.k.sh; p.ks_n = t.k.sn;
  p.vs_b = t.v.sb; p.vs_h = t.v.sh; p.vs_n = t.v.sn;
  p.os_b = t.o.sb; p.os_h = t.o.sh; p.os_n = t.o.sn;
  p.gs_b = t.dout.sb; p.gs_h = t.dout.sh; p.gs_n = t.dout.sn;
  p.dqs_b = t.dq.sb; p.dqs_h = t.dq.sh; p.dqs_n = t.dq.sn;
  p.dks_b = t.dk.sb; p.dks_h = t.dk.sh; p.dks_n = t.dk.sn;
  p.dvs_b = t.dv.sb; p.dvs_h = t.dv.sh; p.dvs_n = t.dv.sn;
  p.mask = mk.ptr;
  p.ms_b = mk.sb; p.ms_h = mk.sh; p.ms_n = mk.sn;
  p.mscale = kLog2e / p.c;
  p.split = split;
  p.part = part;
  p.pair = causal ? bwd_pairs(B, Hkv, N, D, split, mk.type) : 0;
  hipError_t e = dtype == ATTN_BF16 ? dispatch_bwd<ATTN_BF16>(p, D, causal != 0, mk.type, hs)
                                    : dispatch_bwd<ATTN_F16>(p, D, causal != 0, mk.type, hs);
  if (e == hipSuccess && split > 1) e = launch_reduce(t, part, B, Hkv, N, D, split, dtype, hs);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

// Workspace of attn_bwd_scratch, for callers that cannot allocate: a static device array of
// ATTN_SCRATCH_FLOATS floats that each device running this library holds until the process
// ends. Host code never passes `scratch` itself (on the host it names a stand-in, not device
// memory); it uses the device address scratch_ptr looks up once per device.
static __device__ __align__(256) float scratch[ATTN_SCRATCH_FLOATS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices];   // device address of `scratch` per device ordinal

// The device address of `scratch` on the device `stream` belongs to (the current device for the
// null stream), looked up with hipGetSymbolAddress once per device while that device is
// current. nullptr when the runtime reports an error or the ordinal is beyond kMaxDevices.
float* scratch_ptr(hipStream_t stream) {
  int dev = -1;
  if (stream) {
    hipDevice_t d;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return nullptr;
    dev = (int)d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = (float*)ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int attn_bwd_validate(const void* q, const void* k, const void* v, const void* out,
                                 const void* dout, const float* lse, const void* dq,
                                 const void* dk, const void* dv, const float* ws, int B,
                                 int Hq, int Hkv, int N, int D, float scale, int causal,
                                 const int32_t* valid_len, int dtype) {
  (void)causal;
  return bwd_validate(bwd_layouts(q, nullptr, k, nullptr, v, nullptr, out, nullptr, dout,
                                  nullptr, dq, nullptr, dk, nullptr, dv, nullptr, Hq, Hkv, N, D),
                      lse, ws, ws_base_floats(B, Hq, N), B, Hq, Hkv, N, D, scale, valid_len,
                      dtype);
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        float* ws, int B, int Hq, int Hkv, int N, int D, float scale,
                        int causal, const int32_t* valid_len, int dtype, void* stream) {
  return bwd_run(bwd_layouts(q, nullptr, k, nullptr, v, nullptr, out, nullptr, dout, nullptr,
                             dq, nullptr, dk, nullptr, dv, nullptr, Hq, Hkv, N, D),
                 lse, ws, ws_base_floats(B, Hq, N), B, Hq, Hkv, N, D, scale, causal, valid_len,
                 dtype, stream);
}

extern "C" int attn_bwd_strided_validate(
    const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
    const void* v, const int64_t* v_strides, const void* out, const int64_t* out_strides,
    const void* dout, const int64_t* dout_strides, const float* lse, const void* dq,
    const int64_t* dq_strides, const void* dk, const int64_t* dk_strides, const void* dv,
    const int64_t* dv_strides, const float* ws, int B, int Hq, int Hkv, int N, int D,
    float scale, int causal, const int32_t* valid_len, int dtype) {
  (void)causal;
  return bwd_validate(bwd_layouts(q, q_strides, k, k_strides, v, v_strides, out, out_strides,
                                  dout, dout_strides, dq, dq_strides, dk, dk_strides, dv,
                                  dv_strides, Hq, Hkv, N, D),
                      lse, ws, ws_base_floats(B, Hq, N), B, Hq, Hkv, N, D, scale, valid_len,
                      dtype);
}

extern "C" int attn_bwd_strided(
    const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
    const void* v, const int64_t* v_strides, const void* out, const int64_t* out_strides,
    const void* dout, const int64_t* dout_strides, const float* lse, void* dq,
    const int64_t* dq_strides, void* dk, const int64_t* dk_strides, void* dv,
    const int64_t* dv_strides, float* ws, int B, int Hq, int Hkv, int N, int D, float scale,
    int causal, const int32_t* valid_len, int dtype, void* stream) {
  return bwd_run(bwd_layouts(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                             dout_strides, dq, dq_strides, dk, dk_strides, dv, dv_strides, Hq,
                             Hkv, N, D),
                 lse, ws, ws_base_floats(B, Hq, N), B, Hq, Hkv, N, D, scale, causal, valid_len,
                 dtype, stream);
}

extern "C" int attn_bwd_masked_validate(
    const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
    const void* v, const int64_t* v_strides, const void* out, const int64_t* out_strides,
    const void* dout, const int64_t* dout_strides, const float* lse, const void* dq,
    const int64_t* dq_strides, const void* dk, const int64_t* dk_strides, const void* dv,
    const int64_t* dv_strides, const float* ws, int B, int Hq, int Hkv, int N, int D,
    float scale, int causal, const int32_t* valid_len, const void* mask, int mask_type,
    const int64_t* mask_strides, int dtype) {
  (void)causal;
  return bwd_validate(bwd_layouts(q, q_strides, k, k_strides, v, v_strides, out, out_strides,
                                  dout, dout_strides, dq, dq_strides, dk, dk_strides, dv,
                                  dv_strides, Hq, Hkv, N, D),
                      lse, ws, ws_base_floats(B, Hq, N), B, Hq, Hkv, N, D, scale, valid_len,
                      dtype, mask_arg(mask, mask_type, mask_strides, N));
}

extern "C" int attn_bwd_masked(
    const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
    const void* v, const int64_t* v_strides, const void* out, const int64_t* out_strides,
    const void* dout, const int64_t* dout_strides, const float* lse, void* dq,
    const int64_t* dq_strides, void* dk, const int64_t* dk_strides, void* dv,
    const int64_t* dv_strides, float* ws, int B, int Hq, int Hkv, int N, int D, float scale,
    int causal, const int32_t* valid_len, const void* mask, int mask_type,
    const int64_t* mask_strides, int dtype, void* stream) {
  return bwd_run(bwd_layouts(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                             dout_strides, dq, dq_strides, dk, dk_strides, dv, dv_strides, Hq,
                             Hkv, N, D),
                 lse, ws, ws_base_floats(B, Hq, N), B, Hq, Hkv, N, D, scale, causal, valid_len,
                 dtype, stream, mask_arg(mask, mask_type, mask_strides, N));
}

extern "C" int64_t attn_bwd_workspace_floats(int B, int Hq, int Hkv, int N, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1) return -1;
  return ws_floats_for(B, Hq, Hkv, N, D, bwd_split(B, Hq, Hkv, N, D, INT64_MAX));
}

extern "C" int attn_bwd_ws_validate(
    const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
    const void* v, const int64_t* v_strides, const void* out, const int64_t* out_strides,
    const void* dout, const int64_t* dout_strides, const float* lse, const void* dq,
    const int64_t* dq_strides, const void* dk, const int64_t* dk_strides, const void* dv,
    const int64_t* dv_strides, const float* ws, int64_t ws_floats, int B, int Hq, int Hkv,
    int N, int D, float scale, int causal, const int32_t* valid_len, const void* mask,
    int mask_type, const int64_t* mask_strides, int dtype) {
  (void)causal;
  return bwd_validate(bwd_layouts(q, q_strides, k, k_strides, v, v_strides, out, out_strides,
                                  dout, dout_strides, dq, dq_strides, dk, dk_strides, dv,
                                  dv_strides, Hq, Hkv, N, D),
                      lse, ws, ws_floats, B, Hq, Hkv, N, D, scale, valid_len, dtype,
                      mask_arg(mask, mask_type, mask_strides, N));
}

extern "C" int attn_bwd_ws(
    const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
    const void* v, const int64_t* v_strides, const void* out, const int64_t* out_strides,
    const void* dout, const int64_t* dout_strides, const float* lse, void* dq,
    const int64_t* dq_strides, void* dk, const int64_t* dk_strides, void* dv,
    const int64_t* dv_strides, float* ws, int64_t ws_floats, int B, int Hq, int Hkv, int N,
    int D, float scale, int causal, const int32_t* valid_len, const void* mask, int mask_type,
    const int64_t* mask_strides, int dtype, void* stream) {
  return bwd_run(bwd_layouts(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                             dout_strides, dq, dq_strides, dk, dk_strides, dv, dv_strides, Hq,
                             Hkv, N, D),
                 lse, ws, ws_floats, B, Hq, Hkv, N, D, scale, causal, valid_len, dtype, stream,
                 mask_arg(mask, mask_type, mask_strides, N));
}

extern "C" int attn_bwd_scratch(
    const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
    const void* v, const int64_t* v_strides, const void* out, const int64_t* out_strides,
    const void* dout, const int64_t* dout_strides, const float* lse, void* dq,
    const int64_t* dq_strides, void* dk, const int64_t* dk_strides, void* dv,
    const int64_t* dv_strides, int B, int Hq, int Hkv, int N, int D, float scale, int causal,
    const int32_t* valid_len, const void* mask, int mask_type, const int64_t* mask_strides,
    int dtype, void* stream) {
  if (B >= 1 && Hq >= 1 && N >= 1 && ws_base_floats(B, Hq, N) > ATTN_SCRATCH_FLOATS)
    return ATTN_ERR_SCRATCH;
  float* const ws = scratch_ptr((hipStream_t)stream);
  if (!ws) return ATTN_ERR_LAUNCH;
  return bwd_run(bwd_layouts(q, q_strides, k, k_strides, v, v_strides, out, out_strides, dout,
                             dout_strides, dq, dq_strides, dk, dk_strides, dv, dv_strides, Hq,
                             Hkv, N, D),
                 lse, ws, ATTN_SCRATCH_FLOATS, B, Hq, Hkv, N, D, scale, causal, valid_len, dtype,
                 stream, mask_arg(mask, mask_type, mask_strides, N));
}
