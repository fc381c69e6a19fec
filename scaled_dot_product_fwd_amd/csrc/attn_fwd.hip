// Fused masked multi-head attention forward for CDNA4 (gfx950), behind the C ABI in attn.h.
//
// Method: the tiled online softmax of "Triton Cuda Attention" (section on the online softmax
// core algorithm) -- one workgroup owns a tile of query rows of one (batch, query head), keeps
// its Q tile in registers, streams K/V tiles through LDS, and keeps a running row maximum m,
// running denominator l and fp32 accumulator acc, dividing by l once at the end. The block row
// maximum is taken before the exponentials so that each score costs one exp (the masked
// multi-head attention CUDA article, wzjinhao.cn/news/73578, section 4.3), and exponentials are
// exp2 of scores pre-multiplied by scale*log2(e) ("Triton Cuda Attention", performance notes).
//
// CDNA4 mapping (lane layouts of v_mfma_f32_32x32x16_{bf16,f16} and ds_read_b64_tr_b16 were
// measured on the device before use):
//   * Scores are computed transposed, S^T = K Q^T, so the 32x32 MFMA output column a lane holds
//     is one query: lane l owns query (l % 32) and 16 of every 32 keys; lanes l and l^32 share a
//     query. Row max and row sum are in-lane, plus one permlane32 swap.
//   * Output is accumulated transposed, O^T = V^T P^T: the S^T registers, rounded to 16 bits,
//     are the B operand of the second MFMA directly (keys in the order the first MFMA's output
//     layout gives them); V^T fragments come from row-major V in LDS through the transposing LDS
//     read ds_read_b64_tr_b16.
//   * K and V tiles go HBM -> LDS by buffer_load ... lds (no staging registers); the buffer
//     range check returns zeros past the last key, so a ragged tail needs no branches. LDS rows
//     are XOR-swizzled by 16-byte chunk so that the 128-bit K reads and the transposing V reads
//     are free of bank conflicts.
//   * K runs one tile ahead of V: while the MFMAs compute the scores of tile j+1, the VALU does
//     the softmax of tile j, then P_j V_j accumulates. Each wave keeps two score tiles.
//   * Causal and padding masks are implicit: tiles wholly above the diagonal or past valid_len
//     are never loaded; only tiles that straddle a boundary apply a per-element mask, on a
//     separate (slower) code path. An explicit [B, H, N, N] keep or additive mask (the article,
//     sections 2.1-2.2) is streamed per wave into LDS one tile ahead and applied on every tile.
//   * Q, K, V and O are addressed through (batch, head, row) strides with contiguous rows, so
//     [B, N, H, D] and other layouts need no copy ("Triton Cuda Attention"'s kernel takes the
//     same strides).
//   * The running maximum is only raised when a tile's maximum exceeds it by more than
//     RESCALE_THRESHOLD (log2 units). Any reference value gives the same final O = acc / l and
//     LSE = m + log2(l) as long as numerator and denominator share it; a bounded stale maximum
//     only keeps probabilities below 2^RESCALE_THRESHOLD, and saves the accumulator rescale on
//     most tiles.
//   * Workgroups are ordered so that, when the KV heads divide evenly over the 8 XCDs, every
//     query head of one KV head runs on the same XCD (its K/V stay in that XCD's L2), longest
//     causal tiles first.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <type_traits>

#include "attn.h"
#include "attn_common.h"

typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

namespace {

using namespace attn_detail;

constexpr float RESCALE_THRESHOLD = 8.0f;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int32_t* valid_len;
  int B, Hq, Hkv, N;
  int group;         // Hq / Hkv
  int nqt;           // ceil(N / kBM)
  int xcd_order;     // 1: KV heads divide evenly over the 8 XCDs
  // Element strides (batch, head, row) of Q, K, V and O; the D elements of a row are
  // contiguous. Every stride is a multiple of 8 elements (16-byte rows).
  int64_t qs_b, qs_h, qs_n;
  int64_t ks_b, ks_h, ks_n;
  int64_t vs_b, vs_h, vs_n;
  int64_t os_b, os_h, os_n;
  const void* mask;  // explicit mask (kernels with MK != kMaskNone)
  int64_t ms_b, ms_h, ms_n;   // its element strides (batch, query head, query row)
  float mscale;      // log2(e) / c: an additive mask value in raw score units
  float c;           // |scale| * log2(e)
  uint32_t qsign;    // 0x80008000 when scale < 0: Q is negated (exactly) instead
  uint32_t qmask;    // 0 when scale == 0: all scores are exactly 0 (and c is set to 1)
  // Split of each query tile's key range (kernels with SPLIT): chunk c of a query tile covers
  // key tiles [c * split_tiles, (c + 1) * split_tiles) of its range and writes its fp32 partial
  // O (normalised by its own sum) and base-2 LSE for the merge kernel.
  int split_tiles;
  int nchunk;        // chunks per query tile (grid = B * Hq * nqt * nchunk)
  float* part_o;     // [B * Hq * nqt * nchunk][kBM rows][DH]
  float* part_lse;   // [B * Hq * nqt * nchunk][kBM rows]
};

template <int DT, int D>
__device__ inline void qk_tile(f32x16 (&s)[2], const unsigned char* kbuf, const Frag<D>& f,
                               const u32x4 (&qf)[Geo<D>::KSTEPS]) {
  using G = Geo<D>;
  using M = Mfma<DT>;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s[t] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < G::KSTEPS; ++ks) {
      const u32x4 a = *(const u32x4*)(kbuf + f.kaddr[ks] + t * 32 * G::ROW);
      s[t] = M::run(a, qf[ks], s[t]);
    }
  }
}

// O^T += V^T P^T for the 16 keys of k-step s.
template <int DT, int D>
__device__ inline void pv_step(f32x16 (&acc)[Geo<D>::OT], const unsigned char* vbuf,
                               const Frag<D>& f, int s, u32x4 pb) {
  using G = Geo<D>;
  using M = Mfma<DT>;
#pragma unroll
  for (int u = 0; u < G::OT; ++u) {
    const unsigned char* base = vbuf + f.vaddr[u] + 16 * s * G::ROW;
    const u32x2 lo = lds_read_tr16(base);
    const u32x2 hi = lds_read_tr16(base + 8 * G::ROW);
    acc[u] = M::run(u32x4{lo[0], lo[1], hi[0], hi[1]}, pb, acc[u]);
  }
}

// Raise the reference maximum if this tile's maximum exceeds it by more than the threshold.
template <int D>
__device__ inline void update_max(float mx, float c, float& m, float& l,
                                  f32x16 (&acc)[Geo<D>::OT]) {
  const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
  const bool need = mt > m + RESCALE_THRESHOLD;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
    // Rows that keep their maximum keep their state (alpha = 1): one of them may still be at
    // m = -inf (no visible key yet), where exp2(m - m) would be NaN. A raised row from
    // m = -inf gets alpha = exp2(-inf) = 0.
    const float mnew = need ? mt : m;
    const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;
    l *= alpha;
#pragma unroll
    for (int u = 0; u < Geo<D>::OT; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][r] *= alpha;
    m = mnew;
  }
}

// DH is the head dimension of the tensors; head dimensions below 64 run the D = 64 geometry with
// the missing 16-byte chunks of every row zero-filled (their lanes' loads are out of range) and
// never stored: zero chunks add nothing to Q.K and give zero O columns. The work per score is
// then that of D = 64, which is bound by the softmax's VALU work, not by the MFMAs.
template <int DT, int DH, bool CAUSAL, int MK, bool SPLIT>
__device__ __forceinline__ void attn_fwd_body(const Params& p) {
  constexpr int D = DH < 64 ? 64 : DH;   // geometry
  constexpr int DCH = DH / 8;            // 16-byte chunks of a row that exist
  using G = Geo<D>;
  using M = Mfma<DT>;
  using MG = MaskGeo<MK>;
  constexpr int KSTEPS = G::KSTEPS;
  constexpr int OT = G::OT;
  constexpr int MOFF = G::LDS;   // mask slots follow the K/V tiles
  __shared__ __attribute__((aligned(1024))) unsigned char smem[G::LDS + kWaves * MG::WB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;          // which half of the wave
  const int ql = lane & 31;

  // ---- work decomposition
  int qt, b, hq, chunk = 0;
  if constexpr (SPLIT) {
    // small grids: (batch, query head) major, longest query tiles first, chunks minor
    const int wid = blockIdx.x;
    const int rest = wid / p.nchunk;
    chunk = wid - rest * p.nchunk;
    const int bhh = rest / p.nqt;
    const int qi = rest - bhh * p.nqt;
    qt = CAUSAL ? p.nqt - 1 - qi : qi;
    b = bhh / p.Hq;
    hq = bhh - b * p.Hq;
  } else {
    const int wid = blockIdx.x;
    if (p.xcd_order) {
      const int xcd = wid & 7;
      const int local = wid >> 3;
      const int per_head = p.group * p.nqt;
      const int head_local = local / per_head;
      const int r = local - head_local * per_head;
      const int kv_head = head_local * 8 + xcd;          // in [0, B * Hkv)
      const int qi = r / p.group;
      qt = CAUSAL ? p.nqt - 1 - qi : qi;
      b = kv_head / p.Hkv;
      hq = (kv_head - b * p.Hkv) * p.group + (r - qi * p.group);
    } else {
      const int BH = p.B * p.Hq;
      const int qi = wid / BH;
      const int bh = wid - qi * BH;
      qt = CAUSAL ? p.nqt - 1 - qi : qi;
      b = bh / p.Hq;
      hq = bh - b * p.Hq;
    }
  }
  const int bh = b * p.Hq + hq;
  const int kvh = hq / p.group;
  const int q0 = qt * kBM;
  const int qa = q0 + wave * 32;            // first query of this wave
  const int qrow = qa + ql;

  // ---- Q fragments: B operand of S^T = K Q^T. Lane l holds Q[row][16s + 8h .. +7]. Rows past
  // N read row N-1 (in bounds; their outputs are never stored). Issued first, so that their
  // latency from HBM overlaps the rest of the set-up; the sign/zero masks are applied after the
  // prologue's wait.
  const uint16_t* __restrict__ qsrc =
      p.q + b * p.qs_b + hq * p.qs_h + min(qrow, p.N - 1) * p.qs_n + 8 * h;
  u32x4 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    qf[s] = (DCH < G::CH && 2 * s + h >= DCH) ? u32x4{} : *(const u32x4*)(qsrc + 16 * s);

  int kv_end = p.N;
  if (p.valid_len) kv_end = min(max(p.valid_len[b], 0), p.N);
  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, q0 + kBM);
  const int ntiles = (kv_stop + kBN - 1) / kBN;
  // Key tiles [jb, je) of this workgroup: the whole range, or one chunk of it. A chunk that
  // starts past the range has nothing to do (the merge kernel counts the same chunks).
  int jb = 0, je = ntiles;
  if constexpr (SPLIT) {
    jb = chunk * p.split_tiles;
    je = min(jb + p.split_tiles, ntiles);
    if (jb >= je) return;
  }

  // K and V of this (batch, KV head) as buffers spanning exactly its N rows: rows past N read
  // as zeros. Row strides in bytes (the host keeps every span below 2^31 bytes).
  const uint32_t krow = (uint32_t)p.ks_n * 2, vrow = (uint32_t)p.vs_n * 2;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k + b * p.ks_b + kvh * p.ks_h), (short)0, (p.N - 1) * krow + 2 * DH,
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.v + b * p.vs_b + kvh * p.vs_h), (short)0, (p.N - 1) * vrow + 2 * DH,
      kBufferFlags);
  // A lane whose global chunk does not exist (DH < 64) fetches from 2^31, past every buffer
  // (the host keeps each span and scalar tile offset below 2^31), and so writes zeros to LDS.
  constexpr uint32_t kNoChunk = 0x80000000u;

  // ---- DMA offsets: block (wave * LOADS + i) of a tile holds rows [blk * RPB, +RPB); lane
  // writes LDS chunk (lane % CH) of row (lane / CH) and fetches the global chunk that the row's
  // swizzle maps there. V's swizzle depends on row & 3 only, the same in every block.
  // With 512-byte rows (D = 256) a block holds 2 rows and V's swizzle differs between blocks:
  // one V offset per block then.
  constexpr bool VSHARED = G::RPB % 4 == 0;
  uint32_t koff[G::LOADS], voff[VSHARED ? 1 : G::LOADS];
#pragma unroll
  for (int i = 0; i < G::LOADS; ++i) {
    const int row = (wave * G::LOADS + i) * G::RPB + lane / G::CH;
    const int gc = (lane % G::CH) ^ G::kswz(row);
    koff[i] = (DCH < G::CH && gc >= DCH) ? kNoChunk : row * krow + gc * 16;
  }
#pragma unroll
  for (int i = 0; i < (VSHARED ? 1 : G::LOADS); ++i) {
    // VSHARED: block 0's row, the blocks' row offsets go into the scalar offset
    const int row = (wave * G::LOADS + i) * G::RPB + lane / G::CH;
    const int gc = (lane % G::CH) ^ G::vswz(row);
    voff[i] = (DCH < G::CH && gc >= DCH) ? kNoChunk : row * vrow + gc * 16;
  }
  // D <= 128 issues the DMA through inline asm at scalar LDS addresses; D = 256 keeps the
  // builtin (its unpipelined loop reads no V before computing the scores).
  const uint32_t sbase = lds_base(smem);
  auto dma_one = [&](__amdgpu_buffer_rsrc_t rs, int dst, uint32_t voff_, uint32_t soff) {
    if constexpr (D <= 128)
      dma16_at(rs, sbase + (uint32_t)dst, voff_, soff);
    else
      dma16(rs, smem + dst, voff_, soff);
  };
  auto dma = [&](int tile, int kdst, int vdst) {
    const uint32_t row0 = (uint32_t)tile * kBN;
#pragma unroll
    for (int i = 0; i < G::LOADS; ++i) {
      const int blk = (wave * G::LOADS + i) * 1024;
      if (kdst >= 0) dma_one(krs, kdst + blk, koff[i], row0 * krow);
      if (vdst >= 0)
        dma_one(vrs, vdst + blk, voff[VSHARED ? 0 : i], (row0 + (VSHARED ? i * G::RPB : 0)) * vrow);
    }
  };

  // ---- explicit mask: this wave's rows qa .. qa+31 of the (batch, query head) mask matrix as a
  // buffer spanning its N rows, the last one up to its next 16-byte boundary (rows past N read
  // as zeros; key columns past N are read but those keys are hidden anyway).
  const uint32_t mrow = MK != kMaskNone ? (uint32_t)(p.ms_n * MG::ES) : 0;
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      MK != kMaskNone ? (void*)((const unsigned char*)p.mask + (b * p.ms_b + hq * p.ms_h) * MG::ES)
                      : (void*)p.q,
      (short)0, MK != kMaskNone ? (p.N - 1) * mrow + ((p.N * MG::ES + 15) & ~15) : 0,
      kBufferFlags);
  uint32_t moff = 0;
  if constexpr (MK != kMaskNone) {
    const int r = lane / MG::CPR;            // row within a DMA block
    moff = (uint32_t)(qa + r) * mrow + 16 * ((lane % MG::CPR) ^ MG::mswz(r));
  }
  auto mask_dma = [&](int tile) {
    if constexpr (MK != kMaskNone) {
#pragma unroll
      for (int i = 0; i < MG::LOADS; ++i)
        dma_one(mrs, MOFF + wave * MG::WB + i * 1024, moff,
                (uint32_t)tile * MG::RB + (uint32_t)(i * MG::RPL) * mrow);
    }
  };

  // ---- LDS fragment offsets (see the swizzles in Geo)
  Frag<D> f;
  {
    // K: lane reads row ql (+32 for the second half), logical chunk 2s + h.
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      f.kaddr[ks] = ql * G::ROW + 16 * ((2 * ks + h) ^ G::kswz(ql));
    // V^T via ds_read_b64_tr_b16: lane 16g + jj reads row 4(g/2) + jj/4 (+16s, +8 for the
    // second 4 keys), columns 32u + 16(g%2) + 4(jj%4) .. +3, i.e. logical chunk
    // 4u + 2(g%2) + (jj%4)/2 and byte 8(jj%2) within it.
    const int g = lane >> 4;
    const int jj = lane & 15;
    const int row = 4 * (g >> 1) + (jj >> 2);
#pragma unroll
    for (int u = 0; u < OT; ++u)
      f.vaddr[u] = row * G::ROW + 16 * ((4 * u + 2 * (g & 1) + ((jj & 3) >> 1)) ^ G::vswz(row)) +
                   8 * (jj & 1);
  }


  f32x16 acc[OT];
#pragma unroll
  for (int u = 0; u < OT; ++u) acc[u] = f32x16{};
  float m = -INFINITY;    // running reference maximum, log2 units
  float l = 0.f;          // this lane's part of the running denominator
  const float c = p.c;

  // Row maximum (raw score units, both lanes of a query pair) of a score tile.
  auto rowmax = [&](const f32x16 (&sv)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[t][r]);
    return pair_max(mx);
  };

  // Tile j: softmax, O += P V, and (HAS_NEXT) the scores of tile j+1, as an explicit program of
  // 4 * SPS slots with one MFMA each (sched_barrier keeps the compiler from moving work across
  // slots):
  //   * the scores of tile j+1 (QK, both 32-key halves alternating so that consecutive MFMAs
  //     are independent) and O += P_s V_s for the four 16-key steps s of tile j interleave, QPS
  //     QK slots then OT PV slots per step;
  //   * K and V fragments are read from LDS three slots of their kind ahead of their MFMA;
  //   * the wave raises its issue priority for the program, so that of two waves sharing a
  //     SIMD the one inside its MFMA stream is served first;
  //   * the probabilities P_s of tile j are computed in the SPS slots before PV step s (P_0 in
  //     the QK slots of step 0), so the exponentials run under the MFMAs; with fp16 inputs
  //     the rounded P_s is summed in the PV slots of step s;
  //   * the row maximum of tile j+1 is taken under the last PV MFMAs.
  // Scores of hidden keys arrive as -inf (see mask_tile), whose exponential is exactly 0;
  // c > 0 always (scale 0 runs with Q = 0). mxc is the row maximum of tile j; mxn returns that
  // of tile j+1 (before any masking of tile j+1).
  auto tile = [&](auto has_next, const f32x16 (&sc)[2], float mxc, f32x16 (&sn)[2],
                  float& mxn, const unsigned char* kbuf, const unsigned char* vbuf) {
    constexpr bool HAS_NEXT = decltype(has_next)::value;
    update_max<D>(mxc, c, m, l, acc);
    const float mneg = (m == -INFINITY) ? 0.f : -m;
    float lsum = 0.f, pend1 = 0.f, pend2 = 0.f;
    // fp16: the denominator is the sum of the rounded weights that multiply V, two per dot2
    // (relative error of each weight at most 2^-11, so the LSE moves by at most ~5e-4); bf16
    // weights round 4x coarser, so bf16 sums the fp32 exponentials one add each.
    constexpr bool RSUM = DT == ATTN_F16;
    auto psum = [&](u32x4 pk, int i) {
      // (the element is copied out first: a bit cast of the element expression itself
      // compiles to a read of element 0)
      const uint32_t w = pk[i];
      lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w),
                                    f16x2{(_Float16)1.0f, (_Float16)1.0f}, lsum, false);
    };
    auto prob = [&](f32x8& pe, int ps, int e) {
      const float ex =
          __builtin_amdgcn_exp2f(__builtin_fmaf(sc[ps >> 1][8 * (ps & 1) + e], c, mneg));
      if constexpr (RSUM) {
        pe[e] = ex;
        return;
      }
      // Add the exponential from two calls (slots) earlier, so that no instruction in a slot
      // waits on one issued in the same slot, and keep the running sum here: otherwise the
      // compiler sinks all the additions past the MFMA stream.
      lsum += pend2;
      pend2 = pend1;
      pend1 = ex;
      asm volatile("" : "+v"(lsum));
      pe[e] = ex;
    };
    if (!HAS_NEXT) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f32x8 pe;
#pragma unroll
        for (int e = 0; e < 8; ++e) prob(pe, s, e);
        const u32x4 pk = M::pack(pe);
        if constexpr (RSUM)
#pragma unroll
          for (int i = 0; i < 4; ++i) psum(pk, i);
        pv_step<DT, D>(acc, vbuf, f, s, pk);
      }
      l += lsum + pend1 + pend2;
      return;
    }
    constexpr int NQK = 2 * KSTEPS;   // score MFMAs of one tile
    constexpr int QPS = NQK / 4;      // ... per PV step
    constexpr int SPS = QPS + OT;     // slots per PV step
    u32x4 kf[NQK];
    u32x4 vf[4 * OT];
    u32x4 pb[4];
    f32x8 pe;
    float mx = -INFINITY;
    auto kload = [&](int idx) {
      const int t = idx & 1, ks = idx >> 1;
      kf[idx] = *(const u32x4*)(kbuf + f.kaddr[ks] + t * 32 * G::ROW);
    };
    auto vload = [&](int pvi) {
      const int s = pvi / OT, u = pvi % OT;
      const unsigned char* base = vbuf + f.vaddr[u] + 16 * s * G::ROW;
      const u32x2 lo = lds_read_tr16(base);
      const u32x2 hi = lds_read_tr16(base + 8 * G::ROW);
      vf[pvi] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    __builtin_amdgcn_s_setprio(1);
    kload(0);
    kload(1);
    kload(2);
    vload(0);
    vload(1);
    vload(2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 4 * SPS; ++g) {
      const int s = g / SPS, k = g % SPS;
      if (k < QPS) {
        const int idx = s * QPS + k;
        if (idx + 3 < NQK) kload(idx + 3);
        sn[idx & 1] = M::run(kf[idx], qf[idx >> 1], idx < 2 ? f32x16{} : sn[idx & 1]);
      } else {
        const int u = k - QPS, pvi = s * OT + u;
        if (pvi + 3 < 4 * OT) vload(pvi + 3);
        acc[u] = M::run(vf[pvi], pb[s], acc[u]);
        if constexpr (RSUM)
#pragma unroll
          for (int i = u * 4 / OT; i < (u + 1) * 4 / OT; ++i) psum(pb[s], i);
      }
      int ps, e0, ne;
      if (g < QPS) {
        ps = 0;
        ne = 8 / QPS;
        e0 = g * ne;
      } else {
        ps = (g + OT) / SPS;
        ne = SPS <= 8 ? 8 / SPS : 1;   // D = 256: one per slot in the first 8 of SPS = 16
        e0 = (g - (ps * SPS - OT)) * ne;
      }
      if (ps < 4 && e0 < 8) {
#pragma unroll
        for (int e = e0; e < e0 + ne; ++e) prob(pe, ps, e);
        if (e0 + ne == 8) pb[ps] = M::pack(pe);
      }
      if (s == 3 && k >= QPS) {
        const int u = k - QPS;
        if (u == 0)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sn[0][r]);
        if (u == OT / 2)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sn[1][r]);
        if (u == OT - 1) mxn = pair_max(mx);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    l += lsum + pend1 + pend2;
  };

  // ---- prologue: K_0, V_0 (and, software-pipelined, K_1) in flight; scores of tile 0
  if (je > jb) dma(jb, G::K0, G::V0);
  if (D <= 128 && je > jb + 1) dma(jb + 1, G::K1, -1);
  if (je > jb) mask_dma(jb);
  wait_loads_and_lds();
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) qf[s] = (qf[s] ^ p.qsign) & p.qmask;
  __syncthreads();
  f32x16 sA[2], sB[2];
  float mxA = -INFINITY, mxB = -INFINITY;
  if (D <= 128 && je > jb) {
    qk_tile<DT, D>(sA, smem + G::K0, f, qf);
    mxA = rowmax(sA);
  }

  // Tiles that straddle the causal diagonal (for this wave's 32 queries), valid_len or N: set
  // the scores of hidden keys to -inf in place and recompute the row maximum. A tile wholly
  // hidden from this wave (above its diagonal) becomes all -inf and adds exactly nothing.
  // key = kb + 32t + 8(r/4) + 4h + r%4 is visible iff key - kb - 4h <= lim.
  // With an explicit mask every tile takes the per-element path: the wave reads its mask slice
  // of tile j from its LDS slot (the DMA of step j-1 has landed: the step's wait covered it),
  // starts the DMA of tile j+1 into the same slot, and keeps a key iff the mask, causality and
  // valid_len all allow it; an additive value is folded into the raw score before the selects,
  // so that nothing from a hidden key (even a non-finite mask value) reaches the softmax.
  auto mask_tile = [&](f32x16 (&sc)[2], float& mxc, int kb, int j) {
    if constexpr (MK != kMaskNone) {
      const unsigned char* mr = smem + MOFF + wave * MG::WB + ql * MG::RB;
      uint32_t mw[8][2];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        // keys 8g + 4h .. +3 of this query's row slice
        if constexpr (MK == kMaskKeep) {
          mw[g][0] = *(const uint32_t*)(mr + 16 * ((g >> 1) ^ MG::mswz(ql)) + 8 * (g & 1) +
                                        4 * h);
        } else {
          const u32x2 w = *(const u32x2*)(mr + 16 * (g ^ MG::mswz(ql)) + 8 * h);
          mw[g][0] = w[0];
          mw[g][1] = w[1];
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (j + 1 < je) mask_dma(j + 1);
      if constexpr (MK == kMaskKeep) {
        // A tile whose keep bytes are all nonzero for every lane of the wave, and which no
        // causal, valid_len or N boundary crosses, needs nothing (a window or block mask keeps
        // most tiles whole). (w - 0x01..01) & ~w & 0x80..80 is nonzero iff w has a zero byte.
        // A tile with no nonzero keep byte in any lane is wholly hidden: all its scores -inf.
        uint32_t z = 0, any = 0;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          z |= (mw[g][0] - 0x01010101u) & ~mw[g][0] & 0x80808080u;
          any |= mw[g][0];
        }
        const bool pos_full = (!CAUSAL || kb + kBN - 1 <= qa) && kb + kBN <= kv_end;
        if (pos_full && __builtin_amdgcn_ballot_w64(z != 0) == 0) return;
        if (__builtin_amdgcn_ballot_w64(any != 0) == 0) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[t][r] = -INFINITY;
          mxc = -INFINITY;
          return;
        }
      }
      if constexpr (MK == kMaskAdd) {
        // Fold the additive values into every score, then hide keys by position only where a
        // causal, valid_len or N boundary crosses the tile.
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int g = 4 * t + (r >> 2), e = r & 3;
            const uint32_t bits = (mw[g][e >> 1] >> (16 * (e & 1))) & 0xffffu;
            const float a = DT == ATTN_BF16
                                ? __uint_as_float(bits << 16)
                                : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
            sc[t][r] = __builtin_fmaf(a, p.mscale, sc[t][r]);
          }
        if (!((!CAUSAL || kb + kBN - 1 <= qa) && kb + kBN <= kv_end)) {
          int lim = kv_end - 1 - kb - 4 * h;
          if (CAUSAL) lim = min(lim, qrow - kb - 4 * h);
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              sc[t][r] = (32 * t + 8 * (r >> 2) + (r & 3) <= lim) ? sc[t][r] : -INFINITY;
        }
      } else {
        int lim = kv_end - 1 - kb - 4 * h;
        if (CAUSAL) lim = min(lim, qrow - kb - 4 * h);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int g = 4 * t + (r >> 2), e = r & 3;
            const bool vis = 32 * t + 8 * (r >> 2) + e <= lim &&
                             ((mw[g][0] >> (8 * e)) & 0xffu) != 0;
            sc[t][r] = vis ? sc[t][r] : -INFINITY;
          }
      }
      mxc = rowmax(sc);
      return;
    }
    (void)j;
    const bool full = (!CAUSAL || kb + kBN - 1 <= qa) && kb + kBN <= kv_end;
    if (!full) {
      int lim = kv_end - 1 - kb - 4 * h;
      if (CAUSAL) lim = min(lim, qrow - kb - 4 * h);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[t][r] = (32 * t + 8 * (r >> 2) + (r & 3) <= lim) ? sc[t][r] : -INFINITY;
      mxc = rowmax(sc);
    }
  };

  // One iteration: tile j (parity P = j & 1) lives in K[P] / V[P] and its scores in cur;
  // K_{j+1} is in K[P^1]. Every wave of the workgroup runs every tile, so the loop has one code
  // path (apart from the rare masking and rescale branches).
  auto step = [&](int j, auto parity, auto has_next, f32x16 (&cur)[2], float& mxc,
                  f32x16 (&nxt)[2], float& mxn) {
    constexpr int P = decltype(parity)::value;
    constexpr int KCUR = P ? G::K1 : G::K0;
    constexpr int KNXT = P ? G::K0 : G::K1;
    constexpr int VCUR = P ? G::V1 : G::V0;
    constexpr int VNXT = P ? G::V0 : G::V1;
    wait_loads_and_lds();
    __syncthreads();
    // K_{j+2} replaces K_j (its scores were computed last iteration); V_{j+1} replaces V_{j-1}.
    if (j + 2 < je) dma(j + 2, KCUR, -1);
    if (j + 1 < je) dma(j + 1, -1, VNXT);
    mask_tile(cur, mxc, j * kBN, j);
    tile(has_next, cur, mxc, nxt, mxn, smem + KNXT, smem + VCUR);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  if constexpr (D > 128) {
    // 512-byte rows: the next tile's scores do not fit beside the 128 accumulator and 64 Q
    // registers, so each step computes its own scores, then the softmax and P V, while the DMA
    // of the next tile's K and V runs.
    auto step1 = [&](int j, auto parity) {
      constexpr int P = decltype(parity)::value;
      wait_loads_and_lds();
      __syncthreads();
      if (j + 1 < je) dma(j + 1, P ? G::K0 : G::K1, P ? G::V0 : G::V1);
      qk_tile<DT, D>(sA, smem + (P ? G::K1 : G::K0), f, qf);
      mxA = rowmax(sA);
      mask_tile(sA, mxA, j * kBN, j);
      tile(F{}, sA, mxA, sB, mxB, nullptr, smem + (P ? G::V1 : G::V0));
    };
    for (int j = jb; j < je; j += 2) {
      step1(j, I0{});
      if (j + 1 < je) step1(j + 1, I1{});
    }
  } else {
    int j = jb;
    for (; j + 2 < je; j += 2) {
      step(j, I0{}, T{}, sA, mxA, sB, mxB);
      step(j + 1, I1{}, T{}, sB, mxB, sA, mxA);
    }
    // Under causal masking the last tile lies wholly above the diagonal of the waves whose last
    // query comes before its first key (the first two waves of a 128-row tile that reaches the
    // diagonal): its scores are all -inf and its softmax and P V add exactly nothing, so such a
    // wave skips them (its scores are computed with the step before, whose single program
    // keeps the register allocation intact). It still waits, joins the barrier and issues its
    // share of the DMA, like every wave, in every step.
    const bool skip_last = CAUSAL && (je - 1) * kBN > qa + 31;
    auto step_sync = [&](int jj, auto parity) {
      constexpr int P = decltype(parity)::value;
      wait_loads_and_lds();
      __syncthreads();
      if (jj + 2 < je) dma(jj + 2, P ? G::K1 : G::K0, -1);
      if (jj + 1 < je) dma(jj + 1, -1, P ? G::V0 : G::V1);
    };
    if (j + 1 < je) {
      step(j, I0{}, T{}, sA, mxA, sB, mxB);
      if (skip_last)
        step_sync(j + 1, I1{});
      else
        step(j + 1, I1{}, F{}, sB, mxB, sA, mxA);
    } else if (j < je) {
      if (skip_last)
        step_sync(j, I0{});
      else
        step(j, I0{}, F{}, sA, mxA, sB, mxB);
    }
  }

  // ---- epilogue: O = acc / l (0 for a row with no visible key), LSE = m ln2 + ln l; each
  // lane stores 16-byte pieces of its own row straight from registers.
  const float lt = pair_sum(l);
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.0f / lt;
  if constexpr (SPLIT) {
    // this chunk's O (normalised by its own sum, fp32) and base-2 LSE, rows of the query tile
    // in order; the merge kernel weighs the chunks by their LSE
    const size_t slot = ((size_t)bh * p.nqt + qt) * p.nchunk + chunk;
    const int r = wave * 32 + ql;
    float* po = p.part_o + (slot * kBM + r) * DH;
#pragma unroll
    for (int u = 0; u < OT; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * u + 8 * r4 + 4 * h;
        if (d < DH)
          *(f32x4*)(po + d) = f32x4{acc[u][4 * r4 + 0] * inv, acc[u][4 * r4 + 1] * inv,
                                    acc[u][4 * r4 + 2] * inv, acc[u][4 * r4 + 3] * inv};
      }
    if (h == 0) p.part_lse[slot * kBM + r] = empty ? -INFINITY : m + __builtin_log2f(lt);
    return;
  }
  // Each lane holds, per 32-column block u, the columns 32u + 8 r4 + 4h .. +3 of its query
  // row (r4 = 0..3). One swap between the two halves of the wave gives lane l < 32 the 16
  // contiguous bytes 32u + 16j .. +7 and lane l + 32 the 16 bytes 32u + 16j + 8 .. +15 of
  // the same row (j = 0, 1): each lane stores them directly, no staging.
  uint16_t* const orow = p.o + b * p.os_b + hq * p.os_h + (size_t)min(qrow, p.N - 1) * p.os_n;
#pragma unroll
  for (int u = 0; u < OT; ++u)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ra = 4 * (2 * j), rc = 4 * (2 * j + 1);
      const uint32_t a0 = (uint32_t)M::round1(acc[u][ra + 0] * inv) |
                          ((uint32_t)M::round1(acc[u][ra + 1] * inv) << 16);
      const uint32_t a1 = (uint32_t)M::round1(acc[u][ra + 2] * inv) |
                          ((uint32_t)M::round1(acc[u][ra + 3] * inv) << 16);
      const uint32_t c0 = (uint32_t)M::round1(acc[u][rc + 0] * inv) |
                          ((uint32_t)M::round1(acc[u][rc + 1] * inv) << 16);
      const uint32_t c1 = (uint32_t)M::round1(acc[u][rc + 2] * inv) |
                          ((uint32_t)M::round1(acc[u][rc + 3] * inv) << 16);
      const auto x0 = __builtin_amdgcn_permlane32_swap(a0, c0, false, false);
      const auto x1 = __builtin_amdgcn_permlane32_swap(a1, c1, false, false);
      const int d = 32 * u + 16 * j + 8 * h;
      if (qrow < p.N && (DCH == G::CH || d < DH))
        *(u32x4*)(orow + d) = u32x4{x0[0], x1[0], x0[1], x1[1]};
    }
  if (p.lse && h == 0 && qrow < p.N)
    p.lse[(size_t)bh * p.N + qrow] = empty ? -INFINITY : m * kLn2 + logf(lt);
}

// The body uses device-only types (buffer resources), so only the device pass compiles it;
// the host pass needs no more than the kernel's signature to emit its launch stub.
// D = 256 holds 128 KiB of K/V tiles in LDS, one workgroup per CU: one wave per SIMD, which may
// then use the whole register file (256 VGPRs + 256 AGPRs). D <= 64 without an explicit mask
// fits 168 VGPRs (32 KiB of LDS per workgroup): three workgroups per CU, three waves per SIMD
// to share the softmax's VALU work, which bounds these head dimensions.
template <int D, int MK>
constexpr int fwd_waves_per_eu() { return D > 128 ? 1 : (D <= 64 && MK == kMaskNone ? 3 : 2); }

template <int DT, int D, bool CAUSAL, int MK>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_eu<D, MK>(), fwd_waves_per_eu<D, MK>())))
void attn_fwd_kernel(Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
  attn_fwd_body<DT, D, CAUSAL, MK, false>(p);
#endif
}

// One chunk of a query tile's key range per workgroup (no explicit mask): partial results for
// attn_fwd_merge_kernel.
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D > 128 ? 1 : 2, D > 128 ? 1 : 2)))
void attn_fwd_split_kernel(Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
  attn_fwd_body<DT, D, CAUSAL, kMaskNone, true>(p);
#endif
}

// Combination of the chunks of every query row: with the chunks' base-2 LSEs L_c and
// normalised outputs O_c, M = max L_c, w_c = 2^(L_c - M), O = sum w_c O_c / sum w_c and
// LSE = (M + log2 sum w_c) ln 2; a row whose chunks are all empty (L_c = -inf) gets O = 0 and
// LSE = -inf. One thread per 4 consecutive elements of a row.
struct MergeParams {
  const float* part_o;
  const float* part_lse;
  uint16_t* o;
  float* lse;
  const int32_t* valid_len;
  int64_t os_b, os_h, os_n;
  int B, Hq, N, DH, nqt, nchunk, split_tiles;
};

template <int DT, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(MergeParams mp) {
  using M = Mfma<DT>;
  const int per_row = mp.DH / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / per_row;
  if (row >= (int64_t)mp.B * mp.Hq * mp.N) return;
  const int d0 = 4 * (int)(idx - row * per_row);
  const int bh = (int)(row / mp.N);
  const int i = (int)(row - (int64_t)bh * mp.N);
  const int b = bh / mp.Hq;
  const int hq = bh - b * mp.Hq;
  const int qt = i / kBM;
  const int r = i - qt * kBM;
  int kv_end = mp.N;
  if (mp.valid_len) kv_end = min(max(mp.valid_len[b], 0), mp.N);
  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, qt * kBM + kBM);
  const int ntiles = (kv_stop + kBN - 1) / kBN;
  const int nch = (ntiles + mp.split_tiles - 1) / mp.split_tiles;
  const size_t slot0 = ((size_t)bh * mp.nqt + qt) * mp.nchunk;
  float mx = -INFINITY;
  for (int c = 0; c < nch; ++c) mx = fmaxf(mx, mp.part_lse[(slot0 + c) * kBM + r]);
  f32x4 o = f32x4{};
  float lse2 = -INFINITY;
  if (mx != -INFINITY) {
    float ws = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float w = __builtin_amdgcn_exp2f(mp.part_lse[(slot0 + c) * kBM + r] - mx);
      const f32x4 x = *(const f32x4*)(mp.part_o + ((slot0 + c) * kBM + r) * mp.DH + d0);
      ws += w;
      o += w * x;
    }
    o *= 1.0f / ws;
    lse2 = mx + __builtin_log2f(ws);
  }
  const uint32_t w0 = (uint32_t)M::round1(o[0]) | ((uint32_t)M::round1(o[1]) << 16);
  const uint32_t w1 = (uint32_t)M::round1(o[2]) | ((uint32_t)M::round1(o[3]) << 16);
  *(u32x2*)(mp.o + b * mp.os_b + hq * mp.os_h + i * mp.os_n + d0) = u32x2{w0, w1};
  if (mp.lse && d0 == 0)
    mp.lse[(size_t)bh * mp.N + i] = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
}

template <int DT, int D, bool CAUSAL, int MK>
hipError_t launch(const Params& p, int64_t nwg, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<DT, D, CAUSAL, MK>), dim3((unsigned)nwg), dim3(kThreads),
                     0, stream, p);
  return hipGetLastError();
}

template <int DT, int D, bool CAUSAL>
hipError_t launch_split(const Params& p, int64_t nwg, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_split_kernel<DT, D, CAUSAL>), dim3((unsigned)nwg),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int DT>
hipError_t dispatch_split(const Params& p, int D, bool causal, int64_t nwg, hipStream_t s) {
  switch (D) {
    case 16:
      return causal ? launch_split<DT, 16, true>(p, nwg, s)
                    : launch_split<DT, 16, false>(p, nwg, s);
    case 32:
      return causal ? launch_split<DT, 32, true>(p, nwg, s)
                    : launch_split<DT, 32, false>(p, nwg, s);
    case 64:
      return causal ? launch_split<DT, 64, true>(p, nwg, s)
                    : launch_split<DT, 64, false>(p, nwg, s);
    case 256:
      return causal ? launch_split<DT, 256, true>(p, nwg, s)
                    : launch_split<DT, 256, false>(p, nwg, s);
    default:
      return causal ? launch_split<DT, 128, true>(p, nwg, s)
                    : launch_split<DT, 128, false>(p, nwg, s);
  }
}

template <int DT>
hipError_t launch_merge(const MergeParams& mp, bool causal, hipStream_t s) {
  const int64_t n = (int64_t)mp.B * mp.Hq * mp.N * (mp.DH / 4);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (causal)
    hipLaunchKernelGGL((attn_fwd_merge_kernel<DT, true>), grid, dim3(256), 0, s, mp);
  else
    hipLaunchKernelGGL((attn_fwd_merge_kernel<DT, false>), grid, dim3(256), 0, s, mp);
  return hipGetLastError();
}

template <int DT, int MK>
hipError_t dispatch_d(const Params& p, int D, bool causal, int64_t nwg, hipStream_t s) {
  switch (D) {
    case 16:
      return causal ? launch<DT, 16, true, MK>(p, nwg, s) : launch<DT, 16, false, MK>(p, nwg, s);
    case 32:
      return causal ? launch<DT, 32, true, MK>(p, nwg, s) : launch<DT, 32, false, MK>(p, nwg, s);
    case 64:
      return causal ? launch<DT, 64, true, MK>(p, nwg, s) : launch<DT, 64, false, MK>(p, nwg, s);
    case 256:
      return causal ? launch<DT, 256, true, MK>(p, nwg, s) : launch<DT, 256, false, MK>(p, nwg, s);
    default:
      return causal ? launch<DT, 128, true, MK>(p, nwg, s) : launch<DT, 128, false, MK>(p, nwg, s);
  }
}

template <int DT>
hipError_t dispatch_m(const Params& p, int D, bool causal, int mask_type, int64_t nwg,
                      hipStream_t s) {
  if (mask_type == ATTN_MASK_KEEP_U8) return dispatch_d<DT, kMaskKeep>(p, D, causal, nwg, s);
  if (mask_type == ATTN_MASK_ADD) return dispatch_d<DT, kMaskAdd>(p, D, causal, nwg, s);
  return dispatch_d<DT, kMaskNone>(p, D, causal, nwg, s);
}

int validate(const Layout& q, const Layout& k, const Layout& v, const Layout& o,
             const float* lse, int B, int Hq, int Hkv, int N, int D, float scale,
             const int32_t* valid_len, int dtype, const MaskArg& mk = no_mask()) {
  if (!q.ptr || !k.ptr || !v.ptr || !o.ptr) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (N > ATTN_MAX_N) return ATTN_ERR_SHAPE;
  const int64_t ntiles = (int64_t)B * Hq * (((int64_t)N + kBM - 1) / kBM);
  if (ntiles > ATTN_MAX_TILES) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (D != 16 && D != 32 && D != 64 && D != 128 && D != 256) return ATTN_ERR_HEAD_DIM;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  const int es = dtype == ATTN_F32 ? 4 : 2;
  if (!layout_ok(q, D, es) || !layout_ok(k, D, es) || !layout_ok(v, D, es) || !layout_ok(o, D, es))
    return ATTN_ERR_LAYOUT;
  if (!output_disjoint(o, B, Hq, N, D)) return ATTN_ERR_LAYOUT;
  // K and V of one head are read as 32-bit-addressed buffers, including up to one tile of rows
  // past N.
  const int64_t kv_reach = ((int64_t)N + kBN) * std::max(k.sn, v.sn) * es + es * D;
  if (kv_reach > INT32_MAX) return ATTN_ERR_SHAPE;
  const int64_t qbytes = q.span(B, N, D, es), kbytes = k.span(B, N, D, es);
  const int64_t vbytes = v.span(B, N, D, es), obytes = o.span(B, N, D, es);
  const int64_t lbytes = (int64_t)B * Hq * N * 4;
  if (overlaps(o.ptr, obytes, q.ptr, qbytes) || overlaps(o.ptr, obytes, k.ptr, kbytes) ||
      overlaps(o.ptr, obytes, v.ptr, vbytes))
    return ATTN_ERR_ALIAS;
  if (lse && (overlaps(lse, lbytes, q.ptr, qbytes) || overlaps(lse, lbytes, k.ptr, kbytes) ||
              overlaps(lse, lbytes, v.ptr, vbytes) || overlaps(lse, lbytes, o.ptr, obytes)))
    return ATTN_ERR_ALIAS;
  if (valid_len && (overlaps(valid_len, (int64_t)B * 4, o.ptr, obytes) ||
                    (lse && overlaps(valid_len, (int64_t)B * 4, lse, lbytes))))
    return ATTN_ERR_ALIAS;
  if (mk.type != ATTN_MASK_NONE) {
    const int ms = mask_status(mk, N, dtype);
    if (ms != ATTN_OK) return ms;
    const int64_t mbytes = mask_span(mk, B, Hq, N, dtype);
    if (overlaps(o.ptr, obytes, mk.ptr, mbytes) || (lse && overlaps(lse, lbytes, mk.ptr, mbytes)))
      return ATTN_ERR_ALIAS;
  }
  return ATTN_OK;
}

// ---- split of the key range for small grids
// Workgroups the device runs at once: two per CU up to D = 128, one at D = 256 (512 and 256 on
// a whole MI355X).
int resident_slots(int D) { return (D > 128 ? 1 : 2) * device_cus(); }

// Key tiles of query tile qt when every key is visible (the host cannot read valid_len).
int tiles_of(int qt, int N, bool causal) {
  const int nkt = (N + kBN - 1) / kBN;
  return causal ? std::min(2 * (qt + 1), nkt) : nkt;
}

struct Split {
  int tiles = 0;    // key tiles per chunk (0: no split)
  int nchunk = 0;   // chunks per query tile
};

int64_t split_floats(int B, int Hq, int N, int D, const Split& sp) {
  if (sp.tiles == 0) return 0;
  const int64_t slots = (int64_t)B * Hq * ((N + kBM - 1) / kBM) * sp.nchunk;
  return slots * kBM * (D + 1) + 4;
}

// A grid of few query tiles over long key ranges leaves CUs idle and ends when its longest
// query tile ends. Splitting each key range into chunks of `tiles` key tiles gives one workgroup
// per chunk: the smallest chunk for which all chunks still run at once (as far as ws_floats
// holds their partial results). The chunks' outputs then take a second kernel to combine, and
// every workgroup pays a fixed cost (prologue, epilogue, launch) worth several key tiles, so
// the split runs only where the grid fills at most a quarter of the device and the longest key
// range has at least kMinSplitTiles tiles; on the shapes measured below those bounds (e.g.
// B = 2, H = 8, N = 1024, or 256 query tiles of N = 2048 to 4096) it was slower.
constexpr int kMinSplitTiles = 48;

Split choose_split(int B, int Hq, int N, int D, bool causal, int64_t ws_floats) {
  Split sp;
  const int nqt = (N + kBM - 1) / kBM;
  const int64_t items = (int64_t)B * Hq * nqt;
  const int slots = resident_slots(D);
  if (items > slots / 4) return sp;
  int tmax = 0;
  for (int qt = 0; qt < nqt; ++qt) tmax = std::max(tmax, tiles_of(qt, N, causal));
  if (tmax < kMinSplitTiles) return sp;
  for (int ct = 1; ct < tmax; ++ct) {
    int64_t chunks = 0;
    for (int qt = 0; qt < nqt; ++qt) chunks += (tiles_of(qt, N, causal) + ct - 1) / ct;
    chunks *= (int64_t)B * Hq;
    if (chunks > slots) continue;
    Split c;
    c.tiles = ct;
    c.nchunk = (tmax + ct - 1) / ct;
    if (split_floats(B, Hq, N, D, c) <= ws_floats) return c;
  }
  return sp;
}

int run(const Layout& q, const Layout& k, const Layout& v, const Layout& o, float* lse, int B,
        int Hq, int Hkv, int N, int D, float scale, int causal, const int32_t* valid_len,
        int dtype, void* stream, const MaskArg& mk = no_mask(), float* ws = nullptr,
        int64_t ws_floats = 0) {
  const int st = validate(q, k, v, o, lse, B, Hq, Hkv, N, D, scale, valid_len, dtype, mk);
  if (st != ATTN_OK) return st;
  if (dtype == ATTN_F32) {
    F32Params f;
    f.q = (const float*)q.ptr;
    f.k = (const float*)k.ptr;
    f.v = (const float*)v.ptr;
    f.o = (float*)o.ptr;
    f.lse = lse;
    f.valid_len = valid_len;
    f.B = B;
    f.Hq = Hq;
    f.Hkv = Hkv;
    f.N = N;
    f.group = Hq / Hkv;
    f.nqt = (N + kBM - 1) / kBM;
    f.xcd_order = ((int64_t)B * Hkv) % 8 == 0 ? 1 : 0;
    f.qs_b = q.sb; f.qs_h = q.sh; f.qs_n = q.sn;
    f.ks_b = k.sb; f.ks_h = k.sh; f.ks_n = k.sn;
    f.vs_b = v.sb; f.vs_h = v.sh; f.vs_n = v.sn;
    f.os_b = o.sb; f.os_h = o.sh; f.os_n = o.sn;
    f.c = scale == 0.f ? 1.0f : fabsf(scale) * kLog2e;
    f.qmul = scale < 0.f ? -1.0f : (scale == 0.f ? 0.0f : 1.0f);
    f.mask = mk.ptr;
    f.ms_b = mk.sb; f.ms_h = mk.sh; f.ms_n = mk.sn;
    f.mscale = kLog2e / f.c;
    const hipError_t e = launch_fwd_f32(f, D, causal != 0, mk.type, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
  }
  Params p;
  p.q = (const uint16_t*)q.ptr;
  p.k = (const uint16_t*)k.ptr;
  p.v = (const uint16_t*)v.ptr;
  p.o = (uint16_t*)o.ptr;
  p.lse = lse;
  p.valid_len = valid_len;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.group = Hq / Hkv;
  p.nqt = (N + kBM - 1) / kBM;
  p.xcd_order = ((int64_t)B * Hkv) % 8 == 0 ? 1 : 0;
  p.qs_b = q.sb; p.qs_h = q.sh; p.qs_n = q.sn;
  p.ks_b = k.sb; p.ks_h = k.sh; p.ks_n = k.sn;
  p.vs_b = v.sb; p.vs_h = v.sh; p.vs_n = v.sn;
  p.os_b = o.sb; p.os_h = o.sh; p.os_n = o.sn;
  p.mask = mk.ptr;
  p.ms_b = mk.sb; p.ms_h = mk.sh; p.ms_n = mk.sn;
  p.c = fabsf(scale) * kLog2e;
  p.qsign = scale < 0.f ? 0x80008000u : 0u;
  p.qmask = scale == 0.f ? 0u : 0xffffffffu;
  if (scale == 0.f) p.c = 1.0f;
  p.mscale = kLog2e / p.c;
  p.split_tiles = 0;
  p.nchunk = 0;
  p.part_o = p.part_lse = nullptr;
  hipStream_t s = (hipStream_t)stream;
  const Split sp = (ws && mk.type == ATTN_MASK_NONE)
                       ? choose_split(B, Hq, N, D, causal != 0, ws_floats) : Split{};
  if (sp.tiles > 0) {
    const int64_t slots = (int64_t)B * Hq * p.nqt * sp.nchunk;
    p.split_tiles = sp.tiles;
    p.nchunk = sp.nchunk;
    p.part_o = ws;
    p.part_lse = ws + slots * kBM * D;
    hipError_t e = dtype == ATTN_BF16 ? dispatch_split<ATTN_BF16>(p, D, causal != 0, slots, s)
                                      : dispatch_split<ATTN_F16>(p, D, causal != 0, slots, s);
    if (e == hipSuccess) {
      MergeParams mp;
      mp.part_o = p.part_o;
      mp.part_lse = p.part_lse;
      mp.o = p.o;
      mp.lse = lse;
      mp.valid_len = valid_len;
      mp.os_b = o.sb; mp.os_h = o.sh; mp.os_n = o.sn;
      mp.B = B;
      mp.Hq = Hq;
      mp.N = N;
      mp.DH = D;
      mp.nqt = p.nqt;
      mp.nchunk = sp.nchunk;
      mp.split_tiles = sp.tiles;
      e = dtype == ATTN_BF16 ? launch_merge<ATTN_BF16>(mp, causal != 0, s)
                             : launch_merge<ATTN_F16>(mp, causal != 0, s);
    }
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
  }
  const int64_t nwg = (int64_t)B * Hq * p.nqt;
  const hipError_t e =
      dtype == ATTN_BF16 ? dispatch_m<ATTN_BF16>(p, D, causal != 0, mk.type, nwg, s)
                         : dispatch_m<ATTN_F16>(p, D, causal != 0, mk.type, nwg, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" int attn_fwd_validate(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, int B, int Hq, int Hkv, int N, int D,
                                 float scale, int causal, const int32_t* valid_len, int dtype) {
  (void)causal;
  return validate(contiguous(q, Hq, N, D), contiguous(k, Hkv, N, D), contiguous(v, Hkv, N, D),
                  contiguous(out, Hq, N, D), lse, B, Hq, Hkv, N, D, scale, valid_len, dtype);
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                        int Hq, int Hkv, int N, int D, float scale, int causal,
                        const int32_t* valid_len, int dtype, void* stream) {
  return run(contiguous(q, Hq, N, D), contiguous(k, Hkv, N, D), contiguous(v, Hkv, N, D),
             contiguous(out, Hq, N, D), lse, B, Hq, Hkv, N, D, scale, causal, valid_len, dtype,
             stream);
}

extern "C" int attn_fwd_strided_validate(const void* q, const int64_t* q_strides, const void* k,
                                         const int64_t* k_strides, const void* v,
                                         const int64_t* v_strides, const void* out,
                                         const int64_t* out_strides, const float* lse, int B,
                                         int Hq, int Hkv, int N, int D, float scale, int causal,
                                         const int32_t* valid_len, int dtype) {
  (void)causal;
  return validate(strided(q, q_strides, Hq, N, D), strided(k, k_strides, Hkv, N, D),
                  strided(v, v_strides, Hkv, N, D), strided(out, out_strides, Hq, N, D), lse, B,
                  Hq, Hkv, N, D, scale, valid_len, dtype);
}

extern "C" int attn_fwd_strided(const void* q, const int64_t* q_strides, const void* k,
                                const int64_t* k_strides, const void* v,
                                const int64_t* v_strides, void* out, const int64_t* out_strides,
                                float* lse, int B, int Hq, int Hkv, int N, int D, float scale,
                                int causal, const int32_t* valid_len, int dtype, void* stream) {
  return run(strided(q, q_strides, Hq, N, D), strided(k, k_strides, Hkv, N, D),
             strided(v, v_strides, Hkv, N, D), strided(out, out_strides, Hq, N, D), lse, B, Hq,
             Hkv, N, D, scale, causal, valid_len, dtype, stream);
}

namespace {


}  // namespace

namespace {

// attn_fwd_ws's checks beyond those of attn_fwd_strided: the part of the workspace the split
// uses is 16-byte aligned and overlaps no input or output.
int validate_ws(const Layout& q, const Layout& k, const Layout& v, const Layout& o,
                const float* lse, const float* ws, int64_t ws_floats, int B, int Hq, int Hkv,
                int N, int D, float scale, int causal, const int32_t* valid_len, int dtype) {
  const int st = validate(q, k, v, o, lse, B, Hq, Hkv, N, D, scale, valid_len, dtype);
  if (st != ATTN_OK) return st;
  if (ws_floats < 0) return ATTN_ERR_WORKSPACE;
  if (!ws || dtype == ATTN_F32) return ATTN_OK;
  if ((uintptr_t)ws % 16 != 0) return ATTN_ERR_LAYOUT;
  const int64_t used = 4 * split_floats(B, Hq, N, D, choose_split(B, Hq, N, D, causal != 0,
                                                                    ws_floats));
  if (used == 0) return ATTN_OK;
  const int es = 2;
  const void* other[] = {q.ptr, k.ptr, v.ptr, o.ptr, lse, valid_len};
  const int64_t size[] = {q.span(B, N, D, es), k.span(B, N, D, es), v.span(B, N, D, es),
                          o.span(B, N, D, es), (int64_t)B * Hq * N * 4, (int64_t)B * 4};
  for (int i = 0; i < 6; ++i)
    if (other[i] && overlaps(ws, used, other[i], size[i])) return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

}  // namespace

extern "C" int64_t attn_fwd_workspace_floats(int B, int Hq, int Hkv, int N, int D, int causal) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1) return -1;
  return split_floats(B, Hq, N, D, choose_split(B, Hq, N, D, causal != 0, INT64_MAX));
}

extern "C" int attn_fwd_ws_validate(const void* q, const int64_t* q_strides, const void* k,
                                    const int64_t* k_strides, const void* v,
                                    const int64_t* v_strides, const void* out,
                                    const int64_t* out_strides, const float* lse, const float* ws,
                                    int64_t ws_floats, int B, int Hq, int Hkv, int N, int D,
                                    float scale, int causal, const int32_t* valid_len,
                                    int dtype) {
  return validate_ws(strided(q, q_strides, Hq, N, D), strided(k, k_strides, Hkv, N, D),
                     strided(v, v_strides, Hkv, N, D), strided(out, out_strides, Hq, N, D), lse,
                     ws, ws_floats, B, Hq, Hkv, N, D, scale, causal, valid_len, dtype);
}

extern "C" int attn_fwd_ws(const void* q, const int64_t* q_strides, const void* k,
                           const int64_t* k_strides, const void* v, const int64_t* v_strides,
                           void* out, const int64_t* out_strides, float* lse, float* ws,
                           int64_t ws_floats, int B, int Hq, int Hkv, int N, int D, float scale,
                           int causal, const int32_t* valid_len, int dtype, void* stream) {
  const Layout lq = strided(q, q_strides, Hq, N, D), lk = strided(k, k_strides, Hkv, N, D);
  const Layout lv = strided(v, v_strides, Hkv, N, D), lo = strided(out, out_strides, Hq, N, D);
  const int st = validate_ws(lq, lk, lv, lo, lse, ws, ws_floats, B, Hq, Hkv, N, D, scale, causal,
                             valid_len, dtype);
  if (st != ATTN_OK) return st;
  return run(lq, lk, lv, lo, lse, B, Hq, Hkv, N, D, scale, causal, valid_len, dtype, stream,
             no_mask(), ws, ws_floats);
}

extern "C" int attn_fwd_masked_validate(const void* q, const int64_t* q_strides, const void* k,
                                        const int64_t* k_strides, const void* v,
                                        const int64_t* v_strides, const void* out,
                                        const int64_t* out_strides, const float* lse, int B,
                                        int Hq, int Hkv, int N, int D, float scale, int causal,
                                        const int32_t* valid_len, const void* mask,
                                        int mask_type, const int64_t* mask_strides, int dtype) {
  (void)causal;
  return validate(strided(q, q_strides, Hq, N, D), strided(k, k_strides, Hkv, N, D),
                  strided(v, v_strides, Hkv, N, D), strided(out, out_strides, Hq, N, D), lse, B,
                  Hq, Hkv, N, D, scale, valid_len, dtype,
                  mask_arg(mask, mask_type, mask_strides, N));
}

extern "C" int attn_fwd_masked(const void* q, const int64_t* q_strides, const void* k,
                               const int64_t* k_strides, const void* v, const int64_t* v_strides,
                               void* out, const int64_t* out_strides, float* lse, int B, int Hq,
                               int Hkv, int N, int D, float scale, int causal,
                               const int32_t* valid_len, const void* mask, int mask_type,
                               const int64_t* mask_strides, int dtype, void* stream) {
  return run(strided(q, q_strides, Hq, N, D), strided(k, k_strides, Hkv, N, D),
             strided(v, v_strides, Hkv, N, D), strided(out, out_strides, Hq, N, D), lse, B, Hq,
             Hkv, N, D, scale, causal, valid_len, dtype, stream,
             mask_arg(mask, mask_type, mask_strides, N));
}
