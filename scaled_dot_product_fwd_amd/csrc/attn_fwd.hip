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
// CDNA4 mapping (measured lane layouts of v_mfma_f32_32x32x16_{bf16,f16}):
//   * Scores are computed transposed, S^T = K Q^T, so the 32x32 MFMA output column that a lane
//     holds is one query: lane l owns query (l % 32) and 16 of every 32 keys; lanes l and l^32
//     share a query. Row max and row sum are therefore in-lane, plus one permlane32 swap.
//   * Output is accumulated transposed too, O^T = V^T P^T: the S^T accumulator registers, rounded
//     to 16 bits, are the B operand of the second MFMA directly (keys in the order the first
//     MFMA's output layout gives them), and V^T fragments come from row-major V in LDS through
//     the transposing LDS read ds_read_b64_tr_b16.
//   * K and V tiles are double-buffered in LDS with padded rows (no bank conflicts for the
//     128-bit K reads and the transposing V reads); the next tile's global loads are in flight
//     while the current tile is computed.
//   * Causal and padding masks are implicit: tiles wholly above the diagonal or past valid_len
//     are never loaded; only tiles that straddle a boundary apply a per-element mask.
//   * The running maximum is only raised when a tile's maximum exceeds it by more than
//     RESCALE_THRESHOLD (log2 units). Any reference value gives the same final O = acc / l and
//     LSE = m + log2(l) as long as numerator and denominator share it; a bounded stale maximum
//     only keeps probabilities below 2^RESCALE_THRESHOLD, and saves the accumulator rescale on
//     most tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int kBM = 128;        // query rows per workgroup (32 per wave)
constexpr int kBN = 64;         // keys per K/V tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float RESCALE_THRESHOLD = 8.0f;

template <int D>
struct Tile {
  static constexpr int KS = D + 8;    // K row stride in LDS (elements): rows 4 banks apart
  static constexpr int VS = D + 16;   // V row stride in LDS (elements): rows 8 banks apart
  static constexpr int K_ELEMS = kBN * KS;
  static constexpr int V_ELEMS = kBN * VS;
  static constexpr int BUF_ELEMS = K_ELEMS + V_ELEMS;
  static constexpr int LDS_ELEMS = 2 * BUF_ELEMS;
  static constexpr int CHUNKS = D / 8;                      // 16-byte chunks per row
  static constexpr int LOADS = kBN * CHUNKS / kThreads;     // 16-byte loads per thread per tile
  static constexpr int ROWS_PER_PASS = kThreads / CHUNKS;
};

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
  float c;           // |scale| * log2(e)
  uint32_t qsign;    // 0x80008000 when scale < 0: Q is negated (exactly) instead
};

template <int DT>
struct Mfma;

template <>
struct Mfma<ATTN_BF16> {
  __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline u32x4 pack(f32x8 x) {
    return __builtin_bit_cast(u32x4, __builtin_convertvector(x, bf16x8));
  }
  __device__ static inline uint16_t round1(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};

template <>
struct Mfma<ATTN_F16> {
  __device__ static inline f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline u32x4 pack(f32x8 x) {
    return __builtin_bit_cast(u32x4, __builtin_convertvector(x, f16x8));
  }
  __device__ static inline uint16_t round1(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};

// Both members of the lane pair {l, l^32}: returns them in any order.
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline u32x2 lds_read_tr16(const uint16_t* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <int D>
__device__ inline void load_tile(const uint16_t* __restrict__ base, int row0, int N, int tid,
                                 u32x4 (&reg)[Tile<D>::LOADS]) {
  using T = Tile<D>;
  const int c = tid % T::CHUNKS;
  const int r = tid / T::CHUNKS;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i) {
    const int row = row0 + r + i * T::ROWS_PER_PASS;
    if (row < N)
      reg[i] = *(const u32x4*)(base + (size_t)row * D + c * 8);
    else
      reg[i] = u32x4{0, 0, 0, 0};
  }
}

template <int D>
__device__ inline void store_tile(uint16_t* lds, int stride, int tid,
                                  const u32x4 (&reg)[Tile<D>::LOADS]) {
  using T = Tile<D>;
  const int c = tid % T::CHUNKS;
  const int r = tid / T::CHUNKS;
#pragma unroll
  for (int i = 0; i < T::LOADS; ++i)
    *(u32x4*)(lds + (r + i * T::ROWS_PER_PASS) * stride + c * 8) = reg[i];
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(Params p) {
  using T = Tile<D>;
  using M = Mfma<DT>;
  constexpr int KSTEPS = D / 16;   // k-steps of the score MFMA
  constexpr int OT = D / 32;       // 32-row output tiles of O^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[T::LDS_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;          // which half of the wave (which 4-key group in each 8)
  const int ql = lane & 31;

  // Work decomposition: causal tiles in decreasing cost order (the longest start first).
  const int BH = p.B * p.Hq;
  const int bid = blockIdx.x;
  const int qt = CAUSAL ? (p.nqt - 1 - bid / BH) : (bid / BH);
  const int bh = bid % BH;
  const int b = bh / p.Hq;
  const int hq = bh - b * p.Hq;
  const int kvh = hq / p.group;
  const int q0 = qt * kBM;

  int kv_end = p.N;
  if (p.valid_len) kv_end = min(max(p.valid_len[b], 0), p.N);
  int kv_stop = kv_end;
  if (CAUSAL) kv_stop = min(kv_stop, q0 + kBM);
  const int ntiles = (kv_stop + kBN - 1) / kBN;

  const uint16_t* __restrict__ qbase = p.q + (size_t)bh * p.N * D;
  const uint16_t* __restrict__ kbase = p.k + (size_t)(b * p.Hkv + kvh) * p.N * D;
  const uint16_t* __restrict__ vbase = p.v + (size_t)(b * p.Hkv + kvh) * p.N * D;

  // Q fragments: B operand of S^T = K Q^T. Lane l holds Q[row][16s + 8h .. +7].
  const int qa = q0 + wave * 32;            // first query of this wave
  const int qrow = qa + ql;
  u32x4 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    if (qrow < p.N) {
      qf[s] = *(const u32x4*)(qbase + (size_t)qrow * D + 16 * s + 8 * h);
      qf[s] ^= p.qsign;
    } else {
      qf[s] = u32x4{0, 0, 0, 0};
    }
  }

  f32x16 acc[OT];
#pragma unroll
  for (int u = 0; u < OT; ++u) acc[u] = f32x16{};
  float m = -INFINITY;    // running reference maximum, log2 units
  float l = 0.f;          // this lane's part of the running denominator
  const float c = p.c;

  u32x4 kreg[T::LOADS], vreg[T::LOADS];
  if (ntiles > 0) {
    load_tile<D>(kbase, 0, p.N, tid, kreg);
    load_tile<D>(vbase, 0, p.N, tid, vreg);
    store_tile<D>(smem, T::KS, tid, kreg);
    store_tile<D>(smem + T::K_ELEMS, T::VS, tid, vreg);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    const uint16_t* ks = smem + buf * T::BUF_ELEMS;
    const uint16_t* vs = ks + T::K_ELEMS;
    const bool more = j + 1 < ntiles;
    if (more) {
      load_tile<D>(kbase, (j + 1) * kBN, p.N, tid, kreg);
      load_tile<D>(vbase, (j + 1) * kBN, p.N, tid, vreg);
    }
    const int kb = j * kBN;
    // Tile class for this wave's 32 queries.
    const bool hidden = (CAUSAL && kb > qa + 31) || kb >= kv_end;
    if (!hidden) {
      const bool partial = (CAUSAL && kb + kBN - 1 > qa) || kb + kBN > kv_end;
      // ---- S^T = K Q^T: two 32-key halves
      f32x16 sv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sv[t] = f32x16{};
        const uint16_t* krow = ks + (32 * t + ql) * T::KS + 8 * h;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          u32x4 a = *(const u32x4*)(krow + 16 * s);
          sv[t] = M::run(a, qf[s], sv[t]);
        }
      }
      // ---- mask (tiles that straddle the diagonal, valid_len or N only)
      uint32_t vis0 = 0xffffffffu;   // bit (16 t + r): key visible
      if (partial) {
        vis0 = 0;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb + 32 * t + (r >> 2) * 8 + 4 * h + (r & 3);
            const bool ok = key < kv_end && (!CAUSAL || key <= qrow);
            vis0 |= (ok ? 1u : 0u) << (16 * t + r);
            sv[t][r] = ok ? sv[t][r] : -INFINITY;
          }
      }
      // ---- online softmax
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[t][r]);
      mx = pair_max(mx);
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
      const bool need = mt > m + RESCALE_THRESHOLD;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float mnew = need ? mt : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);   // 0 when m = -inf
        l *= alpha;
#pragma unroll
        for (int u = 0; u < OT; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[u][r] *= alpha;
        m = mnew;
      }
      const float mneg = (m == -INFINITY) ? 0.f : -m;
      f32x8 pv[4];
      float lsum = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t][r], c, mneg));
          if (partial) e = ((vis0 >> (16 * t + r)) & 1u) ? e : 0.f;
          lsum += e;
          pv[2 * t + (r >> 3)][r & 7] = e;
        }
      l += lsum;
      // ---- O^T += V^T P^T over four 16-key steps
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 pb = M::pack(pv[s]);
        // V^T fragment for keys 16s + 8e' + 4h + (0..3), e' = 0, 1; lane group g of 16 lanes
        // reads 4 rows x 16 columns.
        const int g = lane >> 4;
        const int jj = lane & 15;
        const int row_a = 16 * s + 4 * (g >> 1) + (jj >> 2);
        const int colb = 16 * (g & 1) + 4 * (jj & 3);
#pragma unroll
        for (int u = 0; u < OT; ++u) {
          const u32x2 lo = lds_read_tr16(vs + row_a * T::VS + 32 * u + colb);
          const u32x2 hi = lds_read_tr16(vs + (row_a + 8) * T::VS + 32 * u + colb);
          const u32x4 a = u32x4{lo[0], lo[1], hi[0], hi[1]};
          acc[u] = M::run(a, pb, acc[u]);
        }
      }
    }
    if (more) {
      uint16_t* nk = smem + (buf ^ 1) * T::BUF_ELEMS;
      store_tile<D>(nk, T::KS, tid, kreg);
      store_tile<D>(nk + T::K_ELEMS, T::VS, tid, vreg);
    }
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (0 for a row with no visible key), LSE = m ln2 + ln l
  const float lt = pair_sum(l);
  if (qrow < p.N) {
    const bool empty = !(lt > 0.f);
    const float inv = empty ? 0.f : 1.0f / lt;
    uint16_t* orow = p.o + ((size_t)bh * p.N + qrow) * D;
#pragma unroll
    for (int u = 0; u < OT; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * u + 8 * r4 + 4 * h;
        uint32_t w0 = (uint32_t)M::round1(acc[u][4 * r4 + 0] * inv) |
                      ((uint32_t)M::round1(acc[u][4 * r4 + 1] * inv) << 16);
        uint32_t w1 = (uint32_t)M::round1(acc[u][4 * r4 + 2] * inv) |
                      ((uint32_t)M::round1(acc[u][4 * r4 + 3] * inv) << 16);
        *(u32x2*)(orow + d0) = u32x2{w0, w1};
      }
    if (p.lse && h == 0)
      p.lse[(size_t)bh * p.N + qrow] = empty ? -INFINITY : m * kLn2 + logf(lt);
  }
}

template <int DT, int D, bool CAUSAL>
hipError_t launch(const Params& p, int64_t nwg, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<DT, D, CAUSAL>), dim3((unsigned)nwg), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <int DT>
hipError_t dispatch_d(const Params& p, int D, bool causal, int64_t nwg, hipStream_t s) {
  if (D == 64) return causal ? launch<DT, 64, true>(p, nwg, s) : launch<DT, 64, false>(p, nwg, s);
  return causal ? launch<DT, 128, true>(p, nwg, s) : launch<DT, 128, false>(p, nwg, s);
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

}  // namespace

extern "C" int attn_fwd_validate(const void* q, const void* k, const void* v, const void* out,
                                 const float* lse, int B, int Hq, int Hkv, int N, int D,
                                 float scale, int causal, const int32_t* valid_len, int dtype) {
  (void)causal;
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (N > ATTN_MAX_N) return ATTN_ERR_SHAPE;
  const int64_t ntiles = (int64_t)B * Hq * (((int64_t)N + kBM - 1) / kBM);
  if (ntiles > ATTN_MAX_TILES) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (!isfinite(scale)) return ATTN_ERR_SCALE;
  const int64_t qbytes = (int64_t)B * Hq * N * D * 2;
  const int64_t kvbytes = (int64_t)B * Hkv * N * D * 2;
  const int64_t lbytes = (int64_t)B * Hq * N * 4;
  if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kvbytes) ||
      overlaps(out, qbytes, v, kvbytes))
    return ATTN_ERR_ALIAS;
  if (lse && (overlaps(lse, lbytes, q, qbytes) || overlaps(lse, lbytes, k, kvbytes) ||
              overlaps(lse, lbytes, v, kvbytes) || overlaps(lse, lbytes, out, qbytes)))
    return ATTN_ERR_ALIAS;
  if (valid_len && (overlaps(valid_len, (int64_t)B * 4, out, qbytes) ||
                    (lse && overlaps(valid_len, (int64_t)B * 4, lse, lbytes))))
    return ATTN_ERR_ALIAS;
  return ATTN_OK;
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                        int Hq, int Hkv, int N, int D, float scale, int causal,
                        const int32_t* valid_len, int dtype, void* stream) {
  const int st =
      attn_fwd_validate(q, k, v, out, lse, B, Hq, Hkv, N, D, scale, causal, valid_len, dtype);
  if (st != ATTN_OK) return st;
  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)out;
  p.lse = lse;
  p.valid_len = valid_len;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.N = N;
  p.group = Hq / Hkv;
  p.nqt = (N + kBM - 1) / kBM;
  p.c = fabsf(scale) * kLog2e;
  p.qsign = scale < 0.f ? 0x80008000u : 0u;
  const int64_t nwg = (int64_t)B * Hq * p.nqt;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = dtype == ATTN_BF16 ? dispatch_d<ATTN_BF16>(p, D, causal != 0, nwg, s)
                                          : dispatch_d<ATTN_F16>(p, D, causal != 0, nwg, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer (q, k, v or out) is NULL";
    case ATTN_ERR_SHAPE:
      return "bad shape: B, Hq, Hkv and N must be >= 1, Hq a multiple of Hkv, within size limits";
    case ATTN_ERR_HEAD_DIM: return "unsupported head dimension: D must be 64 or 128";
    case ATTN_ERR_DTYPE: return "unsupported dtype: must be ATTN_F16 or ATTN_BF16";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_LAUNCH: return "the HIP runtime reported an error at kernel launch";
    case ATTN_ERR_ALIAS: return "out or lse overlaps an input, or out overlaps lse";
    default: return "unknown status";
  }
}

extern "C" int attn_version(void) { return 1; }
