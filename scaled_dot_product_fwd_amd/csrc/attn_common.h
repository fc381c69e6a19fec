// Definitions shared by the forward (attn_fwd.hip) and backward (attn_bwd.hip) kernels for
// CDNA4 (gfx950): vector types, tile geometry and LDS swizzles of the K/V tiles, the 32x32x16
// MFMA wrappers, lane-pair reductions and LDS helpers; on the host, tensor layouts, mask
// arguments and the device's compute-unit count (the only state: one number per device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "attn.h"

namespace attn_detail {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBM = 128;        // query rows per workgroup (32 per wave)
constexpr int kBN = 64;         // keys per K/V tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBufferFlags = 0x00020000;   // raw buffer: dword data, range-checked

// NW: waves sharing the DMA of a tile (the workgroup's waves).
template <int D, int NW = kWaves>
struct Geo {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int ROW = 2 * D;                  // bytes per row
  static constexpr int TILE = kBN * ROW;             // bytes per K or V tile
  static constexpr int LOADS = TILE / 1024 / NW;     // 1 KiB DMA blocks per wave per tile
  static constexpr int RPB = 1024 / ROW;             // rows per 1 KiB block
  static constexpr int KSTEPS = D / 16;              // k-steps of the score MFMA
  static constexpr int OT = D / 32;                  // 32-row tiles of O^T
  static constexpr int K0 = 0, K1 = TILE, V0 = 2 * TILE, V1 = 3 * TILE;
  static constexpr int LDS = 4 * TILE;
  // LDS row r of a tile stores global 16-byte chunk c at chunk c ^ swz(r). The swizzles keep
  // every LDS read phase on distinct banks whether the LDS serves 128 or 256 bytes per clock:
  //  * K is read as 16-byte A fragments, 16 consecutive rows at one logical chunk per phase:
  //    the 16 rows must land in 16 distinct 16-byte bank slots (8 among rows 0..7).
  //  * V is read with ds_read_b64_tr_b16: a 16-lane group reads 4 consecutive rows x 32 bytes,
  //    a 32-lane half the same 4 rows x 64 bytes. XOR of the 32-byte pair index by
  //    F = {0, 3, 5, 6}[r & 3] (D = 128) puts the 4 rows on distinct pairs mod 128 bytes and on
  //    distinct 64-byte blocks mod 256 bytes; with 128-byte rows (D = 64) F = r & 3 does both.
  //  Rows of 256 bytes or more (D >= 128) start on the same bank; rows of 128 bytes (D = 64)
  //  alternate between the two halves of the 256-byte bank set.
  __device__ static constexpr int kswz(int r) {
    return D >= 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
  }
  __device__ static constexpr int vswz(int r) {
    return D >= 128 ? 2 * ((0x6530 >> (4 * (r & 3))) & 15) : 2 * (r & 3);
  }
  //  * A tile read both ways (the backward's K, Q and dO) needs both properties: vswz's pair
  //    XOR on r & 3 for the transposed reads, plus bits that tell apart the 4-row groups of 16
  //    rows for the row reads: the chunk's low bit flips with (r >> 2) & 1 (rows 4..7 of 8 use
  //    the other chunk of each pair) and the pair XOR gains (r >> 3) & 1, which maps the
  //    even-parity set {0, 3, 5, 6} (D = 128) onto the odd one, or shifts F = r & 3 (D = 64).
  //    Rows r and r + 8 therefore differ by chunk XOR 2; rows r and r + 16 share the swizzle.
  __device__ static constexpr int bswz(int r) {
    return D >= 128 ? 2 * (((0x6530 >> (4 * (r & 3))) & 15) ^ ((r >> 3) & 1)) + ((r >> 2) & 1)
                    : 2 * ((r & 3) ^ ((r >> 3) & 1)) + ((r >> 2) & 1);
  }
};

// Explicit [B, H, N, N] masks (template parameter MK of the kernel).
constexpr int kMaskNone = 0;   // causal and valid_len only
constexpr int kMaskKeep = 1;   // uint8: nonzero = the key is visible to the query
constexpr int kMaskAdd = 2;    // the input type (16-bit, or fp32): added to the scaled score

// Each wave keeps the kBN-key slice of its 32 mask rows for the current tile in its own LDS
// slot, fetched by DMA one tile ahead. Row r stores logical 16-byte chunk c at chunk
// c ^ mswz(r); the swizzle depends on r % RPL only, so every DMA block uses the same lane
// offsets.
template <int MK>
struct MaskGeo {
  static constexpr int ES = MK == kMaskKeep ? 1 : 2;            // bytes per element
  static constexpr int RB = kBN * ES;                           // bytes per row slice
  static constexpr int CPR = RB / 16;                           // 16-byte chunks per row slice
  static constexpr int WB = MK == kMaskNone ? 0 : 32 * RB;      // bytes per wave slot
  static constexpr int LOADS = WB / 1024;                       // 1 KiB DMA blocks per slot
  static constexpr int RPL = 1024 / RB;                         // rows per DMA block
  __device__ static constexpr int mswz(int r) {
    return MK == kMaskKeep ? ((r >> 2) & 3) : (r & 7);
  }
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

// permlane32_swap(x, x) returns, in every lane, both members of the lane pair {l, l^32}.
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline u32x2 lds_read_tr16(const unsigned char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ inline void wait_loads_and_lds() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}

// Buffer loads into LDS (16 or 4 bytes per lane, to LDS byte address `lds` + lane * bytes).
// The asm form (ASM = true) exists because the compiler cannot tell a later ds_read_b64_tr_b16
// apart from the DMA's destination and, for the buffer-load-to-LDS builtin, waits for the whole
// DMA before the first such read (measured: the forward's V reads stalled on every tile's
// prefetch). Callers order the asm DMA themselves with an explicit vmcnt wait before reading the
// destination (wait_loads_and_lds at the top of every loop step). The LDS address reaches M0
// through the "{m0}" operand constraint, so the compiler knows M0 is written and sets it itself.
// Addresses are 32-bit LDS byte offsets computed from lds_base() of the kernel's own __shared__
// array: taking a generic pointer back to the LDS address space would cost a null check and a
// v_readfirstlane per load.
// The compiler cannot see the load inside the asm, so it does not insert the wait states the
// hardware needs before it: one after a scalar write of M0 (the compiler sets M0 right before
// the asm), and five after a VALU write (v_readfirstlane, v_readlane restoring a spilled scalar)
// of an SGPR the load reads (the buffer descriptor or the scalar offset). Without them the load
// can use the previous M0 or a stale offset and fill the wrong tile; s_nop 4 gives five.
template <typename T>
__device__ inline uint32_t lds_base(T& shared_array) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(&shared_array);
}

__device__ inline void dma16_at(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff,
                                uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds) : "memory");
}

__device__ inline void dma4_at(__amdgpu_buffer_rsrc_t rs, uint32_t lds, uint32_t voff,
                               uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds) : "memory");
}

// The builtin form, for loops that compute long enough between a DMA and their first transposed
// read (the backward's S and dP products, the unpipelined D = 256 forward) that its wait costs
// nothing measurable.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, unsigned char* lds, uint32_t voff,
                             uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, soff, 0, 0);
}

__device__ inline void dma4(__amdgpu_buffer_rsrc_t rs, unsigned char* lds, uint32_t voff,
                            uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 4, voff, soff, 0, 0);
}

// Per-wave, per-thread state of the main loop (registers).
template <int D>
struct Frag {
  uint32_t kaddr[D / 16];   // LDS byte offsets of this lane's K fragment for each k-step
  uint32_t vaddr[D / 32];   // LDS byte offsets of this lane's V^T fragment for each d-tile u
};

// ---- host-side argument checks shared by the entry points --------------------------------

inline bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// One [B, H, N, D] tensor as (batch, head, row) element strides; rows are D contiguous elements.
struct Layout {
  const void* ptr;
  int64_t sb, sh, sn;
  int64_t H;
  // Bytes from ptr to the end of the last row (elements of es bytes).
  int64_t span(int B, int N, int D, int es) const {
    return ((B - 1) * sb + (H - 1) * sh + (int64_t)(N - 1) * sn + D) * es;
  }
};

inline Layout contiguous(const void* ptr, int H, int N, int D) {
  return Layout{ptr, (int64_t)H * N * D, (int64_t)N * D, (int64_t)D, H};
}

inline Layout strided(const void* ptr, const int64_t* st, int H, int N, int D) {
  if (!st) return contiguous(ptr, H, N, D);
  return Layout{ptr, st[0], st[1], st[2], H};
}

// 16-byte aligned base, non-negative strides that are multiples of 16 bytes, rows of at least
// D elements apart.
inline bool layout_ok(const Layout& t, int D, int es) {
  const int64_t g = 16 / es;   // elements per 16 bytes
  if ((uintptr_t)t.ptr % 16 != 0) return false;
  if (t.sb < 0 || t.sh < 0 || t.sn < 0) return false;
  if (t.sb % g || t.sh % g || t.sn % g) return false;
  return t.sn >= D;
}

// No two (batch, head, row) of an output share an element: ordered by stride, each dimension
// of size > 1 steps past the whole extent of the dimensions below it.
inline bool output_disjoint(const Layout& o, int B, int H, int N, int D) {
  struct Dim { int64_t size, stride; } d[3] = {{B, o.sb}, {H, o.sh}, {N, o.sn}};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (d[j].stride < d[i].stride) {
        const Dim t = d[i];
        d[i] = d[j];
        d[j] = t;
      }
  int64_t extent = D;   // elements spanned by the dimensions below
  for (int i = 0; i < 3; ++i) {
    if (d[i].size <= 1) continue;
    if (d[i].stride < extent) return false;
    extent = (d[i].size - 1) * d[i].stride + extent;
  }
  return true;
}

// An explicit mask: element strides (batch, query head, query row); keys contiguous.
struct MaskArg {
  const void* ptr;
  int type;
  int64_t sb, sh, sn;
};

inline MaskArg no_mask() { return MaskArg{nullptr, ATTN_MASK_NONE, 0, 0, 0}; }

// NULL strides mean one [B, N, N] mask shared by the heads.
inline MaskArg mask_arg(const void* mask, int mask_type, const int64_t* st, int N) {
  if (st) return MaskArg{mask, mask_type, st[0], st[1], st[2]};
  return MaskArg{mask, mask_type, (int64_t)N * N, 0, N};
}

// Bytes per mask element: keep masks are uint8, additive masks have the inputs' type.
inline int64_t mask_es(int type, int dtype) {
  return type == ATTN_MASK_KEEP_U8 ? 1 : (dtype == ATTN_F32 ? 4 : 2);
}

// Type, pointer, layout and size checks of a mask (not its aliasing).
inline int mask_status(const MaskArg& mk, int N, int dtype = ATTN_BF16) {
  if (mk.type != ATTN_MASK_KEEP_U8 && mk.type != ATTN_MASK_ADD) return ATTN_ERR_MASK;
  if (!mk.ptr) return ATTN_ERR_NULL;
  const int64_t es = mask_es(mk.type, dtype);
  if ((uintptr_t)mk.ptr % 16 != 0 || mk.sb < 0 || mk.sh < 0 || mk.sn < N ||
      (mk.sb * es) % 16 || (mk.sh * es) % 16 || (mk.sn * es) % 16)
    return ATTN_ERR_LAYOUT;
  // A wave's DMA addresses rows up to 127 past its first inside one 32-bit buffer.
  if (((int64_t)N + kBM) * mk.sn * es > INT32_MAX) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// Bytes a mask's reads may touch: rows are read in 16-byte units, the last row up to its next
// 16-byte boundary.
inline int64_t mask_span(const MaskArg& mk, int B, int Hq, int N, int dtype = ATTN_BF16) {
  const int64_t es = mask_es(mk.type, dtype);
  return ((B - 1) * mk.sb + (Hq - 1) * mk.sh + (int64_t)(N - 1) * mk.sn) * es +
         ((N * es + 15) & ~15);
}

// fp32 forward (attn_fwd_f32.hip): validated arguments, strides in elements.
struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  const int32_t* valid_len;
  int B, Hq, Hkv, N;
  int group;         // Hq / Hkv
  int nqt;           // ceil(N / kBM)
  int xcd_order;     // 1: KV heads divide evenly over the 8 XCDs
  int64_t qs_b, qs_h, qs_n;
  int64_t ks_b, ks_h, ks_n;
  int64_t vs_b, vs_h, vs_n;
  int64_t os_b, os_h, os_n;
  float c;           // |scale| * log2(e) (1 when scale == 0)
  float qmul;        // sign of scale, 0 when scale == 0: multiplies Q (exact)
  const void* mask;  // explicit mask: uint8 keep or fp32 additive (attn_fwd_masked)
  int64_t ms_b, ms_h, ms_n;   // its element strides (batch, query head, query row)
  float mscale;      // log2(e) / c: an additive mask value in raw score units
};

// Queue the fp32 forward for D in {16, 32, 64, 128, 256} and mask_type an attn_mask_t.
hipError_t launch_fwd_f32(const F32Params& p, int D, bool causal, int mask_type,
                          hipStream_t stream);

// fp32 backward (attn_bwd_f32.hip): validated arguments, strides in elements.
struct F32BwdParams {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;      // workspace row 0: D = rowsum(dO o O)
  float* lse2;       // workspace row 1: L * log2(e) (0 for rows with no visible key)
  const int32_t* valid_len;
  int B, Hq, Hkv, N;
  int group;         // Hq / Hkv
  int nqt, nkt;      // ceil(N / kBM): query tiles (dQ kernel), key tiles (dK/dV kernel)
  int xcd_order;     // 1: KV heads divide evenly over the 8 XCDs
  int64_t qs_b, qs_h, qs_n;
  int64_t ks_b, ks_h, ks_n;
  int64_t vs_b, vs_h, vs_n;
  int64_t os_b, os_h, os_n;
  int64_t gs_b, gs_h, gs_n;
  int64_t dqs_b, dqs_h, dqs_n;
  int64_t dks_b, dks_h, dks_n;
  int64_t dvs_b, dvs_h, dvs_n;
  float c;           // |scale| * log2(e) (1 when scale == 0)
  float qmul;        // sign of scale, 0 when scale == 0: multiplies one operand of the scores
  float scale;       // the signed scale (dQ and dK carry it)
  int split;         // parts per key tile of the dK/dV kernel (1: none; else fp32 partials)
  float* part;       // [2][split][B][Hkv][N][D] partial sums (split > 1)
  const void* mask;  // the forward's explicit mask: uint8 keep or fp32 additive
  int64_t ms_b, ms_h, ms_n;   // its element strides (batch, query head, query row)
  float mscale;      // log2(e) / c: an additive mask value in raw score units
};

// Queue the fp32 backward (dQ kernel, then dK/dV kernel) for D in {16, 32, 64, 128, 256} and
// mask_type an attn_mask_t.
hipError_t launch_bwd_f32(const F32BwdParams& p, int D, bool causal, int mask_type,
                          hipStream_t stream);

// Compute units of the current device: 256 on a whole MI355X, fewer on a partition of one.
// Read once per device; 256 where no device answers (a host without one). Only the launch
// heuristics use it (how many workgroups run at once); no result depends on it.
inline int device_cus() {
  static std::atomic<int> known[64];   // 0: not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int n = known[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  known[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace attn_detail
