// Status strings and the interface version of the C ABI in attn.h (host code only). The codes
// are the argument and launch failures the masked multi-head attention CUDA article describes
// (section 5.2, launch configuration; section 6.2, its table of failure symptoms), reported
// before anything is launched.
#include "attn.h"

extern "C" const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE:
      return "bad shape: B, Hq, Hkv and N must be >= 1, Hq a multiple of Hkv, within size limits";
    case ATTN_ERR_HEAD_DIM:
      return "unsupported head dimension: D must be 16, 32, 64, 128 or 256";
    case ATTN_ERR_DTYPE:
      return "unsupported dtype: ATTN_F16, ATTN_BF16 or ATTN_F32";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_LAUNCH: return "the HIP runtime reported an error at kernel launch";
    case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case ATTN_ERR_LAYOUT:
      return "bad layout: pointers must be 16-byte aligned, strides non-negative multiples of 16 "
             "bytes, rows at least D elements apart, and output rows distinct";
    case ATTN_ERR_MASK: return "unknown mask type";
    case ATTN_ERR_WORKSPACE:
      return "bad workspace size: attn_bwd_ws needs at least 2 * B * Hq * N floats, attn_fwd_ws "
             "a non-negative size";
    case ATTN_ERR_SCRATCH:
      return "the sizes need more than the library's static workspace: 2 * B * Hq * N must be "
             "at most ATTN_SCRATCH_FLOATS (8388608) floats; use attn_bwd_ws";
    default: return "unknown status";
  }
}

extern "C" int attn_version(void) { return 14; }
