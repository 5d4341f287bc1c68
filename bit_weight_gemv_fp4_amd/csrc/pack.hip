// pack.hip -- load-time packer, unpacker and scale validator for the tiled
// weight layout declared in include/fp4gemv.h, plus the library-info entry points.
//
// The packed layout gives every lane of a wave64 one matrix row and 16 bytes per
// load, so each wave-wide load instruction reads 1 KiB of contiguous HBM: a tile
// of 64 rows x 256 columns is eight (NVFP4/MXFP4) or sixteen (FP8) such 1 KiB
// slices, followed by the lanes' block scales.  The feed's NVFP4 section gives the
// 4.5 bits per weight this spends (4-bit element + one 8-bit scale per 16).
#include "common.hpp"

namespace fp4g {

uint64_t packed_bytes_of(uint32_t format, int64_t d_out, int64_t d_in) {
  if (d_out < 1 || d_in < 32 || d_in % 32 != 0) return 0;
  if (format != FP4G_NVFP4 && format != FP4G_MXFP4 && format != FP4G_FP8_ROW) return 0;
  const int64_t R = row_groups(d_out), C = chunks(d_in);
  uint64_t b = (uint64_t)R * (uint64_t)C * (uint64_t)tile_bytes(format);
  if (format == FP4G_FP8_ROW) b += (uint64_t)R * 64u * 4u;
  return b;
}

fp4g_status check_weight(const fp4g_weight* w, bool want_fp4) {
  if (!w || !w->packed) return FP4G_E_NULL;
  if (w->layout_tag != FP4G_LAYOUT_TILE64x256) return FP4G_E_FORMAT;
  if (want_fp4 && w->format != FP4G_NVFP4 && w->format != FP4G_MXFP4) return FP4G_E_FORMAT;
  if (!want_fp4 && w->format != FP4G_FP8_ROW) return FP4G_E_FORMAT;
  if (w->d_out < 1 || w->d_in < 32 || w->d_in % 32 != 0) return FP4G_E_SHAPE;
  if (!aligned(w->packed, 256)) return FP4G_E_ALIGN;
  if (w->packed_bytes < packed_bytes_of(w->format, w->d_out, w->d_in)) return FP4G_E_SHAPE;
  if (!__builtin_isfinite(w->tensor_scale)) return FP4G_E_FORMAT;
  if (w->format != FP4G_NVFP4 && w->tensor_scale != 1.0f) return FP4G_E_FORMAT;
  return FP4G_OK;
}

namespace {

// One workgroup of 64 threads per tile (g, c); lane l copies row 64g + l.
// dir = 0 packs (logical -> tile), dir = 1 unpacks (tile -> logical).
template <int DIR>
__global__ __launch_bounds__(64) void k_pack_fp4(uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                 uint8_t* __restrict__ packed, int d_out, int d_in, int C,
                                                 int sc_per_tile, int tile) {
  const int g = blockIdx.x / C, c = blockIdx.x % C, l = threadIdx.x;
  const int64_t row = (int64_t)g * 64 + l;
  const bool live = row < d_out;
  uint8_t* t = packed + ((int64_t)g * C + c) * tile;
  const int64_t row_code_bytes = d_in / 2;
  for (int j = 0; j < 8; ++j) {
    const int64_t col_byte = (int64_t)c * 128 + j * 16;  // first logical code byte of slot j
    u32x4* tp = reinterpret_cast<u32x4*>(t + j * 1024 + l * 16);
    const bool valid = live && col_byte < row_code_bytes;
    u32x4* lp = valid ? reinterpret_cast<u32x4*>(codes + row * row_code_bytes + col_byte) : nullptr;
    if (DIR == 0) {
      *tp = valid ? *lp : u32x4{0u, 0u, 0u, 0u};
    } else if (valid) {
      *lp = *tp;
    }
  }
  const int64_t row_scales = d_in / (sc_per_tile == 16 ? 16 : 32);
  for (int i = 0; i < sc_per_tile; ++i) {
    const int64_t blk = (int64_t)c * sc_per_tile + i;
    uint8_t* tp = t + kCodeBytes + l * sc_per_tile + i;
    const bool valid = live && blk < row_scales;
    if (DIR == 0) {
      *tp = valid ? scales[row * row_scales + blk] : (uint8_t)0;
    } else if (valid) {
      scales[row * row_scales + blk] = *tp;
    }
  }
}

template <int DIR>
__global__ __launch_bounds__(64) void k_pack_fp8(uint8_t* __restrict__ codes, float* __restrict__ rs,
                                                 uint8_t* __restrict__ packed, int d_out, int d_in, int R,
                                                 int C) {
  const int g = blockIdx.x / C, c = blockIdx.x % C, l = threadIdx.x;
  const int64_t row = (int64_t)g * 64 + l;
  const bool live = row < d_out;
  uint8_t* t = packed + ((int64_t)g * C + c) * kTileF8;
  for (int j = 0; j < kSlotsFp8; ++j) {
    const int64_t col = (int64_t)c * 256 + j * 16;
    u32x4* tp = reinterpret_cast<u32x4*>(t + j * 1024 + l * 16);
    const bool valid = live && col < d_in;
    u32x4* lp = valid ? reinterpret_cast<u32x4*>(codes + row * (int64_t)d_in + col) : nullptr;
    if (DIR == 0) {
      *tp = valid ? *lp : u32x4{0u, 0u, 0u, 0u};
    } else if (valid) {
      *lp = *tp;
    }
  }
  if (c == 0) {
    float* prs = reinterpret_cast<float*>(packed + (int64_t)R * C * kTileF8) + row;
    if (DIR == 0) {
      *prs = live ? rs[row] : 0.0f;
    } else if (live) {
      rs[row] = *prs;
    }
  }
}

__global__ void k_zero_i64(int64_t* p) { *p = 0; }

// Counts NaN scale codes (NVFP4: E4M3 S.1111.111; MXFP4: E8M0 0xFF) of live
// rows and blocks, or, for FP8_ROW, NaN element codes plus non-finite row scales.
__global__ __launch_bounds__(256) void k_validate(const uint8_t* __restrict__ packed, uint32_t fmt, int d_out,
                                                  int d_in, int R, int C, int64_t* bad) {
  int64_t n = 0;
  const int64_t tiles = (int64_t)R * C;
  const int tile = tile_bytes(fmt);
  if (fmt == FP4G_FP8_ROW) {
    // elements: one thread per (tile, lane, slot) 16-byte group
    const int64_t groups = tiles * 64 * kSlotsFp8;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < groups;
         i += (int64_t)gridDim.x * blockDim.x) {
      const int64_t tix = i / (64 * kSlotsFp8);
      const int rem = (int)(i % (64 * kSlotsFp8));
      const int j = rem / 64, l = rem % 64;
      const int64_t g = tix / C, c = tix % C;
      const int64_t row = g * 64 + l, col = c * 256 + j * 16;
      if (row >= d_out || col >= d_in) continue;
      const uint8_t* p = packed + tix * tile + j * 1024 + l * 16;
      for (int b = 0; b < 16; ++b) n += ((p[b] & 0x7f) == 0x7f);
    }
    const float* rs = reinterpret_cast<const float*>(packed + tiles * tile);
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < d_out;
         r += (int64_t)gridDim.x * blockDim.x)
      n += !__builtin_isfinite(rs[r]);
  } else {
    const int per = fmt == FP4G_NVFP4 ? 16 : 8;
    const int64_t row_blocks = d_in / (fmt == FP4G_NVFP4 ? 16 : 32);
    const int64_t total = tiles * 64 * per;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
      const int64_t tix = i / (64 * per);
      const int rem = (int)(i % (64 * per));
      const int l = rem / per, k = rem % per;
      const int64_t g = tix / C, c = tix % C;
      const int64_t row = g * 64 + l, blk = c * per + k;
      if (row >= d_out || blk >= row_blocks) continue;
      const uint8_t b = packed[tix * tile + kCodeBytes + l * per + k];
      n += fmt == FP4G_NVFP4 ? ((b & 0x7f) == 0x7f) : (b == 0xff);
    }
  }
  // wave reduction then one atomic per wave
  for (int off = 32; off > 0; off >>= 1) n += __shfl_down(n, off, 64);
  if ((threadIdx.x & 63) == 0 && n) atomicAdd(reinterpret_cast<unsigned long long*>(bad), (unsigned long long)n);
}

}  // namespace
}  // namespace fp4g

using namespace fp4g;

extern "C" {

uint32_t fp4g_abi_version(void) { return FP4G_ABI_VERSION; }

const char* fp4g_status_string(int32_t s) {
  switch (s) {
    case FP4G_OK: return "ok";
    case FP4G_E_NULL: return "a required pointer is NULL";
    case FP4G_E_SHAPE: return "bad shape, M, expert count, or buffer size";
    case FP4G_E_ALIGN: return "misaligned pointer (packed: 256 B, vectors: 16 B)";
    case FP4G_E_FORMAT: return "format or layout tag not accepted by this call, or bad scale";
    case FP4G_E_WORKSPACE: return "workspace smaller than fp4g_workspace_bytes()";
    case FP4G_E_PATH: return "requested kernel path does not exist for this call";
    case FP4G_E_ALIAS: return "an output overlaps an input or another output";
    case FP4G_E_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

uint64_t fp4g_packed_bytes(uint32_t format, int32_t d_out, int32_t d_in) {
  return packed_bytes_of(format, d_out, d_in);
}

int32_t fp4g_pack(uint32_t format, int32_t d_out, int32_t d_in, const void* codes_dev, const void* scales_dev,
                  float tensor_scale, void* packed_dev, uint64_t packed_bytes, fp4g_weight* out_host,
                  void* stream) {
  if (!codes_dev || !scales_dev || !packed_dev || !out_host) return FP4G_E_NULL;
  if (format != FP4G_NVFP4 && format != FP4G_MXFP4 && format != FP4G_FP8_ROW) return FP4G_E_FORMAT;
  if (d_out < 1 || d_in < 32 || d_in % 32 != 0) return FP4G_E_SHAPE;
  const uint64_t need = packed_bytes_of(format, d_out, d_in);
  if (packed_bytes < need) return FP4G_E_SHAPE;
  if (!aligned(packed_dev, 256) || !aligned(codes_dev, 16) || !aligned(scales_dev, 4)) return FP4G_E_ALIGN;
  if (!__builtin_isfinite(tensor_scale) || (format != FP4G_NVFP4 && tensor_scale != 1.0f)) return FP4G_E_FORMAT;
  const int64_t code_bytes = format == FP4G_FP8_ROW ? (int64_t)d_out * d_in : (int64_t)d_out * d_in / 2;
  const int64_t scale_bytes = format == FP4G_NVFP4   ? (int64_t)d_out * d_in / 16
                              : format == FP4G_MXFP4 ? (int64_t)d_out * d_in / 32
                                                     : (int64_t)d_out * 4;
  if (overlap(codes_dev, code_bytes, packed_dev, need) || overlap(scales_dev, scale_bytes, packed_dev, need))
    return FP4G_E_ALIAS;
  const int R = (int)row_groups(d_out), C = (int)chunks(d_in);
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = (unsigned)((int64_t)R * C);
  uint8_t* codes = (uint8_t*)const_cast<void*>(codes_dev);
  if (format == FP4G_FP8_ROW) {
    k_pack_fp8<0><<<grid, 64, 0, s>>>(codes, (float*)const_cast<void*>(scales_dev), (uint8_t*)packed_dev, d_out,
                                      d_in, R, C);
  } else {
    k_pack_fp4<0><<<grid, 64, 0, s>>>(codes, (uint8_t*)const_cast<void*>(scales_dev), (uint8_t*)packed_dev, d_out,
                                      d_in, C, format == FP4G_NVFP4 ? 16 : 8, tile_bytes(format));
  }
  if (hipGetLastError() != hipSuccess) return FP4G_E_HIP;
  out_host->format = format;
  out_host->layout_tag = FP4G_LAYOUT_TILE64x256;
  out_host->d_out = d_out;
  out_host->d_in = d_in;
  out_host->packed = packed_dev;
  out_host->packed_bytes = packed_bytes;
  out_host->tensor_scale = tensor_scale;
  out_host->reserved = 0;
  return FP4G_OK;
}

int32_t fp4g_unpack(const fp4g_weight* w, void* codes_dev, void* scales_dev, void* stream) {
  if (!w || !codes_dev || !scales_dev) return FP4G_E_NULL;
  fp4g_status st = check_weight(w, w->format != FP4G_FP8_ROW);
  if (st != FP4G_OK) return st;
  if (!aligned(codes_dev, 16) || !aligned(scales_dev, 4)) return FP4G_E_ALIGN;
  const int64_t d_out = w->d_out, d_in = w->d_in;
  const int64_t code_bytes = w->format == FP4G_FP8_ROW ? d_out * d_in : d_out * d_in / 2;
  const int64_t scale_bytes = w->format == FP4G_NVFP4   ? d_out * d_in / 16
                              : w->format == FP4G_MXFP4 ? d_out * d_in / 32
                                                        : d_out * 4;
  if (overlap(codes_dev, code_bytes, w->packed, w->packed_bytes) ||
      overlap(scales_dev, scale_bytes, w->packed, w->packed_bytes) ||
      overlap(codes_dev, code_bytes, scales_dev, scale_bytes))
    return FP4G_E_ALIAS;
  const int R = (int)row_groups(d_out), C = (int)chunks(d_in);
  hipStream_t s = (hipStream_t)stream;
  const unsigned grid = (unsigned)((int64_t)R * C);
  uint8_t* packed = (uint8_t*)const_cast<void*>(w->packed);
  if (w->format == FP4G_FP8_ROW) {
    k_pack_fp8<1><<<grid, 64, 0, s>>>((uint8_t*)codes_dev, (float*)scales_dev, packed, w->d_out, w->d_in, R, C);
  } else {
    k_pack_fp4<1><<<grid, 64, 0, s>>>((uint8_t*)codes_dev, (uint8_t*)scales_dev, packed, w->d_out, w->d_in, C,
                                      w->format == FP4G_NVFP4 ? 16 : 8, tile_bytes(w->format));
  }
  return hipGetLastError() == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

int32_t fp4g_validate(const fp4g_weight* w, int64_t* bad_dev, void* stream) {
  if (!w || !bad_dev) return FP4G_E_NULL;
  fp4g_status st = check_weight(w, w->format != FP4G_FP8_ROW);
  if (st != FP4G_OK) return st;
  if (!aligned(bad_dev, 8)) return FP4G_E_ALIGN;
  if (overlap(bad_dev, 8, w->packed, w->packed_bytes)) return FP4G_E_ALIAS;
  const int R = (int)row_groups(w->d_out), C = (int)chunks(w->d_in);
  hipStream_t s = (hipStream_t)stream;
  k_zero_i64<<<1, 1, 0, s>>>(bad_dev);
  k_validate<<<2048, 256, 0, s>>>((const uint8_t*)w->packed, w->format, w->d_out, w->d_in, R, C, bad_dev);
  return hipGetLastError() == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

}  // extern "C"
