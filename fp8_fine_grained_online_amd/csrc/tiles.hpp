// Tile helpers shared by the gfx950 GEMM kernels: MFMA operand types,
// buffer descriptors, direct global -> LDS copies, the LDS chunk swizzle and
// the XCD-aware, banded order of output tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kXcds = 8;
constexpr int kCus = 256;  // compute units (one large-tile workgroup each)

// Byte offset of 16-byte chunk `chunk` of row `row` in an LDS slab of
// 128-byte rows: chunk positions are XOR row % 8, so the 16 rows read by one
// MFMA operand load fall in distinct banks.
__device__ __forceinline__ int swz(int row, int chunk) { return (row * 8 + (chunk ^ (row & 7))) * 16; }

// Raw buffer descriptor over `bytes` bytes at `base` (dword 3: the gfx9
// raw-buffer format word); loads past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct global -> LDS copy: lane l of the wave writes `size` bytes at
// lds + l * size (lds must be wave-uniform).
__device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int size,
                                         uint32_t voffset, uint32_t soffset) {
  if (size == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voffset, soffset, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voffset, soffset, 0, 0);
}

// Workgroup id -> tile index such that each XCD gets a contiguous run.
__device__ __forceinline__ int xcd_tile(int id, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int x = id % kXcds, local = id / kXcds;
  return x * q + (x < r ? x : r) + local;
}

// Tile index -> (row tile, column tile) in bands of kBand row tiles, column
// by column within a band: a run of 32 consecutive tiles (one XCD's share of
// a wave of workgroups) is a 4 x 8 block that reads 4 A slabs and 8 B slabs,
// instead of 2 x 16 (2 A + 16 B slabs) in plain row-major order.
//
// The grouped GEMM uses bands of kBandGrouped row tiles within each expert.
// Its weights (all experts together) stream from HBM while an expert's rows
// of A stay in the Infinity Cache, so a band as tall as a typical expert has
// each weight panel read by all of the expert's row tiles in a row. Bands of
// 16 (at most 4096 rows of A) beat bands of 4 by 4% on 32 experts of ~2100
// rows, measured on MI355X.
constexpr int kBand = 4;
constexpr int kBandGrouped = 16;
template <int kHeight = kBand>
__device__ __forceinline__ void band_tile(int t, int m_tiles, int n_tiles, int& tm, int& tn) {
  const int band = t / (kHeight * n_tiles);
  const int local = t - band * kHeight * n_tiles;
  const int h = min(kHeight, m_tiles - band * kHeight);  // rows in this (possibly last) band
  tn = local / h;
  tm = band * kHeight + local % h;
}

}  // namespace fp8q
