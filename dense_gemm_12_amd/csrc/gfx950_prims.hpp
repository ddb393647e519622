// gfx950 (CDNA4) device primitives used by the GEMM kernels: vector types,
// buffer-resource loads with out-of-range -> zero, MFMA wrappers, and the
// workgroup -> tile map.  gfx950 only; no portability layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- buffers --
// A raw buffer resource (stride 0): the byte offset is range-checked against
// num_records and an out-of-range load returns zero.  Lanes that must read
// zero are given kOOB as their offset.  The third dword is the CDNA data
// format word for raw 32-bit access.
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kRecords = 0x7fffffffu;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)kRecords,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ------------------------------------------------------------------- MFMA --
// One "chunk step": each lane contributes a 16-byte chunk of the A-side
// operand and of the B-side operand (the same k positions on both sides).
//   f16 / bf16: one v_mfma_f32_16x16x32 (8 k values per lane, 32 per step);
//   f32:        four v_mfma_f32_16x16x4_f32, one per float in the chunk
//               (k = 4*(lane/16) + s for sub-step s; the k assignment is a
//               permutation shared by both operands, so the sum is the same).
// Output layout (16x16 block): lane l holds rows 4*(l/16)+v, column l%16.
template <typename T> struct Mfma;

template <> struct Mfma<_Float16> {
  static constexpr int kInsts = 1;
  static __device__ __forceinline__ void step(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<__bf16> {
  static constexpr int kInsts = 1;
  static __device__ __forceinline__ void step(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int kInsts = 4;
  static __device__ __forceinline__ void step(f32x4 &acc, const u32x4 &a, const u32x4 &b) {
    const f32x4 fa = __builtin_bit_cast(f32x4, a), fb = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[s], fb[s], acc, 0, 0, 0);
  }
};

// ---------------------------------------------------------- tile schedule --
// Workgroups are dispatched round-robin over the 8 XCDs (WG b runs on XCD
// b % 8), and each XCD has its own L2.  remap_xcd turns the launch index into
// a "logical" index such that each XCD receives a contiguous range of
// logical tiles; grouped raster then walks group_m tile-rows at a time so
// tiles that share A rows / B columns run close together in time on the same
// L2.  Both maps are bijections on [0, tiles), so any dispatch order is
// still correct.  They compile for the host too, where a CPU test checks
// the bijections over many grid shapes.
__host__ __device__ __forceinline__ int remap_xcd(int b, int tiles) {
  const int q = tiles >> 3, r = tiles & 7;
  const int xcd = b & 7, idx = b >> 3;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__host__ __device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int group_m, int &tm,
                                                     int &tn) {
  const int per_group = group_m * tiles_n;
  const int g = b / per_group;
  const int first_m = g * group_m;
  const int gsz = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
  const int in_g = b - g * per_group;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

// Workgroup -> (tile row, tile column, K range).  The launch covers
// tiles * splits workgroups; the split index is the slow one, so each XCD's
// contiguous share of logical indices holds whole splits, whose workgroups
// read the same K range of A and B.
__host__ __device__ __forceinline__ void work_coords(int b, int tiles_m, int tiles_n, int group_m,
                                                     int splits, int K, int k_chunk, int &tm, int &tn,
                                                     int &k0, int &kl) {
  const int tiles = tiles_m * tiles_n;
  const int l = remap_xcd(b, tiles * splits);
  const int s = l / tiles;
  tile_coords(l - s * tiles, tiles_m, tiles_n, group_m, tm, tn);
  k0 = s * k_chunk;
  kl = splits > 1 ? (K - k0 < k_chunk ? K - k0 : k_chunk) : K;
}

// ------------------------------------------------------------ conversions --
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

}  // namespace mg
