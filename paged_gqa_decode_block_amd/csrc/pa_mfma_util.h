// pa_mfma_util.h -- gfx950 fragment helpers shared by the MFMA kernels that
// stream 16-token chunks of K and V through LDS (decode and prefill): operand
// types, the bf16 / f16 matrix-core instructions, chunk geometry per head_dim,
// raw buffer descriptors and quad reductions.
#pragma once
#include <type_traits>

#include "pa_kernels.h"

namespace pa {
namespace {

// Compile-time loop: f(integral_constant<int, I>) for I in [I0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;


template <typename T>
struct Mx;

template <>
struct Mx<__bf16> {
  typedef bf16x8 v8;
  typedef s16x4 v4;
  static __device__ __forceinline__ f32x4 mma32(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4 pack(bf16x4 x) { return __builtin_bit_cast(v4, x); }
  typedef bf16x4 e4;
};

template <>
struct Mx<_Float16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ f32x4 mma32(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(v4 a, v4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4 pack(f16x4 x) { return x; }
  typedef f16x4 e4;
};

template <int D>
struct Cfg {
  static constexpr int CPR = D / 8;         // 16-byte chunks per token row
  static constexpr int RPI = 64 / CPR;      // token rows per load instruction (8, 4, 2)
  static constexpr int LPC = 16 / RPI;      // load instructions per 16-token chunk (2, 4, 8)
  static constexpr int KS = D / 32;         // k-steps of the score MFMA
  static constexpr int MB = D / 16;         // 16-dim output tiles
};

// Raw buffer descriptor word 3 for plain 32-bit data on gfx950.
constexpr int kRsrcWord3 = 0x00020000;
// Raw buffer descriptor over [ptr, ptr + bytes); ptr and bytes are the same in
// every lane, which readfirstlane makes visible to the compiler (no waterfall).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const char* ptr, int bytes) {
  const uint64_t a = (uint64_t)ptr;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, kRsrcWord3);
}

// POL: cache policy bits of the K/V loads (0 = default, 2 = non-temporal).
template <int POL>
__device__ __forceinline__ uint4 buf_load(__amdgpu_buffer_rsrc_t r, int voff) {
  const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, POL);
  return make_uint4(t[0], t[1], t[2], t[3]);
}

// Max / sum over the four 16-lane quads (lanes i, i^16, i^32, i^48).
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (int)c[0]), __builtin_bit_cast(float, (int)c[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  return __builtin_bit_cast(float, (int)c[0]) + __builtin_bit_cast(float, (int)c[1]);
}

// Row offsets of the padded K and V tiles (16 rows of DW 16-bit elements).
// Each bank line of the tile (256 bytes: one row at DW = 128, two rows at
// DW = 64; one row at DW = 256) is followed by 32 bytes of pad. Measured with
// gfx950's bank-conflict counter (SQ_LDS_BANK_CONFLICT), this layout makes
// every LDS access of the decode's fold conflict-free: the score MFMA's
// A-fragment read (one 16-byte chunk from each of the 16 rows, 128-bit), the
// transposing 64-bit V^T read (32 contiguous bytes from each of 8 rows) and
// the 128-bit staging writes of whole rows. Unpadded 256-byte rows cost 4 (A
// fragments) and 2 (V^T) conflict cycles per instruction, rows padded by 16
// bytes still 4 for the A fragments. Every fragment address is then a per-lane
// base plus a constant.
template <int DW>
struct TileRows {
  static constexpr int RPL = DW >= 128 ? 1 : 256 / (2 * DW);  // rows per pad
  static constexpr int PAD = 16;                               // elements (32 bytes)
  static constexpr int SIZE = 16 * DW + (16 / RPL) * PAD;
  static __device__ __forceinline__ int row(int r) { return r * DW + (r / RPL) * PAD; }
};

}  // namespace
}  // namespace pa
