// Device helpers shared by the sparse-FFN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfn {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Weight/token storage types. A "chunk" is 16 bytes of a row: 8 bf16 or 4 fp32 values.
enum { WT_F32 = 0, WT_BF16 = 1 };

template <int WT>
struct Chunk;

template <>
struct Chunk<WT_BF16> {
  static constexpr int kVals = 8;
  // sum_j w_j x_j over the 8 bf16 pairs, accumulated into acc (bf16 products are exact
  // in fp32; v_dot2_f32_bf16 adds each pair of products to the running fp32 sum)
  __device__ __forceinline__ static float dot(const uint4& w, const uint4& x, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x),
                                          __builtin_bit_cast(bf16x2_t, x.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y),
                                          __builtin_bit_cast(bf16x2_t, x.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z),
                                          __builtin_bit_cast(bf16x2_t, x.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w),
                                          __builtin_bit_cast(bf16x2_t, x.w), acc, false);
    return acc;
  }
  // acc[j] += h * w_j (bf16 widened exactly to fp32)
  __device__ __forceinline__ static void axpy(float h, const uint4& w, float* acc) {
    const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(h, __uint_as_float(p[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(h, __uint_as_float(p[i] & 0xffff0000u), acc[2 * i + 1]);
    }
  }
};

template <>
struct Chunk<WT_F32> {
  static constexpr int kVals = 4;
  __device__ __forceinline__ static float dot(const uint4& w, const uint4& x, float acc) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
    return acc;
  }
  __device__ __forceinline__ static void axpy(float h, const uint4& w, float* acc) {
    acc[0] = fmaf(h, __uint_as_float(w.x), acc[0]);
    acc[1] = fmaf(h, __uint_as_float(w.y), acc[1]);
    acc[2] = fmaf(h, __uint_as_float(w.z), acc[2]);
    acc[3] = fmaf(h, __uint_as_float(w.w), acc[3]);
  }
};

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// 16-byte streaming load (weights are read once per call: non-temporal hint).
__device__ __forceinline__ uint4 ldg16(const char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// ---- cross-lane moves (wave64) ------------------------------------------------------
// DPP controls: quad_perm [1,0,3,2] swaps lane pairs, [2,3,0,1] swaps pairs of pairs,
// row_half_mirror reverses each group of 8 lanes, row_mirror each row of 16.
#define SFN_DPP_XOR1 0xB1
#define SFN_DPP_XOR2 0x4E
#define SFN_DPP_HALF_MIRROR 0x141
#define SFN_DPP_ROW_MIRROR 0x140

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Sum over all 64 lanes; every lane receives the total. Fixed pairing order, so the
// result is the same on every run.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<SFN_DPP_XOR1>(v);
  v += dpp_mov<SFN_DPP_XOR2>(v);
  v += dpp_mov<SFN_DPP_HALF_MIRROR>(v);
  v += dpp_mov<SFN_DPP_ROW_MIRROR>(v);
  v += shfl_xor_f(v, 16);
  v += shfl_xor_f(v, 32);
  return v;
}

// Reduce V values per lane over the 64 lanes of a wave at once (V a power of two,
// V <= 64). On return lane l holds, in s[0], the wave total of value index
//   vidx(l) = sum over the top log2(V) lane bits, i.e. l >> (6 - log2 V),
// identical in all 64/V lanes that share those bits. Each halving step exchanges half
// of the remaining values with the partner lane across one lane bit, so the work is
// V - 1 + (6 - log2 V) exchanges instead of 6 V.
template <int V>
__device__ __forceinline__ void wave_transpose_sum(float* s) {
  const int lane = threadIdx.x & 63;
  int nv = V;
  int bit = 32;
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    if (nv > 1) {
      const bool upper = (lane & bit) != 0;
      const int half = nv >> 1;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (i < half) {
          const float keep = upper ? s[i + half] : s[i];
          const float send = upper ? s[i] : s[i + half];
          s[i] = keep + shfl_xor_f(send, bit);
        }
      }
      nv = half;
    } else {
      if (bit >= 16) {
        s[0] += shfl_xor_f(s[0], bit);
      } else if (bit == 8) {
        s[0] += dpp_mov<SFN_DPP_ROW_MIRROR>(s[0]);
      } else if (bit == 4) {
        s[0] += dpp_mov<SFN_DPP_HALF_MIRROR>(s[0]);
      } else if (bit == 2) {
        s[0] += dpp_mov<SFN_DPP_XOR2>(s[0]);
      } else {
        s[0] += dpp_mov<SFN_DPP_XOR1>(s[0]);
      }
    }
    bit >>= 1;
  }
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace sfn
