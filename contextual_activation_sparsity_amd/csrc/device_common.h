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
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// Global-address-space pointers. Pointers that arrive inside a by-value argument struct
// are generic; accessing through them would emit flat instructions, which count against
// the LDS wait counter too and serialize LDS waits behind every weight load in flight.
#define SFN_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ SFN_GLOBAL T* gp(T* p) {
  return (SFN_GLOBAL T*)p;
}

// 16-byte streaming load (weights are read once per call: non-temporal hint).
__device__ __forceinline__ uint4 ldg16(const SFN_GLOBAL char* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const SFN_GLOBAL u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 ld16(const SFN_GLOBAL char* p) {
  const u32x4_t v = *reinterpret_cast<const SFN_GLOBAL u32x4_t*>(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 ldg16(const char* p) { return ldg16(gp(p)); }
__device__ __forceinline__ uint4 ld16(const char* p) { return ld16(gp(p)); }

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

// gfx950 lane swaps (v_permlane32_swap / v_permlane16_swap): VALU moves, with no trip
// through the LDS crossbar that a shuffle takes. BIT 32: the upper 32 lanes of a trade
// places with the lower 32 lanes of b. BIT 16: the odd rows of 16 lanes of a trade places
// with the even rows of b. Afterwards a lane without BIT holds in a and b what it and its
// partner lane (l | BIT) held in a; a lane with BIT holds what its partner (l & ~BIT) and
// it held in b. The whole wave must be active.
template <int BIT>
__device__ __forceinline__ void lane_swap(float& a, float& b) {
  static_assert(BIT == 32 || BIT == 16, "half-wave or row swaps");
  if constexpr (BIT == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

// v plus the v of lane l ^ BIT (BIT 16 or 32); the sum is the same in both lanes.
template <int BIT>
__device__ __forceinline__ float swap_pair_sum(float v) {
  float a = v, b = v;
  lane_swap<BIT>(a, b);
  return a + b;
}

// Sum over each aligned group of N consecutive lanes (N a power of two, at most 64);
// every lane of a group receives its total. Each step adds a partner lane that lies in
// the other half of the current group (a mirror or a swap; which lane of that half does
// not matter, since all of them hold the same partial sum by then). Fixed pairing order,
// so the result is the same on every run. The whole wave must be active.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power-of-two group of lanes");
  if constexpr (N >= 2) v += dpp_mov<SFN_DPP_XOR1>(v);
  if constexpr (N >= 4) v += dpp_mov<SFN_DPP_XOR2>(v);
  if constexpr (N >= 8) v += dpp_mov<SFN_DPP_HALF_MIRROR>(v);
  if constexpr (N >= 16) v += dpp_mov<SFN_DPP_ROW_MIRROR>(v);
  if constexpr (N >= 32) v = swap_pair_sum<16>(v);
  if constexpr (N >= 64) v = swap_pair_sum<32>(v);
  return v;
}

// Sum over all 64 lanes; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// Inclusive prefix sum over the 64 lanes of a wave: each row of 16 lanes scans itself
// with DPP right shifts by 1, 2, 4 and 8 (a lane with no source in its row adds 0), then
// row_bcast:15 adds the last lane of row 0 / row 2 to rows 1 / 3 and row_bcast:31 adds
// lane 31 (by then the total of rows 0 and 1) to rows 2 and 3. VALU moves only, no trip
// through the LDS crossbar. The whole wave must be active.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Lane select for the halving steps: hi in the lanes whose index has bit BIT set, lo in
// the others, for BIT in {32, 16, 8, 4}. A DPP identity move whose row mask (lane groups
// of 16) or bank mask (groups of 4 inside a row) enables only those lanes writes hi there
// and leaves lo elsewhere. (A ternary on array elements can turn into a dynamically
// indexed, scratch-backed array; DPP keeps it a register operation the compiler sees.)
template <int BIT>
__device__ __forceinline__ float sel_upper(float lo, float hi) {
  static_assert(BIT == 32 || BIT == 16 || BIT == 8 || BIT == 4, "row/bank granularity");
  constexpr int ROW = BIT == 32 ? 0xC : BIT == 16 ? 0xA : 0xF;
  constexpr int BANK = BIT == 8 ? 0xC : BIT == 4 ? 0xA : 0xF;
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(lo), __float_as_int(hi), 0xE4 /* identity */,
                                                    ROW, BANK, false));
}

// One halving step over lane bit BIT: values [0, H) stay, values [H, 2H) are exchanged,
// so that afterwards slot i holds value i (lanes without BIT) or i + H (lanes with it),
// summed with the partner lane l ^ BIT.
template <int BIT, int H>
__device__ __forceinline__ void halve_step(float* s) {
#pragma unroll
  for (int i = 0; i < H; ++i) {
    if constexpr (BIT >= 16) {
      // one swap puts both operands of each lane's sum in place
      float lo = s[i], hi = s[i + H];
      lane_swap<BIT>(lo, hi);
      s[i] = lo + hi;
    } else {
      const float lo = s[i], hi = s[i + H];
      const float keep = sel_upper<BIT>(lo, hi);
      const float send = sel_upper<BIT>(hi, lo);
      s[i] = keep + shfl_xor_f(send, BIT);
    }
  }
}

template <int BIT>
__device__ __forceinline__ float lane_pair_sum(float v) {
  if constexpr (BIT >= 16) return swap_pair_sum<BIT>(v);
  else if constexpr (BIT == 8) return v + dpp_mov<SFN_DPP_ROW_MIRROR>(v);
  else if constexpr (BIT == 4) return v + dpp_mov<SFN_DPP_HALF_MIRROR>(v);
  else if constexpr (BIT == 2) return v + dpp_mov<SFN_DPP_XOR2>(v);
  else return v + dpp_mov<SFN_DPP_XOR1>(v);
}

template <int NV, int BIT>
__device__ __forceinline__ void transpose_sum_rec(float* s) {
  if constexpr (BIT > 0) {
    if constexpr (NV > 1) {
      halve_step<BIT, NV / 2>(s);
      transpose_sum_rec<NV / 2, BIT / 2>(s);
    } else {
      s[0] = lane_pair_sum<BIT>(s[0]);
      transpose_sum_rec<1, BIT / 2>(s);
    }
  }
}

// Reduce V values per lane over the 64 lanes of a wave at once (V a power of two,
// V <= 16). On return lane l holds, in s[0], the wave total of value index
// l >> (6 - log2 V) (the top log2 V lane bits), identical in the 64/V lanes that share
// those bits. Each halving step exchanges half of the remaining values with the partner
// lane across one lane bit, so the work is V - 1 + (6 - log2 V) exchanges instead of 6 V.
// Larger sets are reduced as independent blocks of 16.
template <int V>
__device__ __forceinline__ void wave_transpose_sum(float* s) {
  static_assert(V <= 16, "reduce larger sets in blocks of 16");
  transpose_sum_rec<V, 32>(s);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

}  // namespace sfn
