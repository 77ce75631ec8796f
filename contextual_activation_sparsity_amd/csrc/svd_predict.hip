// SVD sparsity predictor ("SVD Contextual Sparsity Predictors for Fast LLM Inference",
// abstract and Figures 1-3): z = Q x (Q = V_r^T, [r, d] bf16), p = L z + b
// (L = U_r diag(sigma_r), [f, r] bf16), candidates {i : p_i > tau_i}.
//
// Two launches. The first computes z with one wave per row of Q and clears the scan
// state of the second. The second streams L in tiles of 64 rows, compares with tau and
// writes the candidate list in ascending order with a single-pass decoupled look-back
// scan over tile counts (tiles take dynamic tickets, so every predecessor a tile waits
// on has already started and never waits on a later tile).

#include "device_common.h"
#include "kernels.h"
#include "sparse_ffn.h"

namespace sfn {

namespace {

constexpr int kRowsPerTile = 64;

struct SvdWs {
  uint32_t ticket;
  uint32_t pad[63];
};

// 64-bit tile word: status in the high half (0 none, 1 tile count, 2 inclusive prefix).
__device__ __forceinline__ unsigned long long pack(uint32_t status, uint32_t v) {
  return ((unsigned long long)status << 32) | v;
}

__global__ __launch_bounds__(512) void svd_z_kernel(const char* __restrict__ q, const char* __restrict__ x, int d,
                                                    int r, float* __restrict__ z, SvdWs* st,
                                                    unsigned long long* flags, int ntiles) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 8 + (threadIdx.x >> 6);
  // scan state of the candidate pass
  const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = gtid; i < ntiles; i += gridDim.x * blockDim.x) flags[i] = 0ull;
  if (gtid == 0) st->ticket = 0u;
  if (row >= r) return;
  const int nch = d / 8;
  const size_t rb = (size_t)d * 2;
  float acc = 0.f;
  for (int c = lane; c < nch; c += 64) {
    const uint4 w = ldg16(q + (size_t)row * rb + (size_t)c * 16);
    const uint4 xv = ld16(x + (size_t)c * 16);
    acc = Chunk<WT_BF16>::dot(w, xv, acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) z[row] = acc;
}

// 256 threads; each row of L (r bf16 = r/8 chunks) is handled by TPR = r/8 threads (r <= 512
// -> TPR <= 64 lanes of one wave); rows side by side = 256 / TPR.
template <int TPR>
__global__ __launch_bounds__(256) void svd_p_kernel(const char* __restrict__ l, const float* __restrict__ z,
                                                    const float* __restrict__ bias, const float* __restrict__ tau,
                                                    int f, int r, int32_t* __restrict__ cand, int32_t* n_cand,
                                                    float* __restrict__ p_out, SvdWs* st,
                                                    unsigned long long* flags, int ntiles) {
  constexpr int RPI = 256 / TPR;  // rows side by side
  __shared__ uint32_t s_tile;
  __shared__ float s_p[kRowsPerTile];
  __shared__ uint32_t s_excl;
  const int tid = threadIdx.x;
  if (tid == 0) s_tile = __hip_atomic_fetch_add(&st->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int tile = (int)s_tile;
  const int row0 = tile * kRowsPerTile;
  const int rl = tid / TPR, cl = tid % TPR;
  const int nch = r / 8;
  // z chunk of this lane, widened to fp32
  float zc[8];
  const bool chunk_ok = cl < nch;
#pragma unroll
  for (int j = 0; j < 8; ++j) zc[j] = chunk_ok ? z[cl * 8 + j] : 0.f;
  const size_t rb = (size_t)r * 2;
  constexpr int NIT = kRowsPerTile / RPI;
  uint4 wv[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int row = row0 + rl + RPI * it;
    wv[it] = (chunk_ok && row < f) ? ldg16(l + (size_t)row * rb + (size_t)cl * 16) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const uint32_t p4[4] = {wv[it].x, wv[it].y, wv[it].z, wv[it].w};
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(__uint_as_float(p4[j] << 16), zc[2 * j], acc);
      acc = fmaf(__uint_as_float(p4[j] & 0xffff0000u), zc[2 * j + 1], acc);
    }
    // reduce over the TPR lanes of the row (TPR divides 64, lanes contiguous)
#pragma unroll
    for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (cl == 0) s_p[rl + RPI * it] = acc;
  }
  __syncthreads();
  // wave 0: compare, ballot-compact, look back
  if (tid < 64) {
    const int row = row0 + tid;
    bool on = false;
    if (row < f) {
      const float p = s_p[tid] + (bias ? bias[row] : 0.f);
      if (p_out) p_out[row] = p;
      on = p > tau[row];
    }
    const unsigned long long bal = __ballot(on);
    const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    const uint32_t cnt = (uint32_t)__popcll(bal);
    if (tid == 0) {
      uint32_t excl = 0;
      if (tile == 0) {
        __hip_atomic_store(&flags[0], pack(2u, cnt), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        __hip_atomic_store(&flags[tile], pack(1u, cnt), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        int j = tile - 1;
        while (j >= 0) {
          unsigned long long fl;
          uint32_t spins = 0;
          do {
            fl = __hip_atomic_load(&flags[j], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
            if ((fl >> 32) == 0ull) {
              __builtin_amdgcn_s_sleep(1);
              if (++spins > (1u << 24)) break;  // never expected: predecessors always finish
            }
          } while ((fl >> 32) == 0ull);
          excl += (uint32_t)fl;
          if ((fl >> 32) == 2ull || (fl >> 32) == 0ull) break;
          --j;
        }
        __hip_atomic_store(&flags[tile], pack(2u, excl + cnt), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
      s_excl = excl;
      if (tile == ntiles - 1) *n_cand = (int32_t)(excl + cnt);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const uint32_t base = s_excl;
    if (on) cand[base + pos] = row;
  }
}

}  // namespace

size_t svd_workspace_bytes(int d, int f, int r) {
  (void)d;
  const int ntiles = (f + kRowsPerTile - 1) / kRowsPerTile;
  size_t bytes = kWsHeader + sizeof(SvdWs);
  bytes += (size_t)ntiles * sizeof(unsigned long long);
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += (size_t)r * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_svd_predict(const sfn_svd& s, const void* x, int32_t* cand, int32_t* n_cand, float* p_out,
                              void* ws, hipStream_t stream) {
  const int ntiles = (s.f + kRowsPerTile - 1) / kRowsPerTile;
  char* p = static_cast<char*>(ws) + kWsHeader;
  SvdWs* st = reinterpret_cast<SvdWs*>(p);
  unsigned long long* flags = reinterpret_cast<unsigned long long*>(p + sizeof(SvdWs));
  size_t off = sizeof(SvdWs) + (size_t)ntiles * sizeof(unsigned long long);
  off = (off + 255) & ~(size_t)255;
  float* z = reinterpret_cast<float*>(p + off);
  hipLaunchKernelGGL(svd_z_kernel, dim3((s.r + 7) / 8), dim3(512), 0, stream, static_cast<const char*>(s.q),
                     static_cast<const char*>(x), s.d, s.r, z, st, flags, ntiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nch = s.r / 8;
  const char* l = static_cast<const char*>(s.l);
  if (nch <= 8) {
    hipLaunchKernelGGL((svd_p_kernel<8>), dim3(ntiles), dim3(256), 0, stream, l, z, s.b, s.tau, s.f, s.r, cand, n_cand, p_out, st, flags, ntiles);
  } else if (nch <= 16) {
    hipLaunchKernelGGL((svd_p_kernel<16>), dim3(ntiles), dim3(256), 0, stream, l, z, s.b, s.tau, s.f, s.r, cand, n_cand, p_out, st, flags, ntiles);
  } else if (nch <= 32) {
    hipLaunchKernelGGL((svd_p_kernel<32>), dim3(ntiles), dim3(256), 0, stream, l, z, s.b, s.tau, s.f, s.r, cand, n_cand, p_out, st, flags, ntiles);
  } else if (nch <= 64) {
    hipLaunchKernelGGL((svd_p_kernel<64>), dim3(ntiles), dim3(256), 0, stream, l, z, s.b, s.tau, s.f, s.r, cand, n_cand, p_out, st, flags, ntiles);
  } else {
    return hipErrorInvalidValue;  // r > 512 needs more than one wave per row
  }
  return hipGetLastError();
}

}  // namespace sfn
