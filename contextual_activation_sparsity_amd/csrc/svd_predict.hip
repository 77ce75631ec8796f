// SVD sparsity predictor ("SVD Contextual Sparsity Predictors for Fast LLM Inference",
// abstract and Figures 1-3): z = Q x (Q = V_r^T, [r, d] bf16), p = L z + b
// (L = U_r diag(sigma_r), [f, r] bf16), candidates {i : p_i > tau_i}.
//
// Two launches. The first computes z with two rows of Q per workgroup (256 threads per
// row, 16 bytes each per pass) and clears the scan state of the second. The second
// streams L in tiles of 64 rows, compares with tau and writes the candidate list in
// ascending order: each tile publishes its candidate count in a 64-bit word (a status in
// the high half), then sums the counts of all lower tiles to find where its candidates
// go. Tile = workgroup index: workgroups are dispatched in index order, so every tile
// waited on has already started. Relaxed device-scope atomics suffice: no cache
// writeback or invalidation (a release or acquire at device scope would flush the whole
// L2).

#include "device_common.h"
#include "kernels.h"
#include "sparse_ffn.h"

namespace sfn {

namespace {

constexpr int kRowsPerTile = 64;

// 64-bit tile word: status in the high half (0 not yet published, 1 count published).
__device__ __forceinline__ unsigned long long pack(uint32_t status, uint32_t v) {
  return ((unsigned long long)status << 32) | v;
}

__global__ __launch_bounds__(512) void svd_z_kernel(const char* __restrict__ q, const char* __restrict__ x, int d,
                                                    int r, float* __restrict__ z,
                                                    unsigned long long* flags, int ntiles) {
  __shared__ float part[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = tid >> 8, t = tid & 255;  // row of the pair, thread within the row
  const int row = blockIdx.x * 2 + half;
  // scan state of the candidate pass
  const int gtid = blockIdx.x * blockDim.x + tid;
  for (int i = gtid; i < ntiles; i += gridDim.x * blockDim.x) flags[i] = 0ull;
  const int nch = d / 8;
  const size_t rb = (size_t)d * 2;
  float acc = 0.f;
  if (row < r) {
    constexpr int U = 4;  // chunks in flight per thread
    for (int c0 = t; c0 < nch; c0 += 256 * U) {
      uint4 w[U], xv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 256 * u;
        const bool ok = c < nch;
        w[u] = ok ? ldg16(q + (size_t)row * rb + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
        xv[u] = ok ? ld16(x + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc = Chunk<WT_BF16>::dot(w[u], xv[u], acc);
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (t == 0 && row < r) z[row] = part[4 * half] + part[4 * half + 1] + part[4 * half + 2] + part[4 * half + 3];
}

// 512 threads, kRowsPerTile rows of L per tile; each row (r bf16 = r/8 chunks of 16
// bytes) is handled by TPR <= 64 lanes of one wave, CH chunks each (TPR CH >= r/8, so
// r <= 1024), 512 / TPR rows side by side. One wave per 64 rows then compares and
// compacts.
template <int TPR, int CH>
__global__ __launch_bounds__(512) void svd_p_kernel(const char* __restrict__ l, const float* __restrict__ z,
                                                    const float* __restrict__ bias, const float* __restrict__ tau,
                                                    int f, int r, int32_t* __restrict__ cand, int32_t* n_cand,
                                                    float* __restrict__ p_out,
                                                    unsigned long long* flags, int ntiles, uint32_t* status) {
  constexpr int RPI = 512 / TPR;  // rows side by side
  constexpr int NIT = kRowsPerTile / RPI;
  constexpr int NCW = kRowsPerTile / 64;  // comparing waves
  static_assert(kRowsPerTile % 64 == 0 && NCW <= 512 / 64, "whole waves compare the tile's rows");
  __shared__ float s_p[kRowsPerTile];
  __shared__ uint32_t s_cnt[NCW];
  __shared__ uint32_t s_excl;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x;
  const int row0 = tile * kRowsPerTile;
  const int rl = tid / TPR, cl = tid % TPR;
  // waves 0-3: bias and threshold of row (row0 + tid), read now so the compare need not wait
  float pb = 0.f, pt = 0.f;
  if (tid < kRowsPerTile && row0 + tid < f) {
    pb = bias ? bias[row0 + tid] : 0.f;
    pt = tau[row0 + tid];
  }
  const int nch = r / 8;
  const size_t rb = (size_t)r * 2;
  uint4 wv[NIT][CH];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int row = row0 + rl + RPI * it;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = cl + TPR * c;
      wv[it][c] = (ch < nch && row < f) ? ldg16(l + (size_t)row * rb + (size_t)ch * 16) : make_uint4(0, 0, 0, 0);
    }
  }
  // z chunks of this lane, widened to fp32
  float zc[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) zc[c][j] = cl + TPR * c < nch ? z[(cl + TPR * c) * 8 + j] : 0.f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t p4[4] = {wv[it][c].x, wv[it][c].y, wv[it][c].z, wv[it][c].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(__uint_as_float(p4[j] << 16), zc[c][2 * j], acc);
        acc = fmaf(__uint_as_float(p4[j] & 0xffff0000u), zc[c][2 * j + 1], acc);
      }
    }
    // reduce over the TPR lanes of the row (TPR divides 64, lanes contiguous)
    acc = group_sum<TPR>(acc);
    if (cl == 0) s_p[rl + RPI * it] = acc;
  }
  __syncthreads();
  // waves 0 .. NCW-1: compare and ballot-compact 64 rows each
  const int row = row0 + tid;
  bool on = false;
  unsigned long long bal = 0ull;
  if (wave < NCW) {
    if (row < f) {
      const float p = s_p[tid] + pb;
      if (p_out) p_out[row] = p;
      on = p > pt;
    }
    bal = __ballot(on);
    if (lane == 0) s_cnt[wave] = (uint32_t)__popcll(bal);
  }
  __syncthreads();
  uint32_t cnt = 0;
#pragma unroll
  for (int w2 = 0; w2 < NCW; ++w2) cnt += s_cnt[w2];
  // Prefix over tiles: every tile publishes its count as soon as it has it; wave 0 then
  // reads the counts of all lower tiles (four per lane in flight, waiting for any not yet
  // published: lower tiles have lower workgroup indices, so they are running) and sums
  // them. No tile waits on another tile's prefix, so there is no chain of round trips.
  // The wait is bounded (2^20 round trips, about a second; never expected, since lower
  // tiles always publish). A tile that gives up sets the workspace status word; the last
  // tile waits on every other one, so it gives up too and reports n_cand = -1 instead of
  // a count built from missing words.
  if (wave == 0) {
    if (lane == 0) __hip_atomic_store(&flags[tile], pack(1u, cnt), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t excl = 0;
    bool late = false;
    for (int b0 = 0; b0 < tile; b0 += 256) {
      uint32_t v = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = b0 + 64 * u + lane;
        if (j < tile) {
          unsigned long long fl;
          uint32_t spins = 0;
          while (((fl = __hip_atomic_load(&flags[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) >> 32) == 0ull) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > (1u << 20)) {
              late = true;
              break;
            }
          }
          v += (uint32_t)fl;
        }
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
      excl += v;
    }
    const bool gave_up = __ballot(late) != 0ull;
    if (lane == 0) {
      s_excl = excl;
      if (gave_up) __hip_atomic_store(status, kStatusPredictor, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tile == ntiles - 1) *n_cand = gave_up ? -1 : (int32_t)(excl + cnt);
    }
  }
  __syncthreads();
  if (on) {
    uint32_t base = s_excl;
    for (int w2 = 0; w2 < wave; ++w2) base += s_cnt[w2];
    const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    cand[base + pos] = row;
  }
}

}  // namespace

size_t svd_workspace_bytes(int d, int f, int r) {
  (void)d;
  const int ntiles = (f + kRowsPerTile - 1) / kRowsPerTile;
  size_t bytes = kWsHeader;
  bytes += (size_t)ntiles * sizeof(unsigned long long);
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += (size_t)r * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_svd_z(const sfn_svd& s, const void* x, float* z, hipStream_t stream) {
  hipLaunchKernelGGL(svd_z_kernel, dim3((s.r + 1) / 2), dim3(512), 0, stream, static_cast<const char*>(s.q),
                     static_cast<const char*>(x), s.d, s.r, z, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_svd_predict(const sfn_svd& s, const void* x, int32_t* cand, int32_t* n_cand, float* p_out,
                              void* ws, hipStream_t stream) {
  const int ntiles = (s.f + kRowsPerTile - 1) / kRowsPerTile;
  char* p = static_cast<char*>(ws) + kWsHeader;
  unsigned long long* flags = reinterpret_cast<unsigned long long*>(p);
  size_t off = (size_t)ntiles * sizeof(unsigned long long);
  off = (off + 255) & ~(size_t)255;
  float* z = reinterpret_cast<float*>(p + off);
  uint32_t* status = reinterpret_cast<uint32_t*>(ws) + kWsStatusWord;
  hipLaunchKernelGGL(svd_z_kernel, dim3((s.r + 1) / 2), dim3(512), 0, stream, static_cast<const char*>(s.q),
                     static_cast<const char*>(x), s.d, s.r, z, flags, ntiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nch = s.r / 8;
  const char* l = static_cast<const char*>(s.l);
#define SFN_P_LAUNCH(TPR, CH)                                                                                      \
  hipLaunchKernelGGL((svd_p_kernel<TPR, CH>), dim3(ntiles), dim3(512), 0, stream, l, z, s.b, s.tau, s.f, s.r, cand, \
                     n_cand, p_out, flags, ntiles, status)
  if (nch <= 8) {
    SFN_P_LAUNCH(8, 1);
  } else if (nch <= 16) {
    SFN_P_LAUNCH(16, 1);
  } else if (nch <= 32) {
    SFN_P_LAUNCH(32, 1);
  } else if (nch <= 64) {
    SFN_P_LAUNCH(64, 1);
  } else if (nch <= 128) {
    SFN_P_LAUNCH(64, 2);
  } else {
    return hipErrorInvalidValue;  // r > 1024
  }
#undef SFN_P_LAUNCH
  return hipGetLastError();
}

}  // namespace sfn
