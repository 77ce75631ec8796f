// CATS threshold calibration ("CATS: Contextually-Aware Thresholding for Sparsity in
// Large Language Models", abstract: one threshold per layer sets the activation
// sparsity). Offline: run once per layer, not on the decode path.
//
// 1. Scores S[m, i] = |act(x_m . Wg[i] + b_i)| for n calibration tokens, fp32, with an
//    LDS-tiled vector kernel (16 tokens x 64 neurons per workgroup).
// 2. The K-th smallest score by radix select: non-negative fp32 values order like their
//    bit patterns read as uint32, so four passes of 8-bit digit histograms (most
//    significant first) pin down the exact bit pattern. Each pass is a histogram kernel
//    (integer atomics, so counts do not depend on timing) and a one-workgroup pick
//    kernel that chooses the digit and clears the histogram for the next pass.

#include "device_common.h"
#include "kernels.h"
#include "sparse_ffn.h"

namespace sfn {

namespace {

struct SelState {
  uint32_t prefix;  // digits chosen so far
  uint32_t k_rem;   // 1-based rank inside the current prefix class
  uint32_t pad[62];
  uint32_t hist[256];
};

constexpr int kTokTile = 16, kNeurTile = 64, kKTile = 64;

template <int WT>
__global__ __launch_bounds__(256) void score_kernel(const char* __restrict__ wg, const float* __restrict__ bias,
                                                    const char* __restrict__ x, int n, int d, int f, int act,
                                                    float* __restrict__ S, SelState* st, uint32_t K) {
  __shared__ float s_w[kNeurTile][kKTile + 1];
  __shared__ float s_x[kTokTile][kKTile + 1];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    st->hist[tid] = 0u;
    if (tid == 0) {
      st->prefix = 0u;
      st->k_rem = K;
    }
  }
  const int i0 = blockIdx.x * kNeurTile, m0 = blockIdx.y * kTokTile;
  const int j = tid % kNeurTile, tg = tid / kNeurTile;  // neuron j, tokens tg*4 .. tg*4+3
  constexpr int wb = WT == WT_BF16 ? 2 : 4;
  const size_t rb = (size_t)d * wb;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < d; k0 += kKTile) {
    __syncthreads();
    for (int e = tid; e < kNeurTile * kKTile; e += 256) {
      const int r = e / kKTile, c = e % kKTile;
      float v = 0.f;
      if (i0 + r < f && k0 + c < d) {
        const char* p = wg + (size_t)(i0 + r) * rb + (size_t)(k0 + c) * wb;
        v = WT == WT_BF16 ? __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16)
                          : *reinterpret_cast<const float*>(p);
      }
      s_w[r][c] = v;
    }
    for (int e = tid; e < kTokTile * kKTile; e += 256) {
      const int r = e / kKTile, c = e % kKTile;
      float v = 0.f;
      if (m0 + r < n && k0 + c < d) {
        const char* p = x + (size_t)(m0 + r) * rb + (size_t)(k0 + c) * wb;
        v = WT == WT_BF16 ? __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16)
                          : *reinterpret_cast<const float*>(p);
      }
      s_x[r][c] = v;
    }
    __syncthreads();
    for (int c = 0; c < kKTile; ++c) {
      const float wv = s_w[j][c];
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = fmaf(wv, s_x[tg * 4 + t][c], acc[t]);
    }
  }
  const int i = i0 + j;
  if (i < f) {
    const float bv = bias ? bias[i] : 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = m0 + tg * 4 + t;
      if (m < n) {
        const float g = acc[t] + bv;
        const float a = act == 0 ? silu_f(g) : fmaxf(g, 0.f);
        S[(size_t)m * f + i] = fabsf(a);
      }
    }
  }
}

__global__ __launch_bounds__(256) void hist_kernel(const float* __restrict__ S, long long N, int pass,
                                                   SelState* st) {
  __shared__ uint32_t h[256];
  const int tid = threadIdx.x;
  h[tid] = 0u;
  __syncthreads();
  const int shift = 24 - 8 * pass;
  const uint32_t prefix = st->prefix;
  for (long long e = (long long)blockIdx.x * 256 + tid; e < N; e += (long long)gridDim.x * 256) {
    const uint32_t u = __float_as_uint(S[e]);
    const bool match = pass == 0 || (u >> (shift + 8)) == prefix;
    if (match) atomicAdd(&h[(u >> shift) & 0xFFu], 1u);
  }
  __syncthreads();
  if (h[tid]) atomicAdd(&st->hist[tid], h[tid]);
}

__global__ __launch_bounds__(256) void pick_kernel(int pass, SelState* st, float* t_out) {
  __shared__ uint32_t c[256];
  const int tid = threadIdx.x;
  c[tid] = st->hist[tid];
  __syncthreads();
  if (tid == 0) {
    uint32_t k = st->k_rem, run = 0;
    int digit = 255;
    for (int b = 0; b < 256; ++b) {
      if (run + c[b] >= k) {
        digit = b;
        break;
      }
      run += c[b];
    }
    st->k_rem = k - run;
    st->prefix = (st->prefix << 8) | (uint32_t)digit;
    if (pass == 3) *t_out = __uint_as_float(st->prefix);
  }
  st->hist[tid] = 0u;
}

__global__ void set_kernel(float* t_out, float v) { *t_out = v; }

}  // namespace

size_t calibrate_workspace_bytes(int d, int f, int wdtype, int n) {
  (void)d;
  (void)wdtype;
  return kWsHeader + sizeof(SelState) + (((size_t)n * f * sizeof(float) + 255) & ~(size_t)255);
}

hipError_t launch_calibrate(const sfn_ffn& ffn, const void* x_cal, int n, float k, float* t_out, float* scores_out,
                            void* ws, hipStream_t stream) {
  const long long N = (long long)n * ffn.f;
  const double kd = (double)k;
  long long K = (long long)floor(kd * (double)N + 0.5);
  if (K <= 0) {
    hipLaunchKernelGGL(set_kernel, dim3(1), dim3(1), 0, stream, t_out, -1.0f);
    return hipGetLastError();
  }
  if (K >= N) {
    hipLaunchKernelGGL(set_kernel, dim3(1), dim3(1), 0, stream, t_out, __builtin_huge_valf());
    return hipGetLastError();
  }
  SelState* st = reinterpret_cast<SelState*>(static_cast<char*>(ws) + kWsHeader);
  float* S = scores_out ? scores_out
                        : reinterpret_cast<float*>(static_cast<char*>(ws) + kWsHeader + sizeof(SelState));
  const dim3 sgrid((ffn.f + kNeurTile - 1) / kNeurTile, (n + kTokTile - 1) / kTokTile);
  if (ffn.wdtype == SFN_BF16) {
    hipLaunchKernelGGL(score_kernel<WT_BF16>, sgrid, dim3(256), 0, stream, static_cast<const char*>(ffn.w_gate),
                       ffn.b_gate, static_cast<const char*>(x_cal), n, ffn.d, ffn.f, ffn.act, S, st, (uint32_t)K);
  } else {
    hipLaunchKernelGGL(score_kernel<WT_F32>, sgrid, dim3(256), 0, stream, static_cast<const char*>(ffn.w_gate),
                       ffn.b_gate, static_cast<const char*>(x_cal), n, ffn.d, ffn.f, ffn.act, S, st, (uint32_t)K);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  long long blocks = (N + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  for (int pass = 0; pass < 4; ++pass) {
    hipLaunchKernelGGL(hist_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, S, N, pass, st);
    hipLaunchKernelGGL(pick_kernel, dim3(1), dim3(256), 0, stream, pass, st, t_out);
  }
  return hipGetLastError();
}

}  // namespace sfn
