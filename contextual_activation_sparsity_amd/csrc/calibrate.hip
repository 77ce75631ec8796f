// CATS threshold calibration ("CATS: Contextually-Aware Thresholding for Sparsity in
// Large Language Models", abstract: one threshold per layer sets the activation
// sparsity). Offline: run once per layer, not on the decode path.
//
// 1. Scores S[m, i] = |act(x_m . Wg[i] + b_i)| for n calibration tokens, fp32. bf16
//    weights run on matrix cores (v_mfma_f32_16x16x32_bf16, 16 neurons per workgroup as
//    the N side, 256 tokens per pass as 16 blocks of M): Wg goes through LDS in 1 KB row
//    pieces, the token fragments come from L2, each wave owns 4 token blocks over the
//    whole K range (no cross-wave sums). fp32 weights use an LDS-tiled vector kernel
//    (16 tokens x 64 neurons per workgroup).
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
constexpr int kKT = 512;          // matrix-core scores: K elements per stage (1 KB of a bf16 row)
constexpr int kTokPass = 256;     // tokens per workgroup (16 blocks of 16)

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

__device__ __forceinline__ bf16x8_t as_frag(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ void init_select(SelState* st, uint32_t K) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    st->hist[tid] = 0u;
    if (tid == 0) {
      st->prefix = 0u;
      st->k_rem = K;
    }
  }
}

__global__ __launch_bounds__(256) void score_mfma_kernel(const char* __restrict__ wg, const float* __restrict__ bias,
                                                         const char* __restrict__ x, int n, int d, int f, int act,
                                                         float* __restrict__ S, SelState* st, uint32_t K) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[16][kKT + 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  init_select(st, K);
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * kTokPass;
  const int col = lane & 15, q = lane >> 4;
  const size_t rb = (size_t)d * 2;
  const int nst = (d + kKT - 1) / kKT;
  // this wave's token blocks: m0 + 16 (wave + 4 b) + col for b < 4
  const char* xrow[4];
  bool tok_ok[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int m = m0 + 16 * (wave + 4 * b) + col;
    tok_ok[b] = m < n;
    xrow[b] = x + (size_t)(tok_ok[b] ? m : 0) * rb;
  }
  // loader: round i (0..3) of wave v reads row 4 i + v, bytes [16 lane, +16) of the 1 KB piece
  uint4 wr[4];
  auto load = [&](int stg) {
    const int k = stg * kKT + lane * 8;
    const size_t koff = (size_t)(k < d ? k : 0) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = n0 + 4 * i + wave;
      const uint4 v = ldg16(wg + (size_t)(row < f ? row : 0) * rb + koff);
      wr[i] = (k < d && row < f) ? v : make_uint4(0, 0, 0, 0);
    }
  };
  f32x4_t acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int stg = 0; stg < nst; ++stg) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&s_w[4 * i + wave][lane * 8]) = wr[i];
    __syncthreads();
    if (stg + 1 < nst) load(stg + 1);
    for (int t = 0; t < kKT / 32; ++t) {
      const int kk = t * 32 + q * 8;
      const int kx = stg * kKT + kk;
      const uint4 bw = *reinterpret_cast<const uint4*>(&s_w[col][kk]);
      uint4 xa[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint4 v = ld16(xrow[b] + (size_t)(kx < d ? kx : 0) * 2);
        xa[b] = (tok_ok[b] && kx < d) ? v : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(xa[b]), as_frag(bw), acc[b], 0, 0, 0);
    }
  }
  // acc[b][i]: token m0 + 16 (wave + 4 b) + 4 q + i, neuron n0 + col
  const int i0 = n0 + col;
  if (i0 < f) {
    const float bv = bias ? bias[i0] : 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * (wave + 4 * b) + 4 * q + i;
        if (m < n) {
          const float g = acc[b][i] + bv;
          const float a = act == 0 ? silu_f(g) : fmaxf(g, 0.f);
          S[(size_t)m * f + i0] = fabsf(a);
        }
      }
  }
}

template <int WT>
__global__ __launch_bounds__(256) void score_kernel(const char* __restrict__ wg, const float* __restrict__ bias,
                                                    const char* __restrict__ x, int n, int d, int f, int act,
                                                    float* __restrict__ S, SelState* st, uint32_t K) {
  __shared__ float s_w[kNeurTile][kKTile + 1];
  __shared__ float s_x[kTokTile][kKTile + 1];
  const int tid = threadIdx.x;
  init_select(st, K);
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
  if (ffn.wdtype == SFN_BF16) {
    const dim3 mgrid((ffn.f + 15) / 16, (n + kTokPass - 1) / kTokPass);
    hipLaunchKernelGGL(score_mfma_kernel, mgrid, dim3(256), 0, stream, static_cast<const char*>(ffn.w_gate),
                       ffn.b_gate, static_cast<const char*>(x_cal), n, ffn.d, ffn.f, ffn.act, S, st, (uint32_t)K);
  } else {
    const dim3 sgrid((ffn.f + kNeurTile - 1) / kNeurTile, (n + kTokTile - 1) / kTokTile);
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
