// CATS threshold calibration ("CATS: Contextually-Aware Thresholding for Sparsity in
// Large Language Models", abstract: one threshold per layer sets the activation
// sparsity). Offline: run once per layer, not on the decode path.
//
// 1. Scores S[m, i] = |act(x_m . Wg[i] + b_i)| for n calibration tokens, fp32. bf16
//    weights run on matrix cores (v_mfma_f32_16x16x32_bf16, 64 neurons x 256 tokens per
//    workgroup, 64 x 64 per wave, weights and tokens staged in LDS). fp32 weights use an
//    LDS-tiled vector kernel (16 tokens x 64 neurons per workgroup).
// 2. The K-th smallest score by radix select: non-negative fp32 values order like their
//    bit patterns read as uint32, so four passes of 8-bit digit histograms (most
//    significant first) pin down the exact bit pattern. Each pass is one histogram
//    kernel (integer atomics, so counts do not depend on timing) with a histogram of its
//    own; every workgroup of pass p first derives the digits chosen by passes 0..p-1
//    from their histograms (a block-wide scan per pass), so no kernel sits between the
//    passes. A one-workgroup kernel derives the last digit and writes the threshold.

#include "device_common.h"
#include "kernels.h"
#include "sparse_ffn.h"

namespace sfn {

namespace {

struct SelState {
  uint32_t hist[4][256];  // digit counts of each pass
};

constexpr int kTokTile = 16, kNeurTile = 64, kKTile = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

__device__ __forceinline__ bf16x8_t as_frag(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Clears the histograms of the selection (first workgroup of the score kernel; the
// histogram passes run after it).
__device__ __forceinline__ void init_select(SelState* st) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < 4 * 256; i += blockDim.x) st->hist[i >> 8][i & 255] = 0u;
}

// Digits chosen by passes 0..npass-1 for rank K (1-based): in each pass the digit whose
// cumulative count first reaches the remaining rank; the rank then becomes the rank
// inside that digit's class. Called by all 256 threads of a workgroup; returns the
// prefix of chosen digits and the remaining rank to every thread.
__device__ void chosen_digits(const SelState* st, int npass, uint32_t K, uint32_t& prefix, uint32_t& k_rem) {
  __shared__ uint32_t s_wsum[4];
  __shared__ uint32_t s_pick[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t pre = 0u, k = K;
  for (int p = 0; p < npass; ++p) {
    const uint32_t c = st->hist[p][tid];
    uint32_t v = c;  // inclusive scan over the workgroup
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const uint32_t u = __shfl_up(v, m, 64);
      if (lane >= m) v += u;
    }
    if (lane == 63) s_wsum[wave] = v;
    __syncthreads();
    for (int w = 0; w < wave; ++w) v += s_wsum[w];
    const uint32_t excl = v - c;
    if (excl < k && k <= v) {  // exactly one digit: the counts sum to at least k
      s_pick[0] = (uint32_t)tid;
      s_pick[1] = k - excl;
    }
    __syncthreads();
    pre = (pre << 8) | s_pick[0];
    k = s_pick[1];
    __syncthreads();
  }
  prefix = pre;
  k_rem = k;
}

// Scores on matrix cores with two-level tiling: a workgroup owns 64 neurons and SM
// tokens (256, or 128 when 256-token tiles would leave compute units idle); each of its
// four waves owns SM / 4 tokens x 64 neurons (SM / 64 x 4 blocks of 16 x 16), so every B
// fragment serves SM / 64 MFMAs and every A fragment four. Per stage of 64 K elements
// the 64 weight rows and the SM token rows go through LDS (128-byte pieces, eight rows
// per wave instruction), the next stage's loads in flight meanwhile. Whole calibration
// per layer, 256 tokens: 115 us at d 4096, f 11008 with SM 128 (128 with 256-token
// tiles, 172 workgroups); 270 us at d 8192, f 28672 with SM 256 (343 with 128).
constexpr int kSN = 64;           // neurons per workgroup
constexpr int kSK = 64;           // K elements per stage
constexpr int kSLd = kSK + 8;     // padded LDS row (elements)

template <int SM>
__global__ __launch_bounds__(256) void score_tile_kernel(const char* __restrict__ wg, const float* __restrict__ bias,
                                                         const char* __restrict__ x, int n, int d, int f, int act,
                                                         float* __restrict__ S, SelState* st, uint32_t K) {
  __shared__ __attribute__((aligned(16))) uint16_t s_w[kSN][kSLd];
  __shared__ __attribute__((aligned(16))) uint16_t s_x[SM][kSLd];
  constexpr int MB = SM / 64;  // token blocks per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  (void)K;
  init_select(st);
  const int n0 = blockIdx.x * kSN, m0 = blockIdx.y * SM;
  const int col = lane & 15, q = lane >> 4;
  const size_t rb = (size_t)d * 2;
  const int nst = (d + kSK - 1) / kSK;
  // loader: thread t reads chunk t % 8 (16 bytes) of the 128-byte piece of rows t / 8 + 32 i
  const int lr = tid >> 3, lc = tid & 7;
  uint4 wr[2], xr[SM / 32];
  auto load = [&](int stg) {
    const int k = stg * kSK + lc * 8;
    const bool kok = k < d;
    const size_t koff = (size_t)(kok ? k : 0) * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = n0 + lr + 32 * i;
      const bool ok = kok && row < f;
      wr[i] = ok ? ldg16(wg + (size_t)row * rb + koff) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < SM / 32; ++i) {
      const int tok = m0 + lr + 32 * i;
      const bool ok = kok && tok < n;
      xr[i] = ok ? ld16(x + (size_t)tok * rb + koff) : make_uint4(0, 0, 0, 0);
    }
  };
  f32x4_t acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int stg = 0; stg < nst; ++stg) {
    __syncthreads();  // the previous stage's fragments have been read
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(&s_w[lr + 32 * i][lc * 8]) = wr[i];
#pragma unroll
    for (int i = 0; i < SM / 32; ++i) *reinterpret_cast<uint4*>(&s_x[lr + 32 * i][lc * 8]) = xr[i];
    __syncthreads();
    if (stg + 1 < nst) load(stg + 1);
#pragma unroll
    for (int t = 0; t < kSK / 32; ++t) {
      const int kk = 32 * t + 8 * q;
      uint4 bf[4], af[MB];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bf[nb] = *reinterpret_cast<const uint4*>(&s_w[16 * nb + col][kk]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const uint4*>(&s_x[16 * MB * wave + 16 * mb + col][kk]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(af[mb]), as_frag(bf[nb]), acc[mb][nb], 0, 0, 0);
    }
  }
  // acc[mb][nb][i]: token m0 + 16 MB wave + 16 mb + 4 q + i, neuron n0 + 16 nb + col
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int neuron = n0 + 16 * nb + col;
    if (neuron < f) {
      const float bv = bias ? bias[neuron] : 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 16 * MB * wave + 16 * mb + 4 * q + i;
          if (m < n) {
            const float g = acc[mb][nb][i] + bv;
            const float a = act == 0 ? silu_f(g) : fmaxf(g, 0.f);
            S[(size_t)m * f + neuron] = fabsf(a);
          }
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
  (void)K;
  init_select(st);
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

// One pass of the radix select: counts of the 8-bit digit at `shift` among the scores
// whose higher digits equal the prefix. Each wave counts into its own LDS histogram
// (calibration scores share few exponents, so one shared histogram would serialize on
// a handful of bins); each workgroup then adds its totals to the global histogram, one
// integer atomic per bin. Four float4 loads are in flight per thread.
constexpr int kHistBlocks = 256;

__global__ __launch_bounds__(256) void hist_kernel(const float* __restrict__ S, long long N, int pass,
                                                   SelState* st, uint32_t K) {
  __shared__ uint32_t h[4][256];
  const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
  for (int v = 0; v < 4; ++v) h[v][tid] = 0u;
  uint32_t prefix, k_rem;
  chosen_digits(st, pass, K, prefix, k_rem);
  (void)k_rem;
  __syncthreads();  // the cleared histograms (pass 0 derives no digit, so no barrier yet)
  const int shift = 24 - 8 * pass;
  uint32_t* hw = h[wave];
  auto count = [&](float x) {
    const uint32_t u = __float_as_uint(x);
    if (pass == 0 || (u >> (shift + 8)) == prefix) atomicAdd(&hw[(u >> shift) & 0xFFu], 1u);
  };
  const long long N4 = N / 4;
  const f32x4_t* S4 = reinterpret_cast<const f32x4_t*>(S);
  const long long stride = (long long)gridDim.x * 256;
  for (long long e0 = (long long)blockIdx.x * 256 + tid; e0 < N4; e0 += 4 * stride) {
    f32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long e = e0 + u * stride;
      v[u] = e < N4 ? S4[e] : f32x4_t{-1.f, -1.f, -1.f, -1.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (e0 + u * stride < N4) {
        count(v[u][0]);
        count(v[u][1]);
        count(v[u][2]);
        count(v[u][3]);
      }
  }
  // the N % 4 tail
  if (blockIdx.x == 0 && tid < (int)(N - 4 * N4)) count(S[4 * N4 + tid]);
  __syncthreads();
  const uint32_t tot = h[0][tid] + h[1][tid] + h[2][tid] + h[3][tid];
  if (tot) atomicAdd(&st->hist[pass][tid], tot);
}

// The threshold: the bit pattern of all four chosen digits.
__global__ __launch_bounds__(256) void pick_kernel(const SelState* st, uint32_t K, float* t_out) {
  uint32_t prefix, k_rem;
  chosen_digits(st, 4, K, prefix, k_rem);
  (void)k_rem;
  if (threadIdx.x == 0) *t_out = __uint_as_float(prefix);
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
    const int ntile = (ffn.f + kSN - 1) / kSN;
    if (ntile < 256) {
      const dim3 mgrid(ntile, (n + 127) / 128);
      hipLaunchKernelGGL(score_tile_kernel<128>, mgrid, dim3(256), 0, stream, static_cast<const char*>(ffn.w_gate),
                         ffn.b_gate, static_cast<const char*>(x_cal), n, ffn.d, ffn.f, ffn.act, S, st, (uint32_t)K);
    } else {
      const dim3 mgrid(ntile, (n + 255) / 256);
      hipLaunchKernelGGL(score_tile_kernel<256>, mgrid, dim3(256), 0, stream, static_cast<const char*>(ffn.w_gate),
                         ffn.b_gate, static_cast<const char*>(x_cal), n, ffn.d, ffn.f, ffn.act, S, st, (uint32_t)K);
    }
  } else {
    const dim3 sgrid((ffn.f + kNeurTile - 1) / kNeurTile, (n + kTokTile - 1) / kTokTile);
    hipLaunchKernelGGL(score_kernel<WT_F32>, sgrid, dim3(256), 0, stream, static_cast<const char*>(ffn.w_gate),
                       ffn.b_gate, static_cast<const char*>(x_cal), n, ffn.d, ffn.f, ffn.act, S, st, (uint32_t)K);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  long long blocks = (N / 4 + 255) / 256;
  if (blocks > kHistBlocks) blocks = kHistBlocks;
  if (blocks < 1) blocks = 1;
  for (int pass = 0; pass < 4; ++pass)
    hipLaunchKernelGGL(hist_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, S, N, pass, st, (uint32_t)K);
  hipLaunchKernelGGL(pick_kernel, dim3(1), dim3(256), 0, stream, st, (uint32_t)K, t_out);
  return hipGetLastError();
}

}  // namespace sfn
