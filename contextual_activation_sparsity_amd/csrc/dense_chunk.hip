// Dense FFN over a chunk of up to 16 tokens on matrix cores: the Sirius verification
// pass ("SIRIUS: Contexual Sparisty with Correction for Efficient LLMs", Approach: the
// full model re-runs a chunk of sparse-generated tokens in parallel with the weights the
// sparse model shares).
//
// Stage 1 (gate and up): H[m, i] = act(x_m . Wg[i] + b_i) * (x_m . Wu[i]) for 16 neurons
// per workgroup. v_mfma_f32_16x16x32_bf16 takes the tokens as the M side and 16 neurons
// as the N side; a lane's 8-element K fragment of a weight row is 16 contiguous bytes,
// loaded straight from HBM. The four waves split K and combine through LDS. H is rounded
// to bf16 for stage 2.
// Stage 2 (down): Y = H Dt with Dt = W_down^T [f, d]. The K side (neurons) is the slow
// axis of Dt, so 32x64 tiles of Dt are loaded coalesced, staged in LDS and read back
// transposed into B fragments. K is split over S workgroups per 64-column tile; the last
// of the S to finish adds the partials in a fixed order.
// Both stages are bound by HBM (16 tokens = 16 flop per weight byte).

#include "device_common.h"
#include "kernels.h"
#include "sparse_ffn.h"

namespace sfn {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kPF1 = 8;  // K steps (of 32) in flight per wave in stage 1
constexpr int kPF2 = 8;  // K steps staged per batch in stage 2
constexpr int kColTile = 64;

__device__ __forceinline__ bf16x8_t as_frag(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ __launch_bounds__(256) void chunk_stage1_kernel(const char* __restrict__ wg, const char* __restrict__ wu,
                                                           const float* __restrict__ bias, const char* __restrict__ x,
                                                           int n, int d, int f, int act,
                                                           uint16_t* __restrict__ H) {
  __shared__ f32x4_t s_part[4][2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int col = lane & 15, q = lane >> 4;
  const int neuron = n0 + col;
  const bool nrow_ok = neuron < f;
  const bool tok_ok = col < n;  // A side: lane's token is col
  const int hs = (f + 7) & ~7;  // H row stride (elements)
  const size_t rb = (size_t)d * 2;
  const int nks = (d + 31) / 32;
  const int ks0 = (int)((long long)wave * nks / 4), ks1 = (int)((long long)(wave + 1) * nks / 4);
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  const char* wg_row = wg + (size_t)neuron * rb;
  const char* wu_row = wu + (size_t)neuron * rb;
  const char* x_row = x + (size_t)col * rb;
  for (int ks = ks0; ks < ks1; ks += kPF1) {
    uint4 fa[kPF1], fg[kPF1], fu[kPF1];
#pragma unroll
    for (int p = 0; p < kPF1; ++p) {
      const int k = (ks + p) * 32 + q * 8;
      const bool kok = (ks + p) < ks1 && k < d;
      fa[p] = (kok && tok_ok) ? ld16(x_row + (size_t)k * 2) : make_uint4(0, 0, 0, 0);
      fg[p] = (kok && nrow_ok) ? ldg16(wg_row + (size_t)k * 2) : make_uint4(0, 0, 0, 0);
      fu[p] = (kok && nrow_ok) ? ldg16(wu_row + (size_t)k * 2) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < kPF1; ++p) {
      accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(fa[p]), as_frag(fg[p]), accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(fa[p]), as_frag(fu[p]), accu, 0, 0, 0);
    }
  }
  s_part[wave][0][lane] = accg;
  s_part[wave][1][lane] = accu;
  __syncthreads();
  if (wave == 0) {
    f32x4_t g = s_part[0][0][lane], u = s_part[0][1][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      g += s_part[w][0][lane];
      u += s_part[w][1][lane];
    }
    // lane holds tokens 4q + i (rows of C) for neuron n0 + col (column of C)
    const float bv = (bias && nrow_ok) ? bias[neuron] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * q + i;
      if (m < n && nrow_ok) {
        const float gv = g[i] + bv;
        const float av = act == 0 ? silu_f(gv) : fmaxf(gv, 0.f);
        H[(size_t)m * hs + neuron] = (uint16_t)f32_to_bf16_rne(av * u[i]);
      } else if (m < n && neuron < hs) {
        H[(size_t)m * hs + neuron] = 0;  // row padding read by stage 2's last K step
      }
    }
  }
}

__global__ __launch_bounds__(256) void chunk_stage2_kernel(const uint16_t* __restrict__ H, const char* __restrict__ wd,
                                                           int n, int d, int f, int S,
                                                           float* __restrict__ part, uint32_t* __restrict__ arrive,
                                                           float* __restrict__ y) {
  __shared__ uint16_t s_dt[kPF2][32][kColTile + 8];
  __shared__ uint32_t s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntile = (d + kColTile - 1) / kColTile;
  const int ct = blockIdx.x % ntile, s = blockIdx.x / ntile;
  const int c0 = ct * kColTile;
  const int nks = (f + 31) / 32;
  const int ks0 = (int)((long long)s * nks / S), ks1 = (int)((long long)(s + 1) * nks / S);
  const size_t rb = (size_t)d * 2;
  // loader mapping: thread -> (row tid/8 of the 32-row step, 8 columns at (tid%8)*8)
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  const bool lcol_ok = c0 + lc < d;
  // fragment mapping
  const int col = lane & 15, q = lane >> 4;
  const bool tok_ok = col < n;
  const int hs = (f + 7) & ~7;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  uint4 stage[kPF2];
  auto load_batch = [&](int kb) {
#pragma unroll
    for (int p = 0; p < kPF2; ++p) {
      const int row = (kb + p) * 32 + lr;
      const bool ok = (kb + p) < ks1 && row < f && lcol_ok;
      stage[p] = ok ? ldg16(wd + (size_t)row * rb + (size_t)(c0 + lc) * 2) : make_uint4(0, 0, 0, 0);
    }
  };
  load_batch(ks0);
  for (int kb = ks0; kb < ks1; kb += kPF2) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kPF2; ++p) *reinterpret_cast<uint4*>(&s_dt[p][lr][lc]) = stage[p];
    __syncthreads();
    if (kb + kPF2 < ks1) load_batch(kb + kPF2);
#pragma unroll
    for (int p = 0; p < kPF2; ++p) {
      if (kb + p < ks1) {
        const int k = (kb + p) * 32 + q * 8;
        const uint4 a = (tok_ok && k < f) ? ld16(reinterpret_cast<const char*>(H + (size_t)col * hs + k))
                                          : make_uint4(0, 0, 0, 0);
        // B fragment: Dt[k + j][c0 + 16 wave + col], j < 8, from the staged tile
        uint32_t bw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = s_dt[p][q * 8 + 2 * j][16 * wave + col];
          const uint32_t hi = s_dt[p][q * 8 + 2 * j + 1][16 * wave + col];
          bw[j] = lo | (hi << 16);
        }
        const uint4 b = make_uint4(bw[0], bw[1], bw[2], bw[3]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(a), as_frag(b), acc, 0, 0, 0);
      }
    }
  }
  // C[4q + i][16 wave + col]: token 4q + i, column c0 + 16 wave + col
  const int ycol = c0 + 16 * wave + col;
  if (S == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * q + i;
      if (m < n && ycol < d) y[(size_t)m * d + ycol] = acc[i];
    }
    return;
  }
  // Partials cross workgroups (and XCDs, whose L2s are not coherent with each other):
  // they are written through to memory with relaxed device-scope stores and read back
  // the same way, and the arrival ticket is a relaxed device-scope atomic. Nothing here
  // needs a fence, which at device scope would write back the whole L2.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * q + i;
    if (m < n && ycol < d)
      __hip_atomic_store(&part[((size_t)s * n + m) * d + ycol], acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial is in memory
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&arrive[ct], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == (uint32_t)(S - 1)) ? 1u : 0u;
    if (s_last) __hip_atomic_store(&arrive[ct], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // old >= S means the counter was not zero at launch; no tile is then summed
  }
  __syncthreads();
  if (!s_last) return;
  // sum the S partials of this column tile in split order
  for (int e = tid; e < n * kColTile; e += 256) {
    const int m = e / kColTile, c = c0 + e % kColTile;
    if (c < d) {
      float tot = 0.f;
      for (int s2 = 0; s2 < S; ++s2)
        tot += __hip_atomic_load(&part[((size_t)s2 * n + m) * d + c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      y[(size_t)m * d + c] = tot;
    }
  }
}

int chunk_splits(int d, int f) {
  const int ntile = (d + kColTile - 1) / kColTile;
  int S = (512 + ntile - 1) / ntile;
  const int maxs = (f + 255) / 256;
  if (S > maxs) S = maxs;
  return S < 1 ? 1 : S;
}

}  // namespace

size_t chunk_workspace_bytes(int d, int f, int wdtype, int n) {
  if (wdtype != SFN_BF16) {
    // fp32 weights run through the decode kernel, 4 tokens at a time
    return decode_workspace_bytes(d, f, 4, n > 1 ? 4 : 1);
  }
  const int S = chunk_splits(d, f);
  size_t bytes = kWsHeader;
  bytes += (size_t)SFN_MAX_CHUNK * ((f + 7) & ~7) * sizeof(uint16_t);
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += (size_t)S * SFN_MAX_CHUNK * d * sizeof(float);
  (void)n;
  return bytes;
}

hipError_t launch_dense_chunk(const sfn_ffn& ffn, const void* x, int n, float* y, void* ws, hipStream_t stream) {
  if (ffn.wdtype != SFN_BF16) {
    // |act(g)| > 0 keeps every neuron that contributes, so this is the dense FFN.
    DecodeArgs a{};
    a.wg = static_cast<const char*>(ffn.w_gate);
    a.wu = static_cast<const char*>(ffn.w_up);
    a.wd = static_cast<const char*>(ffn.w_down_t);
    a.bias = ffn.b_gate;
    a.d = ffn.d;
    a.f = ffn.f;
    a.nch = ffn.d * 4 / 16;
    a.row_bytes = ffn.d * 4;
    a.act = ffn.act;
    a.G = decode_grid(ffn.f);
    decode_carve(a, ws, 4);
    for (int j0 = 0; j0 < n; j0 += SFN_MAX_BATCH) {
      const int nb = n - j0 < SFN_MAX_BATCH ? n - j0 : SFN_MAX_BATCH;
      a.x = static_cast<const char*>(x) + (size_t)j0 * a.row_bytes;
      a.y = y + (size_t)j0 * ffn.d;
      a.nb = nb;
      a.n_red = decode_reducers(a.G, nb, ffn.d);
      hipError_t e = launch_decode(a, SFN_F32, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int ntile = (ffn.d + kColTile - 1) / kColTile;
  const int S = chunk_splits(ffn.d, ffn.f);
  if (ntile > kMaxColTiles) return hipErrorInvalidValue;
  char* p = static_cast<char*>(ws);
  uint32_t* arrive = reinterpret_cast<uint32_t*>(p + kWsChunkCounters);
  size_t off = kWsHeader;
  uint16_t* H = reinterpret_cast<uint16_t*>(p + off);
  off += (size_t)SFN_MAX_CHUNK * ((ffn.f + 7) & ~7) * sizeof(uint16_t);
  off = (off + 255) & ~(size_t)255;
  float* part = reinterpret_cast<float*>(p + off);
  hipLaunchKernelGGL(chunk_stage1_kernel, dim3((ffn.f + 15) / 16), dim3(256), 0, stream,
                     static_cast<const char*>(ffn.w_gate), static_cast<const char*>(ffn.w_up), ffn.b_gate,
                     static_cast<const char*>(x), n, ffn.d, ffn.f, ffn.act, H);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_stage2_kernel, dim3(ntile * S), dim3(256), 0, stream, H,
                     static_cast<const char*>(ffn.w_down_t), n, ffn.d, ffn.f, S, part, arrive, y);
  return hipGetLastError();
}

}  // namespace sfn
