// Dense FFN over a chunk of 2 to 16 tokens on matrix cores: the Sirius verification
// pass ("SIRIUS: Contexual Sparisty with Correction for Efficient LLMs", Approach: the
// full model re-runs a chunk of sparse-generated tokens in parallel with the weights the
// sparse model shares).
//
// Stage 1 (gate and up): H[m, i] = act(x_m . Wg[i] + b_i) * (x_m . Wu[i]) for 16 neurons
// per workgroup. v_mfma_f32_16x16x32_bf16 takes the tokens as the M side and 16 neurons
// as the N side. A fragment of a weight row is 16 contiguous bytes, but one wave-wide
// load of fragments would touch 16 rows at 64 bytes each, which HBM serves far below its
// streaming rate; so the weights go through LDS: each stage loads 512-element (1 KB)
// pieces of the 32 rows (Wg and Wu), one row per wave instruction, while the matrix
// cores work on the previous stage. The four waves split each stage's K range and
// combine through LDS at the end. H is rounded to bf16 for stage 2.
// Layers with f > 16384 take a wide variant of stage 1 (chunk_stage1_wide_kernel below).
// Stage 2 (down): Y = H Dt with Dt = W_down^T [f, d]. K (neurons) is the slow axis of
// Dt: a workgroup owns 256 output columns and a range of K, loads 32 x 256 tiles (two
// rows of 512 bytes per wave instruction), stages them in LDS and reads B fragments back
// transposed. K is split over S workgroups per column tile; a third launch adds the S
// partials in split order (deterministic), every output element in parallel.
// Both stages are bound by HBM (16 tokens = 16 flop per weight byte).

#include "device_common.h"
#include "kernels.h"
#include "sparse_ffn.h"

namespace sfn {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kKT = 512;           // stage 1: K elements per stage (1 KB of a bf16 row)
constexpr int kLdsRow1 = kKT + 8;  // padded LDS row (elements)
constexpr int kKTW = 256;              // wide stage 1: K elements per stage (512 bytes of a bf16 row)
constexpr int kLdsRowW = kKTW + 8;     // its padded LDS row (elements)
constexpr int kRowsW = 32;             // its rows per workgroup at most (two 16-neuron MFMA tiles)
constexpr int kGW = 1024;              // its workgroups (four per compute unit, all resident)
constexpr int kCT = 256;           // stage 2: output columns per workgroup
constexpr int kLdsRow2 = kCT + 8;
constexpr int kPB = 2;             // stage 2: K steps (of 32 rows) staged per batch

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
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2][16][kLdsRow1];
  __shared__ f32x4_t s_part[4][2][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int col = lane & 15, q = lane >> 4;
  const bool tok_ok = col < n;  // A side: lane's token is col
  const int hs = (f + 7) & ~7;  // H row stride (elements)
  const size_t rb = (size_t)d * 2;
  const int nst = (d + kKT - 1) / kKT;
  // loader: round i (0..7) of wave v reads row slot 4 i + v (matrix slot / 16, row slot % 16),
  // bytes [16 lane, 16 lane + 16) of the stage's 1 KB piece
  uint4 wr[8], xr[4], xc[4];
  auto load = [&](int st) {
    const int k = st * kKT + lane * 8;
    const bool kok = k < d;
    const size_t koff = (size_t)(kok ? k : 0) * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = 4 * i + wave;
      const int row = n0 + (slot & 15);
      const bool ok = kok && row < f;
      const char* base = (slot < 16 ? wg : wu) + (size_t)(row < f ? row : 0) * rb;
      const uint4 v = ldg16(base + koff);
      wr[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
    // A fragments of this wave's quarter: token col, K = st kKT + 128 wave + 32 t + 8 q
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kx = st * kKT + 128 * wave + 32 * t + 8 * q;
      const bool ok = tok_ok && kx < d;
      const uint4 v = ld16(x + (size_t)(tok_ok ? col : 0) * rb + (size_t)(kx < d ? kx : 0) * 2);
      xr[t] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  };
  f32x4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int st = 0; st < nst; ++st) {
    __syncthreads();  // the previous stage's fragments have been read
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = 4 * i + wave;
      *reinterpret_cast<uint4*>(&s_w[slot >> 4][slot & 15][lane * 8]) = wr[i];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) xc[t] = xr[t];
    __syncthreads();
    if (st + 1 < nst) load(st + 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kk = 128 * wave + 32 * t + 8 * q;
      const uint4 bg = *reinterpret_cast<const uint4*>(&s_w[0][col][kk]);
      const uint4 bu = *reinterpret_cast<const uint4*>(&s_w[1][col][kk]);
      accg = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(xc[t]), as_frag(bg), accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(xc[t]), as_frag(bu), accu, 0, 0, 0);
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
    const int neuron = n0 + col;
    const bool nrow_ok = neuron < f;
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

// Stage 1 for layers with more than 1024 16-neuron tiles (f > 16384): up to 32 neurons per
// workgroup (two 16-neuron tiles), at most 1024 workgroups, so that all of them are
// resident from the start (four per compute unit fit in LDS). The kernel above would run
// f / 16 workgroups in rounds of three per compute unit: 1792 at the Llama-3-70B shape,
// whose last round leaves two thirds of the chip idle. Each stage loads 256-element
// (512-byte) pieces of the workgroup's rows of Wg and Wu, two rows per wave instruction;
// otherwise it works as the kernel above. Llama-3-70B shape, 16 tokens, graph replay:
// 233.6 against 258.9 us per layer (6.03 against 5.44 TB/s). At d 4096 (f 11008 and
// 14336, where the kernel above runs in one round or nearly) it was slower, 76.0 against
// 68.6 and 83.7 against 80.7 us, so those shapes keep the kernel above.
__global__ __launch_bounds__(256) void chunk_stage1_wide_kernel(const char* __restrict__ wg, const char* __restrict__ wu,
                                                           const float* __restrict__ bias, const char* __restrict__ x,
                                                           int n, int d, int f, int act,
                                                           uint16_t* __restrict__ H) {
  // the wave sums at the end reuse this buffer
  __shared__ __attribute__((aligned(16))) uint16_t s_w[2][kRowsW][kLdsRowW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G1 = gridDim.x;
  const int r0 = (int)((uint32_t)blockIdx.x * (uint32_t)f / (uint32_t)G1);
  const int nr = (int)((uint32_t)(blockIdx.x + 1) * (uint32_t)f / (uint32_t)G1) - r0;  // <= kRowsW
  const int col = lane & 15, q = lane >> 4;
  const bool tok_ok = col < n;  // A side: lane's token is col
  const int hs = (f + 7) & ~7;  // H row stride (elements)
  const size_t rb = (size_t)d * 2;
  const int nst = (d + kKTW - 1) / kKTW;
  // loader: round i (0..7) of wave v reads row slot 8 i + 2 v + (lane / 32) of the 64 (the
  // workgroup's rows of Wg, then of Wu), bytes [16 (lane % 32), +16) of the stage's
  // 512-byte piece: two rows per wave instruction
  uint4 wr[8], xr[2], xc[2];
  auto load = [&](int st) {
    const int k = st * kKTW + (lane & 31) * 8;
    const bool kok = k < d;
    const size_t koff = (size_t)(kok ? k : 0) * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = 8 * i + 2 * wave + (lane >> 5);
      const int rr = slot & (kRowsW - 1);
      const bool ok = kok && rr < nr;
      const char* base = (slot < kRowsW ? wg : wu) + (size_t)(r0 + (rr < nr ? rr : 0)) * rb;
      const uint4 v = ldg16(base + koff);
      wr[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
    // A fragments of this wave's quarter: token col, K = st kKTW + 64 wave + 32 t + 8 q
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kx = st * kKTW + 64 * wave + 32 * t + 8 * q;
      const bool ok = tok_ok && kx < d;
      const uint4 v = ld16(x + (size_t)(tok_ok ? col : 0) * rb + (size_t)(kx < d ? kx : 0) * 2);
      xr[t] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  };
  f32x4_t acc[2][2];  // [Wg / Wu][neurons 0-15 / 16-31]
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[m][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int st = 0; st < nst; ++st) {
    __syncthreads();  // the previous stage's fragments have been read
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slot = 8 * i + 2 * wave + (lane >> 5);
      *reinterpret_cast<uint4*>(&s_w[slot / kRowsW][slot & (kRowsW - 1)][(lane & 31) * 8]) = wr[i];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) xc[t] = xr[t];
    __syncthreads();
    if (st + 1 < nst) load(st + 1);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kk = 64 * wave + 32 * t + 8 * q;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 bg = *reinterpret_cast<const uint4*>(&s_w[0][16 * h + col][kk]);
        const uint4 bu = *reinterpret_cast<const uint4*>(&s_w[1][16 * h + col][kk]);
        acc[0][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(xc[t]), as_frag(bg), acc[0][h], 0, 0, 0);
        acc[1][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(xc[t]), as_frag(bu), acc[1][h], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // every wave is done with s_w
  f32x4_t* s_part = reinterpret_cast<f32x4_t*>(&s_w[0][0][0]);  // [wave][Wg / Wu][half][lane]
  static_assert(4 * 2 * 2 * 64 * sizeof(f32x4_t) <= sizeof(s_w), "wave sums fit the stage buffer");
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int h = 0; h < 2; ++h) s_part[((wave * 2 + m) * 2 + h) * 64 + lane] = acc[m][h];
  __syncthreads();
  if (wave < 2) {
    // wave h: lane holds tokens 4q + i (rows of C) for neuron r0 + 16 h + col (column of C)
    const int h = wave;
    f32x4_t g = s_part[((0 * 2 + 0) * 2 + h) * 64 + lane], u = s_part[((0 * 2 + 1) * 2 + h) * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      g += s_part[((w * 2 + 0) * 2 + h) * 64 + lane];
      u += s_part[((w * 2 + 1) * 2 + h) * 64 + lane];
    }
    const int local = 16 * h + col;
    const int neuron = r0 + local;
    const bool nrow_ok = local < nr;
    const float bv = (bias && nrow_ok) ? bias[neuron] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * q + i;
      if (m < n && nrow_ok) {
        const float gv = g[i] + bv;
        const float av = act == 0 ? silu_f(gv) : fmaxf(gv, 0.f);
        H[(size_t)m * hs + neuron] = (uint16_t)f32_to_bf16_rne(av * u[i]);
      }
    }
  } else if (wave == 2 && blockIdx.x == gridDim.x - 1) {
    // row padding [f, hs) that stage 2's last K step reads
    const int np = hs - f;
    for (int e = lane; e < np * n; e += 64) H[(size_t)(e / np) * hs + f + e % np] = 0;
  }
}

__global__ __launch_bounds__(256) void chunk_stage2_kernel(const uint16_t* __restrict__ H, const char* __restrict__ wd,
                                                           int n, int d, int f, int S,
                                                           float* __restrict__ part, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t s_dt[kPB][32][kLdsRow2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ntile = (d + kCT - 1) / kCT;
  const int ct = blockIdx.x % ntile, s = blockIdx.x / ntile;
  const int c0 = ct * kCT;
  const int nks = (f + 31) / 32;
  const int ks0 = (int)((long long)s * nks / S), ks1 = (int)((long long)(s + 1) * nks / S);
  const size_t rb = (size_t)d * 2;
  // loader: K step p, round i (0..3): wave v reads rows 8 i + 2 v + (lane >> 5), bytes
  // [16 (lane & 31), +16) of the 512-byte column range
  const int lrow = 2 * wave + (lane >> 5), lch = (lane & 31) * 8;
  const bool lcol_ok = c0 + lch < d;
  const size_t lcoff = (size_t)(lcol_ok ? c0 + lch : 0) * 2;
  // fragment mapping
  const int col = lane & 15, q = lane >> 4;
  const bool tok_ok = col < n;
  const int hs = (f + 7) & ~7;
  f32x4_t acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 stage[kPB][4];
  auto load_batch = [&](int kb) {
#pragma unroll
    for (int p = 0; p < kPB; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (kb + p) * 32 + 8 * i + lrow;
        const bool ok = (kb + p) < ks1 && row < f && lcol_ok;
        const uint4 v = ldg16(wd + (size_t)(row < f ? row : 0) * rb + lcoff);
        stage[p][i] = ok ? v : make_uint4(0, 0, 0, 0);
      }
  };
  load_batch(ks0);
  for (int kb = ks0; kb < ks1; kb += kPB) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kPB; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&s_dt[p][8 * i + lrow][lch]) = stage[p][i];
    __syncthreads();
    if (kb + kPB < ks1) load_batch(kb + kPB);
#pragma unroll
    for (int p = 0; p < kPB; ++p) {
      if (kb + p < ks1) {
        const int k = (kb + p) * 32 + q * 8;
        const uint4 a = (tok_ok && k < f) ? ld16(reinterpret_cast<const char*>(H + (size_t)col * hs + k))
                                          : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // B fragment: Dt[k + j][c0 + 64 wave + 16 b + col], j < 8, from the staged tile
          const int cc = 64 * wave + 16 * b + col;
          uint32_t bw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = s_dt[p][q * 8 + 2 * j][cc];
            const uint32_t hi = s_dt[p][q * 8 + 2 * j + 1][cc];
            bw[j] = lo | (hi << 16);
          }
          const uint4 bv = make_uint4(bw[0], bw[1], bw[2], bw[3]);
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(a), as_frag(bv), acc[b], 0, 0, 0);
        }
      }
    }
  }
  // C[4q + i][16 b + col] of block b: token 4q + i, column c0 + 64 wave + 16 b + col
  if (S == 1) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int ycol = c0 + 64 * wave + 16 * b + col;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        if (m < n && ycol < d) y[(size_t)m * d + ycol] = acc[b][i];
      }
    }
    return;
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int ycol = c0 + 64 * wave + 16 * b + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * q + i;
      if (m < n && ycol < d) part[((size_t)s * n + m) * d + ycol] = acc[b][i];
    }
  }
}

// y = sum over the S splits of part[s, :, :], in split order; one float4 per thread.
__global__ __launch_bounds__(256) void chunk_reduce_kernel(const float* __restrict__ part, int S, int n4,
                                                           float* __restrict__ y) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n4) return;
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(part) + e;
  f32x4_t tot = {0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 8 <= S; s += 8) {
    f32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(size_t)(s + u) * n4];
#pragma unroll
    for (int u = 0; u < 8; ++u) tot += v[u];
  }
  for (; s < S; ++s) tot += src[(size_t)s * n4];
  reinterpret_cast<f32x4_t*>(y)[e] = tot;
}

int chunk_splits(int d, int f) {
  const int ntile = (d + kCT - 1) / kCT;
  int S = (1024 + ntile - 1) / ntile;  // about 1024 workgroups
  const int maxs = (f + 255) / 256;
  if (S > maxs) S = maxs;
  return S < 1 ? 1 : S;
}

}  // namespace

// Chunks of at most this many bf16 tokens run through the decode kernels with threshold 0
// (every neuron that contributes). One token, graph replay: 48.8 against 58.9 us at d
// 4096, f 11008; 61.0 against 76.4 at f 14336; 218.9 against 249.0 at d 8192, f 28672.
// With two to four tokens neither path wins everywhere (60-79 us against 60-79 at d
// 4096; 230-242 against 249-251 at d 8192), so they stay on the matrix cores.
constexpr int kDecodeDenseMax = 1;

size_t chunk_workspace_bytes(int d, int f, int wdtype, int n) {
  if (wdtype != SFN_BF16) {
    // fp32 weights run through the decode kernel, 4 tokens at a time
    return decode_workspace_bytes(d, f, 4, n > 1 ? 4 : 1);
  }
  if (n <= kDecodeDenseMax) return decode_workspace_bytes(d, f, 2, n);
  const int S = chunk_splits(d, f);
  size_t bytes = kWsHeader;
  bytes += (size_t)SFN_MAX_CHUNK * ((f + 7) & ~7) * sizeof(uint16_t);
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += (size_t)S * SFN_MAX_CHUNK * d * sizeof(float);
  (void)n;
  return bytes;
}

hipError_t launch_dense_chunk(const sfn_ffn& ffn, const void* x, int n, float* y, void* ws, hipStream_t stream) {
  if (ffn.wdtype != SFN_BF16 || n <= kDecodeDenseMax) {
    // |act(g)| > 0 keeps every neuron that contributes, so this is the dense FFN.
    const int wb = ffn.wdtype == SFN_BF16 ? 2 : 4;
    DecodeArgs a{};
    a.wg = static_cast<const char*>(ffn.w_gate);
    a.wu = static_cast<const char*>(ffn.w_up);
    a.wd = static_cast<const char*>(ffn.w_down_t);
    a.bias = ffn.b_gate;
    a.d = ffn.d;
    a.f = ffn.f;
    a.nch = ffn.d * wb / 16;
    a.row_bytes = ffn.d * wb;
    a.act = ffn.act;
    a.G = decode_grid(ffn.f);
    decode_carve(a, ws, wb);
    for (int j0 = 0; j0 < n; j0 += SFN_MAX_BATCH) {
      const int nb = n - j0 < SFN_MAX_BATCH ? n - j0 : SFN_MAX_BATCH;
      a.x = static_cast<const char*>(x) + (size_t)j0 * a.row_bytes;
      a.y = y + (size_t)j0 * ffn.d;
      a.nb = nb;
      a.n_red = decode_reducers(a.G, nb, ffn.d);
      hipError_t e = launch_decode(a, ffn.wdtype, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int ntile = (ffn.d + kCT - 1) / kCT;
  const int S = chunk_splits(ffn.d, ffn.f);
  char* p = static_cast<char*>(ws);
  size_t off = kWsHeader;
  uint16_t* H = reinterpret_cast<uint16_t*>(p + off);
  off += (size_t)SFN_MAX_CHUNK * ((ffn.f + 7) & ~7) * sizeof(uint16_t);
  off = (off + 255) & ~(size_t)255;
  float* part = reinterpret_cast<float*>(p + off);
  if ((ffn.f + 15) / 16 > kGW) {
    // enough rows that kGW workgroups of up to kRowsW rows each are all full-width
    int g1 = kGW;
    if (g1 < (ffn.f + kRowsW - 1) / kRowsW) g1 = (ffn.f + kRowsW - 1) / kRowsW;
    hipLaunchKernelGGL(chunk_stage1_wide_kernel, dim3(g1), dim3(256), 0, stream,
                       static_cast<const char*>(ffn.w_gate), static_cast<const char*>(ffn.w_up), ffn.b_gate,
                       static_cast<const char*>(x), n, ffn.d, ffn.f, ffn.act, H);
  } else {
    hipLaunchKernelGGL(chunk_stage1_kernel, dim3((ffn.f + 15) / 16), dim3(256), 0, stream,
                       static_cast<const char*>(ffn.w_gate), static_cast<const char*>(ffn.w_up), ffn.b_gate,
                       static_cast<const char*>(x), n, ffn.d, ffn.f, ffn.act, H);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_stage2_kernel, dim3(ntile * S), dim3(256), 0, stream, H,
                     static_cast<const char*>(ffn.w_down_t), n, ffn.d, ffn.f, S, part, y);
  if (S > 1) {
    const int n4 = n * ffn.d / 4;
    hipLaunchKernelGGL(chunk_reduce_kernel, dim3((n4 + 255) / 256), dim3(256), 0, stream, part, S, n4, y);
  }
  return hipGetLastError();
}

}  // namespace sfn
