// Sparse gated-FFN decode step: one fused kernel per layer.
//
// What it computes (for each token b of the batch):
//   g = Wg x_b + bias, a = act(g), m_bi = [|a_i| > t] (or the mask override, or the
//   candidate restriction), y_b = sum_i m_bi a_bi (Wu x_b)_i Dt[i, :]
// i.e. the CATS thresholded SwiGLU ("CATS: Contextually-Aware Thresholding for Sparsity
// in Large Language Models", abstract) and the ReGLU sequential pipeline of "SVD
// Contextual Sparsity Predictors for Fast LLM Inference" (Figure 3: gate on the
// predicted rows, up and down only where ReLU(gate) > 0).
//
// How (one launch, G workgroups of 512 threads, all HBM-bound GEMV work):
//   1. Each workgroup owns a contiguous tile of rows (or an equal share of the candidate
//      list). Gate rows are streamed in steps of RG rows; thread t of a row reads 16-byte
//      chunk t, so a 4096-wide bf16 row is one fully coalesced 8 KB sweep of the
//      workgroup. Partial dot products are reduced with a multi-value transposing
//      butterfly (DPP + swizzles) and a per-wave LDS hand-off.
//   2. Wave 0 turns each step's sums into activations, applies the threshold and
//      appends the active rows to an LDS queue with a ballot + mbcnt compaction, in
//      ascending row order.
//   3. Queue rows are consumed in steps of RG: the Wu and Dt rows (each one contiguous
//      row, Dt being W_down transposed) are loaded together, u = Wu x is reduced like
//      the gate, h = m a u goes through LDS, and every thread accumulates h * Dt into
//      fp32 registers for the columns of its chunk.
//   Steps are software pipelined: the loads of the next step (gate or up/down) are in
//   flight while the current one is reduced, so the memory pipe does not drain at the
//   gate -> up/down transition.
//   4. Each workgroup writes its fp32 partial of y. The last n_red workgroups to finish
//      (an arrival ticket) wait for the rest and then sum the partials column slice by
//      column slice in a fixed order, so y is deterministic. Waiting only in the last
//      n_red < resident-capacity arrivals cannot deadlock: every other workgroup has a
//      free slot to run in.

#include "device_common.h"
#include "kernels.h"

namespace sfn {

namespace {

constexpr int kNT = 512;       // threads per workgroup
constexpr int kNW = kNT / 64;  // waves per workgroup
constexpr int kTMax = 256;     // rows per workgroup tile
constexpr int kBMaxAll = 4;

enum StepKind { STEP_NONE = 0, STEP_GATE = 1, STEP_UPDOWN = 2 };

struct StepDesc {
  int kind;
  int base;  // gate: first local row of the step; up/down: first queue position
  int n;     // rows in the step
};

template <int WT, int BMAX, int CPT, int TPR, int R>
struct DecodeKernel {
  using CK = Chunk<WT>;
  static constexpr int RPG = kNT / TPR;  // rows processed side by side
  static constexpr int RG = RPG * R;     // rows per step
  static constexpr int V = R * BMAX;     // values each thread reduces per step
  static constexpr int WPR = TPR / 64;   // waves per row
  static constexpr int KV = CK::kVals;
  static_assert(RG <= 64, "one lane of wave 0 per row of a step");
  static_assert((V & (V - 1)) == 0 && V <= 64, "power-of-two value count");

  struct Smem {
    int rowid[kTMax];            // candidate mode: global row of each local row
    float aval[kTMax][BMAX];     // activation per local row and token
    uint8_t mbits[kTMax];        // bit b: token b active
    int queue[kTMax];            // local rows active for some token, ascending
    float wpart[kNW][V];         // per-wave partial sums of a step
    float h[64][BMAX];           // h = m a u of the rows of an up/down step
    float red[kNT];              // reducer scratch
    int pref[1025];              // tile prefix (index output)
    int qlen;
    int cnt[BMAX];
    uint32_t ticket;
    uint32_t rel0;
  };

  // Loads of one step: gate rows into w0, or Wu rows into w0 and Dt rows into w1.
  __device__ __forceinline__ static void issue(const DecodeArgs& a, const Smem& sm, const StepDesc& sd,
                                               int r0, bool cand_mode, int rl, int cl,
                                               uint4 (&w0)[R][CPT], uint4 (&w1)[R][CPT]) {
    if (sd.kind == STEP_NONE) return;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int j = rl + RPG * k;
      const bool valid = j < sd.n;
      int grow = 0;
      if (valid) {
        const int lr = (sd.kind == STEP_GATE) ? sd.base + j : sm.queue[sd.base + j];
        grow = cand_mode ? sm.rowid[lr] : r0 + lr;
      }
      const size_t roff = (size_t)grow * (size_t)a.row_bytes;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int ch = cl + TPR * c;
        const bool ok = valid && ch < a.nch;
        if (sd.kind == STEP_GATE) {
          w0[k][c] = ok ? ldg16(a.wg + roff + (size_t)ch * 16) : make_uint4(0, 0, 0, 0);
        } else {
          w0[k][c] = ok ? ldg16(a.wu + roff + (size_t)ch * 16) : make_uint4(0, 0, 0, 0);
          w1[k][c] = ok ? ldg16(a.wd + roff + (size_t)ch * 16) : make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  // Dot products of the step's rows with the tokens, reduced to per-wave partials.
  __device__ __forceinline__ static void dots_to_lds(Smem& sm, const uint4 (&w)[R][CPT],
                                                     const uint4 (&xr)[BMAX][CPT]) {
    float s[V];
#pragma unroll
    for (int k = 0; k < R; ++k)
#pragma unroll
      for (int b = 0; b < BMAX; ++b) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc = CK::dot(w[k][c], xr[b][c], acc);
        s[k * BMAX + b] = acc;
      }
    wave_transpose_sum<V>(s);
    const int lane = threadIdx.x & 63;
    constexpr int LOGV = (V >= 64) ? 6 : (V >= 32) ? 5 : (V >= 16) ? 4 : (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;
    constexpr int SH = 6 - LOGV;
    if ((lane & ((1 << SH) - 1)) == 0) sm.wpart[threadIdx.x >> 6][lane >> SH] = s[0];
  }

  // Sum of the wave partials of row j (0 <= j < RG) of a step, token b.
  __device__ __forceinline__ static float row_sum(const Smem& sm, int j, int b) {
    const int rlj = j % RPG, k = j / RPG;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < WPR; ++i) acc += sm.wpart[rlj * WPR + i][k * BMAX + b];
    return acc;
  }

  __device__ static void run(const DecodeArgs& a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = tid / TPR, cl = tid % TPR;
    const int w = blockIdx.x;
    const bool cand_mode = a.cand != nullptr;
    const bool want_y = a.y != nullptr;
    const bool want_idx = a.active_idx != nullptr || a.n_active != nullptr;
    const int nb = a.nb;

    // ---- this workgroup's rows
    int r0, nrows;
    if (cand_mode) {
      const int n = min(max(*a.n_cand, 0), a.f);  // a count beyond f cannot be a valid list
      r0 = (int)((long long)w * n / a.G);
      nrows = (int)((long long)(w + 1) * n / a.G) - r0;
      for (int i = tid; i < nrows; i += kNT) sm.rowid[i] = min(max(a.cand[r0 + i], 0), a.f - 1);  // stay in bounds
    } else {
      r0 = (int)((long long)w * a.f / a.G);
      nrows = (int)((long long)(w + 1) * a.f / a.G) - r0;
    }
    if (tid == 0) sm.qlen = 0;
    if (tid < BMAX) sm.cnt[tid] = 0;

    // ---- token chunks in registers (zero beyond the row or the batch)
    uint4 xr[BMAX][CPT];
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int ch = cl + TPR * c;
        xr[b][c] = (b < nb && ch < a.nch) ? ld16(a.x + (size_t)b * a.row_bytes + (size_t)ch * 16)
                                          : make_uint4(0, 0, 0, 0);
      }
    const float thr = a.t ? *a.t : 0.0f;
    float acc[BMAX][CPT][KV];
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int v = 0; v < KV; ++v) acc[b][c][v] = 0.f;
    __syncthreads();

    // ---- software-pipelined steps
    const int ngate = (nrows + RG - 1) / RG;
    int next_gate = 0;  // gate steps issued
    int qh = 0;         // queue rows handed to up/down steps
    auto next_step = [&]() -> StepDesc {
      StepDesc sd{STEP_NONE, 0, 0};
      if (next_gate < ngate) {
        sd.kind = STEP_GATE;
        sd.base = next_gate * RG;
        sd.n = min(RG, nrows - sd.base);
        ++next_gate;
      } else if (want_y) {
        const int ql = sm.qlen;
        if (qh < ql) {
          sd.kind = STEP_UPDOWN;
          sd.base = qh;
          sd.n = min(RG, ql - qh);
          qh += sd.n;
        }
      }
      return sd;
    };

    auto process = [&](const StepDesc& sd, const uint4 (&w0)[R][CPT], const uint4 (&w1)[R][CPT]) {
      dots_to_lds(sm, w0, xr);
      __syncthreads();
      if (sd.kind == STEP_GATE) {
        if (wave == 0) {
          const int j = lane;
          const bool valid = j < sd.n;
          const int lr = sd.base + j;
          uint32_t bits = 0;
          int grow = 0;
          if (valid) {
            grow = cand_mode ? sm.rowid[lr] : r0 + lr;
            const float bias = a.bias ? a.bias[grow] : 0.f;
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
              if (b < nb) {
                const float g = row_sum(sm, j, b) + bias;
                const float av = (a.act == 0) ? silu_f(g) : fmaxf(g, 0.f);
                bool on;
                if (a.mask_in) on = a.mask_in[(size_t)b * a.f + grow] != 0;
                else on = fabsf(av) > thr;
                sm.aval[lr][b] = av;
                bits |= (uint32_t)on << b;
              }
            }
            sm.mbits[lr] = (uint8_t)bits;
          }
          const unsigned long long ub = __ballot(bits != 0);
          const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(ub >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ub, 0));
          const int q0 = sm.qlen;
          if (bits != 0) sm.queue[q0 + pos] = lr;
          if (want_idx) {
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
              if (b < nb) {
                const bool on = (bits >> b) & 1u;
                const unsigned long long bb = __ballot(on);
                const int pb = __builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0));
                const int c0 = sm.cnt[b];
                if (on) a.tile_idx[(size_t)b * a.f + r0 + c0 + pb] = grow;
                if (lane == 0) sm.cnt[b] = c0 + __popcll(bb);
              }
            }
          }
          if (lane == 0) sm.qlen = q0 + __popcll(ub);
        }
        __syncthreads();
      } else {
        if (wave == 0 && lane < sd.n) {
          const int lr = sm.queue[sd.base + lane];
          const uint32_t bits = sm.mbits[lr];
#pragma unroll
          for (int b = 0; b < BMAX; ++b) {
            const float u = row_sum(sm, lane, b);
            sm.h[lane][b] = ((bits >> b) & 1u) ? sm.aval[lr][b] * u : 0.f;
          }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const int j = rl + RPG * k;
          if (j < sd.n) {
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
              const float hv = sm.h[j][b];
#pragma unroll
              for (int c = 0; c < CPT; ++c) CK::axpy(hv, w1[k][c], acc[b][c]);
            }
          }
        }
      }
    };

    uint4 a0[R][CPT], a1[R][CPT], b0[R][CPT], b1[R][CPT];
    StepDesc da = next_step();
    issue(a, sm, da, r0, cand_mode, rl, cl, a0, a1);
    while (da.kind != STEP_NONE) {
      StepDesc db = next_step();
      issue(a, sm, db, r0, cand_mode, rl, cl, b0, b1);
      process(da, a0, a1);
      if (db.kind == STEP_NONE) {
        db = next_step();
        issue(a, sm, db, r0, cand_mode, rl, cl, b0, b1);
      }
      if (db.kind == STEP_NONE) break;
      StepDesc dn = next_step();
      issue(a, sm, dn, r0, cand_mode, rl, cl, a0, a1);
      process(db, b0, b1);
      if (dn.kind == STEP_NONE) {
        dn = next_step();
        issue(a, sm, dn, r0, cand_mode, rl, cl, a0, a1);
      }
      da = dn;
    }

    // ---- partial of y and the tile's index counts
    if (want_y) {
      float* prow = a.part + ((size_t)(w * RPG + rl) * nb) * a.d;
#pragma unroll
      for (int b = 0; b < BMAX; ++b) {
        if (b < nb) {
#pragma unroll
          for (int c = 0; c < CPT; ++c) {
            const int ch = cl + TPR * c;
            if (ch < a.nch) {
              float* dst = prow + (size_t)b * a.d + (size_t)ch * KV;
#pragma unroll
              for (int v = 0; v < KV; v += 4)
                *reinterpret_cast<float4*>(dst + v) = make_float4(acc[b][c][v], acc[b][c][v + 1], acc[b][c][v + 2], acc[b][c][v + 3]);
            }
          }
        }
      }
    }
    if (want_idx && tid < kBMaxAll) a.tile_cnt[w * kBMaxAll + tid] = (tid < BMAX) ? sm.cnt[tid] : 0;

    // ---- arrival; the last n_red workgroups reduce
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0) {
      sm.rel0 = __hip_atomic_load(&a.ctrl->release, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.ticket = __hip_atomic_fetch_add(&a.ctrl->arrive, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const uint32_t ticket = sm.ticket;
    const uint32_t first_red = (uint32_t)(a.G - a.n_red);
    if (ticket >= (uint32_t)a.G) {
      // control words not zero at launch (workspace not zero-filled, or shared by
      // overlapping calls): flag it and write nothing rather than out of range
      if (tid == 0) __hip_atomic_store(&a.ctrl->error, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (ticket < first_red) return;
    if (tid == 0) {
      if (ticket == (uint32_t)(a.G - 1)) {
        __hip_atomic_store(&a.ctrl->arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(&a.ctrl->release, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const uint32_t r0v = sm.rel0;
        uint32_t spins = 0;
        while (__hip_atomic_load(&a.ctrl->release, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == r0v) {
          __builtin_amdgcn_s_sleep(2);
          if (++spins > (1u << 22)) {
            __hip_atomic_store(&a.ctrl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int ri = (int)(ticket - first_red);

    if (want_y) {
      const int L = nb * a.d;
      const int P = a.G * RPG;
      const int s0 = (int)((long long)ri * L / a.n_red);
      const int s1 = (int)((long long)(ri + 1) * L / a.n_red);
      const int SL = s1 - s0;
      const int slmax = (L + a.n_red - 1) / a.n_red;
      if (slmax <= kNT) {
        const int npg = kNT / slmax;
        const int e = tid % slmax, pg = tid / slmax;
        float sum = 0.f;
        if (pg < npg && e < SL)
          for (int p = pg; p < P; p += npg) sum += a.part[(size_t)p * L + s0 + e];
        sm.red[tid] = sum;
        __syncthreads();
        if (pg == 0 && e < SL) {
          float tot = sm.red[e];
          for (int g2 = 1; g2 < npg; ++g2) tot += sm.red[g2 * slmax + e];
          a.y[s0 + e] = tot;
        }
      } else {
        for (int e = tid; e < SL; e += kNT) {
          float sum = 0.f;
          for (int p = 0; p < P; ++p) sum += a.part[(size_t)p * L + s0 + e];
          a.y[s0 + e] = sum;
        }
      }
    }

    if (want_idx && ri == a.n_red - 1) {
      int n_total = a.f;
      if (cand_mode) n_total = min(max(*a.n_cand, 0), a.f);
      for (int b = 0; b < nb; ++b) {
        __syncthreads();
        // exclusive prefix of the tile counts, tiles in row order
        for (int i = tid; i <= a.G; i += kNT) sm.pref[i] = (i < a.G) ? a.tile_cnt[i * kBMaxAll + b] : 0;
        __syncthreads();
        if (tid == 0) {
          int run = 0;
          for (int i = 0; i <= a.G; ++i) {
            const int c = sm.pref[i];
            sm.pref[i] = run;
            run += c;
          }
        }
        __syncthreads();
        if (a.active_idx) {
          for (int tile = wave; tile < a.G; tile += kNW) {
            const int tr0 = (int)((long long)tile * n_total / a.G);
            const int c = sm.pref[tile + 1] - sm.pref[tile];
            for (int i = lane; i < c; i += 64)
              a.active_idx[(size_t)b * a.f + sm.pref[tile] + i] = a.tile_idx[(size_t)b * a.f + tr0 + i];
          }
        }
        if (tid == 0 && a.n_active) a.n_active[b] = sm.pref[a.G];
      }
    }
  }
};

template <int WT, int BMAX, int CPT, int TPR, int R>
__global__ __launch_bounds__(kNT) void decode_kernel(DecodeArgs a) {
  DecodeKernel<WT, BMAX, CPT, TPR, R>::run(a);
}

template <int WT, int BMAX>
hipError_t dispatch_tpr(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.G), block(kNT);
  if (a.nch > 2048) return hipErrorInvalidValue;
  if (a.nch > 1024) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 4, 512, 2>), grid, block, 0, s, a); }
  else if (a.nch > 512) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 2, 512, 4>), grid, block, 0, s, a); }
  else if (a.nch > 256) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 1, 512, 8>), grid, block, 0, s, a); }
  else if (a.nch > 128) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 1, 256, 4>), grid, block, 0, s, a); }
  else if (a.nch > 64) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 1, 128, 8>), grid, block, 0, s, a); }
  else { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 1, 64, 8>), grid, block, 0, s, a); }
  return hipGetLastError();
}

}  // namespace

int decode_rows_side_by_side(int nch) {
  if (nch > 256) return 1;
  if (nch > 128) return 2;
  if (nch > 64) return 4;
  return 8;
}

int decode_grid(int f) {
  int g = (f + 7) / 8;
  if (g > 256) g = 256;
  const int need = (f + kTMax - 1) / kTMax;
  if (g < need) g = need;
  return g < 1 ? 1 : g;
}

int decode_reducers(int G, int nb, int d) {
  int n = (nb * d + 31) / 32;
  const int cap = G / 2 > 1 ? G / 2 : 1;
  if (n > cap) n = cap;
  return n < 1 ? 1 : n;
}

size_t decode_workspace_bytes(int d, int f, int wb, int nb) {
  const int G = decode_grid(f);
  const int nch = d * wb / 16;
  const size_t rpg = (size_t)decode_rows_side_by_side(nch);
  size_t bytes = kWsHeader;
  bytes += (size_t)G * kBMaxAll * sizeof(int32_t);
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += (size_t)kBMaxAll * f * sizeof(int32_t);
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += (size_t)G * rpg * nb * d * sizeof(float);
  return bytes;
}

void decode_carve(DecodeArgs& a, void* ws, int wb) {
  char* p = static_cast<char*>(ws);
  a.ctrl = reinterpret_cast<Ctrl*>(p);
  size_t off = kWsHeader;
  a.tile_cnt = reinterpret_cast<int32_t*>(p + off);
  off += (size_t)a.G * kBMaxAll * sizeof(int32_t);
  off = (off + 255) & ~(size_t)255;
  a.tile_idx = reinterpret_cast<int32_t*>(p + off);
  off += (size_t)kBMaxAll * a.f * sizeof(int32_t);
  off = (off + 255) & ~(size_t)255;
  a.part = reinterpret_cast<float*>(p + off);
  (void)wb;
}

hipError_t launch_decode(const DecodeArgs& a, int wdtype, hipStream_t s) {
  if (wdtype == WT_BF16) {
    return a.nb == 1 ? dispatch_tpr<WT_BF16, 1>(a, s) : dispatch_tpr<WT_BF16, 4>(a, s);
  }
  return a.nb == 1 ? dispatch_tpr<WT_F32, 1>(a, s) : dispatch_tpr<WT_F32, 4>(a, s);
}

}  // namespace sfn
