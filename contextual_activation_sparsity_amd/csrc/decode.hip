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

// The kernel's view of DecodeArgs: the same fields with global-address-space pointers,
// held in registers (built from the by-value argument at kernel entry).
struct DevArgs {
  const SFN_GLOBAL char* wg;
  const SFN_GLOBAL char* wu;
  const SFN_GLOBAL char* wd;
  const SFN_GLOBAL float* bias;
  const SFN_GLOBAL char* x;
  const SFN_GLOBAL float* t;
  const SFN_GLOBAL int32_t* cand;
  const SFN_GLOBAL int32_t* n_cand;
  const SFN_GLOBAL uint8_t* mask_in;
  SFN_GLOBAL float* y;
  SFN_GLOBAL int32_t* active_idx;
  SFN_GLOBAL int32_t* n_active;
  SFN_GLOBAL Ctrl* ctrl;
  SFN_GLOBAL int32_t* tile_cnt;
  SFN_GLOBAL int32_t* tile_idx;
  SFN_GLOBAL float* part;
  int d, f, nch, row_bytes, nb, act, G, n_red;
};

__device__ __forceinline__ DevArgs dev_args(const DecodeArgs& h) {
  DevArgs a;
  a.wg = gp(h.wg); a.wu = gp(h.wu); a.wd = gp(h.wd); a.bias = gp(h.bias); a.x = gp(h.x); a.t = gp(h.t);
  a.cand = gp(h.cand); a.n_cand = gp(h.n_cand); a.mask_in = gp(h.mask_in); a.y = gp(h.y);
  a.active_idx = gp(h.active_idx); a.n_active = gp(h.n_active); a.ctrl = gp(h.ctrl);
  a.tile_cnt = gp(h.tile_cnt); a.tile_idx = gp(h.tile_idx); a.part = gp(h.part);
  a.d = h.d; a.f = h.f; a.nch = h.nch; a.row_bytes = h.row_bytes; a.nb = h.nb; a.act = h.act; a.G = h.G;
  a.n_red = h.n_red;
  return a;
}

// Zero words that stand in for absent optional inputs, so that every step issues the
// same loads whatever it holds.
__device__ __attribute__((aligned(16))) float g_zero_f32[4];
__device__ __attribute__((aligned(16))) uint8_t g_zero_u8[16];

template <int WT, int BMAX, int CPT, int TPR, int R>
struct DecodeKernel {
  using CK = Chunk<WT>;
  static constexpr int RPG = kNT / TPR;  // rows processed side by side
  static constexpr int RG = RPG * R;     // rows of an up/down step (and of half a gate step)
  static constexpr int RS = 2 * RG;      // rows of a gate step
  static constexpr int VG = 2 * R * BMAX;
  static constexpr int VU = R * BMAX;
  static constexpr int WPR = TPR / 64;   // waves per row
  static constexpr int KV = CK::kVals;
  static_assert(RS <= 64, "one lane of wave 0 per row of a gate step");
  static_assert((VG & (VG - 1)) == 0 && VG <= 64, "power-of-two value count");

  struct Smem {
    int rowid[kTMax];         // candidate mode: global row of each local row
    float aval[kTMax][BMAX];  // activation per local row and token
    uint8_t mbits[kTMax];     // bit b: token b active
    int queue[kTMax];         // local rows active for some token, ascending
    float wpart[kNW][VG];     // per-wave partial sums of a step
    float h[64][BMAX];        // h = m a u of the rows of an up/down step
    float red[kNT];           // reducer scratch
    int pref[1025];           // tile prefix (index output)
    int qlen;
    int cnt[BMAX];
    uint32_t ticket;
    uint32_t rel0;
  };

  // Loads of one step into a buffer. The instruction stream is the same for every kind
  // of step (only addresses differ), so the compiler can count the loads in flight and
  // wait for exactly the older buffer:
  //   gate:    w0 = Wg rows [base, base+RG), w1 = Wg rows [base+RG, base+RS)
  //   up/down: w0 = Wu rows, w1 = Dt rows of queue entries [base, base+n)
  //   none:    both from x (L1-resident), results unused
  // Rows past the end are clamped to a valid row; their results are masked later.
  // Each lane also fetches the bias and mask bytes of gate row (lane % RS).
  __device__ __forceinline__ static void issue(const DevArgs& a, const Smem& sm, const StepDesc& sd, int r0,
                                               int nrows, bool cand_mode, int rl, int cl, int lane,
                                               uint4 (&w0)[R][CPT], uint4 (&w1)[R][CPT], float& bias,
                                               uint32_t (&mraw)[BMAX], uint32_t& valid) {
    const bool gate = sd.kind == STEP_GATE, upd = sd.kind == STEP_UPDOWN;
    const SFN_GLOBAL char* p0 = gate ? a.wg : (upd ? a.wu : a.x);
    const SFN_GLOBAL char* p1 = gate ? a.wg : (upd ? a.wd : a.x);
    const size_t rb = (sd.kind == STEP_NONE) ? 0 : (size_t)a.row_bytes;
    const int lrmax = nrows > 0 ? nrows - 1 : 0;
    valid = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int j = rl + RPG * k;
      int lr0, lr1;
      bool v0, v1;
      if (gate) {
        lr0 = sd.base + j;
        lr1 = sd.base + RG + j;
        v0 = lr0 < nrows;
        v1 = lr1 < nrows;
      } else {
        v0 = v1 = upd && j < sd.n;
        lr0 = lr1 = sm.queue[min(sd.base + j, kTMax - 1)];
      }
      lr0 = min(max(lr0, 0), lrmax);
      lr1 = min(max(lr1, 0), lrmax);
      const int g0 = cand_mode ? sm.rowid[lr0] : r0 + lr0;
      const int g1 = cand_mode ? sm.rowid[lr1] : r0 + lr1;
      valid |= (uint32_t)v0 << k;
      valid |= (uint32_t)v1 << (R + k);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        int ch = cl + TPR * c;
        ch = ch < a.nch ? ch : 0;
        w0[k][c] = ldg16(p0 + (size_t)g0 * rb + (size_t)ch * 16);
        w1[k][c] = ldg16(p1 + (size_t)g1 * rb + (size_t)ch * 16);
      }
    }
    // bias and mask bytes of gate row (lane % RS) of this step
    int lb = gate ? sd.base + (lane % RS) : 0;
    lb = min(max(lb, 0), lrmax);
    const int gb = cand_mode ? sm.rowid[lb] : r0 + lb;
    bias = a.bias ? a.bias[gb] : gp(g_zero_f32)[0];
    // raw bytes: tested only when the step is processed, so no wait is forced here
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      const int bb = b < a.nb ? b : 0;
      mraw[b] = a.mask_in ? a.mask_in[(size_t)bb * a.f + gb] : gp(g_zero_u8)[b];
    }
  }

  // Wave totals of NV values per thread into sm.wpart[wave][0..NV): blocks of up to 16
  // values are transposed and summed across the wave, then written by one lane each.
  template <int NV>
  __device__ __forceinline__ static void reduce_to_lds(Smem& sm, float (&s)[NV]) {
    constexpr int BLK = NV < 16 ? NV : 16;
    constexpr int LOGB = (BLK >= 16) ? 4 : (BLK >= 8) ? 3 : (BLK >= 4) ? 2 : (BLK >= 2) ? 1 : 0;
    constexpr int SH = 6 - LOGB;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int blk = 0; blk < NV / BLK; ++blk) {
      float t[BLK];
#pragma unroll
      for (int i = 0; i < BLK; ++i) t[i] = s[blk * BLK + i];
      wave_transpose_sum<BLK>(t);
      if ((lane & ((1 << SH) - 1)) == 0) sm.wpart[threadIdx.x >> 6][blk * BLK + (lane >> SH)] = t[0];
    }
  }

  __device__ __forceinline__ static float wave_partial_sum(const Smem& sm, int rlj, int v) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < WPR; ++i) acc += sm.wpart[rlj * WPR + i][v];
    return acc;
  }

  __device__ static void run(const DecodeArgs& args) {
    const DevArgs a = dev_args(args);
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

    // ---- software-pipelined steps (one issued ahead of the one processed)
    const int ngate = (nrows + RS - 1) / RS;
    int next_gate = 0;  // gate steps issued
    int gates_done = 0; // gate steps processed
    int qh = 0;         // queue rows handed to up/down steps
    auto next_step = [&]() -> StepDesc {
      StepDesc sd{STEP_NONE, 0, 0};
      if (next_gate < ngate) {
        sd.kind = STEP_GATE;
        sd.base = next_gate * RS;
        sd.n = min(RS, nrows - sd.base);
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

    auto process = [&](const StepDesc& sd, const uint4 (&w0)[R][CPT], const uint4 (&w1)[R][CPT], float bias,
                       const uint32_t (&mraw)[BMAX], uint32_t valid) {
      if (sd.kind == STEP_GATE) {
        float s[VG];
#pragma unroll
        for (int k = 0; k < R; ++k)
#pragma unroll
          for (int b = 0; b < BMAX; ++b) {
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
              d0 = CK::dot(w0[k][c], xr[b][c], d0);
              d1 = CK::dot(w1[k][c], xr[b][c], d1);
            }
            s[k * BMAX + b] = d0;
            s[(R + k) * BMAX + b] = d1;
          }
        reduce_to_lds<VG>(sm, s);
        __syncthreads();
        if (wave == 0) {
          // lane j finalizes row j of the step: half h = j / RG, row-lane j % RPG, slot k
          const int j = lane;
          const int hh = j / RG, jj = j % RG;
          const int rlj = jj % RPG, k = jj / RPG;
          const bool ok = j < sd.n;
          const int lr = sd.base + j;
          uint32_t bits = 0;
          int grow = 0;
          if (ok) {
            grow = cand_mode ? sm.rowid[lr] : r0 + lr;
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
              if (b < nb) {
                const float g = wave_partial_sum(sm, rlj, (hh * R + k) * BMAX + b) + bias;
                const float av = (a.act == 0) ? silu_f(g) : fmaxf(g, 0.f);
                const bool on = a.mask_in ? mraw[b] != 0u : fabsf(av) > thr;
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
                if (on)
                  __hip_atomic_store(&a.tile_idx[(size_t)b * a.f + r0 + c0 + pb], grow, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
                if (lane == 0) sm.cnt[b] = c0 + __popcll(bb);
              }
            }
          }
          if (lane == 0) sm.qlen = q0 + __popcll(ub);
        }
        __syncthreads();
        ++gates_done;
      } else if (sd.kind == STEP_UPDOWN) {
        float s[VU];
#pragma unroll
        for (int k = 0; k < R; ++k)
#pragma unroll
          for (int b = 0; b < BMAX; ++b) {
            float d0 = 0.f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) d0 = CK::dot(w0[k][c], xr[b][c], d0);
            s[k * BMAX + b] = d0;
          }
        reduce_to_lds<VU>(sm, s);
        __syncthreads();
        if (wave == 0 && lane < sd.n) {
          const int lr = sm.queue[sd.base + lane];
          const uint32_t bits = sm.mbits[lr];
          const int rlj = lane % RPG, k = lane / RPG;
#pragma unroll
          for (int b = 0; b < BMAX; ++b) {
            const float u = wave_partial_sum(sm, rlj, k * BMAX + b);
            sm.h[lane][b] = ((bits >> b) & 1u) ? sm.aval[lr][b] * u : 0.f;
          }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < R; ++k) {
          if ((valid >> (R + k)) & 1u) {
            const int j = rl + RPG * k;
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
    float abias, bbias;
    uint32_t amask[BMAX], bmask[BMAX], avalid, bvalid;
    StepDesc sa = next_step();
    issue(a, sm, sa, r0, nrows, cand_mode, rl, cl, lane, a0, a1, abias, amask, avalid);
    while (true) {
      StepDesc sb = next_step();
      issue(a, sm, sb, r0, nrows, cand_mode, rl, cl, lane, b0, b1, bbias, bmask, bvalid);
      process(sa, a0, a1, abias, amask, avalid);
      if (sa.kind == STEP_NONE && sb.kind == STEP_NONE && gates_done == ngate && (!want_y || qh == sm.qlen)) break;
      sa = next_step();
      issue(a, sm, sa, r0, nrows, cand_mode, rl, cl, lane, a0, a1, abias, amask, avalid);
      process(sb, b0, b1, bbias, bmask, bvalid);
      if (sa.kind == STEP_NONE && sb.kind == STEP_NONE && gates_done == ngate && (!want_y || qh == sm.qlen)) break;
    }

    // ---- partial of y (device-coherent stores: read by other workgroups below)
    if (want_y) {
      SFN_GLOBAL float* prow = a.part + ((size_t)(w * RPG + rl) * nb) * a.d;
#pragma unroll
      for (int b = 0; b < BMAX; ++b) {
        if (b < nb) {
#pragma unroll
          for (int c = 0; c < CPT; ++c) {
            const int ch = cl + TPR * c;
            if (ch < a.nch) {
              SFN_GLOBAL float* dst = prow + (size_t)b * a.d + (size_t)ch * KV;
#pragma unroll
              for (int v = 0; v < KV; ++v)
                __hip_atomic_store(dst + v, acc[b][c][v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
    if (want_idx && tid < kBMaxAll)
      __hip_atomic_store(&a.tile_cnt[w * kBMaxAll + tid], (tid < BMAX) ? sm.cnt[tid] : 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);

    // ---- arrival; the last n_red workgroups reduce.
    // No cache-maintenance fences: the partials above are device-scope stores that write
    // through to the coherent level, s_waitcnt 0 waits until every one of them is
    // acknowledged, and the readers use device-scope loads. (An agent-scope release or
    // acquire fence would write back or invalidate the whole L2 of the XCD.)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      sm.rel0 = __hip_atomic_load(&a.ctrl->release, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      sm.ticket = __hip_atomic_fetch_add(&a.ctrl->arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        __builtin_amdgcn_s_waitcnt(0);
        __hip_atomic_fetch_add(&a.ctrl->release, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const uint32_t r0v = sm.rel0;
        uint32_t spins = 0;
        while (__hip_atomic_load(&a.ctrl->release, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == r0v) {
          __builtin_amdgcn_s_sleep(1);
          if (++spins > (1u << 24)) {
            __hip_atomic_store(&a.ctrl->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
        }
      }
    }
    __syncthreads();
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
        if (pg < npg && e < SL) {
          const SFN_GLOBAL float* src = a.part + s0 + e;
          int p = pg;
          // eight device-scope loads in flight, summed in partial order
          for (; p + 7 * npg < P; p += 8 * npg) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
              v[u] = __hip_atomic_load(src + (size_t)(p + u * npg) * L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
          }
          for (; p < P; p += npg) sum += __hip_atomic_load(src + (size_t)p * L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
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
          for (int p = 0; p < P; ++p)
            sum += __hip_atomic_load(a.part + (size_t)p * L + s0 + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        for (int i = tid; i <= a.G; i += kNT)
          sm.pref[i] = (i < a.G) ? __hip_atomic_load(&a.tile_cnt[i * kBMaxAll + b], __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : 0;
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
              a.active_idx[(size_t)b * a.f + sm.pref[tile] + i] =
                  __hip_atomic_load(&a.tile_idx[(size_t)b * a.f + tr0 + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  // rows per thread per half step: 16 weight loads in flight per thread and buffer for
  // one token, 8 for four tokens (the dot-product registers grow with the batch)
  constexpr int RB = BMAX == 1 ? 8 : 4;
  const dim3 grid(a.G), block(kNT);
  if (a.nch > 2048) return hipErrorInvalidValue;
  if (a.nch > 1024) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 4, 512, RB / 4>), grid, block, 0, s, a); }
  else if (a.nch > 512) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 2, 512, RB / 2>), grid, block, 0, s, a); }
  else if (a.nch > 256) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 1, 512, RB>), grid, block, 0, s, a); }
  else if (a.nch > 128) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 1, 256, RB>), grid, block, 0, s, a); }
  else if (a.nch > 64) { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 1, 128, RB>), grid, block, 0, s, a); }
  else { hipLaunchKernelGGL((decode_kernel<WT, BMAX, 1, 64, 4>), grid, block, 0, s, a); }
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
