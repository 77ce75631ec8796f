// Sparse gated-FFN decode step: two launches per layer for one token, three for a batch.
//
// What it computes (for each token b of the batch):
//   g = Wg x_b + bias, a = act(g), m_bi = [|a_i| > t] (or the mask override, or the
//   candidate restriction), y_b = sum_i m_bi a_bi (Wu x_b)_i Dt[i, :]
// i.e. the CATS thresholded SwiGLU ("CATS: Contextually-Aware Thresholding for Sparsity
// in Large Language Models", abstract) and the ReGLU sequential pipeline of "SVD
// Contextual Sparsity Predictors for Fast LLM Inference" (Figure 3: gate on the
// predicted rows, up and down only where ReLU(gate) > 0).
//
// Gate (G workgroups of 512 threads, one tile of rows each, or an equal share of the
// candidate list): streams the gate rows. Thread t of a row reads 16-byte chunk t, so a
// 4096-wide bf16 row is one coalesced 8 KB sweep of the workgroup; partial dot products
// are reduced with a multi-value transposing butterfly (DPP + swizzles) and a per-wave
// LDS hand-off. Wave 0 turns the sums into activations, applies the threshold and
// compacts the active rows with ballot + mbcnt, in ascending order, into the tile's
// slice of a global list (row, activations, per-token bits) plus a count. Batches of 2
// to 4 tokens with bf16 weights take a matrix-core gate over 16-row tiles instead
// (decode_gate_mfma_kernel), with the same outputs. In predict mode each tile first runs
// the SVD predictor on its own rows and gates its candidates (predict_tile).
//
// Up/down: gathers the Wu and Dt rows of a list of active rows (each one contiguous row,
// Dt being W_down transposed), reduces u = Wu x like the gate, forms h = m a u and
// accumulates h * Dt into fp32 registers for the columns of its chunk, then writes the
// workgroup's fp32 partial of y with plain vector stores.
//  * One token (decode_gate_local_kernel, launch 1 of 2): the workgroup that gated a
//    tile streams the up/down rows of that tile's active rows right after, from a copy of
//    the list in LDS. A tile's share follows the spread of its active count, but the
//    separate launch, its scan over the tile counts and its gather of a share cost more.
//    For rows wider than 8 KB the tiles also even out their shares among themselves
//    through count words in the workspace header (Balancer).
//  * Batches (decode_updown_kernel, launch 2 of 3): the active lists of all tiles form one
//    concatenated list and each of Gu workgroups takes an equal share of it (a prefix over
//    the tile counts in LDS): the union rows of several tokens are many, and an even split
//    keeps every share within one row of the mean.
//
// In the streaming loops the loads of the next step are in flight while the current step
// is reduced (the issue sequence is the same for every kind of step, so the compiler's
// wait counts cover exactly the older buffer).
//
// Last launch, reduce kernel: y = the sum of the partials, column slice by column slice,
// in a fixed order, so y is deterministic; its workgroups also assemble the per-token
// active index lists, each the slices of a share of the gate tiles. The kernel boundary
// orders the partial stores before the loads. The decode path uses no fences; only the
// balancer (one token, rows wider than 8 KB) exchanges words between workgroups of one
// launch, with relaxed device-scope atomics.
//
// The one-pass kernel (parallel pipeline of the SVD predictor) reads the gate, up and
// down rows of each candidate together and ends in the same reduce kernel.

#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace sfn {

namespace {

constexpr int kNT = 512;       // threads per workgroup
constexpr int kNW = kNT / 64;  // waves per workgroup
constexpr int kTMax = 256;     // rows per tile / per up-down share
constexpr int kGMax = 1024;    // workgroups per launch
constexpr int kBMaxAll = 4;
constexpr int kCnt = 8;        // tile count stride: union, then one per token

enum StepKind { STEP_NONE = 0, STEP_GATE = 1, STEP_UPDOWN = 2 };

struct StepDesc {
  int kind;
  int base;  // first row (gate: tile-local row; up/down: share-local row)
  int n;     // rows in the step
};

// The kernels' view of DecodeArgs: the same fields with global-address-space pointers,
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
  SFN_GLOBAL int32_t* tile_cnt;
  SFN_GLOBAL int32_t* tile_idx;
  SFN_GLOBAL int32_t* sel_idx;
  SFN_GLOBAL float* sel_a;
  SFN_GLOBAL uint8_t* sel_bits;
  SFN_GLOBAL float* part;
  SFN_GLOBAL uint32_t* flags;
  const SFN_GLOBAL char* pl;
  const SFN_GLOBAL float* pz;
  const SFN_GLOBAL float* ptau;
  const SFN_GLOBAL float* pb;
  int pr;
  int d, f, nch, row_bytes, nb, act, G, n_red, Gu;
};

__device__ __forceinline__ DevArgs dev_args(const DecodeArgs& h) {
  DevArgs a;
  a.wg = gp(h.wg); a.wu = gp(h.wu); a.wd = gp(h.wd); a.bias = gp(h.bias); a.x = gp(h.x); a.t = gp(h.t);
  a.cand = gp(h.cand); a.n_cand = gp(h.n_cand); a.mask_in = gp(h.mask_in); a.y = gp(h.y);
  a.active_idx = gp(h.active_idx); a.n_active = gp(h.n_active);
  a.tile_cnt = gp(h.tile_cnt); a.tile_idx = gp(h.tile_idx); a.sel_idx = gp(h.sel_idx); a.sel_a = gp(h.sel_a);
  a.sel_bits = gp(h.sel_bits); a.part = gp(h.part); a.flags = gp(h.flags);
  a.pl = gp(h.pl); a.pz = gp(h.pz); a.ptau = gp(h.ptau); a.pb = gp(h.pb); a.pr = h.pr;
  a.d = h.d; a.f = h.f; a.nch = h.nch; a.row_bytes = h.row_bytes; a.nb = h.nb; a.act = h.act; a.G = h.G;
  a.n_red = h.n_red;
  a.Gu = h.Gu > 0 ? h.Gu : h.G;
  return a;
}

// Zero words that stand in for absent optional inputs, so that every step issues the
// same loads whatever it holds.
__device__ __attribute__((aligned(16))) float g_zero_f32[4];
__device__ __attribute__((aligned(16))) uint8_t g_zero_u8[16];

// First entry of share w when n entries are split over G workgroups. Here w <= 1024
// workgroups and n <= 2^18 rows (SFN_MAX_F), so w n < 2^28 and 32-bit unsigned
// arithmetic is exact; a 64-bit division would cost over a hundred instructions in every
// workgroup's prologue, ahead of its first weight load.
__device__ __forceinline__ int share_begin(int w, int n, int G) {
  return (int)((uint32_t)w * (uint32_t)n / (uint32_t)G);
}

// Words other workgroups read during the same launch: relaxed device-scope atomics,
// which go through to memory past this XCD's L2 (the L2s of the eight XCDs are not
// coherent with each other) without the whole-L2 writeback or invalidation that a
// release or acquire fence would cost.
__device__ __forceinline__ void st_through(SFN_GLOBAL uint32_t* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_through(const SFN_GLOBAL uint32_t* p) {
  return __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Sets *p to v if it holds expect; returns the value found (== expect iff it was set).
__device__ __forceinline__ uint32_t cas_through(SFN_GLOBAL uint32_t* p, uint32_t expect, uint32_t v) {
  __hip_atomic_compare_exchange_strong((uint32_t*)p, &expect, v, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return expect;
}

template <int WT, int BMAX, int CPT, int TPR, int R>
struct Shape {
  using CK = Chunk<WT>;
  static constexpr int RPG = kNT / TPR;  // rows processed side by side
  static constexpr int RG = RPG * R;     // rows of an up/down step (and of half a gate step)
  static constexpr int RS = 2 * RG;      // rows of a gate step
  static constexpr int VG = 2 * R * BMAX;
  static constexpr int VU = R * BMAX;
  static constexpr int WPR = TPR / 64;  // waves per row
  static constexpr int KV = CK::kVals;
  static_assert(RS <= 64, "one lane of wave 0 per row of a gate step");

  // Token chunks of this thread, zero beyond the row or the batch.
  __device__ __forceinline__ static void load_x(const DevArgs& a, int cl, uint4 (&xr)[BMAX][CPT]) {
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int ch = cl + TPR * c;
        xr[b][c] = (b < a.nb && ch < a.nch) ? ld16(a.x + (size_t)b * a.row_bytes + (size_t)ch * 16)
                                            : make_uint4(0, 0, 0, 0);
      }
  }

  // Wave totals of NV values per thread into wpart[wave][0..NV): the values are cut into
  // power-of-two blocks of at most 16 (e.g. 24 = 16 + 8), each transposed and summed
  // across the wave, then written by one lane per value.
  template <int NV, int OFF, int BLK>
  __device__ __forceinline__ static void reduce_block(float (*wpart)[NV], const float (&s)[NV]) {
    constexpr int LOGB = (BLK >= 16) ? 4 : (BLK >= 8) ? 3 : (BLK >= 4) ? 2 : (BLK >= 2) ? 1 : 0;
    constexpr int SH = 6 - LOGB;
    const int lane = threadIdx.x & 63;
    float t[BLK];
#pragma unroll
    for (int i = 0; i < BLK; ++i) t[i] = s[OFF + i];
    wave_transpose_sum<BLK>(t);
    if ((lane & ((1 << SH) - 1)) == 0) wpart[threadIdx.x >> 6][OFF + (lane >> SH)] = t[0];
  }

  template <int NV, int OFF = 0>
  __device__ __forceinline__ static void reduce_to_lds(float (*wpart)[NV], const float (&s)[NV]) {
    constexpr int REM = NV - OFF;
    if constexpr (REM > 0) {
      constexpr int BLK = REM >= 16 ? 16 : REM >= 8 ? 8 : REM >= 4 ? 4 : REM >= 2 ? 2 : 1;
      reduce_block<NV, OFF, BLK>(wpart, s);
      reduce_to_lds<NV, OFF + BLK>(wpart, s);
    }
  }

  // Sum of the WPR wave partials of row-lane rlj, value v.
  template <int NV>
  __device__ __forceinline__ static float wave_partial_sum(const float (*wpart)[NV], int rlj, int v) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < WPR; ++i) acc += wpart[rlj * WPR + i][v];
    return acc;
  }
};

// ------------------------------------------------------------------ predictor phase
// Predict mode: the SVD predictor on one tile's own rows ("SVD Contextual Sparsity
// Predictors for Fast LLM Inference", Figures 1 and 3): p_i = L_i z + b_i for rows
// [r0, r0 + nt) (z = Q x, computed by the launch before), candidates {i : p_i > tau_i},
// compacted in ascending order into rowid[0, n). The tile then processes its own
// candidates, so no candidate list crosses workgroups and no scan over tiles is needed.
// Each row of L (r bf16 = r/8 chunks) is read by 2^lt lanes of one wave, at most two
// chunks each (r <= 1024); 8 passes of rows are in flight per lane.
struct PredSmem {
  float p[kTMax];
  int wcnt[kNW];
  int n;
};

__device__ __forceinline__ float dot_l_z(const uint4& w, const float (&z)[8], float acc) {
  const uint32_t p4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc = fmaf(__uint_as_float(p4[j] << 16), z[2 * j], acc);
    acc = fmaf(__uint_as_float(p4[j] & 0xffff0000u), z[2 * j + 1], acc);
  }
  return acc;
}

__device__ void predict_tile(const DevArgs& a, PredSmem& ps, int r0, int nt, int* rowid) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // bias and threshold of row tid, read first (the compare below runs on thread tid)
  float pb = 0.f, pt = 0.f;
  if (tid < nt) {
    pb = a.pb ? a.pb[r0 + tid] : 0.f;
    pt = a.ptau[r0 + tid];
  }
  const int nchr = a.pr >> 3;
  const int lt = nchr <= 8 ? 3 : nchr <= 16 ? 4 : nchr <= 32 ? 5 : 6;  // log2 lanes per row
  const int tpr = 1 << lt;
  const int rp = kNT >> lt;  // rows per pass
  const int rl = tid >> lt, cl = tid & (tpr - 1);
  float zc[2][8];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch = cl + tpr * c;
#pragma unroll
    for (int j = 0; j < 8; ++j) zc[c][j] = ch < nchr ? a.pz[ch * 8 + j] : 0.f;
  }
  const size_t rb = (size_t)a.pr * 2;
  const int npass = (nt + rp - 1) / rp;
  for (int p0 = 0; p0 < npass; p0 += 8) {
    uint4 wv[8][2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = (p0 + u) * rp + rl;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ch = cl + tpr * c;
        wv[u][c] = (row < nt && ch < nchr) ? ldg16(a.pl + (size_t)(r0 + row) * rb + (size_t)ch * 16)
                                           : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float acc = dot_l_z(wv[u][1], zc[1], dot_l_z(wv[u][0], zc[0], 0.f));
      acc = lt == 3 ? group_sum<8>(acc) : lt == 4 ? group_sum<16>(acc) : lt == 5 ? group_sum<32>(acc) : group_sum<64>(acc);
      const int row = (p0 + u) * rp + rl;
      if (cl == 0 && row < nt) ps.p[row] = acc;
    }
  }
  __syncthreads();
  // compare and compact, one wave per 64 rows (nt <= kTMax = 4 waves)
  const int nw = (nt + 63) >> 6;
  bool on = false;
  unsigned long long bal = 0ull;
  if (wave < nw) {
    on = tid < nt && ps.p[tid] + pb > pt;
    bal = __ballot(on);
    if (lane == 0) ps.wcnt[wave] = (int)__popcll(bal);
  }
  __syncthreads();
  if (on) {
    int base = 0;
    for (int w2 = 0; w2 < wave; ++w2) base += ps.wcnt[w2];
    rowid[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0))] =
        r0 + tid;
  }
  if (tid == 0) {
    int n = 0;
    for (int w2 = 0; w2 < nw; ++w2) n += ps.wcnt[w2];
    ps.n = n;
  }
  __syncthreads();
}

// ------------------------------------------------------------------------ gate kernel
template <int WT, int BMAX, int CPT, int TPR, int R>
struct GateKernel {
  using S = Shape<WT, BMAX, CPT, TPR, R>;
  using CK = typename S::CK;
  static constexpr int RPG = S::RPG, RG = S::RG, RS = S::RS, VG = S::VG;

  struct Smem {
    int rowid[kTMax];  // candidate and predict modes: global row of each local row
    float wpart[kNW][VG];
    int qlen;
    int cnt[BMAX];
    PredSmem ps;
  };

  // Loads of one gate step: w0 = rows [base, base+RG), w1 = rows [base+RG, base+RS) of Wg,
  // or (step none) both from x, L1-resident, results unused. Rows past the end are
  // clamped to a valid row and masked later. Each lane also fetches the bias and mask
  // bytes of row (lane % RS).
  __device__ __forceinline__ static void issue(const DevArgs& a, const Smem& sm, const StepDesc& sd, int r0,
                                               int nrows, bool cand_mode, int rl, int cl, int lane,
                                               uint4 (&w0)[R][CPT], uint4 (&w1)[R][CPT], float& bias,
                                               uint32_t (&mraw)[BMAX]) {
    const bool gate = sd.kind == STEP_GATE;
    const SFN_GLOBAL char* p = gate ? a.wg : a.x;
    const size_t rb = gate ? (size_t)a.row_bytes : 0;
    const int lrmax = nrows > 0 ? nrows - 1 : 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int j = rl + RPG * k;
      const int lr0 = min(sd.base + j, lrmax), lr1 = min(sd.base + RG + j, lrmax);
      const int g0 = cand_mode ? sm.rowid[lr0] : r0 + lr0;
      const int g1 = cand_mode ? sm.rowid[lr1] : r0 + lr1;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        int ch = cl + TPR * c;
        ch = ch < a.nch ? ch : 0;
        w0[k][c] = ldg16(p + (size_t)g0 * rb + (size_t)ch * 16);
        w1[k][c] = ldg16(p + (size_t)g1 * rb + (size_t)ch * 16);
      }
    }
    // an empty share (no candidates) has no rowid entries: fetch row 0's bytes instead of
    // indexing with whatever the LDS holds
    const int lb = min(sd.base + (lane % RS), lrmax);
    const int gb = nrows == 0 ? 0 : cand_mode ? sm.rowid[lb] : r0 + lb;
    bias = a.bias ? a.bias[gb] : gp(g_zero_f32)[0];
    // raw bytes: tested only when the step is processed, so no wait is forced here
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      const int bb = b < a.nb ? b : 0;
      mraw[b] = a.mask_in ? a.mask_in[(size_t)bb * a.f + gb] : gp(g_zero_u8)[b];
    }
  }

  // rec(slot, row, activations, bits) is called by wave 0 for every selected row, slot
  // being its position in the tile's slice; returns the tile's selected-row count and
  // where its slice of the lists starts. LOCAL: the workgroup streams the up/down rows of
  // its own list, kept in LDS by rec, so the global list is not written.
  template <bool LOCAL, class Rec>
  __device__ static int2 run(const DecodeArgs& args, Rec&& rec) {
    const DevArgs a = dev_args(args);
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = tid / TPR, cl = tid % TPR;
    const int w = blockIdx.x;
    const bool pred_mode = a.pl != nullptr;
    const bool cand_mode = a.cand != nullptr || pred_mode;
    const bool want_idx = a.active_idx != nullptr || a.n_active != nullptr;
    const int nb = a.nb;

    int r0, nrows;
    if (pred_mode) {
      // the tile's own rows; its candidates become the local rows (the slices of the
      // lists stay at the tile's first row)
      r0 = share_begin(w, a.f, a.G);
      predict_tile(a, sm.ps, r0, share_begin(w + 1, a.f, a.G) - r0, sm.rowid);
      nrows = sm.ps.n;
    } else if (cand_mode) {
      const int n = min(max(*a.n_cand, 0), a.f);  // a count beyond f cannot be a valid list
      r0 = share_begin(w, n, a.G);
      nrows = share_begin(w + 1, n, a.G) - r0;
      for (int i = tid; i < nrows; i += kNT) sm.rowid[i] = min(max(a.cand[r0 + i], 0), a.f - 1);  // in bounds
    } else {
      r0 = share_begin(w, a.f, a.G);
      nrows = share_begin(w + 1, a.f, a.G) - r0;
    }
    if (tid == 0) sm.qlen = 0;
    if (tid < BMAX) sm.cnt[tid] = 0;
    uint4 xr[BMAX][CPT];
    S::load_x(a, cl, xr);
    const float thr = a.t ? *a.t : 0.0f;
    __syncthreads();

    auto process = [&](const StepDesc& sd, const uint4 (&w0)[R][CPT], const uint4 (&w1)[R][CPT], float bias,
                       const uint32_t (&mraw)[BMAX]) {
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
      S::template reduce_to_lds<VG>(sm.wpart, s);
      __syncthreads();
      if (wave == 0) {
        // lane j finalizes row j of the step: half hh = j / RG, row-lane jj % RPG, slot k
        const int j = lane;
        const int hh = j / RG, jj = j % RG;
        const int rlj = jj % RPG, k = jj / RPG;
        const bool ok = j < sd.n;
        const int lr = sd.base + j;
        uint32_t bits = 0;
        int grow = 0;
        float av[BMAX];
#pragma unroll
        for (int b = 0; b < BMAX; ++b) av[b] = 0.f;
        if (ok) {
          grow = cand_mode ? sm.rowid[lr] : r0 + lr;
#pragma unroll
          for (int b = 0; b < BMAX; ++b) {
            if (b < nb) {
              const float g = S::template wave_partial_sum<VG>(sm.wpart, rlj, (hh * R + k) * BMAX + b) + bias;
              av[b] = (a.act == 0) ? silu_f(g) : fmaxf(g, 0.f);
              const bool on = a.mask_in ? mraw[b] != 0u : fabsf(av[b]) > thr;
              bits |= (uint32_t)on << b;
            }
          }
        }
        const unsigned long long ub = __ballot(bits != 0);
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(ub >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ub, 0));
        const int q0 = sm.qlen;
        if (bits != 0) {
          if constexpr (!LOCAL) {
            const int o = r0 + q0 + pos;  // this tile's slice of the global lists
            a.sel_idx[o] = grow;
            a.sel_bits[o] = (uint8_t)bits;
#pragma unroll
            for (int b = 0; b < BMAX; ++b)
              if (b < nb) a.sel_a[(size_t)b * a.f + o] = av[b];
          }
          rec(q0 + pos, grow, av, bits);
        }
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
    };

    const int ngate = (nrows + RS - 1) / RS;
    uint4 a0[R][CPT], a1[R][CPT], b0[R][CPT], b1[R][CPT];
    float abias, bbias;
    uint32_t amask[BMAX], bmask[BMAX];
    auto step = [&](int s) -> StepDesc {
      StepDesc sd{STEP_NONE, 0, 0};
      if (s < ngate) {
        sd.kind = STEP_GATE;
        sd.base = s * RS;
        sd.n = min(RS, nrows - sd.base);
      }
      return sd;
    };
    // Two steps per iteration and no exit inside the body: the loop then has a single
    // path back to its head, along which exactly the loads of buffer a are in flight, so
    // the compiler's wait counts let buffer b's loads go out while a's are still on their
    // way. (An exit after the first half gave the head a second incoming path with b's
    // loads in flight, and the head then waited for the older loads before issuing: one
    // step in flight instead of two for much of every iteration.) An even step count ends
    // with one issue of an empty step (loads of x, unused); an odd one processes its last
    // step after the loop.
    StepDesc sa = step(0);
    issue(a, sm, sa, r0, nrows, cand_mode, rl, cl, lane, a0, a1, abias, amask);
    int s = 0;
    for (; s + 1 < ngate; s += 2) {
      const StepDesc sb = step(s + 1);
      issue(a, sm, sb, r0, nrows, cand_mode, rl, cl, lane, b0, b1, bbias, bmask);
      process(sa, a0, a1, abias, amask);
      sa = step(s + 2);
      issue(a, sm, sa, r0, nrows, cand_mode, rl, cl, lane, a0, a1, abias, amask);
      process(sb, b0, b1, bbias, bmask);
    }
    if (s < ngate) process(sa, a0, a1, abias, amask);
    if (tid < kCnt) {
      int v = 0;
      if (tid == 0) v = sm.qlen;
      else if (tid - 1 < BMAX) v = sm.cnt[tid - 1];
      a.tile_cnt[w * kCnt + tid] = v;
    }
    return make_int2(sm.qlen, r0);
  }
};

// ------------------------------------------------------------- matrix-core gate kernel
// Gate on matrix cores for bf16 weights (one to four tokens, no candidate list): the
// same outputs as the gate kernel (tile slices of the union rows, their activations and
// per-token bits, per-token index slices, counts), for tiles of at most 16 rows
// (G = ceil(f / 16)). v_mfma_f32_16x16x32_bf16 takes the tokens as M (rows beyond the
// batch are zero) and the tile's rows as N, so the sum over d happens inside the matrix
// cores and no cross-lane reduction is needed, whatever the batch. A wave-wide load of B
// fragments would touch 16 rows at 64 bytes each, so the rows go through LDS: each stage
// loads 1 KB pieces of the 16 rows, one row per wave instruction, with the next two
// stages in flight while the matrix cores work on the current one; the four waves split
// each stage's K range.
constexpr int kMKT = 512;          // K elements per stage (1 KB of a bf16 row)
constexpr int kMLds = kMKT + 8;    // padded LDS row (elements)
constexpr int kMRows = 16;         // rows per tile

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
__device__ __forceinline__ bf16x8_t as_frag(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

template <int BMAX>
__global__ __launch_bounds__(256) void decode_gate_mfma_kernel(DecodeArgs args) {
  const DevArgs a = dev_args(args);
  __shared__ __attribute__((aligned(16))) uint16_t s_w[kMRows][kMLds];
  __shared__ f32x4_t s_part[4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int w = blockIdx.x;
  const int r0 = share_begin(w, a.f, a.G);
  const int nt = share_begin(w + 1, a.f, a.G) - r0;  // <= 16 rows
  const int col = lane & 15, q = lane >> 4;
  const bool tok_ok = col < a.nb;  // A side: lane's token is col
  const size_t rb = (size_t)a.row_bytes;
  const int d = a.d;
  const int nst = (d + kMKT - 1) / kMKT;
  // loader: round i (0..3) of wave v reads row slot 4 i + v, pieces h (0..kMKT/512-1)
  // of the stage's K range, bytes [16 lane, 16 lane + 16) of each 1 KB piece. Two
  // stages are in flight: the loads of stage st + 2 go out once stage st is in LDS.
  constexpr int NH = kMKT / 512;  // 1 KB pieces per row and stage
  constexpr int NT = kMKT / 128;  // K steps of 32 per wave and stage
  uint4 wa[4 * NH], wb[4 * NH], xa[NT], xb[NT];
  auto load = [&](int st, uint4 (&wr)[4 * NH], uint4 (&xr)[NT]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int slot = 4 * i + wave;
      const bool rok = slot < nt;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int k = st * kMKT + 512 * h + lane * 8;
        const bool ok = rok && k < d;
        wr[NH * i + h] = ok ? ldg16(a.wg + (size_t)(r0 + slot) * rb + (size_t)k * 2) : make_uint4(0, 0, 0, 0);
      }
    }
    // A fragments of this wave's quarter: token col, K = st kMKT + (kMKT/4) wave + 32 t + 8 q
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int kx = st * kMKT + (kMKT / 4) * wave + 32 * t + 8 * q;
      const bool ok = tok_ok && kx < d;
      xr[t] = ok ? ld16(a.x + (size_t)col * rb + (size_t)kx * 2) : make_uint4(0, 0, 0, 0);
    }
  };
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  auto stage = [&](int st, uint4 (&wr)[4 * NH], uint4 (&xr)[NT]) {
    __syncthreads();  // the previous stage's fragments have been read
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        *reinterpret_cast<uint4*>(&s_w[4 * i + wave][512 * h + lane * 8]) = wr[NH * i + h];
    uint4 xc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) xc[t] = xr[t];
    __syncthreads();
    if (st + 2 < nst) load(st + 2, wr, xr);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int kk = (kMKT / 4) * wave + 32 * t + 8 * q;
      const uint4 bg = *reinterpret_cast<const uint4*>(&s_w[col][kk]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_frag(xc[t]), as_frag(bg), acc, 0, 0, 0);
    }
  };
  load(0, wa, xa);
  if (nst > 1) load(1, wb, xb);
  for (int st = 0; st < nst; st += 2) {
    stage(st, wa, xa);
    if (st + 1 < nst) stage(st + 1, wb, xb);
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    // lane (q = 0) holds tokens 0..3 (rows of C) for row r0 + col (column of C)
    f32x4_t g = s_part[0][lane];
#pragma unroll
    for (int v = 1; v < 4; ++v) g += s_part[v][lane];
    const bool ok = q == 0 && col < nt;
    const bool want_idx = a.active_idx != nullptr || a.n_active != nullptr;
    const int row = r0 + (ok ? col : 0);
    const float bias = a.bias ? a.bias[row] : 0.f;
    const float thr = a.t ? *a.t : 0.0f;
    uint32_t bits = 0;
    float av[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      av[b] = 0.f;
      if (ok && b < a.nb) {
        const float gv = g[b] + bias;
        av[b] = (a.act == 0) ? silu_f(gv) : fmaxf(gv, 0.f);
        const bool on = a.mask_in ? a.mask_in[(size_t)b * a.f + row] != 0 : fabsf(av[b]) > thr;
        bits |= (uint32_t)on << b;
      }
    }
    const unsigned long long ub = __ballot(bits != 0);
    const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(ub >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ub, 0));
    if (bits != 0) {
      const int o = r0 + pos;  // this tile's slice of the global lists
      a.sel_idx[o] = row;
      a.sel_bits[o] = (uint8_t)bits;
#pragma unroll
      for (int b = 0; b < BMAX; ++b)
        if (b < a.nb) a.sel_a[(size_t)b * a.f + o] = av[b];
    }
    int cnt[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      const bool on = (bits >> b) & 1u;
      const unsigned long long bb = __ballot(on);
      cnt[b] = (int)__popcll(bb);
      if (on && want_idx) {
        const int pb = __builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0));
        a.tile_idx[(size_t)b * a.f + r0 + pb] = row;
      }
    }
    if (lane < kCnt) {
      int v = 0;
      if (lane == 0) v = (int)__popcll(ub);
#pragma unroll
      for (int b = 0; b < BMAX; ++b)
        if (lane == 1 + b && b < a.nb) v = cnt[b];
      a.tile_cnt[w * kCnt + lane] = v;
    }
  }
}

// --------------------------------------------------------------------- up/down kernel
template <int WT, int BMAX, int CPT, int TPR, int R>
struct UpDownKernel {
  using S = Shape<WT, BMAX, CPT, TPR, R>;
  using CK = typename S::CK;
  static constexpr int RPG = S::RPG, RG = S::RG, VU = S::VU, KV = S::KV;

  struct Smem {
    int qslot[kTMax];         // list slot of each entry of this workgroup's share
    int qrow[kTMax];          // global row of each entry of this workgroup's share
    float qa[kTMax][BMAX];    // activations
    uint8_t qbits[kTMax];     // per-token mask bits
    float wpart[kNW][VU];
    float h[64][BMAX];
    int wsum[kNW];
    // list slots [o_lo, o_hi) around the share, loaded with the tile counts
    int srow[kNT];
    float sa[kNT][BMAX];
    uint8_t sbits[kNT];
  };

  // Loads of one up/down step: w0 = Wu rows, w1 = Dt rows of share entries [base,
  // base+n), or (step none) both from x, L1-resident, results unused.
  __device__ __forceinline__ static void issue(const DevArgs& a, const Smem& sm, const StepDesc& sd, int nq, int rl,
                                               int cl, uint4 (&w0)[R][CPT], uint4 (&w1)[R][CPT]) {
    const bool upd = sd.kind == STEP_UPDOWN;
    const SFN_GLOBAL char* p0 = upd ? a.wu : a.x;
    const SFN_GLOBAL char* p1 = upd ? a.wd : a.x;
    const size_t rb = upd ? (size_t)a.row_bytes : 0;
    const int jmax = nq > 0 ? nq - 1 : 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int j = min(sd.base + rl + RPG * k, jmax);
      const int g = sm.qrow[j];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        int ch = cl + TPR * c;
        ch = ch < a.nch ? ch : 0;
        w0[k][c] = ldg16(p0 + (size_t)g * rb + (size_t)ch * 16);
        w1[k][c] = ldg16(p1 + (size_t)g * rb + (size_t)ch * 16);
      }
    }
  }

  __device__ static void run(const DecodeArgs& args) {
    const DevArgs a = dev_args(args);
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w = blockIdx.x;
    const bool cand_mode = a.cand != nullptr;
    const bool want_y = a.y != nullptr;
    const int nb = a.nb;
    const int n_total = cand_mode ? min(max(*a.n_cand, 0), a.f) : a.f;  // rows the gate tiles cover

    if (want_y) {
      // ---- this workgroup's equal share [s0, s0 + nq) of the concatenated active lists.
      // Each thread owns two consecutive tiles; a scan of the tile counts tells it where
      // their lists sit in the concatenation and the total n, so it can mark, for each
      // share entry inside its tiles, which list slot holds it. Then every thread copies
      // one entry.
      // The list slots of the tiles around the share's expected place (two tiles either side
      // of a proportional split; at most one slot per thread) are loaded together with the
      // counts, so the gather below almost never needs a second round trip (the cumulative
      // counts stray from the proportional split by about one tile); an entry outside the
      // window is fetched from memory.
      int n, s0, nq;
      const int tl = max(0, (int)((uint32_t)w * (uint32_t)a.G / (uint32_t)a.Gu) - 2);
      const int th = min(a.G, (int)(((uint32_t)(w + 1) * (uint32_t)a.G + (uint32_t)a.Gu - 1) / (uint32_t)a.Gu) + 2);
      const int o_lo = share_begin(tl, n_total, a.G);
      const int o_hi = min(share_begin(th, n_total, a.G), o_lo + kNT);
      {
        const int i0 = 2 * tid;  // G <= 1024 = 2 * kNT
        const int c0 = i0 < a.G ? a.tile_cnt[i0 * kCnt] : 0;
        const int c1 = i0 + 1 < a.G ? a.tile_cnt[(i0 + 1) * kCnt] : 0;
        if (tid < o_hi - o_lo) {
          const int o = o_lo + tid;
          sm.srow[tid] = a.sel_idx[o];
          sm.sbits[tid] = a.sel_bits[o];
#pragma unroll
          for (int b = 0; b < BMAX; ++b) sm.sa[tid][b] = b < nb ? a.sel_a[(size_t)b * a.f + o] : 0.f;
        }
        const int v = wave_incl_scan(c0 + c1);  // inclusive scan over the wave (DPP)
        if (lane == 63) sm.wsum[wave] = v;
        __syncthreads();
        int base = 0;
        n = 0;
#pragma unroll
        for (int i = 0; i < kNW; ++i) {
          const int ws = sm.wsum[i];
          base += i < wave ? ws : 0;
          n += ws;
        }
        s0 = share_begin(w, n, a.Gu);
        nq = share_begin(w + 1, n, a.Gu) - s0;
        int p0 = base + v - c0 - c1;  // first position of tile i0's list
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int cnt = t ? c1 : c0;
          const int lo = max(p0, s0), hi = min(p0 + cnt, s0 + nq);
          const int ob = share_begin(i0 + t, n_total, a.G) - p0;  // list slot = ob + position
          for (int pos = lo; pos < hi; ++pos) sm.qslot[pos - s0] = ob + pos;
          p0 += cnt;
        }
      }
      __syncthreads();
      for (int j = tid; j < nq; j += kNT) {
        const int o = sm.qslot[j];
        if (o >= o_lo && o < o_hi) {
          const int k = o - o_lo;
          sm.qrow[j] = sm.srow[k];
          sm.qbits[j] = sm.sbits[k];
#pragma unroll
          for (int b = 0; b < BMAX; ++b) sm.qa[j][b] = sm.sa[k][b];
        } else {
          sm.qrow[j] = a.sel_idx[o];
          sm.qbits[j] = a.sel_bits[o];
#pragma unroll
          for (int b = 0; b < BMAX; ++b) sm.qa[j][b] = b < nb ? a.sel_a[(size_t)b * a.f + o] : 0.f;
        }
      }
      NoBalance nobal;
      stream(a, sm, nq, w, nobal);
    }
  }

  // Up and down rows of list entries (rows, activations and bits in sm), then the
  // workgroup's partial of y in partial rows w RPG .. w RPG + RPG - 1. Without a balancer
  // the entries are [0, nq). With one, the first three steps take entries
  // [0, min(nq, 3 RG)); after the second step is processed the balancer settles the list
  // (the tail of a long one given away, others' entries appended to a short one) and
  // the steps continue from there.
  struct NoBalance {
    __device__ bool active() const { return false; }
    __device__ bool poisoned() const { return false; }
    __device__ void load_counts(const DevArgs&) {}
    __device__ int decide(const DevArgs&, Smem&, int covered) { return covered; }
  };
  template <class Bal>
  __device__ static void stream(const DevArgs& a, Smem& sm, int nq, int w, Bal& bal) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = tid / TPR, cl = tid % TPR;
    const int nb = a.nb;
    float acc[BMAX][CPT][KV];
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
#pragma unroll
      for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int v = 0; v < KV; ++v) acc[b][c][v] = 0.f;
    {
      uint4 xr[BMAX][CPT];
      S::load_x(a, cl, xr);
      __syncthreads();

      auto process = [&](const StepDesc& sd, const uint4 (&w0)[R][CPT], const uint4 (&w1)[R][CPT]) {
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
        S::template reduce_to_lds<VU>(sm.wpart, s);
        __syncthreads();
        if (wave == 0 && lane < sd.n) {
          const int j = sd.base + lane;
          const uint32_t bits = sm.qbits[j];
          const int rlj = lane % RPG, k = lane / RPG;
#pragma unroll
          for (int b = 0; b < BMAX; ++b) {
            const float u = S::template wave_partial_sum<VU>(sm.wpart, rlj, k * BMAX + b);
            sm.h[lane][b] = ((bits >> b) & 1u) ? sm.qa[j][b] * u : 0.f;
          }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < R; ++k) {
          const int jj = rl + RPG * k;
          if (jj < sd.n) {
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
              const float hv = sm.h[jj][b];
#pragma unroll
              for (int c = 0; c < CPT; ++c) CK::axpy(hv, w1[k][c], acc[b][c]);
            }
          }
        }
      };

      // lim: entries the steps may take; steps 0 to 2 cover [0, covered), later steps run
      // on from there
      constexpr int kPre = 3;  // steps issued before the balancer decides
      const bool balanced = bal.active();
      int lim = balanced ? min(nq, kPre * RG) : nq;
      const int covered = min(lim, kPre * RG);
      int nstep = balanced ? kPre : (nq + RG - 1) / RG;
      uint4 a0[R][CPT], a1[R][CPT], b0[R][CPT], b1[R][CPT];
      auto step = [&](int s) -> StepDesc {
        StepDesc sd{STEP_NONE, 0, 0};
        const int base = s < kPre ? s * RG : covered + (s - kPre) * RG;
        if (s < nstep && base < lim) {
          sd.kind = STEP_UPDOWN;
          sd.base = base;
          sd.n = min(RG, lim - base);
        }
        return sd;
      };
      // (the loop shape of the gate: no exit inside the body; see GateKernel::run)
      StepDesc sa = step(0);
      issue(a, sm, sa, lim, rl, cl, a0, a1);
      int s = 0;
      for (; s + 1 < nstep; s += 2) {
        const StepDesc sb = step(s + 1);
        issue(a, sm, sb, lim, rl, cl, b0, b1);
        process(sa, a0, a1);
        if (balanced && s == 0) bal.load_counts(a);
        sa = step(s + 2);
        issue(a, sm, sa, lim, rl, cl, a0, a1);
        process(sb, b0, b1);
        if (balanced && s == 0) {
          lim = bal.decide(a, sm, covered);
          nstep = kPre + (max(lim - covered, 0) + RG - 1) / RG;
        }
      }
      if (s < nstep) process(sa, a0, a1);

      // ---- partial of y (read by the reduce kernel after this launch completes)
      if (bal.poisoned()) {
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
#pragma unroll
          for (int c = 0; c < CPT; ++c)
#pragma unroll
            for (int v = 0; v < KV; ++v) acc[b][c][v] = __builtin_nanf("");
      }
      // one partial row per workgroup and token: with RPG rows side by side the row-lanes'
      // sums are added in LDS first, row-lane 0 + 1 + ... in order, so the reduce kernel
      // reads RPG times fewer rows (at d 256 in fp32, 86 partial rows instead of 688)
      SFN_GLOBAL float* prow = a.part + (size_t)w * nb * a.d;
      if constexpr (RPG > 1) {
        __shared__ float comb[RPG][TPR * CPT * KV];  // each row-lane's columns
        for (int b = 0; b < nb; ++b) {
          __syncthreads();  // the previous token's sums have been read
#pragma unroll
          for (int c = 0; c < CPT; ++c) {
            const int ch = cl + TPR * c;
            if (ch < a.nch) {
#pragma unroll
              for (int v = 0; v < KV; ++v) comb[rl][ch * KV + v] = acc[b][c][v];
            }
          }
          __syncthreads();
          for (int e = tid; e < a.d; e += kNT) {
            float sum = comb[0][e];
#pragma unroll
            for (int r = 1; r < RPG; ++r) sum += comb[r][e];
            prow[(size_t)b * a.d + e] = sum;
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
          if (b < nb) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
              const int ch = cl + TPR * c;
              if (ch < a.nch) {
                SFN_GLOBAL float* dst = prow + (size_t)b * a.d + (size_t)ch * KV;
#pragma unroll
                for (int v = 0; v < KV; v += 4)
                  *reinterpret_cast<SFN_GLOBAL f32x4_t*>(dst + v) =
                      f32x4_t{acc[b][c][v], acc[b][c][v + 1], acc[b][c][v + 2], acc[b][c][v + 3]};
              }
            }
          }
        }
      }
    }
  }
};

// ------------------------------------------------------------ parallel-pipeline kernel
// Candidate rows in one pass ("SVD Contextual Sparsity Predictors for Fast LLM
// Inference", Table 2: the parallel pipeline): for the rows of a candidate list the gate,
// up and down rows are read in the same step, and y = sum over the candidates of
// act(g_i + b_i) u_i Dt[i, :]. Each of the G workgroups takes an equal share of the
// list; one token. With ReLU the result is that of the sequential pipeline (the gate
// zeroes the rest); it reads all three rows of every candidate but needs no gate pass.
template <int WT, int CPT, int TPR, int R>
struct ParKernel {
  using S = Shape<WT, 1, CPT, TPR, R>;
  using CK = typename S::CK;
  static constexpr int RPG = S::RPG, RG = S::RG, KV = S::KV;
  static constexpr int V2 = 2 * R;  // gate and up of the step's rows
  static_assert(RG <= 64, "one lane of wave 0 per row of a step");

  struct Smem {
    int qrow[kTMax];
    float qb[kTMax];
    float wpart[kNW][V2];
    float h[64];
    PredSmem ps;
  };

  // Loads of one step: Wg, Wu and Dt rows of share entries [base, base + n), or (step
  // none) all from x, L1-resident, results unused.
  __device__ __forceinline__ static void issue(const DevArgs& a, const Smem& sm, const StepDesc& sd, int nq, int rl,
                                               int cl, uint4 (&wg)[R][CPT], uint4 (&wu)[R][CPT],
                                               uint4 (&wd)[R][CPT]) {
    const bool live = sd.kind == STEP_UPDOWN;
    const SFN_GLOBAL char* pg = live ? a.wg : a.x;
    const SFN_GLOBAL char* pu = live ? a.wu : a.x;
    const SFN_GLOBAL char* pd = live ? a.wd : a.x;
    const size_t rb = live ? (size_t)a.row_bytes : 0;
    const int jmax = nq > 0 ? nq - 1 : 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int j = min(sd.base + rl + RPG * k, jmax);
      const size_t ro = (size_t)sm.qrow[j] * rb;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        int ch = cl + TPR * c;
        ch = ch < a.nch ? ch : 0;
        wg[k][c] = ldg16(pg + ro + (size_t)ch * 16);
        wu[k][c] = ldg16(pu + ro + (size_t)ch * 16);
        wd[k][c] = ldg16(pd + ro + (size_t)ch * 16);
      }
    }
  }

  __device__ static void run(const DecodeArgs& args) {
    const DevArgs a = dev_args(args);
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rl = tid / TPR, cl = tid % TPR;
    const int w = blockIdx.x;
    int nq;
    if (a.pl) {
      // predict mode: the candidates among the tile's own rows, also written to the
      // tile's slice of the index lists (for the reduce kernel to assemble)
      const int r0 = share_begin(w, a.f, a.G);
      predict_tile(a, sm.ps, r0, share_begin(w + 1, a.f, a.G) - r0, sm.qrow);
      nq = sm.ps.n;
      for (int j = tid; j < nq; j += kNT) {
        const int row = sm.qrow[j];
        sm.qb[j] = a.bias ? a.bias[row] : 0.f;
        a.tile_idx[r0 + j] = row;
      }
      if (tid < kCnt) a.tile_cnt[w * kCnt + tid] = tid < 2 ? nq : 0;
    } else {
      const int n = min(max(*a.n_cand, 0), a.f);  // a count beyond f cannot be a valid list
      const int s0 = share_begin(w, n, a.G);
      nq = share_begin(w + 1, n, a.G) - s0;
      for (int j = tid; j < nq; j += kNT) {
        const int row = min(max(a.cand[s0 + j], 0), a.f - 1);  // in bounds
        sm.qrow[j] = row;
        sm.qb[j] = a.bias ? a.bias[row] : 0.f;
      }
    }
    float acc[CPT][KV];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int v = 0; v < KV; ++v) acc[c][v] = 0.f;
    uint4 xr[1][CPT];
    S::load_x(a, cl, xr);
    __syncthreads();

    auto process = [&](const StepDesc& sd, const uint4 (&wg)[R][CPT], const uint4 (&wu)[R][CPT],
                       const uint4 (&wd)[R][CPT]) {
      float s[V2];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        float dg = 0.f, du = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          dg = CK::dot(wg[k][c], xr[0][c], dg);
          du = CK::dot(wu[k][c], xr[0][c], du);
        }
        s[k] = dg;
        s[R + k] = du;
      }
      S::template reduce_to_lds<V2>(sm.wpart, s);
      __syncthreads();
      if (wave == 0 && lane < sd.n) {
        const int j = sd.base + lane;
        const int rlj = lane % RPG, k = lane / RPG;
        const float g = S::template wave_partial_sum<V2>(sm.wpart, rlj, k) + sm.qb[j];
        const float u = S::template wave_partial_sum<V2>(sm.wpart, rlj, R + k);
        sm.h[lane] = (a.act == 0 ? silu_f(g) : fmaxf(g, 0.f)) * u;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int jj = rl + RPG * k;
        if (jj < sd.n) {
          const float hv = sm.h[jj];
#pragma unroll
          for (int c = 0; c < CPT; ++c) CK::axpy(hv, wd[k][c], acc[c]);
        }
      }
    };

    const int nstep = (nq + RG - 1) / RG;
    uint4 ag[R][CPT], au[R][CPT], ad[R][CPT], bg[R][CPT], bu[R][CPT], bd[R][CPT];
    auto step = [&](int st) -> StepDesc {
      StepDesc sd{STEP_NONE, 0, 0};
      if (st < nstep) {
        sd.kind = STEP_UPDOWN;
        sd.base = st * RG;
        sd.n = min(RG, nq - sd.base);
      }
      return sd;
    };
    // (the loop shape of the gate: no exit inside the body; see GateKernel::run)
    StepDesc sa = step(0);
    issue(a, sm, sa, nq, rl, cl, ag, au, ad);
    int st = 0;
    for (; st + 1 < nstep; st += 2) {
      const StepDesc sb = step(st + 1);
      issue(a, sm, sb, nq, rl, cl, bg, bu, bd);
      process(sa, ag, au, ad);
      sa = step(st + 2);
      issue(a, sm, sa, nq, rl, cl, ag, au, ad);
      process(sb, bg, bu, bd);
    }
    if (st < nstep) process(sa, ag, au, ad);

    // ---- partial of y (read by the reduce kernel after this launch completes)
    SFN_GLOBAL float* prow = a.part + (size_t)(w * RPG + rl) * a.d;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int ch = cl + TPR * c;
      if (ch < a.nch) {
        SFN_GLOBAL float* dst = prow + (size_t)ch * KV;
#pragma unroll
        for (int v = 0; v < KV; v += 4)
          *reinterpret_cast<SFN_GLOBAL f32x4_t*>(dst + v) = f32x4_t{acc[c][v], acc[c][v + 1], acc[c][v + 2], acc[c][v + 3]};
      }
    }
  }
};

// ---------------------------------------------------------------------- reduce kernel
// y = sum of the partials of the up/down kernel, in chunks of 32 columns (128 bytes of
// each partial row). Thread (g, q) of 64 groups x 8 column quads sums 16-byte quad q of
// partials g, g + 64, g + 128, ... (four loads in flight per round, rounds past the last
// partial row masked, so a short list of partials costs one round trip, not one per
// row); then eight threads per column add eight groups each, in order, and one thread
// per column adds those eight, so y is deterministic. The partials are read once, with
// non-temporal loads (with the earlier 4-byte loads these were 0.2-0.3 us per one-token
// call and 1.7 us per four-token call faster than plain loads at d 4096). The workgroups
// also assemble the per-token active index lists.
constexpr int kRedCols = 32;

struct ReduceKernel {
  static constexpr int kRT = 512;                // threads
  static constexpr int kQC = kRedCols / 4;       // 16-byte column quads per chunk
  static constexpr int kNG = kRT / kQC;          // partial-row groups (64 = 8 x 8 in the sums below)
  struct Smem {
    float red4[kNG][kRedCols];   // group sums
    float red8[8][kRedCols];     // sums of eight groups
    int pref[kGMax + 1];
    int wsum[kRT / 64];
  };

  // Exclusive prefix of tile_cnt[i * kCnt + off] over the G tiles into sm.pref[0..G].
  __device__ __forceinline__ static void tile_prefix(const DevArgs& a, Smem& sm, int off) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int PER = kGMax / kRT + 1;  // tiles per thread, G <= kGMax
    const int i0 = tid * PER;
    int c[PER];
    int tot = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      c[i] = i0 + i < a.G ? a.tile_cnt[(i0 + i) * kCnt + off] : 0;
      tot += c[i];
    }
    const int v = wave_incl_scan(tot);  // inclusive scan over the wave (DPP)
    if (lane == 63) sm.wsum[wave] = v;
    __syncthreads();
    int run = v - tot;
    for (int i = 0; i < wave; ++i) run += sm.wsum[i];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (i0 + i <= a.G) sm.pref[i0 + i] = run;
      run += c[i];
    }
    __syncthreads();
  }

  __device__ static void run(const DecodeArgs& args, int P) {
    const DevArgs a = dev_args(args);
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ri = blockIdx.x;
    const int nb = a.nb;
    // the balancer's count words and its decision go back to zero for the next call
    if (a.flags) {
      for (int i = ri * kRT + tid; i < a.G; i += gridDim.x * kRT) a.flags[i] = 0u;
      if (ri == 0 && tid == 0) a.flags[kWsBalDecisionWord] = 0u;
    }
    if (a.y && ri < a.n_red) {
      const int L = nb * a.d;  // a multiple of 4: rows are whole 16-byte chunks
      const int nck = (L + kRedCols - 1) / kRedCols;
      const int c0 = share_begin(ri, nck, a.n_red), c1 = share_begin(ri + 1, nck, a.n_red);
      const int qd = tid % kQC, g = tid / kQC;
      for (int ck = c0; ck < c1; ++ck) {
        const int e = ck * kRedCols + 4 * qd;
        const bool ok = e < L;
        const SFN_GLOBAL float* src = a.part + (ok ? e : 0);
        f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
        for (int p = g; p < P; p += 4 * kNG) {
          f32x4_t v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int pu = p + u * kNG;
            v[u] = pu < P ? __builtin_nontemporal_load(reinterpret_cast<const SFN_GLOBAL f32x4_t*>(src + (size_t)pu * L))
                          : f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) sum += v[u];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.red4[g][4 * qd + j] = sum[j];
        __syncthreads();
        if (tid < 8 * kRedCols) {
          const int col = tid % kRedCols, h = tid / kRedCols;
          float t8 = sm.red4[8 * h][col];
#pragma unroll
          for (int j = 1; j < 8; ++j) t8 += sm.red4[8 * h + j][col];
          sm.red8[h][col] = t8;
        }
        __syncthreads();
        if (tid < kRedCols) {
          const int ee = ck * kRedCols + tid;
          float tot = sm.red8[0][tid];
#pragma unroll
          for (int j = 1; j < 8; ++j) tot += sm.red8[j][tid];
          if (ee < L) a.y[ee] = tot;
        }
        __syncthreads();
      }
    }
    // per-token active rows, ascending: the tiles' slices concatenated. Every workgroup
    // forms the prefix over all tile counts and copies the slices of its own share of the
    // tiles (one tile per wave); workgroup 0 writes the counts.
    const int nw = gridDim.x;
    const int t0 = a.active_idx ? share_begin(ri, a.G, nw) : 0;
    const int t1 = a.active_idx ? share_begin(ri + 1, a.G, nw) : 0;
    if (t0 < t1 || (ri == 0 && a.n_active)) {
      const int n_total = a.cand ? min(max(*a.n_cand, 0), a.f) : a.f;
      for (int b = 0; b < nb; ++b) {
        __syncthreads();
        tile_prefix(a, sm, 1 + b);
        for (int tile = t0 + wave; tile < t1; tile += kRT / 64) {
          const int tr0 = share_begin(tile, n_total, a.G);
          const int c = sm.pref[tile + 1] - sm.pref[tile];
          for (int i = lane; i < c; i += 64)
            a.active_idx[(size_t)b * a.f + sm.pref[tile] + i] = a.tile_idx[(size_t)b * a.f + tr0 + i];
        }
        if (ri == 0 && tid == 0 && a.n_active) a.n_active[b] = sm.pref[a.G];
      }
    }
  }
};

template <int WT, int BMAX, int CPT, int TPR, int R>
__global__ __launch_bounds__(kNT) void decode_gate_kernel(DecodeArgs a) {
  GateKernel<WT, BMAX, CPT, TPR, R>::template run<false>(a, [](int, int, const auto&, uint32_t) {});
}

// Balancer of the one-token up/down (flags non-null, G <= kBalMaxTiles, every tile
// resident at once). A tile's share of up/down rows follows its active count, so the
// slowest tile used to finish about 6 us after the median one. Each tile now publishes
// its count (its entries first, through to memory); during its first two up/down steps
// every workgroup reads all counts and derives the same assignment from them: with
// T = ceil(N / G) for N active rows over G tiles, tile t keeps
// k_t = max(min(c_t, T), min(c_t, 3 RG)) of its c_t entries (its first three steps are
// already under way) and gives the rest away; the given-away entries, in tile order,
// fill the shortfalls T - k_t of the other tiles, in tile order. The assignment depends
// on the counts only, so every workgroup sums the same rows in the same order on every
// run and y stays deterministic. The counts live in the workspace header, which the
// reduce kernel clears again.
// Waiting for every count is safe only if every tile is resident, which a launch does not
// guarantee: with two such calls in flight on different streams, each can hold part of
// the device while its other tiles wait for it. So the launch first settles, in one header
// word, whether it balances at all. The last workgroup, on starting, swaps the word from 0
// to "yes": workgroups are dispatched in index order, so all the others have started, and
// none can finish before the decision, so all are resident. Workgroup 0 (always resident)
// swaps it from 0 to "no" if it is still unset a few microseconds after its own decision
// point. The first swap wins and every workgroup follows the word: "no" means each tile
// keeps its own rows and waits for nothing else.
// It costs a write-through of the tile's list and a wait for it, the count round trip,
// and for a workgroup that takes rows, a round trip for their entries. That pays only
// where tiles carry much up/down work: rows wider than 8 KB. One token, graph replay:
// d 8192, f 28672: 148.3 against 154.0 us per call at 50% sparsity, 109.2 against 112.6
// at 80%, 98.5 against 98.0 at 90%; d 5120, f 13824: 56.5 against 58.1 at 50%. With 8 KB
// rows it lost: 37.6 against 37.2 us at d 4096, f 11008, 50%; 29.6 against 26.7 at 90%;
// 52.2 against 51.5 at d 3584, f 18944.
constexpr int kBalMaxTiles = 256;
constexpr uint32_t kPublished = 0x80000000u;

struct BalSmem {
  uint32_t decision;  // the launch's kBalYes / kBalNo, or 0 if it never arrived
  int cnt[kBalMaxTiles];
  int epre[kBalMaxTiles + 1];  // entries given away by the tiles before t
  int dpre[kBalMaxTiles + 1];  // shortfalls of the tiles before t
  int wsum[3][kNW];
};

template <int RG>
struct Balancer {
  BalSmem& bs;
  bool on;
  int G, w, nown, n_total;
  uint32_t cw;           // count word of tile threadIdx.x, loaded when the up/down starts
  uint32_t dw0 = 0;      // thread 0: the decision word, loaded with the counts
  bool gave_up = false;  // a count never arrived: this workgroup's partial becomes NaN

  __device__ bool active() const { return on; }
  __device__ bool poisoned() const { return gave_up; }

  static constexpr int kPre = 3;  // up/down steps issued before the decision
  __device__ static int keep_of(int c, int T) { return max(min(c, T), min(c, kPre * RG)); }

  // the count words, loaded after the first up/down step (most tiles have published by
  // the time they are used, one step later)
  __device__ void load_counts(const DevArgs& a) {
    if ((int)threadIdx.x < G) cw = ld_through(a.flags + threadIdx.x);
    if (threadIdx.x == 0) dw0 = ld_through(a.flags + kWsBalDecisionWord);
  }

  // Every tile's count (waiting for tiles still gating), the assignment, and this
  // workgroup's list: its first keep entries, then its share of the given-away ones
  // appended. Returns the list length.
  // polls of workgroup 0 for the last workgroup's "yes" before it decides "no"
  static constexpr uint32_t kDecideSpins = 4;

  template <class SmemT>
  __device__ int decide(const DevArgs& a, SmemT& sm, int covered) {
    (void)covered;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the launch's decision (see above); the wait for it ends because workgroup 0 is
    // resident, and is bounded all the same
    if (tid == 0) {
      SFN_GLOBAL uint32_t* dw = a.flags + kWsBalDecisionWord;
      uint32_t dv = dw0;
      const uint32_t bound = w == 0 ? kDecideSpins : (1u << 20);
      for (uint32_t spins = 0; dv == 0u && spins < bound; ++spins) {
        __builtin_amdgcn_s_sleep(2);
        dv = ld_through(dw);
      }
      if (dv == 0u && w == 0) {
        const uint32_t found = cas_through(dw, 0u, kBalNo);
        dv = found == 0u ? kBalNo : found;
      }
      bs.decision = dv;
    }
    __syncthreads();
    if (bs.decision != kBalYes) {
      if (bs.decision != kBalNo) {  // never decided: poison, as for a count that never came
        gave_up = true;
        if (tid == 0) st_through(a.flags + kWsStatusWord, kStatusBalancer);
      }
      return nown;  // every tile streams all of its own entries
    }
    // Every tile is resident at once (G <= CU count), so the wait ends once all have been
    // dispatched; kernels of other streams can only delay that. The bound (2^20 round
    // trips, about a second) is a guard: a workgroup that reaches it poisons its partial,
    // so y is NaN, not wrong, and sets the workspace status word.
    uint32_t v = cw;
    bool late = false;
    if (tid < G) {
      uint32_t spins = 0;
      while (!(v & kPublished)) {
        if (++spins > (1u << 20)) {
          late = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        v = ld_through(a.flags + tid);
      }
    }
    gave_up = __syncthreads_or(late) != 0;
    if (gave_up && tid == 0) st_through(a.flags + kWsStatusWord, kStatusBalancer);
    // a tile has at most kTMax rows; the clamp keeps every index below in bounds even if
    // the header held something other than zeros when the call started
    const int c = tid < G ? min((int)(v & ~kPublished), kTMax) : 0;
    const int ic = wave_incl_scan(c);
    if (lane == 63) bs.wsum[0][wave] = ic;
    if (tid < G) bs.cnt[tid] = c;
    __syncthreads();
    int N = 0;
#pragma unroll
    for (int i = 0; i < kNW; ++i) N += bs.wsum[0][i];
    const int T = (N + G - 1) / G;
    const int kt = keep_of(c, T);
    const int ex = c - kt;                             // given away by tile tid
    const int df = tid < G ? max(T - kt, 0) : 0;       // taken by tile tid
    const int ie = wave_incl_scan(ex), id = wave_incl_scan(df);
    if (lane == 63) {
      bs.wsum[1][wave] = ie;
      bs.wsum[2][wave] = id;
    }
    __syncthreads();
    int be = 0, bd = 0;
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
      be += i < wave ? bs.wsum[1][i] : 0;
      bd += i < wave ? bs.wsum[2][i] : 0;
    }
    if (tid <= G) {  // G < kNT: thread G writes the totals
      bs.epre[tid] = be + ie - ex;
      bs.dpre[tid] = bd + id - df;
    }
    __syncthreads();
    const int keep = keep_of(nown, T);
    const int etot = bs.epre[G];
    const int e0 = min(bs.dpre[w], etot), e1 = min(bs.dpre[w] + max(T - keep, 0), etot);
    const int ns = max(e1 - e0, 0);
    for (int i = tid; i < ns; i += kNT) {
      const int k = e0 + i;
      int lo = 0, hi = G;  // the tile whose given-away range holds k: epre[lo] <= k < epre[lo + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (bs.epre[mid] <= k) lo = mid;
        else hi = mid;
      }
      const int slot = min(share_begin(lo, n_total, G) + keep_of(bs.cnt[lo], T) + (k - bs.epre[lo]), a.f - 1);
      const uint32_t row = ld_through(reinterpret_cast<const SFN_GLOBAL uint32_t*>(a.sel_idx + slot));
      sm.qrow[keep + i] = (int)min(row, (uint32_t)(a.f - 1));
      sm.qa[keep + i][0] = __uint_as_float(ld_through(reinterpret_cast<const SFN_GLOBAL uint32_t*>(a.sel_a + slot)));
      sm.qbits[keep + i] = 1;
    }
    __syncthreads();
    return keep + ns;
  }
};

// Gate and up/down of one tile in one workgroup: the tile's selected rows are recorded
// in LDS as the gate finds them, and the same workgroup then streams their up and down
// rows and writes its partial of y. No list crosses workgroups, so the up/down launch
// and its prologue (a scan over the tile counts, then a gather of the share) disappear;
// the price is that a tile's share follows the spread of its selected-row count. One
// token at d 4096: 37.1-37.3 against 40.4 us per call at f 11008 and 50% sparsity, 29.8
// against 33.4 at 80%, 46.1 against 50.1 at f 14336; 156.6 against 160.8 at d 8192,
// f 28672. Both 1.5x and 2x the tiles, and 1 or 4 up/down rows per step, were slower.
template <int WT, int BMAX, int CPT, int TPR, int RGATE, int RUP>
__global__ __launch_bounds__(kNT) void decode_gate_local_kernel(DecodeArgs args) {
  using UD = UpDownKernel<WT, BMAX, CPT, TPR, RUP>;
  static_assert(BMAX == 1, "one token");
  __shared__ typename UD::Smem usm;
  __shared__ BalSmem bsm;
  // balanced launch: the last workgroup to be dispatched settles "yes" if nothing has
  // settled the launch yet (the decision word in the header; see Balancer)
  if (args.flags && blockIdx.x == gridDim.x - 1 && threadIdx.x == 0)
    (void)cas_through(gp(args.flags) + kWsBalDecisionWord, 0u, kBalYes);
  const int2 go = GateKernel<WT, BMAX, CPT, TPR, RGATE>::template run<true>(
      args, [&](int slot, int row, const auto& av, uint32_t bits) {
        usm.qrow[slot] = row;
        usm.qbits[slot] = (uint8_t)bits;
#pragma unroll
        for (int b = 0; b < BMAX; ++b) usm.qa[slot][b] = av[b];
      });
  const DevArgs a = dev_args(args);
  const int tid = threadIdx.x, w = blockIdx.x;
  const int n_total = a.cand ? min(max(*a.n_cand, 0), a.f) : a.f;
  Balancer<UD::RG> bal{bsm, a.flags != nullptr, a.G, w, go.x, n_total, kPublished};
  if (bal.on) {
    // the tile's entries, then its count, through to memory for the other workgroups
    for (int j = tid; j < go.x; j += kNT) {
      st_through(reinterpret_cast<SFN_GLOBAL uint32_t*>(a.sel_idx + go.y + j), (uint32_t)usm.qrow[j]);
      st_through(reinterpret_cast<SFN_GLOBAL uint32_t*>(a.sel_a + go.y + j), __float_as_uint(usm.qa[j][0]));
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have reached memory
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0) st_through(a.flags + w, kPublished | (uint32_t)go.x);
  }
  UD::stream(a, usm, go.x, w, bal);
}

template <int WT, int BMAX, int CPT, int TPR, int R>
__global__ __launch_bounds__(kNT) void decode_updown_kernel(DecodeArgs a) {
  UpDownKernel<WT, BMAX, CPT, TPR, R>::run(a);
}

__global__ __launch_bounds__(512) void decode_reduce_kernel(DecodeArgs a, int P) { ReduceKernel::run(a, P); }

// Compute units of the current device (cached per device; 0 if unknown). Host threads
// may call this concurrently: every thread that finds the entry empty stores the same
// value.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = -1;
    cache[dev].store(n, std::memory_order_relaxed);
    v = n;
  }
  return v > 0 ? v : 0;
}

// Workgroups of the reduce kernel: the column chunks of y (n_red), and when the index
// lists are asked for, at least one workgroup per four gate tiles (G is the gate's tile
// count, which for the matrix-core gate differs from the up/down grid).
int reduce_grid(const DecodeArgs& g) {
  int n = g.y ? g.n_red : 1;
  if (g.active_idx && (g.G + 3) / 4 > n) n = (g.G + 3) / 4;
  return n;
}

// Batches of at least this many tokens take the matrix-core gate (bf16 weights, at most
// kGMax tiles of 16 rows, no candidate list): its cost per row does not grow with the batch.
constexpr int kMfmaGateMinBatch = 2;

// Tiles of the matrix-core gate: at most 16 rows each (rows split evenly over the tiles),
// rounded up to a multiple of 256 workgroups while that stays within kGMax, so that every
// compute unit of a 256-CU device holds the same number of tiles (all of them are
// resident at once). At f 14336, 1024 tiles of 14 rows took 2.1-2.3 us less per
// four-token call than 896 tiles of 16 rows, and at f 11008 768 tiles about 1 us less
// than 688. The matrix-core gate is taken iff ceil(f / 16) <= kGMax, as before.
int mfma_gate_tiles(int f) {
  const int g = (f + kMRows - 1) / kMRows;
  const int r = (g + 255) / 256 * 256;
  return r <= kGMax ? r : g;
}

// RGATE / RUP: rows each thread holds per half step of the gate / per up-down step.
template <int WT, int BMAX, int CPT, int TPR, int RGATE, int RUP>
hipError_t launch_pair(const DecodeArgs& a, hipStream_t s) {
  DecodeArgs g = a;  // gate tiles G, up/down workgroups Gu
  g.Gu = a.G;
  const bool mfma = WT == WT_BF16 && !a.cand && !a.pl && a.nb >= kMfmaGateMinBatch && mfma_gate_tiles(a.f) <= kGMax;
  // one token: each tile streams the up/down rows of its own selected rows, balanced
  // through the header words for rows wider than 8 KB when every tile can be resident
  // at once
  const bool local = BMAX == 1 && a.y;
  g.flags = local && CPT >= 2 && a.G <= kBalMaxTiles && a.G <= device_cus() ? a.flags : nullptr;
  if (mfma) {
    g.G = mfma_gate_tiles(a.f);
    hipLaunchKernelGGL((decode_gate_mfma_kernel<BMAX>), dim3(g.G), dim3(256), 0, s, g);
  } else if (local) {
    if constexpr (BMAX == 1)
      hipLaunchKernelGGL((decode_gate_local_kernel<WT, BMAX, CPT, TPR, RGATE, RUP>), dim3(g.G), dim3(kNT), 0, s, g);
  } else {
    hipLaunchKernelGGL((decode_gate_kernel<WT, BMAX, CPT, TPR, RGATE>), dim3(g.G), dim3(kNT), 0, s, g);
  }
  if constexpr (BMAX > 1)
    if (a.y) hipLaunchKernelGGL((decode_updown_kernel<WT, BMAX, CPT, TPR, RUP>), dim3(g.Gu), dim3(kNT), 0, s, g);
  // one partial row per up/down workgroup and token (row-lanes combined in LDS)
  if (a.y || a.active_idx || a.n_active)
    hipLaunchKernelGGL(decode_reduce_kernel, dim3(reduce_grid(g)), dim3(ReduceKernel::kRT), 0, s, g, g.Gu);
  return hipGetLastError();
}

template <int WT, int CPT, int TPR, int R>
__global__ __launch_bounds__(kNT) void decode_parallel_kernel(DecodeArgs a) {
  ParKernel<WT, CPT, TPR, R>::run(a);
}

template <int WT, int CPT, int TPR, int R>
hipError_t launch_parallel(const DecodeArgs& a0, hipStream_t s) {
  DecodeArgs a = a0;
  a.flags = nullptr;
  hipLaunchKernelGGL((decode_parallel_kernel<WT, CPT, TPR, R>), dim3(a.G), dim3(kNT), 0, s, a);
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(reduce_grid(a)), dim3(ReduceKernel::kRT), 0, s, a,
                     a.G * (kNT / TPR));
  return hipGetLastError();
}

template <int WT>
hipError_t dispatch_parallel(const DecodeArgs& a, hipStream_t s) {
  // three rows per step entry. With one chunk per thread (d up to 4096 in bf16), one row
  // per step (6 weight loads in flight per thread over both buffers) streamed best:
  // 27.4 / 16.4 / 10.9 us per call at 50 / 20 / 5% candidates of f 11008, against 29.1 /
  // 18.7 / 11.8 with four rows
  if (a.nch > 2048) return hipErrorInvalidValue;
  if (a.nch > 1024) return launch_parallel<WT, 4, 512, 1>(a, s);
  if (a.nch > 512) return launch_parallel<WT, 2, 512, 2>(a, s);
  // predict mode: a tile's own candidates (about 9 of its 43 rows at 22% density) go two
  // rows per step, so its few steps take fewer round trips: 25.2 against 25.7 us per fused
  // call at rank 256, 29.7 against 30.0 at rank 1024 (whitened)
  if (a.nch > 256) return a.pl ? launch_parallel<WT, 1, 512, 2>(a, s) : launch_parallel<WT, 1, 512, 1>(a, s);
  if (a.nch > 128) return launch_parallel<WT, 1, 256, 4>(a, s);
  if (a.nch > 64) return launch_parallel<WT, 1, 128, 4>(a, s);
  return launch_parallel<WT, 1, 64, 2>(a, s);
}

template <int WT, int BMAX>
hipError_t dispatch_tpr(const DecodeArgs& a, hipStream_t s) {
  // rows per thread per half step: 16 weight loads in flight per thread and buffer for
  // one token, 8 for four tokens (the dot-product registers grow with the batch). With
  // one chunk per thread (d up to 4096 in bf16) 2 rows stream faster, i.e. 8 loads in
  // flight per thread over both buffers for one token: 39.8-41.1 against 43.3-44.4 us
  // per call at d 4096, f 11008, and 47.2 against 51.7 us at f 14336 (batches of two:
  // 63.8 against 64.7 us at f 14336; four tokens unchanged).
  constexpr int RB = BMAX == 1 ? 8 : 4;
  constexpr int R1 = 2;
  if (a.nch > 2048) return hipErrorInvalidValue;
  if (a.nch > 1024) return launch_pair<WT, BMAX, 4, 512, RB / 4, RB / 4>(a, s);
  if (a.nch > 512) return launch_pair<WT, BMAX, 2, 512, RB / 2, RB / 2>(a, s);
  if (a.nch > 256) return launch_pair<WT, BMAX, 1, 512, R1, R1>(a, s);
  if (a.nch > 128) return launch_pair<WT, BMAX, 1, 256, RB, RB>(a, s);
  if (a.nch > 64) return launch_pair<WT, BMAX, 1, 128, RB, RB>(a, s);
  return launch_pair<WT, BMAX, 1, 64, 4, 4>(a, s);
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
  (void)G;
  int n = (nb * d + kRedCols - 1) / kRedCols;  // one 32-column chunk per reducing workgroup
  if (n > kGMax) n = kGMax;
  return n < 1 ? 1 : n;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Gate tiles the workspace holds counts for: the vector gate's or the matrix-core gate's.
static int decode_tiles_max(int f) {
  const int g = decode_grid(f), m = mfma_gate_tiles(f);
  return m <= kGMax && m > g ? m : g;
}

size_t decode_workspace_bytes(int d, int f, int wb, int nb) {
  const int G = decode_grid(f);
  const int nch = d * wb / 16;
  const size_t rpg = (size_t)decode_rows_side_by_side(nch);
  size_t bytes = kWsHeader;
  bytes = align256(bytes + (size_t)decode_tiles_max(f) * kCnt * sizeof(int32_t));  // tile_cnt
  bytes = align256(bytes + (size_t)kBMaxAll * f * sizeof(int32_t));  // tile_idx
  bytes = align256(bytes + (size_t)f * sizeof(int32_t));             // sel_idx
  bytes = align256(bytes + (size_t)kBMaxAll * f * sizeof(float));    // sel_a
  bytes = align256(bytes + (size_t)f);                               // sel_bits
  bytes += (size_t)G * rpg * nb * d * sizeof(float);                 // part
  return bytes;
}

void decode_carve(DecodeArgs& a, void* ws, int wb) {
  (void)wb;
  char* p = static_cast<char*>(ws);
  size_t off = kWsHeader;
  a.tile_cnt = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + (size_t)decode_tiles_max(a.f) * kCnt * sizeof(int32_t));
  a.tile_idx = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + (size_t)kBMaxAll * a.f * sizeof(int32_t));
  a.sel_idx = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + (size_t)a.f * sizeof(int32_t));
  a.sel_a = reinterpret_cast<float*>(p + off);
  off = align256(off + (size_t)kBMaxAll * a.f * sizeof(float));
  a.sel_bits = reinterpret_cast<uint8_t*>(p + off);
  off = align256(off + (size_t)a.f);
  a.part = reinterpret_cast<float*>(p + off);
  a.flags = reinterpret_cast<uint32_t*>(p);  // the header (the launcher decides whether to use it)
}

hipError_t launch_decode_parallel(const DecodeArgs& a, int wdtype, hipStream_t s) {
  if (a.G > kGMax) return hipErrorInvalidValue;
  return wdtype == WT_BF16 ? dispatch_parallel<WT_BF16>(a, s) : dispatch_parallel<WT_F32>(a, s);
}

hipError_t launch_decode(const DecodeArgs& a, int wdtype, hipStream_t s) {
  if (a.G > kGMax) return hipErrorInvalidValue;
  if (wdtype == WT_BF16) {
    return a.nb == 1 ? dispatch_tpr<WT_BF16, 1>(a, s) : dispatch_tpr<WT_BF16, 4>(a, s);
  }
  return a.nb == 1 ? dispatch_tpr<WT_F32, 1>(a, s) : dispatch_tpr<WT_F32, 4>(a, s);
}

}  // namespace sfn
