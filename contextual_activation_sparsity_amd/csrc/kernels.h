// Internal launch interface between the C ABI layer (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sparse_ffn.h"

namespace sfn {

// Workspace layout shared by every call on a workspace:
//   [0, kWsHeader)      words that must be zero when a call starts: zero-filled once by
//                       the caller, and every call that sets some clears them again in
//                       its last launch:
//     words [0, 256)      the one-token decode's tile counts (balancer)
//     word kWsStatusWord  status: 0, or the code of a bounded device wait that gave up
//                         (left set for the caller to read; see sparse_ffn.h)
//     word kWsBalDecisionWord  the balancer's decision for the call in flight: 0 until
//                         decided, then kBalYes or kBalNo (cleared by the reduce kernel)
//   [kWsHeader, ...)    per-call scratch, rewritten by each call before it is read
// Scratch of one call may overlap scratch of another.
constexpr size_t kWsHeader = SFN_WORKSPACE_HEADER_BYTES;
constexpr int kWsStatusWord = SFN_WORKSPACE_STATUS_OFFSET / 4;
constexpr uint32_t kStatusBalancer = SFN_STATUS_BALANCER_TIMEOUT;
constexpr uint32_t kStatusPredictor = SFN_STATUS_PREDICTOR_TIMEOUT;
constexpr int kWsBalDecisionWord = kWsStatusWord + 1;
constexpr uint32_t kBalYes = 1u;  // every tile of the launch is resident: balance
constexpr uint32_t kBalNo = 2u;   // some tile was not dispatched in time: each keeps its own rows

struct DecodeArgs {
  const char* wg;
  const char* wu;
  const char* wd;
  const float* bias;  // [f] or null
  const char* x;      // [nb, d]
  const float* t;     // device threshold or null (0)
  const int32_t* cand;
  const int32_t* n_cand;
  const uint8_t* mask_in;  // [nb, f] or null
  float* y;                // [nb, d] or null
  int32_t* active_idx;     // [nb, f] or null
  int32_t* n_active;       // [nb] or null
  int32_t* tile_cnt;  // [G, 8]: union count, then one count per token
  int32_t* tile_idx;  // [4, f]: per-token active rows, by tile
  int32_t* sel_idx;   // [f]: rows active for some token, by tile
  float* sel_a;       // [4, f]: their activations
  uint8_t* sel_bits;  // [f]: their per-token mask bits
  float* part;        // [G * rows side by side, nb, d]
  // One word per gate tile in the workspace header (zero between calls), or null: the
  // one-token decode balances its up/down work through them (the launcher decides).
  uint32_t* flags;
  // Predict mode (pl non-null; one token): each tile's candidates are {i : L_i z + pb_i >
  // ptau_i} over its own rows instead of a share of a candidate list; z = Q x from the
  // predictor's first launch, r = rank.
  const char* pl;     // [f, r] bf16
  const float* pz;    // [r]
  const float* ptau;  // [f]
  const float* pb;    // [f] or null
  int pr;
  // G: gate tiles (tile i covers rows [i f / G, (i + 1) f / G)); Gu: up/down workgroups
  // and partial-row groups (0 means G; the launcher sets it)
  int d, f, nch, row_bytes, nb, act, G, n_red, Gu;
};

// Decode (a gate kernel over tiles of rows that writes compacted active lists; for one
// token each tile then streams the up/down rows of its own active rows, for a batch an
// up/down kernel splits the concatenated list evenly; both write fp32 partials of y, and
// a reduce kernel sums them in a fixed order): workgroups per launch for f neurons,
// reducing workgroups, rows a workgroup handles side by side (partials per workgroup),
// workspace bytes, carving of the workspace.
int decode_grid(int f);
int decode_reducers(int G, int nb, int d);
int decode_rows_side_by_side(int nch);
size_t decode_workspace_bytes(int d, int f, int wb, int nb);
void decode_carve(DecodeArgs& a, void* ws, int wb);
hipError_t launch_decode(const DecodeArgs& a, int wdtype, hipStream_t stream);
// Candidate rows in one pass (gate, up and down rows together), then the reduce kernel.
hipError_t launch_decode_parallel(const DecodeArgs& a, int wdtype, hipStream_t stream);

size_t chunk_workspace_bytes(int d, int f, int wdtype, int n);
hipError_t launch_dense_chunk(const sfn_ffn& ffn, const void* x, int n, float* y, void* ws, hipStream_t stream);

size_t calibrate_workspace_bytes(int d, int f, int wdtype, int n);
hipError_t launch_calibrate(const sfn_ffn& ffn, const void* x_cal, int n, float k, float* t_out,
                            float* scores_out, void* ws, hipStream_t stream);

size_t svd_workspace_bytes(int d, int f, int r);
// z = Q x only (the predictor's first launch), into z [r].
hipError_t launch_svd_z(const sfn_svd& s, const void* x, float* z, hipStream_t stream);
hipError_t launch_svd_predict(const sfn_svd& s, const void* x, int32_t* cand, int32_t* n_cand, float* p_out,
                              void* ws, hipStream_t stream);

}  // namespace sfn
