// moe_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "moe.h"

namespace moe {

constexpr int kGroup = 128;        // int4 group size and the k-tile of every layout
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kBlobAlign = 256;
constexpr int kPermSmallT = 1024;  // largest T grouped by the single-workgroup kernel
constexpr int kPermChunk = 256;    // tokens per block of the multi-block grouping
constexpr int kCertifiedMinT = 256;   // fewest tokens routed by the MFMA router
constexpr int kCertifiedMinE = 32;    // fewest experts for it
constexpr double kCertifiedMinFma = 536870912.0;  // fewest T*E*H for it (2^29)
constexpr int kRouterMaxSplit = 8;    // most K splits across blocks of the MFMA router

// Whether a routing call that wants no logits takes the MFMA router
// (router_certified.hip): in auto mode, calls large enough for it to beat the
// canonical fp32 kernel (which costs T*E*H FMAs).
inline bool use_certified_router(int mode, int T, int E, int H) {
  if (mode == MOE_ROUTER_CANONICAL) return false;
  if (mode == MOE_ROUTER_MFMA) return T > 0;
  return T >= kCertifiedMinT && E >= kCertifiedMinE && (double)T * E * H >= kCertifiedMinFma;
}

// K splits across blocks of the MFMA router logits: a power of two dividing
// H / 256 (so each wave's K slice is a multiple of 64), raised until the grid
// has about four blocks per CU.
inline int router_split(int T, int E, int H) {
  const long blocks = (long)((T + 31) / 32) * ((E + 63) / 64);
  const int m = H / 256;
  int S = 1;
  while (2 * S <= kRouterMaxSplit && m % (2 * S) == 0 && blocks * S < 1024) S *= 2;
  return S;
}

// Device copy of one expert handle (same field order as moe_expert_handle).
struct DevHandle {
  int32_t tier;
  int32_t flags;
  const uint8_t* w13;
  const uint8_t* w2;
};
static_assert(sizeof(DevHandle) == sizeof(moe_expert_handle), "handle layout");

// One M-tile of a grouped GEMM: rows [row_start, row_start + rows) of the
// grouped (sorted) route order, all owned by `expert`.  The grouping kernel
// copies the expert's current tier and the packed blob this GEMM reads (w13
// for the gate/up table, w2 for the down table) out of the handle table, so a
// GEMM workgroup finds its weights with one load instead of two dependent ones.
struct TileEntry {
  int32_t expert;
  int32_t row_start;
  int32_t rows;
  int32_t tier;
  const uint8_t* w;
  int64_t pad;
};
static_assert(sizeof(TileEntry) == 32, "tile entry is one 32-byte scalar load");

// Kernel family and M-tile size for one forward, picked on the host from T
// and the layer: decode (few routes per expert, weight streaming, exact
// integer MFMA operands) or prefill (many routes per expert, fp16 MFMA).
enum GemmKind { kGemmDecode = 1, kGemmPrefill = 2 };
// Each grouped GEMM takes its own kernel family and M-tiling.  The one mixed
// plan is a large-batch gate/up GEMM feeding a decode down GEMM: its epilogue
// then writes bf16 activations and their 32-column row sums, as the decode
// gate/up epilogue does.
struct GemmPlan {
  int bm13;   // rows per M-tile, gate/up GEMM
  int bm2;    // rows per M-tile, down GEMM
  int kind;   // GemmKind of the gate/up GEMM
  int kind2;  // GemmKind of the down GEMM
};

// Byte offsets of the workspace regions for T tokens.
struct WsPlan {
  size_t logits, ids, weights, offsets, sorted, pos, tiles13, ntiles13, tiles2, ntiles2;
  size_t rank, chunk_counts, chunk_tot, xn2, wn2;
  size_t r13, act, r2, rows, x16;
  size_t total;
  int max_tiles13, max_tiles2;
};

struct Layer {
  int32_t H, I, E, k;
  DevHandle* table;      // device [E]
  // wave execution: resident slots (up to E) and the global-expert-to-slot
  // map (-1 = inactive sentinel), both stream-ordered device state; slot_set
  // records on the host which slots hold a validated handle
  DevHandle* slots;      // device [E]
  int32_t* slot_map;     // device [E]
  uint8_t* slot_set;     // host [E]
  // usage trace over many calls: each forward sets hot[e] = decay * hot[e] + its
  // routes to e (caller-owned device [E], or null)
  float* hot;
  float hot_decay;
  void* stage_events[9];
  int32_t n_stage_events;
  int32_t router_mode;   // moe_router_mode
};

// Wave mode of one forward: expert e runs from slots[slot_map[e]] when that
// is >= 0 and contributes nothing otherwise.  Both null: every expert runs
// from the layer's handle table.
struct WaveMap {
  const int32_t* slot_map;
  const DevHandle* slots;
};

// Optional start/stop events that receive one kernel's own timestamps
// (hipExtLaunchKernelGGL); both null: an ordinary launch.
struct KernelTimer {
  hipEvent_t start, stop;
};

// Per-forward hotness update of the grouping kernels (hot null: none).
struct Hotness {
  float* hot;
  float decay;
};

// error state ---------------------------------------------------------------
int set_error(int status, const char* fmt, ...);
int check_hip(hipError_t e, const char* what);
void clear_error();

// Kernels that take more than 64 KB of dynamic LDS need an opt-in per kernel
// and device (hipFuncSetAttribute acts on the current device).  One bit per
// device records that it was made; concurrent first calls may both set it,
// which is harmless.
struct DeviceOnce {
  std::atomic<uint64_t> done{0};
};
inline hipError_t ensure_dynamic_lds(DeviceOnce& once, const void* kern, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (once.done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) once.done.fetch_or(bit, std::memory_order_release);
  return e;
}

// planning ------------------------------------------------------------------
GemmPlan plan_gemm(const Layer& L, int T);
WsPlan plan_workspace(const Layer& L, int T, const GemmPlan& gp);

// launchers (return hipError_t of the launch) --------------------------------
// Zero bytes [p, p + bytes) with a kernel (bytes a multiple of 4; usable
// where a memset node is not wanted).
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_quantize_pack(int tier, int layout, const uint16_t* w, int64_t n, int64_t k,
                                uint8_t* dst, int* err_flag, hipStream_t s);
hipError_t launch_set_slot_map(int32_t* map, const int32_t* host_map, int E, hipStream_t s);
hipError_t launch_set_handles(DevHandle* table, int first, int count,
                              const moe_expert_handle* h, hipStream_t s);
hipError_t launch_router_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                                int H, int E, float* logits, float* r13, hipStream_t s);
// Routing for many tokens with the logits on MFMA, certified against the
// canonical order: writes ids and weights as launch_topk does.  Workspace,
// with S = router_split(T, E, H): v [S, T, E], xn2 [S, T], wn2 [S, E].
hipError_t launch_router_certified(const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                                   int H, int E, int k, float* v, float* xn2, float* wn2,
                                   int32_t* ids, float* w, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                       hipStream_t s);
// R13 [T, H/128] alone (the fixed-order logits kernel also writes it), bit for
// bit the same sums.
hipError_t launch_group_sums(const uint16_t* x, int T, int H, float* r13, hipStream_t s);
// Few tokens: logits (canonical order), the group sums r13 and the top k in
// one launch, one block per token; the logits stay on chip.  Same ids,
// weights and r13, bit for bit, as launch_router_logits + launch_topk.
constexpr int kSmallRouteMaxT = 64;
constexpr int kSmallRouteMaxE = 128;
// Router weights one block streams: one CU reads 512 KiB (E 128, H 2048) in
// about 11 us, slower than the two-kernel path's 9.7 us; 256 KiB takes 7.8 us
// against 9.2.
constexpr size_t kSmallRouteMaxBytes = 256 * 1024;
bool use_small_router(int T, int E, int H);
hipError_t launch_router_topk_small(const uint16_t* x, const uint16_t* wr, const float* bias,
                                    int T, int H, int E, int k, float* r13, int32_t* ids,
                                    float* w, hipStream_t s);
// Grouping: one workgroup for T <= kPermSmallT, else a rank pass, a
// per-expert scan over the token blocks and a scatter pass, over blocks of
// kPermChunk tokens (rank [T*k], chunk_counts [ceil(T / kPermChunk) * E] and
// chunk_tot [E] are workspace).
hipError_t launch_permute(const DevHandle* table, WaveMap wave, Hotness hotness, const int32_t* ids, int T, int k,
                          int E, int32_t* offsets, int32_t* sorted, int32_t* pos,
                          TileEntry* tiles13, int32_t* ntiles13, int bm13, TileEntry* tiles2,
                          int32_t* ntiles2, int bm2, int32_t* rank, int32_t* chunk_counts,
                          int32_t* chunk_tot, hipStream_t s);
hipError_t launch_gemm13(const Layer& L, const GemmPlan& gp, int T, const uint16_t* x,
                         const int32_t* sorted, const TileEntry* tiles, const int32_t* ntiles,
                         int max_tiles, const float* r13, uint16_t* act, float* r2,
                         hipStream_t s, KernelTimer kt = KernelTimer{nullptr, nullptr});
hipError_t launch_gemm2(const Layer& L, const GemmPlan& gp, int T, const uint16_t* act,
                        const int32_t* sorted, const float* topk_w, const TileEntry* tiles,
                        const int32_t* ntiles, int max_tiles, const float* r2, float* rows,
                        hipStream_t s);
size_t prefill_lds_bytes();
hipError_t launch_x_to_f16(const uint16_t* x, uint16_t* x16, size_t n, hipStream_t s);
hipError_t launch_prefill(bool gate_up, const Layer& L, int T, const uint16_t* a16, const int32_t* sorted,
                          const TileEntry* tiles, const int32_t* ntiles, int max_tiles,
                          uint16_t* act16, float* r2, const float* topk_w, float* rows,
                          hipStream_t s, KernelTimer kt = KernelTimer{nullptr, nullptr});
// y[t] (=|+=) sum over the token's routes in ascending expert order (rows
// [T k, H] by route id); with a slot map, routes whose expert maps to the
// sentinel are skipped.
hipError_t launch_combine(const float* rows, const int32_t* ids, const int32_t* slot_map, int T,
                          int H, int k, void* y, int y_dtype, bool accumulate, hipStream_t s);

}  // namespace moe
