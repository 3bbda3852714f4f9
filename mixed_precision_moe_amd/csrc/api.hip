// api.hip -- the C ABI: validation, layer object, workspace plan, launch order.
//
// The launch order of one forward follows the call stack of "Every Expert
// Counts: ExactMoE ..." §3.4 with every expert resident (one wave holding all
// experts): router -> top-k -> group tokens by expert -> one gate/up grouped
// GEMM (+SwiGLU) -> one down grouped GEMM (x routing weight) -> sum of the
// experts' contributions.  Nothing here allocates, synchronizes or copies to
// the host on that path.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

static thread_local char g_err[512] = "";

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = 0; }

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return set_error(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

WsPlan plan_workspace(const Layer& L, int T, const GemmPlan& gp) {
  WsPlan w{};
  const size_t R = (size_t)T * L.k;
  w.max_tiles13 = (int)(R / gp.bm13) + (int)(R < (size_t)L.E ? R : (size_t)L.E);
  w.max_tiles2 = (int)(R / gp.bm2) + (int)(R < (size_t)L.E ? R : (size_t)L.E);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = round_up(o + bytes, kBlobAlign);
    return at;
  };
  // the MFMA router (any call of this size may take it) keeps S partial
  // logit rows per token here
  const bool cert = use_certified_router(L.router_mode, T, L.E, L.H);
  const size_t S = cert ? (size_t)router_split(T, L.E, L.H) : 1;
  w.logits = take(sizeof(float) * T * (size_t)L.E * S);
  w.ids = take(sizeof(int32_t) * R);
  w.weights = take(sizeof(float) * R);
  w.offsets = take(sizeof(int32_t) * (L.E + 1));
  w.sorted = take(sizeof(int32_t) * R);
  w.pos = take(sizeof(int32_t) * R);
  w.rank = take(sizeof(int32_t) * R);
  w.chunk_counts = take(sizeof(int32_t) * (size_t)((T + kPermChunk - 1) / kPermChunk) * L.E);
  w.chunk_tot = take(sizeof(int32_t) * (size_t)L.E);
  w.xn2 = take(sizeof(float) * (size_t)T * S);
  w.wn2 = take(sizeof(float) * (size_t)L.E * S);
  w.tiles13 = take(sizeof(TileEntry) * (size_t)(w.max_tiles13 > 0 ? w.max_tiles13 : 1));
  w.ntiles13 = take(2 * sizeof(int32_t));   // [tile count, decode grouping flag]
  w.tiles2 = take(sizeof(TileEntry) * (size_t)(w.max_tiles2 > 0 ? w.max_tiles2 : 1));
  w.ntiles2 = take(2 * sizeof(int32_t));
  w.r13 = take(sizeof(float) * T * (size_t)(L.H / kGroup));
  w.act = take(sizeof(uint16_t) * R * L.I);
  w.r2 = take(sizeof(float) * R * (L.I / 32));
  w.rows = take(sizeof(float) * R * L.H);
  w.x16 = take(gp.kind == kGemmPrefill ? sizeof(uint16_t) * T * (size_t)L.H : 0);
  w.total = o;
  return w;
}

namespace {

constexpr int kHandlesPerLaunch = 64;
struct HandleBatch {
  moe_expert_handle h[kHandlesPerLaunch];
};

__global__ void set_handles_kernel(DevHandle* table, int first, int count, HandleBatch b) {
  const int i = threadIdx.x;
  if (i < count) {
    DevHandle d;
    d.tier = b.h[i].tier;
    d.flags = b.h[i].flags;
    d.w13 = reinterpret_cast<const uint8_t*>(b.h[i].w13);
    d.w2 = reinterpret_cast<const uint8_t*>(b.h[i].w2);
    table[first + i] = d;
  }
}

constexpr int kMapPerLaunch = 256;
struct MapBatch {
  int32_t v[kMapPerLaunch];
};

__global__ void set_map_kernel(int32_t* map, int first, int count, MapBatch b) {
  const int i = threadIdx.x;
  if (i < count) map[first + i] = b.v[i];
}

int validate_handles(const moe_expert_handle* h, int count) {
  for (int i = 0; i < count; ++i) {
    if (h[i].tier < MOE_TIER_BF16 || h[i].tier > MOE_TIER_INT4)
      return set_error(MOE_EINVAL, "handle %d: bad tier %d", i, h[i].tier);
    if (h[i].flags != 0) return set_error(MOE_EINVAL, "handle %d: flags must be 0", i);
    if (!h[i].w13 || !h[i].w2) return set_error(MOE_EINVAL, "handle %d: null weight pointer", i);
    if (!aligned(h[i].w13, kBlobAlign) || !aligned(h[i].w2, kBlobAlign))
      return set_error(MOE_EINVAL, "handle %d: weight blobs must be 256-byte aligned", i);
  }
  return MOE_OK;
}

}  // namespace

hipError_t launch_set_slot_map(int32_t* map, const int32_t* host_map, int E, hipStream_t s) {
  for (int done = 0; done < E; done += kMapPerLaunch) {
    const int n = E - done < kMapPerLaunch ? E - done : kMapPerLaunch;
    MapBatch b;
    for (int i = 0; i < kMapPerLaunch; ++i) b.v[i] = i < n ? (host_map ? host_map[done + i] : -1) : -1;
    hipLaunchKernelGGL(set_map_kernel, dim3(1), dim3(kMapPerLaunch), 0, s, map, done, n, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_set_handles(DevHandle* table, int first, int count,
                              const moe_expert_handle* h, hipStream_t s) {
  for (int done = 0; done < count; done += kHandlesPerLaunch) {
    const int n = count - done < kHandlesPerLaunch ? count - done : kHandlesPerLaunch;
    HandleBatch b;
    memset(&b, 0, sizeof b);
    memcpy(b.h, h + done, sizeof(moe_expert_handle) * n);
    hipLaunchKernelGGL(set_handles_kernel, dim3(1), dim3(kHandlesPerLaunch), 0, s, table,
                       first + done, n, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ESHAPE: return "unsupported shape";
    case MOE_ERANGE: return "value out of range";
    case MOE_ENOSPC: return "buffer too small";
    case MOE_EHIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

size_t moe_packed_size(int tier, int64_t n_out, int64_t k_in) {
  if (n_out <= 0 || k_in <= 0 || k_in % kGroup || n_out % 64) return 0;
  size_t bytes;
  switch (tier) {
    case MOE_TIER_INT4: bytes = (size_t)n_out * k_in / 2 + (size_t)n_out * (k_in / kGroup) * 2; break;
    case MOE_TIER_INT8: bytes = (size_t)n_out * k_in + 2 * (size_t)n_out; break;
    case MOE_TIER_BF16: bytes = 2 * (size_t)n_out * k_in; break;
    default: return 0;
  }
  return round_up(bytes, kBlobAlign);
}

static int check_pack_args(int tier, int layout, const uint16_t* w_bf16, int64_t n_out,
                           int64_t k_in, void* dst, size_t dst_bytes, size_t* need, size_t* payload) {
  if (tier < MOE_TIER_BF16 || tier > MOE_TIER_INT4)
    return set_error(MOE_EINVAL, "bad tier %d", tier);
  if (layout != MOE_LAYOUT_PLAIN && layout != MOE_LAYOUT_GATE_UP)
    return set_error(MOE_EINVAL, "bad layout %d", layout);
  if (!w_bf16 || !dst) return set_error(MOE_EINVAL, "null pointer");
  if (!aligned(dst, kBlobAlign)) return set_error(MOE_EINVAL, "dst must be 256-byte aligned");
  if (!aligned(w_bf16, 16)) return set_error(MOE_EINVAL, "weights must be 16-byte aligned");
  if (n_out <= 0 || k_in <= 0 || k_in % kGroup || n_out % 64 || n_out > (1 << 30) ||
      k_in > (1 << 30))
    return set_error(MOE_ESHAPE, "need k_in %% 128 == 0 and n_out %% 64 == 0 (got %lld x %lld)",
                     (long long)n_out, (long long)k_in);
  if ((uint64_t)n_out * (uint64_t)k_in * 2 > 0xffffffffull)
    return set_error(MOE_ESHAPE, "a packed matrix must stay below 4 GiB");
  *need = moe_packed_size(tier, n_out, k_in);
  if (dst_bytes < *need)
    return set_error(MOE_ENOSPC, "dst has %zu bytes, %zu needed", dst_bytes, *need);
  switch (tier) {
    case MOE_TIER_INT4: *payload = (size_t)n_out * k_in / 2 + (size_t)n_out * (k_in / kGroup) * 2; break;
    case MOE_TIER_INT8: *payload = (size_t)n_out * k_in + 2 * (size_t)n_out; break;
    default: *payload = 2 * (size_t)n_out * k_in; break;
  }
  return MOE_OK;
}

int moe_quantize_pack(int tier, int layout, const uint16_t* w_bf16, int64_t n_out, int64_t k_in,
                      void* dst, size_t dst_bytes, void* stream) {
  g_err[0] = 0;
  size_t need = 0, payload = 0;
  int rc = check_pack_args(tier, layout, w_bf16, n_out, k_in, dst, dst_bytes, &need, &payload);
  if (rc) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int* flag = nullptr;
  rc = check_hip(hipMalloc(&flag, sizeof(int)), "hipMalloc(flag)");
  if (rc) return rc;
  int host_flag = 0;
  if (!rc) rc = check_hip(hipMemsetAsync(flag, 0, sizeof(int), s), "hipMemsetAsync(flag)");
  if (!rc && need > payload)
    rc = check_hip(hipMemsetAsync(static_cast<uint8_t*>(dst) + payload, 0, need - payload, s),
                   "hipMemsetAsync(pad)");
  if (!rc)
    rc = check_hip(launch_quantize_pack(tier, layout, w_bf16, n_out, k_in,
                                        static_cast<uint8_t*>(dst), flag, s),
                   "quantize_pack launch");
  if (!rc)
    rc = check_hip(hipMemcpyAsync(&host_flag, flag, sizeof(int), hipMemcpyDeviceToHost, s),
                   "hipMemcpyAsync(flag)");
  if (!rc) rc = check_hip(hipStreamSynchronize(s), "hipStreamSynchronize");
  (void)hipFree(flag);
  if (!rc && host_flag)
    rc = set_error(MOE_ERANGE, "non-finite weight or fp16 scale overflow");
  return rc;
}

int moe_quantize_pack_async(int tier, int layout, const uint16_t* w_bf16, int64_t n_out,
                            int64_t k_in, void* dst, size_t dst_bytes, int32_t* status,
                            void* stream) {
  g_err[0] = 0;
  size_t need = 0, payload = 0;
  int rc = check_pack_args(tier, layout, w_bf16, n_out, k_in, dst, dst_bytes, &need, &payload);
  if (rc) return rc;
  if (!status || !aligned(status, 4)) return set_error(MOE_EINVAL, "status must be a 4-byte aligned device int");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = launch_fill_zero(status, sizeof(int32_t), s);
  if (e == hipSuccess && need > payload)   // payload and need are multiples of 4
    e = launch_fill_zero(static_cast<uint8_t*>(dst) + payload, need - payload, s);
  if (e == hipSuccess)
    e = launch_quantize_pack(tier, layout, w_bf16, n_out, k_in, static_cast<uint8_t*>(dst), status, s);
  return check_hip(e, "quantize_pack launch");
}

int moe_layer_create(const moe_layer_desc* d, const moe_expert_handle* table, void* stream,
                     moe_layer_t* out) {
  g_err[0] = 0;
  if (!d || !table || !out) return set_error(MOE_EINVAL, "null pointer");
  *out = nullptr;
  if (d->hidden <= 0 || d->hidden % 256)
    return set_error(MOE_ESHAPE, "hidden must be a positive multiple of 256 (got %d)", d->hidden);
  if (d->inter <= 0 || d->inter % 128)
    return set_error(MOE_ESHAPE, "inter must be a positive multiple of 128 (got %d)", d->inter);
  if (d->n_experts < 1 || d->n_experts > kMaxExperts)
    return set_error(MOE_ESHAPE, "n_experts must be in [1, %d] (got %d)", kMaxExperts, d->n_experts);
  if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->n_experts)
    return set_error(MOE_ESHAPE, "top_k must be in [1, min(n_experts, %d)] (got %d)", kMaxTopK,
                     d->top_k);
  // the GEMMs address an expert's blob through 32-bit buffer records: the
  // largest tier (bf16) of the gate/up matrix must stay below 4 GiB
  if ((uint64_t)2 * d->inter * 2 * (uint64_t)d->hidden > 0xffffffffull)
    return set_error(MOE_ESHAPE, "an expert's bf16 gate/up matrix (2 x %d x %d x 2 bytes) must stay below 4 GiB",
                     d->inter, d->hidden);
  int rc = validate_handles(table, d->n_experts);
  if (rc) return rc;
  Layer* L = new (std::nothrow) Layer();
  if (!L) return set_error(MOE_EINVAL, "out of host memory");
  L->H = d->hidden;
  L->I = d->inter;
  L->E = d->n_experts;
  L->k = d->top_k;
  L->n_stage_events = 0;
  L->router_mode = MOE_ROUTER_AUTO;
  L->table = nullptr;
  L->hot = nullptr;
  L->hot_decay = 1.0f;
  L->slots = nullptr;
  L->slot_map = nullptr;
  L->slot_set = new (std::nothrow) uint8_t[L->E]();
  if (!L->slot_set) {
    delete L;
    return set_error(MOE_EINVAL, "out of host memory");
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  rc = check_hip(hipMalloc(&L->table, sizeof(DevHandle) * L->E), "hipMalloc(table)");
  if (!rc) rc = check_hip(hipMalloc(&L->slots, sizeof(DevHandle) * L->E), "hipMalloc(slots)");
  if (!rc) rc = check_hip(hipMalloc(&L->slot_map, sizeof(int32_t) * L->E), "hipMalloc(slot_map)");
  if (!rc) rc = check_hip(launch_set_handles(L->table, 0, L->E, table, s), "set_handles launch");
  if (!rc) rc = check_hip(launch_set_slot_map(L->slot_map, nullptr, L->E, s), "set_slot_map launch");
  if (rc) {
    if (L->table) (void)hipFree(L->table);
    if (L->slots) (void)hipFree(L->slots);
    if (L->slot_map) (void)hipFree(L->slot_map);
    delete[] L->slot_set;
    delete L;
    return rc;
  }
  *out = reinterpret_cast<moe_layer_t>(L);
  return MOE_OK;
}

int moe_layer_set_experts(moe_layer_t layer, int32_t first, int32_t count,
                          const moe_expert_handle* handles, void* stream) {
  g_err[0] = 0;
  Layer* L = reinterpret_cast<Layer*>(layer);
  if (!L || (!handles && count > 0)) return set_error(MOE_EINVAL, "null pointer");
  if (first < 0 || count < 0 || first + count > L->E)
    return set_error(MOE_ESHAPE, "handle range [%d, %d) outside [0, %d)", first, first + count, L->E);
  int rc = validate_handles(handles, count);
  if (rc) return rc;
  return check_hip(launch_set_handles(L->table, first, count, handles,
                                      reinterpret_cast<hipStream_t>(stream)),
                   "set_handles launch");
}

int moe_layer_set_slots(moe_layer_t layer, int32_t first, int32_t count,
                        const moe_expert_handle* handles, void* stream) {
  g_err[0] = 0;
  Layer* L = reinterpret_cast<Layer*>(layer);
  if (!L || (!handles && count > 0)) return set_error(MOE_EINVAL, "null pointer");
  if (first < 0 || count < 0 || first + count > L->E)
    return set_error(MOE_ESHAPE, "slot range [%d, %d) outside [0, %d)", first, first + count, L->E);
  int rc = validate_handles(handles, count);
  if (rc) return rc;
  rc = check_hip(launch_set_handles(L->slots, first, count, handles,
                                    reinterpret_cast<hipStream_t>(stream)),
                 "set_slots launch");
  if (!rc)
    for (int i = 0; i < count; ++i) L->slot_set[first + i] = 1;
  return rc;
}

int moe_layer_set_slot_map(moe_layer_t layer, const int32_t* expert_to_slot, void* stream) {
  g_err[0] = 0;
  Layer* L = reinterpret_cast<Layer*>(layer);
  if (!L || !expert_to_slot) return set_error(MOE_EINVAL, "null pointer");
  for (int e = 0; e < L->E; ++e) {
    const int v = expert_to_slot[e];
    if (v == -1) continue;
    if (v < 0 || v >= L->E)
      return set_error(MOE_EINVAL, "expert %d: slot %d outside [-1, %d)", e, v, L->E);
    if (!L->slot_set[v]) return set_error(MOE_EINVAL, "expert %d: slot %d holds no handle", e, v);
  }
  return check_hip(launch_set_slot_map(L->slot_map, expert_to_slot, L->E,
                                       reinterpret_cast<hipStream_t>(stream)),
                   "set_slot_map launch");
}

int moe_layer_set_hotness(moe_layer_t layer, float* hot, float decay) {
  g_err[0] = 0;
  Layer* L = reinterpret_cast<Layer*>(layer);
  if (!L) return set_error(MOE_EINVAL, "null layer");
  if (!(decay >= 0.0f && decay <= 1.0f)) return set_error(MOE_EINVAL, "decay must be in [0, 1]");
  if (hot && !aligned(hot, 4)) return set_error(MOE_EINVAL, "hot must be 4-byte aligned");
  L->hot = hot;
  L->hot_decay = decay;
  return MOE_OK;
}

int moe_plan_tiers(const float* hot, int32_t n_experts, const size_t* bytes_per_tier,
                   size_t budget_bytes, int32_t hi_tier, int32_t lo_tier, int32_t* tiers_out,
                   int32_t* n_hi_out) {
  g_err[0] = 0;
  if (!hot || !bytes_per_tier || !tiers_out) return set_error(MOE_EINVAL, "null pointer");
  if (n_experts < 1 || n_experts > kMaxExperts)
    return set_error(MOE_ESHAPE, "n_experts must be in [1, %d]", kMaxExperts);
  if (hi_tier < MOE_TIER_BF16 || hi_tier > MOE_TIER_INT4 || lo_tier < MOE_TIER_BF16 ||
      lo_tier > MOE_TIER_INT4)
    return set_error(MOE_EINVAL, "bad tier");
  for (int e = 0; e < n_experts; ++e)
    if (!(hot[e] == hot[e])) return set_error(MOE_EINVAL, "hotness of expert %d is NaN", e);
  const size_t lo = bytes_per_tier[lo_tier], hi = bytes_per_tier[hi_tier];
  if (lo > budget_bytes / (size_t)n_experts || (size_t)n_experts * lo > budget_bytes)
    return set_error(MOE_ENOSPC, "%d experts at the low tier need %zu bytes, budget %zu", n_experts,
                     (size_t)n_experts * lo, budget_bytes);
  // top-n: experts ranked by hotness (descending, ties to the lower id); the
  // n hottest take the high tier, n the largest that fits the budget
  int order[kMaxExperts];
  for (int e = 0; e < n_experts; ++e) order[e] = e;
  for (int i = 1; i < n_experts; ++i) {   // insertion sort: stable, so ties keep the lower id first
    const int e = order[i];
    int j = i - 1;
    while (j >= 0 && hot[order[j]] < hot[e]) {
      order[j + 1] = order[j];
      --j;
    }
    order[j + 1] = e;
  }
  const size_t spare = budget_bytes - (size_t)n_experts * lo;
  int n_hi = 0;
  if (hi <= lo)
    n_hi = n_experts;
  else
    n_hi = (int)((spare / (hi - lo)) < (size_t)n_experts ? spare / (hi - lo) : (size_t)n_experts);
  for (int e = 0; e < n_experts; ++e) tiers_out[e] = lo_tier;
  for (int i = 0; i < n_hi; ++i) tiers_out[order[i]] = hi_tier;
  if (n_hi_out) *n_hi_out = n_hi;
  return MOE_OK;
}

int moe_layer_destroy(moe_layer_t layer) {
  g_err[0] = 0;
  Layer* L = reinterpret_cast<Layer*>(layer);
  if (!L) return set_error(MOE_EINVAL, "null layer");
  int rc = check_hip(hipFree(L->table), "hipFree(table)");
  const int rc2 = check_hip(hipFree(L->slots), "hipFree(slots)");
  const int rc3 = check_hip(hipFree(L->slot_map), "hipFree(slot_map)");
  delete[] L->slot_set;
  delete L;
  return rc ? rc : rc2 ? rc2 : rc3;
}

int moe_layer_plan(moe_layer_t layer, int32_t T, int32_t* path, int32_t* tile_rows,
                   int32_t* down_path, int32_t* down_tile_rows) {
  g_err[0] = 0;
  const Layer* L = reinterpret_cast<const Layer*>(layer);
  if (!L || !path || !tile_rows) return set_error(MOE_EINVAL, "null pointer");
  if (T < 0 || T > (1 << 24)) return set_error(MOE_ESHAPE, "bad token count %d", T);
  const GemmPlan gp = plan_gemm(*L, T);
  *path = gp.kind;
  *tile_rows = gp.bm13;
  if (down_path) *down_path = gp.kind2;
  if (down_tile_rows) *down_tile_rows = gp.bm2;
  return MOE_OK;
}

size_t moe_workspace_size(moe_layer_t layer, int32_t T) {
  const Layer* L = reinterpret_cast<const Layer*>(layer);
  if (!L || T < 0) return 0;
  const GemmPlan gp = plan_gemm(*L, T);
  return plan_workspace(*L, T, gp).total;
}

int moe_layer_set_stage_events(moe_layer_t layer, void* const* events, int32_t n) {
  g_err[0] = 0;
  Layer* L = reinterpret_cast<Layer*>(layer);
  if (!L) return set_error(MOE_EINVAL, "null layer");
  if (n != 0 && n != 7 && n != 9) return set_error(MOE_EINVAL, "need 0, 7 or 9 events (got %d)", n);
  if (n && !events) return set_error(MOE_EINVAL, "null events");
  for (int i = 0; i < n; ++i) {
    if (!events[i]) return set_error(MOE_EINVAL, "null event %d", i);
    L->stage_events[i] = events[i];
  }
  L->n_stage_events = n;
  return MOE_OK;
}

int moe_layer_set_router_mode(moe_layer_t layer, int32_t mode) {
  g_err[0] = 0;
  Layer* L = reinterpret_cast<Layer*>(layer);
  if (!L) return set_error(MOE_EINVAL, "null layer");
  if (mode != MOE_ROUTER_AUTO && mode != MOE_ROUTER_CANONICAL && mode != MOE_ROUTER_MFMA)
    return set_error(MOE_EINVAL, "bad router mode %d", mode);
  L->router_mode = mode;
  return MOE_OK;
}

}  // extern "C"

namespace {

// gemm: the call runs the grouped GEMMs (a forward), not only the routing.
int check_common(const Layer* L, const uint16_t* x, const uint16_t* wr, int32_t T, void* ws,
                 size_t ws_bytes, WsPlan* plan, GemmPlan* gp, bool gemm) {
  if (!L) return set_error(MOE_EINVAL, "null layer");
  if (T < 0 || T > (1 << 24)) return set_error(MOE_ESHAPE, "bad token count %d", T);
  if ((size_t)T * L->k > (size_t)1 << 28) return set_error(MOE_ESHAPE, "too many routes");
  if (T > 0 && (!x || !wr || !ws)) return set_error(MOE_EINVAL, "null pointer");
  if (T > 0 && (!aligned(x, 16) || !aligned(wr, 16)))
    return set_error(MOE_EINVAL, "x and wr must be 16-byte aligned");
  if (T > 0 && !aligned(ws, kBlobAlign))
    return set_error(MOE_EINVAL, "workspace must be 256-byte aligned");
  *gp = plan_gemm(*L, T);
  // The large-batch GEMMs read their 16-bit activations (x [T, H] and the
  // SwiGLU output [T k, I]) through 32-bit buffer records and offsets, so each
  // array must stay below 4 GiB; larger batches are split by the caller.
  if (gemm && (gp->kind == kGemmPrefill || gp->kind2 == kGemmPrefill) &&
      ((uint64_t)T * L->H * 2 > 0xffffffffull || (uint64_t)T * L->k * L->I * 2 > 0xffffffffull))
    return set_error(MOE_ESHAPE,
                     "%d tokens: the large-batch path needs T*H*2 and T*k*I*2 below 4 GiB "
                     "(H %d, k %d, I %d); split the batch",
                     T, L->H, L->k, L->I);
  *plan = plan_workspace(*L, T, *gp);
  if (T > 0 && ws_bytes < plan->total)
    return set_error(MOE_ENOSPC, "workspace has %zu bytes, %zu needed", ws_bytes, plan->total);
  return MOE_OK;
}

// Optional per-stage timing events (moe_layer_set_stage_events).
struct Stages {
  const Layer* L;
  hipStream_t s;
  bool on;
  void rec(int i) const {
    if (on && L->n_stage_events >= 7)
      (void)hipEventRecord(reinterpret_cast<hipEvent_t>(L->stage_events[i]), s);
  }
  // events 7 and 8: the gate/up GEMM kernel's own start and end
  KernelTimer gate_up_timer() const {
    if (on && L->n_stage_events == 9)
      return KernelTimer{reinterpret_cast<hipEvent_t>(L->stage_events[7]),
                         reinterpret_cast<hipEvent_t>(L->stage_events[8])};
    return KernelTimer{nullptr, nullptr};
  }
};

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

hipError_t enqueue_route(const Layer& L, WaveMap wave, Hotness hotness, const WsPlan& p, const GemmPlan& gp, const uint16_t* x,
                         const uint16_t* wr, const float* bias, int T, float* logits,
                         int32_t* ids, float* w, int32_t* offsets, int32_t* sorted, int32_t* pos,
                         float* r13, void* ws, const Stages& st, bool reuse_topk = false) {
  st.rec(0);
  hipError_t e = hipSuccess;
  // Many tokens, logits not wanted (null): logits on MFMA, the top k taken
  // from the candidates the error bound leaves, recomputed in the canonical
  // order (the same routing bit for bit, see router_certified.hip).
  if (!reuse_topk && !logits && use_certified_router(L.router_mode, T, L.E, L.H)) {
    e = launch_router_certified(x, wr, bias, T, L.H, L.E, L.k, at<float>(ws, p.logits),
                                at<float>(ws, p.xn2), at<float>(ws, p.wn2), ids, w, st.s);
    // the decode GEMMs' group sums, which the fixed-order kernel would write
    if (e == hipSuccess && r13) e = launch_group_sums(x, T, L.H, r13, st.s);
    if (e != hipSuccess) return e;
    st.rec(1);
  } else if (!reuse_topk && !logits && use_small_router(T, L.E, L.H)) {
    // few tokens: logits, group sums and top k in one launch
    e = launch_router_topk_small(x, wr, bias, T, L.H, L.E, L.k, r13, ids, w, st.s);
    if (e != hipSuccess) return e;
    st.rec(1);
  } else {
    float* z = logits ? logits : at<float>(ws, p.logits);
    if (!reuse_topk) {   // later waves of a layer call keep the first wave's routing
      e = launch_router_logits(x, wr, bias, T, L.H, L.E, z, r13, st.s);
      if (e != hipSuccess) return e;
    }
    st.rec(1);
    if (!reuse_topk) {
      e = launch_topk(z, T, L.E, L.k, ids, w, st.s);
      if (e != hipSuccess) return e;
    }
  }
  st.rec(2);
  return launch_permute(L.table, wave, hotness, ids, T, L.k, L.E, offsets, sorted, pos, at<TileEntry>(ws, p.tiles13),
                        at<int32_t>(ws, p.ntiles13), gp.bm13, at<TileEntry>(ws, p.tiles2),
                        at<int32_t>(ws, p.ntiles2), gp.bm2, at<int32_t>(ws, p.rank),
                        at<int32_t>(ws, p.chunk_counts), at<int32_t>(ws, p.chunk_tot), st.s);
}

}  // namespace

namespace {

int forward_impl(const Layer* L, WaveMap wave, bool accumulate, const uint16_t* x,
                        const uint16_t* wr, const float* bias, int32_t T, void* y, int y_dtype,
                        void* ws, size_t ws_bytes, void* stream) {
  WsPlan p;
  GemmPlan gp;
  int rc = check_common(L, x, wr, T, ws, ws_bytes, &p, &gp, true);
  if (rc) return rc;
  if (y_dtype != MOE_DTYPE_BF16 && y_dtype != MOE_DTYPE_F32)
    return set_error(MOE_EINVAL, "bad y_dtype %d", y_dtype);
  if (accumulate && y_dtype != MOE_DTYPE_F32)
    return set_error(MOE_EINVAL, "accumulating needs an fp32 y");
  if (T == 0) return MOE_OK;
  if (!y || !aligned(y, 16)) return set_error(MOE_EINVAL, "y must be non-null and 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const Stages st{L, s, true};
  const bool prefill = gp.kind == kGemmPrefill;     // the gate/up GEMM's family
  const bool prefill2 = gp.kind2 == kGemmPrefill;   // the down GEMM's
  // a large-batch down GEMM reads fp16 activations, which only the
  // large-batch gate/up GEMM writes (plan_gemm never pairs it otherwise)
  if (prefill2 && !prefill) return set_error(MOE_EINVAL, "unsupported GEMM plan");
  // the hotness trace counts each layer call once: a plain forward, or the
  // first wave of a layer call (the one that does not accumulate)
  const Hotness hotness{accumulate ? nullptr : L->hot, L->hot_decay};
  hipError_t e = enqueue_route(*L, wave, hotness, p, gp, x, wr, bias, T, nullptr,
                               at<int32_t>(ws, p.ids), at<float>(ws, p.weights),
                               at<int32_t>(ws, p.offsets), at<int32_t>(ws, p.sorted),
                               at<int32_t>(ws, p.pos), prefill ? nullptr : at<float>(ws, p.r13),
                               ws, st, wave.slot_map != nullptr && accumulate);
  if (e != hipSuccess) return check_hip(e, "route launch");
  st.rec(3);
  if (prefill) {
    e = launch_x_to_f16(x, at<uint16_t>(ws, p.x16), (size_t)T * L->H, s);
    if (e == hipSuccess)
      e = launch_prefill(true, *L, T, at<uint16_t>(ws, p.x16), at<int32_t>(ws, p.sorted),
                         at<TileEntry>(ws, p.tiles13), at<int32_t>(ws, p.ntiles13), p.max_tiles13,
                         at<uint16_t>(ws, p.act), prefill2 ? nullptr : at<float>(ws, p.r2), nullptr,
                         nullptr, s, st.gate_up_timer());
  } else {
    e = launch_gemm13(*L, gp, T, x, at<int32_t>(ws, p.sorted), at<TileEntry>(ws, p.tiles13),
                      at<int32_t>(ws, p.ntiles13), p.max_tiles13, at<float>(ws, p.r13),
                      at<uint16_t>(ws, p.act), at<float>(ws, p.r2), s, st.gate_up_timer());
  }
  if (e != hipSuccess) return check_hip(e, "gate/up GEMM launch");
  st.rec(4);
  if (prefill2) {
    e = launch_prefill(false, *L, T, at<uint16_t>(ws, p.act), at<int32_t>(ws, p.sorted),
                       at<TileEntry>(ws, p.tiles2), at<int32_t>(ws, p.ntiles2), p.max_tiles2,
                       nullptr, nullptr, at<float>(ws, p.weights), at<float>(ws, p.rows), s);
  } else {
    e = launch_gemm2(*L, gp, T, at<uint16_t>(ws, p.act), at<int32_t>(ws, p.sorted),
                     at<float>(ws, p.weights), at<TileEntry>(ws, p.tiles2),
                     at<int32_t>(ws, p.ntiles2), p.max_tiles2, at<float>(ws, p.r2),
                     at<float>(ws, p.rows), s);
  }
  if (e != hipSuccess) return check_hip(e, "down GEMM launch");
  st.rec(5);
  e = launch_combine(at<float>(ws, p.rows), at<int32_t>(ws, p.ids), wave.slot_map, T, L->H, L->k,
                     y, y_dtype, accumulate, s);
  if (e != hipSuccess) return check_hip(e, "combine launch");
  st.rec(6);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_route(moe_layer_t layer, const uint16_t* x, const uint16_t* wr, const float* bias,
              int32_t T, int32_t* topk_ids, float* topk_w, float* logits, int32_t* expert_offsets,
              int32_t* sorted_routes, int32_t* route_pos, void* ws, size_t ws_bytes,
              void* stream) {
  g_err[0] = 0;
  const Layer* L = reinterpret_cast<const Layer*>(layer);
  WsPlan p;
  GemmPlan gp;
  int rc = check_common(L, x, wr, T, ws, ws_bytes, &p, &gp, false);
  if (rc) return rc;
  if (!expert_offsets || (T > 0 && (!topk_ids || !topk_w || !sorted_routes || !route_pos)))
    return set_error(MOE_EINVAL, "null output pointer");
  if (!aligned(expert_offsets, 4)) return set_error(MOE_EINVAL, "expert_offsets must be 4-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // no tokens: all offsets are zero (a fill kernel, not a memset node, so a
  // captured graph replays it correctly)
  if (T == 0)
    return check_hip(launch_fill_zero(expert_offsets, sizeof(int32_t) * (L->E + 1), s),
                     "fill(offsets)");
  const Stages st{L, s, false};
  const hipError_t e = enqueue_route(*L, WaveMap{nullptr, nullptr}, Hotness{nullptr, 1.0f}, p, gp,
                                     x, wr, bias, T, logits, topk_ids, topk_w,
                                     expert_offsets, sorted_routes, route_pos, nullptr, ws, st);
  return check_hip(e, "route launch");
}

int moe_layer_forward(moe_layer_t layer, const uint16_t* x, const uint16_t* wr, const float* bias,
                      int32_t T, void* y, int y_dtype, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  return forward_impl(reinterpret_cast<const Layer*>(layer), WaveMap{nullptr, nullptr}, false, x,
                      wr, bias, T, y, y_dtype, ws, ws_bytes, stream);
}

int moe_layer_forward_wave(moe_layer_t layer, const uint16_t* x, const uint16_t* wr,
                           const float* bias, int32_t T, void* y, int y_dtype, int accumulate,
                           void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  const Layer* L = reinterpret_cast<const Layer*>(layer);
  if (!L) return set_error(MOE_EINVAL, "null layer");
  if (accumulate != 0 && accumulate != 1) return set_error(MOE_EINVAL, "accumulate must be 0 or 1");
  return forward_impl(L, WaveMap{L->slot_map, L->slots}, accumulate == 1, x, wr, bias, T, y,
                      y_dtype, ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free forward.  Its workspace is `scratch`, a file-scope device
// array (one per GPU, held by the loaded library until the process ends).  In
// host code the array's name only stands in for it; its device address on
// each GPU comes from hipGetSymbolAddress, asked once per device with that
// device current, and only that address is ever handed to kernels.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (set up on its first use
// there).
int scratch_address(void** out) {
  int dev = -1;
  int rc = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (rc) return rc;
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(MOE_EINVAL, "device %d: the allocation-free forward serves devices 0..%d", dev,
                     kMaxDevices - 1);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      rc = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
      if (rc) return rc;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" int moe_layer_forward_noalloc(moe_layer_t layer, const uint16_t* x, const uint16_t* wr,
                                         const float* bias, int32_t T, void* y, int y_dtype,
                                         void* stream) {
  g_err[0] = 0;
  const Layer* L = reinterpret_cast<const Layer*>(layer);
  if (!L) return set_error(MOE_EINVAL, "null layer");
  if (T < 0 || T > (1 << 24)) return set_error(MOE_ESHAPE, "bad token count %d", T);
  const size_t need = moe_workspace_size(layer, T);
  if (need > kScratchBytes)
    return set_error(MOE_ENOSPC,
                     "%d tokens need %zu bytes of workspace; the allocation-free forward has a "
                     "fixed scratch of %zu bytes per device (use moe_layer_forward with a "
                     "workspace, or fewer tokens per call)",
                     T, need, kScratchBytes);
  if (T == 0)
    return forward_impl(L, WaveMap{nullptr, nullptr}, false, x, wr, bias, T, y, y_dtype, nullptr, 0,
                        stream);
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  // every workspace region a forward reads is written earlier in the same
  // forward, so nothing needs clearing between calls
  return forward_impl(L, WaveMap{nullptr, nullptr}, false, x, wr, bias, T, y, y_dtype, ws,
                      kScratchBytes, stream);
}
