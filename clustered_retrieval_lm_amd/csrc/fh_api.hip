// C ABI of the FlashHead library: host-side validation and dispatch to the kernel
// launchers.  The declarations, argument meanings and error behaviour are in
// include/flashhead.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/flashhead.h"
#include "fh_device.h"
#include "fh_internal.h"

namespace {

thread_local std::string g_last_error;

fh_status fail(fh_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fh_status hip_fail(hipError_t e, const char* what) {
  return fail(FH_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxC = 32768;
constexpr int64_t kMaxB = 65535;
constexpr int64_t kMaxTile = 256;
constexpr int64_t kMaxSets = (int64_t(1) << 31) - 1;

int fmt_of(int32_t dt) { return dt == FH_F32 ? fh::RF_F32 : dt == FH_BF16 ? fh::RF_BF16 : fh::RF_INT4; }

// Checks shared by every entry point that takes a desc.
fh_status check_desc(const fh_desc* d, bool need_tiles) {
  if (!d) return fail(FH_ERR_ARG, "desc is NULL");
  if (d->reserved != 0) return fail(FH_ERR_ARG, "desc.reserved must be 0");
  if (d->B < 1 || d->d < 1 || d->V < 1 || d->c < 1)
    return fail(FH_ERR_SHAPE, "B, d, V and c must be >= 1 (B=%lld d=%lld V=%lld c=%lld)",
                (long long)d->B, (long long)d->d, (long long)d->V, (long long)d->c);
  if (d->B > kMaxB) return fail(FH_ERR_UNSUPPORTED, "B=%lld exceeds %lld", (long long)d->B, (long long)kMaxB);
  if (d->V >= (int64_t(1) << 31)) return fail(FH_ERR_UNSUPPORTED, "V must be < 2^31");
  if (d->V % d->c != 0)
    return fail(FH_ERR_SHAPE, "c=%lld does not divide V=%lld (clusters must have equal size)",
                (long long)d->c, (long long)d->V);
  if (d->h_dtype != FH_F32 && d->h_dtype != FH_BF16) return fail(FH_ERR_DTYPE, "h_dtype must be F32 or BF16");
  if (d->c_dtype != FH_F32 && d->c_dtype != FH_BF16 && d->c_dtype != FH_INT4_G128)
    return fail(FH_ERR_DTYPE, "c_dtype must be F32, BF16 or INT4_G128");
  if (d->c_dtype == FH_INT4_G128 && d->d % 128 != 0)
    return fail(FH_ERR_SHAPE, "int4 centroids need d %% 128 == 0 (d=%lld)", (long long)d->d);
  if (d->e_dtype != FH_F32 && d->e_dtype != FH_BF16 && d->e_dtype != FH_INT4_G128)
    return fail(FH_ERR_DTYPE, "e_dtype must be F32, BF16 or INT4_G128");
  if (d->d % 8 != 0) return fail(FH_ERR_SHAPE, "d=%lld must be a multiple of 8", (long long)d->d);
  const int64_t b = d->V / d->c;
  if (need_tiles) {
    if (b > kMaxTile) return fail(FH_ERR_UNSUPPORTED, "cluster size b=%lld exceeds %lld", (long long)b, (long long)kMaxTile);
    if (d->c > kMaxC) return fail(FH_ERR_UNSUPPORTED, "c=%lld exceeds %lld", (long long)d->c, (long long)kMaxC);
  }
  if (d->e_dtype == FH_INT4_G128 && d->d % 128 != 0)
    return fail(FH_ERR_SHAPE, "int4 token embeddings need d %% 128 == 0 (d=%lld)", (long long)d->d);
  auto fits = [&](int32_t dt) {
    const int f = fmt_of(dt);
    return fh::chunk_slots(f, (int)d->d) <= fh::max_chunk_slots(f);
  };
  if (d->d > 16384 || !fits(d->c_dtype) || !fits(d->e_dtype))
    return fail(FH_ERR_UNSUPPORTED, "d=%lld too large for these dtypes (bf16 <= 4096, f32 <= 2048, int4 <= 8192)",
                (long long)d->d);
  return FH_OK;
}

fh_status check_sampling(int32_t mode, float tau) {
  if (mode != FH_GREEDY && mode != FH_SAMPLE) return fail(FH_ERR_ARG, "mode must be FH_GREEDY or FH_SAMPLE");
  if (mode == FH_SAMPLE && !(tau > 0.f && std::isfinite(tau)))
    return fail(FH_ERR_ARG, "temperature must be finite and > 0 when sampling (got %g)", (double)tau);
  return FH_OK;
}

fh_status check_p(const fh_desc* d, int64_t p) {
  if (p < 1 || p > d->c) return fail(FH_ERR_ARG, "p=%lld must satisfy 1 <= p <= c=%lld", (long long)p, (long long)d->c);
  return FH_OK;
}

fh_status check_ws(const fh_desc* d, int64_t p, void* ws, size_t ws_bytes, fh::Workspace* out) {
  const fh::Workspace need = fh::carve_workspace(nullptr, (int)d->B, (int)d->c, (int)p);
  if (!ws) return fail(FH_ERR_WORKSPACE, "workspace is NULL");
  if (ws_bytes < need.bytes)
    return fail(FH_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes, need.bytes);
  *out = fh::carve_workspace(ws, (int)d->B, (int)d->c, (int)p);
  return FH_OK;
}

fh::HeadShape shape_of(const fh_desc* d) {
  fh::HeadShape s;
  s.B = (int)d->B;
  s.d = (int)d->d;
  s.c = (int)d->c;
  s.b = (int)(d->V / d->c);
  s.h_bf16 = d->h_dtype == FH_BF16;
  s.c_fmt = fmt_of(d->c_dtype);
  s.e_fmt = fmt_of(d->e_dtype);
  return s;
}

fh::Sampling sampling_of(int32_t mode, float tau, uint64_t seed, uint64_t step) {
  return fh::Sampling{mode == FH_SAMPLE ? 1 : 0, tau, seed, step};
}

// Scratch of flashhead_forward_noalloc: a workspace the library owns, one copy per device, held
// until the process ends.  The array's name is a host-side stand-in; kernels get the device
// address that hipGetSymbolAddress returns for the current device (kept in g_scratch_ptr).
constexpr size_t kStaticScratchBytes = size_t(4) << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fh_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FH_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FH_OK;
}

}  // namespace

extern "C" {

const char* flashhead_version(void) { return "flashhead 0.1.0 gfx950"; }

const char* flashhead_last_error(void) { return g_last_error.c_str(); }

fh_status flashhead_workspace_bytes(const fh_desc* desc, int64_t p, size_t* bytes) {
  fh_status st = check_desc(desc, true);
  if (st != FH_OK) return st;
  if ((st = check_p(desc, p)) != FH_OK) return st;
  if (!bytes) return fail(FH_ERR_ARG, "bytes is NULL");
  *bytes = fh::carve_workspace(nullptr, (int)desc->B, (int)desc->c, (int)p).bytes;
  return FH_OK;
}

fh_status flashhead_pack(const fh_desc* desc, int32_t src_dtype, const void* E, const int32_t* cluster_tokens,
                         void* E_tiles, void* E_scales, void* stream) {
  fh_status st = check_desc(desc, false);
  if (st != FH_OK) return st;
  if (src_dtype != FH_F32 && src_dtype != FH_BF16) return fail(FH_ERR_DTYPE, "src_dtype must be F32 or BF16");
  if (!E || !cluster_tokens || !E_tiles) return fail(FH_ERR_ARG, "E, cluster_tokens and E_tiles must be non-NULL");
  const bool int4 = desc->e_dtype == FH_INT4_G128;
  if (int4 && !E_scales) return fail(FH_ERR_ARG, "E_scales must be non-NULL for INT4_G128");
  if (!int4 && E_scales) return fail(FH_ERR_ARG, "E_scales must be NULL unless e_dtype is INT4_G128");
  hipStream_t s = (hipStream_t)stream;
  const int V = (int)desc->V;
  uint32_t* tmp = nullptr;   // counts[V], the empty-slot count, the error flags
  hipError_t e = hipMalloc(&tmp, (size_t)(V + 2) * sizeof(uint32_t));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc");
  e = hipMemsetAsync(tmp, 0, (size_t)(V + 2) * sizeof(uint32_t), s);
  if (e == hipSuccess)
    e = fh::launch_pack(V, (int)desc->d, (int)desc->c, (int)(desc->V / desc->c), src_dtype == FH_BF16,
                        fmt_of(desc->e_dtype), E, cluster_tokens, E_tiles, (uint16_t*)E_scales, tmp,
                        tmp + V + 1, s);
  uint32_t bad = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&bad, tmp + V + 1, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  hipError_t e2 = hipFree(tmp);
  if (e != hipSuccess) return hip_fail(e, "flashhead_pack");
  if (e2 != hipSuccess) return hip_fail(e2, "hipFree");
  if (bad)
    return fail(FH_ERR_ARG, "cluster_tokens must hold the tokens 0 .. n-1 once each and -1 in its other slots");
  return FH_OK;
}

fh_status flashhead_centroids(const fh_desc* desc, int32_t src_dtype, const void* E, const int32_t* cluster_tokens,
                              int32_t unit, void* centroids, void* stream) {
  fh_status st = check_desc(desc, false);
  if (st != FH_OK) return st;
  if (src_dtype != FH_F32 && src_dtype != FH_BF16) return fail(FH_ERR_DTYPE, "src_dtype must be F32 or BF16");
  if (unit != 0 && unit != 1) return fail(FH_ERR_ARG, "unit must be 0 or 1");
  if (!E || !cluster_tokens || !centroids) return fail(FH_ERR_ARG, "E, cluster_tokens and centroids must be non-NULL");
  if (desc->V / desc->c > kMaxTile)
    return fail(FH_ERR_UNSUPPORTED, "cluster size b=%lld exceeds %lld", (long long)(desc->V / desc->c), (long long)kMaxTile);
  const int c = (int)desc->c, d = (int)desc->d, b = (int)(desc->V / desc->c);
  hipStream_t hs = (hipStream_t)stream;
  if (desc->c_dtype != FH_INT4_G128) {
    hipError_t e = fh::launch_centroids(d, c, b, src_dtype == FH_BF16, desc->c_dtype == FH_BF16, unit, E,
                                        cluster_tokens, centroids, hs);
    if (e != hipSuccess) return hip_fail(e, "centroids launch");
    return FH_OK;
  }
  // int4: the bf16 centroids, quantised per group of 128 (a temporary bf16 copy)
  uint16_t* tmp = nullptr;
  hipError_t e = hipMalloc(&tmp, (size_t)c * d * sizeof(uint16_t));
  if (e != hipSuccess) return hip_fail(e, "hipMalloc");
  e = fh::launch_centroids(d, c, b, src_dtype == FH_BF16, 1, unit, E, cluster_tokens, tmp, hs);
  if (e == hipSuccess)
    e = fh::launch_quant_int4_rows(tmp, c, d, (uint8_t*)centroids,
                                   (uint16_t*)((char*)centroids + fh::int4_scales_offset(c, d)), hs);
  if (e == hipSuccess) e = hipStreamSynchronize(hs);
  hipError_t e2 = hipFree(tmp);
  if (e != hipSuccess) return hip_fail(e, "int4 centroids");
  if (e2 != hipSuccess) return hip_fail(e2, "hipFree");
  return FH_OK;
}

fh_status flashhead_centroids_bytes(const fh_desc* desc, size_t* bytes) {
  fh_status st = check_desc(desc, false);
  if (st != FH_OK) return st;
  if (!bytes) return fail(FH_ERR_ARG, "bytes is NULL");
  const size_t c = (size_t)desc->c, d = (size_t)desc->d;
  *bytes = desc->c_dtype == FH_F32 ? c * d * 4 : desc->c_dtype == FH_BF16 ? c * d * 2 : fh::int4_rows_bytes(c, d);
  return FH_OK;
}

static fh_status check_clusters_args(const fh_desc* desc, int32_t src_dtype) {
  fh_status st = check_desc(desc, false);
  if (st != FH_OK) return st;
  if (desc->c_dtype == FH_INT4_G128)
    return fail(FH_ERR_DTYPE, "build_clusters stores F32 or BF16 centroids (quantise with flashhead_centroids)");
  if (src_dtype != FH_F32 && src_dtype != FH_BF16) return fail(FH_ERR_DTYPE, "src_dtype must be F32 or BF16");
  if (desc->c > kMaxC) return fail(FH_ERR_UNSUPPORTED, "c=%lld exceeds %lld", (long long)desc->c, (long long)kMaxC);
  if (desc->V / desc->c > kMaxTile)
    return fail(FH_ERR_UNSUPPORTED, "cluster size b=%lld exceeds %lld", (long long)(desc->V / desc->c),
                (long long)kMaxTile);
  return FH_OK;
}

fh_status flashhead_build_clusters_workspace_bytes(const fh_desc* desc, int32_t src_dtype, size_t* bytes) {
  fh_status st = check_clusters_args(desc, src_dtype);
  if (st != FH_OK) return st;
  if (!bytes) return fail(FH_ERR_ARG, "bytes is NULL");
  *bytes = fh::build_clusters_workspace_bytes((int)desc->V, (int)desc->d, (int)desc->c);
  return FH_OK;
}

fh_status flashhead_build_clusters(const fh_desc* desc, int32_t src_dtype, const void* E, int32_t iters,
                                   uint64_t seed, int32_t unit, void* centroids, int32_t* cluster_tokens,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  fh_status st = check_clusters_args(desc, src_dtype);
  if (st != FH_OK) return st;
  if (iters < 1 || iters > 100000) return fail(FH_ERR_ARG, "iters=%d must be in [1, 100000]", (int)iters);
  if (unit != 0 && unit != 1) return fail(FH_ERR_ARG, "unit must be 0 or 1");
  if (!E || !centroids || !cluster_tokens) return fail(FH_ERR_ARG, "E, centroids and cluster_tokens must be non-NULL");
  const size_t need = fh::build_clusters_workspace_bytes((int)desc->V, (int)desc->d, (int)desc->c);
  if (!workspace || workspace_bytes < need)
    return fail(FH_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  hipError_t e = fh::launch_build_clusters((int)desc->V, (int)desc->d, (int)desc->c, src_dtype == FH_BF16, E, iters,
                                           seed, unit, desc->c_dtype == FH_BF16, centroids, cluster_tokens, workspace,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "build_clusters");
  return FH_OK;
}

fh_status flashhead_centroid_scores(const fh_desc* desc, const void* h, const void* centroids, int32_t mode,
                                    float temperature, uint64_t seed, uint64_t step, void* workspace,
                                    size_t workspace_bytes, float* keys_out, void* stream) {
  fh_status st = check_desc(desc, true);
  if (st != FH_OK) return st;
  if ((st = check_sampling(mode, temperature)) != FH_OK) return st;
  if (!h || !centroids) return fail(FH_ERR_ARG, "h and centroids must be non-NULL");
  fh::Workspace ws;
  if ((st = check_ws(desc, 1, workspace, workspace_bytes, &ws)) != FH_OK) return st;
  hipError_t e = fh::launch_scores(shape_of(desc), h, centroids, sampling_of(mode, temperature, seed, step), ws,
                                   keys_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "centroid scores launch");
  return FH_OK;
}

fh_status flashhead_select_probes(const fh_desc* desc, int64_t p, void* workspace, size_t workspace_bytes,
                                  int32_t* probe_ids_out, void* stream) {
  fh_status st = check_desc(desc, true);
  if (st != FH_OK) return st;
  if ((st = check_p(desc, p)) != FH_OK) return st;
  fh::Workspace ws;
  if ((st = check_ws(desc, p, workspace, workspace_bytes, &ws)) != FH_OK) return st;
  // the B > 1 per-cluster state starts cleared whatever ran on this workspace before
  hipError_t e = fh::launch_clear_select(ws, (int)desc->c, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "selection state reset");
  e = fh::launch_select(shape_of(desc), (int)p, ws, probe_ids_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "probe selection launch");
  return FH_OK;
}

static fh_status check_tiles_args(const fh_desc* desc, const void* h, const int32_t* c2t, const void* tiles,
                                  const void* scales, const fh_outputs* out) {
  if (!h || !c2t || !tiles) return fail(FH_ERR_ARG, "h, cluster_tokens and E_tiles must be non-NULL");
  const bool int4 = desc->e_dtype == FH_INT4_G128;
  if (int4 && !scales) return fail(FH_ERR_ARG, "E_scales must be non-NULL for INT4_G128");
  if (!out || !out->token) return fail(FH_ERR_ARG, "out and out->token must be non-NULL");
  return FH_OK;
}

fh_status flashhead_probe_logits(const fh_desc* desc, int64_t p, const void* h, const int32_t* cluster_tokens,
                                 const void* E_tiles, const void* E_scales, int32_t mode, float temperature,
                                 uint64_t seed, uint64_t step, void* workspace, size_t workspace_bytes,
                                 const fh_outputs* out, void* stream) {
  fh_status st = check_desc(desc, true);
  if (st != FH_OK) return st;
  if ((st = check_p(desc, p)) != FH_OK) return st;
  if ((st = check_sampling(mode, temperature)) != FH_OK) return st;
  if ((st = check_tiles_args(desc, h, cluster_tokens, E_tiles, E_scales, out)) != FH_OK) return st;
  fh::Workspace ws;
  if ((st = check_ws(desc, p, workspace, workspace_bytes, &ws)) != FH_OK) return st;
  hipError_t e = fh::launch_tiles(shape_of(desc), (int)p, h, cluster_tokens, E_tiles, (const uint16_t*)E_scales,
                                  sampling_of(mode, temperature, seed, step), ws, out->probe_logits,
                                  out->probe_tokens, out->token, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "probe logits launch");
  return FH_OK;
}

// Probe selection and stage 2: at B = 1 one fused kernel, else the select and tile kernels.
static fh_status select_and_probe(const fh::HeadShape& s, int p, const void* h, const int32_t* c2t,
                                  const void* tiles, const void* scales, const fh::Sampling& smp,
                                  const fh::Workspace& ws, const fh_outputs* out, bool state_clear,
                                  hipStream_t hs) {
  hipError_t e;
  if (s.B == 1) {
    e = fh::launch_stage2_b1(s, p, h, c2t, tiles, (const uint16_t*)scales, smp, ws, out->probe_ids,
                             out->probe_logits, out->probe_tokens, out->token, hs);
    if (e != hipSuccess) return hip_fail(e, "fused selection and probe logits launch");
    return FH_OK;
  }
  if (!state_clear) {           // no stage-1 launch of this call cleared the per-cluster state
    e = fh::launch_clear_select(ws, s.c, hs);
    if (e != hipSuccess) return hip_fail(e, "selection state reset");
  }
  e = fh::launch_select(s, p, ws, out->probe_ids, hs);
  if (e != hipSuccess) return hip_fail(e, "probe selection launch");
  e = fh::launch_tiles(s, p, h, c2t, tiles, (const uint16_t*)scales, smp, ws, out->probe_logits, out->probe_tokens,
                       out->token, hs);
  if (e != hipSuccess) return hip_fail(e, "probe logits launch");
  return FH_OK;
}

fh_status flashhead_select_and_probe(const fh_desc* desc, int64_t p, const void* h, const int32_t* cluster_tokens,
                                     const void* E_tiles, const void* E_scales, int32_t mode, float temperature,
                                     uint64_t seed, uint64_t step, void* workspace, size_t workspace_bytes,
                                     const fh_outputs* out, void* stream) {
  fh_status st = check_desc(desc, true);
  if (st != FH_OK) return st;
  if ((st = check_p(desc, p)) != FH_OK) return st;
  if ((st = check_sampling(mode, temperature)) != FH_OK) return st;
  if ((st = check_tiles_args(desc, h, cluster_tokens, E_tiles, E_scales, out)) != FH_OK) return st;
  fh::Workspace ws;
  if ((st = check_ws(desc, p, workspace, workspace_bytes, &ws)) != FH_OK) return st;
  return select_and_probe(shape_of(desc), (int)p, h, cluster_tokens, E_tiles, E_scales,
                          sampling_of(mode, temperature, seed, step), ws, out, false, (hipStream_t)stream);
}

// The forward path of flashhead_forward and flashhead_forward_noalloc on a carved workspace.
static fh_status forward_on(const fh_desc* desc, const void* h, const void* centroids, const int32_t* cluster_tokens,
                            const void* E_tiles, const void* E_scales, int64_t p, int32_t mode, float temperature,
                            uint64_t seed, uint64_t step, const fh::Workspace& ws, const fh_outputs* out,
                            void* stream) {
  const fh::HeadShape s = shape_of(desc);
  const fh::Sampling smp = sampling_of(mode, temperature, seed, step);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = fh::launch_scores(s, h, centroids, smp, ws, nullptr, hs);
  if (e != hipSuccess) return hip_fail(e, "centroid scores launch");
  return select_and_probe(s, (int)p, h, cluster_tokens, E_tiles, E_scales, smp, ws, out, true, hs);
}

static fh_status check_forward_args(const fh_desc* desc, const void* h, const void* centroids,
                                    const int32_t* cluster_tokens, const void* E_tiles, const void* E_scales, int64_t p,
                                    int32_t mode, float temperature, const fh_outputs* out) {
  fh_status st = check_desc(desc, true);
  if (st != FH_OK) return st;
  if ((st = check_p(desc, p)) != FH_OK) return st;
  if ((st = check_sampling(mode, temperature)) != FH_OK) return st;
  if (!centroids) return fail(FH_ERR_ARG, "centroids must be non-NULL");
  return check_tiles_args(desc, h, cluster_tokens, E_tiles, E_scales, out);
}

fh_status flashhead_forward(const fh_desc* desc, const void* h, const void* centroids, const int32_t* cluster_tokens,
                            const void* E_tiles, const void* E_scales, int64_t p, int32_t mode, float temperature,
                            uint64_t seed, uint64_t step, void* workspace, size_t workspace_bytes,
                            const fh_outputs* out, void* stream) {
  fh_status st = check_forward_args(desc, h, centroids, cluster_tokens, E_tiles, E_scales, p, mode, temperature, out);
  if (st != FH_OK) return st;
  fh::Workspace ws;
  if ((st = check_ws(desc, p, workspace, workspace_bytes, &ws)) != FH_OK) return st;
  return forward_on(desc, h, centroids, cluster_tokens, E_tiles, E_scales, p, mode, temperature, seed, step, ws, out,
                    stream);
}

fh_status flashhead_forward_noalloc(const fh_desc* desc, const void* h, const void* centroids,
                                    const int32_t* cluster_tokens, const void* E_tiles, const void* E_scales,
                                    int64_t p, int32_t mode, float temperature, uint64_t seed, uint64_t step,
                                    const fh_outputs* out, void* stream) {
  fh_status st = check_forward_args(desc, h, centroids, cluster_tokens, E_tiles, E_scales, p, mode, temperature, out);
  if (st != FH_OK) return st;
  const size_t need = fh::carve_workspace(nullptr, (int)desc->B, (int)desc->c, (int)p).bytes;
  if (need > kStaticScratchBytes)
    return fail(FH_ERR_UNSUPPORTED, "this head needs %zu bytes of workspace; the static scratch holds %zu "
                "(use flashhead_forward with a caller workspace)", need, kStaticScratchBytes);
  void* base = nullptr;
  if ((st = scratch_of_current_device(&base)) != FH_OK) return st;
  const fh::Workspace ws = fh::carve_workspace(base, (int)desc->B, (int)desc->c, (int)p);
  return forward_on(desc, h, centroids, cluster_tokens, E_tiles, E_scales, p, mode, temperature, seed, step, ws, out,
                    stream);
}

fh_status flashhead_mc_marginal_workspace_bytes(const fh_desc* desc, size_t* bytes) {
  fh_status st = check_desc(desc, true);
  if (st != FH_OK) return st;
  if (!bytes) return fail(FH_ERR_ARG, "bytes is NULL");
  *bytes = fh::carve_mc_workspace(nullptr, (int)desc->B, (int)desc->c, (int)(desc->V / desc->c)).bytes;
  return FH_OK;
}

fh_status flashhead_mc_marginal(const fh_desc* desc, const void* h, const void* centroids,
                                const int32_t* cluster_tokens, const void* E_tiles, const void* E_scales, int64_t p,
                                float temperature, uint64_t seed, int64_t n_sets, int32_t clip, void* workspace,
                                size_t workspace_bytes, double* out, void* stream) {
  fh_status st = check_desc(desc, true);
  if (st != FH_OK) return st;
  if ((st = check_p(desc, p)) != FH_OK) return st;
  if ((st = check_sampling(FH_SAMPLE, temperature)) != FH_OK) return st;
  if (!h || !centroids || !cluster_tokens || !E_tiles || !out)
    return fail(FH_ERR_ARG, "h, centroids, cluster_tokens, E_tiles and out must be non-NULL");
  if (desc->e_dtype == FH_INT4_G128 && !E_scales) return fail(FH_ERR_ARG, "E_scales must be non-NULL for INT4_G128");
  if (n_sets < 1 || n_sets > kMaxSets)
    return fail(FH_ERR_ARG, "n_sets=%lld must satisfy 1 <= n_sets <= %lld", (long long)n_sets, (long long)kMaxSets);
  if (clip != 0 && clip != 1) return fail(FH_ERR_ARG, "clip must be 0 or 1");
  const fh::HeadShape s = shape_of(desc);
  const fh::McWorkspace w = fh::carve_mc_workspace(workspace, s.B, s.c, s.b);
  if (!workspace) return fail(FH_ERR_WORKSPACE, "workspace is NULL");
  if (workspace_bytes < w.bytes)
    return fail(FH_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes,
                w.bytes);
  hipStream_t hs = (hipStream_t)stream;
  // every logit of the head: the centroid scores (greedy keys are the logits), then the token
  // logits in tile order -- bf16 / fp32 tiles are a dense [V][d] matrix for the dense GEMV;
  // int4 tiles go through the forward pass with p = c
  const fh::Sampling plain = sampling_of(FH_GREEDY, 1.0f, 0, 0);
  hipError_t e = fh::launch_scores(s, h, centroids, plain, w.fw, w.s, hs);
  if (e != hipSuccess) return hip_fail(e, "centroid scores launch");
  if (desc->e_dtype == FH_INT4_G128) {
    const fh_outputs all{w.token, nullptr, w.z, nullptr};
    if ((st = select_and_probe(s, s.c, h, cluster_tokens, E_tiles, E_scales, plain, w.fw, &all, true, hs)) != FH_OK)
      return st;
  } else {
    e = fh::launch_dense(s, s.c * s.b, h, E_tiles, plain, w.fw.best, w.token, w.z, hs);
    if (e != hipSuccess) return hip_fail(e, "tile logits launch");
  }
  e = fh::launch_mc(s, (int)p, temperature, seed, n_sets, clip, cluster_tokens, w, out, hs);
  if (e != hipSuccess) return hip_fail(e, "Monte-Carlo marginal launch");
  return FH_OK;
}

fh_status flashhead_dense_workspace_bytes(const fh_desc* desc, size_t* bytes) {
  fh_status st = check_desc(desc, false);
  if (st != FH_OK) return st;
  if (!bytes) return fail(FH_ERR_ARG, "bytes is NULL");
  *bytes = fh::dense_workspace_bytes((int)desc->B);
  return FH_OK;
}

fh_status flashhead_dense_forward(const fh_desc* desc, const void* h, const void* E, int32_t mode, float temperature,
                                  uint64_t seed, uint64_t step, void* workspace, size_t workspace_bytes,
                                  int32_t* token, float* logits, void* stream) {
  fh_status st = check_desc(desc, false);
  if (st != FH_OK) return st;
  if ((st = check_sampling(mode, temperature)) != FH_OK) return st;
  if (!h || !E || !token) return fail(FH_ERR_ARG, "h, E and token must be non-NULL");
  if (!workspace) return fail(FH_ERR_WORKSPACE, "workspace is NULL");
  const size_t need = fh::dense_workspace_bytes((int)desc->B);
  if (workspace_bytes < need)
    return fail(FH_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", workspace_bytes, need);
  hipError_t e = fh::launch_dense(shape_of(desc), (int)desc->V, h, E, sampling_of(mode, temperature, seed, step),
                                  (uint64_t*)workspace, token, logits, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "dense head launch");
  return FH_OK;
}

fh_status flashhead_philox_words(uint64_t seed, uint32_t row, uint64_t step, uint32_t rng_stream, uint32_t n0,
                                 int64_t count, uint32_t* words_out, float* gumbel_out, void* stream) {
  if (rng_stream > 3) return fail(FH_ERR_ARG, "rng_stream=%u must be 0, 1, 2 or 3", (unsigned)rng_stream);
  if (count < 0 || (uint64_t)n0 + (uint64_t)count > (uint64_t(1) << 32))
    return fail(FH_ERR_ARG, "count=%lld must be >= 0 with n0 + count <= 2^32", (long long)count);
  if (!words_out && !gumbel_out) return fail(FH_ERR_ARG, "words_out and gumbel_out are both NULL");
  if (count == 0) return FH_OK;
  hipError_t e = fh::launch_philox_words(seed, row, step, rng_stream, n0, count, words_out, gumbel_out,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "philox launch");
  return FH_OK;
}

}  // extern "C"
