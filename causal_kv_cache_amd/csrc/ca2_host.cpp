// Host side of libca2: cache object, validation, queue / spatial-buffer / TPE
// bookkeeping and kernel launches behind the C ABI declared in include/ca2.h.
//
// The whole queue state is one counter, frames_written (F_w). Clean frame F
// lives in ring slot F mod R, R the ring's slot count (P_max, or P_max + l for
// a cache created with staging slots); the queue holds the last
// P_k = min(F_w, P_max) frames, the oldest in slot (F_w - P_k) mod R
// (Ca2-VDM notes, key design 4: FIFO queue capped at P_max, oldest leaves
// first). With R >= P_max + l the next chunk's slots hold no queued frame, so
// the cache-writing projection can store the chunk's K/V there before the
// chunk's own attention has read the queue; a commit then advances F_w. The spatial buffer keeps the last P' clean frames, frame F in slot
// F mod P' (key design 5); while fewer than P' exist, the oldest fills the
// missing logical positions. TPE index of frame F is F mod L_tpe (key design
// 4, Cyclic-TPEs).
#include "ca2.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "kernels.hpp"

struct ca2_cache {
  ca2_config cfg;
  int64_t frames_written;
  int64_t frame_bytes;   // S * H * d * elem: one (batch entry, frame) block
  int32_t ring_slots;    // R: P_max, or P_max + chunk with staging slots
  int32_t staged_n;      // frames written by ca2_qkv_proj_stage, not yet committed
  int32_t staged_targets;
  uint32_t generation;   // +1 on every state change (write, stage, commit)
  void* ring_k;
  void* ring_v;
  void* sp_k;
  void* sp_v;
};

namespace {

thread_local std::string g_last_error;

ca2_status fail(ca2_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

ca2_status ok() {
  g_last_error.clear();
  return CA2_OK;
}

int elem_bytes(int dtype) { return dtype == CA2_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ca2_status check_config(const ca2_config* c) {
  if (!c) return fail(CA2_ERR_INVALID_ARG, "config is NULL");
  if (c->dtype != CA2_F32 && c->dtype != CA2_BF16) return fail(CA2_ERR_INVALID_ARG, "dtype %d", c->dtype);
  if (c->batch < 1 || c->heads < 1 || c->tokens < 1 || c->head_dim < 1)
    return fail(CA2_ERR_INVALID_ARG, "batch/heads/tokens/head_dim must be >= 1");
  if (c->chunk < 1 || c->chunk > 16) return fail(CA2_ERR_INVALID_ARG, "chunk %d not in [1, 16]", c->chunk);
  if (c->p_max < 1) return fail(CA2_ERR_INVALID_ARG, "p_max %d < 1", c->p_max);
  if (c->p_spatial < 0 || c->p_spatial >= c->chunk)
    return fail(CA2_ERR_INVALID_ARG, "p_spatial %d must satisfy 0 <= P' < chunk (%d)", c->p_spatial, c->chunk);
  if ((int64_t)c->tpe_len < (int64_t)c->p_max + c->chunk)
    return fail(CA2_ERR_INVALID_ARG, "tpe_len %d < p_max + chunk", c->tpe_len);
  const int64_t rows = (int64_t)c->batch * c->tokens * c->heads;
  if (rows > (int64_t)1 << 30) return fail(CA2_ERR_INVALID_ARG, "B*S*H too large");
  const int64_t frame = (int64_t)c->tokens * c->heads * c->head_dim * elem_bytes(c->dtype);
  if ((int64_t)c->batch * (c->p_max + c->p_spatial) * frame > ((int64_t)1 << 46))
    return fail(CA2_ERR_INVALID_ARG, "cache too large");
  if (!ca2::temporal_supported(c->dtype, c->head_dim) || !ca2::spatial_supported(c->dtype, c->head_dim))
    return fail(CA2_ERR_UNSUPPORTED, "head_dim %d not built for dtype %d", c->head_dim, c->dtype);
  return CA2_OK;
}

ca2_status check_frames(const ca2_cache* c, int32_t n) {
  if (!c) return fail(CA2_ERR_INVALID_ARG, "cache is NULL");
  if (n < 1 || n > c->cfg.chunk) return fail(CA2_ERR_INVALID_ARG, "n_frames %d not in [1, %d]", n, c->cfg.chunk);
  return CA2_OK;
}

ca2_status check_ptrs(std::initializer_list<const void*> ps) {
  int i = 0;
  for (const void* p : ps) {
    if (!p) return fail(CA2_ERR_INVALID_ARG, "device pointer argument %d is NULL", i);
    if (!aligned16(p)) return fail(CA2_ERR_INVALID_ARG, "device pointer argument %d is not 16-byte aligned", i);
    ++i;
  }
  return CA2_OK;
}

// Shape checks of the cache-less entry points ([B][T][S][H][d] tensors).
ca2_status check_frames_shape(int32_t B, int32_t T, int32_t S, int32_t H, int32_t d, int32_t dtype,
                              float scale) {
  if (dtype != CA2_F32 && dtype != CA2_BF16) return fail(CA2_ERR_INVALID_ARG, "dtype %d", dtype);
  if (B < 1 || T < 1 || S < 1 || H < 1 || d < 1)
    return fail(CA2_ERR_INVALID_ARG, "batch/frames/tokens/heads/head_dim must be >= 1");
  if (T > 4096) return fail(CA2_ERR_INVALID_ARG, "frames %d > 4096", T);
  if ((int64_t)T * H > 65535) return fail(CA2_ERR_INVALID_ARG, "frames * heads > 65535");
  if ((int64_t)B * S * H > ((int64_t)1 << 30)) return fail(CA2_ERR_INVALID_ARG, "B*S*H too large");
  if ((int64_t)B * T * S * H * d * elem_bytes(dtype) > ((int64_t)1 << 46))
    return fail(CA2_ERR_INVALID_ARG, "tensor too large");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(CA2_ERR_INVALID_ARG, "scale must be finite and > 0");
  return CA2_OK;
}

ca2_status hip_fail(hipError_t e, const char* what) {
  return fail(CA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int32_t queue_len(const ca2_cache* c) {
  return (int32_t)(c->frames_written < c->cfg.p_max ? c->frames_written : c->cfg.p_max);
}

int32_t queue_head(const ca2_cache* c) {
  return (int32_t)((c->frames_written - queue_len(c)) % c->ring_slots);
}

ca2_status check_not_staged(const ca2_cache* c, const char* what) {
  if (c->staged_n)
    return fail(CA2_ERR_STATE, "%s: %d staged frames are not committed (call ca2_cache_commit)", what,
                c->staged_n);
  return CA2_OK;
}

// Logical spatial position j -> absolute frame (oldest first, padded by the
// oldest while fewer than P' clean frames exist).
int64_t spatial_frame(int64_t fw, int32_t p, int32_t j) {
  const int64_t f = fw - p + j;
  return f < 0 ? 0 : f;
}

}  // namespace

extern "C" {

const char* ca2_status_string(int32_t s) {
  switch (s) {
    case CA2_OK: return "ok";
    case CA2_ERR_INVALID_ARG: return "invalid argument";
    case CA2_ERR_OUT_OF_MEMORY: return "out of device memory";
    case CA2_ERR_HIP: return "HIP runtime error";
    case CA2_ERR_STATE: return "invalid in the cache's current state";
    case CA2_ERR_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

const char* ca2_last_error(void) { return g_last_error.c_str(); }

int32_t ca2_abi_version(void) { return CA2_ABI_VERSION; }

uint64_t ca2_bytes_resident(const ca2_config* cfg) {
  if (check_config(cfg) != CA2_OK) return 0;
  const uint64_t frame = (uint64_t)cfg->tokens * cfg->heads * cfg->head_dim * elem_bytes(cfg->dtype);
  return 2ull * cfg->batch * (uint64_t)(cfg->p_max + cfg->p_spatial) * frame;
}

}  // extern "C"

namespace {

ca2_status create_impl(const ca2_config* cfg, bool staging, ca2_cache** out) {
  if (!out) return fail(CA2_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  ca2_status st = check_config(cfg);
  if (st != CA2_OK) return st;
  const int64_t slots = (int64_t)cfg->p_max + (staging ? cfg->chunk : 0);
  const int64_t frame = (int64_t)cfg->tokens * cfg->heads * cfg->head_dim * elem_bytes(cfg->dtype);
  if (slots > 0x7fffffff || (int64_t)cfg->batch * (slots + cfg->p_spatial) * frame > ((int64_t)1 << 46))
    return fail(CA2_ERR_INVALID_ARG, "cache too large");
  ca2_cache* c = new (std::nothrow) ca2_cache();
  if (!c) return fail(CA2_ERR_OUT_OF_MEMORY, "host allocation failed");
  c->cfg = *cfg;
  c->frames_written = 0;
  c->frame_bytes = frame;
  c->ring_slots = (int32_t)slots;
  c->staged_n = 0;
  c->staged_targets = 0;
  c->generation = 0;
  const size_t ring_bytes = (size_t)cfg->batch * c->ring_slots * c->frame_bytes;
  const size_t sp_bytes = (size_t)cfg->batch * cfg->p_spatial * c->frame_bytes;
  // Unwritten slots are filled with 0xFF bytes (a NaN in both dtypes) when
  // CA2_NAN_CANARY=1, so a kernel reading a slot it should not shows up as NaN.
  const char* canary = getenv("CA2_NAN_CANARY");
  const int fill = (canary && canary[0] == '1') ? 0xFF : 0x00;
  void** bufs[4] = {&c->ring_k, &c->ring_v, &c->sp_k, &c->sp_v};
  const size_t sizes[4] = {ring_bytes, ring_bytes, sp_bytes, sp_bytes};
  for (int i = 0; i < 4; ++i) {
    *bufs[i] = nullptr;
    if (!sizes[i]) continue;
    hipError_t e = hipMalloc(bufs[i], sizes[i]);
    if (e != hipSuccess) {
      ca2_cache_destroy(c);
      (void)hipGetLastError();
      return e == hipErrorOutOfMemory ? fail(CA2_ERR_OUT_OF_MEMORY, "hipMalloc(%zu) failed", sizes[i])
                                      : hip_fail(e, "hipMalloc");
    }
    e = hipMemset(*bufs[i], fill, sizes[i]);
    if (e != hipSuccess) {
      ca2_cache_destroy(c);
      return hip_fail(e, "hipMemset");
    }
  }
  *out = c;
  return ok();
}

}  // namespace

extern "C" {

ca2_status ca2_cache_create(const ca2_config* cfg, ca2_cache** out) { return create_impl(cfg, false, out); }

ca2_status ca2_cache_create_staged(const ca2_config* cfg, ca2_cache** out) { return create_impl(cfg, true, out); }

void ca2_cache_destroy(ca2_cache* c) {
  if (!c) return;
  if (c->ring_k) (void)hipFree(c->ring_k);
  if (c->ring_v) (void)hipFree(c->ring_v);
  if (c->sp_k) (void)hipFree(c->sp_k);
  if (c->sp_v) (void)hipFree(c->sp_v);
  delete c;
}

ca2_status ca2_cache_write(ca2_cache* c, const void* k_t, const void* v_t, const void* k_s,
                           const void* v_s, int32_t n, void* stream) {
  ca2_status st = check_frames(c, n);
  if (st != CA2_OK) return st;
  st = check_not_staged(c, "ca2_cache_write");
  if (st != CA2_OK) return st;
  st = check_ptrs({k_t, v_t});
  if (st != CA2_OK) return st;
  const int32_t P = c->cfg.p_max, Ps = c->cfg.p_spatial, R = c->ring_slots;
  if (Ps > 0) {
    st = check_ptrs({k_s, v_s});
    if (st != CA2_OK) return st;
  }
  ca2::CopyArgs a;
  memset(&a, 0, sizeof(a));
  a.batch = c->cfg.batch;
  a.frame_bytes = c->frame_bytes;
  const int64_t fw = c->frames_written;
  const int64_t fb = c->frame_bytes;
  int nj = 0;
  // temporal ring: frame fw+i -> slot (fw+i) mod R; only the last P stay queued
  for (int32_t i = (n > P ? n - P : 0); i < n; ++i) {
    const int64_t slot = (fw + i) % R;
    const void* srcs[2] = {k_t, v_t};
    void* dsts[2] = {c->ring_k, c->ring_v};
    for (int t = 0; t < 2; ++t) {
      a.job[nj].src = static_cast<const unsigned char*>(srcs[t]) + i * fb;
      a.job[nj].dst = static_cast<unsigned char*>(dsts[t]) + slot * fb;
      a.job[nj].src_bstride = (int64_t)n * fb;
      a.job[nj].dst_bstride = (int64_t)R * fb;
      ++nj;
    }
  }
  // spatial buffer: last P' frames, frame F -> slot F mod P'
  for (int32_t i = (n > Ps ? n - Ps : 0); Ps > 0 && i < n; ++i) {
    const int64_t slot = (fw + i) % Ps;
    const void* srcs[2] = {k_s, v_s};
    void* dsts[2] = {c->sp_k, c->sp_v};
    for (int t = 0; t < 2; ++t) {
      a.job[nj].src = static_cast<const unsigned char*>(srcs[t]) + i * fb;
      a.job[nj].dst = static_cast<unsigned char*>(dsts[t]) + slot * fb;
      a.job[nj].src_bstride = (int64_t)n * fb;
      a.job[nj].dst_bstride = (int64_t)Ps * fb;
      ++nj;
    }
  }
  a.n_jobs = nj;
  hipError_t e = ca2::launch_copy(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache_write launch");
  c->frames_written += n;
  ++c->generation;
  return ok();
}

}  // extern "C"

namespace {

// Validation and kernel arguments of one temporal-attention call over the
// cache (ca2_temporal_attn, ca2_denoise_attn).
ca2_status temporal_args(const ca2_cache* c, const void* q, const void* k_new, const void* v_new, void* out,
                         int32_t n, float scale, ca2::TemporalArgs* a) {
  ca2_status st = check_frames(c, n);
  if (st != CA2_OK) return st;
  // new frames already in the ring: staged by ca2_qkv_proj_stage, not committed
  const bool from_ring = !k_new && !v_new && c->staged_n > 0 && (c->staged_targets & CA2_STAGE_RING);
  if (!k_new && !v_new && !from_ring)
    return fail(CA2_ERR_INVALID_ARG, "k_new and v_new are NULL but no frames are staged in the ring");
  if (from_ring && n != c->staged_n)
    return fail(CA2_ERR_INVALID_ARG, "n_frames %d differs from the %d staged frames", n, c->staged_n);
  st = from_ring ? check_ptrs({q, out}) : check_ptrs({q, k_new, v_new, out});
  if (st != CA2_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(CA2_ERR_INVALID_ARG, "scale must be finite and > 0");
  a->q = q; a->k_new = k_new; a->v_new = v_new; a->out = out;
  a->ring_k = c->ring_k; a->ring_v = c->ring_v;
  a->rows_per_batch = c->cfg.tokens * c->cfg.heads;
  a->rows_total = c->cfg.batch * a->rows_per_batch;
  a->n = n;
  a->p_k = queue_len(c);
  a->head = queue_head(c);
  a->p_max = c->ring_slots;
  a->ring_keys = from_ring ? a->p_k + n : a->p_k;
  a->causal = 1;
  a->scale_log2e = scale * 1.4426950408889634f;
  return CA2_OK;
}

// Validation and kernel arguments of one spatial-attention call over the
// cache (ca2_spatial_attn, ca2_denoise_attn).
ca2_status spatial_args(const ca2_cache* c, const void* q, const void* k, const void* v, void* out, int32_t n,
                        int32_t mode, float scale, ca2::SpatialArgs* a) {
  ca2_status st = check_frames(c, n);
  if (st != CA2_OK) return st;
  st = check_ptrs({q, k, v, out});
  if (st != CA2_OK) return st;
  if (mode != CA2_SPATIAL_PREFIX && mode != CA2_SPATIAL_SELF) return fail(CA2_ERR_INVALID_ARG, "mode %d", mode);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(CA2_ERR_INVALID_ARG, "scale must be finite and > 0");
  const int32_t Ps = c->cfg.p_spatial;
  memset(a, 0, sizeof(*a));
  a->q = q; a->k = k; a->v = v; a->out = out;
  a->sp_k = c->sp_k; a->sp_v = c->sp_v;
  a->batch = c->cfg.batch; a->n = n; a->tokens = c->cfg.tokens; a->heads = c->cfg.heads;
  a->p_slots = Ps;
  a->n_prefix = 0;
  if (mode == CA2_SPATIAL_PREFIX && Ps > 0) {
    if (c->frames_written < 1)
      return fail(CA2_ERR_STATE, "prefix mode needs at least one clean frame in the cache");
    if (c->staged_targets & CA2_STAGE_SPATIAL)
      return fail(CA2_ERR_STATE, "prefix mode while the spatial buffer holds staged, uncommitted frames");
    a->n_prefix = Ps;
    for (int32_t j = 0; j < Ps; ++j) a->prefix_slot[j] = (int32_t)(spatial_frame(c->frames_written, Ps, j) % Ps);
  }
  a->scale_log2e = scale * 1.4426950408889634f;
  return CA2_OK;
}

bool overlap(const void* a, const void* b, size_t bytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bytes && y < x + bytes;
}

}  // namespace

extern "C" {

ca2_status ca2_temporal_attn(const ca2_cache* c, const void* q, const void* k_new, const void* v_new,
                             void* out, int32_t n, float scale, void* stream) {
  ca2::TemporalArgs a;
  ca2_status st = temporal_args(c, q, k_new, v_new, out, n, scale, &a);
  if (st != CA2_OK) return st;
  hipError_t e = ca2::launch_temporal(c->cfg.dtype, c->cfg.head_dim, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "temporal_attn launch");
  return ok();
}

ca2_status ca2_spatial_attn(const ca2_cache* c, const void* q, const void* k, const void* v, void* out,
                            int32_t n, int32_t mode, float scale, void* stream) {
  ca2::SpatialArgs a;
  ca2_status st = spatial_args(c, q, k, v, out, n, mode, scale, &a);
  if (st != CA2_OK) return st;
  hipError_t e = ca2::launch_spatial(c->cfg.dtype, c->cfg.head_dim, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spatial_attn launch");
  return ok();
}

ca2_status ca2_denoise_attn(const ca2_cache* c, const void* q_s, const void* k_s, const void* v_s, void* out_s,
                            int32_t mode, float scale_s, const void* q_t, const void* k_t, const void* v_t,
                            void* out_t, float scale_t, int32_t n, int32_t* fused, void* stream) {
  ca2::SpatialArgs sa;
  ca2::TemporalArgs ta;
  ca2_status st = spatial_args(c, q_s, k_s, v_s, out_s, n, mode, scale_s, &sa);
  if (st != CA2_OK) return st;
  st = temporal_args(c, q_t, k_t, v_t, out_t, n, scale_t, &ta);
  if (st != CA2_OK) return st;
  const size_t bytes = (size_t)c->cfg.batch * n * c->frame_bytes;
  if (overlap(out_s, out_t, bytes)) return fail(CA2_ERR_INVALID_ARG, "out_s and out_t overlap");
  for (const void* in : {q_s, k_s, v_s, q_t, k_t, v_t})
    if (in && (overlap(in, out_s, bytes) || overlap(in, out_t, bytes)))
      return fail(CA2_ERR_INVALID_ARG, "an input overlaps an output");
  bool f = false;
  hipError_t e = ca2::launch_denoise_call(c->cfg.dtype, c->cfg.head_dim, sa, ta, static_cast<hipStream_t>(stream), &f);
  if (e != hipSuccess) return hip_fail(e, "denoise_attn launch");
  if (fused) *fused = f ? 1 : 0;
  return ok();
}

ca2_status ca2_temporal_attn_frames(const void* q, const void* k, const void* v, void* out, int32_t B,
                                    int32_t T, int32_t S, int32_t H, int32_t d, int32_t dtype, int32_t causal,
                                    float scale, void* stream) {
  ca2_status st = check_frames_shape(B, T, S, H, d, dtype, scale);
  if (st != CA2_OK) return st;
  st = check_ptrs({q, k, v, out});
  if (st != CA2_OK) return st;
  if (causal != 0 && causal != 1) return fail(CA2_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!ca2::temporal_supported(dtype, d))
    return fail(CA2_ERR_UNSUPPORTED, "head_dim %d not built for dtype %d", d, dtype);
  ca2::TemporalArgs a;
  a.q = q; a.k_new = k; a.v_new = v; a.out = out;
  a.ring_k = k; a.ring_v = v;   // never read: the queue is empty
  a.rows_per_batch = S * H;
  a.rows_total = B * a.rows_per_batch;
  a.n = T;
  a.p_k = 0;
  a.head = 0;
  a.p_max = 1;
  a.ring_keys = 0;
  a.causal = causal;
  a.scale_log2e = scale * 1.4426950408889634f;
  hipError_t e = ca2::launch_temporal(dtype, d, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "temporal_attn_frames launch");
  return ok();
}

ca2_status ca2_spatial_attn_frames(const void* q, const void* k, const void* v, void* out, int32_t B,
                                   int32_t T, int32_t S, int32_t H, int32_t d, int32_t dtype, float scale,
                                   void* stream) {
  ca2_status st = check_frames_shape(B, T, S, H, d, dtype, scale);
  if (st != CA2_OK) return st;
  st = check_ptrs({q, k, v, out});
  if (st != CA2_OK) return st;
  if (!ca2::spatial_supported(dtype, d))
    return fail(CA2_ERR_UNSUPPORTED, "head_dim %d not built for dtype %d", d, dtype);
  ca2::SpatialArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.sp_k = nullptr; a.sp_v = nullptr;
  a.batch = B; a.n = T; a.tokens = S; a.heads = H;
  a.p_slots = 0;
  a.n_prefix = 0;
  a.scale_log2e = scale * 1.4426950408889634f;
  hipError_t e = ca2::launch_spatial(dtype, d, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "spatial_attn_frames launch");
  return ok();
}

ca2_status ca2_set_spatial_variant(int32_t variant) {
  if (variant < 0 || variant > 4) return fail(CA2_ERR_INVALID_ARG, "variant %d not in [0, 4]", variant);
  ca2::set_spatial_variant(variant);
  return ok();
}

ca2_status ca2_set_temporal_variant(int32_t variant) {
  if (variant < 0 || variant > 2) return fail(CA2_ERR_INVALID_ARG, "variant %d not in [0, 2]", variant);
  ca2::set_temporal_variant(variant);
  return ok();
}

ca2_status ca2_tpe_index_raw(int64_t first, int32_t n, int32_t L, int32_t* out) {
  if (first < 0 || n < 0 || L < 1) return fail(CA2_ERR_INVALID_ARG, "first >= 0, n >= 0, tpe_len >= 1");
  if (n > 0 && !out) return fail(CA2_ERR_INVALID_ARG, "host_out is NULL");
  for (int32_t i = 0; i < n; ++i) out[i] = (int32_t)((first + i) % L);
  return ok();
}

ca2_status ca2_tpe_index(const ca2_cache* c, int32_t n, int32_t* out) {
  ca2_status st = check_frames(c, n);
  if (st != CA2_OK) return st;
  return ca2_tpe_index_raw(c->frames_written, n, c->cfg.tpe_len, out);
}

ca2_status ca2_cache_info_get(const ca2_cache* c, ca2_cache_info* out) {
  if (!c || !out) return fail(CA2_ERR_INVALID_ARG, "NULL argument");
  out->p_k = queue_len(c);
  out->head_slot = queue_head(c);
  const int64_t fw = c->frames_written;
  out->spatial_frames = (int32_t)(fw < c->cfg.p_spatial ? fw : c->cfg.p_spatial);
  out->staged_frames = c->staged_n;
  out->ring_slots = c->ring_slots;
  out->generation = c->generation;
  out->frames_written = fw;
  out->bytes_resident = 2ull * c->cfg.batch * (uint64_t)(c->ring_slots + c->cfg.p_spatial) * c->frame_bytes;
  return ok();
}

ca2_status ca2_ring_slot_map_raw(int64_t fw, int32_t P, int32_t* out, int32_t* p_k_out) {
  if (fw < 0 || P < 1) return fail(CA2_ERR_INVALID_ARG, "frames_written >= 0, p_max >= 1");
  const int32_t pk = (int32_t)(fw < P ? fw : P);
  if (pk > 0 && !out) return fail(CA2_ERR_INVALID_ARG, "host_out is NULL");
  for (int32_t j = 0; j < pk; ++j) out[j] = (int32_t)((fw - pk + j) % P);
  if (p_k_out) *p_k_out = pk;
  return ok();
}

ca2_status ca2_spatial_slot_map_raw(int64_t fw, int32_t Ps, int64_t* frames_out, int32_t* slots_out) {
  if (fw < 0 || Ps < 0) return fail(CA2_ERR_INVALID_ARG, "frames_written >= 0, p_spatial >= 0");
  if (fw == 0 || Ps == 0) return ok();
  for (int32_t j = 0; j < Ps; ++j) {
    const int64_t f = spatial_frame(fw, Ps, j);
    if (frames_out) frames_out[j] = f;
    if (slots_out) slots_out[j] = (int32_t)(f % Ps);
  }
  return ok();
}

ca2_status ca2_cache_slot_map(const ca2_cache* c, int32_t* out) {
  if (!c) return fail(CA2_ERR_INVALID_ARG, "cache is NULL");
  const int32_t pk = queue_len(c);
  if (pk > 0 && !out) return fail(CA2_ERR_INVALID_ARG, "host_out is NULL");
  for (int32_t j = 0; j < pk; ++j) out[j] = (int32_t)((c->frames_written - pk + j) % c->ring_slots);
  return ok();
}

ca2_status ca2_cache_frame_ids(const ca2_cache* c, int64_t* t_out, int64_t* s_out, int32_t* s_slots) {
  if (!c) return fail(CA2_ERR_INVALID_ARG, "cache is NULL");
  const int32_t pk = queue_len(c);
  if (t_out)
    for (int32_t j = 0; j < pk; ++j) t_out[j] = c->frames_written - pk + j;
  return ca2_spatial_slot_map_raw(c->frames_written, c->cfg.p_spatial, s_out, s_slots);
}

ca2_status ca2_cache_debug_copy(const ca2_cache* c, void* hk, void* hv, void* hks, void* hvs, void* stream) {
  if (!c) return fail(CA2_ERR_INVALID_ARG, "cache is NULL");
  const size_t ring = (size_t)c->cfg.batch * c->ring_slots * c->frame_bytes;
  const size_t sp = (size_t)c->cfg.batch * c->cfg.p_spatial * c->frame_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  struct { void* dst; const void* src; size_t n; } cp[4] = {
      {hk, c->ring_k, ring}, {hv, c->ring_v, ring}, {hks, c->sp_k, sp}, {hvs, c->sp_v, sp}};
  for (auto& x : cp) {
    if (!x.dst || !x.n) continue;
    hipError_t e = hipMemcpyAsync(x.dst, x.src, x.n, hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return ok();
}

ca2_status ca2_qkv_proj(const void* x, const void* w, void* q, void* k, void* v, int32_t m, int32_t c_in,
                        int32_t c_out, void* stream) {
  ca2_status st = check_ptrs({x, w, q, k, v});
  if (st != CA2_OK) return st;
  if (m < 1 || c_in < 64 || c_out < 64 || c_in % 64 || c_out % 64)
    return fail(CA2_ERR_INVALID_ARG, "m >= 1, c_in and c_out multiples of 64");
  if (m > 0x7fffff00) return fail(CA2_ERR_INVALID_ARG, "m too large");   // token index + tile stays in int32
  if (c_in > (1 << 20) || c_out > (1 << 20)) return fail(CA2_ERR_INVALID_ARG, "c_in, c_out <= 2^20");
  if ((int64_t)m * c_in > ((int64_t)1 << 40)) return fail(CA2_ERR_INVALID_ARG, "too large");
  ca2::ProjArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.w = w; a.q = q; a.k = k; a.v = v;
  a.m = m; a.c_in = c_in; a.c_out = c_out;
  hipError_t e = ca2::launch_qkv_proj(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "qkv_proj launch");
  return ok();
}

ca2_status ca2_qkv_proj_stage(ca2_cache* c, const void* x, const void* w, const float* tpe_rows, void* q,
                              void* k, void* v, int32_t c_in, int32_t n, int32_t targets, void* stream) {
  ca2_status st = check_frames(c, n);
  if (st != CA2_OK) return st;
  if (c->cfg.dtype != CA2_BF16) return fail(CA2_ERR_UNSUPPORTED, "the projection is built for bf16 caches only");
  st = check_ptrs({x, w});
  if (st != CA2_OK) return st;
  for (const void* p : {(const void*)tpe_rows, (const void*)q, (const void*)k, (const void*)v})
    if (p && !aligned16(p)) return fail(CA2_ERR_INVALID_ARG, "tpe_rows / q / k / v must be 16-byte aligned");
  if (targets < 1 || targets > (CA2_STAGE_RING | CA2_STAGE_SPATIAL))
    return fail(CA2_ERR_INVALID_ARG, "targets %d: a nonempty combination of CA2_STAGE_RING, CA2_STAGE_SPATIAL",
                targets);
  const int32_t c_out = c->cfg.heads * c->cfg.head_dim;
  if (c_in < 64 || c_in % 64 || c_out % 64 || c_in > (1 << 20))
    return fail(CA2_ERR_INVALID_ARG, "c_in (%d, at most 2^20) and heads * head_dim (%d) must be multiples of 64",
                c_in, c_out);
  const int64_t m = (int64_t)c->cfg.batch * n * c->cfg.tokens;
  if (m > 0x7fffff00 || m * c_in > ((int64_t)1 << 40)) return fail(CA2_ERR_INVALID_ARG, "too large");
  // Either target needs staging slots: a commit needs the ring staged, so a
  // spatial-only staging on a plain cache would overwrite the prefix frames
  // with no way to commit them.
  if (c->ring_slots < c->cfg.p_max + n)
    return fail(CA2_ERR_STATE, "staging needs a cache created with ca2_cache_create_staged");
  if (c->staged_n && (c->staged_n != n || (c->staged_targets & targets)))
    return fail(CA2_ERR_STATE, "already staged: %d frames, targets %d", c->staged_n, c->staged_targets);
  const int64_t fw = c->frames_written;
  const int32_t Ps = c->cfg.p_spatial;
  ca2::ProjArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x; a.w = w; a.q = q; a.k = k; a.v = v;
  a.m = (int32_t)m; a.c_in = c_in; a.c_out = c_out;
  a.tpe = tpe_rows;
  a.tokens = c->cfg.tokens;
  a.frames = n;
  a.tpe_len = c->cfg.tpe_len;
  a.tpe_first = (int32_t)(fw % c->cfg.tpe_len);
  a.ring_slots = c->ring_slots;
  a.ring_first = (int32_t)(fw % c->ring_slots);
  if (targets & CA2_STAGE_RING) {
    a.ring_k = c->ring_k;
    a.ring_v = c->ring_v;
  }
  if ((targets & CA2_STAGE_SPATIAL) && Ps > 0) {
    a.sp_k = c->sp_k;
    a.sp_v = c->sp_v;
    a.sp_slots = Ps;
    a.sp_first = (int32_t)(fw % Ps);
    a.sp_from = n > Ps ? n - Ps : 0;
  }
  hipError_t e = ca2::launch_qkv_proj_stage(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "qkv_proj_stage launch");
  c->staged_n = n;
  c->staged_targets |= targets;
  ++c->generation;
  return ok();
}

ca2_status ca2_cache_commit(ca2_cache* c) {
  if (!c) return fail(CA2_ERR_INVALID_ARG, "cache is NULL");
  if (!c->staged_n) return fail(CA2_ERR_STATE, "no staged frames to commit");
  const int32_t need = CA2_STAGE_RING | (c->cfg.p_spatial > 0 ? CA2_STAGE_SPATIAL : 0);
  if ((c->staged_targets & need) != need)
    return fail(CA2_ERR_STATE, "staged targets %d; a commit needs the ring%s", c->staged_targets,
                c->cfg.p_spatial > 0 ? " and the spatial buffer" : "");
  c->frames_written += c->staged_n;
  c->staged_n = 0;
  c->staged_targets = 0;
  ++c->generation;
  return ok();
}

ca2_status ca2_toy_temb_mod(const float* t, int32_t frames, const float* wmod, int32_t temb_dim, int32_t width,
                            float* out, void* stream) {
  ca2_status st = check_ptrs({t, wmod, out});
  if (st != CA2_OK) return st;
  if (frames < 1 || frames > 65535 || temb_dim < 2 || temb_dim % 2 || width < 1)
    return fail(CA2_ERR_INVALID_ARG, "frames in [1, 65535], temb_dim even >= 2, width >= 1");
  hipError_t e = ca2::launch_toy_temb_mod(t, frames, wmod, temb_dim, width, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "toy_temb_mod launch");
  return ok();
}

ca2_status ca2_toy_ln_mod(const float* x, const float* mod, int32_t mod_stride, int32_t shift_off,
                          int32_t scale_off, int32_t frames, int32_t tokens, int32_t channels, float* out,
                          void* stream) {
  ca2_status st = check_ptrs({x, mod, out});
  if (st != CA2_OK) return st;
  if (frames < 1 || tokens < 1 || channels < 1 || (int64_t)frames * tokens > 0x7fffffff)
    return fail(CA2_ERR_INVALID_ARG, "frames, tokens, channels >= 1");
  if (shift_off < 0 || scale_off < 0 || shift_off + channels > mod_stride || scale_off + channels > mod_stride)
    return fail(CA2_ERR_INVALID_ARG, "shift/scale ranges must lie inside a mod row");
  hipError_t e = ca2::launch_toy_ln_mod(x, mod, mod_stride, shift_off, scale_off, tokens, frames * tokens, channels,
                                        out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "toy_ln_mod launch");
  return ok();
}

ca2_status ca2_toy_linear(const float* x, int32_t ldx, const float* w, int32_t ldw, const float* r, int32_t ldr,
                          float* y, int32_t ldy, int32_t m, int32_t n, int32_t k, int32_t act, void* stream) {
  if (!x || !w || !y) return fail(CA2_ERR_INVALID_ARG, "x, w and y must not be NULL");
  if (m < 1 || n < 1 || k < 1 || m > (1 << 20) || n > (1 << 20))
    return fail(CA2_ERR_INVALID_ARG, "m, n, k >= 1 (m, n <= 2^20)");
  if (ldx < k || ldw < n || ldy < n || (r && ldr < n))
    return fail(CA2_ERR_INVALID_ARG, "leading dimensions smaller than the rows they hold");
  if (act != 0 && act != 1) return fail(CA2_ERR_INVALID_ARG, "act must be 0 (identity) or 1 (GELU)");
  ca2::ToyLinearArgs a{x, w, r, y, m, n, k, ldx, ldw, r ? ldr : 0, ldy, act};
  hipError_t e = ca2::launch_toy_linear(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "toy_linear launch");
  return ok();
}

}  // extern "C"
