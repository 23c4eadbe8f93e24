// Internal launcher interface between the host state machine (ca2_host.cpp)
// and the HIP kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ca2 {

// Temporal attention over the queue + new frames (one launch). With
// causal = 1, new frame i sees the queue and new frames 0..i; with causal = 0
// every new frame sees every key (the cache-less recompute form, p_k = 0).
// The launch covers any n >= 1: query frames are cut into blocks along grid y.
struct TemporalArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* out;
  const void* ring_k;
  const void* ring_v;
  int32_t rows_total;      // B * S * H
  int32_t rows_per_batch;  // S * H
  int32_t n;               // new frames (queries per row)
  int32_t p_k;             // queued frames
  int32_t head;            // ring slot of the oldest queued frame
  int32_t p_max;           // ring slots R (the modulus of the slot arithmetic): P_max, or
                           // P_max + chunk for a cache with staging slots
  int32_t ring_keys;       // keys 0..ring_keys-1 are read from ring slots (head + j) mod p_max:
                           // p_k, or p_k + n when the new frames were already written
                           // into the slots after the queue (k_new / v_new unused)
  int32_t causal;          // 1: lower-triangular mask over the new frames; 0: no mask
  float scale_log2e;       // softmax scale * log2(e)
};

// Spatial attention of every (b, frame, head), prefix or self mode.
struct SpatialArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const void* sp_k;        // spatial buffer [B][P'][S][H][d]
  const void* sp_v;
  int32_t batch, n, tokens, heads;
  int32_t p_slots;         // physical slots of the spatial buffer (P')
  int32_t n_prefix;        // prefix frames used (0 in self mode)
  int32_t prefix_slot[16]; // logical -> physical slot
  float scale_log2e;
};

// Bitwise frame copies for the cache write. Job j copies `frame_elems`
// elements for each batch entry b from src + b*src_bstride to
// dst + b*dst_bstride (element offsets, 16-byte chunks).
struct CopyJob {
  const void* src;
  void* dst;
  int64_t src_bstride;  // bytes
  int64_t dst_bstride;  // bytes
};
static constexpr int kMaxCopyJobs = 64;
struct CopyArgs {
  CopyJob job[kMaxCopyJobs];
  int32_t n_jobs;
  int32_t batch;
  int64_t frame_bytes;
};

// [Q K V] = X W^T. The plain projection writes q/k/v ([m][c_out]). The
// cache-writing form (kernel template kStage) takes rows as (b, f, s) of
// B x frames x tokens, adds the frame's table row to every output (fp32, before
// rounding), writes any of q/k/v that is not NULL, and also writes the K and
// V columns straight into the ring (frame f -> slot (ring_first + f) mod
// ring_slots) and, for frames f >= sp_from, into the spatial buffer
// (slot (sp_first + f) mod sp_slots). Ring and buffer are [B][slots][tokens][c_out].
struct ProjArgs {
  const void* x;
  const void* w;
  void* q;
  void* k;
  void* v;
  int32_t m, c_in, c_out;
  const float* tpe;              // [tpe_len][3 * c_out] or NULL
  void* ring_k;                  // or NULL
  void* ring_v;
  void* sp_k;                    // or NULL
  void* sp_v;
  int32_t tokens, frames;        // row m = (b * frames + f) * tokens + s
  int32_t tpe_len, tpe_first;    // row of frame f: (tpe_first + f) mod tpe_len
  int32_t ring_slots, ring_first;
  int32_t sp_slots, sp_first, sp_from;
};

// fp32 linear layer of the toy block: y = act(x w) (+ r), row-major with
// leading dimensions in elements; act 0 = identity, 1 = tanh-form GELU.
struct ToyLinearArgs {
  const float* x;
  const float* w;
  const float* r;   // may be NULL; may alias y
  float* y;
  int32_t m, n, k;
  int32_t ldx, ldw, ldr, ldy;
  int32_t act;
};

// Each launcher returns hipSuccess or the launch error; it returns
// hipErrorInvalidValue for a (dtype, head_dim) pair that is not built.
hipError_t launch_temporal(int dtype, int head_dim, const TemporalArgs& a, hipStream_t s);
hipError_t launch_spatial(int dtype, int head_dim, const SpatialArgs& a, hipStream_t s);
hipError_t launch_copy(const CopyArgs& a, hipStream_t s);
hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s);
hipError_t launch_qkv_proj_stage(const ProjArgs& a, hipStream_t s);

hipError_t launch_toy_temb_mod(const float* t, int frames, const float* wmod, int temb_dim, int width, float* out,
                               hipStream_t s);
hipError_t launch_toy_ln_mod(const float* x, const float* mod, int mod_stride, int shift_off, int scale_off,
                             int tokens, int rows, int C, float* out, hipStream_t s);
hipError_t launch_toy_linear(const ToyLinearArgs& a, hipStream_t s);

// One denoising call's two attention layers, on independent tensors: the
// spatial attention `sa` and the temporal attention `ta`. One fused launch
// where denoise_call_fusable() holds (bf16, head_dim 64 or 72, whole 64-token
// tiles, causal, n <= 8, the spatial grid within one round of workgroups, no
// forced spatial variant); otherwise the two kernels back to back on `s`.
// *fused (if not NULL) tells which.
bool denoise_call_fusable(int dtype, int head_dim, const SpatialArgs& sa, const TemporalArgs& ta);
hipError_t launch_denoise_call(int dtype, int head_dim, const SpatialArgs& sa, const TemporalArgs& ta, hipStream_t s,
                               bool* fused);

// Process-wide launch variant of the bf16 spatial kernel (0 = by size, 1..4).
void set_spatial_variant(int v);
// Process-wide kernel choice for bf16 temporal attention (0 and 1 =
// dimension-split VALU kernel, 2 = matrix-core rows where n <= 16), in the
// stand-alone kernels and in the fused denoising launch's temporal
// wavefronts alike; temporal_variant() reads it back.
void set_temporal_variant(int v);
int temporal_variant();

bool temporal_supported(int dtype, int head_dim);
bool spatial_supported(int dtype, int head_dim);

}  // namespace ca2
