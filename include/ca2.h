/*
 * ca2.h -- C ABI of libca2: shared causal KV-cache attention for
 * autoregressive video diffusion (Ca2-VDM), on AMD MI355X (gfx950).
 *
 * Source pages cited below:
 *   [notes]    papernotes.org, "Ca2-VDM: Efficient Autoregressive Video Diffusion
 *              Model with Causal Generation and Cache Sharing" (ICML 2025 notes).
 *              Sections: overall framework (整体框架), key designs 1-5 (关键设计),
 *              training strategy, GPU-memory table.
 *   [abstract] bohrium.dp.tech abstract page of arXiv 2411.16375, section
 *              "Formula Representation".
 *
 * What the library holds: one cache object per (layer, batch) = a temporal
 * KV ring of P_max frame slots ([notes] key design 4: FIFO queue capped at
 * P_max) plus a spatial KV buffer of P' frame slots ([notes] key design 5:
 * one chunk's spatial K/V, overwritten every autoregressive step). The cache is
 * read by every denoising call and written only by ca2_cache_write, so one
 * copy serves all T denoising steps ([notes] key design 2, cache sharing).
 * A cache created with staging slots (ca2_cache_create_staged) can instead
 * receive a clean chunk's K/V straight from the cache-writing projection
 * (ca2_qkv_proj_stage, which also binds the cyclic TPE row into them) and
 * take it into the queue with ca2_cache_commit, with no separate copy.
 * Beside the cache object: the QKV projection of the cache-writing pass,
 * cache-less attention over T frames (the recompute baseline the cache
 * removes), and the pieces of a small random-weight block used to check the
 * cache end to end (ca2_toy_*).
 *
 * Conventions (all entry points):
 *   - Layout of every activation tensor: [B][n][S][H][d] contiguous
 *     (batch, frame, spatial token, head, head dim); the ring is
 *     [B][R][S][H][d] with R = P_max ring slots (P_max + chunk for a cache
 *     with staging slots) and the spatial buffer [B][P'][S][H][d].
 *   - Device pointers are owned by the caller, must be 16-byte aligned and
 *     must not alias the output. The library never frees them.
 *   - `stream` is a hipStream_t passed as void* (NULL = legacy default stream).
 *     Every compute call is asynchronous on that stream. Host-side cache state
 *     (queue head, P_k, frames written) is updated when the call is enqueued,
 *     so later calls must be ordered after earlier ones on the device (same
 *     stream, or caller-managed events).
 *   - HIP graphs: an attention call reads the queue state (head slot, P_k,
 *     prefix slots) on the host when it is enqueued and passes it to its
 *     kernel as arguments, so a captured graph keeps the state of the moment
 *     of capture. Replaying it after a later ca2_cache_write,
 *     ca2_qkv_proj_stage or ca2_cache_commit on that cache attends over the
 *     old queue: a captured denoising loop is valid only until the next
 *     state change. ca2_cache_info.generation changes with every such call,
 *     so a caller can tell a stale graph (compare it with the value read at
 *     capture).
 *   - Arguments are validated before anything is launched; on error nothing
 *     is enqueued, the state is unchanged, and ca2_last_error() gives detail.
 *     No call aborts or throws across the ABI.
 *   - Dtypes: CA2_F32 (float) or CA2_BF16 (bfloat16 storage); accumulation,
 *     softmax statistics and the normaliser are float32 in both.
 */
#ifndef CA2_H
#define CA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ca2_cache ca2_cache;   /* opaque; owns its ring + spatial HBM buffers */

typedef enum {
  CA2_OK = 0,
  CA2_ERR_INVALID_ARG = 1,   /* bad pointer, size, alignment or config */
  CA2_ERR_OUT_OF_MEMORY = 2, /* hipMalloc failed at create */
  CA2_ERR_HIP = 3,           /* a HIP runtime call failed (see ca2_last_error) */
  CA2_ERR_STATE = 4,         /* call not valid in the cache's current state */
  CA2_ERR_UNSUPPORTED = 5    /* valid but not built (e.g. head_dim) */
} ca2_status;

typedef enum { CA2_F32 = 0, CA2_BF16 = 1 } ca2_dtype;

typedef enum {
  CA2_SPATIAL_PREFIX = 0,    /* keys = own frame + the P' cached frames */
  CA2_SPATIAL_SELF = 1       /* keys = own frame only */
} ca2_spatial_mode;

typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t heads;       /* H >= 1 */
  int32_t head_dim;    /* d: f32 {16,32,64,72,128}, bf16 {64,72,128} */
  int32_t tokens;      /* S = HW latent tokens per frame, >= 1 */
  int32_t chunk;       /* l: frames per autoregressive chunk, 1..16 */
  int32_t p_max;       /* temporal queue capacity P_max >= 1 */
  int32_t p_spatial;   /* spatial prefix frames P', 0 <= P' < l */
  int32_t tpe_len;     /* cyclic TPE table length, >= p_max + chunk */
  int32_t dtype;       /* ca2_dtype */
} ca2_config;

/* Where ca2_qkv_proj_stage writes a chunk's K/V (bit flags). */
typedef enum {
  CA2_STAGE_RING = 1,        /* the temporal ring's slots after the queue */
  CA2_STAGE_SPATIAL = 2      /* the spatial buffer (the chunk's last P' frames) */
} ca2_stage_target;

typedef struct {
  int32_t p_k;              /* frames in the temporal queue, min(frames_written, p_max) */
  int32_t head_slot;        /* ring slot of the oldest queued frame */
  int32_t spatial_frames;   /* distinct clean frames held by the spatial buffer */
  int32_t staged_frames;    /* frames staged by ca2_qkv_proj_stage, not yet committed */
  int64_t frames_written;   /* clean frames ever written (committed) */
  uint64_t bytes_resident;  /* device bytes of ring + spatial buffer */
  int32_t ring_slots;       /* R: physical ring slots (p_max, or p_max + chunk) */
  uint32_t generation;      /* state generation: +1 (mod 2^32) on every ca2_cache_write,
                               ca2_qkv_proj_stage and ca2_cache_commit that succeeds */
} ca2_cache_info;

/*
 * Create a cache for `cfg`: allocates the ring (2 * B*P_max*S*H*d elements)
 * and the spatial buffer (2 * B*P'*S*H*d) once; nothing is reallocated later.
 * Starts empty (frames_written = 0). Checks P' < l ([notes] key design 5
 * relies on it) and tpe_len >= p_max + chunk (so every window of queued plus
 * new frames has distinct TPE indices, [notes] key design 4).
 * Errors: INVALID_ARG (null, bad config), UNSUPPORTED (head_dim/dtype pair
 * not built), OUT_OF_MEMORY, HIP. On error *out is set to NULL.
 */
ca2_status ca2_cache_create(const ca2_config* cfg, ca2_cache** out);

/*
 * Same, with a ring of R = P_max + chunk slots (2 * B*(P_max+chunk)*S*H*d
 * elements). Frame F lives in slot F mod R, so the slots of the next chunk
 * never hold a queued frame: the chunk's K/V can be written there by
 * ca2_qkv_proj_stage while the queue still holds the frames the chunk's own
 * attention must see ([notes] overall framework: the cache-writing pass
 * attends with the context it was denoised with; eviction comes after).
 * Every other entry point works on such a cache as on a plain one.
 */
ca2_status ca2_cache_create_staged(const ca2_config* cfg, ca2_cache** out);

/* Free the cache's device buffers and the object. NULL-safe. The caller must
 * make sure no enqueued work still uses the cache. */
void ca2_cache_destroy(ca2_cache* cache);

/*
 * Cache-writing stage ([notes] overall framework: after denoising, one pass
 * of the clean chunk at t = 0 computes K/V that are stored for later steps).
 * k_t, v_t: temporal-layer K/V of the n clean frames, [B][n][S][H][d].
 * k_s, v_s: spatial-layer K/V of the same frames, [B][n][S][H][d]; may be
 *           NULL only when p_spatial == 0.
 * Appends the frames to the temporal queue -- frame F goes to ring slot
 * F mod R, which is the slot right after the newest queued frame -- and,
 * past P_max, drops the oldest frames (FIFO eviction, [notes] key design 4).
 * An over-full write is the normal case, not an error. Keeps the last P'
 * clean frames in the spatial buffer (frame F at slot F mod P'). Copies are
 * bitwise. 1 <= n_frames <= chunk. Enqueue this after the cache-writing
 * pass's attention calls: they must see the queue before eviction.
 * STATE while frames staged by ca2_qkv_proj_stage are not committed.
 */
ca2_status ca2_cache_write(ca2_cache* cache, const void* k_t, const void* v_t,
                           const void* k_s, const void* v_s, int32_t n_frames,
                           void* stream);

/*
 * Causal temporal attention ([notes] key design 1, CausalAttn equation with
 * its lower-triangular mask; [abstract] Formula Representation).
 * For each row (b, s, h) and new frame i in [0, n): keys/values are the P_k
 * queued frames (oldest first) followed by new frames 0..i; out_i =
 * softmax(scale * q_i . K^T) V over exactly those P_k + i + 1 keys.
 * q, k_new, v_new, out: [B][n][S][H][d] in the cache's dtype.
 * 1 <= n_frames <= chunk; scale > 0 and finite (normally 1/sqrt(d)); the
 * scaled scores scale * q . k must be finite in float32 (any magnitude up to
 * that is handled).
 * k_new and v_new may both be NULL when n_frames frames are staged in the
 * ring by ca2_qkv_proj_stage: the new keys/values are then read from their
 * ring slots (the cache-writing pass's attention before the commit).
 * Reads the cache, never writes it.
 */
ca2_status ca2_temporal_attn(const ca2_cache* cache, const void* q, const void* k_new,
                             const void* v_new, void* out, int32_t n_frames,
                             float scale, void* stream);

/*
 * Spatial attention of each of the n frames ([notes] key design 3).
 * CA2_SPATIAL_PREFIX: keys/values of frame f are its own S tokens followed by
 *   the S tokens of each of the P' spatial-buffer frames (oldest first), a
 *   map of S x (P'+1)S. While fewer than P' clean frames exist the oldest one
 *   fills the missing positions. Needs frames_written >= 1 (else STATE).
 *   STATE while staged frames in the spatial buffer are not committed.
 * CA2_SPATIAL_SELF: keys/values are the frame's own S tokens (the clean-frame
 *   self-repeat case, whose value equals plain self-attention).
 * q, k, v, out: [B][n][S][H][d]. 1 <= n_frames <= chunk; scale > 0 and
 * finite. bf16: the scores must satisfy |scale * q . k| < 1e9 (they are
 * formed in float32 with the running maximum subtracted -- by one fused
 * multiply-add per score, or at head_dim 72 inside the matrix product, whose
 * Q operand is then q * scale * log2(e) rounded once to bf16 -- and equal
 * keys keep bitwise equal scores at any magnitude below that).
 */
ca2_status ca2_spatial_attn(const ca2_cache* cache, const void* q, const void* k,
                            const void* v, void* out, int32_t n_frames, int32_t mode,
                            float scale, void* stream);

/*
 * Both attention layers of one denoising call over the shared cache, in one
 * launch where the shapes allow it ([notes] overall framework: every
 * denoising step runs the model over the noisy chunk against the same
 * cache; key design 3 for the spatial layer, key designs 1 and 4 for the
 * temporal layer). Computes exactly what
 *   ca2_spatial_attn(cache, q_s, k_s, v_s, out_s, n, mode, scale_s) and
 *   ca2_temporal_attn(cache, q_t, k_t, v_t, out_t, n, scale_t)
 * compute on the same cache state, with the same arguments, layouts and
 * errors (k_t = v_t = NULL reads staged frames from the ring). The two must
 * be independent: no input may overlap an output, nor out_s overlap out_t
 * (INVALID_ARG). The spatial work is MFMA-bound and the temporal work
 * HBM-bound, so one workgroup runs both: its four spatial wavefronts and four
 * temporal wavefronts share every SIMD.
 * Fused when: bf16 cache, head_dim 64 or 72, tokens a multiple of 64,
 * n_frames <= 8, the spatial work fits the chip's compute units in one round
 * (ceil(tokens/128) * n * heads * batch workgroups), one frame of K or V
 * (tokens * heads * head_dim * 2 bytes) under 4 GiB, and no spatial launch
 * variant is forced (ca2_set_spatial_variant). Otherwise the two kernels
 * run back to back on `stream`. *fused (may be NULL) is set to 1 or 0.
 */
ca2_status ca2_denoise_attn(const ca2_cache* cache, const void* q_s, const void* k_s, const void* v_s,
                            void* out_s, int32_t mode, float scale_s, const void* q_t, const void* k_t,
                            const void* v_t, void* out_t, float scale_t, int32_t n_frames, int32_t* fused,
                            void* stream);

/*
 * Cache-less temporal attention over T frames, [B][T][S][H][d] tensors in
 * `dtype` (ca2_dtype): for each row (b, s, h) and frame t, out_t =
 * softmax(scale * q_t . K^T) V over keys 0..t (causal = 1: full causal
 * attention over the concatenated sequence, which the cached path must
 * reproduce -- [notes] key design 1) or over all T keys (causal = 0: the
 * bidirectional temporal attention of the recompute baseline, which must see
 * every conditional frame again at every step -- [abstract] problem
 * statement; [notes] speed comparison with OS-Ext). 1 <= T <= 4096,
 * T * heads <= 65535; head_dim as for the cache. Touches no cache.
 */
ca2_status ca2_temporal_attn_frames(const void* q, const void* k, const void* v, void* out,
                                    int32_t batch, int32_t frames, int32_t tokens, int32_t heads,
                                    int32_t head_dim, int32_t dtype, int32_t causal, float scale,
                                    void* stream);

/*
 * Cache-less spatial self attention of each of T frames (keys/values are the
 * frame's own S tokens): the spatial layer of the recompute baseline, which
 * recomputes every conditional frame's spatial attention at every step
 * ([notes] FLOPs comparison of the attention layers under extended
 * conditioning). Same tensors and limits as ca2_temporal_attn_frames.
 */
ca2_status ca2_spatial_attn_frames(const void* q, const void* k, const void* v, void* out,
                                   int32_t batch, int32_t frames, int32_t tokens, int32_t heads,
                                   int32_t head_dim, int32_t dtype, float scale, void* stream);

/*
 * Cyclic TPE indices of the next n frames ([notes] key design 4,
 * Cyclic-TPEs): host_out[i] = (frames_written + i) mod tpe_len, frame 0 being
 * the conditioning frame. Host-only; host_out has n_frames entries.
 */
ca2_status ca2_tpe_index(const ca2_cache* cache, int32_t n_frames, int32_t* host_out);

/* Same arithmetic without a cache (pure host function, no GPU needed). */
ca2_status ca2_tpe_index_raw(int64_t first_frame, int32_t n, int32_t tpe_len,
                             int32_t* host_out);

/* Snapshot of the host-side state. */
ca2_status ca2_cache_info_get(const ca2_cache* cache, ca2_cache_info* out);

/* Ring slot of each logical queue position, oldest first: host_out[p_k]
 * (slot = (frames_written - p_k + j) mod R). */
ca2_status ca2_cache_slot_map(const ca2_cache* cache, int32_t* host_out);

/* Absolute frame ids held: temporal_out[p_k] oldest first (may be NULL);
 * spatial_out[p_spatial] in logical order, padded with the oldest frame while
 * fewer than P' exist (may be NULL); spatial_slots_out[p_spatial] the buffer
 * slot of each logical position (may be NULL). */
ca2_status ca2_cache_frame_ids(const ca2_cache* cache, int64_t* temporal_out,
                               int64_t* spatial_out, int32_t* spatial_slots_out);

/* Pure host versions of the slot arithmetic, for CPU tests:
 * ring: p_k = min(frames_written, p_max); slot of logical j =
 * (frames_written - p_k + j) mod p_max; host_out has p_max entries (p_k used).
 * spatial: logical j holds frame max(0, frames_written - p_spatial + j),
 * slot = frame mod p_spatial; frames_out/slots_out have p_spatial entries. */
ca2_status ca2_ring_slot_map_raw(int64_t frames_written, int32_t p_max,
                                 int32_t* host_out, int32_t* p_k_out);
ca2_status ca2_spatial_slot_map_raw(int64_t frames_written, int32_t p_spatial,
                                    int64_t* frames_out, int32_t* slots_out);

/* Bytes the cache for `cfg` holds on the device: 2 * B * (P_max + P') * S *
 * H * d * elem ([notes] GPU-memory table: independent of T). 0 if cfg is
 * invalid. Pure host function. A cache with staging slots holds chunk more
 * ring frames (ca2_cache_info_get reports the actual bytes). */
uint64_t ca2_bytes_resident(const ca2_config* cfg);

/* Synchronous copy of the whole ring and spatial buffer to host memory
 * (physical slot order). Any of the pointers may be NULL. Sizes:
 * host_k/host_v B*R*S*H*d elements, host_ks/host_vs B*P'*S*H*d. */
ca2_status ca2_cache_debug_copy(const ca2_cache* cache, void* host_k, void* host_v,
                                void* host_ks, void* host_vs, void* stream);

/*
 * QKV projection of the clean chunk for the cache-writing stage ([notes]
 * overall framework: one forward pass of the denoised chunk produces the K/V
 * that are stored). x: [m][c_in] bf16 tokens; w: [3*c_out][c_in] bf16,
 * row-major weight of a linear layer; q, k, v: [m][c_out] bf16 outputs =
 * columns [0,c), [c,2c), [2c,3c) of x * w^T, accumulated in float32.
 * m >= 1; c_in and c_out multiples of 64, at most 2^20.
 */
ca2_status ca2_qkv_proj(const void* x, const void* w, void* q, void* k, void* v,
                        int32_t m, int32_t c_in, int32_t c_out, void* stream);

/*
 * The cache-writing projection with the cache write fused into it
 * ([notes] overall framework, cache-writing stage; key design 4, Cyclic-TPEs:
 * the temporal position embedding is bound into the cached K/V and keeps the
 * cyclic index the frame was computed with). For the n clean frames that
 * follow the committed ones (frames F_w .. F_w+n-1):
 *   Y = x w^T + tpe_rows[(F_w + f) mod tpe_len]   (row of each token's frame f)
 * accumulated in float32 and rounded once to bf16; columns [0,C) are Q,
 * [C,2C) K, [2C,3C) V with C = heads * head_dim.
 * x: [B][n][S][c_in] bf16; w: [3C][c_in] bf16 (row-major linear weight);
 * tpe_rows: [tpe_len][3C] float32 table of projected embedding rows (the
 *   embedding e_i added to the tokens before the projection contributes
 *   e_i w^T), or NULL for none;
 * q, k, v: [B][n][S][H][d] bf16 outputs, each may be NULL (not written).
 * targets (ca2_stage_target flags): CA2_STAGE_RING writes K/V into ring
 *   slots (F_w + f) mod R; CA2_STAGE_SPATIAL writes the K/V of the last P'
 *   frames into the spatial buffer (frame F at slot F mod P'). The two may
 *   come from two calls (two layers' projections) for the same n. Either
 *   target needs a cache from ca2_cache_create_staged: the commit needs the
 *   ring staged, so on a plain cache even a spatial-only staging is refused
 *   (it would overwrite the prefix frames with no way to commit them).
 * The frames stay staged: the queue and the frame count do not move until
 * ca2_cache_commit, so the chunk's temporal attention still sees the queue
 * before eviction (pass k_new = v_new = NULL to read the new frames from the
 * ring). Bf16 caches only; c_in and C multiples of 64, c_in at most 2^20.
 * Errors: INVALID_ARG (NULL x/w, misaligned pointer, bad sizes or targets),
 * STATE (a cache without staging slots; a target already staged, or a
 * different n, since the last commit), UNSUPPORTED (fp32 cache), HIP.
 */
ca2_status ca2_qkv_proj_stage(ca2_cache* cache, const void* x, const void* w,
                              const float* tpe_rows, void* q, void* k, void* v,
                              int32_t c_in, int32_t n_frames, int32_t targets,
                              void* stream);

/*
 * Take the staged frames into the queue: frames_written += n, which appends
 * them and evicts past P_max exactly as ca2_cache_write does ([notes] key
 * design 4), and makes the spatial buffer's new frames the prefix. Host state
 * only (no launch). Needs the ring staged, and the spatial buffer too when
 * P' > 0; STATE otherwise.
 */
ca2_status ca2_cache_commit(ca2_cache* cache);

/*
 * Pieces of a small spatial-temporal transformer block (random weights) for
 * end-to-end checks of the shared cache on the GPU: the block's attention
 * runs through ca2_spatial_attn / ca2_temporal_attn / ca2_cache_write, these
 * compute what surrounds it. Clean frames take timestep 0 and targets the
 * denoising timestep, one entry per frame ([notes] key design 2, cache
 * sharing with tEmb(0); training section, per-frame timestep vector). All
 * device buffers are fp32, row-major, owned by the caller.
 *
 * ca2_toy_temb_mod: out[f][j] = sum_i emb(t[f])[i] * wmod[i][j] with
 *   emb(t) = [sin(t w_0), .., sin(t w_{h-1}), cos(t w_0), .., cos(t w_{h-1})],
 *   h = temb_dim / 2, w_i = 1000^(-i/h) (evaluated in double). t: [frames];
 *   wmod: [temb_dim][width]; out: [frames][width]. temb_dim even.
 * ca2_toy_ln_mod: for each token row (f, s) of x [frames][tokens][channels]:
 *   out = (x - mean) / sqrt(var + 1e-6) * (1 + mod[f][scale_off + c])
 *         + mod[f][shift_off + c]; mod rows have mod_stride floats.
 * ca2_toy_linear: y[i][j] = act(sum_k x[i][k] w[k][j]) + (r ? r[i][j] : 0),
 *   x [m][k] (ldx), w [k][n] (ldw), r and y [m][n] (ldr, ldy; y may equal r);
 *   act 0 = identity, 1 = GELU, tanh form. Pointers need 4-byte alignment.
 * Errors: INVALID_ARG for NULL or out-of-range sizes, HIP for launch failures.
 */
ca2_status ca2_toy_temb_mod(const float* t, int32_t frames, const float* wmod, int32_t temb_dim,
                            int32_t width, float* out, void* stream);
ca2_status ca2_toy_ln_mod(const float* x, const float* mod, int32_t mod_stride, int32_t shift_off,
                          int32_t scale_off, int32_t frames, int32_t tokens, int32_t channels,
                          float* out, void* stream);
ca2_status ca2_toy_linear(const float* x, int32_t ldx, const float* w, int32_t ldw, const float* r,
                          int32_t ldr, float* y, int32_t ldy, int32_t m, int32_t n, int32_t k,
                          int32_t act, void* stream);

/*
 * Test and measurement switch: force the launch variant of the bf16 spatial
 * attention kernel for every later call in the process (0 = chosen by grid
 * size, the default; 1 = 4 wavefronts x 32 queries; 2 = 4 x 64 queries,
 * head_dim <= 72; 3 = 8 wavefronts, 4 x 32 queries x 2 key halves; 4 = 4 x 32
 * queries plus a wavefront that issues every tile copy). Every variant
 * computes the same attention. INVALID_ARG outside [0, 4]. Not synchronised
 * with calls in flight on other host threads.
 */
ca2_status ca2_set_spatial_variant(int32_t variant);

/*
 * Test and measurement switch: force the kernel of bf16 temporal attention
 * (ca2_temporal_attn, ca2_temporal_attn_frames, and the temporal half of
 * ca2_denoise_attn, whether it runs as two launches or in the fused launch's
 * temporal wavefronts) for every later call in the
 * process: 0 = the default (the dimension-split kernel: VALU dot products),
 * 1 = the same, 2 = matrix-core rows wherever they apply (n <= 16, head_dim
 * 64 or 72; slower, kept for comparison). Every choice computes the same
 * attention. INVALID_ARG outside [0, 2]. Not synchronised with calls in
 * flight on other host threads.
 */
ca2_status ca2_set_temporal_variant(int32_t variant);

/* Version of this ABI (entry points, argument lists, struct layouts):
 * CA2_ABI_VERSION. A binding compares it with the value it was written for
 * and refuses a library built from other sources. */
#define CA2_ABI_VERSION 4
int32_t ca2_abi_version(void);

/* Static description of a status code; any other integer gives
 * "unknown status". Takes a plain integer so that codes from any caller,
 * valid or not, are well defined. */
const char* ca2_status_string(int32_t status);

/* Detail of the last failing call on this thread ("" if none). */
const char* ca2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CA2_H */
