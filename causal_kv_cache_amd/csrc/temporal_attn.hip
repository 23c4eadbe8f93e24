// Causal temporal attention over the shared temporal KV queue (gfx950).
//
// Computes, for every row (b, s, h) and new frame i < n, softmax over the
// P_k queued frames plus new frames 0..i of scale * q_i . k, times V
// (Ca2-VDM notes, key design 1: CausalAttn equation with a lower-triangular
// mask; key design 4: the queue of at most P_max cached frames). With the
// mask switched off and an empty queue the same kernels compute the
// bidirectional temporal attention of the recompute baseline (abstract page:
// problem statement; notes: speed comparison with OS-Ext).
//
// Two kernels. bf16 caches use the dimension-split kernel further down (K/V
// streamed from HBM straight into registers). fp32 caches use this one.
// Work mapping of the fp32 kernel (HBM-bound: each K/V byte is used by at
// most n queries):
//   * a wavefront owns ROWS = 64/QL consecutive rows; lane = (row, query),
//     QL = lanes per row >= n, so the n queries of a row sit in adjacent
//     lanes and read the same staged key row (LDS broadcast);
//   * a workgroup is NW wavefronts on the same rows; the key frames are cut
//     into blocks of F frames and dealt round-robin to the wavefronts, which
//     run without block-wide barriers on wave-private LDS;
//   * per block, the wavefront copies F frames x ROWS rows of K and V from
//     HBM into its LDS slice with 16-byte loads: for one frame the ROWS rows
//     are contiguous (heads innermost), so a wavefront reads whole runs of
//     ROWS*d*elem bytes;
//   * online softmax in base 2 with one rescale per block; partial
//     (max, sum, acc) of the NW wavefronts are merged through LDS at the end.
#include "device_common.hpp"
#include "kernels.hpp"
#include "temporal_common.hpp"
#include "temporal_mfma.hpp"

#include <atomic>

namespace ca2 {
namespace {

constexpr int kWaves = 4;              // wavefronts per workgroup

// Compute units of the current device (queried once per device).
int device_cus_t() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
constexpr int kStageBudget = 20480;    // LDS bytes per wavefront for K+V staging

template <typename T, int D, int QL>
struct TCfg {
  static constexpr int ROWS = 64 / QL;
  static constexpr int EB = (int)sizeof(T);
  static constexpr int VPC = Elem<T>::kPerChunk;       // values per 16-byte chunk
  static constexpr int CPR = D * EB / 16;              // chunks per row
  static constexpr int FRAME_BYTES = ROWS * D * EB;    // one frame of the wave's rows
  static constexpr int F_RAW = kStageBudget / (2 * FRAME_BYTES);
  static constexpr int F = F_RAW >= 8 ? 8 : F_RAW >= 4 ? 4 : F_RAW >= 2 ? 2 : 1;
  static constexpr int CHUNKS = F * ROWS * CPR;        // per tensor per block
  static constexpr int CPL = (CHUNKS + 63) / 64;       // chunks per lane
  static constexpr int STAGE_U4 = 2 * CHUNKS;          // uint4 per wave (K then V)
  static constexpr int MERGE_F = 64 * (D + 2);         // floats per wave for the merge
  static constexpr int LDS_U4_STAGE = kWaves * STAGE_U4;
  static constexpr int LDS_U4_MERGE = ((kWaves - 1) * MERGE_F * 4 + 15) / 16;
  static constexpr int LDS_U4 = LDS_U4_STAGE > LDS_U4_MERGE ? LDS_U4_STAGE : LDS_U4_MERGE;
  static_assert(D * EB % 16 == 0, "row must be a whole number of 16-byte chunks");
};

template <typename T, int D, int QL>
__global__ __launch_bounds__(64 * kWaves) void temporal_attn_kernel(TemporalArgs a) {
  using C = TCfg<T, D, QL>;
  constexpr int ROWS = C::ROWS, CPR = C::CPR, F = C::F, CHUNKS = C::CHUNKS, CPL = C::CPL;
  constexpr int VPC = C::VPC;
  __shared__ uint4 lds[C::LDS_U4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: key ranges, branches
  const int row0 = blockIdx.x * ROWS;
  const int ri = lane / QL;
  const int q0 = blockIdx.y * QL;           // first query frame of this block
  const int qi = q0 + lane % QL;
  const int row = row0 + ri;
  const bool active = row < a.rows_total && qi < a.n;
  const int rpb = a.rows_per_batch;

  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ knp = static_cast<const T*>(a.k_new);
  const T* __restrict__ vnp = static_cast<const T*>(a.v_new);
  const T* __restrict__ rkp = static_cast<const T*>(a.ring_k);
  const T* __restrict__ rvp = static_cast<const T*>(a.ring_v);

  // ---- this lane's query, in float32 registers --------------------------
  float qf[D];
  {
    const int b = row / rpb, rr = row % rpb;
    const int64_t off = ((int64_t)(b * a.n + qi) * rpb + rr) * D;
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (active) u = *reinterpret_cast<const uint4*>(qp + off + c * VPC);
      Elem<T>::unpack(u, qf + c * VPC);
    }
  }

  // ---- per-chunk staging coordinates (same every block) -----------------
  // chunk e of a block = (frame fo, row r, piece cc) with e = (fo*ROWS + r)*CPR + cc
  int64_t ch_rowoff[CPL];   // element offset of (row, piece) inside a frame of its batch
  int ch_b[CPL], ch_fo[CPL];
  bool ch_ok[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = c * 64 + lane;
    const int fo = e / (ROWS * CPR);
    const int rem = e % (ROWS * CPR);
    const int r = rem / CPR, cc = rem % CPR;
    const int grow = row0 + r;
    ch_ok[c] = e < CHUNKS && grow < a.rows_total;
    const int b = grow / rpb, rr = grow % rpb;
    ch_b[c] = b;
    ch_fo[c] = fo;
    ch_rowoff[c] = (int64_t)rr * D + cc * VPC;
  }

  uint4* stage = lds + wave * C::STAGE_U4;
  const int k_total = a.p_k + a.n;
  // keys any query of the block can see
  const int k_lim = a.causal ? min(k_total, a.p_k + q0 + QL) : k_total;
  const int n_blocks = (k_lim + F - 1) / F;
  const int last_key = a.causal ? a.p_k + qi : k_total - 1;   // keys 0..last_key are visible
  const int64_t frame_elems = (int64_t)rpb * D;

  float m = -INFINITY, l = 0.f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;

  for (int blk = wave; blk < n_blocks; blk += kWaves) {
    const int j0 = blk * F;
    // -- stage F key frames (K then V) of this wave's rows into LDS --
    uint4 kr[CPL], vr[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = j0 + ch_fo[c];
      kr[c] = make_uint4(0, 0, 0, 0);
      vr[c] = make_uint4(0, 0, 0, 0);
      if (ch_ok[c] && j < k_lim) {
        const T* kb;
        const T* vb;
        int64_t base;
        if (j < a.ring_keys) {
          int slot = a.head + j;
          if (slot >= a.p_max) slot -= a.p_max;
          base = ((int64_t)ch_b[c] * a.p_max + slot) * frame_elems;
          kb = rkp; vb = rvp;
        } else {
          base = ((int64_t)ch_b[c] * a.n + (j - a.p_k)) * frame_elems;
          kb = knp; vb = vnp;
        }
        kr[c] = *reinterpret_cast<const uint4*>(kb + base + ch_rowoff[c]);
        vr[c] = *reinterpret_cast<const uint4*>(vb + base + ch_rowoff[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = c * 64 + lane;
      if (e < CHUNKS) {
        stage[e] = kr[c];
        stage[CHUNKS + e] = vr[c];
      }
    }
    // LDS accesses of one wavefront complete in order; this only stops the
    // compiler from moving the reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // -- scores of the block --
    float sc[F];
    float mb = -INFINITY;
#pragma unroll
    for (int fo = 0; fo < F; ++fo) {
      const uint4* krow = stage + (fo * ROWS + ri) * CPR;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < CPR; ++c) {
        float kv[VPC];
        Elem<T>::unpack(krow[c], kv);
#pragma unroll
        for (int e = 0; e < VPC; ++e) s = fmaf(qf[c * VPC + e], kv[e], s);
      }
      const int j = j0 + fo;
      const bool vis = active && j <= last_key && j < k_lim;
      sc[fo] = vis ? s * a.scale_log2e : -INFINITY;
      mb = fmaxf(mb, sc[fo]);
    }
    const float m_new = fmaxf(m, mb);
    if (m_new != -INFINITY) {
      const float corr = fast_exp2(m - m_new);   // 0 when m was -inf
      l *= corr;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= corr;
#pragma unroll
      for (int fo = 0; fo < F; ++fo) {
        const float p = fast_exp2(sc[fo] - m_new);   // 0 for hidden keys
        l += p;
        const uint4* vrow = stage + CHUNKS + (fo * ROWS + ri) * CPR;
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
          float vv[VPC];
          Elem<T>::unpack(vrow[c], vv);
#pragma unroll
          for (int e = 0; e < VPC; ++e) acc[c * VPC + e] = fmaf(p, vv[e], acc[c * VPC + e]);
        }
      }
      m = m_new;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the wavefronts' partial results -------------------------------
  __syncthreads();   // staging slices are reused for the merge
  float* mf = reinterpret_cast<float*>(lds);
  if (wave > 0) {
    float* dst = mf + (wave - 1) * C::MERGE_F + lane;
    dst[0] = m;
    dst[64] = l;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[(d + 2) * 64] = acc[d];
  }
  __syncthreads();
  if (wave == 0) {
    float mw[kWaves];
    mw[0] = m;
    float m_all = m;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      mw[w] = mf[(w - 1) * C::MERGE_F + lane];
      m_all = fmaxf(m_all, mw[w]);
    }
    if (active && m_all != -INFINITY) {
      const float s0 = fast_exp2(m - m_all);
      float lt = l * s0;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= s0;
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        const float* src = mf + (w - 1) * C::MERGE_F + lane;
        const float sw = fast_exp2(mw[w] - m_all);   // 0 for a wave with no visible key
        lt = fmaf(src[64], sw, lt);
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(src[(d + 2) * 64], sw, acc[d]);
      }
      const float inv = 1.f / lt;
      T* op = static_cast<T*>(a.out);
      const int b = row / rpb, rr = row % rpb;
      const int64_t off = ((int64_t)(b * a.n + qi) * rpb + rr) * D;
#pragma unroll
      for (int c = 0; c < CPR; ++c) {
        float o[VPC];
#pragma unroll
        for (int e = 0; e < VPC; ++e) o[e] = acc[c * VPC + e] * inv;
        *reinterpret_cast<uint4*>(op + off + c * VPC) = Elem<T>::pack(o);
      }
    }
  }
}

// ----------------------------------------------------------------------------
// bf16 kernel: dimension-split rows, K/V streamed from HBM into registers
// ----------------------------------------------------------------------------
// A row (b, s, h) is served by 4*QH lanes: 4 dimension groups x QH query
// groups of 4 queries. Lane g of a quad holds dims {chunks g, g+4, ...} of the
// row (16-byte pieces) plus dword g of a leftover chunk (d = 72: 2 chunks + 1
// dword = 18 dims), so every load is aligned and the quad covers the row.
// q.k is a v_dot2_f32_bf16 partial sum reduced across the quad with two DPP
// adds; the softmax statistics and the accumulators for the lane's dims stay
// in registers. Keys are taken in pairs from a 4-slot register ring (one
// pair in flight while the other is processed): the pair's P is rounded to
// bf16 and O += P V is one v_dot2_f32_bf16 per dimension and query over the
// two keys (fp32 accumulate), the normaliser the same dot product with (1, 1).
// The running maximum is only raised when a score exceeds it by more than
// 2^8 (base-2 units), so the accumulators are rescaled a handful of times per
// row instead of once per key.
// When rows are few, the key range is split over up to 4 wavefronts of a
// workgroup and the partial results are merged through LDS. Pairs of queued
// keys skip the causal mask (every query sees them), and the raise test is
// two compares against a threshold kept beside the maximum.

constexpr int kQPL = 4;              // queries per lane

// U: the workgroup's rows lie in one batch and a frame is under 4 GiB
// (checked at launch), so a key's address is a wavefront-uniform frame base
// plus per-lane 32-bit offsets (no vector address arithmetic per key).
template <int D, int QH, bool U>
__global__ __launch_bounds__(256) void temporal_attn_ds_kernel(TemporalArgs a, int splits) {
  using G = DsGeom<D>;
  constexpr int DW = G::DW, DPL = G::DPL;
  constexpr int LPR = 4 * QH;          // lanes per row
  constexpr int ROWS = 64 / LPR;       // rows per wavefront
  extern __shared__ float merge_lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: key ranges, branches
  const int g = lane & 3;                          // dimension group
  const int qg = (lane >> 2) % QH;                 // query group
  const int ri = lane / LPR;
  const int q0 = blockIdx.y * (kQPL * QH);         // first query frame of this block
  const int row = blockIdx.x * ROWS + ri;
  const bool row_ok = row < a.rows_total;
  const int rpb = a.rows_per_batch;
  const int b = U ? min(blockIdx.x * ROWS, a.rows_total - 1) / rpb : row_ok ? row / rpb : 0;
  const int rr = U ? min(row, a.rows_total - 1) - b * rpb : row_ok ? row % rpb : 0;
  const int64_t row_bytes = (int64_t)rr * D * 2;
  const int64_t frame_bytes = (int64_t)rpb * D * 2;
  const uint32_t o16 = (uint32_t)row_bytes + 16 * g;                    // (U)
  const uint32_t o4 = (uint32_t)row_bytes + 64 * G::FULL + 4 * g;

  const unsigned char* qb = static_cast<const unsigned char*>(a.q);
  const unsigned char* knb = static_cast<const unsigned char*>(a.k_new);
  const unsigned char* vnb = static_cast<const unsigned char*>(a.v_new);
  const unsigned char* rkb = static_cast<const unsigned char*>(a.ring_k);
  const unsigned char* rvb = static_cast<const unsigned char*>(a.ring_v);

  // queries of this lane: frames q0+qg*4 .. q0+qg*4+3 (dims of this lane only)
  const int k_total = a.p_k + a.n;
  Slice<D> qs[kQPL];
  bool qok[kQPL];
  int last_key[kQPL];
#pragma unroll
  for (int qq = 0; qq < kQPL; ++qq) {
    const int qi = q0 + qg * kQPL + qq;
    qok[qq] = row_ok && qi < a.n;
    last_key[qq] = !qok[qq] ? -1 : a.causal ? a.p_k + qi : k_total - 1;
    if (qok[qq]) {
      if (U) load_slice_at<D>(qs[qq], qb + ((int64_t)b * a.n + qi) * frame_bytes, o16, o4);
      else load_slice<D>(qs[qq], qb + ((int64_t)b * a.n + qi) * frame_bytes + row_bytes, g);
    } else {
#pragma unroll
      for (int w = 0; w < DW; ++w) qs[qq].w[w] = 0u;
    }
  }

  // key range of this wavefront, within the keys the block's queries can see
  const int k_lim = a.causal ? min(k_total, a.p_k + q0 + kQPL * QH) : k_total;
  const int per = (k_lim + splits - 1) / splits;
  const int kb = wave * per;
  const int ke = min(k_lim, kb + per);

  auto key_row = [&](int j, const unsigned char* ring, const unsigned char* fresh) -> const unsigned char* {
    if (j < a.ring_keys) {
      int slot = a.head + j;
      if (slot >= a.p_max) slot -= a.p_max;
      return ring + ((int64_t)b * a.p_max + slot) * frame_bytes + row_bytes;
    }
    return fresh + ((int64_t)b * a.n + (j - a.p_k)) * frame_bytes + row_bytes;
  };

  // K/V slices of keys j .. j+3 in a 4-slot register ring, consumed in pairs:
  // while the pair (j, j+1) is processed the pair (j+2, j+3) is in flight,
  // and the slots of (j, j+1) are refilled with (j+4, j+5) right after.
  constexpr int kPF = 4;
  Slice<D> kr[kPF], vr[kPF];
  // K and V of key jn into ring slot u, if jn is in the range (U: the queue
  // or the new frames by a uniform select, the same per-lane offsets for both)
  auto refill = [&](int u, int jn) {
    if (jn >= ke) return;
    if constexpr (U) {
      const bool queued = jn < a.ring_keys;
      int slot = a.head + jn;
      if (slot >= a.p_max) slot -= a.p_max;
      const int64_t fo = queued ? ((int64_t)b * a.p_max + slot) * frame_bytes
                                : ((int64_t)b * a.n + (jn - a.p_k)) * frame_bytes;
      load_slice_at<D>(kr[u], (queued ? rkb : knb) + fo, o16, o4);
      load_slice_at<D>(vr[u], (queued ? rvb : vnb) + fo, o16, o4);
    } else if (row_ok) {
      load_slice<D>(kr[u], key_row(jn, rkb, knb), g);
      load_slice<D>(vr[u], key_row(jn, rvb, vnb), g);
    }
  };

  float m[kQPL], thr[kQPL], l[kQPL], acc[kQPL][DPL];
#pragma unroll
  for (int qq = 0; qq < kQPL; ++qq) {
    m[qq] = kNoMax;
    thr[qq] = kNoMax;
    l[qq] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[qq][e] = 0.f;
  }

#pragma unroll
  for (int u = 0; u < kPF; ++u) refill(u, kb + u);
  // One key pair: scores, lazy rescale, then P of the pair rounded to bf16 and
  // O += P V as bf16 dot products over the two keys (one v_dot2 per dimension
  // and query; the row sum is the same dot product with (1, 1), so numerator
  // and normaliser use the same rounded P). `two` (wavefront-uniform) is false
  // when key j+1 is past the range: its score is -inf and its V words are
  // zeroed, so a stale slot cannot turn 0 * V into NaN. Pairs of keys that
  // every query of the range sees (queued keys, both within the range) skip
  // the mask.
  const int unmasked_end = min(a.p_k, ke);
  auto process2 = [&](int j, const Slice<D>& k0, const Slice<D>& v0, const Slice<D>& k1, const Slice<D>& v1,
                      bool two) {
    const bool mask = j + 1 >= unmasked_end;       // wavefront-uniform
    float x0[kQPL], x1[kQPL];
    bool raise = false;
#pragma unroll
    for (int qq = 0; qq < kQPL; ++qq) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int w = 0; w < DW; ++w) {
        s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, qs[qq].w[w]),
                                             __builtin_bit_cast(bf16x2v, k0.w[w]), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, qs[qq].w[w]),
                                             __builtin_bit_cast(bf16x2v, k1.w[w]), s1, false);
      }
      x0[qq] = quad_sum(s0) * a.scale_log2e;
      x1[qq] = quad_sum(s1) * a.scale_log2e;
      if (mask) {
        if (j > last_key[qq]) x0[qq] = -INFINITY;
        if (!two || j + 1 > last_key[qq]) x1[qq] = -INFINITY;
      }
      raise |= (x0[qq] > thr[qq]) | (x1[qq] > thr[qq]);
    }
    if (raise) {
#pragma unroll
      for (int qq = 0; qq < kQPL; ++qq) {
        const float mn = fmaxf(m[qq], fmaxf(x0[qq], x1[qq]));
        const float corr = fast_exp2(m[qq] - mn);
        m[qq] = mn;
        thr[qq] = mn + kLazy;
        l[qq] *= corr;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[qq][e] *= corr;
      }
    }
    // V of the pair by dimension: word 2w+h holds (v0, v1) of dimension 2w+h
    uint32_t vp[DPL];
#pragma unroll
    for (int w = 0; w < DW; ++w) {
      const uint32_t b = two ? v1.w[w] : 0u;
      vp[2 * w] = __builtin_amdgcn_perm(b, v0.w[w], 0x05040100u);       // low halves
      vp[2 * w + 1] = __builtin_amdgcn_perm(b, v0.w[w], 0x07060302u);   // high halves
    }
#pragma unroll
    for (int qq = 0; qq < kQPL; ++qq) {
      const bf16x2v pp = __builtin_bit_cast(bf16x2v, pack_bf16x2(fast_exp2(x0[qq] - m[qq]), fast_exp2(x1[qq] - m[qq])));
      l[qq] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2v, 0x3F803F80u), l[qq], false);
#pragma unroll
      for (int e = 0; e < DPL; ++e)
        acc[qq][e] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2v, vp[e]), acc[qq][e], false);
    }
  };
  for (int j = kb; j < ke; j += kPF) {                   // bounds are uniform per wavefront
    process2(j, kr[0], vr[0], kr[1], vr[1], j + 1 < ke);
    refill(0, j + 4);
    refill(1, j + 5);
    if (j + 2 < ke) {
      process2(j + 2, kr[2], vr[2], kr[3], vr[3], j + 3 < ke);
      refill(2, j + 6);
      refill(3, j + 7);
    }
  }

  // merge the wavefronts of a split key range: query qq of every lane is
  // merged and stored by wave qq % splits; the other waves hand over their
  // partial state for it through LDS (slot per (query, writer))
  constexpr int SLOT = (DPL + 2) * 64;
  unsigned char* ob = static_cast<unsigned char*>(a.out);
  if (splits > 1) {
#pragma unroll
    for (int qq = 0; qq < kQPL; ++qq) {
      const int own = qq % splits;
      if (own != wave) {
        float* dst = merge_lds + (qq * (splits - 1) + (wave < own ? wave : wave - 1)) * SLOT + lane;
        dst[0] = m[qq];
        dst[64] = l[qq];
#pragma unroll
        for (int e = 0; e < DPL; ++e) dst[(2 + e) * 64] = acc[qq][e];
      }
    }
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < kQPL; ++qq) {
      if (qq % splits != wave) continue;
      for (int w = 0; w < splits - 1; ++w) {
        const float* src = merge_lds + (qq * (splits - 1) + w) * SLOT + lane;
        const float mw = src[0];
        const float mn = fmaxf(m[qq], mw);
        const float s0 = fast_exp2(m[qq] - mn);
        const float s1 = fast_exp2(mw - mn);
        m[qq] = mn;
        l[qq] = l[qq] * s0 + src[64] * s1;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[qq][e] = acc[qq][e] * s0 + src[(2 + e) * 64] * s1;
      }
    }
  }
#pragma unroll
  for (int qq = 0; qq < kQPL; ++qq) {
    if (!qok[qq] || qq % splits != wave) continue;
    const int qi = q0 + qg * kQPL + qq;
    const float inv = 1.f / l[qq];
    float o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = acc[qq][e] * inv;
    store_slice<D>(ob + ((int64_t)b * a.n + qi) * frame_bytes + row_bytes, g, o);
  }
}

template <int D, int QH>
hipError_t launch_ds_q(const TemporalArgs& a, hipStream_t s) {
  constexpr int ROWS = 64 / (4 * QH);
  constexpr int QB = kQPL * QH;                    // query frames per block
  const int groups = (a.rows_total + ROWS - 1) / ROWS;
  const int qblocks = (a.n + QB - 1) / QB;
  if (qblocks > 65535) return hipErrorInvalidValue;
  // split the key range when there are too few workgroups to fill the chip
  const int64_t wgs = (int64_t)groups * qblocks;
  int splits = (int)((2048 + wgs - 1) / wgs);
  splits = splits < 1 ? 1 : splits > 4 ? 4 : splits;
  const int k_min = a.causal ? a.p_k + (a.n < QB ? a.n : QB) : a.p_k + a.n;   // fewest keys of a block
  if (splits > k_min) splits = k_min;
  const size_t lds = splits > 1 ? (size_t)(splits - 1) * 64 * kQPL * (DsGeom<D>::DPL + 2) * sizeof(float) : 0;
  const int64_t frame_bytes = (int64_t)a.rows_per_batch * D * 2;
  if (a.rows_per_batch % ROWS == 0 && frame_bytes <= 0xFFFFFFFFll)
    hipLaunchKernelGGL((temporal_attn_ds_kernel<D, QH, true>), dim3(groups, qblocks), dim3(64 * splits), lds, s, a, splits);
  else
    hipLaunchKernelGGL((temporal_attn_ds_kernel<D, QH, false>), dim3(groups, qblocks), dim3(64 * splits), lds, s, a, splits);
  return hipGetLastError();
}

template <int D>
hipError_t launch_ds(const TemporalArgs& a, hipStream_t s) {
  if (a.n <= 4) return launch_ds_q<D, 1>(a, s);
  if (a.n <= 8) return launch_ds_q<D, 2>(a, s);
  return launch_ds_q<D, 4>(a, s);
}

// ----------------------------------------------------------------------------
// bf16 kernel on the matrix cores: whole rows per wavefront (selectable)
// ----------------------------------------------------------------------------
// Each wavefront computes `rpw` consecutive rows with temporal_mfma_rows
// (scores, the transposition of V and O = P V on v_mfma_f32_16x16x32_bf16,
// 32 keys per step, one step's loads in flight while the previous step is
// computed). Up to 16 query frames per row. Rows per wavefront are chosen so
// that the launch is about one round of two wavefronts per SIMD (the register
// budget), which keeps eight steps' K/V in flight per compute unit. It cuts
// the VALU work per row about fourfold but is slower than the dimension-split
// kernel: a wavefront reads one row's keys at a time (16 scattered 64-byte
// pieces per load instead of whole runs of adjacent rows) and each 32-key
// step is a dependent chain of MFMAs, two cross-lane exchanges and the
// exponentials, so it is only run when forced (ca2_set_temporal_variant(2)).
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void temporal_mfma_kernel(TemporalArgs a, int rpw) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int first = (blockIdx.x * 4 + wave) * rpw;
  const int rows = max(0, min(rpw, a.rows_total - first));
  temporal_mfma_rows<D>(a, [&](int i) { return first + i; }, rows, 0);
}

template <int D>
hipError_t launch_tm(const TemporalArgs& a, hipStream_t s) {
  const int waves_target = 8 * device_cus_t();
  int rpw = (a.rows_total + waves_target - 1) / waves_target;
  rpw = rpw < 1 ? 1 : rpw;
  const int64_t waves = ((int64_t)a.rows_total + rpw - 1) / rpw;
  const int64_t wgs = (waves + 3) / 4;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((temporal_mfma_kernel<D>), dim3((unsigned)wgs), dim3(256), 0, s, a, rpw);
  return hipGetLastError();
}

// Launch variant forced by ca2_set_temporal_variant (0 = chosen by shape).
std::atomic<int> g_forced_temporal{0};

template <typename T, int D>
hipError_t launch_td(const TemporalArgs& a, hipStream_t s) {
  const int ql = a.n <= 4 ? 4 : a.n <= 8 ? 8 : 16;
  const int rows = 64 / ql;
  const int qblocks = (a.n + ql - 1) / ql;
  if (qblocks > 65535) return hipErrorInvalidValue;
  const dim3 grid((a.rows_total + rows - 1) / rows, qblocks);
  const dim3 block(64 * kWaves);
  if (ql == 4) hipLaunchKernelGGL((temporal_attn_kernel<T, D, 4>), grid, block, 0, s, a);
  else if (ql == 8) hipLaunchKernelGGL((temporal_attn_kernel<T, D, 8>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((temporal_attn_kernel<T, D, 16>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool temporal_supported(int dtype, int d) {
  if (dtype == 0) return d == 16 || d == 32 || d == 64 || d == 72 || d == 128;
  if (dtype == 1) return d == 64 || d == 72 || d == 128;
  return false;
}

hipError_t launch_temporal(int dtype, int d, const TemporalArgs& a, hipStream_t s) {
  if (a.n < 1 || a.p_k < 0) return hipErrorInvalidValue;
  // ring keys: the queue, or the queue and the new frames; slot = head + j
  // needs at most one wrap
  if (a.ring_keys != a.p_k && a.ring_keys != a.p_k + a.n) return hipErrorInvalidValue;
  if (a.ring_keys > 0 && (a.head < 0 || a.head >= a.p_max || a.ring_keys > a.p_max)) return hipErrorInvalidValue;
  if (dtype == 0) {
    switch (d) {
      case 16: return launch_td<float, 16>(a, s);
      case 32: return launch_td<float, 32>(a, s);
      case 64: return launch_td<float, 64>(a, s);
      case 72: return launch_td<float, 72>(a, s);
      case 128: return launch_td<float, 128>(a, s);
    }
  } else if (dtype == 1) {
    // the dimension-split kernel; the matrix-core rows only when forced
    // (they measured slower at every shape: the 256-token call 16.7 vs
    // 14.7 us, the 32x32-latent batch 435 vs 318 us)
    const bool mfma = g_forced_temporal.load(std::memory_order_relaxed) == 2;
    switch (d) {
      case 64: return mfma && a.n <= kTmMaxQ ? launch_tm<64>(a, s) : launch_ds<64>(a, s);
      case 72: return mfma && a.n <= kTmMaxQ ? launch_tm<72>(a, s) : launch_ds<72>(a, s);
      case 128: return launch_ds<128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

void set_temporal_variant(int v) { g_forced_temporal.store(v, std::memory_order_relaxed); }
int temporal_variant() { return g_forced_temporal.load(std::memory_order_relaxed); }

}  // namespace ca2
