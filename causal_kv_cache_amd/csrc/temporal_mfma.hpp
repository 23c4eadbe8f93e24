// Causal temporal attention of whole rows on the matrix cores (gfx950): the
// selectable alternative to the dimension-split VALU kernel.
//
// Ca2-VDM notes, key design 1 (CausalAttn with its lower-triangular mask) and
// key design 4 (the FIFO queue of at most P_max cached frames): for a row
// (b, s, h) and new frame i < n, softmax over the P_k queued frames and new
// frames 0..i of scale * q_i . k, times V.
//
// One wavefront computes one row at a time with v_mfma_f32_16x16x32_bf16
// (lane l, r = l % 16, g = l / 16: A operand row r, k = 8g..8g+7; B operand
// column r, k = 8g..8g+7; result column r, rows 4g..4g+3):
//   * scores S^T = K Q^T per block of 16 keys (A = 16 key rows x 32 dims in
//     their natural layout, B = the row's queries as columns, up to 16), so a
//     lane holds 4 keys of one query;
//   * V is turned into V^T by the matrix cores themselves: a block of 16 keys
//     x 32 dims times a 32 x 16 selection matrix (entries 1.0) yields 16 keys
//     x 16 dims exactly, laid out with one dim per lane and 4 keys per lane,
//     which is the A-operand layout of O^T = V^T P^T;
//   * keys are taken 32 at a time (two blocks; the k index of the PV product
//     runs over keys 4g..4g+3 of the first block, then of the second, the
//     same order for V^T and P^T), with an online softmax in base 2 whose
//     maximum is raised lazily (past 2^kLazy);
//   * V has a column of 1.0 at dim d, so row d of O^T is the softmax
//     normaliser, computed from the same bf16-rounded P as the numerator.
// Work per row is padded to 16 queries and 32-key steps; the exponentials and
// conversions left on the VALU are about a quarter of what the
// dimension-split kernel's dot products cost, but the kernel measured slower
// than it (see temporal_attn.hip), so it runs only when forced.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"
#include "temporal_common.hpp"

namespace ca2 {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kTmMaxQ = 16;   // query frames of a row (the columns of one MFMA)

template <int D>
struct TmGeom {
  static constexpr int KU = (D + 31) / 32;       // QK k-steps of 32 dims
  static constexpr int VU = (D + 1 + 31) / 32;   // 32-dim blocks of V including the 1.0 column at dim D
  static constexpr int DT = (D + 1 + 15) / 16;   // 16-dim blocks of O^T including the normaliser row
  static_assert(D % 8 == 0, "rows are whole 16-byte chunks");
};

// K and V of one block of 16 keys, as this lane holds them (key r, dims 32u + 8g .. +7)
template <int D>
struct TmBlock {
  uint4 k[TmGeom<D>::KU];
  uint4 v[TmGeom<D>::VU];
};

__device__ __forceinline__ f32x4v mfma16(const uint4& a, const uint4& b, f32x4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a), __builtin_bit_cast(bf16x8v, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ uint4 pack_bf16x8(const f32x4v& lo, const f32x4v& hi) {
  return make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                    pack_bf16x2(hi[2], hi[3]));
}

// Loads of one 16-key block: key j = first + r of the row (clamped into the
// row's keys; the caller masks the rest), 16 bytes per lane per 32-dim step.
// Entries past d are 0 for K and, for V, 1.0 at dim d.
template <int D, typename RowFn>
__device__ __forceinline__ void tm_load_block(TmBlock<D>& blk, int first, int k_total, int r, int g, RowFn key_row) {
  using G = TmGeom<D>;
  const int j = min(first + r, k_total - 1);
  const unsigned char* kp = key_row(j, true);
  const unsigned char* vp = key_row(j, false);
#pragma unroll
  for (int u = 0; u < G::KU; ++u) {
    const int d0 = 32 * u + 8 * g;
    blk.k[u] = make_uint4(0, 0, 0, 0);
    if (d0 < D) blk.k[u] = *reinterpret_cast<const uint4*>(kp + d0 * 2);
  }
#pragma unroll
  for (int u = 0; u < G::VU; ++u) {
    const int d0 = 32 * u + 8 * g;
    blk.v[u] = make_uint4(d0 == D ? 0x3F80u : 0u, 0, 0, 0);
    if (d0 < D) blk.v[u] = *reinterpret_cast<const uint4*>(vp + d0 * 2);
  }
}

// One row's running state and the operations on it.
template <int D>
struct TmRow {
  using G = TmGeom<D>;
  uint4 qop[G::KU];          // B operand: query r, dims 32u + 8g .. +7 (0 past n and past d)
  f32x4v acc[G::DT];         // O^T: query r, dims 16t + 4g .. +3
  float m;                   // running maximum (base 2) of query r, kNoMax before the first raise
  int last_key;              // keys 0..last_key are visible to query r (-1: query past n)

  // a new row: qop already holds its queries
  __device__ __forceinline__ void start(int last) {
#pragma unroll
    for (int t = 0; t < G::DT; ++t) acc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
    m = kNoMax;
    last_key = last;
  }

  // Keys first .. first+31 from blocks b0 (keys first..+15) and b1 (+16..+31).
  // sel0 / sel1: the selection matrices that pick dims 32u .. +15 and
  // 32u + 16 .. +31 of a 32-dim block.
  __device__ __forceinline__ void step(const TmBlock<D>& b0, const TmBlock<D>& b1, int first, float c, int g,
                                       const uint4& sel0, const uint4& sel1) {
    const f32x4v z = {0.f, 0.f, 0.f, 0.f};
    f32x4v s0 = z, s1 = z;
#pragma unroll
    for (int u = 0; u < G::KU; ++u) {
      s0 = mfma16(b0.k[u], qop[u], s0);
      s1 = mfma16(b1.k[u], qop[u], s1);
    }
    // V^T of both blocks, 16 dims at a time, rounded back to bf16 (exact)
    uint4 vt[G::DT];
#pragma unroll
    for (int t = 0; t < G::DT; ++t) {
      const uint4& sel = (t & 1) ? sel1 : sel0;
      vt[t] = pack_bf16x8(mfma16(b0.v[t / 2], sel, z), mfma16(b1.v[t / 2], sel, z));
    }
    // scaled scores, masked past each query's last visible key
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j0 = first + 4 * g + e, j1 = first + 16 + 4 * g + e;
      x[e] = j0 <= last_key ? s0[e] * c : -INFINITY;
      x[4 + e] = j1 <= last_key ? s1[e] * c : -INFINITY;
    }
    float mx = __builtin_fmaxf(__builtin_fmaxf(x[0], x[1]), __builtin_fmaxf(x[2], x[3]));
    mx = __builtin_fmaxf(mx, __builtin_fmaxf(__builtin_fmaxf(x[4], x[5]), __builtin_fmaxf(x[6], x[7])));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = mx > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float mn = need ? mx : m;
      const float corr = fast_exp2(m - mn);
      m = mn;
#pragma unroll
      for (int t = 0; t < G::DT; ++t) acc[t] *= corr;
    }
    f32x4v p0, p1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p0[e] = fast_exp2(x[e] - m);
      p1[e] = fast_exp2(x[4 + e] - m);
    }
    const uint4 pt = pack_bf16x8(p0, p1);
#pragma unroll
    for (int t = 0; t < G::DT; ++t) acc[t] = mfma16(vt[t], pt, acc[t]);
  }

  // out row of query r (bf16, d values): O = acc / normaliser, stored 4 dims per lane and block
  __device__ __forceinline__ void finish(unsigned char* orow, bool q_ok, int r, int g) {
    constexpr int TONE = D / 16, GONE = (D % 16) / 4, EONE = D % 4;
    const float l = __shfl(acc[TONE][EONE], r + 16 * GONE);
    const float inv = 1.f / l;
    if (!q_ok) return;
#pragma unroll
    for (int t = 0; t < G::DT; ++t) {
      const int d0 = 16 * t + 4 * g;
      if (d0 + 4 <= D) {
        uint2 w;
        w.x = pack_bf16x2(acc[t][0] * inv, acc[t][1] * inv);
        w.y = pack_bf16x2(acc[t][2] * inv, acc[t][3] * inv);
        *reinterpret_cast<uint2*>(orow + d0 * 2) = w;
      }
    }
  }
};

// Selection matrix operand (B, 32 x 16) picking dims 16h .. 16h+15 of a
// 32-dim block: lane (column r, g) holds entries k = 8g .. 8g+7, with 1.0 at
// k = r + 16h.
__device__ __forceinline__ uint4 tm_select(int h, int r, int g) {
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  const int e = r & 7;
  if (g == 2 * h + (r >> 3)) w[e >> 1] = (e & 1) ? 0x3F800000u : 0x3F80u;
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The rows row_of(0) .. row_of(rows - 1) of a launch, one wavefront, taking
// exactly `bars` workgroup barriers (0 for a wavefront that shares no
// barriers), spread evenly over its 32-key steps. The loads of the next step
// (and of the next row's queries) are issued before the barriers that precede
// the current step, so they arrive while other work runs.
template <int D, typename RowOf>
__device__ __forceinline__ void temporal_mfma_rows(const TemporalArgs& a, RowOf row_of, int rows, int bars) {
  using G = TmGeom<D>;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int rpb = a.rows_per_batch;
  const int64_t frame_bytes = (int64_t)rpb * D * 2;
  const unsigned char* qb = static_cast<const unsigned char*>(a.q);
  const unsigned char* knb = static_cast<const unsigned char*>(a.k_new);
  const unsigned char* vnb = static_cast<const unsigned char*>(a.v_new);
  const unsigned char* rkb = static_cast<const unsigned char*>(a.ring_k);
  const unsigned char* rvb = static_cast<const unsigned char*>(a.ring_v);
  unsigned char* ob = static_cast<unsigned char*>(a.out);
  const int k_total = a.p_k + a.n;
  const int steps = (k_total + 31) / 32;          // 32-key steps per row
  const int items = rows * steps;
  auto base = [&](int row, int64_t& row_bytes) {
    row_bytes = (int64_t)(row % rpb) * D * 2;
    return row / rpb;
  };
  auto load_item = [&](int it, TmBlock<D>& b0, TmBlock<D>& b1, uint4 (&qn)[G::KU]) {
    const int row = row_of(it / steps), st = it % steps;
    int64_t rb;
    const int b = base(row, rb);
    auto key_row = [&](int j, bool isk) -> const unsigned char* {
      if (j < a.ring_keys) {
        int slot = a.head + j;
        if (slot >= a.p_max) slot -= a.p_max;
        return (isk ? rkb : rvb) + ((int64_t)b * a.p_max + slot) * frame_bytes + rb;
      }
      return (isk ? knb : vnb) + ((int64_t)b * a.n + (j - a.p_k)) * frame_bytes + rb;
    };
    tm_load_block<D>(b0, 32 * st, k_total, r, g, key_row);
    tm_load_block<D>(b1, 32 * st + 16, k_total, r, g, key_row);
    if (st == 0) {                                  // the row's queries (query r)
      const unsigned char* qrow = qb + ((int64_t)b * a.n + min(r, a.n - 1)) * frame_bytes + rb;
#pragma unroll
      for (int u = 0; u < G::KU; ++u) {
        const int d0 = 32 * u + 8 * g;
        qn[u] = make_uint4(0, 0, 0, 0);
        if (r < a.n && d0 < D) qn[u] = *reinterpret_cast<const uint4*>(qrow + d0 * 2);
      }
    }
  };
  const uint4 sel0 = tm_select(0, r, g), sel1 = tm_select(1, r, g);
  TmRow<D> row_st;
  TmBlock<D> x0, x1, y0, y1;
  uint4 qn[G::KU];
  int taken = 0;
  auto item = [&](TmBlock<D>& c0, TmBlock<D>& c1, TmBlock<D>& n0, TmBlock<D>& n1, int it) {
    const int st = it % steps;
    if (st == 0) {                                  // a new row: its queries were loaded with this item
#pragma unroll
      for (int u = 0; u < G::KU; ++u) row_st.qop[u] = qn[u];
      row_st.start(r < a.n ? (a.causal ? a.p_k + r : k_total - 1) : -1);
    }
    if (it + 1 < items) load_item(it + 1, n0, n1, qn);
    const int upto = (int)(((int64_t)(it + 1) * bars) / items);
    while (taken < upto) {
      __builtin_amdgcn_s_barrier();
      ++taken;
    }
    row_st.step(c0, c1, 32 * st, a.scale_log2e, g, sel0, sel1);
    if (st == steps - 1) {
      int64_t rb;
      const int b = base(row_of(it / steps), rb);
      row_st.finish(ob + ((int64_t)b * a.n + min(r, a.n - 1)) * frame_bytes + rb, r < a.n, r, g);
    }
  };
  if (items > 0) {
    load_item(0, x0, x1, qn);
    for (int it = 0; it < items; it += 2) {
      item(x0, x1, y0, y1, it);
      if (it + 1 < items) item(y0, y1, x0, x1, it + 1);
    }
  }
  while (taken < bars) {
    __builtin_amdgcn_s_barrier();
    ++taken;
  }
}

}  // namespace ca2
