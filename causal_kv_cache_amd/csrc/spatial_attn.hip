// Prefix-enhanced spatial attention (gfx950).
//
// Ca2-VDM notes, key design 3: each target frame's S queries attend to its own
// S keys concatenated (along the token axis) with the S keys of each of the
// last P' prefix frames -- an S x (P'+1)S map; clean frames use their own keys
// only (the self-repeat case). Key design 5: those prefix frames come from the
// one-chunk spatial KV buffer.
//
// bf16 path = flash attention on MFMA (v_mfma_f32_32x32x16_bf16):
//   * workgroup = 4 wavefronts x 32 queries of one (b, frame, head);
//   * key tiles of 64 keys are staged in LDS: K row-major (row stride d*2
//     bytes: 16-byte reads by 8 consecutive rows hit distinct banks), V
//     transposed (V^T[dim][key], row stride 136 bytes) while staging;
//   * per tile each wavefront computes S^T = K Q^T (keys x queries) so a lane
//     owns one query column: the softmax row statistics are per lane, shared
//     with the partner lane (lane ^ 32) by one exchange, and the exponentiated
//     scores are already laid out as the B operand of O^T = V^T P^T -- they
//     never leave registers;
//   * online softmax in base 2 (scale * log2 e folded into one FMA), fp32
//     statistics, P rounded to bf16 for the PV product, fp32 accumulators.
// The fp32 path (for fp32 caches) is a plain LDS-tiled VALU kernel.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ca2 {
namespace {

// ----------------------------------------------------------------------------
// bf16 MFMA kernel
// ----------------------------------------------------------------------------
constexpr int kBN = 64;                  // keys per tile
constexpr int kSW = 4;                   // wavefronts per workgroup
constexpr int kVtStride = kBN * 2 + 8;   // bytes per V^T row in LDS
constexpr float kNoMax = -1.0e30f;       // running max before the first tile
constexpr float kLazy = 8.0f;            // raise the running max only past this margin (base 2)

template <int D>
struct SCfg {
  static constexpr int KSTEPS = (D + 15) / 16;     // QK^T contraction steps of 16 dims
  static constexpr int DBLK = (D + 31) / 32;       // PV output blocks of 32 dims
  static constexpr int DP = DBLK * 32;             // V^T rows incl. padding rows
  static constexpr bool ONES = DP > D;             // padding row D holds 1.0: MFMA row sums
  static constexpr int CPR = D / 8;                // 16-byte chunks per key row
  // K row stride in LDS: d*2 bytes, +16 when d*2 is a multiple of 128 so that
  // 8 consecutive rows start in distinct banks
  static constexpr int KSTR = D * 2 + ((D * 2) % 128 == 0 ? 16 : 0);
  static constexpr int K_BYTES = kBN * KSTR + 32;  // + zero pad read by the last k-step
  static constexpr int VT_BYTES = DP * kVtStride;
  static constexpr int BUF = K_BYTES + VT_BYTES;   // one stage
  static constexpr int K_CHUNKS = kBN * CPR;       // 16-byte K pieces per tile
  static constexpr int K_PER_T = (K_CHUNKS + 64 * kSW - 1) / (64 * kSW);
  static constexpr int V_UNITS = (kBN / 4) * CPR;  // (4 keys x 8 dims) V pieces per tile
  static_assert(D % 8 == 0, "head_dim must be a multiple of 8");
  static_assert(V_UNITS <= 64 * kSW, "one V unit per thread");
};

// max of a lane's value and its partner lane (lane ^ 32)
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// QB query blocks of 32 per wavefront (32*QB*kSW queries per workgroup).
template <int D, int QB>
__global__ __launch_bounds__(64 * kSW) void spatial_attn_mfma_kernel(SpatialArgs a) {
  using C = SCfg<D>;
  constexpr int KSTEPS = C::KSTEPS, DBLK = C::DBLK, DP = C::DP, CPR = C::CPR, KSTR = C::KSTR;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;            // k-half of the MFMA operands
  const int col = lane & 31;             // query column owned by this lane
  const int head = blockIdx.y % a.heads;
  const int f = blockIdx.y / a.heads;
  const int b = blockIdx.z;
  const int S = a.tokens;
  const int64_t tok_stride = (int64_t)a.heads * D;           // elements between tokens
  const int64_t own_off = (((int64_t)b * a.n + f) * S) * tok_stride + (int64_t)head * D;
  const int q_base = blockIdx.x * (32 * QB * kSW) + wave * (32 * QB);

  // Q^T operands (B of S^T = K Q^T): dims 16s + 8*half .. +7 of each query column
  bf16x8v qop[QB][KSTEPS];
  bool q_ok[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int query = q_base + 32 * qb + col;
    q_ok[qb] = query < S;
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + own_off + (int64_t)query * tok_stride;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int d0 = 16 * s + 8 * half;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (q_ok[qb] && d0 < D) u = *reinterpret_cast<const uint4*>(qp + d0);
      qop[qb][s] = __builtin_bit_cast(bf16x8v, u);
    }
  }

  // padding of both stages: V^T rows D..DP-1 (row D = 1.0 for the row sums)
  // and the tail of the K tile read by the last k-step
  for (int st = 0; st < 2; ++st) {
    unsigned char* vt = smem + st * C::BUF + C::K_BYTES;
    for (int i = tid; i < (DP - D) * (kVtStride / 4); i += 64 * kSW) {
      const int r = i / (kVtStride / 4);
      reinterpret_cast<uint32_t*>(vt + D * kVtStride)[i] = (C::ONES && r == 0) ? 0x3F803F80u : 0u;
    }
    if (tid < 8) reinterpret_cast<uint32_t*>(smem + st * C::BUF + kBN * KSTR)[tid] = 0u;
  }

  const int tiles_per_frame = (S + kBN - 1) / kBN;
  const int n_tiles = (1 + a.n_prefix) * tiles_per_frame;

  auto frame_ptrs = [&](int kf, const bf16_t*& kbase, const bf16_t*& vbase) {
    if (kf == 0) {
      kbase = static_cast<const bf16_t*>(a.k) + own_off;
      vbase = static_cast<const bf16_t*>(a.v) + own_off;
    } else {
      const int64_t off = (((int64_t)b * a.p_slots + a.prefix_slot[kf - 1]) * S) * tok_stride +
                          (int64_t)head * D;
      kbase = static_cast<const bf16_t*>(a.sp_k) + off;
      vbase = static_cast<const bf16_t*>(a.sp_v) + off;
    }
  };

  // register staging of one tile: K pieces and one V unit per thread
  uint4 kreg[C::K_PER_T];
  uint4 vreg[4];
  const int v_unit = tid;                 // (key group kg, dim chunk c)
  const int v_kg = v_unit / CPR, v_c = v_unit % CPR;
  auto load_tile = [&](int t) {
    const int kf = t / tiles_per_frame;
    const int t0 = (t % tiles_per_frame) * kBN;
    const int nk = min(kBN, S - t0);
    const bf16_t* kbase;
    const bf16_t* vbase;
    frame_ptrs(kf, kbase, vbase);
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int e = tid + i * 64 * kSW;
      const int key = e / CPR, c = e % CPR;
      kreg[i] = make_uint4(0, 0, 0, 0);
      if (e < C::K_CHUNKS && key < nk)
        kreg[i] = *reinterpret_cast<const uint4*>(kbase + (int64_t)(t0 + key) * tok_stride + c * 8);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int key = v_kg * 4 + kk;
      vreg[kk] = make_uint4(0, 0, 0, 0);
      if (v_unit < C::V_UNITS && key < nk)
        vreg[kk] = *reinterpret_cast<const uint4*>(vbase + (int64_t)(t0 + key) * tok_stride + v_c * 8);
    }
  };
  auto store_tile = [&](int st) {
    unsigned char* ks = smem + st * C::BUF;
    unsigned char* vt = ks + C::K_BYTES;
#pragma unroll
    for (int i = 0; i < C::K_PER_T; ++i) {
      const int e = tid + i * 64 * kSW;
      if (e < C::K_CHUNKS) {
        const int key = e / CPR, c = e % CPR;
        *reinterpret_cast<uint4*>(ks + key * KSTR + c * 16) = kreg[i];
      }
    }
    if (v_unit < C::V_UNITS) {
      const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
      const uint32_t* x2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
      const uint32_t* x3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        uint2 lo, hi;     // dims 8c + 2qd and 8c + 2qd + 1, keys 4kg .. 4kg+3
        lo.x = __builtin_amdgcn_perm(x1[qd], x0[qd], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(x3[qd], x2[qd], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(x1[qd], x0[qd], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(x3[qd], x2[qd], 0x07060302u);
        const int dim = v_c * 8 + 2 * qd;
        *reinterpret_cast<uint2*>(vt + dim * kVtStride + v_kg * 8) = lo;
        *reinterpret_cast<uint2*>(vt + (dim + 1) * kVtStride + v_kg * 8) = hi;
      }
    }
  };

  f32x16 acc[QB][DBLK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][i][r] = 0.f;
  float m_run[QB];
  float l_run[QB];            // explicit row sums (only without the ones row)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = kNoMax; l_run[qb] = 0.f; }

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int st = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);       // in flight during this tile's math
    const unsigned char* ks = smem + st * C::BUF;
    const unsigned char* vt = ks + C::K_BYTES;
    const int nk = min(kBN, S - (t % tiles_per_frame) * kBN);

    // -- S^T = K Q^T: two key blocks of 32, each query block --
    f32x16 sc[QB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[qb][kb][r] = 0.f;
      const unsigned char* krow = ks + (kb * 32 + col) * KSTR;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8v kop = *reinterpret_cast<const bf16x8v*>(krow + (16 * s + 8 * half) * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[qb][s], sc[qb][kb], 0, 0, 0);
      }
    }
    // register r of sc[.][kb] holds key kb*32 + 8*(r/4) + 4*half + r%4
    if (nk < kBN) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key >= nk) sc[qb][kb][r] = -INFINITY;
          }
    }

    bf16x8v pf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // -- tile max (max3 tree), shared with the partner half --
      float mx = fmaxf(sc[qb][0][0], sc[qb][0][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sc[qb][0][r]), sc[qb][0][r + 1]);
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sc[qb][1][r]), sc[qb][1][r + 1]);
      mx = max_halves(mx) * a.scale_log2e;
      // -- lazy rescale: only when the tile max passes the running max by > 2^8 --
      if (mx > m_run[qb] + kLazy) {
        const float corr = fast_exp2(m_run[qb] - mx);
        m_run[qb] = mx;
        l_run[qb] *= corr;
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][i][r] *= corr;
      }
      const float mneg = -m_run[qb];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int kb = mm >> 1, r0 = 8 * (mm & 1);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(sc[qb][kb][r0 + 2 * e], a.scale_log2e, mneg));
          const float p1 = fast_exp2(fmaf(sc[qb][kb][r0 + 2 * e + 1], a.scale_log2e, mneg));
          if constexpr (!C::ONES) l_run[qb] += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[qb][mm] = __builtin_bit_cast(bf16x8v, make_uint4(w[0], w[1], w[2], w[3]));
      }
    }
    // -- O^T += V^T P^T: k-steps of 16 keys; element e of the operands is key
    //    16*mm + 4*half + e (+4 for e >= 4) --
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
      for (int i = 0; i < DBLK; ++i) {
        const unsigned char* vrow = vt + (i * 32 + col) * kVtStride;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (16 * mm + 4 * half) * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (16 * mm + 8 + 4 * half) * 2);
        const bf16x8v vop = __builtin_bit_cast(bf16x8v, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pf[qb][mm], acc[qb][i], 0, 0, 0);
      }
    }
    if (t + 1 < n_tiles) store_tile(st ^ 1);   // the other stage was last read in tile t-1
    __syncthreads();
  }

  // -- normalise and write: register r of acc[.][i] is dim 32i + 8(r/4) + 4*half + r%4 --
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l_tot;
    if constexpr (C::ONES) {
      // row sum = O^T row D (the ones row): register 4*((D%32)/8) + D%4 of
      // block D/32 in the lanes of half (D%8)/4; the same register of the other
      // half holds row D+4, an all-zero padding row, so adding the halves gives
      // the sum in every lane
      constexpr int RD = D % 32;
      constexpr int REG = 4 * (RD / 8) + (RD % 4);
      static_assert(RD % 8 == 0 && D + 4 < DP, "row D+4 must be a zero padding row");
      l_tot = sum_halves(acc[qb][D / 32][REG]);
    } else {
      l_tot = sum_halves(l_run[qb]);
    }
    const int query = q_base + 32 * qb + col;
    if (!q_ok[qb]) continue;
    const float inv = 1.f / l_tot;
    bf16_t* op = static_cast<bf16_t*>(a.out) + own_off + (int64_t)query * tok_stride;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * i + 8 * g + 4 * half;
        if (dim < D) {
          uint2 w;
          w.x = pack_bf16x2(acc[qb][i][4 * g + 0] * inv, acc[qb][i][4 * g + 1] * inv);
          w.y = pack_bf16x2(acc[qb][i][4 * g + 2] * inv, acc[qb][i][4 * g + 3] * inv);
          *reinterpret_cast<uint2*>(op + dim) = w;
        }
      }
  }
}

// ----------------------------------------------------------------------------
// fp32 kernel: one lane per query, K/V tiles of 32 keys in LDS
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void spatial_attn_f32_kernel(SpatialArgs a) {
  constexpr int TK = 32;
  __shared__ float kt[TK][D];
  __shared__ float vtl[TK][D];
  const int lane = threadIdx.x;
  const int head = blockIdx.y % a.heads;
  const int f = blockIdx.y / a.heads;
  const int b = blockIdx.z;
  const int S = a.tokens;
  const int64_t tok_stride = (int64_t)a.heads * D;
  const int64_t own_off = (((int64_t)b * a.n + f) * S) * tok_stride + (int64_t)head * D;
  const int query = blockIdx.x * 64 + lane;
  const bool q_ok = query < S;

  float qf[D];
  const float* qp = static_cast<const float*>(a.q) + own_off + (int64_t)query * tok_stride;
#pragma unroll
  for (int d = 0; d < D; ++d) qf[d] = q_ok ? qp[d] : 0.f;
  float m = -INFINITY, l = 0.f, acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;

  const int n_kf = 1 + a.n_prefix;
  for (int kf = 0; kf < n_kf; ++kf) {
    const float* kb;
    const float* vb;
    if (kf == 0) {
      kb = static_cast<const float*>(a.k) + own_off;
      vb = static_cast<const float*>(a.v) + own_off;
    } else {
      const int64_t off = (((int64_t)b * a.p_slots + a.prefix_slot[kf - 1]) * S) * tok_stride +
                          (int64_t)head * D;
      kb = static_cast<const float*>(a.sp_k) + off;
      vb = static_cast<const float*>(a.sp_v) + off;
    }
    for (int t0 = 0; t0 < S; t0 += TK) {
      const int nk = min(TK, S - t0);
      __syncthreads();
      for (int e = lane; e < TK * D; e += 64) {
        const int key = e / D, d = e % D;
        kt[key][d] = key < nk ? kb[(int64_t)(t0 + key) * tok_stride + d] : 0.f;
        vtl[key][d] = key < nk ? vb[(int64_t)(t0 + key) * tok_stride + d] : 0.f;
      }
      __syncthreads();
      for (int j = 0; j < nk; ++j) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(qf[d], kt[j][d], s);
        s *= a.scale_log2e;
        const float m_new = fmaxf(m, s);
        const float corr = fast_exp2(m - m_new);
        const float p = fast_exp2(s - m_new);
        l = fmaf(l, corr, p);
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(acc[d], corr, p * vtl[j][d]);
        m = m_new;
      }
    }
  }
  if (q_ok) {
    float* op = static_cast<float*>(a.out) + own_off + (int64_t)query * tok_stride;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  }
}

template <int D, int QB>
hipError_t launch_mfma_qb(const SpatialArgs& a, hipStream_t s) {
  constexpr int BM = 32 * QB * kSW;
  const dim3 grid((a.tokens + BM - 1) / BM, a.n * a.heads, a.batch);
  hipLaunchKernelGGL((spatial_attn_mfma_kernel<D, QB>), grid, dim3(64 * kSW), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const SpatialArgs& a, hipStream_t s) {
  // two query blocks per wavefront when that still gives >= 2 workgroups per CU
  const int64_t wg2 = (int64_t)((a.tokens + 255) / 256) * a.n * a.heads * a.batch;
  if (wg2 >= 512) return launch_mfma_qb<D, 2>(a, s);
  return launch_mfma_qb<D, 1>(a, s);
}

template <int D>
hipError_t launch_f32(const SpatialArgs& a, hipStream_t s) {
  const dim3 grid((a.tokens + 63) / 64, a.n * a.heads, a.batch);
  hipLaunchKernelGGL((spatial_attn_f32_kernel<D>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool spatial_supported(int dtype, int d) {
  if (dtype == 0) return d == 16 || d == 32 || d == 64 || d == 72 || d == 128;
  if (dtype == 1) return d == 64 || d == 72 || d == 128;
  return false;
}

hipError_t launch_spatial(int dtype, int d, const SpatialArgs& a, hipStream_t s) {
  if (dtype == 0) {
    switch (d) {
      case 16: return launch_f32<16>(a, s);
      case 32: return launch_f32<32>(a, s);
      case 64: return launch_f32<64>(a, s);
      case 72: return launch_f32<72>(a, s);
      case 128: return launch_f32<128>(a, s);
    }
  } else if (dtype == 1) {
    switch (d) {
      case 64: return launch_mfma<64>(a, s);
      case 72: return launch_mfma<72>(a, s);
      case 128: return launch_mfma<128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ca2
