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
constexpr int kBN = 64;            // keys per tile
constexpr int kQW = 32;            // queries per wavefront
constexpr int kSW = 4;             // wavefronts per workgroup
constexpr int kVtStride = kBN * 2 + 8;   // bytes per V^T row in LDS

template <int D>
struct SCfg {
  static constexpr int KSTEPS = (D + 15) / 16;     // QK^T contraction steps of 16 dims
  static constexpr int DBLK = (D + 31) / 32;       // PV output blocks of 32 dims
  static constexpr int DP = DBLK * 32;             // V^T rows incl. zero rows
  static constexpr int CPR = D / 8;                // 16-byte chunks per key row
  // K row stride in LDS: d*2 bytes, +16 when d*2 is a multiple of 128 so that
  // 8 consecutive rows start in distinct banks
  static constexpr int KSTR = D * 2 + ((D * 2) % 128 == 0 ? 16 : 0);
  static constexpr int K_BYTES = kBN * KSTR + 32;  // + zero pad read by the last k-step
  static constexpr int VT_BYTES = DP * kVtStride;
  static_assert(D % 8 == 0, "head_dim must be a multiple of 8");
};

template <int D>
__global__ __launch_bounds__(64 * kSW) void spatial_attn_mfma_kernel(SpatialArgs a) {
  using C = SCfg<D>;
  constexpr int KSTEPS = C::KSTEPS, DBLK = C::DBLK, DP = C::DP, CPR = C::CPR, KSTR = C::KSTR;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::K_BYTES + C::VT_BYTES];
  unsigned char* ks = smem;
  unsigned char* vt = smem + C::K_BYTES;

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

  const int query = blockIdx.x * (kQW * kSW) + wave * kQW + col;
  const bool q_ok = query < S;

  // Q^T operand (B of S^T = K Q^T): dims 16s + 8*half .. +7 of this query.
  bf16x8v qop[KSTEPS];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + own_off + (int64_t)query * tok_stride;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const int d0 = 16 * s + 8 * half;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (q_ok && d0 < D) u = *reinterpret_cast<const uint4*>(qp + d0);
      qop[s] = __builtin_bit_cast(bf16x8v, u);
    }
  }

  // zero the pad regions once: V^T rows D..DP-1 and the tail of the K tile
  for (int i = tid; i < (DP - D) * (kVtStride / 4); i += 64 * kSW)
    reinterpret_cast<uint32_t*>(vt + D * kVtStride)[i] = 0u;
  if (tid < 8) reinterpret_cast<uint32_t*>(ks + kBN * KSTR)[tid] = 0u;

  f32x16 acc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_run = -INFINITY;   // running max (base-2 scaled) of this query
  float l_run = 0.f;         // this lane's partial normaliser

  const int n_kf = 1 + a.n_prefix;
  for (int kf = 0; kf < n_kf; ++kf) {
    const bf16_t* kbase;
    const bf16_t* vbase;
    if (kf == 0) {
      kbase = static_cast<const bf16_t*>(a.k) + own_off;
      vbase = static_cast<const bf16_t*>(a.v) + own_off;
    } else {
      const int64_t off = (((int64_t)b * a.p_slots + a.prefix_slot[kf - 1]) * S) * tok_stride +
                          (int64_t)head * D;
      kbase = static_cast<const bf16_t*>(a.sp_k) + off;
      vbase = static_cast<const bf16_t*>(a.sp_v) + off;
    }
    for (int t0 = 0; t0 < S; t0 += kBN) {
      const int nk = min(kBN, S - t0);
      __syncthreads();   // previous tile fully consumed (and pads written)
      // -- K tile, row-major --
      for (int e = tid; e < kBN * CPR; e += 64 * kSW) {
        const int key = e / CPR, c = e % CPR;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (key < nk) u = *reinterpret_cast<const uint4*>(kbase + (int64_t)(t0 + key) * tok_stride + c * 8);
        *reinterpret_cast<uint4*>(ks + key * KSTR + c * 16) = u;
      }
      // -- V tile, transposed: unit = (group of 4 keys, 8 dims) --
      for (int u_ = tid; u_ < (kBN / 4) * CPR; u_ += 64 * kSW) {
        const int kg = u_ / CPR, c = u_ % CPR;
        uint4 x[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int key = kg * 4 + kk;
          x[kk] = make_uint4(0, 0, 0, 0);
          if (key < nk) x[kk] = *reinterpret_cast<const uint4*>(vbase + (int64_t)(t0 + key) * tok_stride + c * 8);
        }
        const uint32_t* x0 = reinterpret_cast<const uint32_t*>(&x[0]);
        const uint32_t* x1 = reinterpret_cast<const uint32_t*>(&x[1]);
        const uint32_t* x2 = reinterpret_cast<const uint32_t*>(&x[2]);
        const uint32_t* x3 = reinterpret_cast<const uint32_t*>(&x[3]);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          // dims 8c + 2qd (low halves) and 8c + 2qd + 1 (high halves)
          uint2 lo, hi;
          lo.x = (x0[qd] & 0xffffu) | (x1[qd] << 16);
          lo.y = (x2[qd] & 0xffffu) | (x3[qd] << 16);
          hi.x = (x0[qd] >> 16) | (x1[qd] & 0xffff0000u);
          hi.y = (x2[qd] >> 16) | (x3[qd] & 0xffff0000u);
          const int dim = c * 8 + 2 * qd;
          *reinterpret_cast<uint2*>(vt + dim * kVtStride + kg * 8) = lo;
          *reinterpret_cast<uint2*>(vt + (dim + 1) * kVtStride + kg * 8) = hi;
        }
      }
      __syncthreads();

      // -- S^T = K Q^T for two blocks of 32 keys --
      f32x16 st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) st[kb][r] = 0.f;
        const unsigned char* krow = ks + (kb * 32 + col) * KSTR;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const bf16x8v kop = *reinterpret_cast<const bf16x8v*>(krow + (16 * s + 8 * half) * 2);
          st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[s], st[kb], 0, 0, 0);
        }
      }
      // register r of st[kb] holds key kb*32 + 8*(r/4) + 4*half + r%4
      if (nk < kBN) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key >= nk) st[kb][r] = -INFINITY;
          }
      }
      // -- online softmax (base 2) --
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * a.scale_log2e);
      const float corr = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < DBLK; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= corr;
      bf16x8v pf[4];
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
        const int kb = mm >> 1, r0 = 8 * (mm & 1);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(st[kb][r0 + 2 * e], a.scale_log2e, -m_new));
          const float p1 = fast_exp2(fmaf(st[kb][r0 + 2 * e + 1], a.scale_log2e, -m_new));
          l_run += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[mm] = __builtin_bit_cast(bf16x8v, make_uint4(w[0], w[1], w[2], w[3]));
      }
      // -- O^T += V^T P^T: k-steps of 16 keys; element e of this lane's
      //    operands is key 16*mm + 4*half + e (+4 for e >= 4) --
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) {
#pragma unroll
        for (int i = 0; i < DBLK; ++i) {
          const unsigned char* vrow = vt + (i * 32 + col) * kVtStride;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (16 * mm + 4 * half) * 2);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (16 * mm + 8 + 4 * half) * 2);
          const bf16x8v vop = __builtin_bit_cast(bf16x8v, make_uint4(lo.x, lo.y, hi.x, hi.y));
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pf[mm], acc[i], 0, 0, 0);
        }
      }
    }
  }

  // -- normalise and write: register r of acc[i] is dim 32i + 8(r/4) + 4*half + r%4 --
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (q_ok) {
    const float inv = 1.f / l_tot;
    bf16_t* op = static_cast<bf16_t*>(a.out) + own_off + (int64_t)query * tok_stride;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dim = 32 * i + 8 * g + 4 * half;
        if (dim < D) {
          uint2 w;
          w.x = pack_bf16x2(acc[i][4 * g + 0] * inv, acc[i][4 * g + 1] * inv);
          w.y = pack_bf16x2(acc[i][4 * g + 2] * inv, acc[i][4 * g + 3] * inv);
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

template <int D>
hipError_t launch_mfma(const SpatialArgs& a, hipStream_t s) {
  const dim3 grid((a.tokens + kQW * kSW - 1) / (kQW * kSW), a.n * a.heads, a.batch);
  hipLaunchKernelGGL((spatial_attn_mfma_kernel<D>), grid, dim3(64 * kSW), 0, s, a);
  return hipGetLastError();
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
