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

#include <cstdlib>

namespace ca2 {
namespace {

// ----------------------------------------------------------------------------
// bf16 MFMA kernel
// ----------------------------------------------------------------------------
// Pipeline: key tiles of 64 keys stream through a 3-stage LDS ring. Each tile
// is copied HBM -> LDS by global_load_lds_dwordx4 (asynchronous DMA, 16 bytes
// per lane, no register staging) two tiles ahead of its use; a wavefront waits
// only for its own copies of the tile it is about to read (s_waitcnt vmcnt),
// then one barrier per tile publishes it to the workgroup. K and V stay
// row-major in LDS; the V^T operand of the PV product is read with
// ds_read_b64_tr_b16, which transposes 16-bit data across each 16-lane group.
constexpr int kBN = 64;                  // keys per tile
constexpr float kNoMax = -1.0e30f;       // running max before the first tile
constexpr float kLazy = 8.0f;            // raise the running max only past this margin (base 2)

template <int D, int kSW>
struct SCfg {
  static constexpr int KSTEPS = (D + 15) / 16;     // QK^T contraction steps of 16 dims
  static constexpr int DBLK = (D + 31) / 32;       // PV output blocks of 32 dims
  static constexpr int DP = DBLK * 32;
  static constexpr bool ONES = DP > D;             // V row padding holds 1.0 at dim D: MFMA row sums
  static constexpr int CH = D / 8;                 // 16-byte chunks of data per key row
  // K row = KSL 16-byte slots. 8 rows read by one ds_read_b128 pass must start
  // in distinct banks: odd slot counts do that.
  static constexpr int KSL = CH % 2 ? CH : CH + 1;
  // V row = VSL slots. The transposing read touches 4 consecutive rows x 32
  // bytes per 16-lane group: rows must be 8 or 24 dwords apart mod 32.
  static constexpr int VSL = (CH + 1) % 8 == 2 || (CH + 1) % 8 == 6 ? CH + 1 : (CH + 2) % 8 == 2 || (CH + 2) % 8 == 6 ? CH + 2 : CH + 3;
  static constexpr int KROW = KSL * 16, VROW = VSL * 16;
  static constexpr int K_BYTES = kBN * KROW + 32;   // + pad read by the last QK k-step
  static constexpr int V_OFF = K_BYTES;
  static constexpr int V_BYTES = kBN * VROW + 64;   // + pad read past the last row
  static constexpr int STAGE = (K_BYTES + V_BYTES + 15) / 16 * 16;
  static constexpr int NI = KSL + VSL;              // 64-lane copy instructions per tile
  static constexpr int MAXI = (NI + kSW - 1) / kSW; // per wavefront
  static_assert(D % 8 == 0, "head_dim must be a multiple of 8");
  static_assert((VSL * 4) % 32 == 8 || (VSL * 4) % 32 == 24, "V row stride");
  static_assert(!ONES || VSL > CH, "ones column needs a padding slot");
};

// max / sum of a lane's value and its partner lane (lane ^ 32)
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// 16-byte global -> LDS copy for every active lane: lane i writes
// lds_addr + 16*i (lds_addr is wavefront-uniform, held in M0). The copy has
// no register result; completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* gptr, unsigned lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds_addr) : "memory", "m0");
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;

// Block index -> work index such that XCD x (which receives blocks x, x+8,
// x+16, ...) processes work items [start_x, start_x + count_x) in order.
__device__ __forceinline__ int xcd_work_index(int block, int nblocks) {
  constexpr int kXcds = 8;
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  const int x = block % kXcds, local = block / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

// QB query blocks of 32 per wavefront, kSW wavefronts per workgroup (32*QB*kSW
// queries), kStages-deep LDS ring (prefetch distance kStages-1).
template <int D, int QB, int kSW, int kStages>
__global__ __launch_bounds__(64 * kSW) __attribute__((amdgpu_waves_per_eu(2, 8))) void spatial_attn_mfma_kernel(SpatialArgs a) {
  using C = SCfg<D, kSW>;
  static_assert(kStages == 2 || kStages == 3, "ring depth");
  constexpr int KSTEPS = C::KSTEPS, DBLK = C::DBLK, KSL = C::KSL, VSL = C::VSL, CH = C::CH;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps per-wave state scalar
  const int half = lane >> 5;            // k-half of the MFMA operands
  const int col = lane & 31;             // query column owned by this lane
  const int S = a.tokens;
  // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).
  // Give every XCD a contiguous run of work items ordered (b, head, frame,
  // query block), so the query blocks of one frame and the frames sharing the
  // same prefix frames read their K/V through the same L2.
  const int nq = (S + 32 * QB * kSW - 1) / (32 * QB * kSW);
  const int w = xcd_work_index(blockIdx.x, gridDim.x);
  const int qblk = w % nq;
  const int f = (w / nq) % a.n;
  const int head = (w / (nq * a.n)) % a.heads;
  const int b = w / (nq * a.n * a.heads);
  const int64_t tok_stride = (int64_t)a.heads * D;           // elements between tokens
  const int64_t own_off = (((int64_t)b * a.n + f) * S) * tok_stride + (int64_t)head * D;
  const int q_base = qblk * (32 * QB * kSW) + wave * (32 * QB);

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

  // The Q operands must be complete before the copy stream starts: vmcnt also
  // counts the copies, so a wait for Q inside the loop would drain them too.
  wait_vmcnt<0>();

  // LDS init: zero everything once (rows past a partial tile stay finite)
  for (int i = tid; i < kStages * C::STAGE / 16; i += 64 * kSW)
    reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;

  // Copy instructions of this wavefront: j = wave, wave+4, ... < NI
  // (j < KSL: K slots j*64 .. +63; else V slots (j-KSL)*64 .. +63). A lane's
  // source offset inside a tile is fixed; lanes on padding slots copy from
  // pad_src instead (1.0 at dim d for V rows with the ones column, else
  // zeros), so every lane of a full tile is active.
  const int n_mine = (C::NI - wave + kSW - 1) / kSW;
  int g_off[C::MAXI], g_row[C::MAXI];
  bool g_pad[C::MAXI];
#pragma unroll
  for (int i = 0; i < C::MAXI; ++i) {
    const int j = wave + kSW * i;
    const bool isv = j >= KSL;
    const int slot = (isv ? j - KSL : j) * 64 + lane;
    const int row = slot / (isv ? VSL : KSL), c = slot % (isv ? VSL : KSL);
    g_pad[i] = c >= CH;
    g_row[i] = row;
    g_off[i] = row * (int)tok_stride + c * 8;
  }
  const unsigned char* pad_ones = static_cast<const unsigned char*>(a.pad_src);
  const unsigned char* pad_zero = pad_ones + 16;

  const int tiles_per_frame = (S + kBN - 1) / kBN;
  const int n_tiles = (1 + a.n_prefix) * tiles_per_frame;
  // copy stream state (scalar): next tile to copy = (frame kf_c, first key t0_c), into stage st_c
  int kf_c = 0, t0_c = 0, st_c = 0;
  auto issue_next = [&]() {
    const int nk = min(kBN, S - t0_c);
    int64_t off;
    const bf16_t* kb;
    const bf16_t* vb;
    if (kf_c == 0) {
      off = own_off;
      kb = static_cast<const bf16_t*>(a.k);
      vb = static_cast<const bf16_t*>(a.v);
    } else {
      off = (((int64_t)b * a.p_slots + a.prefix_slot[kf_c - 1]) * S) * tok_stride + (int64_t)head * D;
      kb = static_cast<const bf16_t*>(a.sp_k);
      vb = static_cast<const bf16_t*>(a.sp_v);
    }
    off += (int64_t)t0_c * tok_stride;
    const unsigned st = lds_base + st_c * C::STAGE;
    const bf16_t* kt = kb + off;
    const bf16_t* vt = vb + off;
#pragma unroll
    for (int i = 0; i < C::MAXI; ++i) {
      const int j = wave + kSW * i;
      if (j < C::NI) {                                  // uniform per wavefront
        const bool isv = j >= KSL;
        const unsigned dst = st + (isv ? C::V_OFF + (j - KSL) * 1024 : j * 1024);
        const void* src = (isv ? vt : kt) + g_off[i];
        if (g_pad[i]) src = (isv && C::ONES) ? (const void*)pad_ones : (const void*)pad_zero;
        if (nk == kBN) {
          dma16(src, dst);
        } else if (g_row[i] < nk || g_pad[i]) {           // last, partial tile of a frame
          dma16(src, dst);
        }
      }
    }
    t0_c += kBN;
    if (t0_c >= S) { t0_c = 0; ++kf_c; }
    st_c = st_c == kStages - 1 ? 0 : st_c + 1;
  };

  f32x16 acc[QB][DBLK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][i][r] = 0.f;
  float m_run[QB];
  float l_run[QB];            // explicit row sums (only without the ones column)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = kNoMax; l_run[qb] = 0.f; }

  issue_next();                                    // tile 0
  if (kStages == 3 && n_tiles > 1) issue_next();   // tile 1
  int st_r = 0;                    // stage being read
  int t0_r = 0;                    // first key of the tile being read (within its frame)

  for (int t = 0; t < n_tiles; ++t) {
    // wait for this wavefront's copies of tile t (tile t+1's may stay in
    // flight when it is a full tile, whose copy count is exact), then publish
    if (kStages == 3 && S % kBN == 0 && t + 1 < n_tiles) {
      if (n_mine == C::MAXI) wait_vmcnt<C::MAXI>(); else wait_vmcnt<C::MAXI - 1>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();                     // also: every wavefront is done with tile t-1
    if (t + kStages - 1 < n_tiles) issue_next();   // into the stage tile t-1 used

    const unsigned char* ks = smem + st_r * C::STAGE;
    const unsigned char* vs = ks + C::V_OFF;
    const int nk = min(kBN, S - t0_r);
    st_r = st_r == kStages - 1 ? 0 : st_r + 1;
    t0_r = t0_r + kBN >= S ? 0 : t0_r + kBN;
    const f32x16 zero16 = {};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // -- S^T = K Q^T for keys kb*32 .. +31 --
      f32x16 sc[QB];
      const unsigned char* krow = ks + (kb * 32 + col) * C::KROW;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8v kop = *reinterpret_cast<const bf16x8v*>(krow + (16 * s + 8 * half) * 2);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[qb][s], s == 0 ? zero16 : sc[qb], 0, 0, 0);
      }
      // register r of sc[.] holds key kb*32 + 8*(r/4) + 4*half + r%4
      if (nk < kBN) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (key >= nk) sc[qb][r] = -INFINITY;
          }
      }
      bf16x8v pf[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = __builtin_fmaxf(sc[qb][0], sc[qb][1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sc[qb][r]), sc[qb][r + 1]);
        mx = max_halves(mx) * a.scale_log2e;
        // lazy rescale: only when the max passes the running max by > 2^8
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
        for (int h2 = 0; h2 < 2; ++h2) {
          uint32_t wv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(fmaf(sc[qb][8 * h2 + 2 * e], a.scale_log2e, mneg));
            const float p1 = fast_exp2(fmaf(sc[qb][8 * h2 + 2 * e + 1], a.scale_log2e, mneg));
            if constexpr (!C::ONES) l_run[qb] += p0 + p1;
            wv[e] = pack_bf16x2(p0, p1);
          }
          pf[qb][h2] = __builtin_bit_cast(bf16x8v, make_uint4(wv[0], wv[1], wv[2], wv[3]));
        }
      }
      // -- O^T += V^T P^T over these 32 keys, k-steps of 16 (mm = 2kb + h2).
      //    Element e of the operands is key 16mm + 4*half + e (+4 for e >= 4).
      //    Transposing read: lane 16g + j addresses key row 16mm + 4*(g/2) +
      //    j/4 (+8 for the second read) at dims 32i + 16*(g%2) + 4*(j%4); it
      //    receives dim 32i + (lane%32) of keys 16mm + 4*(g/2) + 0..3.
      const int g16 = lane >> 4, j16 = lane & 15;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int mm = 2 * kb + h2;
#pragma unroll
        for (int i = 0; i < DBLK; ++i) {
          const unsigned char* p0 = vs + (16 * mm + 4 * (g16 >> 1) + (j16 >> 2)) * C::VROW +
                                    (32 * i + 16 * (g16 & 1) + 4 * (j16 & 3)) * 2;
          const bf16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
          const bf16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 8 * C::VROW));
          const bf16x8v vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pf[qb][h2], acc[qb][i], 0, 0, 0);
        }
      }
    }
  }

  // -- normalise and write: register r of acc[.][i] is dim 32i + 8(r/4) + 4*half + r%4 --
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l_tot;
    if constexpr (C::ONES) {
      // row sum = O^T row D (the ones column): register 4*((D%32)/8) + D%4 of
      // block D/32 in the lanes of half 0; the same register of half 1 holds
      // row D+4, whose V column is zero padding, so adding the halves gives
      // the sum in every lane
      constexpr int RD = D % 32;
      constexpr int REG = 4 * (RD / 8) + (RD % 4);
      static_assert(RD % 8 == 0 && D + 4 < C::DP, "row D+4 must be a zero padding row");
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
          uint2 wv;
          wv.x = pack_bf16x2(acc[qb][i][4 * g + 0] * inv, acc[qb][i][4 * g + 1] * inv);
          wv.y = pack_bf16x2(acc[qb][i][4 * g + 2] * inv, acc[qb][i][4 * g + 3] * inv);
          *reinterpret_cast<uint2*>(op + dim) = wv;
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

template <int D, int QB, int SW, int ST>
hipError_t launch_mfma_cfg(const SpatialArgs& a, hipStream_t s) {
  constexpr int BM = 32 * QB * SW;
  const int64_t nwg = (int64_t)((a.tokens + BM - 1) / BM) * a.n * a.heads * a.batch;
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((spatial_attn_mfma_kernel<D, QB, SW, ST>), dim3((unsigned)nwg), dim3(64 * SW), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const SpatialArgs& a, hipStream_t s) {
  // Large grids: 4 wavefronts x 64 queries (each LDS operand feeds two MFMAs),
  // 3-stage ring, 2 workgroups per CU. Small grids (fewer than ~4 such
  // workgroups per CU): 2 wavefronts x 32 queries with a 2-stage ring, so 4
  // workgroups fit per CU and every SIMD still runs two wavefronts.
  const int64_t frames = (int64_t)a.n * a.heads * a.batch;
  const int64_t wg_big = (int64_t)((a.tokens + 255) / 256) * frames;
  const char* force = getenv("CA2_SPATIAL_CFG");
  int cfg = wg_big >= 1024 ? 2 : 1;
  if (force) cfg = force[0] - '0';
  if constexpr (D <= 72) {
    if (cfg == 2) return launch_mfma_cfg<D, 2, 4, 3>(a, s);
  }
  if (cfg == 1) return launch_mfma_cfg<D, 1, 4, 3>(a, s);
  return launch_mfma_cfg<D, 1, 2, 2>(a, s);
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
