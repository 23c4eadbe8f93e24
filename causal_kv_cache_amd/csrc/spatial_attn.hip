// Prefix-enhanced spatial attention (gfx950).
//
// Ca2-VDM notes, key design 3: each target frame's S queries attend to its own
// S keys concatenated (along the token axis) with the S keys of each of the
// last P' prefix frames -- an S x (P'+1)S map; clean frames use their own keys
// only (the self-repeat case). Key design 5: those prefix frames come from the
// one-chunk spatial KV buffer.
//
// bf16 path = flash attention on MFMA (v_mfma_f32_32x32x16_bf16):
//   * a workgroup covers 4 wavefronts x 32*QB queries of one (b, frame, head)
//     (at one workgroup per CU, plus a fifth wavefront that only copies);
//   * per key tile each wavefront computes S^T = K Q^T (keys x queries) so a
//     lane owns one query column: the softmax row statistics are per lane,
//     shared with the partner lane (lane ^ 32) by one exchange, and the
//     exponentiated scores are already laid out as the B operand of
//     O^T = V^T P^T -- they never leave registers;
//   * online softmax in base 2, fp32 statistics, P rounded to bf16 for the
//     PV product, fp32 accumulators. Where d % 16 == 8 (d = 72) the last
//     16-dim QK step is half padding; there Q is multiplied by
//     scale * log2 e once (rounded to bf16) and the padding carries the
//     running maximum as three more product terms (-m split into three bf16
//     parts, against key entries of 1), so the product yields the shifted
//     base-2 scores and P is exp2 of the MFMA output with no other per-score
//     arithmetic. Elsewhere the scale and the maximum enter through one FMA
//     per score;
//     the V row padding holds 1.0 at dim d, so row d of O^T is the softmax
//     normaliser, computed by the MFMA from the same bf16 P as the numerator.
// The fp32 path (for fp32 caches) is a plain LDS-tiled VALU kernel.
#include "device_common.hpp"
#include "kernels.hpp"
#include "temporal_common.hpp"
#include "temporal_mfma.hpp"

#include <atomic>
#include <cstdlib>

namespace ca2 {
namespace {

// ----------------------------------------------------------------------------
// bf16 MFMA kernel: tile geometry and helpers
// ----------------------------------------------------------------------------
constexpr int kBN = 64;                  // keys per tile
// The running maximum starts at kNoMax (the most negative finite float, so
// any finite score raises it) and is raised lazily, only past kLazy (base 2);
// both constants come with the temporal helpers.

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

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4v lds_bf16x4;


// Lazy rescale of one query block's running state: only when a lane's new
// maximum passes its running maximum m by more than 2^kLazy (base 2). The
// test runs on the raw score maximum against thr = (m + kLazy) / c, c =
// scale * log2 e (kept with m, changed only here), and is made wave-uniform
// so the common case is one compare and one scalar branch; inside, lanes that
// keep their maximum get a factor of exactly 1.
template <int DBLK>
__device__ __forceinline__ void lazy_rescale(float mx_raw, float c, float& m_run, float& thr, float& l_run,
                                             f32x16 (&acc)[DBLK]) {
  const bool need = mx_raw > thr;
  if (__builtin_amdgcn_ballot_w64(need) == 0) return;
  const float m_new = need ? mx_raw * c : m_run;
  const float corr = fast_exp2(m_run - m_new);
  m_run = m_new;
  thr = (m_new + kLazy) / c;
  l_run *= corr;
#pragma unroll
  for (int i = 0; i < DBLK; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] *= corr;
}

// The same for scores that the product already shifts (d % 16 == 8): the
// product yields y = c s - m_run (the running maximum enters it as a sum of
// three bf16 terms, which hold a float32 value exactly), so P = exp2(y) and
// the threshold is kLazy itself (-inf: no score seen yet; m_run is then 0).
// The caller puts the new maximum's three bf16 terms into its Q operand and
// scores the chunk again.
template <int DBLK>
__device__ __forceinline__ void lazy_rescale_shifted(float mx, float& m_run, float& thr, float& l_run,
                                                     f32x16 (&acc)[DBLK]) {
  const bool need = mx > thr;          // the caller has seen some lane need it
  const bool have = thr != -INFINITY;
  const float m_new = need ? m_run + mx : m_run;
  const float corr = !need ? 1.f : have ? fast_exp2(m_run - m_new) : 0.f;   // 0: acc, l_run still 0
  thr = need ? kLazy : thr;
  m_run = m_new;
  l_run *= corr;
#pragma unroll
  for (int i = 0; i < DBLK; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] *= corr;
}

// -m as three bf16 terms whose sum is -m (a float32 has 24 significant bits,
// a bf16 8), packed as the first three entries of a bf16x8 Q operand slice.
__device__ __forceinline__ uint2 neg_bf16x3(float m) {
  const float x = -m;
  const float h = __builtin_bit_cast(float, pack_bf16x2(x, 0.f) << 16);
  const float r1 = x - h;
  const float md = __builtin_bit_cast(float, pack_bf16x2(r1, 0.f) << 16);
  const float r2 = r1 - md;
  return make_uint2(pack_bf16x2(h, md), pack_bf16x2(r2, 0.f));
}

// ----------------------------------------------------------------------------
// bf16 MFMA kernel, software-pipelined
// ----------------------------------------------------------------------------
// Data movement: key tiles of 64 keys stream through a kStages-deep LDS ring,
// row-major (K rows KROW bytes, V rows VROW bytes, both padded for
// conflict-free reads). A tile is copied HBM -> LDS by global_load_lds_dwordx4
// (asynchronous, 16 bytes per lane, no register staging): copy instruction j
// of a tile covers 16-byte slots 64j .. 64j+63 of the tile's rows, so each
// lane's global offset from the tile base is a constant, and the tile base is
// a wavefront-uniform 64-bit value -- issuing a tile takes scalar
// instructions only. Padding slots (zeros, and for d % 32 != 0 a 1.0 at dim
// d that turns row d of the PV accumulator into the softmax row sum) are
// written once at the start and never copied over (their lanes are masked).
// A wavefront waits only for its own copies of the tile it needs (s_waitcnt
// vmcnt), then one barrier per tile publishes it. With PROD an extra
// wavefront issues every copy and does that wait alone: a copy instruction
// holds its wavefront for as long as the CU's memory pipeline takes to accept
// 64 x 16 bytes, and that time then no longer falls on the wavefronts that
// compute, which only take the barrier.
//
// Compute: each wavefront cuts a tile into two chunks of 32 keys and, with
// S(c) the scores of chunk c, overlaps
//   S(c+1) = K(c+1) Q^T        (MFMA)  ||  P(c) = exp2(S(c) - m)   (VALU)
//   O     += V(c) P(c)         (MFMA)  ||  max of S(c+1)           (VALU)
// then the (rare) lazy rescale for chunk c+1. The second chunk of tile t+1 is
// scored during tile t, so tile t+1 must be resident one iteration early: at
// iteration t a wavefront waits for its copies of tile t+1 and, after the
// barrier, refills the stage of tile t-1 with tile t+kStages-1.

// The body, for the kSW (+ PROD) wavefronts of a workgroup with thread
// index tid < 64 * (kSW + PROD), work item w (frame-head-query block) and the
// ring `smem` (kStages * STAGE bytes of LDS). Every wavefront that runs it
// takes exactly n_tiles workgroup barriers.
template <int D, int QB, int kSW, bool FULL, int kStages, int KS, bool PROD>
__device__ __forceinline__ void spatial_pipe(const SpatialArgs& a, int w, int tid, unsigned char* smem) {
  using C = SCfg<D, PROD ? 1 : kSW>;
  static_assert(KS == 1 || KS == 2, "key split over one or two wavefronts");
  static_assert(!PROD || KS == 1, "a copy wavefront only with one key range per wavefront");
  constexpr int kThreads = 64 * (kSW + PROD);
  constexpr int G = kSW / KS;                      // query groups of 32*QB per workgroup
  static_assert(kStages >= 3, "the pipeline reads tile t+1 while tile t+2 is copied");
  constexpr int KSTEPS = C::KSTEPS, DBLK = C::DBLK, KSL = C::KSL, VSL = C::VSL, CH = C::CH;
  constexpr int MAXI = C::MAXI;                    // copies per wavefront per tile (upper bound)
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // PROD: wavefront kSW issues every copy and computes nothing
  const bool producer = PROD && wave == kSW;
  const int cw = PROD ? 0 : wave;                  // copy instructions cw, cw + CSW, ...
  constexpr int CSW = PROD ? 1 : kSW;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int S = a.tokens;
  const int nq = (S + 32 * QB * G - 1) / (32 * QB * G);
  const int qblk = w % nq;
  const int f = (w / nq) % a.n;
  const int head = (w / (nq * a.n)) % a.heads;
  const int b = w / (nq * a.n * a.heads);
  const int64_t tok_stride = (int64_t)a.heads * D;
  const int64_t own_off = (((int64_t)b * a.n + f) * S) * tok_stride + (int64_t)head * D;
  const int grp = wave % G;                        // query group of this wavefront
  const int kh = wave / G;                         // with KS == 2: key half of every tile
  const int q_base = qblk * (32 * QB * G) + grp * (32 * QB);

  // kShifted (d % 16 == 8): the upper half of the last QK step is padding;
  // there the Q operand holds -m_run as three bf16 terms (lanes of the upper
  // half, first three entries) against key entries of 1.0, and the rest of
  // Q holds c q
  constexpr bool kShifted = D % 16 == 8;
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
      uint4 u = make_uint4(0, 0, 0, 0);   // the upper half's shift terms start at m_run = 0
      if (!producer && q_ok[qb] && d0 < D) u = *reinterpret_cast<const uint4*>(qp + d0);
      if constexpr (kShifted) {           // c q, rounded once to bf16
        float qf[8];
        Elem<bf16_t>::unpack(u, qf);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[e] *= a.scale_log2e;
        u = Elem<bf16_t>::pack(qf);
      }
      qop[qb][s] = __builtin_bit_cast(bf16x8v, u);
    }
  }
  const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  // Padding slots and the bytes past the last K / V row are never copied:
  // write them once (the V slot at dim d holds the 1.0 of the row-sum trick).
  // Partial tiles also leave key rows uncopied, so without full tiles the
  // whole ring starts zeroed.
  if constexpr (!FULL) {
    for (int i = tid; i < kStages * C::STAGE / 16; i += kThreads)
      reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }
  {
    constexpr int KP = KSL - CH, VP = VSL - CH;           // padding slots per row
    constexpr int PER = kBN * (KP + VP) + 6;              // + 32 B after K, 64 B after V
    for (int i = tid; i < kStages * PER; i += kThreads) {
      const int st = i / PER, k = i % PER;
      int off;
      bool ones = false;
      if (KP > 0 && k < kBN * KP) {
        constexpr int kp = KP > 0 ? KP : 1;
        off = (k / kp) * C::KROW + (CH + k % kp) * 16;
      } else if (k < kBN * (KP + VP)) {
        const int kv = k - kBN * KP, c = CH + kv % VP;
        off = C::V_OFF + (kv / VP) * C::VROW + c * 16;
        ones = C::ONES && c == CH;
      } else {
        const int e = k - kBN * (KP + VP);
        off = e < 2 ? kBN * C::KROW + 16 * e : C::V_OFF + kBN * C::VROW + 16 * (e - 2);
      }
      *reinterpret_cast<uint4*>(smem + st * C::STAGE + off) = make_uint4(ones ? 0x3F80u : 0u, 0, 0, 0);
    }
  }
  if constexpr (!FULL) __syncthreads();   // ones land before any copy into the zeroed ring
  // copy stream: per-lane byte offsets of each of this wavefront's copy
  // instructions from the tile base (tile-independent), padding lanes masked
  const int n_mine = (C::NI - cw + CSW - 1) / CSW;
  const unsigned row_bytes = (unsigned)(tok_stride * 2);
  unsigned g_off[MAXI];
  int g_row[MAXI];
  bool g_pad[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int j = cw + CSW * i;
    const bool isv = j >= KSL;
    const int slot = (isv ? j - KSL : j) * 64 + lane;
    const int row = slot / (isv ? VSL : KSL), c = slot % (isv ? VSL : KSL);
    g_pad[i] = c >= CH;
    g_row[i] = row;
    g_off[i] = (unsigned)row * row_bytes + 16u * c;
  }
  // tile base pointers (bytes, this head, key 0 of the tile); the empty asm
  // keeps the argument pointers from being re-read per tile
  const unsigned char* sp_k = static_cast<const unsigned char*>(a.sp_k);
  const unsigned char* sp_v = static_cast<const unsigned char*>(a.sp_v);
  const unsigned char* fk = static_cast<const unsigned char*>(a.k) + own_off * 2;
  const unsigned char* fv = static_cast<const unsigned char*>(a.v) + own_off * 2;
  // prefix slots (< 16 each) packed 4 bits apiece into one scalar
  uint64_t pslots = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) pslots |= (uint64_t)(a.prefix_slot[i] & 15) << (4 * i);
  // key frames are streamed prefix frames first (shared by every frame of the
  // chunk, so likely already in L2) and the frame's own keys last
  const unsigned char* own_k = fk;
  const unsigned char* own_v = fv;
  asm volatile("" : "+s"(sp_k), "+s"(sp_v), "+s"(fk), "+s"(fv), "+s"(pslots), "+s"(own_k), "+s"(own_v));
  const int64_t pbase = ((int64_t)b * a.p_slots * S) * tok_stride * 2 + (int64_t)head * D * 2;
  if (a.n_prefix > 0) {
    const int64_t off0 = pbase + (int64_t)(pslots & 15) * S * tok_stride * 2;
    fk = sp_k + off0;
    fv = sp_v + off0;
  }
  const int64_t tile_bytes = (int64_t)kBN * tok_stride * 2;
  const int tiles_per_frame = (S + kBN - 1) / kBN;
  const int n_tiles = (1 + a.n_prefix) * tiles_per_frame;
  int kf_c = 0, t0_c = 0, st_c = 0;
  auto issue_next = [&]() {
    const unsigned st = lds_base + st_c * C::STAGE;
    const uint64_t bk = uniform64(reinterpret_cast<uint64_t>(fk));
    const uint64_t bv = uniform64(reinterpret_cast<uint64_t>(fv));
    const int nk = S - t0_c;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int j = cw + CSW * i;
      if (j < C::NI) {                                  // uniform per wavefront
        const bool isv = j >= KSL;
        const unsigned dst = st + (isv ? C::V_OFF + (j - KSL) * 1024 : j * 1024);
        if (!g_pad[i] && (FULL || g_row[i] < nk)) dma16s(g_off[i], isv ? bv : bk, dst);
      }
    }
    t0_c += kBN;
    fk += tile_bytes;
    fv += tile_bytes;
    if (t0_c >= S) {
      t0_c = 0;
      ++kf_c;
      if (kf_c < a.n_prefix) {
        const int slot = (int)((pslots >> (4 * kf_c)) & 15);
        const int64_t off = pbase + (int64_t)slot * S * tok_stride * 2;
        fk = sp_k + off;
        fv = sp_v + off;
      } else {
        fk = own_k;
        fv = own_v;
      }
    }
    st_c = st_c == kStages - 1 ? 0 : st_c + 1;
  };
  // wait until this wavefront's copies of the oldest outstanding tile are done
  // while `ahead` younger tiles stay in flight (exact counts need full tiles)
  auto wait_tiles = [&](int ahead) {
    if (!FULL) wait_vmcnt<0>();
    else if (n_mine == MAXI) wait_vmcnt_tiles<MAXI>(ahead);
    else wait_vmcnt_tiles<MAXI - 1>(ahead);
  };

  f32x16 acc[QB][DBLK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][i][r] = 0.f;
  float m_run[QB], l_run[QB], thr[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kShifted ? 0.f : kNoMax;
    l_run[qb] = 0.f;
    thr[qb] = kShifted ? -INFINITY : (kNoMax + kLazy) / a.scale_log2e;
  }

  const f32x16 zero16 = {};
  // S^T = K Q^T for keys kb*32 .. +31 of a tile (kShifted: c K Q^T - m_run):
  // sc[qb] register r holds key kb*32 + 8(r/4) + 4*half + r%4 of query 32*qb + col
  auto qk = [&](const unsigned char* ks, int kb, f32x16 (&sc)[QB]) {
    const unsigned char* krow = ks + (kb * 32 + col) * C::KROW;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      bf16x8v kop = *reinterpret_cast<const bf16x8v*>(krow + (16 * s + 8 * half) * 2);
      if (kShifted && s == KSTEPS - 1)      // the padding half: key entries 1.0 against -m_run
        kop = half ? __builtin_bit_cast(bf16x8v, make_uint4(0x3F803F80u, 0x3F80u, 0, 0)) : kop;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[qb][s], s == 0 ? zero16 : sc[qb], 0, 0, 0);
    }
  };
  // the same for one query block (re-scoring after a raise)
  auto qk1 = [&](const unsigned char* ks, int kb, int qb, f32x16& sc) {
    const unsigned char* krow = ks + (kb * 32 + col) * C::KROW;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      bf16x8v kop = *reinterpret_cast<const bf16x8v*>(krow + (16 * s + 8 * half) * 2);
      if (kShifted && s == KSTEPS - 1)
        kop = half ? __builtin_bit_cast(bf16x8v, make_uint4(0x3F803F80u, 0x3F80u, 0, 0)) : kop;
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[qb][s], s == 0 ? zero16 : sc, 0, 0, 0);
    }
  };
  auto mask1 = [&](f32x16& sc, int kb, int nk) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nk) sc[r] = -INFINITY;
  };
  auto mask_tail = [&](f32x16 (&sc)[QB], int kb, int nk) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= nk) sc[qb][r] = -INFINITY;
  };
  // chunk max (base 2; kShifted: of the shifted scores) and lazy rescale of
  // the running state. kShifted: a raise re-scores the chunk (keys kb*32 ..
  // +31 of the tile at ks, nk keys valid) with the new maximum in the
  // product, so that every chunk's scores come out of the same arithmetic --
  // scores of equal keys stay bitwise equal whatever their magnitude.
  auto max_rescale = [&](f32x16 (&sc)[QB], const unsigned char* ks, int kb, int nk) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = __builtin_fmaxf(sc[qb][0], sc[qb][1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, sc[qb][r]), sc[qb][r + 1]);
      mx = max_halves(mx);
      if constexpr (kShifted) {
        if (__builtin_amdgcn_ballot_w64(mx > thr[qb]) != 0) {
          lazy_rescale_shifted(mx, m_run[qb], thr[qb], l_run[qb], acc[qb]);
          uint4 u = __builtin_bit_cast(uint4, qop[qb][KSTEPS - 1]);
          const uint2 t = neg_bf16x3(m_run[qb]);
          u.x = half ? t.x : u.x;
          u.y = half ? t.y : u.y;
          qop[qb][KSTEPS - 1] = __builtin_bit_cast(bf16x8v, u);
          qk1(ks, kb, qb, sc[qb]);
          if (!FULL) mask1(sc[qb], kb, nk);
        }
      } else {
        lazy_rescale(mx, a.scale_log2e, m_run[qb], thr[qb], l_run[qb], acc[qb]);
      }
    }
  };
  // P of one chunk as the B operands of two 16-key k-steps (kShifted: exp2 of
  // the scores as they stand)
  auto expc = [&](const f32x16 (&sc)[QB], bf16x8v (&pf)[QB][2]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mneg = -m_run[qb];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        uint32_t wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x0 = sc[qb][8 * h2 + 2 * e], x1 = sc[qb][8 * h2 + 2 * e + 1];
          if constexpr (!kShifted) {
            x0 = fmaf(x0, a.scale_log2e, mneg);
            x1 = fmaf(x1, a.scale_log2e, mneg);
          }
          const float p0 = fast_exp2(x0);
          const float p1 = fast_exp2(x1);
          if constexpr (!C::ONES) l_run[qb] += p0 + p1;
          wv[e] = pack_bf16x2(p0, p1);
        }
        pf[qb][h2] = __builtin_bit_cast(bf16x8v, make_uint4(wv[0], wv[1], wv[2], wv[3]));
      }
    }
  };
  // V^T operand of lane (g16, j16): dims 32i + 16(g16&1) + 4(j16&3) .. +3 of
  // keys 16mm + 4(g16>>1) + (j16>>2) (+8 for the upper half), by transposing reads
  const int g16 = lane >> 4, j16 = lane & 15;
  auto pv = [&](const unsigned char* vs, int kb, const bf16x8v (&pf)[QB][2]) {
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
  };

  // ---- prologue: tile 0 copied while Q is loaded, tiles 1..kStages-2 in flight, first chunk scored ----
  // tiles 0 .. kStages-2 are all requested before the first wait; loads
  // complete in issue order, so once only the younger tiles' copies are
  // outstanding, Q (loaded first) and tile 0 have arrived. With PROD the
  // copy wavefront (which loads no Q) does this wait alone; the compute
  // wavefronts issue no copies, so the compiler's own waits for their Q
  // loads are exact.
  if (!PROD || producer) {
    issue_next();
    int pre = 0;
    for (int t = 1; t <= kStages - 2 && t < n_tiles; ++t, ++pre) issue_next();
    wait_tiles(pre);
  }
  lds_barrier();
  if constexpr (PROD) {
    if (producer) {   // the same barriers as the loop below, one per tile
      for (int t = 0; t + 1 < n_tiles; ++t) {
        wait_tiles(min(kStages - 3, n_tiles - t - 2));
        lds_barrier();
        if (t + kStages - 1 < n_tiles) issue_next();
      }
      return;
    }
  }
  f32x16 s0[QB], s1[QB];
  bf16x8v pf[QB][2];
  int nk_t = min(kBN, S);             // keys in tile t
  qk(smem, KS == 2 ? kh : 0, s0);
  if (!FULL && nk_t < (KS == 2 ? kBN : 32)) mask_tail(s0, KS == 2 ? kh : 0, nk_t);
  max_rescale(s0, smem, KS == 2 ? kh : 0, nk_t);

  int st_r = 0;                       // stage of tile t
  int t0_n = kBN >= S ? 0 : kBN;      // first key of tile t+1 within its frame
  if constexpr (KS == 1) {
    for (int t = 0; t + 1 < n_tiles; ++t) {
      const unsigned char* ks = smem + st_r * C::STAGE;
      const unsigned char* vs = ks + C::V_OFF;
      // chunk 2t+1 (same tile) is scored while chunk 2t is exponentiated
      qk(ks, 1, s1);
      expc(s0, pf);
      pv(vs, 0, pf);
      if (!FULL && nk_t < kBN) mask_tail(s1, 1, nk_t);
      max_rescale(s1, ks, 1, nk_t);
      st_r = st_r == kStages - 1 ? 0 : st_r + 1;
      if constexpr (!PROD) wait_tiles(min(kStages - 3, n_tiles - t - 2));   // tile t+1; younger tiles stay in flight
      lds_barrier();                                    // every wavefront is done with tile t-1
      if constexpr (!PROD)
        if (t + kStages - 1 < n_tiles) issue_next();    // into tile t-1's stage
      // chunk 2t+2 (next tile) is scored while chunk 2t+1 is exponentiated
      qk(smem + st_r * C::STAGE, 0, s0);
      expc(s1, pf);
      pv(vs, 1, pf);
      nk_t = min(kBN, S - t0_n);
      if (!FULL && nk_t < 32) mask_tail(s0, 0, nk_t);
      max_rescale(s0, smem + st_r * C::STAGE, 0, nk_t);
      t0_n = t0_n + kBN >= S ? 0 : t0_n + kBN;
    }
    {  // last tile
      const unsigned char* ks = smem + st_r * C::STAGE;
      const unsigned char* vs = ks + C::V_OFF;
      qk(ks, 1, s1);
      expc(s0, pf);
      pv(vs, 0, pf);
      if (!FULL && nk_t < kBN) mask_tail(s1, 1, nk_t);
      max_rescale(s1, ks, 1, nk_t);
      expc(s1, pf);
      pv(vs, 1, pf);
    }
  } else {
    // one chunk (key half kh) per tile: this wavefront's chunk of tile t+1 is
    // scored while its chunk of tile t is exponentiated and accumulated
    auto step = [&](f32x16 (&sa)[QB], f32x16 (&sb)[QB], int t) {
      const unsigned char* vs = smem + st_r * C::STAGE + C::V_OFF;
      st_r = st_r == kStages - 1 ? 0 : st_r + 1;
      wait_tiles(min(kStages - 3, n_tiles - t - 2));   // tile t+1; younger tiles stay in flight
      lds_barrier();                                    // every wavefront is done with tile t-1
      if (t + kStages - 1 < n_tiles) issue_next();      // into tile t-1's stage
      qk(smem + st_r * C::STAGE, kh, sb);
      expc(sa, pf);
      pv(vs, kh, pf);
      nk_t = min(kBN, S - t0_n);
      if (!FULL && nk_t < kBN) mask_tail(sb, kh, nk_t);
      max_rescale(sb, smem + st_r * C::STAGE, kh, nk_t);
      t0_n = t0_n + kBN >= S ? 0 : t0_n + kBN;
    };
    auto last = [&](const f32x16 (&sa)[QB]) {
      expc(sa, pf);
      pv(smem + st_r * C::STAGE + C::V_OFF, kh, pf);
    };
    for (int t = 0;; t += 2) {
      if (t + 1 >= n_tiles) { last(s0); break; }
      step(s0, s1, t);
      if (t + 2 >= n_tiles) { last(s1); break; }
      step(s1, s0, t + 1);
    }
    // merge the two key halves (flash attention partial states combine by
    // rescaling to the larger running maximum): half 1 hands over to half 0
    constexpr int PER = QB * (DBLK * 16 + 2);         // floats per lane
    static_assert(G * 64 * PER * 4 <= kStages * C::STAGE, "merge area");
    lds_barrier();                                    // the ring is no longer read
    float* mg = reinterpret_cast<float*>(smem) + grp * 64 * PER;
    if (kh == 1) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float* d = mg + qb * (DBLK * 16 + 2) * 64 + lane;
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) d[(i * 16 + r) * 64] = acc[qb][i][r];
        d[(DBLK * 16) * 64] = kShifted && thr[qb] == -INFINITY ? kNoMax : m_run[qb];
        d[(DBLK * 16 + 1) * 64] = l_run[qb];
      }
    }
    lds_barrier();
    if (kh == 1) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float* d = mg + qb * (DBLK * 16 + 2) * 64 + lane;
      const float m_o = d[(DBLK * 16) * 64];
      const float m_me = kShifted && thr[qb] == -INFINITY ? kNoMax : m_run[qb];
      const float m_new = __builtin_fmaxf(m_me, m_o);
      const float c_me = fast_exp2(m_me - m_new), c_o = fast_exp2(m_o - m_new);
#pragma unroll
      for (int i = 0; i < DBLK; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][i][r] = acc[qb][i][r] * c_me + d[(i * 16 + r) * 64] * c_o;
      l_run[qb] = l_run[qb] * c_me + d[(DBLK * 16 + 1) * 64] * c_o;
      m_run[qb] = m_new;
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float l_tot;
    if constexpr (C::ONES) {
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

template <int D, int QB, int kSW, bool FULL, int kStages, int KS, bool PROD>
// (d > 72: the ring of one workgroup takes most of the CU's LDS, so one
// wavefront per SIMD is all that can be resident)
__global__ __launch_bounds__(64 * (kSW + PROD)) __attribute__((amdgpu_waves_per_eu(D <= 72 ? 2 : 1, 8))) void spatial_attn_pipe_kernel(SpatialArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * SCfg<D, PROD ? 1 : kSW>::STAGE];
  spatial_pipe<D, QB, kSW, FULL, kStages, KS, PROD>(a, xcd_work_index(blockIdx.x, gridDim.x), threadIdx.x, smem);
}

// ----------------------------------------------------------------------------
// One denoising call in one launch: prefix spatial attention of the chunk
// (MFMA-bound) and causal temporal attention over the queue (HBM-bound)
// ----------------------------------------------------------------------------
// A workgroup holds the four compute wavefronts of one spatial work item
// (4 x 32 queries, each issuing its share of the tile copies) and kDcTW
// temporal wavefronts that serve a block of temporal rows, so every SIMD runs
// one MFMA-and-softmax wavefront beside one wavefront that mostly waits for
// HBM. The workgroup barriers of the spatial tile ring count every wavefront
// of the workgroup, so the temporal wavefronts take the same number of
// barriers, one after each key pair they process: their work advances one
// key pair per spatial tile, with loads kDcRing keys ahead in a register
// ring, and whatever is left after the spatial loop's last barrier runs free.
// Measured alternatives, all within 3 % of this form at the 256-token shape
// (27-28 us per call against 16.8 + 14.5 us for the two kernels alone):
// the temporal keys staged through LDS by the same copies as the spatial
// tiles (4 copies per key pair instead of 12 lane-duplicated loads, 140
// VGPRs), the same plus the spatial copy wavefront (9 wavefronts), and the
// two halves as separate workgroups of one launch with no shared barriers;
// the matrix-core temporal rows in the temporal wavefronts (kTm) are slower.
// Rows of a temporal wavefront: 4 dimension groups x kDcQH query groups of
// kDcQPL queries, so a row's 8 new frames are covered and 4 rows share a
// wavefront; the key range is not split, so no partial results are merged.
constexpr int kDcQH = 4;                         // query groups per temporal row
constexpr int kDcQPL = 2;                        // queries per lane
constexpr int kDcTW = 4;                         // temporal wavefronts per workgroup
constexpr int kDcRows = 64 / (4 * kDcQH);        // rows per temporal wavefront
constexpr int kDcBlockRows = kDcTW * kDcRows;    // rows per row block of a workgroup
constexpr int kDcRing = 6;                       // keys in flight per temporal lane (register ring)

// A wavefront-uniform barrier for wavefronts that share nothing through LDS
// (they only keep count with the spatial wavefronts' barriers).
__device__ __forceinline__ void count_barrier(int& bars) {
  if (bars > 0) {
    __builtin_amdgcn_s_barrier();
    --bars;
  }
}

// Temporal wavefront tw of a workgroup: row blocks blk0 .. blk0 + nblk - 1
// (kDcBlockRows rows each), taking exactly `bars` workgroup barriers.
template <int D, int kPF>
__device__ __forceinline__ void temporal_lockstep(const TemporalArgs& a, int tw, int blk0, int nblk, int bars) {
  static_assert(kPF % 2 == 0 && kPF >= 4, "register ring of whole key pairs");
  // The temporal wavefronts set the pace of the shared barriers (the spatial
  // wavefronts wait for them there), so their instructions take issue
  // priority over the spatial wavefront on the same SIMD, which fills the
  // gaps while they wait for memory (step 1.420 -> 1.373 ms on one box).
  __builtin_amdgcn_s_setprio(2);
  using G = DsGeom<D>;
  constexpr int DW = G::DW, DPL = G::DPL, QPL = kDcQPL, QH = kDcQH, LPR = 4 * QH;
  const int lane = threadIdx.x & 63;
  const int g = lane & 3;                          // dimension group
  const int qg = (lane >> 2) % QH;                 // query group
  const int ri = lane / LPR;
  const int rpb = a.rows_per_batch;
  const int64_t frame_bytes = (int64_t)rpb * D * 2;
  const unsigned char* qb = static_cast<const unsigned char*>(a.q);
  const unsigned char* knb = static_cast<const unsigned char*>(a.k_new);
  const unsigned char* vnb = static_cast<const unsigned char*>(a.v_new);
  const unsigned char* rkb = static_cast<const unsigned char*>(a.ring_k);
  const unsigned char* rvb = static_cast<const unsigned char*>(a.ring_v);
  unsigned char* ob = static_cast<unsigned char*>(a.out);
  const int k_total = a.p_k + a.n;
  // every query of the row is served here (n <= QPL * QH), so the keys are
  // all k_total of them; query i stops at key p_k + i (causal)
  const int ke = k_total;
  const float c = a.scale_log2e;
  bool first = true;

  for (int blk = blk0; blk < blk0 + nblk; ++blk) {
    // Addresses: a wavefront-uniform frame base plus a per-lane 32-bit offset
    // within the frame (the rows of a wavefront lie in one batch: the launch
    // checks rows_per_batch % kDcRows == 0 and frames under 4 GiB). Rows past
    // the end are clamped to the last row: loaded, never stored.
    const int row0 = (blk * kDcTW + tw) * kDcRows;
    const bool row_ok = row0 + ri < a.rows_total;
    const int rc = min(row0 + ri, a.rows_total - 1);
    const int b = min(row0, a.rows_total - 1) / rpb;
    const uint32_t lrow = (uint32_t)(rc - b * rpb) * (D * 2);
    const uint32_t o16 = lrow + 16 * g, o4 = lrow + 64 * G::FULL + 4 * g;
    Slice<D> qs[QPL];
    int last_key[QPL];
    // every load is unconditional, indices clamped into range (as in the
    // stand-alone temporal kernel: the compiler's wait counts then keep the
    // refills in flight across iterations); clamped reads are masked
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) {
      const int qi = qg * QPL + qq;
      last_key[qq] = !(row_ok && qi < a.n) ? -1 : a.p_k + qi;
      const int64_t fo = ((int64_t)b * a.n + min(qi, a.n - 1)) * frame_bytes;
      load_slice_at<D>(qs[qq], qb + fo, o16, o4);
    }
    float m[QPL], thr[QPL], l[QPL], acc[QPL][DPL];
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) {
      m[qq] = kNoMax;
      thr[qq] = kNoMax;
      l[qq] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[qq][e] = 0.f;
    }
    Slice<D> kr[kPF], vr[kPF];
    // keys past the end read the last key again; their scores are masked to
    // -inf, so their P is exactly 0 (and the slot never holds stale data)
    auto refill = [&](int u, int jn) {
      const int jc = jn < ke ? jn : ke - 1;
      const bool queued = jc < a.ring_keys;
      int slot = a.head + jc;
      if (slot >= a.p_max) slot -= a.p_max;
      const int64_t fo = queued ? ((int64_t)b * a.p_max + slot) * frame_bytes
                                : ((int64_t)b * a.n + (jc - a.p_k)) * frame_bytes;
      load_slice_at<D>(kr[u], (queued ? rkb : knb) + fo, o16, o4);
      load_slice_at<D>(vr[u], (queued ? rvb : vnb) + fo, o16, o4);
    };
#pragma unroll
    for (int u = 0; u < kPF; ++u) refill(u, u);
    // The first barrier once the first keys are in flight. It also fences the
    // compiler's scheduling: with the ring loads free to move into the loop,
    // its wait counts fall back to waiting for every load in each pair.
    if (first) {
      count_barrier(bars);
      first = false;
    }
    // one key pair: scores, lazy rescale, P rounded to bf16, O += P V by bf16
    // dot products over the two keys (as the stand-alone temporal kernel).
    // Pairs of queued keys, which every query sees, skip the mask (a lane
    // with no query then computes on clamped rows and stores nothing).
    auto process2 = [&](int j, const Slice<D>& k0, const Slice<D>& v0, const Slice<D>& k1, const Slice<D>& v1) {
      const bool mask = j + 1 >= a.p_k;              // wavefront-uniform
      float x0[QPL], x1[QPL];
      bool raise = false;
#pragma unroll
      for (int qq = 0; qq < QPL; ++qq) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int x = 0; x < DW; ++x) {
          s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, qs[qq].w[x]),
                                               __builtin_bit_cast(bf16x2v, k0.w[x]), s0, false);
          s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, qs[qq].w[x]),
                                               __builtin_bit_cast(bf16x2v, k1.w[x]), s1, false);
        }
        x0[qq] = quad_sum(s0) * c;
        x1[qq] = quad_sum(s1) * c;
        if (mask) {
          if (j > last_key[qq]) x0[qq] = -INFINITY;
          if (j + 1 > last_key[qq]) x1[qq] = -INFINITY;
        }
        raise |= (x0[qq] > thr[qq]) | (x1[qq] > thr[qq]);
      }
      if (raise) {
#pragma unroll
        for (int qq = 0; qq < QPL; ++qq) {
          const float mn = fmaxf(m[qq], fmaxf(x0[qq], x1[qq]));
          const float corr = fast_exp2(m[qq] - mn);
          m[qq] = mn;
          thr[qq] = mn + kLazy;
          l[qq] *= corr;
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[qq][e] *= corr;
        }
      }
      uint32_t vp[DPL];
#pragma unroll
      for (int x = 0; x < DW; ++x) {
        vp[2 * x] = __builtin_amdgcn_perm(v1.w[x], v0.w[x], 0x05040100u);       // low halves
        vp[2 * x + 1] = __builtin_amdgcn_perm(v1.w[x], v0.w[x], 0x07060302u);   // high halves
      }
#pragma unroll
      for (int qq = 0; qq < QPL; ++qq) {
        const bf16x2v pp = __builtin_bit_cast(bf16x2v, pack_bf16x2(fast_exp2(x0[qq] - m[qq]),
                                                                   fast_exp2(x1[qq] - m[qq])));
        l[qq] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2v, 0x3F803F80u), l[qq], false);
#pragma unroll
        for (int e = 0; e < DPL; ++e)
          acc[qq][e] = __builtin_amdgcn_fdot2_f32_bf16(pp, __builtin_bit_cast(bf16x2v, vp[e]), acc[qq][e], false);
      }
    };
    for (int j = 0; j < ke; j += kPF) {              // bounds are uniform per wavefront
#pragma unroll
      for (int u = 0; u < kPF; u += 2) {             // ring slots are compile-time constants
        if (j + u >= ke) break;                      // no pair left (uniform)
        process2(j + u, kr[u], vr[u], kr[u + 1], vr[u + 1]);
        refill(u, j + u + kPF);
        refill(u + 1, j + u + 1 + kPF);
        count_barrier(bars);
      }
    }
#pragma unroll
    for (int qq = 0; qq < QPL; ++qq) {
      if (last_key[qq] < 0) continue;
      const int qi = qg * QPL + qq;
      const float inv = 1.f / l[qq];
      float o[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = acc[qq][e] * inv;
      store_slice<D>(ob + ((int64_t)b * a.n + qi) * frame_bytes + lrow, g, o);
    }
  }
  if (first) count_barrier(bars);
  while (bars > 0) count_barrier(bars);          // the rest of the spatial wavefronts' barriers
}

// Wavefronts 0..3: spatial work item w (4 x 32 queries, whole 64-key tiles,
// copies issued by the computing wavefronts); wavefronts 4..4+kDcTW-1:
// temporal row blocks [blockIdx.x * nblk, +nblk), by the dimension-split
// lockstep loop or, with kTm (the forced matrix-core temporal variant, slower
// here too), by the matrix-core rows over the same rows. Launched only when
// the spatial grid fits on the chip in one round (one workgroup per CU).
template <int D, int kStages, int kPF, bool kTm>
__global__ __launch_bounds__(64 * (4 + kDcTW)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void denoise_call_kernel(SpatialArgs sa, TemporalArgs ta, int nblk) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * SCfg<D, 4>::STAGE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4) {
    spatial_pipe<D, 1, 4, true, kStages, 1, false>(sa, xcd_work_index(blockIdx.x, gridDim.x), threadIdx.x, smem);
  } else {
    const int n_tiles = (1 + sa.n_prefix) * (sa.tokens / kBN);   // the spatial wavefronts' barrier count
    if constexpr (kTm) {
      __builtin_amdgcn_s_setprio(2);
      const int tw = wave - 4;
      auto row_of = [&](int i) { return ((blockIdx.x * nblk + i / kDcRows) * kDcTW + tw) * kDcRows + i % kDcRows; };
      int rows = 0;
      for (int i = 0; i < nblk * kDcRows; ++i)
        if (row_of(i) < ta.rows_total) rows = i + 1;
      temporal_mfma_rows<D>(ta, row_of, rows, n_tiles);
    } else {
      temporal_lockstep<D, kPF>(ta, wave - 4, blockIdx.x * nblk, nblk, n_tiles);
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

template <int D, int QB, int SW, int ST, int KS, bool PROD = false>
hipError_t launch_pipe_cfg(const SpatialArgs& a, hipStream_t s) {
  constexpr int BM = 32 * QB * SW / KS;
  const int64_t nwg = (int64_t)((a.tokens + BM - 1) / BM) * a.n * a.heads * a.batch;
  if (nwg > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 block(64 * (SW + PROD));
  if (a.tokens % kBN == 0)
    hipLaunchKernelGGL((spatial_attn_pipe_kernel<D, QB, SW, true, ST, KS, PROD>), dim3((unsigned)nwg), block, 0, s, a);
  else
    hipLaunchKernelGGL((spatial_attn_pipe_kernel<D, QB, SW, false, ST, KS, PROD>), dim3((unsigned)nwg), block, 0, s, a);
  return hipGetLastError();
}

// Compute units of the current device (queried once per device).
int device_cus() {
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

// Launch variant forced by ca2_set_spatial_variant (a test and measurement
// switch; 0 = the size-based choice). One relaxed load per launch.
std::atomic<int> g_forced_variant{0};

template <int D>
hipError_t launch_mfma(const SpatialArgs& a, hipStream_t s) {
  // Large grids: 4 wavefronts x 64 queries (each K/V operand read from LDS
  // feeds two MFMAs), two workgroups per CU. Below ~4 such workgroups per CU:
  // 4 x 32 queries, which doubles the wavefronts in flight. Both use a 4-stage
  // ring: at 256 tokens 3 stages time faster launched alone (18.5 vs 19.7 us)
  // but slower in the denoising step that alternates with the temporal kernel
  // (1.86 vs 1.80 ms per step); 5 and 6 stages take 23.5 us.
  // At d = 72 with at most one workgroup per CU the 4 x 32 form gets a fifth
  // wavefront that issues every copy: the compute wavefronts no longer stall
  // on copy issue (256-token shape 18.6 -> 17.3 us). With two workgroups per
  // CU, or at d = 64 / 128 (SGPR and VGPR spills under the two-wavefront
  // register cap), it measured slower.
  // Forced variants 1|2|3|4: 32 queries, 64 queries, 8 wavefronts of
  // 32 queries x 2 key halves (two wavefronts per SIMD even at one workgroup
  // per CU; measured slower than 4 x 32 at the 256-token shape, kept
  // selectable), or 32 queries with the copy wavefront.
  const int64_t frames = (int64_t)a.n * a.heads * a.batch;
  const int64_t wg_big = (int64_t)((a.tokens + 255) / 256) * frames;
  const int64_t wg_small = (int64_t)((a.tokens + 127) / 128) * frames;
  // (the 64-query form only over whole 64-key tiles: with partial tiles its
  // register budget is exceeded)
  int cfg = wg_big >= 1024 && a.tokens % kBN == 0 ? 2 : D == 72 && wg_small <= device_cus() ? 4 : 1;
  if (const int force = g_forced_variant.load(std::memory_order_relaxed)) cfg = force;
  if constexpr (D <= 72) {
    if (cfg == 2) return launch_pipe_cfg<D, 2, 4, 4, 1>(a, s);
  }
  if (cfg == 3) return launch_pipe_cfg<D, 1, 8, 4, 2>(a, s);
  if (cfg == 4) return launch_pipe_cfg<D, 1, 4, 4, 1, true>(a, s);
  return launch_pipe_cfg<D, 1, 4, 4, 1>(a, s);
}

template <int D>
hipError_t launch_f32(const SpatialArgs& a, hipStream_t s) {
  const dim3 grid((a.tokens + 63) / 64, a.n * a.heads, a.batch);
  hipLaunchKernelGGL((spatial_attn_f32_kernel<D>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

void set_spatial_variant(int v) { g_forced_variant.store(v, std::memory_order_relaxed); }

bool denoise_call_fusable(int dtype, int d, const SpatialArgs& sa, const TemporalArgs& ta) {
  if (dtype != 1 || (d != 64 && d != 72)) return false;                // the bf16 MFMA path, 2 waves per SIMD
  if (sa.tokens % kBN != 0 || ta.n > kDcQH * kDcQPL || !ta.causal) return false;
  if (g_forced_variant.load(std::memory_order_relaxed) != 0) return false;   // a forced spatial variant wins
  // the temporal wavefronts' addressing: the rows of a wavefront in one
  // batch, per-lane 32-bit offsets within a frame
  if (ta.rows_per_batch % kDcRows != 0 || (int64_t)ta.rows_per_batch * d * 2 > 0xFFFFFFFFll) return false;
  const int64_t nwg = (int64_t)((sa.tokens + 127) / 128) * sa.n * sa.heads * sa.batch;
  return nwg <= device_cus();                                          // one round of workgroups
}

hipError_t launch_denoise_call(int dtype, int d, const SpatialArgs& sa, const TemporalArgs& ta, hipStream_t s,
                               bool* fused) {
  const bool f = denoise_call_fusable(dtype, d, sa, ta);
  if (fused) *fused = f;
  if (!f) {
    hipError_t e = launch_spatial(dtype, d, sa, s);
    if (e != hipSuccess) return e;
    return launch_temporal(dtype, d, ta, s);
  }
  // same ring-key rule as the stand-alone temporal launch
  if (ta.n < 1 || ta.p_k < 0) return hipErrorInvalidValue;
  if (ta.ring_keys != ta.p_k && ta.ring_keys != ta.p_k + ta.n) return hipErrorInvalidValue;
  if (ta.ring_keys > 0 && (ta.head < 0 || ta.head >= ta.p_max || ta.ring_keys > ta.p_max)) return hipErrorInvalidValue;
  const int64_t nwg = (int64_t)((sa.tokens + 127) / 128) * sa.n * sa.heads * sa.batch;
  const int64_t blocks = ((int64_t)ta.rows_total + kDcBlockRows - 1) / kDcBlockRows;
  const int nblk = (int)((blocks + nwg - 1) / nwg);
  const dim3 grid((unsigned)nwg), block(64 * (4 + kDcTW));
  const bool tm = temporal_variant() == 2;
  if (d == 64) {
    if (tm) hipLaunchKernelGGL((denoise_call_kernel<64, 4, kDcRing, true>), grid, block, 0, s, sa, ta, nblk);
    else hipLaunchKernelGGL((denoise_call_kernel<64, 4, kDcRing, false>), grid, block, 0, s, sa, ta, nblk);
  } else {
    if (tm) hipLaunchKernelGGL((denoise_call_kernel<72, 4, kDcRing, true>), grid, block, 0, s, sa, ta, nblk);
    else hipLaunchKernelGGL((denoise_call_kernel<72, 4, kDcRing, false>), grid, block, 0, s, sa, ta, nblk);
  }
  return hipGetLastError();
}

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
