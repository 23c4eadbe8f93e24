// QKV projection of the clean chunk (gfx950 bf16 MFMA GEMM).
//
// The cache-writing stage of the Ca2-VDM notes (overall framework) runs one
// forward pass of the denoised chunk to produce the K/V that are stored; this
// is that pass's linear projection: [Q K V] = X W^T, X: [m][c_in] tokens,
// W: [3c][c_in] (row-major linear weight), fp32 accumulation, bf16 outputs
// split into three [m][c] tensors in the activation layout the cache write
// consumes.
//
// Tiling: workgroup tile 256 output channels (n) x 256 tokens (m), 8
// wavefronts (two per SIMD) of 128 x 64 (4 x 2 v_mfma_f32_32x32x16_bf16
// blocks, 128 accumulators per lane). The product is formed as C^T = W X^T so that a lane owns
// one token row and its accumulator registers hold runs of 4 consecutive
// channels (8-byte stores). k-tiles of 64 are double-buffered in LDS and
// filled by global_load_lds_dwordx4 in its scalar-base form: an LDS row is
// 144 bytes (128 of data + a 16-byte pad slot, so 8 consecutive rows read
// distinct banks), copy instruction j covers 16-byte slots 64j..64j+63 of the
// 256 rows, each lane's offset from the k-tile base is a constant, and the
// pad lanes are masked. Within a k-tile the operands of k-step s+1 are read
// from LDS into a second register set while the 16 MFMAs of k-step s run
// (two wavefronts per SIMD, both of the same workgroup and on the same k-tile
// schedule, so they hide little of each other's LDS latency).
// Workgroups are dealt so that each XCD takes a contiguous run of tiles
// sharing token panels.
//
// Cache-writing form (the stage that stores a clean chunk's K/V): the
// epilogue adds the projected cyclic temporal position embedding row of each
// token's frame (Ca2-VDM notes, key design 4, Cyclic-TPEs: the embedding is
// bound into the cached K/V) and writes the K/V columns straight into their
// ring slots and spatial-buffer slots, so no separate copy of the chunk is
// needed.
#include "device_common.hpp"
#include "kernels.hpp"

namespace ca2 {
namespace {

constexpr int TN = 256;                 // output channels per workgroup
constexpr int TM = 256;                 // tokens per workgroup
constexpr int TK = 64;                  // contraction per k-tile
constexpr int kSlots = TK * 2 / 16 + 1; // 16-byte slots per LDS row (data + pad)
constexpr int ROWB = kSlots * 16;       // 144
constexpr int OPB = TN * ROWB;          // one operand tile
constexpr int STAGE = 2 * OPB;          // W tile, then X tile
constexpr int kStages = 2;
constexpr int kThreads = 512;
constexpr int kGroupM = 8;              // token panels per tile group (see the work order below)
constexpr int kWaves = kThreads / 64;
constexpr int NI = TN * kSlots / 64;    // copy instructions per operand per k-tile (36)
constexpr int kPer = 2 * NI / kWaves;   // per wavefront per k-tile (9)
static_assert(TN == TM && (TN * kSlots) % 64 == 0 && (2 * NI) % kWaves == 0, "copy geometry");

template <bool kStage>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void qkv_proj_kernel(ProjArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * STAGE];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int wn = wave & 1, wm = wave >> 1;       // 128 channels x 64 tokens per wavefront
  const int N = 3 * a.c_out;
  const int tiles_n = (N + TN - 1) / TN;
  // Tiles in groups of kGroupM token panels: within a group the token panel
  // runs fastest, so a run of consecutive work items (what one XCD holds at
  // once, dealt by xcd_work_index) covers kGroupM token panels x a few
  // channel panels and each panel's k-slab is read once into that XCD's L2.
  const int w = xcd_work_index(blockIdx.x, gridDim.x);
  const int tiles_m = (a.m + TM - 1) / TM;
  const int grp = w / (kGroupM * tiles_n);
  const int gm = min(kGroupM, tiles_m - grp * kGroupM);   // token panels in this group
  const int wi = w - grp * kGroupM * tiles_n;
  const int n0 = (wi / gm) * TN;
  const int m0 = (grp * kGroupM + wi % gm) * TM;
  const int KT = a.c_in / TK;

  // per-lane copy offsets (bytes from the k-tile base) for this wavefront's
  // instructions: j = wave + 4i over the W tile (j < NI) then the X tile
  unsigned g_off[kPer];
  bool g_ok[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = wave + kWaves * i;
    const bool isx = j >= NI;
    const int slot = (isx ? j - NI : j) * 64 + lane;
    const int row = slot / kSlots, c = slot % kSlots;
    g_ok[i] = c < kSlots - 1 && (isx ? m0 + row < a.m : n0 + row < N);
    g_off[i] = (unsigned)row * (unsigned)(a.c_in * 2) + 16u * c;
  }
  const uint64_t wbase = reinterpret_cast<uint64_t>(a.w) + (uint64_t)n0 * a.c_in * 2;
  const uint64_t xbase = reinterpret_cast<uint64_t>(a.x) + (uint64_t)m0 * a.c_in * 2;
  const unsigned lds_base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  auto issue = [&](int t) {                        // k-tile t into stage t % kStages
    const unsigned st = lds_base + (t % kStages) * STAGE;
    const uint64_t kb = (uint64_t)t * TK * 2;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int j = wave + kWaves * i;
      const bool isx = j >= NI;
      if (g_ok[i]) dma16s(g_off[i], (isx ? xbase : wbase) + kb, st + (isx ? OPB + (j - NI) * 1024 : j * 1024));
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  bf16x8v wa[2][4], xb[2][2];
  auto load_ops = [&](const unsigned char* sw, int s, int buf) {
    const unsigned char* sx = sw + OPB;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wa[buf][i] = *reinterpret_cast<const bf16x8v*>(sw + (wn * 128 + i * 32 + col) * ROWB + (16 * s + 8 * half) * 2);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      xb[buf][j] = *reinterpret_cast<const bf16x8v*>(sx + (wm * 64 + j * 32 + col) * ROWB + (16 * s + 8 * half) * 2);
  };
  issue(0);
  for (int t = 0; t < KT; ++t) {
    wait_vmcnt<0>();                               // this wavefront's copies of k-tile t
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();                  // k-tile t visible; stage of k-tile t-1 free
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    // A copy instruction holds its wavefront while the memory pipeline takes
    // it, so the next k-tile's copies are issued at two times: by waves 0-3
    // right after the barrier and by waves 4-7 after their first k-step.
    // Waves are dealt to the SIMDs in turn, so waves w and w + 4 share one and
    // each SIMD has one wavefront running MFMAs while the other issues copies.
    if (t + 1 < KT && wave < 4) issue(t + 1);
    const unsigned char* sw = smem + (t % kStages) * STAGE;
    load_ops(sw, 0, 0);
#pragma unroll
    for (int s = 0; s < TK / 16; ++s) {
      // the reads of k-step s+1 are issued before the MFMAs of k-step s (the
      // scheduling barriers keep the compiler from sinking them to their uses)
      if (s + 1 < TK / 16) load_ops(sw, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[s & 1][i], xb[s & 1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0 && t + 1 < KT && wave >= 4) issue(t + 1);
    }
  }

  // register r of acc[i][j]: channel n0 + wn*128 + 32i + 8(r/4) + 4*half + r%4,
  // token m0 + wm*64 + 32j + col
  if constexpr (!kStage) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + wm * 64 + 32 * j + col;
      if (m >= a.m) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 128 + 32 * i + 8 * g + 4 * half;
          if (n >= N) continue;
          const int seg = n / a.c_out;
          bf16_t* dst = static_cast<bf16_t*>(seg == 0 ? a.q : seg == 1 ? a.k : a.v);
          uint2 v;
          v.x = pack_bf16x2(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]);
          v.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
          *reinterpret_cast<uint2*>(dst + (int64_t)m * a.c_out + (n - seg * a.c_out)) = v;
        }
    }
  } else {
    // cache-writing epilogue: + the frame's table row, then the caller's
    // outputs and the cache slots of the K and V columns. A run of 4
    // channels never crosses a Q/K/V boundary (c_out is a multiple of 64).
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int m = m0 + wm * 64 + 32 * j + col;
      if (m >= a.m) continue;
      const int bf = m / a.tokens;                 // b * frames + f
      const int s_tok = m - bf * a.tokens;
      const int b = bf / a.frames;
      const int f = bf - b * a.frames;
      const float* trow = a.tpe ? a.tpe + (int64_t)((a.tpe_first + f) % a.tpe_len) * N : nullptr;
      const int64_t ring_row =
          ((int64_t)b * a.ring_slots + (a.ring_first + f) % a.ring_slots) * a.tokens + s_tok;
      const bool to_sp = a.sp_k != nullptr && f >= a.sp_from;
      const int64_t sp_row = to_sp ? ((int64_t)b * a.sp_slots + (a.sp_first + f) % a.sp_slots) * a.tokens + s_tok : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 128 + 32 * i + 8 * g + 4 * half;
          if (n >= N) continue;
          float o0 = acc[i][j][4 * g + 0], o1 = acc[i][j][4 * g + 1];
          float o2 = acc[i][j][4 * g + 2], o3 = acc[i][j][4 * g + 3];
          if (trow) {
            const float4 t = *reinterpret_cast<const float4*>(trow + n);
            o0 += t.x; o1 += t.y; o2 += t.z; o3 += t.w;
          }
          uint2 v;
          v.x = pack_bf16x2(o0, o1);
          v.y = pack_bf16x2(o2, o3);
          const int seg = n / a.c_out;
          const int c = n - seg * a.c_out;
          void* own = seg == 0 ? a.q : seg == 1 ? a.k : a.v;
          if (own) *reinterpret_cast<uint2*>(static_cast<bf16_t*>(own) + (int64_t)m * a.c_out + c) = v;
          if (seg == 0) continue;
          void* rd = seg == 1 ? a.ring_k : a.ring_v;
          if (rd) *reinterpret_cast<uint2*>(static_cast<bf16_t*>(rd) + ring_row * a.c_out + c) = v;
          if (to_sp)
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(seg == 1 ? a.sp_k : a.sp_v) + sp_row * a.c_out + c) = v;
        }
    }
  }
}

}  // namespace

namespace {
bool proj_geometry(const ProjArgs& a, int64_t& tiles) {
  if (a.m < 1 || a.c_in < TK || a.c_in % TK || a.c_out < 64 || a.c_out % 64) return false;
  if ((int64_t)TN * a.c_in * 2 > 0xffffffffLL) return false;   // 32-bit copy offsets
  tiles = (int64_t)((3 * a.c_out + TN - 1) / TN) * ((a.m + TM - 1) / TM);
  return tiles <= 0x7fffffff;
}
}  // namespace

hipError_t launch_qkv_proj(const ProjArgs& a, hipStream_t s) {
  int64_t tiles;
  if (!proj_geometry(a, tiles)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(qkv_proj_kernel<false>, dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_qkv_proj_stage(const ProjArgs& a, hipStream_t s) {
  int64_t tiles;
  if (!proj_geometry(a, tiles)) return hipErrorInvalidValue;
  // rows are whole (b, frame) blocks; every modulus is positive and every
  // first index already reduced
  if (a.tokens < 1 || a.frames < 1 || a.m % ((int64_t)a.tokens * a.frames)) return hipErrorInvalidValue;
  if (a.tpe && (a.tpe_len < 1 || a.tpe_first < 0 || a.tpe_first >= a.tpe_len)) return hipErrorInvalidValue;
  if ((a.ring_k != nullptr) != (a.ring_v != nullptr) || (a.sp_k != nullptr) != (a.sp_v != nullptr))
    return hipErrorInvalidValue;
  if (a.ring_slots < 1 || a.ring_first < 0 || a.ring_first >= a.ring_slots) return hipErrorInvalidValue;
  if (a.sp_k && (a.sp_slots < 1 || a.sp_first < 0 || a.sp_first >= a.sp_slots || a.sp_from < 0))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(qkv_proj_kernel<true>, dim3((unsigned)tiles), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ca2
