// Host-side checks of libca2's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py
// builds and runs it; no GPU is needed). Exercises every pure host function
// over wide ranges and every validation path of the other entry points; the
// sanitizers turn any out-of-bounds access, leak or undefined operation into
// a failure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ca2.h"

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static ca2_config cfg_ok() {
  ca2_config c;
  c.batch = 1; c.heads = 2; c.head_dim = 64; c.tokens = 16; c.chunk = 4;
  c.p_max = 9; c.p_spatial = 1; c.tpe_len = 13; c.dtype = CA2_BF16;
  return c;
}

int main() {
  // cyclic TPE indices
  for (int L = 1; L < 60; L += 7)
    for (int64_t first = 0; first < 200; first += 3) {
      std::vector<int32_t> out(17, -1);
      CHECK(ca2_tpe_index_raw(first, 17, L, out.data()) == CA2_OK);
      for (int i = 0; i < 17; ++i) CHECK(out[i] == (int32_t)((first + i) % L));
    }
  CHECK(ca2_tpe_index_raw(0, 0, 13, nullptr) == CA2_OK);
  CHECK(ca2_tpe_index_raw(-1, 2, 13, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(std::strlen(ca2_last_error()) > 0);
  CHECK(ca2_tpe_index_raw(0, 2, 13, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_tpe_index_raw(0, 2, 0, nullptr) == CA2_ERR_INVALID_ARG);

  // ring and spatial slot maps
  for (int32_t P = 1; P <= 41; P += 4)
    for (int64_t fw = 0; fw < 3 * P + 5; ++fw) {
      std::vector<int32_t> slots(P, -1);
      int32_t pk = -1;
      CHECK(ca2_ring_slot_map_raw(fw, P, slots.data(), &pk) == CA2_OK);
      CHECK(pk == (fw < P ? fw : P));
      for (int32_t j = 0; j < pk; ++j) CHECK(slots[j] == (int32_t)((fw - pk + j) % P));
    }
  for (int32_t Ps = 1; Ps < 16; Ps += 2)
    for (int64_t fw = 1; fw < 40; ++fw) {
      std::vector<int64_t> frames(Ps, -1);
      std::vector<int32_t> sl(Ps, -1);
      CHECK(ca2_spatial_slot_map_raw(fw, Ps, frames.data(), sl.data()) == CA2_OK);
      for (int32_t j = 0; j < Ps; ++j) {
        const int64_t f = fw - Ps + j < 0 ? 0 : fw - Ps + j;
        CHECK(frames[j] == f);
        CHECK(sl[j] == (int32_t)(f % Ps));
      }
    }

  // bytes resident: closed form, and 0 for an invalid config
  ca2_config c = cfg_ok();
  CHECK(ca2_bytes_resident(&c) == 2ull * 1 * (9 + 1) * 16 * 2 * 64 * 2);
  c.p_spatial = 4;  // must stay below the chunk
  CHECK(ca2_bytes_resident(&c) == 0);
  CHECK(ca2_bytes_resident(nullptr) == 0);

  CHECK(ca2_abi_version() == CA2_ABI_VERSION);

  // the fused denoising call validates like its two halves
  CHECK(ca2_denoise_attn(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1.f, nullptr, nullptr, nullptr,
                         nullptr, 1.f, 1, nullptr, nullptr) == CA2_ERR_INVALID_ARG);

  // spatial launch-variant switch: range checked, host state only
  CHECK(ca2_set_spatial_variant(-1) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_set_spatial_variant(5) == CA2_ERR_INVALID_ARG);
  for (int32_t v = 4; v >= 0; --v) CHECK(ca2_set_spatial_variant(v) == CA2_OK);
  CHECK(ca2_set_temporal_variant(-1) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_set_temporal_variant(3) == CA2_ERR_INVALID_ARG);
  for (int32_t v = 2; v >= 0; --v) CHECK(ca2_set_temporal_variant(v) == CA2_OK);

  // status strings
  for (int32_t s = 0; s <= 5; ++s) CHECK(std::strlen(ca2_status_string(s)) > 0);
  CHECK(std::strcmp(ca2_status_string(99), "unknown status") == 0);
  CHECK(std::strcmp(ca2_status_string(-1), "unknown status") == 0);

  // create: argument validation field by field
  ca2_cache* h = nullptr;
  CHECK(ca2_cache_create(nullptr, &h) == CA2_ERR_INVALID_ARG && h == nullptr);
  c = cfg_ok();
  CHECK(ca2_cache_create(&c, nullptr) == CA2_ERR_INVALID_ARG);
  struct Bad { int field; int32_t value; ca2_status want; };
  const Bad bads[] = {{0, 0, CA2_ERR_INVALID_ARG},  {1, 0, CA2_ERR_INVALID_ARG},  {2, 0, CA2_ERR_INVALID_ARG},
                      {3, 0, CA2_ERR_INVALID_ARG},  {4, 0, CA2_ERR_INVALID_ARG},  {4, 17, CA2_ERR_INVALID_ARG},
                      {5, 0, CA2_ERR_INVALID_ARG},  {6, 4, CA2_ERR_INVALID_ARG},  {6, -1, CA2_ERR_INVALID_ARG},
                      {7, 12, CA2_ERR_INVALID_ARG}, {8, 7, CA2_ERR_INVALID_ARG},  {2, 16, CA2_ERR_UNSUPPORTED},
                      {2, 80, CA2_ERR_UNSUPPORTED}};
  for (const Bad& b : bads) {
    c = cfg_ok();
    int32_t* f[] = {&c.batch, &c.heads, &c.head_dim, &c.tokens, &c.chunk, &c.p_max, &c.p_spatial, &c.tpe_len,
                    &c.dtype};
    *f[b.field] = b.value;
    h = reinterpret_cast<ca2_cache*>(0x1);
    CHECK(ca2_cache_create(&c, &h) == b.want);
    CHECK(h == nullptr);
  }
  // a valid config: succeeds on a machine with a GPU, fails cleanly (HIP error, nothing leaked) without one
  c = cfg_ok();
  const ca2_status st = ca2_cache_create(&c, &h);
  CHECK(st == CA2_OK || st == CA2_ERR_HIP || st == CA2_ERR_OUT_OF_MEMORY);
  if (st == CA2_OK) {
    ca2_cache_info info;
    CHECK(ca2_cache_info_get(h, &info) == CA2_OK && info.p_k == 0 && info.frames_written == 0);
    CHECK(info.ring_slots == c.p_max && info.staged_frames == 0);
    CHECK(ca2_cache_write(h, nullptr, nullptr, nullptr, nullptr, 1, nullptr) == CA2_ERR_INVALID_ARG);
    CHECK(ca2_cache_commit(h) == CA2_ERR_STATE);   // nothing staged
    ca2_cache_destroy(h);
  } else {
    CHECK(h == nullptr);
  }
  const ca2_status st2 = ca2_cache_create_staged(&c, &h);
  CHECK(st2 == CA2_OK || st2 == CA2_ERR_HIP || st2 == CA2_ERR_OUT_OF_MEMORY);
  if (st2 == CA2_OK) {
    ca2_cache_info info;
    CHECK(ca2_cache_info_get(h, &info) == CA2_OK && info.ring_slots == c.p_max + c.chunk);
    ca2_cache_destroy(h);
  } else {
    CHECK(h == nullptr);
  }
  ca2_cache_destroy(nullptr);
  CHECK(ca2_cache_create_staged(nullptr, &h) == CA2_ERR_INVALID_ARG && h == nullptr);

  // calls on a NULL cache
  int32_t tpe[4];
  CHECK(ca2_tpe_index(nullptr, 4, tpe) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_temporal_attn(nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0.1f, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_spatial_attn(nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 0.1f, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_cache_write(nullptr, nullptr, nullptr, nullptr, nullptr, 1, nullptr) == CA2_ERR_INVALID_ARG);
  ca2_cache_info info;
  CHECK(ca2_cache_info_get(nullptr, &info) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_cache_slot_map(nullptr, tpe) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_cache_commit(nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_qkv_proj_stage(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 64, 1, 3, nullptr) ==
        CA2_ERR_INVALID_ARG);

  // cache-less and toy entry points: validation before any launch
  void* p = reinterpret_cast<void*>(4096);
  CHECK(ca2_temporal_attn_frames(p, p, p, p, 1, 0, 16, 2, 64, CA2_BF16, 0, 0.125f, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_temporal_attn_frames(p, p, p, p, 1, 4, 16, 2, 16, CA2_BF16, 0, 0.125f, nullptr) == CA2_ERR_UNSUPPORTED);
  CHECK(ca2_spatial_attn_frames(p, p, p, nullptr, 1, 4, 16, 2, 64, CA2_BF16, 0.125f, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_qkv_proj(p, p, p, p, p, 8, 65, 64, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_qkv_proj(p, p, p, p, p, 8, 1 << 21, 64, nullptr) == CA2_ERR_INVALID_ARG);
  const float* fp = reinterpret_cast<const float*>(p);
  float* fo = reinterpret_cast<float*>(p);
  CHECK(ca2_toy_temb_mod(fp, 2, fp, 7, 32, fo, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_toy_ln_mod(fp, fp, 64, 0, 40, 2, 16, 32, fo, nullptr) == CA2_ERR_INVALID_ARG);
  CHECK(ca2_toy_linear(fp, 4, fp, 16, nullptr, 0, fo, 16, 4, 16, 8, 0, nullptr) == CA2_ERR_INVALID_ARG);

  // the last error string clears on success
  CHECK(ca2_tpe_index_raw(0, 1, 5, tpe) == CA2_OK);
  CHECK(ca2_last_error()[0] == '\0');

  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
