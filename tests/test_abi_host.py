"""C-ABI checks that run without a GPU: the library loads, exports every entry
point include/ca2.h declares, and its pure host functions agree bit-exactly
with the oracle's independent constructions. Error paths that return before
any HIP call are forced from the host."""
import ctypes
import os
import re

import pytest

from oracle import TemporalQueue, SpatialCache, tpe_index_ref, bytes_resident_ref
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ca2.h")
LIB = os.path.join(ROOT, "causal_kv_cache_amd", "libca2.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libca2.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ca2_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from causal_kv_cache_amd import ca2
    ca2.load()
    return ca2


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 15
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n
    assert sorted(lib.EXPORTS) == names


def test_tpe_index_raw_matches_oracle(lib):
    for L in (13, 33, 49):
        for first in list(range(0, 120)) + [10 ** 6 + 3]:
            assert lib.ca2_tpe_index_raw(first, 8, L) == tpe_index_ref(first, 8, L)


def test_ring_slot_map_matches_oracle_queue(lib):
    for p_max, writes in ((9, [1, 4, 4, 4, 4, 4]), (41, [1] + [8] * 12), (25, [1, 8, 8, 8, 8, 8]),
                          (5, [1, 2, 3, 7, 1, 1, 9])):
        q = TemporalQueue(p_max)
        fw = 0
        assert lib.ca2_ring_slot_map_raw(0, p_max) == []
        for w in writes:
            q.write(range(fw, fw + w))
            fw += w
            assert lib.ca2_ring_slot_map_raw(fw, p_max) == q.slot_map()


def test_spatial_map_matches_oracle_frames(lib):
    for p, writes in ((3, [1, 8, 8, 1, 2, 8]), (1, [1, 4, 4, 4]), (2, [1, 1, 3, 1])):
        c = SpatialCache(p)
        fw = 0
        for w in writes:
            c.write(range(fw, fw + w))
            fw += w
            frames, slots = lib.ca2_spatial_slot_map_raw(fw, p)
            assert frames == c.logical_frames()
            # each logical frame sits in slot frame mod P' (distinct for distinct frames)
            assert slots == [f % p for f in frames]


def test_bytes_resident_matches_oracle(lib):
    for name, sh in synth.WORKLOADS.items():
        cfg = lib.make_config(sh["B"], sh["H"], sh["d"], sh["S"], sh["l"], sh["p_max"],
                              sh["p_spatial"], sh["tpe_len"], sh["dtype"])
        eb = 2 if sh["dtype"] == "bf16" else 4
        assert lib.ca2_bytes_resident(cfg) == bytes_resident_ref(
            sh["B"], sh["S"], sh["H"], sh["d"], sh["p_max"], sh["p_spatial"], eb), name


@pytest.mark.parametrize("field,value", [
    ("batch", 0), ("heads", 0), ("tokens", 0), ("chunk", 0), ("chunk", 17), ("p_max", 0),
    ("p_spatial", -1), ("p_spatial", 8), ("tpe_len", 32), ("dtype", 7),
])
def test_create_rejects_bad_config_before_any_device_call(lib, field, value):
    sh = synth.WORKLOADS["ar_step_s256"]
    cfg = lib.make_config(sh["B"], sh["H"], sh["d"], sh["S"], sh["l"], sh["p_max"],
                          sh["p_spatial"], sh["tpe_len"], sh["dtype"])
    setattr(cfg, field, value)
    for create in (lib.ca2_cache_create, lib.ca2_cache_create_staged):
        with pytest.raises(lib.Ca2Error) as e:
            create(cfg)
        assert e.value.status == lib.CA2_ERR_INVALID_ARG
    assert lib.ca2_bytes_resident(cfg) == 0


def test_create_rejects_unbuilt_head_dim(lib):
    cfg = lib.make_config(1, 2, 16, 16, 4, 9, 1, 13, "bf16")
    with pytest.raises(lib.Ca2Error) as e:
        lib.ca2_cache_create(cfg)
    assert e.value.status == lib.CA2_ERR_UNSUPPORTED


def test_null_and_range_errors(lib):
    raw = lib.load()
    assert raw.ca2_cache_create(None, None) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_temporal_attn(None, None, None, None, None, 1, 1.0, None) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_tpe_index_raw(-1, 2, 13, None) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_tpe_index_raw(0, 2, 0, None) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_qkv_proj(None, None, None, None, None, 8, 64, 64, None) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_cache_create_staged(None, None) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_qkv_proj_stage(None, None, None, None, None, None, None, 64, 1, 3, None) == \
        lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_cache_commit(None) == lib.CA2_ERR_INVALID_ARG
    raw.ca2_cache_destroy(None)   # NULL-safe
    for s in range(6):
        assert lib.ca2_status_string(s)
    assert raw.ca2_tpe_index_raw(-1, 2, 13, None) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_last_error().decode()        # the failing call left a detail string


def test_frames_entry_points_reject_bad_arguments(lib):
    # every case fails validation before anything is launched
    raw = lib.load()
    p = ctypes.c_void_p(4096)          # aligned, never dereferenced
    t, s = raw.ca2_temporal_attn_frames, raw.ca2_spatial_attn_frames
    BAD, UNS = lib.CA2_ERR_INVALID_ARG, lib.CA2_ERR_UNSUPPORTED
    assert t(None, p, p, p, 1, 4, 16, 2, 64, 1, 0, 0.125, None) == BAD        # NULL q
    assert t(p, p, p, ctypes.c_void_p(4100), 1, 4, 16, 2, 64, 1, 0, 0.125, None) == BAD   # misaligned
    assert t(p, p, p, p, 1, 0, 16, 2, 64, 1, 0, 0.125, None) == BAD           # T = 0
    assert t(p, p, p, p, 1, 4097, 16, 2, 64, 1, 0, 0.125, None) == BAD        # T > 4096
    assert t(p, p, p, p, 1, 4096, 16, 16, 64, 1, 0, 0.125, None) == BAD       # T * H > 65535
    assert t(p, p, p, p, 1, 4, 16, 2, 64, 1, 2, 0.125, None) == BAD           # causal not 0/1
    assert t(p, p, p, p, 1, 4, 16, 2, 64, 1, 0, 0.0, None) == BAD             # scale 0
    assert t(p, p, p, p, 1, 4, 16, 2, 64, 7, 0, 0.125, None) == BAD           # dtype
    assert t(p, p, p, p, 1, 4, 16, 2, 16, 1, 0, 0.125, None) == UNS           # bf16 d=16 not built
    assert s(p, p, p, p, 1, 4, 16, 2, 16, 1, 0.125, None) == UNS
    assert s(p, p, p, p, 1, 4, 16, 2, 64, 1, float("nan"), None) == BAD
    assert s(p, p, p, None, 1, 4, 16, 2, 64, 1, 0.125, None) == BAD
    assert "NULL" in raw.ca2_last_error().decode()


def test_toy_entry_points_reject_bad_arguments(lib):
    raw = lib.load()
    p = ctypes.c_void_p(4096)          # aligned, never dereferenced
    BAD = lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_toy_temb_mod(p, 2, p, 7, 32, p, None) == BAD            # odd embedding width
    assert raw.ca2_toy_temb_mod(p, 0, p, 8, 32, p, None) == BAD            # no frames
    assert raw.ca2_toy_ln_mod(p, p, 64, 0, 40, 2, 16, 32, p, None) == BAD  # scale range past the mod row
    assert raw.ca2_toy_ln_mod(None, p, 64, 0, 32, 2, 16, 32, p, None) == BAD
    assert raw.ca2_toy_linear(p, 8, p, 16, None, 0, p, 16, 4, 16, 8, 2, None) == BAD   # act
    assert raw.ca2_toy_linear(p, 4, p, 16, None, 0, p, 16, 4, 16, 8, 0, None) == BAD   # ldx < k
    assert raw.ca2_toy_linear(p, 8, p, 16, p, 8, p, 16, 4, 16, 8, 0, None) == BAD      # ldr < n
    assert raw.ca2_toy_linear(p, 8, None, 16, None, 0, p, 16, 4, 16, 8, 0, None) == BAD


def test_slot_maps_random_write_sequences(lib):
    """Property check over random chunked write sequences: after every write the
    library's ring and spatial slot maps (one counter and modular arithmetic)
    equal the oracle's step-by-step simulations (deque with explicit eviction;
    replace-oldest spatial slots), and the TPE indices of the next chunk are the
    oracle's table walk."""
    hypothesis = pytest.importorskip("hypothesis")
    st = hypothesis.strategies

    @hypothesis.settings(max_examples=150, deadline=None, derandomize=True)
    @hypothesis.given(p_max=st.integers(1, 64), p_spatial=st.integers(0, 15),
                      writes=st.lists(st.integers(1, 16), min_size=1, max_size=25),
                      tpe_extra=st.integers(0, 9))
    def check(p_max, p_spatial, writes, tpe_extra):
        q, sc = TemporalQueue(p_max), SpatialCache(p_spatial)
        fw = 0
        for w in writes:
            q.write(range(fw, fw + w))
            if p_spatial:
                sc.write(range(fw, fw + w))
            fw += w
            assert lib.ca2_ring_slot_map_raw(fw, p_max) == q.slot_map()
            if p_spatial:
                frames, slots = lib.ca2_spatial_slot_map_raw(fw, p_spatial)
                assert frames == sc.logical_frames()
                assert slots == [f % p_spatial for f in frames]
            L = p_max + 16 + tpe_extra
            assert lib.ca2_tpe_index_raw(fw, 16, L) == tpe_index_ref(fw, 16, L)

    check()


def test_abi_version_matches_header(lib):
    """The library reports the ABI version the header declares, and the
    binding was written for the same one."""
    import re
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ca2.h")).read()
    declared = int(re.search(r"#define CA2_ABI_VERSION (\d+)", hdr).group(1))
    assert lib.load().ca2_abi_version() == declared == lib.ABI_VERSION


def test_temporal_variant_switch_range(lib):
    raw = lib.load()
    assert raw.ca2_set_temporal_variant(-1) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_set_temporal_variant(3) == lib.CA2_ERR_INVALID_ARG
    for v in (2, 1, 0):
        assert raw.ca2_set_temporal_variant(v) == lib.CA2_OK


def test_spatial_variant_switch_range(lib):
    raw = lib.load()
    assert raw.ca2_set_spatial_variant(-1) == lib.CA2_ERR_INVALID_ARG
    assert raw.ca2_set_spatial_variant(5) == lib.CA2_ERR_INVALID_ARG
    for v in (4, 3, 2, 1, 0):
        assert raw.ca2_set_spatial_variant(v) == lib.CA2_OK
