"""Guard for the LDS copies written in inline asm (CPU only).

The scalar-base form of global_load_lds_dwordx4 takes its LDS destination in
M0, and the copy helper writes M0 itself right before the copy (the
compiler's builtin for this copy only offers a 64-bit per-lane address, one
extra VALU add and two registers per copy, and makes every workgroup-scope
release fence wait for all outstanding copies, which would drain the copy
pipeline at every tile barrier). The compiler treats M0 as its own register,
so this stays correct only while nothing the compiler emits lives in M0.
This test compiles the kernels that use the helper to gfx950 assembly with
the library's own flags and checks, over every line that names M0:
  * each one is the helper's `s_mov_b32 m0, sN`, and the very next
    instruction is the copy that consumes it;
  * every copy is directly preceded by such a write.
So no compiler-generated instruction writes or reads M0 anywhere in these
kernels, and the asm's clobber can never destroy a value the compiler keeps
there.
"""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ["spatial_attn.hip", "qkv_proj.hip"]


def _assembly(src, out_dir):
    from causal_kv_cache_amd import build
    out = os.path.join(out_dir, src + ".s")
    cmd = ([build.hipcc()] + build.flags() + build.SOURCE_FLAGS.get(src, []) +
           ["-x", "hip", "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _instructions(text):
    """Instruction lines of an assembly listing (comments, labels and
    directives removed)."""
    out = []
    for line in text.splitlines():
        line = line.split(";", 1)[0].strip()
        if not line or line.endswith(":") or line.startswith("."):
            continue
        out.append(line)
    return out


@pytest.fixture(scope="module")
def listings(tmp_path_factory):
    try:
        from causal_kv_cache_amd import build
        build.hipcc()
    except Exception as e:   # pragma: no cover - the image always has hipcc
        pytest.skip(f"hipcc not available: {e}")
    d = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        texts = list(ex.map(lambda s: _assembly(s, d), SOURCES))
    return dict(zip(SOURCES, texts))


def m0_problems(text):
    """Every violation of the M0 rule in an assembly listing, and the number
    of copies checked."""
    ins = _instructions(text)
    m0 = re.compile(r"\bm0\b")
    # opcodes that read M0 without naming it (messages, relative register
    # moves, GWS / ordered-count LDS operations, interpolation, and the LDS
    # forms of buffer loads)
    implicit = re.compile(r"(s_sendmsg|s_movrel|v_movrel|ds_gws|ds_ordered_count|v_interp)\w*$")
    write = re.compile(r"s_mov_b32 m0, s\d+")
    bad, copies, writes = [], 0, 0
    for i, line in enumerate(ins):
        op = line.split()[0]
        if implicit.match(op) or (op.startswith("buffer_load") and re.search(r"\blds\b", line)):
            bad.append(f"implicit M0 use: {line!r}")
        if op == "global_load_lds_dwordx4":
            copies += 1
            if i == 0 or not write.fullmatch(ins[i - 1]):
                bad.append(f"copy not preceded by its M0 write: {line!r}")
        if m0.search(line):
            writes += 1
            if not write.fullmatch(line):
                bad.append(f"other M0 use: {line!r}")
            elif i + 1 >= len(ins) or ins[i + 1].split()[0] != "global_load_lds_dwordx4":
                bad.append(f"M0 write not followed by its copy: {line!r}")
    if copies != writes:
        bad.append(f"{copies} copies, {writes} M0 references")
    return bad, copies


@pytest.mark.parametrize("src", SOURCES)
def test_m0_written_only_by_the_copy_helper(listings, src):
    bad, copies = m0_problems(listings[src])
    assert copies > 0, src
    assert not bad, (src, bad[:5])


def test_checker_rejects_stray_m0_uses():
    ok = "\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v1, s[6:7]\n\tv_add_u32 v2, v3, v4\n"
    assert m0_problems(ok) == ([], 1)
    cases = ["\ts_mov_b32 m0, -1\n",                        # the compiler setting M0 for itself
             "\tv_movrels_b32 v0, v1\n",                       # implicit readers
             "\ts_sendmsg sendmsg(MSG_INTERRUPT)\n",
             "\tbuffer_load_dword v1, s[8:11], 0 offen lds\n"]
    for stray in cases:
        bad, _ = m0_problems(ok + stray)
        assert bad, stray
    bad, _ = m0_problems("\ts_mov_b32 m0, s4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v1, s[6:7]\n")
    assert bad                                                  # write and copy split apart
