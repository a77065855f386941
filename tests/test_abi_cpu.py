"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments on the host before touching the device."""
import ctypes
import math
import os
import subprocess

import pytest

import head_latent_attention_absorbed_amd as mla
from head_latent_attention_absorbed_amd import MlaShape, split_plan


def _lib():
    if not os.path.exists(mla.library_path):
        pytest.fail("libmla_absorbed.so is not built (run __graft_entry__.build())")
    return mla.library()


def test_exports_every_declared_symbol():
    lib = _lib()
    declared = mla.exported_symbols()
    assert set(declared) >= {"mla_absorb_q", "mla_decode_num_parts", "mla_decode_paged", "mla_combine_lse",
                             "mla_up_v", "mla_combine_up_v", "mla_append_kv", "mla_append_kv_workspace_bytes",
                             "mla_append_kv_noalloc",
                             "mla_prefill_workspace_bytes", "mla_prefill_kv_elems", "mla_prefill_kv", "mla_prefill_attention",
                             "mla_tpla_split_weights", "mla_tpla_rotate_cache", "mla_tpla_reduce",
                             "mla_gqa_queries", "mla_gqa_output",
                             "mla_status_string", "mla_last_error"}
    out = subprocess.run(["nm", "-D", "--defined-only", mla.library_path], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, f"{name} declared in the header but not exported"
        assert hasattr(lib, name)


def test_struct_layout_matches_header(tmp_path):
    """Compile a C program against the header and compare sizeof/offsetof of
    mla_shape_t with the ctypes mirror field by field."""
    names = [f[0] for f in MlaShape._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        "#include <stdio.h>\n#include <stddef.h>\n#include \"mla_absorbed.h\"\n"
        "int main(void) {\n  printf(\"%zu\\n\", sizeof(mla_shape_t));\n"
        + "".join(f'  printf("%zu\\n", offsetof(mla_shape_t, {n}));\n' for n in names)
        + '  printf("%zu\\n", (size_t)MLA_APPEND_NOALLOC_MAX_BYTES);\n'
        + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    from head_latent_attention_absorbed_amd import binding
    inc = os.path.dirname(binding.header_path)
    r = subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", f"-I{inc}", "-I/opt/rocm/include", str(src),
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(MlaShape)
    for n, off in zip(names, vals[1:]):
        assert getattr(MlaShape, n).offset == off, n
    assert vals[-1] == mla.MLA_APPEND_NOALLOC_MAX_BYTES


def _shape(**kw):
    base = dict(batch=2, num_heads=16, q_len=1, d_latent=512, max_blocks_per_seq=4, softmax_scale=192 ** -0.5)
    base.update(kw)
    return MlaShape.make(**base)


FAKE = 1 << 40  # a 16-byte aligned address; never dereferenced by failing calls


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), mla.MLA_ERR_INVALID_ARG),
    (dict(num_heads=-1), mla.MLA_ERR_INVALID_ARG),
    (dict(softmax_scale=math.inf), mla.MLA_ERR_INVALID_ARG),
    (dict(softmax_scale=-0.07), mla.MLA_ERR_UNSUPPORTED),
    (dict(softmax_scale=0.0), mla.MLA_ERR_UNSUPPORTED),
    (dict(cache_dtype=7), mla.MLA_ERR_INVALID_ARG),
    (dict(out_dtype=mla.MLA_FP8_E4M3), mla.MLA_ERR_INVALID_ARG),
    (dict(partial_dtype=mla.MLA_BF16), mla.MLA_ERR_INVALID_ARG),
    (dict(d_latent=384), mla.MLA_ERR_UNSUPPORTED),
    (dict(d_rope=32), mla.MLA_ERR_UNSUPPORTED),
    (dict(block_size=48), mla.MLA_ERR_UNSUPPORTED),
    (dict(q_len=9), mla.MLA_ERR_UNSUPPORTED),
    (dict(batch=4096), mla.MLA_ERR_UNSUPPORTED),
])
def test_shape_validation(kw, status):
    lib = _lib()
    sh = _shape(**kw)
    st = lib.mla_absorb_q(ctypes.byref(sh), FAKE, FAKE, FAKE, None)
    assert st == status, mla.mla_last_error()
    assert mla.mla_last_error() != ""


def test_null_and_alignment_checks():
    lib = _lib()
    sh = _shape()
    assert lib.mla_absorb_q(None, FAKE, FAKE, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(ctypes.byref(sh), None, FAKE, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(ctypes.byref(sh), FAKE + 2, FAKE, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_up_v(ctypes.byref(sh), FAKE, None, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_combine_lse(ctypes.byref(sh), 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == mla.MLA_ERR_INVALID_ARG


def _combine_up(sh, num_parts=8, **kw):
    a = dict(o_part=FAKE, lse_part=FAKE, seq_lens=FAKE, w_uv=FAKE, out=FAKE, lse=FAKE)
    a.update(kw)
    return _lib().mla_combine_up_v(ctypes.byref(sh), num_parts, a["o_part"], a["lse_part"], a["seq_lens"],
                                   a["w_uv"], a["out"], a["lse"], None)


def test_combine_up_argument_checks():
    sh = _shape()
    for name in ("o_part", "lse_part", "seq_lens", "w_uv", "out", "lse"):
        assert _combine_up(sh, **{name: None}) == mla.MLA_ERR_INVALID_ARG, name
    for name in ("o_part", "w_uv", "out"):
        assert _combine_up(sh, **{name: FAKE + 4}) == mla.MLA_ERR_INVALID_ARG, name
    assert _combine_up(sh, num_parts=1) == mla.MLA_ERR_INVALID_ARG              # fewer parts than sequences
    assert _combine_up(_shape(d_v=256)) == mla.MLA_ERR_UNSUPPORTED              # no fused kernel: two calls
    assert "d_v 256" in mla.mla_last_error()
    assert _combine_up(_shape(d_v=192)) == mla.MLA_ERR_UNSUPPORTED
    assert _lib().mla_combine_up_v(None, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    from head_latent_attention_absorbed_amd import combine_up_supported
    assert combine_up_supported(512, 128) and combine_up_supported(256, 64)
    assert not combine_up_supported(512, 256) and not combine_up_supported(384, 128)


def _decode(sh, **kw):
    lib = _lib()
    a = dict(q_lat=FAKE, q_rope=FAKE, c_kv=FAKE, k_rope=FAKE + 1024, token_stride=1152, block_stride=64 * 1152,
             kv_scale=None, block_table=FAKE, seq_lens=FAKE, num_parts=8, o_part=FAKE, lse_part=FAKE)
    a.update(kw)
    return lib.mla_decode_paged(ctypes.byref(sh), a["q_lat"], a["q_rope"], a["c_kv"], a["k_rope"],
                                a["token_stride"], a["block_stride"], a["kv_scale"], a["block_table"],
                                a["seq_lens"], a["num_parts"], a["o_part"], a["lse_part"], None)


def test_decode_argument_checks():
    sh = _shape()
    assert _decode(sh, block_table=None) == mla.MLA_ERR_INVALID_ARG
    assert _decode(sh, kv_scale=FAKE) == mla.MLA_ERR_INVALID_ARG                 # scale with a bf16 cache
    assert _decode(_shape(cache_dtype=mla.MLA_FP8_E4M3), k_rope=FAKE + 512, token_stride=576,
                   block_stride=64 * 576) == mla.MLA_ERR_INVALID_ARG             # fp8 needs kv_scale
    assert _decode(sh, token_stride=1000) == mla.MLA_ERR_INVALID_ARG             # not a multiple of 16
    assert _decode(sh, block_stride=32 * 1152) == mla.MLA_ERR_INVALID_ARG        # page smaller than 64 records
    assert _decode(sh, k_rope=FAKE + 512) == mla.MLA_ERR_INVALID_ARG             # RoPE key overlaps the latent
    assert _decode(sh, k_rope=FAKE + 1152) == mla.MLA_ERR_INVALID_ARG            # RoPE key past the record
    assert _decode(sh, num_parts=1) == mla.MLA_ERR_INVALID_ARG                   # fewer parts than sequences
    assert _decode(sh, q_lat=FAKE + 8) == mla.MLA_ERR_INVALID_ARG                # misaligned


def _tile_copy(sh, **kw):
    a = dict(c_kv=FAKE, k_rope=FAKE + 1024, token_stride=1152, block_stride=64 * 1152, block_table=FAKE,
             seq_lens=FAKE, num_parts=8, sink=FAKE)
    a.update(kw)
    return _lib().mla_probe_tile_copy(ctypes.byref(sh), a["c_kv"], a["k_rope"], a["token_stride"],
                                      a["block_stride"], a["block_table"], a["seq_lens"], a["num_parts"],
                                      a["sink"], None)


def test_probe_argument_checks():
    lib = _lib()
    flops = ctypes.c_int64(0)
    assert lib.mla_probe_hbm_read(None, 1 << 20, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_hbm_read(FAKE, 1 << 20, None, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_hbm_read(FAKE + 4, 1 << 20, FAKE, None) == mla.MLA_ERR_INVALID_ARG   # misaligned
    assert lib.mla_probe_hbm_read(FAKE, 1000, FAKE, None) == mla.MLA_ERR_INVALID_ARG          # not x16
    assert lib.mla_probe_hbm_read(FAKE, 0, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_mfma(0, FAKE, ctypes.byref(flops), None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_mfma(10, None, ctypes.byref(flops), None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_probe_mfma(10, FAKE, None, None) == mla.MLA_ERR_INVALID_ARG
    wide = _shape(num_heads=128)
    assert _tile_copy(_shape()) == mla.MLA_ERR_UNSUPPORTED                    # 16 rows: no 128-row kernel
    assert _tile_copy(_shape(num_heads=128, cache_dtype=mla.MLA_FP8_E4M3), k_rope=FAKE + 512, token_stride=576,
                      block_stride=64 * 576) == mla.MLA_ERR_UNSUPPORTED      # bf16 only
    assert _tile_copy(wide, sink=None) == mla.MLA_ERR_INVALID_ARG
    assert _tile_copy(wide, k_rope=FAKE + 512) == mla.MLA_ERR_INVALID_ARG    # RoPE key overlaps the latent
    assert _tile_copy(wide, num_parts=1) == mla.MLA_ERR_INVALID_ARG
    assert _tile_copy(wide, c_kv=FAKE + 8, k_rope=FAKE + 1032) == mla.MLA_ERR_INVALID_ARG


def test_validate_argument_checks():
    lib = _lib()
    s = _shape()
    sp = ctypes.byref(s)
    assert lib.mla_validate_decode_inputs(sp, None, FAKE, 100, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_validate_decode_inputs(sp, FAKE, None, 100, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_validate_decode_inputs(sp, FAKE, FAKE, 100, None, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_validate_decode_inputs(sp, FAKE, FAKE, 0, FAKE, None) == mla.MLA_ERR_INVALID_ARG
    assert lib.mla_validate_decode_inputs(sp, FAKE, FAKE, 100, FAKE + 2, None) == mla.MLA_ERR_INVALID_ARG
    bad = _shape(block_size=48)
    assert lib.mla_validate_decode_inputs(ctypes.byref(bad), FAKE, FAKE, 100, FAKE, None) != mla.MLA_OK


def test_status_strings():
    _lib()
    assert mla.mla_status_string(0) == "MLA_OK"
    for st in (1, 2, 3):
        assert mla.mla_status_string(st).startswith("MLA_ERR")


def test_split_plan_covers_every_tile_once():
    lens = [0, 1, 31, 32, 33, 700, 0, 64]
    for parts in (8, 9, 12, 40, 300):
        plan = split_plan(lens, parts)
        # parts never cross a sequence, take consecutive slots in sequence order,
        # and W is the smallest tile count per part that fits the slots
        assert [s for s, *_ in plan] == list(range(len(plan)))
        assert [b for _, b, *_ in plan] == sorted(b for _, b, *_ in plan)
        W = max((t1 - t0 + 31) // 32 for _, _, t0, t1 in plan)
        n = [(L + 31) // 32 for L in lens]
        assert sum(-(-x // W) for x in n) <= parts
        assert W == 1 or sum(-(-x // (W - 1)) for x in n) > parts
        covered = {b: [] for b in range(len(lens))}
        slots = set()
        for slot, b, t0, t1 in plan:
            assert slot not in slots and 0 <= slot < parts
            slots.add(slot)
            covered[b].append((t0, t1))
        for b, L in enumerate(lens):
            segs = sorted(covered[b])
            pos = 0
            for t0, t1 in segs:
                assert t0 == pos and t1 > t0
                pos = t1
            assert pos == L


def _append(sh, d_model=4096, ws_bytes=None, **kw):
    lib = _lib()
    need = ctypes.c_size_t(0)
    st = lib.mla_append_kv_workspace_bytes(ctypes.byref(sh), d_model, ctypes.byref(need))
    a = dict(x=FAKE, w=FAKE, base=10000.0, c_kv=FAKE, k_rope=FAKE + 1024, ts=1152, bst=64 * 1152, kv_scale=None,
             bt=FAKE, sl=FAKE, ws=FAKE)
    a.update(kw)
    nbytes = need.value if ws_bytes is None else ws_bytes
    return lib.mla_append_kv(ctypes.byref(sh), d_model, a["x"], a["w"], a["base"], a["c_kv"], a["k_rope"], a["ts"],
                             a["bst"], a["kv_scale"], a["bt"], a["sl"], a["ws"], nbytes, None), st, need.value


def test_append_workspace_size():
    lib = _lib()
    sh = _shape(batch=3, q_len=2)
    n = ctypes.c_size_t(0)
    assert lib.mla_append_kv_workspace_bytes(ctypes.byref(sh), 4096, ctypes.byref(n)) == mla.MLA_OK
    assert n.value == 3 * 2 * (4096 // 256) * (512 + 64) * 4
    assert lib.mla_append_kv_workspace_bytes(ctypes.byref(sh), 1000, ctypes.byref(n)) == mla.MLA_ERR_UNSUPPORTED
    assert lib.mla_append_kv_workspace_bytes(ctypes.byref(sh), 4096, None) == mla.MLA_ERR_INVALID_ARG


def test_append_argument_checks():
    sh = _shape()
    for name in ("x", "w", "c_kv", "bt", "sl", "ws"):
        assert _append(sh, **{name: None})[0] == mla.MLA_ERR_INVALID_ARG, name
    assert _append(sh, x=FAKE + 2)[0] == mla.MLA_ERR_INVALID_ARG                     # misaligned
    assert _append(sh, base=1.0)[0] == mla.MLA_ERR_INVALID_ARG                       # rope_base must exceed 1
    assert _append(sh, base=math.nan)[0] == mla.MLA_ERR_INVALID_ARG
    assert _append(sh, kv_scale=FAKE)[0] == mla.MLA_ERR_INVALID_ARG                  # scale with a bf16 cache
    assert _append(_shape(cache_dtype=mla.MLA_FP8_E4M3), k_rope=FAKE + 512, ts=576,
                   bst=64 * 576)[0] == mla.MLA_ERR_INVALID_ARG                       # fp8 needs kv_scale
    assert _append(sh, k_rope=FAKE + 512)[0] == mla.MLA_ERR_INVALID_ARG              # RoPE key overlaps the latent
    assert _append(sh, d_model=1000)[0] == mla.MLA_ERR_UNSUPPORTED                   # not a multiple of 256
    st, _, need = _append(sh)
    assert _append(sh, ws_bytes=need - 4)[0] == mla.MLA_ERR_INVALID_ARG              # workspace too small
    assert "workspace" in mla.mla_last_error()


def _append_noalloc(sh, d_model=4096, **kw):
    lib = _lib()
    a = dict(x=FAKE, w=FAKE, base=10000.0, c_kv=FAKE, k_rope=FAKE + 1024, ts=1152, bst=64 * 1152, kv_scale=None,
             bt=FAKE, sl=FAKE)
    a.update(kw)
    return lib.mla_append_kv_noalloc(ctypes.byref(sh), d_model, a["x"], a["w"], a["base"], a["c_kv"], a["k_rope"],
                                     a["ts"], a["bst"], a["kv_scale"], a["bt"], a["sl"], None)


def test_append_noalloc_argument_checks():
    """The no-allocation append checks its arguments like mla_append_kv, and
    refuses, before touching the device, a request whose partial products do
    not fit the library's fixed scratch array."""
    sh = _shape()
    for name in ("x", "w", "c_kv", "bt", "sl"):
        assert _append_noalloc(sh, **{name: None}) == mla.MLA_ERR_INVALID_ARG, name
    assert _append_noalloc(sh, x=FAKE + 2) == mla.MLA_ERR_INVALID_ARG
    assert _append_noalloc(sh, base=1.0) == mla.MLA_ERR_INVALID_ARG
    assert _append_noalloc(sh, k_rope=FAKE + 512) == mla.MLA_ERR_INVALID_ARG
    assert _append_noalloc(sh, d_model=1000) == mla.MLA_ERR_UNSUPPORTED
    # 228 rows x 16 slices x 576 values x 4 bytes > 8 MiB; 227 rows fit
    lib = _lib()
    for rows, fits in ((227, True), (228, False)):
        big = _shape(batch=rows)
        need = ctypes.c_size_t(0)
        assert lib.mla_append_kv_workspace_bytes(ctypes.byref(big), 4096, ctypes.byref(need)) == mla.MLA_OK
        assert (need.value <= mla.MLA_APPEND_NOALLOC_MAX_BYTES) == fits
    assert _append_noalloc(_shape(batch=228)) == mla.MLA_ERR_UNSUPPORTED
    assert "scratch" in mla.mla_last_error()
    assert _append_noalloc(_shape(batch=57, q_len=4)) == mla.MLA_ERR_UNSUPPORTED   # 228 rows again
    assert _append_noalloc(_shape(batch=16), d_model=65536) == mla.MLA_ERR_UNSUPPORTED  # 16 rows x 256 slices


def test_prefill_argument_checks():
    lib = _lib()
    sh = _shape()
    need = ctypes.c_size_t(0)
    assert lib.mla_prefill_workspace_bytes(ctypes.byref(sh), ctypes.byref(need)) == mla.MLA_OK
    assert need.value == 16 * 512 * 128 * 2
    kv = lambda shp, **kw: lib.mla_prefill_kv(ctypes.byref(shp), kw.get("P", 64), kw.get("ckr", FAKE), FAKE, FAKE,
                                             kw.get("lens", FAKE), FAKE, FAKE, kw.get("ws", FAKE),
                                             kw.get("nb", need.value), None)
    att = lambda shp, **kw: lib.mla_prefill_attention(ctypes.byref(shp), kw.get("P", 64), FAKE, FAKE, FAKE,
                                                      kw.get("ckr", FAKE), FAKE, FAKE, kw.get("out", FAKE), FAKE, None)
    assert kv(sh, ckr=None) == mla.MLA_ERR_INVALID_ARG
    assert kv(sh, ws=FAKE + 8) == mla.MLA_ERR_INVALID_ARG          # misaligned workspace
    assert kv(sh, nb=need.value - 2) == mla.MLA_ERR_INVALID_ARG    # workspace too small
    assert kv(sh, P=0) == mla.MLA_ERR_INVALID_ARG
    assert kv(sh, P=(1 << 20) + 1) == mla.MLA_ERR_INVALID_ARG     # positions must fit 32-bit offsets
    assert kv(sh, lens=None) == mla.MLA_ERR_INVALID_ARG
    n = ctypes.c_int64(0)
    assert lib.mla_prefill_kv_elems(ctypes.byref(sh), 65, ctypes.byref(n)) == mla.MLA_OK
    assert n.value == sh.batch * sh.num_heads * 3 * 32 * 128      # three 32-position tiles per sequence
    assert kv(_shape(d_v=64)) == mla.MLA_ERR_UNSUPPORTED           # kernels exist for d_v 128
    assert att(sh, out=None) == mla.MLA_ERR_INVALID_ARG
    assert att(sh, ckr=FAKE + 4) == mla.MLA_ERR_INVALID_ARG
    assert att(_shape(d_nope=192)) == mla.MLA_ERR_UNSUPPORTED
    # records and outputs are bf16 only: other dtypes in the shape are refused
    assert kv(_shape(cache_dtype=mla.MLA_FP8_E4M3)) == mla.MLA_ERR_UNSUPPORTED
    assert att(_shape(out_dtype=mla.MLA_FP32)) == mla.MLA_ERR_UNSUPPORTED
    assert att(_shape(cache_dtype=mla.MLA_FP8_E4M3)) == mla.MLA_ERR_UNSUPPORTED


def test_tpla_argument_checks():
    lib = _lib()
    sh = _shape()
    split = lambda shp, n=2, **kw: lib.mla_tpla_split_weights(ctypes.byref(shp), n, 1, kw.get("w_uk", FAKE), FAKE,
                                                               FAKE, kw.get("out", FAKE), None)
    assert split(sh, n=3) == mla.MLA_ERR_UNSUPPORTED
    assert split(sh, n=8) == mla.MLA_ERR_UNSUPPORTED
    assert split(sh, w_uk=None) == mla.MLA_ERR_INVALID_ARG
    assert split(sh, out=FAKE + 2) == mla.MLA_ERR_INVALID_ARG
    rot = lambda shp, **kw: lib.mla_tpla_rotate_cache(ctypes.byref(shp), kw.get("c", FAKE), kw.get("ts", 1152),
                                                      kw.get("bs", 1152 * 64), kw.get("np", 4), None)
    assert rot(_shape(cache_dtype=mla.MLA_FP8_E4M3), ts=576, bs=576 * 64) == mla.MLA_ERR_UNSUPPORTED
    assert rot(sh, c=None) == mla.MLA_ERR_INVALID_ARG
    assert rot(sh, ts=1000) == mla.MLA_ERR_INVALID_ARG               # latent does not fit the record
    assert rot(sh, bs=1152 * 63) == mla.MLA_ERR_INVALID_ARG          # pages overlap
    assert rot(sh, np=-1) == mla.MLA_ERR_INVALID_ARG
    red = lambda shp, n=2, **kw: lib.mla_tpla_reduce(ctypes.byref(shp), n, kw.get("parts", FAKE), FAKE, None)
    assert red(sh, n=0) == mla.MLA_ERR_INVALID_ARG
    assert red(sh, parts=None) == mla.MLA_ERR_INVALID_ARG
    assert red(sh, parts=FAKE + 4) == mla.MLA_ERR_INVALID_ARG


def test_gqa_argument_checks():
    lib = _lib()
    q = lambda shp, g=4, **kw: lib.mla_gqa_queries(ctypes.byref(shp), g, kw.get("qn", FAKE), FAKE, FAKE,
                                                   kw.get("qr", FAKE), None)
    o = lambda shp, g=4, **kw: lib.mla_gqa_output(ctypes.byref(shp), g, FAKE, FAKE, kw.get("out", FAKE), FAKE, None)
    sh = _shape()                                              # 16 heads
    assert q(sh, g=3) == mla.MLA_ERR_INVALID_ARG                # 16 heads do not split into 3 groups
    assert q(sh, g=0) == mla.MLA_ERR_INVALID_ARG
    assert q(_shape(d_v=64)) == mla.MLA_ERR_UNSUPPORTED         # d_nope + d_v = 192: no decode of that width
    assert q(_shape(batch=300), g=4) == mla.MLA_ERR_UNSUPPORTED  # 1200 streams
    assert q(sh, qn=None) == mla.MLA_ERR_INVALID_ARG
    assert q(sh, qr=FAKE + 2) == mla.MLA_ERR_INVALID_ARG
    assert o(sh, out=None) == mla.MLA_ERR_INVALID_ARG
    assert o(sh, out=FAKE + 8) == mla.MLA_ERR_INVALID_ARG
