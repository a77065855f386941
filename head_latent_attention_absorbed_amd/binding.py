"""ctypes binding of libmla_absorbed.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
import re

MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_HIP = 3

MLA_BF16 = 0
MLA_FP8_E4M3 = 1
MLA_FP32 = 2
MLA_FP16 = 3

MLA_TILE_TOKENS = 32

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
library_path = os.path.join(_HERE, "libmla_absorbed.so")
header_path = os.path.join(_ROOT, "include", "mla_absorbed.h")


class MlaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("d_nope", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("cache_dtype", ctypes.c_int),
        ("out_dtype", ctypes.c_int),
        ("partial_dtype", ctypes.c_int),
    ]

    @classmethod
    def make(cls, *, batch, num_heads, q_len, d_latent, max_blocks_per_seq, softmax_scale,
             cache_dtype=MLA_BF16, out_dtype=MLA_BF16, partial_dtype=MLA_FP32, d_nope=128, d_rope=64, d_v=128,
             block_size=64):
        return cls(batch, num_heads, q_len, d_nope, d_rope, d_latent, d_v, block_size, max_blocks_per_seq,
                   softmax_scale, cache_dtype, out_dtype, partial_dtype)


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {message}")


def _status_name(st):
    return {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_HIP"}.get(st, str(st))


_lib = None


def library() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it first (python -m head_latent_attention_absorbed_amd.build_lib "
            "or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(library_path)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    SP = ctypes.POINTER(MlaShape)
    lib.mla_absorb_q.argtypes = [SP, P, P, P, P]
    lib.mla_decode_num_parts.argtypes = [SP, ctypes.POINTER(I32)]
    lib.mla_decode_paged.argtypes = [SP, P, P, P, P, I64, I64, P, P, P, I32, P, P, P]
    lib.mla_combine_lse.argtypes = [SP, I32, P, P, P, P, P, P]
    lib.mla_up_v.argtypes = [SP, P, P, P, P]
    lib.mla_combine_up_v.argtypes = [SP, I32, P, P, P, P, P, P, P]
    lib.mla_append_kv_workspace_bytes.argtypes = [SP, I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_append_kv.argtypes = [SP, I32, P, P, F, P, P, I64, I64, P, P, P, P, ctypes.c_size_t, P]
    lib.mla_append_kv_noalloc.argtypes = [SP, I32, P, P, F, P, P, I64, I64, P, P, P, P]
    lib.mla_prefill_workspace_bytes.argtypes = [SP, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_prefill_kv_elems.argtypes = [SP, I32, ctypes.POINTER(ctypes.c_int64)]
    lib.mla_prefill_kv.argtypes = [SP, I32, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.mla_prefill_attention.argtypes = [SP, I32, P, P, P, P, P, P, P, P, P]
    lib.mla_tpla_split_weights.argtypes = [SP, I32, I32, P, P, P, P, P]
    lib.mla_tpla_rotate_cache.argtypes = [SP, P, I64, I64, I32, P]
    lib.mla_tpla_reduce.argtypes = [SP, I32, P, P, P]
    lib.mla_gqa_queries.argtypes = [SP, I32, P, P, P, P, P]
    lib.mla_gqa_output.argtypes = [SP, I32, P, P, P, P, P]
    for fn in ("mla_absorb_q", "mla_decode_num_parts", "mla_decode_paged", "mla_combine_lse", "mla_up_v",
               "mla_combine_up_v", "mla_append_kv_workspace_bytes", "mla_append_kv", "mla_append_kv_noalloc",
               "mla_prefill_workspace_bytes",
               "mla_prefill_kv_elems", "mla_prefill_kv", "mla_prefill_attention", "mla_tpla_split_weights",
               "mla_tpla_rotate_cache", "mla_tpla_reduce", "mla_gqa_queries", "mla_gqa_output"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.mla_probe_hbm_read.argtypes = [P, I64, P, P]
    lib.mla_probe_mfma.argtypes = [I32, P, ctypes.POINTER(ctypes.c_int64), P]
    lib.mla_probe_tile_copy.argtypes = [SP, P, P, I64, I64, P, P, I32, P, P]
    lib.mla_validate_decode_inputs.argtypes = [SP, P, P, I64, P, P]
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def exported_symbols() -> list[str]:
    """Function names the public header declares."""
    with open(header_path) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(mla_\w+)\s*\(", text, flags=re.M)))


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError(f"expected a tensor, an int address or None, got {type(x)!r}")


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st: int, where: str):
    if st != MLA_OK:
        raise MlaError(st, where, library().mla_last_error().decode())


def mla_status_string(status: int) -> str:
    return library().mla_status_string(status).decode()


def mla_last_error() -> str:
    return library().mla_last_error().decode()


def mla_absorb_q(shape: MlaShape, q_nope, w_uk, q_lat, stream=None) -> None:
    _check(library().mla_absorb_q(ctypes.byref(shape), _ptr(q_nope), _ptr(w_uk), _ptr(q_lat), _stream(stream)),
           "mla_absorb_q")


def mla_decode_num_parts(shape: MlaShape) -> int:
    n = ctypes.c_int32(0)
    _check(library().mla_decode_num_parts(ctypes.byref(shape), ctypes.byref(n)), "mla_decode_num_parts")
    return n.value


def mla_decode_paged(shape: MlaShape, q_lat, q_rope, c_kv, k_rope, token_stride: int, block_stride: int, kv_scale,
                     block_table, seq_lens, num_parts: int, o_part, lse_part, stream=None) -> None:
    _check(library().mla_decode_paged(ctypes.byref(shape), _ptr(q_lat), _ptr(q_rope), _ptr(c_kv), _ptr(k_rope),
                                      int(token_stride), int(block_stride), _ptr(kv_scale), _ptr(block_table),
                                      _ptr(seq_lens), int(num_parts), _ptr(o_part), _ptr(lse_part), _stream(stream)),
           "mla_decode_paged")


def mla_combine_lse(shape: MlaShape, num_parts: int, o_part, lse_part, seq_lens, o_lat, lse, stream=None) -> None:
    _check(library().mla_combine_lse(ctypes.byref(shape), int(num_parts), _ptr(o_part), _ptr(lse_part),
                                     _ptr(seq_lens), _ptr(o_lat), _ptr(lse), _stream(stream)), "mla_combine_lse")


def mla_up_v(shape: MlaShape, o_lat, w_uv, out, stream=None) -> None:
    _check(library().mla_up_v(ctypes.byref(shape), _ptr(o_lat), _ptr(w_uv), _ptr(out), _stream(stream)),
           "mla_up_v")


def mla_combine_up_v(shape: MlaShape, num_parts: int, o_part, lse_part, seq_lens, w_uv, out, lse,
                     stream=None) -> None:
    _check(library().mla_combine_up_v(ctypes.byref(shape), int(num_parts), _ptr(o_part), _ptr(lse_part),
                                      _ptr(seq_lens), _ptr(w_uv), _ptr(out), _ptr(lse), _stream(stream)),
           "mla_combine_up_v")


def mla_append_kv_workspace_bytes(shape: MlaShape, d_model: int) -> int:
    n = ctypes.c_size_t(0)
    _check(library().mla_append_kv_workspace_bytes(ctypes.byref(shape), int(d_model), ctypes.byref(n)),
           "mla_append_kv_workspace_bytes")
    return n.value


def mla_append_kv(shape: MlaShape, d_model: int, x, w_dkv, rope_base: float, c_kv, k_rope, token_stride: int,
                  block_stride: int, kv_scale, block_table, seq_lens, workspace, workspace_bytes: int,
                  stream=None) -> None:
    _check(library().mla_append_kv(ctypes.byref(shape), int(d_model), _ptr(x), _ptr(w_dkv), float(rope_base),
                                   _ptr(c_kv), _ptr(k_rope), int(token_stride), int(block_stride), _ptr(kv_scale),
                                   _ptr(block_table), _ptr(seq_lens), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream)), "mla_append_kv")


MLA_APPEND_NOALLOC_MAX_BYTES = 8 << 20


def mla_append_kv_noalloc(shape: MlaShape, d_model: int, x, w_dkv, rope_base: float, c_kv, k_rope, token_stride: int,
                          block_stride: int, kv_scale, block_table, seq_lens, stream=None) -> None:
    _check(library().mla_append_kv_noalloc(ctypes.byref(shape), int(d_model), _ptr(x), _ptr(w_dkv), float(rope_base),
                                           _ptr(c_kv), _ptr(k_rope), int(token_stride), int(block_stride),
                                           _ptr(kv_scale), _ptr(block_table), _ptr(seq_lens), _stream(stream)),
           "mla_append_kv_noalloc")


def mla_probe_hbm_read(buf, nbytes: int, sink, stream=None) -> None:
    _check(library().mla_probe_hbm_read(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream)), "mla_probe_hbm_read")


def mla_probe_mfma(iters: int, sink, stream=None) -> int:
    """Enqueues the MFMA probe; returns its flop count."""
    flops = ctypes.c_int64(0)
    _check(library().mla_probe_mfma(int(iters), _ptr(sink), ctypes.byref(flops), _stream(stream)), "mla_probe_mfma")
    return flops.value


def mla_probe_tile_copy(shape: MlaShape, c_kv, k_rope, token_stride: int, block_stride: int, block_table, seq_lens,
                        num_parts: int, sink, stream=None) -> None:
    _check(library().mla_probe_tile_copy(ctypes.byref(shape), _ptr(c_kv), _ptr(k_rope), int(token_stride),
                                         int(block_stride), _ptr(block_table), _ptr(seq_lens), int(num_parts),
                                         _ptr(sink), _stream(stream)), "mla_probe_tile_copy")


def mla_validate_decode_inputs(shape: MlaShape, block_table, seq_lens, num_pages: int, violations,
                               stream=None) -> None:
    """Enqueue the device check of the decode's lengths and block table;
    ``violations`` (device int32) holds the count once the stream has run."""
    _check(library().mla_validate_decode_inputs(ctypes.byref(shape), _ptr(block_table), _ptr(seq_lens),
                                                int(num_pages), _ptr(violations), _stream(stream)),
           "mla_validate_decode_inputs")


def mla_prefill_workspace_bytes(shape: MlaShape) -> int:
    n = ctypes.c_size_t(0)
    _check(library().mla_prefill_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)), "mla_prefill_workspace_bytes")
    return n.value


def mla_prefill_kv_elems(shape: MlaShape, prompt_len: int) -> int:
    """bf16 values in each of the tile-native k_nope and v buffers."""
    n = ctypes.c_int64(0)
    _check(library().mla_prefill_kv_elems(ctypes.byref(shape), int(prompt_len), ctypes.byref(n)),
           "mla_prefill_kv_elems")
    return n.value


def mla_prefill_kv(shape: MlaShape, prompt_len: int, ckr, w_uk, w_uv, seq_lens, k_nope, v, workspace,
                   workspace_bytes: int, stream=None) -> None:
    _check(library().mla_prefill_kv(ctypes.byref(shape), int(prompt_len), _ptr(ckr), _ptr(w_uk), _ptr(w_uv),
                                    _ptr(seq_lens), _ptr(k_nope), _ptr(v), _ptr(workspace), int(workspace_bytes),
                                    _stream(stream)),
           "mla_prefill_kv")


def mla_prefill_attention(shape: MlaShape, prompt_len: int, q_nope, q_rope, k_nope, ckr, v, seq_lens, out, lse,
                          stream=None) -> None:
    _check(library().mla_prefill_attention(ctypes.byref(shape), int(prompt_len), _ptr(q_nope), _ptr(q_rope),
                                           _ptr(k_nope), _ptr(ckr), _ptr(v), _ptr(seq_lens), _ptr(out), _ptr(lse),
                                           _stream(stream)), "mla_prefill_attention")


def mla_tpla_split_weights(shape: MlaShape, n_shards: int, hadamard: bool, w_uk, w_uv, w_uk_shards, w_uv_shards,
                           stream=None) -> None:
    _check(library().mla_tpla_split_weights(ctypes.byref(shape), int(n_shards), int(bool(hadamard)), _ptr(w_uk),
                                            _ptr(w_uv), _ptr(w_uk_shards), _ptr(w_uv_shards), _stream(stream)),
           "mla_tpla_split_weights")


def mla_tpla_rotate_cache(shape: MlaShape, c_kv, token_stride: int, block_stride: int, num_pages: int,
                          stream=None) -> None:
    _check(library().mla_tpla_rotate_cache(ctypes.byref(shape), _ptr(c_kv), int(token_stride), int(block_stride),
                                           int(num_pages), _stream(stream)), "mla_tpla_rotate_cache")


def mla_tpla_reduce(shape: MlaShape, n_shards: int, parts, out, stream=None) -> None:
    _check(library().mla_tpla_reduce(ctypes.byref(shape), int(n_shards), _ptr(parts), _ptr(out), _stream(stream)),
           "mla_tpla_reduce")


def mla_gqa_queries(shape: MlaShape, groups: int, q_nope, q_rope, q_cat, q_rope_g, stream=None) -> None:
    _check(library().mla_gqa_queries(ctypes.byref(shape), int(groups), _ptr(q_nope), _ptr(q_rope), _ptr(q_cat),
                                     _ptr(q_rope_g), _stream(stream)), "mla_gqa_queries")


def mla_gqa_output(shape: MlaShape, groups: int, o_lat, lse_g, out, lse, stream=None) -> None:
    _check(library().mla_gqa_output(ctypes.byref(shape), int(groups), _ptr(o_lat), _ptr(lse_g), _ptr(out), _ptr(lse),
                                    _stream(stream)), "mla_gqa_output")
