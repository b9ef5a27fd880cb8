"""ctypes binding of libatw (include/atw.h): argument marshalling only.

Every computation runs in the HIP library; PyTorch supplies device memory
and the current stream.  If libatw.so is missing the functions raise -- there
is no fallback implementation.
"""

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libatw.so")

ATW_OK, ATW_EINVAL, ATW_EUNSUPPORTED, ATW_EWORKSPACE, ATW_EHIP = 0, -1, -2, -3, -4
ATW_F32, ATW_BF16, ATW_BF16_F32OUT = 0, 1, 2
UNBOUNDED = 1 << 62

EXPORTED = [
    "atw_prefill", "atw_prefill_workspace_bytes", "atw_decode", "atw_decode_banded", "atw_kcache_band",
    "atw_decode_workspace_bytes", "atw_pruned_terms",
    "atw_window_widths", "atw_window_plan", "atw_window_plan_device", "atw_last_error",
    "atw_version", "atw_rope_theta", "atw_window_widths_rope", "atw_pruned_terms_rope",
    "atw_prefill_rope", "atw_decode_rope", "atw_decode_banded_rope", "atw_decode_multi",
    "atw_decode_multi_workspace_bytes", "atw_prefill_sparse", "atw_block_mask_words",
    "atw_pruned_terms_sparse", "atw_decode_sparse", "atw_decode_noalloc", "atw_decode_noalloc_max_bytes",
]

SPARSE_BLOCK = 64

ATW_ROPE_PLAIN, ATW_ROPE_LINEAR, ATW_ROPE_LLAMA3, ATW_ROPE_TABLE = 0, 1, 2, 3
ATW_ROPE_HAS_WIDTHS = 1


class Rope(ctypes.Structure):
    """Mirror of struct atw_rope (include/atw.h)."""
    _fields_ = [("kind", ctypes.c_int32), ("flags", ctypes.c_int32), ("base", ctypes.c_double),
                ("factor", ctypes.c_double), ("low_freq_factor", ctypes.c_double),
                ("high_freq_factor", ctypes.c_double), ("original_max_position", ctypes.c_double),
                ("theta", ctypes.POINTER(ctypes.c_double)), ("widths", ctypes.POINTER(ctypes.c_int64))]


def rope_descriptor(rope_base, rope_scaling, head_dim):
    """atw_rope for a model's RoPE: rope_scaling None (plain) or a dict in the
    style of a model config: {"rope_type": "linear", "factor": f},
    {"rope_type": "llama3", "factor", "low_freq_factor", "high_freq_factor",
    "original_max_position_embeddings"}, or {"rope_type": "table", "theta":
    [theta_0, ...]} (explicit per-pair frequencies).  "type" is accepted for
    "rope_type".  Any of these may carry "widths": [W_0, ...], explicit
    integer windows used in place of floor(k * lambda_r) (a dict with only
    "widths" keeps the plain frequencies)."""
    r = Rope()
    r.base = float(rope_base) if rope_base is not None else 0.0
    if rope_scaling is None:
        r.kind = ATW_ROPE_PLAIN
        return r
    if rope_scaling.get("widths") is not None:
        wv = [int(x) for x in rope_scaling["widths"]]
        if len(wv) != head_dim // 2:
            raise ValueError(f"widths needs head_dim/2 = {head_dim // 2} entries (got {len(wv)})")
        wbuf = (ctypes.c_int64 * len(wv))(*wv)
        r.widths = ctypes.cast(wbuf, ctypes.POINTER(ctypes.c_int64))
        r.flags = ATW_ROPE_HAS_WIDTHS
        r._keep_widths = wbuf
    kind = rope_scaling.get("rope_type", rope_scaling.get("type"))
    if kind is None or kind == "default":
        r.kind = ATW_ROPE_PLAIN
    elif kind == "linear":
        r.kind = ATW_ROPE_LINEAR
        r.factor = float(rope_scaling["factor"])
    elif kind == "llama3":
        r.kind = ATW_ROPE_LLAMA3
        r.factor = float(rope_scaling["factor"])
        r.low_freq_factor = float(rope_scaling["low_freq_factor"])
        r.high_freq_factor = float(rope_scaling["high_freq_factor"])
        r.original_max_position = float(rope_scaling.get("original_max_position_embeddings",
                                                         rope_scaling.get("original_max_position")))
    elif kind == "table":
        vals = [float(x) for x in rope_scaling["theta"]]
        if len(vals) != head_dim // 2:
            raise ValueError(f"theta needs head_dim/2 = {head_dim // 2} entries (got {len(vals)})")
        buf = (ctypes.c_double * len(vals))(*vals)
        r.kind = ATW_ROPE_TABLE
        r.theta = ctypes.cast(buf, ctypes.POINTER(ctypes.c_double))
        r._keep = buf
    else:
        raise ValueError(f"unknown rope_scaling type {kind!r}")
    return r


class AtwError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"atw error {code}: {msg}")
        self.code = code


_lib = None

_i32, _i64, _f64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
_pi64 = ctypes.POINTER(ctypes.c_int64)
_pi32 = ctypes.POINTER(ctypes.c_int32)


def load_library(path=LIB_PATH):
    """Load libatw.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run rope_frequency_pair_amd.build.build() "
                           "(hipcc, gfx950) first; there is no fallback path")
    lib = ctypes.CDLL(path)
    lib.atw_prefill.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _i32, _i32, _pi32,
                                _i32, _pi64, _pi64, _pi64, _pi64, _f64, _f64, _i32, _i32, _f64, _vp,
                                ctypes.c_size_t, _vp]
    lib.atw_prefill.restype = ctypes.c_int
    lib.atw_prefill_workspace_bytes.argtypes = [_i32, _i64, _i32, _i64, _i32]
    lib.atw_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.atw_decode.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _pi64, _pi64, _i32, _i32, _pi32, _i32,
                               _pi64, _pi64, _pi64, _pi64, _f64, _f64, _i32, _i32, _f64, _i32, _vp,
                               ctypes.c_size_t, _vp]
    lib.atw_decode.restype = ctypes.c_int
    lib.atw_decode_banded.argtypes = lib.atw_decode.argtypes
    lib.atw_decode_banded.restype = ctypes.c_int
    lib.atw_decode_noalloc.argtypes = lib.atw_decode.argtypes[:22] + [_vp]
    lib.atw_decode_noalloc.restype = ctypes.c_int
    lib.atw_decode_noalloc_max_bytes.argtypes = []
    lib.atw_decode_noalloc_max_bytes.restype = ctypes.c_size_t
    lib.atw_kcache_band.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _i64, _i64, _pi64, _pi64, _vp]
    lib.atw_kcache_band.restype = ctypes.c_int
    lib.atw_decode_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32]
    lib.atw_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.atw_pruned_terms.argtypes = [_i64, _i64, _i64, _i32, _f64, _f64, _i32, _i32, _pi64, _pi64]
    lib.atw_pruned_terms.restype = ctypes.c_int
    lib.atw_window_widths.argtypes = [_i32, _f64, _f64, _i32, _pi64]
    lib.atw_window_widths.restype = ctypes.c_int
    lib.atw_window_plan.argtypes = [_i32, _f64, _f64, _i32, _i64, _i64, _i64, _i32, _i32, _i32, _pi32]
    lib.atw_window_plan.restype = ctypes.c_int
    lib.atw_window_plan_device.argtypes = [_i32, _f64, _f64, _i32, _i64, _i64, _i64, _i32, _i32, _i32,
                                           _vp, _vp, _vp]
    lib.atw_window_plan_device.restype = ctypes.c_int
    _prope = ctypes.POINTER(Rope)
    lib.atw_rope_theta.argtypes = [_prope, _i32, ctypes.POINTER(ctypes.c_double)]
    lib.atw_rope_theta.restype = ctypes.c_int
    lib.atw_window_widths_rope.argtypes = [_prope, _i32, _f64, _i32, _pi64]
    lib.atw_window_widths_rope.restype = ctypes.c_int
    lib.atw_pruned_terms_rope.argtypes = [_i64, _i64, _i64, _i32, _prope, _f64, _i32, _i32, _pi64, _pi64]
    lib.atw_pruned_terms_rope.restype = ctypes.c_int
    lib.atw_prefill_rope.argtypes = lib.atw_prefill.argtypes[:17] + [_prope] + lib.atw_prefill.argtypes[18:]
    lib.atw_prefill_rope.restype = ctypes.c_int
    lib.atw_decode_rope.argtypes = lib.atw_decode.argtypes[:16] + [_prope] + lib.atw_decode.argtypes[17:]
    lib.atw_decode_rope.restype = ctypes.c_int
    lib.atw_decode_banded_rope.argtypes = lib.atw_decode_rope.argtypes
    lib.atw_decode_banded_rope.restype = ctypes.c_int
    lib.atw_decode_multi.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _i32, _pi64, _pi64, _i32, _i32, _pi32,
                                     _i32, _pi64, _pi64, _pi64, _pi64, _i32, _prope, _f64, _i32, _f64,
                                     _i32, _vp, ctypes.c_size_t, _vp]
    lib.atw_decode_multi.restype = ctypes.c_int
    lib.atw_decode_multi_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, _i32]
    lib.atw_decode_multi_workspace_bytes.restype = ctypes.c_size_t
    # prefill_rope's arguments with the block mask before the workspace
    lib.atw_prefill_sparse.argtypes = lib.atw_prefill_rope.argtypes[:22] + [_vp] + lib.atw_prefill_rope.argtypes[22:]
    lib.atw_prefill_sparse.restype = ctypes.c_int
    lib.atw_block_mask_words.argtypes = [_i64]
    lib.atw_block_mask_words.restype = ctypes.c_int64
    lib.atw_pruned_terms_sparse.argtypes = [_i64, _i64, _i64, _i32, _prope, _f64, _i32, _i32, _vp, _pi64, _pi64]
    lib.atw_pruned_terms_sparse.restype = ctypes.c_int
    lib.atw_decode_sparse.argtypes = (lib.atw_decode_rope.argtypes[:22] + [_vp, _i64, _i32] +
                                      lib.atw_decode_rope.argtypes[22:])
    lib.atw_decode_sparse.restype = ctypes.c_int
    lib.atw_last_error.argtypes = []
    lib.atw_last_error.restype = ctypes.c_char_p
    lib.atw_version.argtypes = []
    lib.atw_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(code):
    if code != ATW_OK:
        raise AtwError(code, _lib.atw_last_error().decode())


def _arr64(vals):
    vals = list(vals)
    return (ctypes.c_int64 * len(vals))(*vals)


def _arr32(vals):
    vals = list(vals)
    return (ctypes.c_int32 * len(vals))(*vals)


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return ATW_BF16
    if t.dtype == torch.float32:
        return ATW_F32
    raise AtwError(ATW_EUNSUPPORTED, f"unsupported dtype {t.dtype}")


def _io_code(q, out):
    """Element-type code of a call: the inputs' type, or ATW_BF16_F32OUT for
    bf16 inputs written to an fp32 output tensor."""
    import torch
    if q.dtype == torch.bfloat16 and out.dtype == torch.float32:
        return ATW_BF16_F32OUT
    if out.dtype != q.dtype:
        raise AtwError(ATW_EUNSUPPORTED, f"output dtype {out.dtype} with inputs of dtype {q.dtype}")
    return _dtype_code(q)


def _head_map(kv_head_of_q):
    if kv_head_of_q is None:
        return None
    return _arr32(int(x) for x in kv_head_of_q)


def version():
    return load_library().atw_version().decode()


def window_widths(head_dim, rope_base, k_turns, window_on=True, rope_scaling=None):
    """Integer windows W_r (list of int) computed by the library."""
    lib = load_library()
    out = (ctypes.c_int64 * (head_dim // 2))()
    if rope_scaling is None:
        _check(lib.atw_window_widths(head_dim, float(rope_base), float(k_turns), int(window_on), out))
    else:
        r = rope_descriptor(rope_base, rope_scaling, head_dim)
        _check(lib.atw_window_widths_rope(ctypes.byref(r), head_dim, float(k_turns), int(window_on), out))
    return list(out)


def rope_theta(head_dim, rope_base, rope_scaling=None):
    """theta_r of every pair (list of float) as the library computes them."""
    lib = load_library()
    out = (ctypes.c_double * (head_dim // 2))()
    r = rope_descriptor(rope_base, rope_scaling, head_dim)
    _check(lib.atw_rope_theta(ctypes.byref(r), head_dim, out))
    return list(out)


def pruned_terms(n_q, n_kv, q_pos0, head_dim, rope_base, k_turns, causal=True, window_on=True,
                 rope_scaling=None):
    """(pruned, total) pair-term counts per (batch, query head)."""
    lib = load_library()
    p, t = ctypes.c_int64(), ctypes.c_int64()
    if rope_scaling is None:
        _check(lib.atw_pruned_terms(n_q, n_kv, q_pos0, head_dim, float(rope_base), float(k_turns),
                                    int(causal), int(window_on), ctypes.byref(p), ctypes.byref(t)))
    else:
        r = rope_descriptor(rope_base, rope_scaling, head_dim)
        _check(lib.atw_pruned_terms_rope(n_q, n_kv, q_pos0, head_dim, ctypes.byref(r), float(k_turns),
                                         int(causal), int(window_on), ctypes.byref(p), ctypes.byref(t)))
    return p.value, t.value


def block_mask_words(n_kv):
    """uint32 words per block-mask row: ceil(ceil(n_kv / 64) / 32)."""
    return load_library().atw_block_mask_words(int(n_kv))


def pack_block_mask(selected):
    """Bit-pack a boolean block selection [..., n_qb, n_kb] (query block qb
    attends key block kb) into the int32 words atw_prefill_sparse reads
    [..., n_qb, ceil(n_kb / 32)] (bit kb % 32 of word kb / 32).  Host-side
    marshalling of a torch bool tensor; the result is on the same device."""
    import torch
    n_kb = selected.shape[-1]
    words = -(-n_kb // 32)
    pad = words * 32 - n_kb
    sel = torch.nn.functional.pad(selected.to(torch.int64), (0, pad))
    sel = sel.reshape(*selected.shape[:-1], words, 32)
    weights = torch.ones(32, dtype=torch.int64, device=selected.device) << torch.arange(32, device=selected.device)
    packed = (sel * weights).sum(-1)
    return torch.where(packed >= 2 ** 31, packed - 2 ** 32, packed).to(torch.int32).contiguous()


def pruned_terms_sparse(n_q, n_kv, q_pos0, head_dim, rope_base, k_turns, block_mask, causal=True,
                        window_on=True, rope_scaling=None):
    """(pruned, total) pair-term counts over the cells one head's block-sparse
    selection attends; block_mask: packed int32 words [ceil(n_q/64), words]
    (any device; copied to the host)."""
    import numpy as np
    lib = load_library()
    m = np.ascontiguousarray(block_mask.cpu().numpy().astype(np.int32).view(np.uint32))
    if m.shape != (-(-n_q // SPARSE_BLOCK), block_mask_words(n_kv)):
        raise ValueError("block_mask must be [ceil(n_q/64), block_mask_words(n_kv)]")
    r = rope_descriptor(rope_base, rope_scaling, head_dim)
    p, t = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.atw_pruned_terms_sparse(n_q, n_kv, q_pos0, head_dim, ctypes.byref(r), float(k_turns),
                                       int(causal), int(window_on), m.ctypes.data_as(ctypes.c_void_p),
                                       ctypes.byref(p), ctypes.byref(t)))
    return p.value, t.value


def window_plan(head_dim, rope_base, k_turns, window_on, n_q, n_kv, q_pos0, causal, tile_q, tile_k):
    """Host tile plan as a nested list [n_qt][n_kt] of (r_any, r_full)."""
    lib = load_library()
    n_qt, n_kt = -(-n_q // tile_q), -(-n_kv // tile_k)
    buf = (ctypes.c_int32 * (2 * n_qt * n_kt))()
    _check(lib.atw_window_plan(head_dim, float(rope_base), float(k_turns), int(window_on), n_q, n_kv,
                               q_pos0, int(causal), tile_q, tile_k, buf))
    return [[(buf[(a * n_kt + b) * 2], buf[(a * n_kt + b) * 2 + 1]) for b in range(n_kt)]
            for a in range(n_qt)]


def window_plan_device(head_dim, rope_base, k_turns, window_on, n_q, n_kv, q_pos0, causal, tile_q,
                       tile_k, stream=None):
    """Tile plan and per-tile pruned counts computed by the GPU's device code.

    Returns (plan int32 [n_qt, n_kt, 2], pruned int64 [n_qt, n_kt]) as CUDA tensors.
    """
    import torch
    lib = load_library()
    n_qt, n_kt = -(-n_q // tile_q), -(-n_kv // tile_k)
    plan = torch.empty((n_qt, n_kt, 2), dtype=torch.int32, device="cuda")
    pruned = torch.empty((n_qt, n_kt), dtype=torch.int64, device="cuda")
    _check(lib.atw_window_plan_device(head_dim, float(rope_base), float(k_turns), int(window_on), n_q,
                                      n_kv, q_pos0, int(causal), tile_q, tile_k,
                                      ctypes.c_void_p(plan.data_ptr()),
                                      ctypes.c_void_p(pruned.data_ptr()), _stream_ptr(stream)))
    return plan, pruned


def prefill_workspace_bytes(dtype_code, batch, h_kv, n_kv, head_dim):
    return load_library().atw_prefill_workspace_bytes(dtype_code, batch, h_kv, n_kv, head_dim)


def prefill(q, k, v, *, rope_base, k_turns, q_pos0=0, causal=True, window_on=True, scale=None,
            kv_head_of_q=None, out=None, workspace=None, stream=None, rope_scaling=None):
    """Windowed prefill.  q [B, Hq, Nq, d]; k, v [B, Hkv, Nkv, d] (any strides
    with d contiguous), bf16 or fp32 CUDA tensors.  Returns out [B, Hq, Nq, d].
    workspace: device buffer of prefill_workspace_bytes(...) bytes, allocated
    per call when None."""
    import torch
    lib = load_library()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise AtwError(ATW_EINVAL, f"{name} must be 4-D with a contiguous last dim")
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    need = lib.atw_prefill_workspace_bytes(_dtype_code(q), B, Hkv, Nkv, D)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if rope_scaling is None:
        entry, rope_arg = lib.atw_prefill, float(rope_base)
    else:
        rdesc = rope_descriptor(rope_base, rope_scaling, D)
        entry, rope_arg = lib.atw_prefill_rope, ctypes.byref(rdesc)
    _check(entry(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), _io_code(q, out), B, Nq, Nkv, int(q_pos0), Hq, Hkv,
        _head_map(kv_head_of_q), D, _arr64(q.stride()[:3]), _arr64(k.stride()[:3]),
        _arr64(v.stride()[:3]), _arr64(out.stride()[:3]), rope_arg, float(k_turns),
        int(causal), int(window_on), float(scale or 0.0), ws_ptr, ws_len, _stream_ptr(stream)))
    return out


def prefill_sparse(q, k, v, block_mask, *, rope_base, k_turns, q_pos0=0, causal=True, window_on=True,
                   scale=None, kv_head_of_q=None, out=None, workspace=None, stream=None,
                   rope_scaling=None):
    """prefill() restricted to a block-sparse key selection: block_mask is the
    packed int32 device tensor [B, Hq, ceil(Nq/64), block_mask_words(Nkv)]
    (pack_block_mask).  bf16 only."""
    import torch
    lib = load_library()
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dim() != 4 or t.stride(-1) != 1:
            raise AtwError(ATW_EINVAL, f"{name} must be 4-D with a contiguous last dim")
    B, Hq, Nq, D = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    want = (B, Hq, -(-Nq // SPARSE_BLOCK), block_mask_words(Nkv))
    if (block_mask.dtype != torch.int32 or tuple(block_mask.shape) != want or not block_mask.is_contiguous()
            or block_mask.device != q.device):
        raise ValueError(f"block_mask must be a contiguous int32 tensor {want} on {q.device}")
    need = lib.atw_prefill_workspace_bytes(_dtype_code(q), B, Hkv, Nkv, D)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rdesc = rope_descriptor(rope_base, rope_scaling, D)
    _check(lib.atw_prefill_sparse(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), _io_code(q, out), B, Nq, Nkv, int(q_pos0), Hq, Hkv,
        _head_map(kv_head_of_q), D, _arr64(q.stride()[:3]), _arr64(k.stride()[:3]),
        _arr64(v.stride()[:3]), _arr64(out.stride()[:3]), ctypes.byref(rdesc), float(k_turns),
        int(causal), int(window_on), float(scale or 0.0), ctypes.c_void_p(block_mask.data_ptr()),
        ws_ptr, ws_len, _stream_ptr(stream)))
    return out


def decode_workspace_bytes(batch, h_q, head_dim, num_splits):
    return load_library().atw_decode_workspace_bytes(batch, h_q, head_dim, num_splits)


def decode(q, k_cache, v_cache, kv_len, q_pos, *, rope_base, k_turns, causal=True, window_on=True,
           scale=None, num_splits=64, kv_head_of_q=None, workspace=None, out=None, stream=None,
           rope_scaling=None):
    """Windowed split-KV decode.  q [B, Hq, d]; caches [B, Hkv, L, d] bf16 CUDA
    tensors; kv_len, q_pos: per-sequence ints.  Returns out [B, Hq, d]."""
    return _decode("atw_decode", q, k_cache, v_cache, kv_len, q_pos, rope_base, k_turns, causal,
                   window_on, scale, num_splits, kv_head_of_q, workspace, out, stream, rope_scaling)


def decode_banded(q, k_bands, v_cache, kv_len, q_pos, *, rope_base, k_turns, causal=True,
                  window_on=True, scale=None, num_splits=64, kv_head_of_q=None, workspace=None,
                  out=None, stream=None, rope_scaling=None):
    """decode() over a pair-banded K cache k_bands [B, Hkv, d/16, L, 16] (token
    stride 16); v_cache [B, Hkv, L, d] as for decode()."""
    if k_bands.dim() != 5 or k_bands.shape[-1] != 16 or k_bands.stride(3) != 16:
        raise ValueError("k_bands must be [B, Hkv, d/16, L, 16] with token stride 16")
    return _decode("atw_decode_banded", q, k_bands, v_cache, kv_len, q_pos, rope_base, k_turns,
                   causal, window_on, scale, num_splits, kv_head_of_q, workspace, out, stream,
                   rope_scaling)


def kcache_band(k_rows, k_bands=None, *, t0=0, n_tokens=None, stream=None):
    """Copy keys [t0, t0 + n_tokens) of a row-layout K cache [B, Hkv, L, d] into
    a pair-banded one [B, Hkv, d/16, L, 16] (allocated when k_bands is None).
    Returns k_bands."""
    import torch
    lib = load_library()
    B, Hkv, L, D = k_rows.shape
    if k_bands is None:
        k_bands = torch.empty((B, Hkv, D // 16, L, 16), dtype=k_rows.dtype, device=k_rows.device)
    if k_bands.dim() != 5 or k_bands.shape[-1] != 16 or k_bands.stride(3) != 16:
        raise ValueError("k_bands must be [B, Hkv, d/16, L, 16] with token stride 16")
    if tuple(k_bands.shape[:3]) != (B, Hkv, D // 16) or k_bands.stride(4) != 1:
        raise ValueError("k_bands shape does not match k_rows")
    if n_tokens is None:
        n_tokens = L - t0
    if t0 < 0 or n_tokens < 0 or t0 + n_tokens > min(L, k_bands.shape[3]):
        raise ValueError("token range outside the caches")
    _check(lib.atw_kcache_band(
        ctypes.c_void_p(k_rows.data_ptr()), ctypes.c_void_p(k_bands.data_ptr()),
        _dtype_code(k_rows), B, Hkv, D, int(t0), int(n_tokens), _arr64(k_rows.stride()[:3]),
        _arr64(k_bands.stride()[:3]), _stream_ptr(stream)))
    return k_bands


def _decode(entry, q, k_cache, v_cache, kv_len, q_pos, rope_base, k_turns, causal, window_on,
            scale, num_splits, kv_head_of_q, workspace, out, stream, rope_scaling=None):
    import torch
    lib = load_library()
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    need = lib.atw_decode_workspace_bytes(B, Hq, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    kv_len = [int(x) for x in (kv_len if hasattr(kv_len, "__len__") else [kv_len] * B)]
    q_pos = [int(x) for x in (q_pos if hasattr(q_pos, "__len__") else [q_pos] * B)]
    if rope_scaling is None:
        rope_arg = float(rope_base)
    else:
        rdesc = rope_descriptor(rope_base, rope_scaling, D)
        entry, rope_arg = entry + "_rope", ctypes.byref(rdesc)
    _check(getattr(lib, entry)(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
        ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(out.data_ptr()), _io_code(q, out), B,
        _arr64(kv_len), _arr64(q_pos), Hq, Hkv, _head_map(kv_head_of_q), D,
        _arr64(q.stride()[:2]), _arr64(k_cache.stride()[:3]), _arr64(v_cache.stride()[:3]),
        _arr64(out.stride()[:2]), rope_arg, float(k_turns), int(causal), int(window_on),
        float(scale or 0.0), int(num_splits), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _stream_ptr(stream)))
    return out


def decode_noalloc(q, k_cache, v_cache, kv_len, q_pos, *, rope_base, k_turns, causal=True, window_on=True,
                   scale=None, num_splits=64, kv_head_of_q=None, out=None, stream=None):
    """decode() through atw_decode_noalloc: no workspace; the split partials
    live in the library's per-device array (decode_noalloc_max_bytes())."""
    import torch
    lib = load_library()
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    kv_len = [int(x) for x in (kv_len if hasattr(kv_len, "__len__") else [kv_len] * B)]
    q_pos = [int(x) for x in (q_pos if hasattr(q_pos, "__len__") else [q_pos] * B)]
    _check(lib.atw_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
        ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(out.data_ptr()), _io_code(q, out), B,
        _arr64(kv_len), _arr64(q_pos), Hq, Hkv, _head_map(kv_head_of_q), D,
        _arr64(q.stride()[:2]), _arr64(k_cache.stride()[:3]), _arr64(v_cache.stride()[:3]),
        _arr64(out.stride()[:2]), float(rope_base), float(k_turns), int(causal), int(window_on),
        float(scale or 0.0), int(num_splits), _stream_ptr(stream)))
    return out


def decode_noalloc_max_bytes():
    return int(load_library().atw_decode_noalloc_max_bytes())


def decode_sparse(q, k_cache, v_cache, kv_len, q_pos, block_mask, *, rope_base, k_turns, causal=True,
                  window_on=True, scale=None, num_splits=64, kv_head_of_q=None, k_banded=False,
                  workspace=None, out=None, stream=None, rope_scaling=None):
    """decode() / decode_banded() restricted to a block-sparse key selection:
    block_mask is the packed int32 device tensor [B, Hkv, words] (pack_block_mask
    of a boolean [B, Hkv, n_blocks]), words >= block_mask_words(max kv_len)."""
    import torch
    lib = load_library()
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if k_banded and (k_cache.dim() != 5 or k_cache.shape[-1] != 16 or k_cache.stride(3) != 16):
        raise ValueError("k_banded: k_cache must be [B, Hkv, d/16, L, 16] with token stride 16")
    if (block_mask.dtype != torch.int32 or block_mask.dim() != 3 or tuple(block_mask.shape[:2]) != (B, Hkv)
            or not block_mask.is_contiguous() or block_mask.device != q.device):
        raise ValueError(f"block_mask must be a contiguous int32 tensor [{B}, {Hkv}, words] on {q.device}")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    need = lib.atw_decode_workspace_bytes(B, Hq, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    kv_len = [int(x) for x in (kv_len if hasattr(kv_len, "__len__") else [kv_len] * B)]
    q_pos = [int(x) for x in (q_pos if hasattr(q_pos, "__len__") else [q_pos] * B)]
    rdesc = rope_descriptor(rope_base, rope_scaling, D)
    _check(lib.atw_decode_sparse(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
        ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(out.data_ptr()), _io_code(q, out), B,
        _arr64(kv_len), _arr64(q_pos), Hq, Hkv, _head_map(kv_head_of_q), D,
        _arr64(q.stride()[:2]), _arr64(k_cache.stride()[:3]), _arr64(v_cache.stride()[:3]),
        _arr64(out.stride()[:2]), ctypes.byref(rdesc), float(k_turns), int(causal), int(window_on),
        float(scale or 0.0), int(num_splits), ctypes.c_void_p(block_mask.data_ptr()),
        int(block_mask.shape[2]), int(bool(k_banded)), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _stream_ptr(stream)))
    return out


def decode_multi(q, k_cache, v_cache, kv_len, q_pos, *, rope_base, k_turns, window_on=True,
                 scale=None, num_splits=64, kv_head_of_q=None, k_banded=False, workspace=None,
                 out=None, stream=None, rope_scaling=None):
    """Causal decode of q_len tokens per sequence at positions q_pos[b] ..
    q_pos[b] + q_len - 1.  q [B, T, Hq, d] (T = q_len, any strides with d
    contiguous); k_cache [B, Hkv, L, d] (or the banded layout when k_banded);
    v_cache [B, Hkv, L, d].  Returns out [B, T, Hq, d]."""
    import torch
    lib = load_library()
    B, T, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=q.dtype, device=q.device)
    need = lib.atw_decode_multi_workspace_bytes(B, T, Hq, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    kv_len = [int(x) for x in (kv_len if hasattr(kv_len, "__len__") else [kv_len] * B)]
    q_pos = [int(x) for x in (q_pos if hasattr(q_pos, "__len__") else [q_pos] * B)]
    rdesc = rope_descriptor(rope_base, rope_scaling, D)
    qs = (q.stride(0), q.stride(2), q.stride(1))
    os_ = (out.stride(0), out.stride(2), out.stride(1))
    _check(lib.atw_decode_multi(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k_cache.data_ptr()),
        ctypes.c_void_p(v_cache.data_ptr()), ctypes.c_void_p(out.data_ptr()), _io_code(q, out), B, T,
        _arr64(kv_len), _arr64(q_pos), Hq, Hkv, _head_map(kv_head_of_q), D, _arr64(qs),
        _arr64(k_cache.stride()[:3]), _arr64(v_cache.stride()[:3]), _arr64(os_), int(bool(k_banded)),
        ctypes.byref(rdesc), float(k_turns), int(window_on), float(scale or 0.0), int(num_splits),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _stream_ptr(stream)))
    return out


def decode_multi_workspace_bytes(batch, q_len, h_q, head_dim, num_splits):
    return load_library().atw_decode_multi_workspace_bytes(batch, q_len, h_q, head_dim, num_splits)


def default_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)
