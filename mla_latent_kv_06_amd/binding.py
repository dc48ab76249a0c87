"""ctypes binding of libmla (C ABI in include/mla.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their data pointers and torch's current HIP stream are handed
to the library.  Every step of the computation runs in the library's kernels.
Importing this module loads ``libmla.so`` and raises if it has not been built
(``python -m mla_latent_kv_06_amd.build``).
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime the library binds to

# MLA_LIBRARY names another build of the same library (e.g. one with host
# sanitizers); by default the in-tree libmla.so.
_LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libmla.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"libmla.so not found at {_LIB_PATH}; build it with "
                      "`python -m mla_latent_kv_06_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

# ---- mirror of include/mla.h ---------------------------------------------------

MLA_OK = 0
STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_NULL_POINTER", 2: "MLA_ERR_BAD_SHAPE",
                3: "MLA_ERR_UNSUPPORTED", 4: "MLA_ERR_ALIGNMENT",
                5: "MLA_ERR_WORKSPACE_TOO_SMALL", 6: "MLA_ERR_HIP"}
MLA_F32, MLA_BF16, MLA_FP8_E4M3 = 0, 1, 2
STAGE_ABSORB_Q, STAGE_SPLIT_KV, STAGE_COMBINE, STAGE_ALL = 1, 2, 4, 7
PREFILL_GATHER, PREFILL_DECOMPRESS, PREFILL_ATTEND, PREFILL_ALL = 1, 2, 4, 7
STEP_PROJECT, STEP_FINALIZE_ABSORB, STEP_SPLIT_KV, STEP_COMBINE, STEP_ALL = 1, 2, 4, 8, 15

DTYPE_CODES = {"f32": MLA_F32, "bf16": MLA_BF16, "fp8": MLA_FP8_E4M3}
_TORCH_OF = {MLA_F32: (torch.float32,), MLA_BF16: (torch.bfloat16,),
             MLA_FP8_E4M3: (torch.uint8, torch.float8_e4m3fn)}

EXPORTED = ("mla_status_string", "mla_last_error", "mla_cache_row_bytes",
            "mla_cache_block_bytes", "mla_cache_append_workspace_size", "mla_cache_append",
            "mla_decode_default_splits", "mla_decode_workspace_size", "mla_decode_absorbed",
            "mla_decode_absorbed_stages", "mla_query_workspace_size", "mla_query_project",
            "mla_prefill_workspace_size", "mla_prefill", "mla_prefill_stages",
            "mla_decode_absorbed_noalloc", "mla_output_workspace_size", "mla_output_project",
            "mla_decode_output_workspace_size", "mla_decode_output", "mla_check_block_table",
            "mla_decode_step_workspace_size", "mla_decode_step", "mla_decode_step_stages")


class Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_rope_dim", ctypes.c_int32), ("qk_nope_dim", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("cache_dtype", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("flags", ctypes.c_int32)]

    @classmethod
    def make(cls, n_heads, kv_lora_rank, qk_rope_dim, qk_nope_dim, v_head_dim, block_size,
             cache_dtype="bf16", act_dtype="bf16", softmax_scale=0.0, flags=0):
        cd = DTYPE_CODES[cache_dtype] if isinstance(cache_dtype, str) else cache_dtype
        ad = DTYPE_CODES[act_dtype] if isinstance(act_dtype, str) else act_dtype
        return cls(n_heads, kv_lora_rank, qk_rope_dim, qk_nope_dim, v_head_dim, block_size,
                   cd, ad, softmax_scale, flags)

    @classmethod
    def from_workload(cls, wl, softmax_scale=0.0, flags=0):
        return cls.make(wl.n_heads, wl.kv_lora_rank, wl.qk_rope_dim, wl.qk_nope_dim,
                        wl.v_head_dim, wl.block_size, wl.cache_dtype, wl.act_dtype,
                        softmax_scale, flags)


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_DP = ctypes.POINTER(Dims)

_lib.mla_status_string.restype = ctypes.c_char_p
_lib.mla_status_string.argtypes = [ctypes.c_int]
_lib.mla_last_error.restype = ctypes.c_char_p
_lib.mla_last_error.argtypes = []
_lib.mla_cache_row_bytes.restype = _SZ
_lib.mla_cache_row_bytes.argtypes = [_DP]
_lib.mla_cache_block_bytes.restype = _SZ
_lib.mla_cache_block_bytes.argtypes = [_DP]
_lib.mla_cache_append_workspace_size.restype = ctypes.c_int
_lib.mla_cache_append_workspace_size.argtypes = [_DP, _I, _I, _I, ctypes.POINTER(_SZ)]
_lib.mla_cache_append.restype = ctypes.c_int
_lib.mla_cache_append.argtypes = [_DP, _I, _I, _I, _P, _P, _P, ctypes.c_float, ctypes.c_float,
                                  _P, _I, _P, _P, _P, _P, _SZ, _P]
_lib.mla_decode_step_workspace_size.restype = ctypes.c_int
_lib.mla_decode_step_workspace_size.argtypes = [_DP, _I, _I, _I, _I, ctypes.POINTER(_SZ)]
_lib.mla_decode_step_stages.restype = ctypes.c_int
_lib.mla_decode_step_stages.argtypes = [_DP, _I, _I, _I, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P,
                                        _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _P, _P, _SZ,
                                        ctypes.c_uint32, _P]
_lib.mla_decode_step.restype = ctypes.c_int
_lib.mla_decode_step.argtypes = _lib.mla_decode_step_stages.argtypes[:-2] + [_P]
_lib.mla_decode_default_splits.restype = _I
_lib.mla_decode_default_splits.argtypes = [_DP, _I, _I]
_lib.mla_decode_workspace_size.restype = ctypes.c_int
_lib.mla_decode_workspace_size.argtypes = [_DP, _I, _I, _I, ctypes.POINTER(_SZ)]
_lib.mla_decode_absorbed.restype = ctypes.c_int
_lib.mla_decode_absorbed.argtypes = [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I,
                                     _P, _P, _P, _SZ, _P]
_lib.mla_decode_absorbed_noalloc.restype = ctypes.c_int
_lib.mla_decode_absorbed_noalloc.argtypes = [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I,
                                             _P, _P, _P]
_lib.mla_query_workspace_size.restype = ctypes.c_int
_lib.mla_query_workspace_size.argtypes = [_DP, _I, _I, _I, _I, ctypes.POINTER(_SZ)]
_lib.mla_query_project.restype = ctypes.c_int
_lib.mla_query_project.argtypes = [_DP, _I, _I, _I, _I, _P, _P, _P, ctypes.c_float, _P, _P,
                                   ctypes.c_float, _P, _P, _P, _P, _SZ, _P]
_lib.mla_decode_absorbed_stages.restype = ctypes.c_int
_lib.mla_decode_absorbed_stages.argtypes = [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I,
                                            _P, _P, _P, _SZ, ctypes.c_uint32, _P]
_lib.mla_output_workspace_size.restype = ctypes.c_int
_lib.mla_output_workspace_size.argtypes = [_I, _I, _I, ctypes.POINTER(_SZ)]
_lib.mla_output_project.restype = ctypes.c_int
_lib.mla_output_project.argtypes = [_I, _I, _I, _P, _P, _P, _P, _SZ, _P]
_lib.mla_decode_output_workspace_size.restype = ctypes.c_int
_lib.mla_decode_output_workspace_size.argtypes = [_DP, _I, _I, _I, _I, ctypes.POINTER(_SZ)]
_lib.mla_decode_output.restype = ctypes.c_int
_lib.mla_decode_output.argtypes = [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _P, _P,
                                   _P, _P, _SZ, _P]
_lib.mla_check_block_table.restype = ctypes.c_int
_lib.mla_check_block_table.argtypes = [_DP, _I, _P, _I, _P, _I, _P, _P]

_lib.mla_prefill_workspace_size.restype = ctypes.c_int
_lib.mla_prefill_workspace_size.argtypes = [_DP, _I, _I, _I, ctypes.POINTER(_SZ)]
_lib.mla_prefill.restype = ctypes.c_int
_lib.mla_prefill.argtypes = [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _SZ, _P]
_lib.mla_prefill_stages.restype = ctypes.c_int
_lib.mla_prefill_stages.argtypes = [_DP, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _SZ,
                                    ctypes.c_uint32, _P]


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.mla_last_error().decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def _check(st: int, where: str):
    if st != MLA_OK:
        raise MLAError(st, where)


def lib() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.mla_status_string(status).decode()


def cache_row_bytes(dims: Dims) -> int:
    return _lib.mla_cache_row_bytes(ctypes.byref(dims))


def cache_block_bytes(dims: Dims) -> int:
    return _lib.mla_cache_block_bytes(ctypes.byref(dims))


def default_splits(dims: Dims, batch: int, q_len: int) -> int:
    return _lib.mla_decode_default_splits(ctypes.byref(dims), batch, q_len)


def decode_workspace_size(dims: Dims, batch: int, q_len: int, num_splits: int = 0) -> int:
    n = _SZ(0)
    _check(_lib.mla_decode_workspace_size(ctypes.byref(dims), batch, q_len, num_splits,
                                          ctypes.byref(n)), "mla_decode_workspace_size")
    return n.value


def append_workspace_size(dims: Dims, batch: int, n_new: int, d_model: int) -> int:
    n = _SZ(0)
    _check(_lib.mla_cache_append_workspace_size(ctypes.byref(dims), batch, n_new, d_model,
                                                ctypes.byref(n)), "mla_cache_append_workspace_size")
    return n.value


def query_workspace_size(dims: Dims, batch: int, q_len: int, d_model: int, q_lora_rank: int) -> int:
    n = _SZ(0)
    _check(_lib.mla_query_workspace_size(ctypes.byref(dims), batch, q_len, d_model, q_lora_rank,
                                         ctypes.byref(n)), "mla_query_workspace_size")
    return n.value


def prefill_workspace_size(dims: Dims, batch: int, q_len: int, max_blocks_per_seq: int) -> int:
    n = _SZ(0)
    _check(_lib.mla_prefill_workspace_size(ctypes.byref(dims), batch, q_len, max_blocks_per_seq,
                                           ctypes.byref(n)), "mla_prefill_workspace_size")
    return n.value


# ---- tensor marshalling ------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes, shape=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _decode_tensors(dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale, block_table,
                    seq_lens, out, lse, want_lse, need_out=True):
    """Check the decode's tensors; create out (and lse) when not given
    (need_out False: no out tensor at all)."""
    act = _TORCH_OF[dims.act_dtype]
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    H, N, R = dims.n_heads, dims.qk_nope_dim, dims.qk_rope_dim
    dc, V = dims.kv_lora_rank, dims.v_head_dim
    dev = q_nope.device
    _need(q_nope, "q_nope", act, (B, Sq, H, N), dev)
    _need(q_pe, "q_pe", act, (B, Sq, H, R), dev)
    _need(w_uk, "w_uk", act, (H, N, dc), dev)
    _need(w_uv, "w_uv", act, (H, V, dc), dev)
    _need(cache_pool, "cache_pool", _TORCH_OF[dims.cache_dtype], None, dev)
    if cache_pool.dim() != 3 or cache_pool.shape[1:] != (dims.block_size, dc + R):
        raise ValueError(f"cache_pool shape {tuple(cache_pool.shape)}")
    if dims.cache_dtype == MLA_FP8_E4M3:
        _need(cache_scale, "cache_scale", (torch.float32,), cache_pool.shape[:2], dev)
    _need(block_table, "block_table", (torch.int32,), None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table shape {tuple(block_table.shape)}")
    _need(seq_lens, "seq_lens", (torch.int32,), (B,), dev)
    if need_out:
        if out is None:
            out = torch.empty((B, Sq, H, V), dtype=act[0], device=dev)
        _need(out, "out", act, (B, Sq, H, V), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (B, Sq, H), dev)
    return B, Sq, dev, out, lse


def decode(dims: Dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale, block_table, seq_lens,
           num_splits: int = 0, out=None, lse=None, workspace=None,
           stages: int = STAGE_ALL, want_lse: bool = True):
    """One absorbed-MLA decode step (mla_decode_absorbed[_stages]).

    q_nope [B, Sq, H, N], q_pe [B, Sq, H, R] (act dtype); w_uk [H, N, d_c],
    w_uv [H, V, d_c]; cache_pool [num_blocks, block_size, d_c + R] (cache dtype);
    cache_scale [num_blocks, block_size] float32 (fp8 only); block_table
    [B, max_blocks] int32; seq_lens [B] int32.  Returns (out, lse)."""
    B, Sq, dev, out, lse = _decode_tensors(dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                                           block_table, seq_lens, out, lse, want_lse)
    ws_bytes = decode_workspace_size(dims, B, Sq, num_splits)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), None, dev)
    st = _lib.mla_decode_absorbed_stages(
        ctypes.byref(dims), B, Sq, _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
        _ptr(cache_pool), _ptr(cache_scale), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), num_splits, _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), stages, _stream(dev))
    _check(st, "mla_decode_absorbed_stages")
    return out, lse


def decode_noalloc(dims: Dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale, block_table,
                   seq_lens, out, lse=None, num_splits: int = 0):
    """mla_decode_absorbed_noalloc: the decode on the library's static scratch.
    Arguments as for ``decode``; out (and lse, if wanted) must be given, so
    that nothing is allocated.  Returns (out, lse)."""
    if out is None:
        raise ValueError("out is required (this call allocates nothing)")
    B, Sq, dev, out, lse = _decode_tensors(dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                                           block_table, seq_lens, out, lse, False)
    st = _lib.mla_decode_absorbed_noalloc(
        ctypes.byref(dims), B, Sq, _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
        _ptr(cache_pool), _ptr(cache_scale), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), num_splits, _ptr(out), _ptr(lse), _stream(dev))
    _check(st, "mla_decode_absorbed_noalloc")
    return out, lse


def check_block_table(dims: Dims, block_table, seq_lens, num_blocks: int):
    """mla_check_block_table: returns (violations, first b, first k) after a
    device synchronisation (k = -1 for a bad length)."""
    dev = block_table.device
    _need(block_table, "block_table", (torch.int32,), None, dev)
    _need(seq_lens, "seq_lens", (torch.int32,), (block_table.shape[0],), dev)
    report = torch.full((3,), -7, dtype=torch.int32, device=dev)
    _check(_lib.mla_check_block_table(ctypes.byref(dims), block_table.shape[0], _ptr(block_table),
                                      block_table.shape[1], _ptr(seq_lens), num_blocks, _ptr(report),
                                      _stream(dev)), "mla_check_block_table")
    r = report.cpu().tolist()
    return r[0], r[1], r[2]


def output_workspace_size(rows: int, k: int, n: int) -> int:
    b = _SZ(0)
    _check(_lib.mla_output_workspace_size(rows, k, n, ctypes.byref(b)), "mla_output_workspace_size")
    return b.value


def output_project(x, w, out=None, workspace=None):
    """out = x W^T (mla_output_project): x [rows, k] and w [n, k] bf16 (x may
    carry more leading axes, flattened to rows; its last axis is k).
    Returns out [..., n] bf16."""
    if x is None or w is None:
        raise ValueError("x and w are required")
    k = x.shape[-1]
    rows = x.numel() // k if k else 0
    n = w.shape[0]
    dev = x.device
    _need(x, "x", (torch.bfloat16,), None, dev)
    _need(w, "w", (torch.bfloat16,), (n, k), dev)
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (n,), dtype=torch.bfloat16, device=dev)
    _need(out, "out", (torch.bfloat16,), tuple(x.shape[:-1]) + (n,), dev)
    ws_bytes = output_workspace_size(rows, k, n)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), None, dev)
    _check(_lib.mla_output_project(rows, k, n, _ptr(x), _ptr(w), _ptr(out), _ptr(workspace),
                                   workspace.numel(), _stream(dev)), "mla_output_project")
    return out


def decode_output_workspace_size(dims: Dims, batch: int, q_len: int, num_splits: int,
                                 d_model: int) -> int:
    b = _SZ(0)
    _check(_lib.mla_decode_output_workspace_size(ctypes.byref(dims), batch, q_len, num_splits,
                                                 d_model, ctypes.byref(b)),
           "mla_decode_output_workspace_size")
    return b.value


def decode_output(dims: Dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale, block_table,
                  seq_lens, w_o, num_splits: int = 0, u=None, lse=None, workspace=None,
                  want_lse: bool = True):
    """Decode then output projection (mla_decode_output): the decode's
    arguments as for ``decode``, w_o [d_model, H * V] bf16.  Returns
    (u [B, Sq, d_model] bf16, lse)."""
    B, Sq, dev, _, lse = _decode_tensors(dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                                         block_table, seq_lens, None, lse, want_lse, need_out=False)
    _need(w_o, "w_o", (torch.bfloat16,), None, dev)
    if w_o.dim() != 2 or w_o.shape[1] != dims.n_heads * dims.v_head_dim:
        raise ValueError(f"w_o shape {tuple(w_o.shape)}")
    d_model = w_o.shape[0]
    if u is None:
        u = torch.empty((B, Sq, d_model), dtype=torch.bfloat16, device=dev)
    _need(u, "u", (torch.bfloat16,), (B, Sq, d_model), dev)
    ws_bytes = decode_output_workspace_size(dims, B, Sq, num_splits, d_model)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), None, dev)
    st = _lib.mla_decode_output(
        ctypes.byref(dims), B, Sq, _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
        _ptr(cache_pool), _ptr(cache_scale), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), num_splits, d_model, _ptr(w_o), _ptr(u), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(dev))
    _check(st, "mla_decode_output")
    return u, lse


def prefill(dims: Dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale, block_table, seq_lens,
            out=None, lse=None, workspace=None, stages: int = PREFILL_ALL, want_lse: bool = True):
    """Causal prefill attention in the decompressed form (mla_prefill[_stages]).
    Arguments and result as for ``decode``.  Returns (out, lse)."""
    act = _TORCH_OF[dims.act_dtype]
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    H, N, R = dims.n_heads, dims.qk_nope_dim, dims.qk_rope_dim
    dc, V = dims.kv_lora_rank, dims.v_head_dim
    dev = q_nope.device
    _need(q_nope, "q_nope", act, (B, Sq, H, N), dev)
    _need(q_pe, "q_pe", act, (B, Sq, H, R), dev)
    _need(w_uk, "w_uk", act, (H, N, dc), dev)
    _need(w_uv, "w_uv", act, (H, V, dc), dev)
    _need(cache_pool, "cache_pool", _TORCH_OF[dims.cache_dtype], None, dev)
    if cache_pool.dim() != 3 or cache_pool.shape[1:] != (dims.block_size, dc + R):
        raise ValueError(f"cache_pool shape {tuple(cache_pool.shape)}")
    if dims.cache_dtype == MLA_FP8_E4M3:
        _need(cache_scale, "cache_scale", (torch.float32,), cache_pool.shape[:2], dev)
    _need(block_table, "block_table", (torch.int32,), None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table shape {tuple(block_table.shape)}")
    _need(seq_lens, "seq_lens", (torch.int32,), (B,), dev)
    if out is None:
        out = torch.empty((B, Sq, H, V), dtype=act[0], device=dev)
    _need(out, "out", act, (B, Sq, H, V), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Sq, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (torch.float32,), (B, Sq, H), dev)
    ws_bytes = prefill_workspace_size(dims, B, Sq, block_table.shape[1])
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), None, dev)
    st = _lib.mla_prefill_stages(
        ctypes.byref(dims), B, Sq, _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
        _ptr(cache_pool), _ptr(cache_scale), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), stages,
        _stream(dev))
    _check(st, "mla_prefill_stages")
    return out, lse


def append(dims: Dims, h, w_kv_a, kv_norm_gamma, block_table, start_pos, cache_pool,
           cache_scale=None, rms_eps: float = 1e-6, rope_base: float = 10000.0, workspace=None):
    """Write the cache rows of h's new tokens (mla_cache_append).

    h [B, n_new, d] (act dtype); w_kv_a [d_c + R, d]; kv_norm_gamma [d_c];
    block_table [B, max_blocks] int32; start_pos [B] int32."""
    act = _TORCH_OF[dims.act_dtype]
    B, n_new, d = h.shape
    dc, R = dims.kv_lora_rank, dims.qk_rope_dim
    dev = h.device
    _need(h, "h", act, None, dev)
    _need(w_kv_a, "w_kv_a", act, (dc + R, d), dev)
    _need(kv_norm_gamma, "kv_norm_gamma", act, (dc,), dev)
    _need(block_table, "block_table", (torch.int32,), None, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table shape {tuple(block_table.shape)}")
    _need(start_pos, "start_pos", (torch.int32,), (B,), dev)
    _need(cache_pool, "cache_pool", _TORCH_OF[dims.cache_dtype], None, dev)
    if dims.cache_dtype == MLA_FP8_E4M3:
        _need(cache_scale, "cache_scale", (torch.float32,), cache_pool.shape[:2], dev)
    ws_bytes = append_workspace_size(dims, B, n_new, d)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), None, dev)
    st = _lib.mla_cache_append(
        ctypes.byref(dims), B, n_new, d, _ptr(h), _ptr(w_kv_a), _ptr(kv_norm_gamma),
        float(rms_eps), float(rope_base), _ptr(block_table), block_table.shape[1],
        _ptr(start_pos), _ptr(cache_pool), _ptr(cache_scale), _ptr(workspace),
        workspace.numel(), _stream(dev))
    _check(st, "mla_cache_append")



def step_workspace_size(dims: Dims, batch: int, q_len: int, d_model: int, num_splits: int = 0) -> int:
    n = _SZ(0)
    _check(_lib.mla_decode_step_workspace_size(ctypes.byref(dims), batch, q_len, d_model, num_splits,
                                               ctypes.byref(n)), "mla_decode_step_workspace_size")
    return n.value


def decode_step(dims: Dims, h, w_kv_a, kv_norm_gamma, start_pos, q_nope, q_pe, w_uk, w_uv,
                cache_pool, cache_scale, block_table, seq_lens, num_splits: int = 0,
                rms_eps: float = 1e-6, rope_base: float = 10000.0, out=None, lse=None,
                workspace=None, stages: int = STEP_ALL, want_lse: bool = True):
    """One decode step with its cache append (mla_decode_step[_stages]): the
    q_len new tokens h [B, q_len, d] are appended at start_pos, then their
    queries q_nope / q_pe attend over the cache (seq_lens = start_pos + q_len).
    Other arguments as append() and decode().  Returns (out, lse)."""
    act = _TORCH_OF[dims.act_dtype]
    B, Sq, dev, out, lse = _decode_tensors(dims, q_nope, q_pe, w_uk, w_uv, cache_pool, cache_scale,
                                           block_table, seq_lens, out, lse, want_lse)
    dc, R = dims.kv_lora_rank, dims.qk_rope_dim
    d = h.shape[-1]
    _need(h, "h", act, (B, Sq, d), dev)
    _need(w_kv_a, "w_kv_a", act, (dc + R, d), dev)
    _need(kv_norm_gamma, "kv_norm_gamma", act, (dc,), dev)
    _need(start_pos, "start_pos", (torch.int32,), (B,), dev)
    ws_bytes = step_workspace_size(dims, B, Sq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), None, dev)
    st = _lib.mla_decode_step_stages(
        ctypes.byref(dims), B, Sq, d, _ptr(h), _ptr(w_kv_a), _ptr(kv_norm_gamma), float(rms_eps),
        float(rope_base), _ptr(start_pos), _ptr(q_nope), _ptr(q_pe), _ptr(w_uk), _ptr(w_uv),
        _ptr(cache_pool), _ptr(cache_scale), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        num_splits, _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), stages, _stream(dev))
    _check(st, "mla_decode_step_stages")
    return out, lse


def query_project(dims: Dims, h, w_dq, q_norm_gamma, w_uq, w_qr, start_pos,
                  rms_eps: float = 1e-6, rope_base: float = 10000.0, q_nope=None, q_pe=None,
                  workspace=None):
    """The decode's query inputs from the layer input (mla_query_project).

    h [B, Sq, d] bf16; w_dq [d_q, d] bf16, or None for full-rank queries
    (d_q = 0); q_norm_gamma [d_q] bf16 or None; w_uq [H N, f], w_qr [H R, f]
    bf16 (f = d_q, or d); start_pos [B] int32.  Returns (q_nope [B, Sq, H, N],
    q_pe [B, Sq, H, R])."""
    B, Sq, d = h.shape
    H, N, R = dims.n_heads, dims.qk_nope_dim, dims.qk_rope_dim
    dq = 0 if w_dq is None else w_dq.shape[0]
    f = dq if dq else d
    dev = h.device
    bf = (torch.bfloat16,)
    _need(h, "h", bf, None, dev)
    if w_dq is not None:
        _need(w_dq, "w_dq", bf, (dq, d), dev)
    if q_norm_gamma is not None:
        _need(q_norm_gamma, "q_norm_gamma", bf, (dq,), dev)
    _need(w_uq, "w_uq", bf, (H * N, f), dev)
    _need(w_qr, "w_qr", bf, (H * R, f), dev)
    _need(start_pos, "start_pos", (torch.int32,), (B,), dev)
    if q_nope is None:
        q_nope = torch.empty((B, Sq, H, N), dtype=torch.bfloat16, device=dev)
    if q_pe is None:
        q_pe = torch.empty((B, Sq, H, R), dtype=torch.bfloat16, device=dev)
    _need(q_nope, "q_nope", bf, (B, Sq, H, N), dev)
    _need(q_pe, "q_pe", bf, (B, Sq, H, R), dev)
    ws_bytes = query_workspace_size(dims, B, Sq, d, dq)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", (torch.uint8,), None, dev)
    st = _lib.mla_query_project(
        ctypes.byref(dims), B, Sq, d, dq, _ptr(h), _ptr(w_dq), _ptr(q_norm_gamma), float(rms_eps),
        _ptr(w_uq), _ptr(w_qr), float(rope_base), _ptr(start_pos), _ptr(q_nope), _ptr(q_pe),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev))
    _check(st, "mla_query_project")
    return q_nope, q_pe


# ---- streaming-read probe (include/mla_probe.h; a separate library) -----------

PROBE_SINK_BYTES = 8192
_probe = None


def probe_read(buf, sink=None):
    """Enqueue libmla_probe's streaming read of every byte of the contiguous
    device tensor `buf` on torch's current stream; returns the sink tensor
    (allocated here when not given)."""
    global _probe
    if _probe is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_probe.so")
        if not os.path.exists(path):
            raise ImportError(f"libmla_probe.so not found at {path}; build it with "
                              "`python -m mla_latent_kv_06_amd.build`")
        lp = ctypes.CDLL(path)
        lp.mla_probe_read.restype = ctypes.c_int
        lp.mla_probe_read.argtypes = [_P, _SZ, _P, _P]
        _probe = lp
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("probe_read: buf must be a contiguous device tensor")
    if sink is None:
        sink = torch.empty(PROBE_SINK_BYTES, dtype=torch.uint8, device=buf.device)
    st = _probe.mla_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                               _stream(buf.device))
    if st != 0:
        raise RuntimeError(f"mla_probe_read failed with status {st}")
    return sink
