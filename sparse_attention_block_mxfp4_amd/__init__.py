"""Python binding of ``libmi_idx.so``, the MXFP4 lightning indexer for MI355X.

Argument marshalling only: every function here checks the tensors it is given
(device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream to the C ABI declared in ``include/mi_idx.h`` (same names),
and raises ``MiIdxError`` on a non-zero status.  All the work runs in the HIP
kernels of ``csrc/``.  There is no fallback: importing this package fails if
the library has not been built.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (one runtime per process, shared streams).
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MI_IDX_LIB selects another build of the same library (the sanitizer build
# of build.py --sanitize-check); by default the in-tree libmi_idx.so.
LIB_PATH = os.environ.get("MI_IDX_LIB") or os.path.join(_HERE, "libmi_idx.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python sparse_attention_block_mxfp4_amd/build.py` "
        "(or __graft_entry__.build()) with the ROCm toolchain")
lib = ctypes.CDLL(LIB_PATH)

_c = ctypes
_vp, _i32, _i64, _sz, _f32 = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_size_t, _c.c_float
_SIGS = {
    "mi_idx_version": (_c.c_char_p, []),
    "mi_idx_last_error": (_c.c_char_p, []),
    "mi_idx_unsupported_reason": (_c.c_char_p, [_i32, _i32, _i32, _i32, _i32, _c.c_char_p,
                                                _i32, _i32]),
    "mi_idx_insert_mxfp4": (_i32, [_vp, _i32, _i64, _vp, _i64, _vp, _i64, _vp]),
    "mi_idx_decode_plan_bytes": (_sz, [_i32]),
    "mi_idx_decode_plan_capacity": (_sz, [_i32, _i32, _i32, _i32]),
    "mi_idx_decode_noalloc": (_i32, [_vp, _i32, _vp, _i64, _vp, _i64, _vp, _i32, _i32, _i32,
                                     _i32, _f32, _vp, _vp, _vp]),
    "mi_idx_decode_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "mi_idx_plan_decode": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp, _sz, _vp]),
    "mi_idx_score_topk_decode": (_i32, [_vp, _i32, _vp, _i64, _vp, _i64, _vp, _i32, _i32, _i32,
                                        _i32, _f32, _vp, _sz, _vp, _sz, _vp, _vp, _vp]),
    "mi_idx_prefill_plan_bytes": (_sz, [_i32, _i64, _i32]),
    "mi_idx_prefill_workspace_bytes": (_sz, []),
    "mi_idx_plan_prefill": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp, _vp]),
    "mi_idx_score_topk_prefill": (_i32, [_vp, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32,
                                         _i64, _i32, _i32, _f32, _vp, _sz, _vp, _vp, _sz, _vp,
                                         _vp, _vp]),
    "mi_idx_select_forced": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp]),
    "mi_idx_score_local": (_i32, [_vp, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _i32,
                                  _i64, _i32, _i32, _f32, _vp, _vp]),
    "mi_idx_select_topk": (_i32, [_vp, _i64, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp]),
    "mi_idx_norm_rope_insert_mxfp4": (_i32, [_vp, _i32, _i64, _vp, _f32, _vp, _i32, _c.c_double,
                                             _i32, _vp, _i64, _vp, _i64, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

PAGE_TOKENS = 128
HEAD_DIM = 128
TOKEN_BYTES = 68
PAGE_BYTES = 8704
TOPK = 16
MAX_QUERY_LEN = 8
MAX_HEADS = 8
NOALLOC_SCRATCH_BYTES = 32 << 20

OK, EINVAL, EUNSUPPORTED, ECAPACITY, EHIP = 0, 1, 2, 3, 4


class MiIdxError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


def _check(status, name):
    if status != OK:
        raise MiIdxError(status, f"{name}: {lib.mi_idx_last_error().decode()} (status {status})")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtypes, cuda=True, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if cuda and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_U8 = (torch.uint8,)
_Q8 = (torch.uint8, torch.float8_e4m3fn)
_QALL = _Q8 + (torch.bfloat16,)
Q_E4M3, Q_BF16 = 0, 1


def _q_dtype(q):
    """The C ABI's index-Q dtype code of a query tensor."""
    return Q_BF16 if q.dtype == torch.bfloat16 else Q_E4M3
_I32 = (torch.int32,)


def mi_idx_version():
    return lib.mi_idx_version().decode()


def mi_idx_unsupported_reason(topk_blocks=16, init_blocks=0, local_blocks=1, block_size=128,
                              head_dim=128, score_type="max", num_heads=1, max_query_len=1):
    r = lib.mi_idx_unsupported_reason(topk_blocks, init_blocks, local_blocks, block_size,
                                      head_dim, score_type.encode(), num_heads, max_query_len)
    return None if r is None else r.decode()


def mi_idx_insert_mxfp4(k, slot_mapping, pages, stream=None):
    """Quantise K rows [n, >=128] (fp32 or bf16, unit stride in the last dim)
    to MXFP4 and write them to ``pages`` at ``slot_mapping`` [n] (int64)."""
    _need(k, "k", (torch.float32, torch.bfloat16), contiguous=False)
    if k.dim() != 2 or k.shape[1] < HEAD_DIM or k.stride(1) != 1:
        raise ValueError("k must be [n, >=128] with unit stride in the last dim")
    _need(slot_mapping, "slot_mapping", (torch.int64,))
    _need(pages, "pages", _U8)
    if slot_mapping.numel() != k.shape[0]:
        raise ValueError("slot_mapping must have one slot per row of k")
    num_blocks = pages.numel() // PAGE_BYTES
    st = lib.mi_idx_insert_mxfp4(_ptr(k), 0 if k.dtype == torch.float32 else 1, k.stride(0),
                                 _ptr(slot_mapping), k.shape[0], _ptr(pages), num_blocks,
                                 _stream(stream))
    _check(st, "mi_idx_insert_mxfp4")


ROPE_NEOX, ROPE_INTERLEAVED = 0, 1


def mi_idx_norm_rope_insert_mxfp4(k, slot_mapping, pages, norm_weight=None, norm_eps=1e-6,
                                  positions=None, rotary_dim=0, rope_base=10000.0,
                                  rope_style=ROPE_NEOX, stream=None):
    """As mi_idx_insert_mxfp4, with the rows first RMS-normalised (norm_weight
    [128] fp32, or None for no norm) and their first rotary_dim dims rotated
    at positions [n] int64."""
    _need(k, "k", (torch.float32, torch.bfloat16), contiguous=False)
    if k.dim() != 2 or k.shape[1] != HEAD_DIM or k.stride(1) != 1:
        raise ValueError("k must be [n, 128] with unit column stride")
    _need(slot_mapping, "slot_mapping", (torch.int64,))
    _need(pages, "pages", _U8)
    if slot_mapping.numel() != k.shape[0]:
        raise ValueError("slot_mapping must have one entry per row of k")
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", (torch.float32,))
        if norm_weight.numel() != HEAD_DIM:
            raise ValueError("norm_weight must have 128 entries")
    if rotary_dim:
        _need(positions, "positions", (torch.int64,))
        if positions.numel() != k.shape[0]:
            raise ValueError("positions must have one entry per row of k")
    st = lib.mi_idx_norm_rope_insert_mxfp4(
        _ptr(k), 0 if k.dtype == torch.float32 else 1, k.stride(0), _ptr(norm_weight),
        float(norm_eps), _ptr(positions) if rotary_dim else None, int(rotary_dim),
        float(rope_base), int(rope_style), _ptr(slot_mapping), k.shape[0], _ptr(pages),
        pages.numel() // PAGE_BYTES, _stream(stream))
    _check(st, "mi_idx_norm_rope_insert_mxfp4")


def mi_idx_decode_plan_bytes(max_reqs):
    return int(lib.mi_idx_decode_plan_bytes(max_reqs))


def mi_idx_decode_plan_capacity(max_reqs, max_pages, query_len, num_heads):
    """Work items (rows of four int32) of a decode plan for max_reqs requests."""
    return int(lib.mi_idx_decode_plan_capacity(max_reqs, max_pages, query_len, num_heads))


def mi_idx_decode_workspace_bytes(max_reqs, query_len, num_heads):
    return int(lib.mi_idx_decode_workspace_bytes(max_reqs, query_len, num_heads))


def mi_idx_plan_decode(seq_lens, query_len, num_heads, max_pages, plan, workspace,
                       stream=None):
    _need(seq_lens, "seq_lens", _I32)
    _need(plan, "plan", _U8)
    _need(workspace, "workspace", _U8)
    st = lib.mi_idx_plan_decode(_ptr(seq_lens), seq_lens.numel(), query_len, num_heads,
                                max_pages, _ptr(plan), plan.numel(), _ptr(workspace),
                                workspace.numel(), _stream(stream))
    _check(st, "mi_idx_plan_decode")


def mi_idx_score_topk_decode(q, pages, block_table, seq_lens, query_len, max_pages, plan,
                             workspace, topk_out, scale=1.0, scores_out=None, stream=None):
    """q [R*query_len, H, 128] E4M3 (uint8 or float8_e4m3fn) or bfloat16;
    topk_out [R*query_len, H, 16] int32; block_table [R, >=max_pages] int32
    (row stride taken from the tensor)."""
    R, H = _decode_args(q, pages, block_table, seq_lens, query_len, max_pages, topk_out,
                        scores_out)
    _need(plan, "plan", _U8)
    _need(workspace, "workspace", _U8)
    st = lib.mi_idx_score_topk_decode(
        _ptr(q), _q_dtype(q), _ptr(pages), pages.numel() // PAGE_BYTES, _ptr(block_table),
        block_table.stride(0), _ptr(seq_lens), R, query_len, H, max_pages, float(scale),
        _ptr(plan), plan.numel(), _ptr(workspace), workspace.numel(), _ptr(topk_out),
        _ptr(scores_out), _stream(stream))
    _check(st, "mi_idx_score_topk_decode")


def _decode_args(q, pages, block_table, seq_lens, query_len, max_pages, topk_out, scores_out):
    _need(q, "q", _QALL)
    _need(pages, "pages", _U8)
    _need(block_table, "block_table", _I32, contiguous=False)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be 2-D with unit column stride")
    _need(seq_lens, "seq_lens", _I32)
    _need(topk_out, "topk_out", _I32)
    R = seq_lens.numel()
    H = q.shape[1] if q.dim() == 3 else 0
    if q.dim() != 3 or q.shape[0] != R * query_len or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [{R}*{query_len}, H, 128], got {tuple(q.shape)}")
    if tuple(topk_out.shape) != (R * query_len, H, TOPK):
        raise ValueError(f"topk_out must be [{R * query_len}, {H}, 16]")
    if block_table.shape[0] < R:
        raise ValueError("block_table has fewer rows than seq_lens")
    if scores_out is not None:
        _need(scores_out, "scores_out", (torch.float32,))
        if tuple(scores_out.shape) != (R * query_len, H, max_pages):
            raise ValueError("scores_out must be [rows, H, max_pages]")
    return R, H


def mi_idx_decode_noalloc(q, pages, block_table, seq_lens, query_len, max_pages, topk_out,
                          scale=1.0, scores_out=None, stream=None):
    """Plan + score + merge of the decode rows with the library's static
    device scratch (no plan or workspace, nothing allocated); the same
    arguments and result as mi_idx_plan_decode + mi_idx_score_topk_decode.
    Calls that overlap on one GPU race."""
    R, H = _decode_args(q, pages, block_table, seq_lens, query_len, max_pages, topk_out,
                        scores_out)
    st = lib.mi_idx_decode_noalloc(
        _ptr(q), _q_dtype(q), _ptr(pages), pages.numel() // PAGE_BYTES, _ptr(block_table),
        block_table.stride(0), _ptr(seq_lens), R, query_len, H, max_pages, float(scale),
        _ptr(topk_out), _ptr(scores_out), _stream(stream))
    _check(st, "mi_idx_decode_noalloc")


def mi_idx_prefill_plan_bytes(num_reqs, total_q, num_heads):
    return int(lib.mi_idx_prefill_plan_bytes(num_reqs, total_q, num_heads))


class PrefillLaunch(ctypes.Structure):
    """mi_idx_prefill_launch: the launch shape of a prefill plan."""
    _fields_ = [("num_lists", ctypes.c_int32), ("num_pieces", ctypes.c_int32),
                ("num_merges", ctypes.c_int32), ("num_chunks", ctypes.c_int32)]


def mi_idx_prefill_workspace_bytes():
    return int(lib.mi_idx_prefill_workspace_bytes())


def mi_idx_plan_prefill(cu_seqlens_q_host, seq_lens_host, num_heads, gather_budget_pages,
                        staging, plan, stream=None):
    """Host plan of the prefill work lists; one async copy of ``staging``
    (pinned host uint8 tensor) into ``plan`` (device uint8 tensor).  Returns
    the plan's PrefillLaunch (work lists, pieces, split tiles, chunks)."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_q_host, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    if cu.ndim != 1 or sl.ndim != 1 or cu.size != sl.size + 1:
        raise ValueError("cu_seqlens_q must have one more entry than seq_lens")
    _need(staging, "staging", _U8, cuda=False)
    if not staging.is_pinned():
        raise ValueError("staging must be pinned host memory")
    _need(plan, "plan", _U8)
    if staging.numel() < plan.numel():
        raise ValueError("staging must be at least as large as plan")
    launch = PrefillLaunch()
    st = lib.mi_idx_plan_prefill(cu.ctypes.data, sl.ctypes.data, sl.size, num_heads,
                                 int(gather_budget_pages), _ptr(staging), _ptr(plan),
                                 plan.numel(), ctypes.byref(launch), _stream(stream))
    _check(st, "mi_idx_plan_prefill")
    return launch


def mi_idx_score_topk_prefill(q, pages, block_table, cu_seqlens_q, seq_lens, context_lens,
                              max_pages, plan, launch, workspace, topk_out, scale=1.0,
                              scores_out=None, stream=None):
    """q [total_q, H, 128] E4M3 or bfloat16; topk_out [total_q, H, 16] int32
    (may be a row slice of a larger contiguous buffer); launch: the
    PrefillLaunch of the plan; workspace: device uint8 tensor of
    mi_idx_prefill_workspace_bytes() (None when launch.num_merges is 0)."""
    _need(q, "q", _QALL)
    _need(pages, "pages", _U8)
    _need(block_table, "block_table", _I32, contiguous=False)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be 2-D with unit column stride")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seq_lens", seq_lens),
                    ("context_lens", context_lens)):
        _need(t, name, _I32)
    _need(topk_out, "topk_out", _I32)
    R = seq_lens.numel()
    if cu_seqlens_q.numel() != R + 1 or context_lens.numel() != R or block_table.shape[0] < R:
        raise ValueError("cu_seqlens_q / context_lens / block_table do not match seq_lens")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [total_q, H, 128]")
    T, H = q.shape[0], q.shape[1]
    if tuple(topk_out.shape) != (T, H, TOPK):
        raise ValueError(f"topk_out must be [{T}, {H}, 16]")
    if scores_out is not None:
        _need(scores_out, "scores_out", (torch.float32,))
        if tuple(scores_out.shape) != (T, H, max_pages):
            raise ValueError("scores_out must be [total_q, H, max_pages]")
    if workspace is not None:
        _need(workspace, "workspace", _U8)
    st = lib.mi_idx_score_topk_prefill(
        _ptr(q), _q_dtype(q), _ptr(pages), pages.numel() // PAGE_BYTES, _ptr(block_table),
        block_table.stride(0), _ptr(cu_seqlens_q), _ptr(seq_lens), _ptr(context_lens), R, T, H,
        max_pages, float(scale), _ptr(plan), plan.numel(), ctypes.byref(launch),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _ptr(topk_out),
        _ptr(scores_out), _stream(stream))
    _check(st, "mi_idx_score_topk_prefill")


def mi_idx_select_forced(ranked, topk, init_blocks, local_blocks, max_k_tiles, out=None,
                         stream=None):
    """ranked [..., 16] int32 rows as the score calls write them; returns out
    [..., topk] int32 (allocated when not given): the forced windows, the best
    pages between them, ascending, -1 tail."""
    _need(ranked, "ranked", _I32)
    if ranked.dim() < 1 or ranked.shape[-1] != TOPK:
        raise ValueError("ranked must be [..., 16]")
    shape = tuple(ranked.shape[:-1]) + (int(topk),)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=ranked.device)
    _need(out, "out", _I32)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must be {list(shape)}")
    n = ranked.numel() // TOPK
    st = lib.mi_idx_select_forced(_ptr(ranked), n, int(topk), int(init_blocks),
                                  int(local_blocks), int(max_k_tiles), _ptr(out), _stream(stream))
    _check(st, "mi_idx_select_forced")
    return out


MAX_TOPK = 1024


def mi_idx_score_local(q, pages, block_table, max_pages, local_out=None, seq_lens=None,
                       query_len=None, cu_seqlens_q=None, context_lens=None, scale=1.0,
                       stream=None):
    """Causal score of each row's own page ([rows, H] fp32, NaN where a row
    has none): decode rows from seq_lens and query_len, or prefill rows from
    cu_seqlens_q and context_lens (device int32 tensors)."""
    _need(q, "q", _QALL)
    _need(pages, "pages", _U8)
    _need(block_table, "block_table", _I32, contiguous=False)
    if block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be 2-D with unit column stride")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [rows, H, 128]")
    T, H = q.shape[0], q.shape[1]
    if cu_seqlens_q is None:
        _need(seq_lens, "seq_lens", _I32)
        R = seq_lens.numel()
        ql = int(query_len)
        if T != R * ql:
            raise ValueError("decode q must have num_reqs * query_len rows")
    else:
        _need(cu_seqlens_q, "cu_seqlens_q", _I32)
        _need(context_lens, "context_lens", _I32)
        R = context_lens.numel()
        ql = 0
        if cu_seqlens_q.numel() != R + 1:
            raise ValueError("cu_seqlens_q must have num_reqs + 1 entries")
    if local_out is None:
        local_out = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _need(local_out, "local_out", (torch.float32,))
    if tuple(local_out.shape) != (T, H):
        raise ValueError(f"local_out must be [{T}, {H}]")
    st = lib.mi_idx_score_local(_ptr(q), _q_dtype(q), _ptr(pages), pages.numel() // PAGE_BYTES,
                                _ptr(block_table), block_table.stride(0), _ptr(seq_lens),
                                _ptr(cu_seqlens_q), _ptr(context_lens), R, ql, T, H,
                                int(max_pages), float(scale), _ptr(local_out), _stream(stream))
    _check(st, "mi_idx_score_local")
    return local_out


def mi_idx_select_topk(ranked, scores, topk, init_blocks, local_blocks, max_k_tiles,
                       local_scores=None, out=None, stream=None):
    """General selection: ranked [..., 16] and scores [..., W] (a score call's
    outputs), local_scores [...] (mi_idx_score_local) when the local page can
    compete; returns out [..., topk] int32."""
    _need(ranked, "ranked", _I32)
    _need(scores, "scores", (torch.float32,))
    if ranked.shape[-1] != TOPK or tuple(scores.shape[:-1]) != tuple(ranked.shape[:-1]):
        raise ValueError("ranked must be [..., 16] and scores [..., W] over the same rows")
    n = ranked.numel() // TOPK
    if local_scores is not None:
        _need(local_scores, "local_scores", (torch.float32,))
        if local_scores.numel() != n:
            raise ValueError("local_scores must hold one score per (row, head)")
    shape = tuple(ranked.shape[:-1]) + (int(topk),)
    if out is None:
        out = torch.empty(shape, dtype=torch.int32, device=ranked.device)
    _need(out, "out", _I32)
    if tuple(out.shape) != shape:
        raise ValueError(f"out must be {list(shape)}")
    st = lib.mi_idx_select_topk(_ptr(scores), scores.shape[-1], _ptr(local_scores), _ptr(ranked),
                                n, int(topk), int(init_blocks), int(local_blocks),
                                int(max_k_tiles), _ptr(out), _stream(stream))
    _check(st, "mi_idx_select_topk")
    return out


__all__ = [n for n in dir() if n.startswith("mi_idx_")] + ["MiIdxError", "lib", "LIB_PATH"]
