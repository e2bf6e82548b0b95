"""Python binding of libmsa, the MI355X MiniMax Sparse Attention hot path.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/msa.h. torch supplies device
memory (inputs, outputs, workspace) and the current stream. There is no CPU or
eager fallback: if libmsa.so is missing the import of the library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsa.so")

MSA_OK = 0
_STATUS = {0: "MSA_OK", -1: "MSA_ERR_INVALID_ARG", -2: "MSA_ERR_UNSUPPORTED",
           -3: "MSA_ERR_WORKSPACE_TOO_SMALL", -4: "MSA_ERR_HIP"}

EXPORTED = ("msa_prefill_workspace_bytes", "msa_prefill", "msa_prefill_varlen_workspace_bytes",
            "msa_prefill_varlen", "msa_decode_workspace_bytes", "msa_decode", "msa_prefill_profiled",
            "msa_decode_profiled", "msa_index_kl_workspace_bytes", "msa_index_kl_backward", "msa_index_scores",
            "msa_select_blocks", "msa_status_string", "msa_index_project_workspace_bytes", "msa_index_project",
            "msa_index_project_decode", "msa_decode_noalloc", "msa_prefill_schedule_layout",
            "msa_prefill_timed", "msa_decode_timed", "msa_stage_timer_read")
PREFILL_STAGES = ("index_score", "select", "reverse_index", "kv_outer_attn", "dense_attn_merge")
DECODE_STAGES = ("index_score", "select_attn")


class MsaParams(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


_SCHED_OFFSETS = ("tile_info", "chunk_off", "entries", "tiles", "tile_visits", "wg_trace", "dense_cnt",
                  "dense_list", "dense_qmask", "dense_slots")


class MsaScheduleMap(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in _SCHED_OFFSETS] + [
        ("dense_max", ctypes.c_int32), ("tile_queries", ctypes.c_int32), ("claim", ctypes.c_int32),
        ("dense_min", ctypes.c_int32), ("wall_clock_khz", ctypes.c_int64)]


class MsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_STATUS.get(status, status)}")
        self.status = status


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmsa.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} not found: build it with `python -m block_sparse_long_07_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    P = ctypes.POINTER(MsaParams)
    lib.msa_prefill_workspace_bytes.argtypes = [P, i32, i64]
    lib.msa_prefill_workspace_bytes.restype = sz
    lib.msa_prefill.argtypes = [P, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_prefill.restype = ctypes.c_int
    lib.msa_prefill_varlen_workspace_bytes.argtypes = [P, i64, i64]
    lib.msa_prefill_varlen_workspace_bytes.restype = sz
    lib.msa_prefill_varlen.argtypes = [P, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_prefill_varlen.restype = ctypes.c_int
    lib.msa_decode_workspace_bytes.argtypes = [P, i32, i64]
    lib.msa_decode_workspace_bytes.restype = sz
    lib.msa_decode.argtypes = [P, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_decode.restype = ctypes.c_int
    lib.msa_decode_noalloc.argtypes = [P, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.msa_decode_noalloc.restype = ctypes.c_int
    fp = ctypes.POINTER(ctypes.c_float)
    lib.msa_prefill_profiled.argtypes = [P, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, fp]
    lib.msa_prefill_profiled.restype = ctypes.c_int
    lib.msa_decode_profiled.argtypes = [P, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, fp]
    lib.msa_decode_profiled.restype = ctypes.c_int
    lib.msa_index_kl_workspace_bytes.argtypes = [P, i64]
    lib.msa_index_kl_workspace_bytes.restype = sz
    lib.msa_index_kl_backward.argtypes = [P, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_index_kl_backward.restype = ctypes.c_int
    lib.msa_index_scores.argtypes = [P, i64, vp, vp, vp, vp]
    lib.msa_index_scores.restype = ctypes.c_int
    lib.msa_select_blocks.argtypes = [P, i64, vp, vp, vp]
    lib.msa_select_blocks.restype = ctypes.c_int
    lib.msa_index_project_workspace_bytes.argtypes = [P, i64, i32]
    lib.msa_index_project_workspace_bytes.restype = sz
    lib.msa_index_project.argtypes = [P, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_index_project.restype = ctypes.c_int
    lib.msa_index_project_decode.argtypes = [P, i32, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.msa_index_project_decode.restype = ctypes.c_int
    vpp = ctypes.POINTER(ctypes.c_void_p)
    lib.msa_prefill_timed.argtypes = [P, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vpp]
    lib.msa_prefill_timed.restype = ctypes.c_int
    lib.msa_decode_timed.argtypes = [P, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vpp]
    lib.msa_decode_timed.restype = ctypes.c_int
    lib.msa_stage_timer_read.argtypes = [vp, ctypes.POINTER(ctypes.c_float)]
    lib.msa_stage_timer_read.restype = ctypes.c_int
    lib.msa_prefill_schedule_layout.argtypes = [P, i64, i64, ctypes.POINTER(MsaScheduleMap)]
    lib.msa_prefill_schedule_layout.restype = ctypes.c_int
    lib.msa_status_string.argtypes = [ctypes.c_int]
    lib.msa_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def params(num_q_heads=64, num_kv_heads=4, head_dim=128, index_dim=64, block_size=128, topk=16,
           softmax_scale: Optional[float] = None) -> MsaParams:
    return MsaParams(num_q_heads, num_kv_heads, head_dim, index_dim, block_size, topk,
                     float(softmax_scale) if softmax_scale else 0.0)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int, what: str):
    if status != MSA_OK:
        raise MsaError(status, what)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def prefill_workspace_bytes(p: MsaParams, batch: int, seq_len: int) -> int:
    return int(load().msa_prefill_workspace_bytes(ctypes.byref(p), batch, seq_len))


def prefill(q, k, v, q_idx, k_idx, *, topk=16, block_size=128, softmax_scale=None,
            want_sel=False, want_lse=False, workspace: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, stage_ms: Optional[list] = None,
            stage_timers: Optional[list] = None):
    """Causal MSA prefill. q [B,N,Hq,d], k/v [B,N,G,d], q_idx [B,N,G,d_idx],
    k_idx [B,N,d_idx], all bf16 on one device. Returns (out, sel or None, lse or None).
    With stage_timers (a list) the timed entry point runs without synchronising
    and a handle is appended; read_stage_timers() later gives the per-stage
    milliseconds. With stage_ms (a list) the profiled entry point runs, synchronises, and the
    per-stage milliseconds (PREFILL_STAGES order) are appended to it."""
    lib = load()
    B, N, Hq, d = q.shape
    G = k.shape[2]
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (q_idx, "q_idx"), (k_idx, "k_idx")):
        _need(t, torch.bfloat16, name)
    p = params(Hq, G, d, q_idx.shape[-1], block_size, topk, softmax_scale)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    sel = torch.empty((B, G, N, topk), dtype=torch.int32, device=dev) if want_sel else None
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev) if want_lse else None
    nbytes = int(lib.msa_prefill_workspace_bytes(ctypes.byref(p), B, N))
    if nbytes == 0:
        raise MsaError(-2, "msa_prefill_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    args = (ctypes.byref(p), B, N, _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx),
            _ptr(out), _ptr(sel), _ptr(lse), _ptr(workspace), nbytes, _stream(dev))
    if stage_timers is not None:
        h = ctypes.c_void_p()
        _check(lib.msa_prefill_timed(*args, ctypes.byref(h)), "msa_prefill_timed")
        stage_timers.append((h, len(PREFILL_STAGES)))
    elif stage_ms is None:
        _check(lib.msa_prefill(*args), "msa_prefill")
    else:
        ms = (ctypes.c_float * len(PREFILL_STAGES))()
        _check(lib.msa_prefill_profiled(*args, ms), "msa_prefill_profiled")
        stage_ms.extend(float(x) for x in ms)
    return out, sel, lse


def prefill_schedule_layout(p: MsaParams, max_q_len: int, max_ctx: int) -> MsaScheduleMap:
    """Where a prefill workspace keeps the KV-outer schedule of its last window."""
    m = MsaScheduleMap()
    _check(load().msa_prefill_schedule_layout(ctypes.byref(p), max_q_len, max_ctx, ctypes.byref(m)),
           "msa_prefill_schedule_layout")
    return m


def read_prefill_schedule(workspace: torch.Tensor, m: MsaScheduleMap, num_kv_heads: int) -> dict:
    """Copies the schedule of the last window a completed prefill left in
    `workspace` (laid out as `m` says) to host tensors: tile_info, chunk_off,
    entries, tiles [T,4], tile_visits [T], wg_trace [workgroups,4],
    dense_cnt [G,units], dense_list / dense_qmask [G,units,dense_max],
    dense_slots [G,rows]."""
    def part(name, count, dtype=torch.int32):
        off = getattr(m, name)
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return workspace[off:off + nbytes].view(dtype).cpu()

    info = part("tile_info", 16)
    T, lists, nch, nwg, n = (int(info[i]) for i in (0, 2, 3, 4, 5))
    G, units = num_kv_heads, (n + 15) // 16
    chunk_off = part("chunk_off", lists * nch + 1)
    return dict(
        tile_info=info, chunk_off=chunk_off, entries=part("entries", int(chunk_off[-1])),
        tiles=part("tiles", 4 * T).view(T, 4), tile_visits=part("tile_visits", T),
        wg_trace=part("wg_trace", 4 * nwg, torch.int64).view(nwg, 4),
        dense_cnt=part("dense_cnt", G * units).view(G, units),
        dense_list=part("dense_list", G * units * m.dense_max).view(G, units, m.dense_max),
        dense_qmask=part("dense_qmask", G * units * m.dense_max).view(G, units, m.dense_max),
        dense_slots=part("dense_slots", G * n).view(G, n))


def prefill_varlen_workspace_bytes(p: MsaParams, max_q_len: int, max_ctx: int) -> int:
    return int(load().msa_prefill_varlen_workspace_bytes(ctypes.byref(p), max_q_len, max_ctx))


def prefill_varlen(q, q_idx, k_cache, v_cache, k_idx_cache, q_start, q_len, *, topk=16,
                   block_size=128, softmax_scale=None, want_sel=False, want_lse=False,
                   workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """Variable-length / chunked prefill against per-sequence caches.
    q [T,Hq,d] and q_idx [T,G,d_idx] hold the sequences' query rows packed in
    order; sequence b's rows are positions q_start[b] .. q_start[b]+q_len[b]-1
    (q_start, q_len: host sequences of ints). k_cache/v_cache [B,max_ctx,G,d],
    k_idx_cache [B,max_ctx,d_idx] already hold those positions. Returns
    (out [T,Hq,d], sel [G,T,topk] or None, lse [T,Hq] or None)."""
    lib = load()
    T, Hq, d = q.shape
    B, max_ctx, G = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    for t, name in ((q, "q"), (q_idx, "q_idx"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                    (k_idx_cache, "k_idx_cache")):
        _need(t, torch.bfloat16, name)
    starts = [int(x) for x in q_start]
    lens = [int(x) for x in q_len]
    if len(starts) != B or len(lens) != B:
        raise ValueError("q_start and q_len need one entry per cache sequence")
    if sum(lens) != T:
        raise ValueError(f"q has {T} rows but q_len sums to {sum(lens)}")
    p = params(Hq, G, d, q_idx.shape[-1], block_size, topk, softmax_scale)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    sel = torch.empty((G, T, topk), dtype=torch.int32, device=dev) if want_sel else None
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev) if want_lse else None
    if T == 0:
        return out, sel, lse
    nbytes = int(lib.msa_prefill_varlen_workspace_bytes(ctypes.byref(p), max(lens), max_ctx))
    if nbytes == 0:
        raise MsaError(-2, "msa_prefill_varlen_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    c_start = (ctypes.c_int64 * B)(*starts)
    c_len = (ctypes.c_int64 * B)(*lens)
    _check(lib.msa_prefill_varlen(ctypes.byref(p), B, max_ctx, c_start, c_len, _ptr(q), _ptr(q_idx),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(k_idx_cache), _ptr(out),
                                  _ptr(sel), _ptr(lse), _ptr(workspace), nbytes, _stream(dev)),
           "msa_prefill_varlen")
    return out, sel, lse


def decode_workspace_bytes(p: MsaParams, batch: int, max_ctx: int) -> int:
    return int(load().msa_decode_workspace_bytes(ctypes.byref(p), batch, max_ctx))


def decode(q, q_idx, k_cache, v_cache, k_idx_cache, ctx_lens, *, topk=16, block_size=128,
           softmax_scale=None, want_sel=False, want_lse=False,
           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
           stage_ms: Optional[list] = None, stage_timers: Optional[list] = None):
    """One decode step. q [B,Hq,d], q_idx [B,G,d_idx], k_cache/v_cache
    [B,max_ctx,G,d], k_idx_cache [B,max_ctx,d_idx] (bf16), ctx_lens int32 [B]
    on the device (the new token is row ctx_lens[b]-1). Returns (out, sel, lse)."""
    lib = load()
    B, Hq, d = q.shape
    max_ctx, G = k_cache.shape[1], k_cache.shape[2]
    for t, name in ((q, "q"), (q_idx, "q_idx"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                    (k_idx_cache, "k_idx_cache")):
        _need(t, torch.bfloat16, name)
    _need(ctx_lens, torch.int32, "ctx_lens")
    p = params(Hq, G, d, q_idx.shape[-1], block_size, topk, softmax_scale)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    sel = torch.empty((B, G, topk), dtype=torch.int32, device=dev) if want_sel else None
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if want_lse else None
    nbytes = int(lib.msa_decode_workspace_bytes(ctypes.byref(p), B, max_ctx))
    if nbytes == 0:
        raise MsaError(-1, "msa_decode_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    args = (ctypes.byref(p), B, max_ctx, _ptr(q), _ptr(q_idx), _ptr(k_cache), _ptr(v_cache),
            _ptr(k_idx_cache), _ptr(ctx_lens), _ptr(out), _ptr(sel), _ptr(lse),
            _ptr(workspace), nbytes, _stream(dev))
    if stage_timers is not None:
        h = ctypes.c_void_p()
        _check(lib.msa_decode_timed(*args, ctypes.byref(h)), "msa_decode_timed")
        stage_timers.append((h, len(DECODE_STAGES)))
    elif stage_ms is None:
        _check(lib.msa_decode(*args), "msa_decode")
    else:
        ms = (ctypes.c_float * len(DECODE_STAGES))()
        _check(lib.msa_decode_profiled(*args, ms), "msa_decode_profiled")
        stage_ms.extend(float(x) for x in ms)
    return out, sel, lse


def read_stage_timers(timers: list) -> list:
    """Per-stage milliseconds of each handle that prefill/decode appended to
    `timers` (waits for each call's last event; every handle is released)."""
    lib = load()
    res = []
    for h, n in timers:
        ms = (ctypes.c_float * n)()
        _check(lib.msa_stage_timer_read(h, ms), "msa_stage_timer_read")
        res.append([float(x) for x in ms])
    timers.clear()
    return res


def decode_noalloc(q, q_idx, k_cache, v_cache, k_idx_cache, ctx_lens, *, topk=16, block_size=128,
                   softmax_scale=None, want_sel=False, want_lse=False, out: Optional[torch.Tensor] = None):
    """msa_decode_noalloc: one decode step with the library's own fixed device
    workspace (no workspace argument; the library allocates nothing). Same
    arguments and results as decode()."""
    lib = load()
    B, Hq, d = q.shape
    max_ctx, G = k_cache.shape[1], k_cache.shape[2]
    for t, name in ((q, "q"), (q_idx, "q_idx"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                    (k_idx_cache, "k_idx_cache")):
        _need(t, torch.bfloat16, name)
    _need(ctx_lens, torch.int32, "ctx_lens")
    p = params(Hq, G, d, q_idx.shape[-1], block_size, topk, softmax_scale)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    sel = torch.empty((B, G, topk), dtype=torch.int32, device=dev) if want_sel else None
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if want_lse else None
    _check(lib.msa_decode_noalloc(ctypes.byref(p), B, max_ctx, _ptr(q), _ptr(q_idx), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(k_idx_cache), _ptr(ctx_lens), _ptr(out), _ptr(sel), _ptr(lse),
                                  _stream(dev)), "msa_decode_noalloc")
    return out, sel, lse


def index_kl_workspace_bytes(p: MsaParams, seq_len: int) -> int:
    return int(load().msa_index_kl_workspace_bytes(ctypes.byref(p), seq_len))


def index_kl_backward(q, k, q_idx, k_idx, sel, lse, *, topk=16, block_size=128, softmax_scale=None,
                      workspace: Optional[torch.Tensor] = None):
    """KL alignment of the Index Branch to the Main Branch for one sequence:
    q [N,Hq,d], k [N,G,d], q_idx [N,G,d_idx], k_idx [N,d_idx] (bf16), sel
    int32 [G,N,topk] and lse fp32 [N,Hq] as returned by prefill (batch entry).
    Returns (loss fp32 [G,N], dq_idx fp32 [N,G,d_idx], dk_idx fp32 [N,d_idx]):
    the per-(group, row) divergences and the gradients of their sum."""
    lib = load()
    N, Hq, d = q.shape
    G = k.shape[1]
    for t, name in ((q, "q"), (k, "k"), (q_idx, "q_idx"), (k_idx, "k_idx")):
        _need(t, torch.bfloat16, name)
    _need(sel, torch.int32, "sel")
    _need(lse, torch.float32, "lse")
    p = params(Hq, G, d, q_idx.shape[-1], block_size, topk, softmax_scale)
    dev = q.device
    loss = torch.empty((G, N), dtype=torch.float32, device=dev)
    dq = torch.empty((N, G, q_idx.shape[-1]), dtype=torch.float32, device=dev)
    dk = torch.empty((N, k_idx.shape[-1]), dtype=torch.float32, device=dev)
    nbytes = int(lib.msa_index_kl_workspace_bytes(ctypes.byref(p), N))
    if nbytes == 0:
        raise MsaError(-2, "msa_index_kl_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib.msa_index_kl_backward(ctypes.byref(p), N, _ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(sel),
                                     _ptr(lse), _ptr(loss), _ptr(dq), _ptr(dk), _ptr(workspace), nbytes,
                                     _stream(dev)), "msa_index_kl_backward")
    return loss, dq, dk


def index_project_workspace_bytes(p: MsaParams, n_tokens: int, d_model: int) -> int:
    return int(load().msa_index_project_workspace_bytes(ctypes.byref(p), n_tokens, d_model))


def _project_args(x, w_qi, w_ki):
    for t, name in ((x, "x"), (w_qi, "w_qi"), (w_ki, "w_ki")):
        _need(t, torch.bfloat16, name)
    n, dm = x.shape
    G, di, dm2 = w_qi.shape
    if dm2 != dm or tuple(w_ki.shape) != (di, dm):
        raise ValueError(f"weights {tuple(w_qi.shape)} / {tuple(w_ki.shape)} do not match x {tuple(x.shape)}")
    return n, dm, G, di, params(16 * G, G, 128, di)


def _project_workspace(lib, p, n, dm, workspace, dev, what):
    nbytes = int(lib.msa_index_project_workspace_bytes(ctypes.byref(p), n, dm))
    if nbytes == 0:
        raise MsaError(-2, what)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    return workspace, nbytes


def index_project(x, w_qi, w_ki, *, q_idx=None, k_idx=None, workspace: Optional[torch.Tensor] = None):
    """Index Branch projections of hidden states x [n, d_model] (bf16):
    q_idx [n, G, d_idx] = x W_qi[g]^T per group, k_idx [n, d_idx] = x W_ki^T,
    with w_qi [G, d_idx, d_model] and w_ki [d_idx, d_model]. k_idx may be a
    contiguous slice of a cache (the chunk's rows); both are written."""
    lib = load()
    n, dm, G, di, p = _project_args(x, w_qi, w_ki)
    dev = x.device
    if q_idx is None:
        q_idx = torch.empty((n, G, di), dtype=torch.bfloat16, device=dev)
    if k_idx is None:
        k_idx = torch.empty((n, di), dtype=torch.bfloat16, device=dev)
    _need(q_idx, torch.bfloat16, "q_idx")
    _need(k_idx, torch.bfloat16, "k_idx")
    workspace, nbytes = _project_workspace(lib, p, n, dm, workspace, dev, "msa_index_project_workspace_bytes")
    _check(lib.msa_index_project(ctypes.byref(p), n, dm, _ptr(x), _ptr(w_qi), _ptr(w_ki), _ptr(q_idx), _ptr(k_idx),
                                 _ptr(workspace), nbytes, _stream(dev)), "msa_index_project")
    return q_idx, k_idx


def index_project_decode(x, w_qi, w_ki, k_idx_cache, ctx_lens, *, q_idx=None,
                         workspace: Optional[torch.Tensor] = None):
    """Decode-step projections: x [B, d_model] -> q_idx [B, G, d_idx]
    (returned), and the key head appended in place at row ctx_lens[b]-1 of
    k_idx_cache [B, max_ctx, d_idx]."""
    lib = load()
    B, dm, G, di, p = _project_args(x, w_qi, w_ki)
    dev = x.device
    _need(k_idx_cache, torch.bfloat16, "k_idx_cache")
    _need(ctx_lens, torch.int32, "ctx_lens")
    if k_idx_cache.dim() != 3 or k_idx_cache.shape[0] != B or k_idx_cache.shape[2] != di or ctx_lens.numel() != B:
        raise ValueError("k_idx_cache must be [B, max_ctx, d_idx] and ctx_lens [B]")
    if q_idx is None:
        q_idx = torch.empty((B, G, di), dtype=torch.bfloat16, device=dev)
    _need(q_idx, torch.bfloat16, "q_idx")
    workspace, nbytes = _project_workspace(lib, p, B, dm, workspace, dev, "msa_index_project_workspace_bytes")
    _check(lib.msa_index_project_decode(ctypes.byref(p), B, k_idx_cache.shape[1], dm, _ptr(x), _ptr(w_qi),
                                        _ptr(w_ki), _ptr(ctx_lens), _ptr(q_idx), _ptr(k_idx_cache),
                                        _ptr(workspace), nbytes, _stream(dev)), "msa_index_project_decode")
    return q_idx


def index_scores(q_idx, k_idx, *, num_q_heads=None, topk=16, block_size=128, scores=None):
    """Pooled index scores of one sequence: q_idx [N,G,d_idx], k_idx [N,d_idx]
    -> scores fp32 [N,G,nb] (defined for rows whose own block is >= topk, b < own block)."""
    lib = load()
    N, G, di = q_idx.shape
    _need(q_idx, torch.bfloat16, "q_idx")
    _need(k_idx, torch.bfloat16, "k_idx")
    nb = (N + block_size - 1) // block_size
    p = params(num_q_heads or 16 * G, G, 128, di, block_size, topk)
    if scores is None:
        scores = torch.full((N, G, nb), float("nan"), dtype=torch.float32, device=q_idx.device)
    _check(lib.msa_index_scores(ctypes.byref(p), N, _ptr(q_idx), _ptr(k_idx), _ptr(scores),
                                _stream(q_idx.device)), "msa_index_scores")
    return scores


def select_blocks(scores, *, topk=16, block_size=128, sel=None):
    """Top-k block selection from pooled scores [N,G,nb] -> sel int32 [G,N,topk]."""
    lib = load()
    N, G, nb = scores.shape
    _need(scores, torch.float32, "scores")
    p = params(16 * G, G, 128, 64, block_size, topk)
    if sel is None:
        sel = torch.empty((G, N, topk), dtype=torch.int32, device=scores.device)
    _check(lib.msa_select_blocks(ctypes.byref(p), N, _ptr(scores), _ptr(sel), _stream(scores.device)),
           "msa_select_blocks")
    return sel


def status_string(status: int) -> str:
    return load().msa_status_string(status).decode()
