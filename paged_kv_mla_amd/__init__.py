"""MI355X (gfx950) batched paged-KV MLA decode, absorbed form.

Thin ctypes binding over the C ABI in include/pkvmla.h (libpkvmla.so, built in
this directory by ``python paged_kv_mla_amd/build.py``).  Argument marshalling
only: every step of the decode runs in the library's HIP kernels.  PyTorch is
used for device memory and streams; there is no CPU or PyTorch fallback, and
importing this package fails if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

# PyTorch-ROCm ships its own HIP runtime under the same SONAME as the system
# one (libamdhip64.so.7).  Importing torch first makes libpkvmla.so bind to the
# runtime torch already loaded, so one process never mixes two HIP/HSA runtimes.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkvmla.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python paged_kv_mla_amd/build.py` "
        "(hipcc, gfx950).  There is no fallback implementation.")

_lib = ctypes.CDLL(LIB_PATH)

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p

_lib.pkvmla_plan_create.argtypes = [_i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_float, _vp, ctypes.POINTER(_vp)]
_lib.pkvmla_plan_create_cascade.argtypes = [_i32p, ctypes.c_int32, _i32p, _i32p, _i32p,
                                            _i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_float, _vp,
                                            ctypes.POINTER(_vp)]
_lib.pkvmla_plan_create_cascade_with_capacity.argtypes = [
    _i32p, ctypes.c_int32, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p, ctypes.c_int32,
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
    ctypes.c_float, ctypes.c_int64, _vp, ctypes.POINTER(_vp)]
_lib.pkvmla_plan_update_cascade.argtypes = [_vp, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p, _i32p,
                                            _vp]
_lib.pkvmla_plan_create_with_capacity.argtypes = [_i32p, _i32p, _i32p, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                                  ctypes.c_int64, _vp, ctypes.POINTER(_vp)]
_lib.pkvmla_plan_update.argtypes = [_vp, _i32p, _i32p, _i32p, _vp]
_lib.pkvmla_plan_create_qo.argtypes = [_i32p, _i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_float, _vp, ctypes.POINTER(_vp)]
_lib.pkvmla_plan_create_qo_layout.argtypes = [_i32p, _i32p, _i32p, _i32p, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                              ctypes.c_int32, _vp, ctypes.POINTER(_vp)]
_lib.pkvmla_plan_create_qo_with_capacity.argtypes = [
    _i32p, _i32p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
    ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int64, _vp,
    ctypes.POINTER(_vp)]
_lib.pkvmla_plan_update_qo.argtypes = [_vp, _i32p, _i32p, _i32p, _i32p, _vp]
_lib.pkvmla_schedule_qo_rows_host.argtypes = [_i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              _i32p, ctypes.c_int64, _i32p, ctypes.c_int64,
                                              _i32p, ctypes.c_int64, _i32p, ctypes.c_int64,
                                              _i32p]
_lib.pkvmla_run.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.pkvmla_run_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.pkvmla_run_strided.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64,
                                    _vp, _vp, _vp]
_lib.pkvmla_run_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64,
                                ctypes.c_float, ctypes.c_float, _vp, _vp, _vp]
_lib.pkvmla_plan_destroy.argtypes = [_vp]
_lib.pkvmla_plan_destroy.restype = None
_lib.pkvmla_last_error.restype = ctypes.c_char_p
_lib.pkvmla_kernel_config.argtypes = [ctypes.c_int32, _i32p]
_lib.pkvmla_schedule_host.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int64,
                                      _i32p, ctypes.c_int64, _i32p, ctypes.c_int64, _i32p]
_lib.pkvmla_schedule_rows_host.argtypes = [_i32p, ctypes.c_int32, _i32p, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int64,
                                           _i32p, ctypes.c_int64, _i32p]
_lib.pkvmla_schedule_chain_host.argtypes = [_i32p, ctypes.c_int32, _i32p, _i32p, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int64,
                                            _i32p, ctypes.c_int64, _i32p, ctypes.c_int64, _i32p,
                                            ctypes.c_int64, _i32p]
_lib.pkvmla_plan_export.argtypes = [_vp, _i32p, ctypes.c_int64, _i64p]
_lib.pkvmla_gather.argtypes = [_vp, _vp, _vp, _vp, _vp]
_lib.pkvmla_gather_rows.argtypes = [_vp, _i64p]
_lib.pkvmla_plan_set_timing.argtypes = [_vp, ctypes.c_int32]
_lib.pkvmla_plan_set_wait_limit.argtypes = [_vp, ctypes.c_int32]
_lib.pkvmla_plan_timing_runs.argtypes = [_vp, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double), ctypes.c_int64,
                                         ctypes.POINTER(ctypes.c_int64)]
_lib.pkvmla_plan_timing.argtypes = [_vp, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double), _i64p]

EXPORTED_SYMBOLS = (
    "pkvmla_plan_create", "pkvmla_plan_create_with_capacity", "pkvmla_plan_update",
    "pkvmla_plan_create_cascade", "pkvmla_run", "pkvmla_run_strided", "pkvmla_plan_destroy",
    "pkvmla_last_error", "pkvmla_kernel_config", "pkvmla_schedule_host", "pkvmla_plan_export",
    "pkvmla_gather", "pkvmla_gather_rows", "pkvmla_plan_set_timing", "pkvmla_plan_timing",
    "pkvmla_run_noalloc", "pkvmla_plan_create_qo", "pkvmla_schedule_rows_host",
    "pkvmla_plan_create_cascade_with_capacity", "pkvmla_plan_update_cascade", "pkvmla_run_fp8",
    "pkvmla_schedule_chain_host", "pkvmla_plan_create_qo_layout", "pkvmla_schedule_qo_rows_host",
    "pkvmla_plan_create_qo_with_capacity", "pkvmla_plan_update_qo", "pkvmla_plan_timing_runs",
    "pkvmla_plan_set_wait_limit",
)

# work layouts of a plan with several query tokens per request
QO_AUTO, QO_TOKENS, QO_ROW_BLOCKS = 0, 1, 2

OK, EINVAL, EUNSUPPORTED, EHIP, ENOMEM = 0, 1, 2, 3, 4
_NAMES = {EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", EHIP: "EHIP", ENOMEM: "ENOMEM"}


class PkvmlaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkvmla {_NAMES.get(code, code)}: {msg}")
        self.code = code


def last_error() -> str:
    return (_lib.pkvmla_last_error() or b"").decode()


def _check(rc: int) -> None:
    if rc != OK:
        raise PkvmlaError(rc, last_error())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_i32p)


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _check_csr(what: str, indptr: np.ndarray, indices: np.ndarray, lens: np.ndarray) -> None:
    """Array lengths the C layer trusts (it reads indptr[n] and indices[:indptr[n]])."""
    if lens.ndim != 1 or indptr.ndim != 1 or indices.ndim != 1:
        raise ValueError(f"{what}: indptr, indices and lengths must be 1-D")
    if len(indptr) != len(lens) + 1:
        raise ValueError(f"{what}: indptr needs {len(lens) + 1} entries (got {len(indptr)})")
    if len(indptr) and indptr[-1] > len(indices):
        raise ValueError(f"{what}: indptr[-1] = {indptr[-1]} exceeds the {len(indices)} indices")


def _current_device() -> int:
    import torch
    return int(torch.cuda.current_device()) if torch.cuda.is_available() else 0


def kernel_config(num_heads: int) -> dict:
    cfg = np.zeros(7, dtype=np.int32)
    _check(_lib.pkvmla_kernel_config(int(num_heads), _ptr(cfg)))
    keys = ("tile", "waves", "heads_per_wave", "stages", "wg_per_cu", "fixed_cost", "head_groups")
    return {k: int(v) for k, v in zip(keys, cfg)}


def schedule_host(items, batch: int, num_wg: int, tile: int, fixed_cost: int):
    """The library's split-KV schedule for (request, sequence, length) items,
    computed on the host.  Returns (wg_indptr, units [n, 8], merges [m, 4])."""
    it = _i32(items).reshape(-1, 3)
    n_tok_tiles = int(sum(-(-int(L) // tile) for L in it[:, 2]))
    cap_u = 8 * (n_tok_tiles + num_wg + 8)
    cap_m = 4 * (batch + 1)
    wg = np.zeros(num_wg + 1, np.int32)
    units = np.zeros(cap_u, np.int32)
    merges = np.zeros(cap_m, np.int32)
    counts = np.zeros(3, np.int32)
    _check(_lib.pkvmla_schedule_host(_ptr(it), len(it), int(batch), int(num_wg), int(tile),
                                     int(fixed_cost), _ptr(wg), wg.size, _ptr(units), units.size,
                                     _ptr(merges), merges.size, _ptr(counts)))
    grid, nu, nm = (int(c) for c in counts)
    return wg[:grid + 1].copy(), units[:8 * nu].reshape(nu, 8).copy(), merges[:4 * nm].reshape(nm, 4).copy()


def schedule_rows_host(group_req_indptr, prefix_lens, num_heads: int, num_wg: int,
                       tile: int = 32):
    """The library's level-0 (shared-prefix) schedule of a cascade plan,
    computed on the host.  Returns (wg_indptr, units [n, 8], n_slots)."""
    gi, pl = _i32(group_req_indptr), _i32(prefix_lens)
    if gi.ndim != 1 or pl.ndim != 1 or len(gi) != len(pl) + 1:
        raise ValueError("group_req_indptr needs len(prefix_lens) + 1 entries")
    rows = int(gi[-1]) * int(num_heads)
    n_blocks = rows // 64 + len(pl) + 1
    cap_u = 8 * (n_blocks + 1) * max(1, int(num_wg))
    wg = np.zeros(int(num_wg) + 1, np.int32)
    units = np.zeros(cap_u, np.int32)
    counts = np.zeros(3, np.int32)
    _check(_lib.pkvmla_schedule_rows_host(_ptr(gi), len(pl), _ptr(pl), int(num_heads),
                                          int(num_wg), int(tile), _ptr(wg), wg.size, _ptr(units),
                                          units.size, _ptr(counts)))
    grid, nu, ns = (int(c) for c in counts)
    return wg[:grid + 1].copy(), units[:8 * nu].reshape(nu, 8).copy(), ns


def schedule_chain_host(group_req_indptr, prefix_lens, kv_lens, num_wg: int, tile: int = 32):
    """The library's one-launch cascade schedule, computed on the host.
    Returns (wg_indptr, units [n, 8], merges [m, 4], slot_list)."""
    gi, pl, kl = _i32(group_req_indptr), _i32(prefix_lens), _i32(kv_lens)
    if gi.ndim != 1 or len(gi) != len(pl) + 1:
        raise ValueError("group_req_indptr needs len(prefix_lens) + 1 entries")
    B = len(kl)
    cap = 2 * (B + int(num_wg)) + 8
    wg = np.zeros(int(num_wg) + 1, np.int32)
    units = np.zeros(8 * cap, np.int32)
    merges = np.zeros(4 * (B + 1), np.int32)
    lst = np.zeros(cap, np.int32)
    counts = np.zeros(4, np.int32)
    _check(_lib.pkvmla_schedule_chain_host(_ptr(gi), len(pl), _ptr(pl), _ptr(kl), B, int(num_wg),
                                           int(tile), _ptr(wg), wg.size, _ptr(units), units.size,
                                           _ptr(merges), merges.size, _ptr(lst), lst.size,
                                           _ptr(counts)))
    grid, nu, nm, nl = (int(c) for c in counts)
    return (wg[:grid + 1].copy(), units[:8 * nu].reshape(nu, 8).copy(),
            merges[:4 * nm].reshape(nm, 4).copy(), lst[:nl].copy())


def schedule_qo_rows_host(qo_indptr, kv_lens, num_heads: int, num_wg: int, tile: int = 32,
                          fixed_cost: int = 4):
    """The library's row-block schedule of several query tokens per request,
    computed on the host.  Returns (wg_indptr, units [n, 8], merges [m, 4],
    slot_list, n_slots, auto_picks_rows)."""
    qi, kl = _i32(qo_indptr), _i32(kv_lens)
    if qi.ndim != 1 or len(qi) != len(kl) + 1:
        raise ValueError("qo_indptr needs len(kv_lens) + 1 entries")
    B = len(kl)
    blocks = int(sum(-(-int(qi[b + 1] - qi[b]) * int(num_heads) // 64) for b in range(B)))
    ucap = blocks + int(num_wg) + 8
    tokens = int(qi[-1])
    wg = np.zeros(int(num_wg) + 1, np.int32)
    units = np.zeros(8 * ucap, np.int32)
    merges = np.zeros(4 * (tokens + 1), np.int32)
    lst = np.zeros(ucap * 4 + 8, np.int32)
    counts = np.zeros(6, np.int32)
    _check(_lib.pkvmla_schedule_qo_rows_host(_ptr(qi), _ptr(kl), B, int(num_heads), int(num_wg),
                                             int(tile), int(fixed_cost), _ptr(wg), wg.size,
                                             _ptr(units), units.size, _ptr(merges), merges.size,
                                             _ptr(lst), lst.size, _ptr(counts)))
    grid, nu, nm, nl, ns, auto = (int(c) for c in counts)
    return (wg[:grid + 1].copy(), units[:8 * nu].reshape(nu, 8).copy(),
            merges[:4 * nm].reshape(nm, 4).copy(), lst[:nl].copy(), ns, bool(auto))


@dataclass
class PlanExport:
    header: np.ndarray
    sm_scale: float
    wg_indptr: np.ndarray
    units: np.ndarray
    merges: np.ndarray
    seq_indptr: np.ndarray
    seq_lens: np.ndarray
    seq_indices: np.ndarray
    wg_indptr0: np.ndarray = None   # cascade level 0, or the row blocks of several
                                    # query tokens per request (empty for other plans)
    units0: np.ndarray = None
    slot_list: np.ndarray = None

    @property
    def grid(self) -> int:
        return int(self.header[12])

    @property
    def num_cu(self) -> int:
        return int(self.header[18])

    @property
    def head_groups(self) -> int:
        return int(self.header[22])


class Plan:
    """A decode plan (page table + work schedule on the device).  Build with
    :func:`plan` or :func:`plan_cascade`; run it with :meth:`run` for every
    set of tensors (e.g. once per layer) that shares the page table."""

    def __init__(self, handle: int, batch: int, num_heads: int, page_size: int = 0,
                 num_pages: int = 0, device: int = 0):
        self._h = ctypes.c_void_p(handle)
        self.batch = batch
        self.num_heads = num_heads
        self.page_size = page_size
        self.num_pages = num_pages
        self.device = device

    def __del__(self):
        h = getattr(self, "_h", None)
        # (at interpreter exit the module globals may already be gone)
        if h is not None and h.value and _lib is not None:
            _lib.pkvmla_plan_destroy(h)
            self._h = None

    def destroy(self) -> None:
        self.__del__()

    def run(self, q_nope, q_pe, ckv_cache, kpe_cache, out=None, lse=None, stream=None,
            kv_scales=None):
        """Decode on the device.  q_nope [B,H,512], q_pe [B,H,64] are
        contiguous bf16 CUDA tensors; ckv_cache [P,ps,512] and kpe_cache
        [P,ps,64] are bf16 with unit stride inside a row and packed rows within
        a page (row stride S, page stride ps*S): contiguous tensors, or the two
        views [..., :512] and [..., 512:] of one [P,ps,576] cache.  With
        kv_scales = (ckv_scale, kpe_scale) the caches hold OCP E4M3 codes
        (uint8 or float8_e4m3fn tensors of the same shapes) and a value is its
        scale times its code's value.  Returns (out bf16 [B,H,512], lse fp32
        [B,H]); out/lse are allocated when not given.  Asynchronous on
        `stream` (default: current stream)."""
        import torch
        B, H = self.batch, self.num_heads
        fp8 = kv_scales is not None
        kv_dtypes = (torch.uint8, torch.float8_e4m3fn) if fp8 else (torch.bfloat16,)
        # The C layer sees raw pointers only: every bound it cannot check
        # (device, shape, dtype, pool size) is checked here, before a launch.
        for name, t, shape in (("q_nope", q_nope, (B, H, 512)), ("q_pe", q_pe, (B, H, 64))):
            if tuple(t.shape) != shape or t.dtype != torch.bfloat16 or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous bf16 tensor of shape {shape}")
        strides = []
        for name, t, d in (("ckv_cache", ckv_cache, 512), ("kpe_cache", kpe_cache, 64)):
            ok = t.dim() == 3 and t.shape[2] == d and t.dtype in kv_dtypes
            S = t.stride(1) if ok else 0
            if not ok or t.stride(2) != 1 or t.stride(0) != t.shape[1] * S:
                raise ValueError(f"{name} must be a {'fp8' if fp8 else 'bf16'} "
                                 f"[pages, page_size, {d}] tensor with unit stride in a row "
                                 "and packed rows")
            if t.shape[0] < self.num_pages or t.shape[1] != self.page_size:
                raise ValueError(f"{name} holds {t.shape[0]} pages of {t.shape[1]} slots; the "
                                 f"plan needs >= {self.num_pages} pages of {self.page_size}")
            strides.append(S)
        if out is None:
            out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=q_nope.device)
        elif tuple(out.shape) != (B, H, 512) or out.dtype != torch.bfloat16 or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous bf16 tensor of shape {(B, H, 512)}")
        if lse is None:
            lse = torch.empty((B, H), dtype=torch.float32, device=q_nope.device)
        elif tuple(lse.shape) != (B, H) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError(f"lse must be a contiguous float32 tensor of shape {(B, H)}")
        for name, t in (("q_nope", q_nope), ("q_pe", q_pe), ("ckv_cache", ckv_cache),
                        ("kpe_cache", kpe_cache), ("out", out), ("lse", lse)):
            if not t.is_cuda or t.device.index != self.device:
                raise ValueError(f"{name} must live on cuda:{self.device}, the plan's device "
                                 f"(got {t.device})")
        if fp8:
            _check(_lib.pkvmla_run_fp8(self._h, q_nope.data_ptr(), q_pe.data_ptr(),
                                       ckv_cache.data_ptr(), kpe_cache.data_ptr(), strides[0],
                                       strides[1], float(kv_scales[0]), float(kv_scales[1]),
                                       out.data_ptr(), lse.data_ptr(), _stream_handle(stream)))
        else:
            _check(_lib.pkvmla_run_strided(self._h, q_nope.data_ptr(), q_pe.data_ptr(),
                                           ckv_cache.data_ptr(), kpe_cache.data_ptr(),
                                           strides[0], strides[1], out.data_ptr(),
                                           lse.data_ptr(), _stream_handle(stream)))
        return out, lse

    def update(self, kv_indptr, kv_indices, kv_lens, stream=None) -> None:
        """Replace the page table and lengths of a flat plan in place (same
        batch): no pointer or launch shape changes, so a HIP graph captured
        around :meth:`run` replays the new tables.  Waits for earlier work on
        `stream` (default: current stream)."""
        ip, ix, ln = _i32(kv_indptr), _i32(kv_indices), _i32(kv_lens)
        if len(ln) != self.batch or len(ip) != self.batch + 1:
            raise ValueError(f"update needs batch {self.batch} (kv_lens) and batch + 1 (kv_indptr)")
        _check_csr("kv", ip, ix, ln)
        if ix.size == 0:
            ix = np.zeros(1, np.int32)
        _check(_lib.pkvmla_plan_update(self._h, _ptr(ip), _ptr(ix), _ptr(ln),
                                       _stream_handle(stream)))

    def update_cascade(self, group_req_indptr, prefix_indptr, prefix_indices, prefix_lens,
                       kv_indptr, kv_indices, kv_lens, stream=None) -> None:
        """Replace a cascade plan's groups, prefixes and suffixes in place (same
        number of groups and batch), as :meth:`update` does for flat plans."""
        g, pip, pix, pl, ip, ix, ln = _cascade_arrays(group_req_indptr, prefix_indptr,
                                                      prefix_indices, prefix_lens, kv_indptr,
                                                      kv_indices, kv_lens)
        if len(ln) != self.batch or len(pl) != getattr(self, "num_groups", -1):
            raise ValueError(f"update_cascade needs batch {self.batch} and the plan's "
                             f"{getattr(self, 'num_groups', None)} groups")
        _check(_lib.pkvmla_plan_update_cascade(self._h, _ptr(g), _ptr(pip), _ptr(pix), _ptr(pl),
                                               _ptr(ip), _ptr(ix), _ptr(ln),
                                               _stream_handle(stream)))

    def update_qo(self, qo_indptr, kv_indptr, kv_indices, kv_lens, stream=None) -> None:
        """Replace the page tables and token split of a plan with several query
        tokens per request in place (same number of requests and of query
        tokens), as :meth:`update` does for flat plans."""
        qi = _i32(qo_indptr)
        ip, ix, ln = _i32(kv_indptr), _i32(kv_indices), _i32(kv_lens)
        _check_csr("kv", ip, ix, ln)
        nreq = getattr(self, "num_requests", None)
        if nreq is None:
            raise ValueError("update_qo needs a plan built by plan_qo")
        if len(ln) != nreq or qi.ndim != 1 or len(qi) != nreq + 1:
            raise ValueError(f"update_qo needs {nreq} requests and {nreq + 1} qo_indptr entries")
        if int(qi[-1]) != self.batch:
            raise ValueError(f"update_qo needs {self.batch} query tokens (got {int(qi[-1])})")
        if ix.size == 0:
            ix = np.zeros(1, np.int32)
        _check(_lib.pkvmla_plan_update_qo(self._h, _ptr(qi), _ptr(ip), _ptr(ix), _ptr(ln),
                                          _stream_handle(stream)))

    def run_ptrs(self, q_nope: int, q_pe: int, ckv: int, kpe: int, out: int, lse: int,
                 stream: int) -> None:
        """Raw-pointer form of :meth:`run` (no checks beyond the library's)."""
        _check(_lib.pkvmla_run(self._h, q_nope, q_pe, ckv, kpe, out, lse, stream))

    def run_fp8_ptrs(self, q_nope: int, q_pe: int, ckv: int, kpe: int, ckv_row_stride: int,
                     kpe_row_stride: int, ckv_scale: float, kpe_scale: float, out: int, lse: int,
                     stream: int) -> None:
        """Raw-pointer form of :meth:`run` for fp8 caches (row strides in bytes)."""
        _check(_lib.pkvmla_run_fp8(self._h, q_nope, q_pe, ckv, kpe, int(ckv_row_stride),
                                   int(kpe_row_stride), float(ckv_scale), float(kpe_scale), out,
                                   lse, stream))

    def run_noalloc_ptrs(self, q_nope: int, q_pe: int, ckv: int, kpe: int, out: int, lse: int,
                         stream: int) -> None:
        """Raw-pointer form of the allocation-free run (the split workspace is
        the library's static per-device scratch; packed caches)."""
        _check(_lib.pkvmla_run_noalloc(self._h, q_nope, q_pe, ckv, kpe, out, lse, stream))

    def set_wait_limit(self, polls: int = 1 << 20) -> None:
        """Polls before a progress-counter wait of the 16- and 32-head decode
        kernels gives up (outputs of later units then read NaN); 2^20 by
        default.  0 makes every such wait give up at once: the failure path,
        for tests."""
        _check(_lib.pkvmla_plan_set_wait_limit(self._h, int(polls)))

    def set_timing(self, enable=True, events: bool = False) -> None:
        """Record every later run's decode span (per-workgroup in-kernel
        stamps); with events=True also a HIP event pair around the launch."""
        _check(_lib.pkvmla_plan_set_timing(self._h, (2 if events else 1) if enable else 0))

    def timing_runs(self):
        """(span_us, start_us, merge_start_us) arrays of the last timed runs,
        oldest first; starts relative to the first run's start (merge start
        -1 for a run without a merge launch)."""
        n = ctypes.c_int64(0)
        cap = 256
        span = (ctypes.c_double * cap)()
        start = (ctypes.c_double * cap)()
        mstart = (ctypes.c_double * cap)()
        _check(_lib.pkvmla_plan_timing_runs(self._h, span, start, mstart, cap, ctypes.byref(n)))
        k = int(n.value)
        return np.array(span[:k]), np.array(start[:k]), np.array(mstart[:k])

    def kernel_timing(self):
        """(summed decode-kernel event ms, summed in-kernel span ms, number of
        timed runs), over the last 256 runs."""
        ms = ctypes.c_double(0.0)
        span = ctypes.c_double(0.0)
        n = ctypes.c_int64(0)
        _check(_lib.pkvmla_plan_timing(self._h, ctypes.byref(ms), ctypes.byref(span),
                                       ctypes.byref(n)))
        return float(ms.value), float(span.value), int(n.value)

    def gather_rows(self) -> int:
        n = ctypes.c_int64(0)
        _check(_lib.pkvmla_gather_rows(self._h, ctypes.byref(n)))
        return int(n.value)

    def gather(self, ckv_cache, kpe_cache, stream=None):
        """Rows [n, 576] bf16: ckv then kpe of every attended token, gathered
        through the decode kernel's page-table load path."""
        import torch
        rows = torch.empty((self.gather_rows(), 576), dtype=torch.bfloat16, device=ckv_cache.device)
        _check(_lib.pkvmla_gather(self._h, ckv_cache.data_ptr(), kpe_cache.data_ptr(),
                                  rows.data_ptr(), _stream_handle(stream)))
        return rows

    def export(self) -> PlanExport:
        used = ctypes.c_int64(0)
        _lib.pkvmla_plan_export(self._h, None, 0, ctypes.byref(used))
        buf = np.zeros(int(used.value), np.int32)
        _check(_lib.pkvmla_plan_export(self._h, _ptr(buf), buf.size, ctypes.byref(used)))
        hdr = buf[:32].copy()
        grid, nu, nm, ns, ni = int(hdr[12]), int(hdr[13]), int(hdr[14]), int(hdr[16]), int(hdr[17])
        g0, nu0, nsl = int(hdr[28]), int(hdr[29]), int(hdr[30])
        o = 32
        parts = []
        for n in (grid + 1, 8 * nu, 4 * nm, ns + 1, ns, ni,
                  (g0 + 1) if (int(hdr[20]) or int(hdr[26]) == 2) else 0, 8 * nu0, nsl):
            parts.append(buf[o:o + n].copy())
            o += n
        return PlanExport(header=hdr, sm_scale=float(hdr[19:20].view(np.float32)[0]),
                          wg_indptr=parts[0], units=parts[1].reshape(nu, 8),
                          merges=parts[2].reshape(nm, 4), seq_indptr=parts[3],
                          seq_lens=parts[4], seq_indices=parts[5], wg_indptr0=parts[6],
                          units0=parts[7].reshape(nu0, 8), slot_list=parts[8])


def plan(kv_indptr, kv_indices, kv_lens, num_heads: int, page_size: int, num_pages: int,
         ckv_dim: int = 512, kpe_dim: int = 64, sm_scale: Optional[float] = None,
         stream=None, index_capacity: int = 0) -> Plan:
    """Flat decode plan from host page-table arrays (int32): kv_indptr [B+1],
    kv_indices [kv_indptr[B]], kv_lens [B].  sm_scale None selects
    1/sqrt(ckv_dim + kpe_dim).  index_capacity > 0 sizes the plan for later
    :meth:`Plan.update` calls with up to that many page ids and fixes its
    launch shapes (for HIP-graph capture of :meth:`Plan.run`)."""
    ip, ix, ln = _i32(kv_indptr), _i32(kv_indices), _i32(kv_lens)
    _check_csr("kv", ip, ix, ln)
    if ix.size == 0:
        ix = np.zeros(1, np.int32)
    h = ctypes.c_void_p()
    _check(_lib.pkvmla_plan_create_with_capacity(
        _ptr(ip), _ptr(ix), _ptr(ln), int(len(ln)), int(num_pages), int(num_heads), int(ckv_dim),
        int(kpe_dim), int(page_size), float(sm_scale or 0.0), int(index_capacity),
        _stream_handle(stream) if stream else None, ctypes.byref(h)))
    return Plan(h.value, int(len(ln)), int(num_heads), int(page_size), int(num_pages),
                _current_device())


def plan_qo(qo_indptr, kv_indptr, kv_indices, kv_lens, num_heads: int, page_size: int,
            num_pages: int, ckv_dim: int = 512, kpe_dim: int = 64,
            sm_scale: Optional[float] = None, stream=None, layout: int = QO_AUTO,
            index_capacity: int = 0) -> Plan:
    """Plan with qo_indptr[b+1] - qo_indptr[b] new query tokens for request b,
    causal among them (they are the request's last tokens).  The run takes and
    returns one row per query token ([qo_indptr[-1], H, ...]); the Plan's
    ``batch`` is that row count.  ``layout``: QO_AUTO, QO_TOKENS (a work item
    per token) or QO_ROW_BLOCKS (16 or 32 heads: blocks of 64 query rows that
    score each KV tile once for several tokens).  index_capacity > 0 sizes the
    plan for :meth:`Plan.update_qo` (same batch and token count) and fixes its
    launch shapes."""
    qi = _i32(qo_indptr)
    ip, ix, ln = _i32(kv_indptr), _i32(kv_indices), _i32(kv_lens)
    _check_csr("kv", ip, ix, ln)
    if qi.ndim != 1 or len(qi) != len(ln) + 1:
        raise ValueError(f"qo_indptr needs {len(ln) + 1} entries (got {len(qi)})")
    if ix.size == 0:
        ix = np.zeros(1, np.int32)
    h = ctypes.c_void_p()
    _check(_lib.pkvmla_plan_create_qo_with_capacity(
        _ptr(qi), _ptr(ip), _ptr(ix), _ptr(ln), int(len(ln)), int(num_pages), int(num_heads),
        int(ckv_dim), int(kpe_dim), int(page_size), float(sm_scale or 0.0), int(layout),
        int(index_capacity), _stream_handle(stream) if stream else None, ctypes.byref(h)))
    p = Plan(h.value, int(qi[-1]), int(num_heads), int(page_size), int(num_pages),
             _current_device())
    p.num_requests = int(len(ln))
    return p


def _cascade_arrays(group_req_indptr, prefix_indptr, prefix_indices, prefix_lens, kv_indptr,
                    kv_indices, kv_lens):
    g, pip, pix, pl = (_i32(group_req_indptr), _i32(prefix_indptr), _i32(prefix_indices),
                       _i32(prefix_lens))
    ip, ix, ln = _i32(kv_indptr), _i32(kv_indices), _i32(kv_lens)
    if g.ndim != 1 or len(g) != len(pl) + 1:
        raise ValueError("group_req_indptr needs num_groups + 1 entries")
    _check_csr("prefix", pip, pix, pl)
    _check_csr("suffix", ip, ix, ln)
    if pix.size == 0:
        pix = np.zeros(1, np.int32)
    if ix.size == 0:
        ix = np.zeros(1, np.int32)
    return g, pip, pix, pl, ip, ix, ln


def plan_cascade(group_req_indptr, prefix_indptr, prefix_indices, prefix_lens,
                 kv_indptr, kv_indices, kv_lens, num_heads: int, page_size: int,
                 num_pages: int, ckv_dim: int = 512, kpe_dim: int = 64,
                 sm_scale: Optional[float] = None, stream=None, index_capacity: int = 0) -> Plan:
    """Two-level plan: per group a shared prefix page list, per request its
    own suffix list (kv_lens may be 0); states are merged by log-sum-exp.
    index_capacity > 0 sizes the plan for later :meth:`Plan.update_cascade`
    calls (prefix and suffix page ids together) and fixes its launch shapes."""
    g, pip, pix, pl, ip, ix, ln = _cascade_arrays(group_req_indptr, prefix_indptr,
                                                  prefix_indices, prefix_lens, kv_indptr,
                                                  kv_indices, kv_lens)
    h = ctypes.c_void_p()
    _check(_lib.pkvmla_plan_create_cascade_with_capacity(
        _ptr(g), int(len(pl)), _ptr(pip), _ptr(pix), _ptr(pl), _ptr(ip), _ptr(ix), _ptr(ln),
        int(len(ln)), int(num_pages), int(num_heads), int(ckv_dim), int(kpe_dim), int(page_size),
        float(sm_scale or 0.0), int(index_capacity),
        _stream_handle(stream) if stream else None, ctypes.byref(h)))
    p = Plan(h.value, int(len(ln)), int(num_heads), int(page_size), int(num_pages),
             _current_device())
    p.num_groups = int(len(pl))
    return p


def plan_for(inp, stream=None, qo_layout: int = QO_AUTO) -> Plan:
    """Plan for an input bundle from mla_workloads (flat, several query
    tokens per request, or cascade)."""
    if getattr(inp, "qo_indptr", None) is not None:
        return plan_qo(inp.qo_indptr, inp.kv_indptr, inp.kv_indices, inp.kv_lens, inp.num_heads,
                       inp.page_size, inp.num_pages, sm_scale=inp.sm_scale, stream=stream,
                       layout=qo_layout)
    if hasattr(inp, "prefix_lens"):
        return plan_cascade(inp.group_req_indptr, inp.prefix_indptr, inp.prefix_indices,
                            inp.prefix_lens, inp.kv_indptr, inp.kv_indices, inp.kv_lens,
                            inp.num_heads, inp.page_size, inp.num_pages, sm_scale=inp.sm_scale,
                            stream=stream)
    return plan(inp.kv_indptr, inp.kv_indices, inp.kv_lens, inp.num_heads, inp.page_size,
                inp.num_pages, sm_scale=inp.sm_scale, stream=stream)
