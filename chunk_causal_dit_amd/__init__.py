"""Python binding of libwf: the chunk-wise causal attention round of Wave Forcing on MI355X.

Argument marshalling only. Every step of the round runs in the HIP kernels of
``libwf.so`` (built by ``python -m chunk_causal_dit_amd.build``); torch is used
to hold device memory and to name the stream. There is no fallback: if the
library is missing, importing the calls raises.

Calls mirror include/wf.h:
    KVCache(...)                 wf_kv_pool_bytes / wf_kv_cache_create
      .append / .refresh / .evict / .set_table / .table
    rope3d(x, ...)               wf_rope3d (in place)
    chunk_causal_attn_fwd(...)   wf_chunk_causal_attn_fwd, or wf_chunk_causal_attn_fwd_ws
                                 with a workspace (attn_fwd_workspace_bytes)
    chunk_causal_attn_fwd_i8qk(...), attn_i8qk_workspace_bytes(...)
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Callable, List, Optional, Sequence, Tuple

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

__all__ = [
    "WFError", "lib", "library_path", "exported_symbols", "header_symbols",
    "WF_F32", "WF_BF16", "KVCache", "kv_pool_bytes", "rope3d",
    "chunk_causal_attn_fwd", "attn_fwd_workspace_bytes", "attn_fwd_workspace", "attn_i8qk_workspace_bytes", "chunk_causal_attn_fwd_i8qk",
    "quant_rows_i8", "gemm_w8a8", "WF_I32",
    "WF_MAX_TABLE", "RoundPlan", "device_peak_info", "rounds_1f1c", "plan_1f1c", "run_round", "Rollout1F1C",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
HEADER = os.path.join(_ROOT, "include", "wf.h")

WF_F32, WF_BF16, WF_I32 = 0, 1, 2
WF_MAX_TABLE = 64
WF_KV_ADOPT, WF_KV_ZERO_FILL = 0, 1
_DTYPE = {torch.float32: WF_F32, torch.bfloat16: WF_BF16}


class WFError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: status {status} ({text})")
        self.status = status


def library_path() -> str:
    return os.environ.get("WF_LIBRARY", os.path.join(_HERE, "libwf.so"))


_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p


class RoundPlan(ctypes.Structure):
    """One round of a 1F1C rollout (the C struct wf_round_plan)."""

    _fields_ = [
        ("round", _c_int), ("n_inflight", _c_int),
        ("inflight_chunk", _c_int * WF_MAX_TABLE), ("inflight_stage", _c_int * WF_MAX_TABLE),
        ("n_hist", _c_int), ("hist_chunk", _c_int * WF_MAX_TABLE),
        ("new_chunk", _c_int), ("output_chunk", _c_int), ("evict_after", _c_int),
    ]

    @property
    def inflight(self) -> List[Tuple[int, int]]:
        """(chunk, stage) cleanest first; stage n_steps is the refresh pass."""
        return [(self.inflight_chunk[i], self.inflight_stage[i]) for i in range(self.n_inflight)]

    @property
    def hist(self) -> List[int]:
        return [self.hist_chunk[i] for i in range(self.n_hist)]

    @property
    def new(self) -> Optional[int]:
        return None if self.new_chunk < 0 else self.new_chunk

    @property
    def output(self) -> Optional[int]:
        return None if self.output_chunk < 0 else self.output_chunk


_SIGNATURES = {
    "wf_kv_pool_bytes": (_c_size, [_c_int] * 5),
    "wf_kv_cache_create": (_c_int, [ctypes.POINTER(_vp), _vp, _vp] + [_c_int] * 6 + [_vp]),
    "wf_kv_cache_destroy": (_c_int, [_vp]),
    "wf_kv_append": (_c_int, [_vp, _vp, _vp, _vp, ctypes.POINTER(_c_int)]),
    "wf_kv_refresh": (_c_int, [_vp, _c_int, _vp, _vp, _vp]),
    "wf_kv_evict": (_c_int, [_vp, _c_int]),
    "wf_kv_set_table": (_c_int, [_vp, ctypes.POINTER(_c_int), _c_int]),
    "wf_kv_get_table": (_c_int, [_vp, ctypes.POINTER(_c_int), _c_int, ctypes.POINTER(_c_int)]),
    "wf_rope3d": (_c_int, [_vp] + [_c_int] * 11 + [ctypes.c_float, _vp]),
    "wf_chunk_causal_attn_fwd": (_c_int, [_vp, _vp, _c_int, ctypes.c_float, _vp, _vp, _vp]),
    "wf_attn_fwd_workspace_bytes": (_c_size, [_vp]),
    "wf_chunk_causal_attn_fwd_ws": (_c_int, [_vp, _vp, _c_int, ctypes.c_float, _vp, _vp, _vp, _vp]),
    "wf_chunk_causal_attn_fwd_static": (_c_int, [_vp, _vp, _c_int, ctypes.c_float, _vp, _vp, _vp]),
    "wf_kv_set_rope": (_c_int, [_vp] + [_c_int] * 6 + [ctypes.c_float]),
    "wf_kv_append_rope": (_c_int, [_vp, _vp, _vp, _c_int, _vp, ctypes.POINTER(_c_int)]),
    "wf_kv_refresh_rope": (_c_int, [_vp, _c_int, _vp, _vp, _c_int, _vp]),
    "wf_attn_i8qk_workspace_bytes": (_c_size, [_vp, _c_int]),
    "wf_chunk_causal_attn_fwd_i8qk": (_c_int, [_vp, _vp, _c_int, ctypes.c_float, _vp, _vp, _vp, _vp]),
    "wf_quant_rows_i8": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "wf_gemm_w8a8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "wf_1f1c_rounds": (_c_int, [_c_int, _c_int]),
    "wf_1f1c_plan": (_c_int, [_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(RoundPlan)]),
    "wf_1f1c_run_round": (_c_int, [_vp, ctypes.POINTER(RoundPlan), _vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                   ctypes.c_float, _vp, _vp, _vp, _vp]),
    "wf_status_str": (ctypes.c_char_p, [_c_int]),
    "wf_last_error": (ctypes.c_char_p, []),
    "wf_version": (_c_int, []),
    "wf_device_peak_info": (_c_int, [_c_int, ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libwf.so (loaded on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m chunk_causal_dit_amd.build`")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def header_symbols() -> List[str]:
    """Function names declared in include/wf.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wf_[a-z0-9_]+)\s*\(", text)))


def exported_symbols() -> List[str]:
    """wf_* function names exported by the built library (dynamic symbol table)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", library_path()], capture_output=True, text=True,
                         check=True).stdout
    return sorted({l.split()[-1] for l in out.splitlines() if l.split()[-1].startswith("wf_")})


def _check(status: int, where: str) -> None:
    if status != 0:
        L = lib()
        raise WFError(status, where, f"{L.wf_status_str(status).decode()}; {L.wf_last_error().decode()}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str) -> _vp:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _vp(t.data_ptr())


def _workspace(ws: Optional[torch.Tensor], need: int, where: str) -> Optional[_vp]:
    """Device pointer of a caller's workspace after checking that it holds need bytes (the
    C calls take no size: a short buffer would be written past its end)."""
    if ws is None:
        return None
    have = ws.numel() * ws.element_size()
    if have < need:
        raise ValueError(f"{where}: workspace holds {have} bytes, the call needs {need}")
    return _dev(ws, "workspace")


def kv_pool_bytes(n_slots: int, chunk_tokens: int, n_heads: int, head_dim: int, dtype: torch.dtype) -> int:
    return int(lib().wf_kv_pool_bytes(n_slots, chunk_tokens, n_heads, head_dim, _DTYPE[dtype]))


class KVCache:
    """Ring-buffer history cache over two device pools (owned by this object)."""

    def __init__(self, n_slots: int, chunk_tokens: int, n_heads: int, head_dim: int,
                 dtype: torch.dtype = torch.bfloat16, device="cuda", stream=None):
        if dtype not in _DTYPE:
            raise ValueError(f"unsupported dtype {dtype}")
        nbytes = kv_pool_bytes(n_slots, chunk_tokens, n_heads, head_dim, dtype)
        if nbytes == 0:  # the shape check recorded why
            raise WFError(-2, "wf_kv_pool_bytes", lib().wf_last_error().decode())
        self.n_slots, self.chunk_tokens, self.n_heads, self.head_dim = n_slots, chunk_tokens, n_heads, head_dim
        self.dtype = dtype
        self.s_pad = (chunk_tokens + 127) // 128 * 128
        self.k_pool = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.v_pool = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = _vp()
        _check(lib().wf_kv_cache_create(ctypes.byref(h), _dev(self.k_pool, "k_pool"), _dev(self.v_pool, "v_pool"),
                                        n_slots, chunk_tokens, n_heads, head_dim, _DTYPE[dtype],
                                        WF_KV_ZERO_FILL, _vp(_stream(stream))), "wf_kv_cache_create")
        self._h = h

    # decoded contents of one physical slot, [H][S_pad][D] (for inspection and tests)
    def _slot_raw(self, pool: torch.Tensor, slot: int) -> torch.Tensor:
        n = self.n_heads * self.s_pad * self.head_dim
        return pool.view(self.dtype)[slot * n:(slot + 1) * n]

    def k_slot(self, slot: int) -> torch.Tensor:
        """K tile images [H][S_pad/64][D/E][64][E] (E = 16 bytes of elements) -> [H][S_pad][D]."""
        H, S, D = self.n_heads, self.s_pad, self.head_dim
        E = 16 // self.k_pool.view(self.dtype).element_size()
        raw = self._slot_raw(self.k_pool, slot).view(H, S // 64, D // E, 64, E)
        return raw.permute(0, 1, 3, 2, 4).reshape(H, S, D)

    def v_slot(self, slot: int) -> torch.Tensor:
        """V tile images [H][S_pad/64][64/E][D][E] -> [H][S_pad][D]."""
        H, S, D = self.n_heads, self.s_pad, self.head_dim
        E = 16 // self.v_pool.view(self.dtype).element_size()
        raw = self._slot_raw(self.v_pool, slot).view(H, S // 64, 64 // E, D, E)
        return raw.permute(0, 1, 2, 4, 3).reshape(H, S, D)

    @property
    def handle(self) -> _vp:
        if self._h is None:
            raise ValueError("cache is closed")
        return self._h

    def _chunk(self, t: torch.Tensor, name: str) -> _vp:
        if t.dtype != self.dtype or tuple(t.shape) != (self.chunk_tokens, self.n_heads, self.head_dim):
            raise ValueError(f"{name} must be {self.dtype} [{self.chunk_tokens}][{self.n_heads}][{self.head_dim}],"
                             f" got {t.dtype} {tuple(t.shape)}")
        return _dev(t, name)

    def append(self, k: torch.Tensor, v: torch.Tensor, stream=None) -> int:
        slot = ctypes.c_int(-1)
        _check(lib().wf_kv_append(self.handle, self._chunk(k, "k"), self._chunk(v, "v"), _vp(_stream(stream)),
                                  ctypes.byref(slot)), "wf_kv_append")
        return slot.value

    def refresh(self, logical_idx: int, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        _check(lib().wf_kv_refresh(self.handle, logical_idx, self._chunk(k, "k"), self._chunk(v, "v"),
                                   _vp(_stream(stream))), "wf_kv_refresh")

    def set_rope(self, frames_per_chunk: int, grid_h: int, grid_w: int,
                 split: Tuple[int, int, int] = (44, 42, 42), theta: float = 10000.0) -> None:
        """RoPE geometry for append_rope / refresh_rope (same convention as rope3d)."""
        _check(lib().wf_kv_set_rope(self.handle, frames_per_chunk, grid_h, grid_w, split[0], split[1], split[2],
                                    float(theta)), "wf_kv_set_rope")

    def append_rope(self, k: torch.Tensor, v: torch.Tensor, global_chunk: int, stream=None) -> int:
        """append with K rotated at the positions of global chunk global_chunk (k is not modified)."""
        slot = ctypes.c_int(-1)
        _check(lib().wf_kv_append_rope(self.handle, self._chunk(k, "k"), self._chunk(v, "v"), global_chunk,
                                       _vp(_stream(stream)), ctypes.byref(slot)), "wf_kv_append_rope")
        return slot.value

    def refresh_rope(self, logical_idx: int, k: torch.Tensor, v: torch.Tensor, global_chunk: int,
                     stream=None) -> None:
        """refresh with K rotated at the positions of global chunk global_chunk."""
        _check(lib().wf_kv_refresh_rope(self.handle, logical_idx, self._chunk(k, "k"), self._chunk(v, "v"),
                                        global_chunk, _vp(_stream(stream))), "wf_kv_refresh_rope")

    def evict(self, n_oldest: int) -> None:
        _check(lib().wf_kv_evict(self.handle, n_oldest), "wf_kv_evict")

    def set_table(self, slots: Sequence[int]) -> None:
        arr = (ctypes.c_int * max(1, len(slots)))(*slots)
        _check(lib().wf_kv_set_table(self.handle, arr, len(slots)), "wf_kv_set_table")

    def table(self) -> List[int]:
        arr = (ctypes.c_int * 64)()
        n = ctypes.c_int(0)
        _check(lib().wf_kv_get_table(self.handle, arr, 64, ctypes.byref(n)), "wf_kv_get_table")
        return list(arr[: n.value])

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and _lib is not None:
            _lib.wf_kv_cache_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rope3d(x: torch.Tensor, first_global_chunk: int, frames_per_chunk: int, grid_h: int, grid_w: int,
           split: Tuple[int, int, int] = (44, 42, 42), theta: float = 10000.0, stream=None) -> torch.Tensor:
    """In-place 3D rotary embedding of x [n_tokens][H][D]; returns x."""
    if x.dim() != 3 or x.dtype not in _DTYPE:
        raise ValueError("x must be [tokens][heads][head_dim] float32 or bfloat16")
    n, H, D = x.shape
    _check(lib().wf_rope3d(_dev(x, "x"), n, H, D, _DTYPE[x.dtype], first_global_chunk, frames_per_chunk,
                           grid_h, grid_w, split[0], split[1], split[2], float(theta), _vp(_stream(stream))),
           "wf_rope3d")
    return x


def _attn_io(q, cache, n_inflight, out, lse, with_lse):
    nq = n_inflight * cache.chunk_tokens
    shape = (nq, cache.n_heads, cache.head_dim)
    if q.dtype != cache.dtype or tuple(q.shape) != shape:
        raise ValueError(f"q must be {cache.dtype} {shape}, got {q.dtype} {tuple(q.shape)}")
    if out is None:
        out = torch.empty_like(q)
    elif out.dtype != q.dtype or tuple(out.shape) != shape:
        raise ValueError("out must match q")
    if lse is None and with_lse:
        lse = torch.empty((cache.n_heads, nq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (cache.n_heads, nq)):
        raise ValueError(f"lse must be float32 [{cache.n_heads}][{nq}]")
    return out, lse


def attn_fwd_workspace_bytes(cache: KVCache) -> int:
    """Bytes of the key-split workspace of wf_chunk_causal_attn_fwd_ws (0 for fp32 caches)."""
    return int(lib().wf_attn_fwd_workspace_bytes(cache.handle))


def attn_fwd_workspace(cache: KVCache) -> Optional[torch.Tensor]:
    """A device workspace for the key split of this cache's rounds, or None when it has none."""
    n = attn_fwd_workspace_bytes(cache)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None


def chunk_causal_attn_fwd(q: torch.Tensor, cache: KVCache, n_inflight: int, scale: float,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          with_lse: bool = True, stream=None, workspace: Optional[torch.Tensor] = None):
    """Chunk-wise causal attention of the round. Returns (out, lse or None). With a workspace
    (attn_fwd_workspace) it calls wf_chunk_causal_attn_fwd_ws, which may split chunk 0's keys."""
    out, lse = _attn_io(q, cache, n_inflight, out, lse, with_lse)
    lse_p = _dev(lse, "lse") if lse is not None else None
    if workspace is None:
        _check(lib().wf_chunk_causal_attn_fwd(_dev(q, "q"), cache.handle, n_inflight, float(scale),
                                              _dev(out, "out"), lse_p, _vp(_stream(stream))),
               "wf_chunk_causal_attn_fwd")
    else:
        ws = _workspace(workspace, attn_fwd_workspace_bytes(cache), "wf_chunk_causal_attn_fwd_ws")
        _check(lib().wf_chunk_causal_attn_fwd_ws(_dev(q, "q"), cache.handle, n_inflight, float(scale), ws,
                                                 _dev(out, "out"), lse_p, _vp(_stream(stream))),
               "wf_chunk_causal_attn_fwd_ws")
    return out, lse


def chunk_causal_attn_fwd_static(q: torch.Tensor, cache: KVCache, n_inflight: int, scale: float,
                                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                                 with_lse: bool = True, stream=None):
    """wf_chunk_causal_attn_fwd_static: the key-split call with its partials in the library's
    static device scratch (the C call allocates nothing; out and lse are allocated here when
    not given). Calls that overlap on one GPU race on the scratch. Returns (out, lse or None)."""
    out, lse = _attn_io(q, cache, n_inflight, out, lse, with_lse)
    _check(lib().wf_chunk_causal_attn_fwd_static(_dev(q, "q"), cache.handle, n_inflight, float(scale),
                                                 _dev(out, "out"), _dev(lse, "lse") if lse is not None else None,
                                                 _vp(_stream(stream))),
           "wf_chunk_causal_attn_fwd_static")
    return out, lse


def attn_i8qk_workspace_bytes(cache: KVCache, n_inflight: int) -> int:
    return int(lib().wf_attn_i8qk_workspace_bytes(cache.handle, n_inflight))


def chunk_causal_attn_fwd_i8qk(q: torch.Tensor, cache: KVCache, n_inflight: int, scale: float,
                               workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None, with_lse: bool = True, stream=None):
    """int8-QK variant. Returns (out, lse or None)."""
    out, lse = _attn_io(q, cache, n_inflight, out, lse, with_lse)
    need = attn_i8qk_workspace_bytes(cache, n_inflight)
    if workspace is None:
        workspace = torch.empty(max(1, need), dtype=torch.uint8, device=q.device)
    _check(lib().wf_chunk_causal_attn_fwd_i8qk(_dev(q, "q"), cache.handle, n_inflight, float(scale),
                                               _workspace(workspace, need, "wf_chunk_causal_attn_fwd_i8qk"),
                                               _dev(out, "out"),
                                               _dev(lse, "lse") if lse is not None else None,
                                               _vp(_stream(stream))),
           "wf_chunk_causal_attn_fwd_i8qk")
    return out, lse


def quant_rows_i8(x: torch.Tensor, codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                  stream=None):
    """Per-row int8 quantization of x [rows][cols] bf16. Returns (codes int8, scales fp32)."""
    if x.dim() != 2 or x.dtype != torch.bfloat16:
        raise ValueError("x must be a 2-D bfloat16 tensor")
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.int8, device=x.device) if codes is None else codes
    scales = torch.empty(rows, dtype=torch.float32, device=x.device) if scales is None else scales
    if codes.shape != (rows, cols) or codes.dtype != torch.int8 or scales.shape != (rows,) \
            or scales.dtype != torch.float32:
        raise ValueError("codes must be int8 [rows][cols] and scales float32 [rows]")
    _check(lib().wf_quant_rows_i8(_dev(x, "x"), rows, cols, WF_BF16, _dev(codes, "codes"), _dev(scales, "scales"),
                                  _vp(_stream(stream))), "wf_quant_rows_i8")
    return codes, scales


def gemm_w8a8(xq: torch.Tensor, sx: Optional[torch.Tensor], wq: torch.Tensor, sw: Optional[torch.Tensor],
              bias: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
              out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """W8A8 linear: y[m][n] = s_x[m] s_w[n] sum_k xq[m,k] wq[n,k] + bias[n] (bf16), or the raw
    int32 accumulators with out_dtype=torch.int32."""
    if xq.dtype != torch.int8 or wq.dtype != torch.int8 or xq.dim() != 2 or wq.dim() != 2 or xq.shape[1] != wq.shape[1]:
        raise ValueError("xq [M][K] and wq [N][K] must be int8 with the same K")
    M, K = xq.shape
    N = wq.shape[0]
    code = {torch.bfloat16: WF_BF16, torch.int32: WF_I32}[out_dtype]
    out = torch.empty((M, N), dtype=out_dtype, device=xq.device) if out is None else out
    if tuple(out.shape) != (M, N) or out.dtype != out_dtype:
        raise ValueError(f"out must be {out_dtype} [{M}][{N}]")
    for t, name, n, dt in ((sx, "sx", M, torch.float32), (sw, "sw", N, torch.float32), (bias, "bias", N, torch.bfloat16)):
        if t is not None and (tuple(t.shape) != (n,) or t.dtype != dt):
            raise ValueError(f"{name} must be {dt} [{n}]")
    _check(lib().wf_gemm_w8a8(_dev(xq, "xq"), _dev(sx, "sx") if sx is not None else None, _dev(wq, "wq"),
                              _dev(sw, "sw") if sw is not None else None,
                              _dev(bias, "bias") if bias is not None else None, M, N, K, code, _dev(out, "out"),
                              _vp(_stream(stream))), "wf_gemm_w8a8")
    return out


def device_peak_info(device: int = 0) -> Tuple[int, int]:
    """(compute units, peak shader clock in kHz) of a device, as the HIP runtime reports them."""
    cu, clk = _c_int(), _c_int()
    _check(lib().wf_device_peak_info(device, ctypes.byref(cu), ctypes.byref(clk)), "wf_device_peak_info")
    return cu.value, clk.value


def rounds_1f1c(n_steps: int, n_chunks: int) -> int:
    """Rounds of a 1F1C rollout of n_chunks chunks with n_steps denoising steps."""
    n = lib().wf_1f1c_rounds(n_steps, n_chunks)
    if n < 0:
        _check(n, "wf_1f1c_rounds")
    return n


def plan_1f1c(n_steps: int, n_chunks: int, hist_window: int, r: int) -> RoundPlan:
    """The plan of round r (host only)."""
    p = RoundPlan()
    _check(lib().wf_1f1c_plan(n_steps, n_chunks, hist_window, r, ctypes.byref(p)), "wf_1f1c_plan")
    return p


def run_round(cache: KVCache, plan: RoundPlan, q: torch.Tensor, ks: Sequence[torch.Tensor],
              vs: Sequence[torch.Tensor], scale: float, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, with_lse: bool = True, stream=None,
              workspace: Optional[torch.Tensor] = None):
    """One round on the stream: append the new chunk, refresh the other in-flight entries,
    attention over the round's query block, evict. ks[i], vs[i] are this round's K/V of
    in-flight chunk i (cleanest first). With a RoPE geometry on the cache (set_rope), q is
    rotated in place and K inside the cache writes. A workspace (attn_fwd_workspace) lets the
    attention split chunk 0's keys. Returns (out, lse or None)."""
    N = plan.n_inflight
    if len(ks) != N or len(vs) != N:
        raise ValueError(f"need {N} K and V chunks, got {len(ks)} and {len(vs)}")
    out, lse = _attn_io(q, cache, N, out, lse, with_lse)
    kp = (_vp * N)(*[cache._chunk(t, "k").value for t in ks])
    vp = (_vp * N)(*[cache._chunk(t, "v").value for t in vs])
    _check(lib().wf_1f1c_run_round(cache.handle, ctypes.byref(plan), _dev(q, "q"), kp, vp, float(scale),
                                   _workspace(workspace, attn_fwd_workspace_bytes(cache), "wf_1f1c_run_round"),
                                   _dev(out, "out"), _dev(lse, "lse") if lse is not None else None,
                                   _vp(_stream(stream))), "wf_1f1c_run_round")
    return out, lse


class Rollout1F1C:
    """Drives a whole 1F1C rollout of one layer through the library.

    model(plan) returns the round's query block [n_inflight*C][H][D] and the lists of
    this round's K and V chunks of the in-flight chunks, cleanest first. Each call of
    step() plans the next round (wf_1f1c_plan) and enqueues it (wf_1f1c_run_round).
    With rope (the 3D geometry of wf_kv_set_rope), the query block is rotated in place
    each round and K inside the cache writes, at the chunks' global indices. With split
    (default), the rounds' attention runs with a key-split workspace held by the rollout."""

    def __init__(self, n_steps: int, n_chunks: int, hist_window: int, chunk_tokens: int, n_heads: int,
                 head_dim: int, scale: float, dtype: torch.dtype = torch.bfloat16, n_slots: Optional[int] = None,
                 stream=None, rope: Optional[dict] = None, split: bool = True):
        self.n_steps, self.n_chunks, self.hist_window, self.scale = n_steps, n_chunks, hist_window, scale
        self.n_rounds = rounds_1f1c(n_steps, n_chunks)
        plan_1f1c(n_steps, n_chunks, hist_window, 0)  # validates the window
        need = hist_window + n_steps + 1
        self.cache = KVCache(n_slots or need, chunk_tokens, n_heads, head_dim, dtype, stream=stream)
        if rope is not None:  # {"frames_per_chunk", "grid_h", "grid_w", optional "split", "theta"}
            self.cache.set_rope(rope["frames_per_chunk"], rope["grid_h"], rope["grid_w"],
                                tuple(rope.get("split", (44, 42, 42))), rope.get("theta", 10000.0))
        self.workspace = attn_fwd_workspace(self.cache) if split else None
        self.round = 0
        self.stream = stream

    def step(self, model: Callable, out: Optional[torch.Tensor] = None, with_lse: bool = False):
        """Runs the next round. Returns (plan, out, lse or None)."""
        if self.round >= self.n_rounds:
            raise StopIteration("the rollout is complete")
        plan = plan_1f1c(self.n_steps, self.n_chunks, self.hist_window, self.round)
        q, ks, vs = model(plan)
        o, l = run_round(self.cache, plan, q, ks, vs, self.scale, out=out, with_lse=with_lse, stream=self.stream,
                         workspace=self.workspace)
        self.round += 1
        return plan, o, l
