"""Python binding of libsmla: argument marshalling only.

Every function has the name of the C entry point it calls and passes torch tensors'
device pointers, strides and the current HIP stream through ctypes. torch provides
device memory and streams; every step of the computation runs in libsmla's kernels.
If libsmla.so is missing, importing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmla.so")

SMLA_F32, SMLA_BF16, SMLA_FP8_E4M3 = 0, 1, 2
LATENT, ROPE, ROW = 512, 64, 576
FP8_ROW_BYTES, FP8_ROPE_OFFSET, FP8_SCALE_OFFSET = 656, 512, 640
UNION_MAX_SLOTS = (1 << 24) - 2

STATUS = {0: "SMLA_OK", 1: "SMLA_ERR_NULL", 2: "SMLA_ERR_SHAPE", 3: "SMLA_ERR_ALIGN",
          4: "SMLA_ERR_UNSUPPORTED", 5: "SMLA_ERR_RANGE", 6: "SMLA_ERR_WORKSPACE", 7: "SMLA_ERR_DEVICE"}
STATUS_CODES = {v: k for k, v in STATUS.items()}

EXPORTS = ["smla_resolve_slots", "smla_sparse_decode_workspace", "smla_sparse_decode_workspace_init",
           "smla_sparse_decode_splits",
           "smla_sparse_decode", "smla_sparse_decode_stage1", "smla_sparse_decode_stage2",
           "smla_sparse_decode_topk", "smla_sparse_decode_topk_stage1", "smla_sparse_decode_noalloc",
           "smla_build_group_union", "smla_grouped_prefill", "smla_kv_write",
           "smla_status_str", "smla_last_error", "smla_abi_version", "smla_sizeof_kv",
           "smla_sizeof_decode_args", "smla_sizeof_prefill_args", "smla_sizeof_page_map"]


class SmlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_mla_attention_resolve_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_p, c_f32, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t


class smla_kv(ctypes.Structure):
    _fields_ = [("dtype", c_i32), ("reserved0", c_i32), ("num_slots", c_i64),
                ("rows", c_p), ("row_stride", c_i64),
                ("lat8", c_p), ("lat8_stride", c_i64),
                ("rope16", c_p), ("rope16_stride", c_i64),
                ("scale", c_p), ("scale_stride", c_i64)]


class smla_decode_args(ctypes.Structure):
    _fields_ = [("T", c_i32), ("H", c_i32), ("q_dtype", c_i32), ("page_size", c_i32),
                ("q", c_p), ("q_tok_stride", c_i64), ("q_head_stride", c_i64),
                ("kv", smla_kv),
                ("table", c_p), ("table_stride", c_i64), ("table_width", c_i32),
                ("num_splits", c_i32), ("lens", c_p), ("scale", c_f32), ("reserved0", c_i32),
                ("out", c_p), ("out_tok_stride", c_i64), ("out_head_stride", c_i64),
                ("lse", c_p), ("lse_tok_stride", c_i64)]


class smla_prefill_args(ctypes.Structure):
    _fields_ = [("Q", c_i32), ("H", c_i32), ("G", c_i32), ("enc_width", c_i32),
                ("q", c_p), ("q_tok_stride", c_i64), ("q_head_stride", c_i64),
                ("kv", smla_kv),
                ("enc", c_p), ("enc_stride", c_i64), ("lens", c_p), ("scale", c_f32),
                ("reserved1", c_i32),
                ("out", c_p), ("out_tok_stride", c_i64), ("out_head_stride", c_i64),
                ("lse", c_p), ("lse_tok_stride", c_i64)]


class smla_page_map(ctypes.Structure):
    _fields_ = [("tok_req", c_p), ("page_table", c_p), ("pt_stride", c_i64), ("seq_lens", c_p),
                ("R", c_i32), ("pt_width", c_i32), ("page_size", c_i32), ("reserved0", c_i32)]


_sig = {
    "smla_resolve_slots": [c_p, c_i64, c_p, c_p, c_i32, c_p, c_i64, c_i32, c_p, c_i32, c_i32, c_i32, c_p, c_i64, c_p],
    "smla_sparse_decode_workspace": [ctypes.POINTER(smla_decode_args), ctypes.POINTER(c_sz)],
    "smla_sparse_decode_workspace_init": [c_p, c_sz, c_p],
    "smla_sparse_decode_splits": [ctypes.POINTER(smla_decode_args), ctypes.POINTER(c_i32)],
    "smla_sparse_decode": [ctypes.POINTER(smla_decode_args), c_p, c_sz, c_p],
    "smla_sparse_decode_stage1": [ctypes.POINTER(smla_decode_args), c_p, c_sz, c_p],
    "smla_sparse_decode_stage2": [ctypes.POINTER(smla_decode_args), c_p, c_sz, c_p],
    "smla_sparse_decode_topk": [ctypes.POINTER(smla_decode_args), ctypes.POINTER(smla_page_map), c_p, c_sz, c_p],
    "smla_sparse_decode_topk_stage1": [ctypes.POINTER(smla_decode_args), ctypes.POINTER(smla_page_map), c_p, c_sz,
                                       c_p],
    "smla_sparse_decode_noalloc": [ctypes.POINTER(smla_decode_args), ctypes.POINTER(smla_page_map), c_p],
    "smla_build_group_union": [c_p, c_i64, c_p, c_i32, c_i32, c_i32, c_i64, c_p, c_i64, c_p, c_p],
    "smla_grouped_prefill": [ctypes.POINTER(smla_prefill_args), c_p],
    "smla_kv_write": [c_p, c_i32, c_i64, c_p, c_i32, ctypes.POINTER(smla_kv), c_p],
    "smla_status_str": [c_i32],
    "smla_last_error": [],
    "smla_abi_version": [],
    "smla_sizeof_kv": [], "smla_sizeof_decode_args": [], "smla_sizeof_prefill_args": [], "smla_sizeof_page_map": [],
}
for _name, _args in _sig.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_char_p if _name in ("smla_status_str", "smla_last_error") else c_i32

assert _lib.smla_sizeof_kv() == ctypes.sizeof(smla_kv), "smla_kv layout mismatch"
assert _lib.smla_sizeof_decode_args() == ctypes.sizeof(smla_decode_args), "smla_decode_args layout mismatch"
assert _lib.smla_sizeof_prefill_args() == ctypes.sizeof(smla_prefill_args), "smla_prefill_args layout mismatch"
assert _lib.smla_sizeof_page_map() == ctypes.sizeof(smla_page_map), "smla_page_map layout mismatch"


def lib():
    return _lib


def _check(status: int):
    if status != 0:
        raise SmlaError(status, _lib.smla_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _rs(t: torch.Tensor) -> int:
    """Row stride of a 2-D (or leading-dim) tensor; a single row may carry any stride."""
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t[0].numel())


def _i32(t: torch.Tensor, name: str):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


# ---------------------------------------------------------------------------------- cache

FP8_ALIGNED_ROW_BYTES = 640     # e4m3 codes (0..511) + bf16 rope (512..639): five aligned 128-byte lines


class KvCache:
    """A latent KV pool in device memory (torch-allocated) and its smla_kv descriptor.

    bf16 / f32: one [num_slots, 576] tensor.
    fp8, layout "aligned" (the default): uint8 [num_slots, 640] rows holding the e4m3 codes
    (bytes 0..511) and the bf16 rope (512..639), each row five whole 128-byte lines, and a
    separate fp32 [num_slots] scale plane.
    fp8, layout "packed": one uint8 [num_slots, 656] tensor holding the codes (0..511), the rope
    (512..639) and the scale (640..643), the SMLA_FP8_ROW_BYTES row of smla.h.
    """

    def __init__(self, dtype: int, num_slots: int, storage: torch.Tensor, scale_plane: Optional[torch.Tensor] = None):
        self.dtype = dtype
        self.num_slots = num_slots
        self.storage = storage
        self.scale_plane = scale_plane

    @staticmethod
    def empty(dtype: int, num_slots: int, device="cuda", poison: bool = True, layout: str = "aligned") -> "KvCache":
        sc = None
        if dtype == SMLA_BF16:
            st = torch.empty((num_slots, ROW), dtype=torch.bfloat16, device=device)
            if poison:
                st.fill_(float("nan"))
        elif dtype == SMLA_F32:
            st = torch.empty((num_slots, ROW), dtype=torch.float32, device=device)
            if poison:
                st.fill_(float("nan"))
        elif dtype == SMLA_FP8_E4M3:
            if layout not in ("aligned", "packed"):
                raise ValueError(layout)
            width = FP8_ALIGNED_ROW_BYTES if layout == "aligned" else FP8_ROW_BYTES
            st = torch.empty((num_slots, width), dtype=torch.uint8, device=device)
            if layout == "aligned":
                sc = torch.empty((num_slots,), dtype=torch.float32, device=device)
            if poison:
                st.fill_(0x7F)                                   # e4m3 NaN codes, NaN rope and scale
                st[:, FP8_ROPE_OFFSET:FP8_SCALE_OFFSET].view(torch.int16).fill_(0x7FC0)
                if sc is None:
                    st[:, FP8_SCALE_OFFSET:FP8_SCALE_OFFSET + 4].view(torch.float32).fill_(float("nan"))
                else:
                    sc.fill_(float("nan"))
        else:
            raise ValueError(dtype)
        return KvCache(dtype, num_slots, st, sc)

    def desc(self) -> smla_kv:
        d = smla_kv()
        d.dtype = self.dtype
        d.num_slots = self.num_slots
        base = self.storage.data_ptr()
        if self.dtype in (SMLA_BF16, SMLA_F32):
            d.rows = base
            d.row_stride = self.storage.stride(0) * self.storage.element_size()
        else:
            rs = self.storage.stride(0)
            d.lat8, d.lat8_stride = base, rs
            d.rope16, d.rope16_stride = base + FP8_ROPE_OFFSET, rs
            if self.scale_plane is None:
                d.scale, d.scale_stride = base + FP8_SCALE_OFFSET, rs
            else:
                d.scale, d.scale_stride = self.scale_plane.data_ptr(), 4
        return d

    # views of the stored planes (for tests and for building inputs)
    def lat8(self):
        return self.storage[:, :LATENT]

    def rope16(self):
        return self.storage[:, FP8_ROPE_OFFSET:FP8_SCALE_OFFSET].view(torch.int16)

    def scale(self):
        if self.scale_plane is not None:
            return self.scale_plane
        return self.storage[:, FP8_SCALE_OFFSET:FP8_SCALE_OFFSET + 4].view(torch.float32)[:, 0]


# ---------------------------------------------------------------------------------- calls

def smla_resolve_slots(idx, valid, tok_req, page_table, seq_lens, page_size: int,
                       slots: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    T, W = idx.shape
    if slots is None:
        slots = torch.empty((T, W), dtype=torch.int32, device=idx.device)
    for t, n in ((idx, "idx"), (tok_req, "tok_req"), (page_table, "page_table"), (seq_lens, "seq_lens"),
                 (slots, "slots")):
        _i32(t, n)
    if valid is not None:
        _i32(valid, "valid")
    R, ptw = page_table.shape
    _check(_lib.smla_resolve_slots(_ptr(idx), _rs(idx), _ptr(valid), _ptr(tok_req), R, _ptr(page_table),
                                   _rs(page_table), ptw, _ptr(seq_lens), page_size, T, W, _ptr(slots),
                                   _rs(slots), _stream(stream)))
    return slots


def _decode_args(q, kv: KvCache, table, lens, page_size, scale, out, lse, num_splits) -> smla_decode_args:
    a = smla_decode_args()
    T, H, D = q.shape
    assert D == ROW and q.stride(2) == 1
    a.T, a.H = T, H
    a.q_dtype = SMLA_BF16 if q.dtype == torch.bfloat16 else SMLA_F32
    a.page_size = page_size
    a.q, a.q_tok_stride, a.q_head_stride = q.data_ptr(), _rs(q), q.stride(1)
    a.kv = kv.desc()
    _i32(table, "table")
    _i32(lens, "lens")
    a.table, a.table_stride, a.table_width = table.data_ptr(), _rs(table), table.shape[1]
    a.num_splits = num_splits
    a.lens = lens.data_ptr()
    a.scale = scale
    if out is not None:
        a.out, a.out_tok_stride, a.out_head_stride = out.data_ptr(), _rs(out), out.stride(1)
    if lse is not None:
        a.lse, a.lse_tok_stride = lse.data_ptr(), _rs(lse)
    return a


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A decode workspace of at least nbytes bytes, zero-filled: its leading counter region
    must hold zeros before first use, and every decode leaves it so (see smla.h)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def smla_sparse_decode_workspace_init(workspace: torch.Tensor, stream=None):
    """Zero the merge counters of an existing workspace (a fill kernel on the stream)."""
    _check(_lib.smla_sparse_decode_workspace_init(_ptr(workspace), workspace.numel(), _stream(stream)))


def smla_sparse_decode_workspace(q, kv: KvCache, table, lens, page_size: int, scale: float,
                                 num_splits: int = 0) -> int:
    a = _decode_args(q, kv, table, lens, page_size, scale, None, None, num_splits)
    n = c_sz(0)
    _check(_lib.smla_sparse_decode_workspace(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def smla_sparse_decode_splits(q, kv: KvCache, table, lens, page_size: int, scale: float,
                              num_splits: int = 0) -> int:
    a = _decode_args(q, kv, table, lens, page_size, scale, None, None, num_splits)
    n = c_i32(0)
    _check(_lib.smla_sparse_decode_splits(ctypes.byref(a), ctypes.byref(n)))
    return n.value


def smla_sparse_decode(q, kv: KvCache, table, lens, page_size: int, scale: float,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       want_lse: bool = True, num_splits: int = 0,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Split decode (stage 1 + stage 2). q [T, H, 576] bf16 or fp32; returns (out, lse)."""
    T, H, _ = q.shape
    if out is None:
        out = torch.empty((T, H, LATENT), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    a = _decode_args(q, kv, table, lens, page_size, scale, out, lse, num_splits)
    need = c_sz(0)
    _check(_lib.smla_sparse_decode_workspace(ctypes.byref(a), ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = new_workspace(need.value, q.device)
    _check(_lib.smla_sparse_decode(ctypes.byref(a), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def _page_map(tok_req, page_table, seq_lens, page_size: int) -> smla_page_map:
    for t, n in ((tok_req, "tok_req"), (page_table, "page_table"), (seq_lens, "seq_lens")):
        _i32(t, n)
    m = smla_page_map()
    m.tok_req, m.page_table, m.pt_stride = tok_req.data_ptr(), page_table.data_ptr(), _rs(page_table)
    m.seq_lens = seq_lens.data_ptr()
    m.R, m.pt_width = page_table.shape
    m.page_size = page_size
    return m


def smla_sparse_decode_topk(q, kv: KvCache, idx, valid, tok_req, page_table, seq_lens, page_size: int,
                            scale: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            want_lse: bool = True, num_splits: int = 0,
                            workspace: Optional[torch.Tensor] = None, stream=None):
    """Decode straight from logical top-k indices idx [T, W] (valid counts `valid` [T]),
    resolved through the page table inside stage 1. Returns (out, lse)."""
    T, H, _ = q.shape
    if out is None:
        out = torch.empty((T, H, LATENT), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    a = _decode_args(q, kv, idx, valid, 1, scale, out, lse, num_splits)
    m = _page_map(tok_req, page_table, seq_lens, page_size)
    need = c_sz(0)
    _check(_lib.smla_sparse_decode_workspace(ctypes.byref(a), ctypes.byref(need)))
    if workspace is None or workspace.numel() < need.value:
        workspace = new_workspace(need.value, q.device)
    _check(_lib.smla_sparse_decode_topk(ctypes.byref(a), ctypes.byref(m), _ptr(workspace), workspace.numel(),
                                        _stream(stream)))
    return out, lse


def smla_sparse_decode_noalloc(q, kv: KvCache, table, lens, page_size: int, scale: float,
                               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                               want_lse: bool = True, num_splits: int = 0, page_map=None, stream=None):
    """The decode with the library's static workspace (no workspace argument, nothing allocated
    by the library). page_map=(tok_req, page_table, seq_lens, page_size) makes `table` logical
    top-k indices resolved inside stage 1, as smla_sparse_decode_topk. Returns (out, lse)."""
    T, H, _ = q.shape
    if out is None:
        out = torch.empty((T, H, LATENT), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    a = _decode_args(q, kv, table, lens, page_size, scale, out, lse, num_splits)
    m = None if page_map is None else ctypes.byref(_page_map(*page_map))
    _check(_lib.smla_sparse_decode_noalloc(ctypes.byref(a), m, _stream(stream)))
    return out, lse


class DecodeCall:
    """Prepared arguments for repeated decode calls on fixed tensors (no per-call allocation);
    `stage1()`, `stage2()` and `__call__()` enqueue on the current stream. With
    `page_map=(tok_req, page_table, seq_lens, page_size)` the table holds logical top-k
    indices and stage 1 resolves them (smla_sparse_decode_topk)."""

    def __init__(self, q, kv: KvCache, table, lens, page_size: int, scale: float, out, lse, num_splits: int = 0,
                 workspace: Optional[torch.Tensor] = None, page_map=None):
        self.args = _decode_args(q, kv, table, lens, page_size, scale, out, lse, num_splits)
        need = c_sz(0)
        _check(_lib.smla_sparse_decode_workspace(ctypes.byref(self.args), ctypes.byref(need)))
        if workspace is None:
            workspace = new_workspace(need.value, q.device)
        self.workspace = workspace
        self.map = None if page_map is None else _page_map(*page_map)
        self.keep = (q, kv, table, lens, out, lse, page_map)
        self.splits = smla_sparse_decode_splits(q, kv, table, lens, page_size, scale, num_splits)

    def _run(self, fn, stream):
        _check(fn(ctypes.byref(self.args), _ptr(self.workspace), self.workspace.numel(), _stream(stream)))

    def _run_map(self, fn, stream):
        _check(fn(ctypes.byref(self.args), ctypes.byref(self.map), _ptr(self.workspace), self.workspace.numel(),
                  _stream(stream)))

    def __call__(self, stream=None):
        if self.map is None:
            self._run(_lib.smla_sparse_decode, stream)
        else:
            self._run_map(_lib.smla_sparse_decode_topk, stream)

    def stage1(self, stream=None):
        if self.map is None:
            self._run(_lib.smla_sparse_decode_stage1, stream)
        else:
            self._run_map(_lib.smla_sparse_decode_topk_stage1, stream)

    def stage2(self, stream=None):
        self._run(_lib.smla_sparse_decode_stage2, stream)


def smla_build_group_union(slots, valid, G: int, num_slots: int, enc: Optional[torch.Tensor] = None,
                           lens: Optional[torch.Tensor] = None, stream=None):
    _i32(slots, "slots")
    Q, W = slots.shape
    ng = -(-Q // G)
    if enc is None:
        enc = torch.empty((ng, G * W), dtype=torch.int32, device=slots.device)
    if lens is None:
        lens = torch.empty((ng,), dtype=torch.int32, device=slots.device)
    if valid is not None:
        _i32(valid, "valid")
    _check(_lib.smla_build_group_union(_ptr(slots), _rs(slots), _ptr(valid), Q, W, G, num_slots,
                                       _ptr(enc), _rs(enc), _ptr(lens), _stream(stream)))
    return enc, lens


def smla_grouped_prefill(q, kv: KvCache, enc, lens, G: int, scale: float,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         want_lse: bool = True, stream=None):
    Q, H, D = q.shape
    assert D == ROW and q.stride(2) == 1
    if out is None:
        out = torch.empty((Q, H, LATENT), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Q, H), dtype=torch.float32, device=q.device)
    a = smla_prefill_args()
    a.Q, a.H, a.G, a.enc_width = Q, H, G, enc.shape[1]
    a.q, a.q_tok_stride, a.q_head_stride = q.data_ptr(), _rs(q), q.stride(1)
    a.kv = kv.desc()
    a.enc, a.enc_stride = enc.data_ptr(), _rs(enc)
    _i32(lens, "lens")
    a.lens = lens.data_ptr()
    a.scale = scale
    a.out, a.out_tok_stride, a.out_head_stride = out.data_ptr(), _rs(out), out.stride(1)
    if lse is not None:
        a.lse, a.lse_tok_stride = lse.data_ptr(), _rs(lse)
    _check(_lib.smla_grouped_prefill(ctypes.byref(a), _stream(stream)))
    return out, lse


def smla_kv_write(src: torch.Tensor, slot_mapping: torch.Tensor, kv: KvCache, stream=None):
    T = src.shape[0]
    assert src.shape[1] == ROW and src.stride(1) == 1
    sd = SMLA_F32 if src.dtype == torch.float32 else SMLA_BF16
    _i32(slot_mapping, "slot_mapping")
    d = kv.desc()
    _check(_lib.smla_kv_write(_ptr(src), sd, _rs(src), _ptr(slot_mapping), T, ctypes.byref(d),
                              _stream(stream)))
    return kv
