"""ctypes binding over libmoe.so (include/moe.h): argument marshalling only.

Every step of the layer runs in the library's HIP kernels. PyTorch supplies
device memory and the current stream; outputs the caller does not pass are
allocated with torch before the call. If the library is missing the first
call raises: there is no other implementation to fall back to.
"""
import ctypes
import os
import re
from ctypes import c_int, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_EHIP = 0, -1, -2
FMT_FP8_E4M3_ROW, FMT_INT4_G128 = 0, 1
ACT_BF16, ACT_FP8_G128_POW2 = 0, 1


class MoeError(RuntimeError):
    pass


class moe_slot_pool(ctypes.Structure):
    _fields_ = [("d_base", c_void_p), ("slot_bytes", c_size_t), ("n_slots", c_int),
                ("d_slot_fmt", c_void_p), ("hidden", c_int), ("inter", c_int)]


_lib = None


def _declare(lib):
    P = c_void_p
    sig = {
        "moe_abi_version": (c_int, []),
        "moe_strerror": (ctypes.c_char_p, [c_int]),
        "moe_last_hip_error": (c_int, []),
        "moe_route": (c_int, [P, P, c_int, c_int, c_int, P, P, P, P]),
        "moe_align_capacity": (c_int, [c_int, c_int, c_int, c_int]),
        "moe_route_gemm": (c_int, [P, P, P, P, c_int, c_int, c_int, c_int, P, P, P, P, P]),
        "moe_align_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
        "moe_align": (c_int, [P, c_int, c_int, c_int, c_int, P, P, P, P, P, P, P, P, c_size_t, P]),
        "moe_route_align_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
        "moe_route_align": (c_int, [P, P, c_int, c_int, c_int, c_int, P, P, P, P, P, P, P, P, P, P, c_size_t, P]),
        "moe_slot_bytes": (c_size_t, [c_int, c_int, c_int]),
        "moe_slot_part_offset": (c_size_t, [c_int, c_int, c_int, c_int]),
        "moe_ffn_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
        "moe_expert_ffn": (c_int, [ctypes.POINTER(moe_slot_pool), P, c_int, c_int, c_int, P, P, P, P,
                                   c_int, c_int, P, P, c_size_t, P]),
        "moe_pager_create": (c_void_p, [c_int, c_int, c_int]),
        "moe_pager_destroy": (None, [c_void_p]),
        "moe_pager_plan": (c_int, [c_void_p, c_int, P, c_int, P, P, P, ctypes.POINTER(c_int)]),
        "moe_pager_stats": (c_int, [c_void_p, c_int, ctypes.POINTER(ctypes.c_longlong),
                                    ctypes.POINTER(ctypes.c_longlong)]),
        "moe_pager_fill": (c_int, [ctypes.POINTER(moe_slot_pool), P, c_size_t, P, P, P, c_int, P]),
        "moe_fp8_pack_bound": (c_size_t, [c_int, c_int]),
        "moe_fp8_pack": (c_size_t, [P, c_int, c_int, P, c_size_t]),
        "moe_fp8_unpack": (c_int, [ctypes.POINTER(moe_slot_pool), P, c_int, P, P]),
        "moe_pager_fill_packed": (c_int, [ctypes.POINTER(moe_slot_pool), P, P, P, P, P, c_int, P, c_size_t, P, P]),
        "moe_expert_ffn_pass": (c_int, [ctypes.POINTER(moe_slot_pool), P, c_int, c_int, c_int, P, P, P, P,
                                        c_int, c_int, c_int, P, P, c_size_t, P]),
        "moe_layer_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int, c_int]),
        "moe_layer_noalloc": (c_int, [ctypes.POINTER(moe_slot_pool), P, P, P, c_int, c_int, c_int, c_int, c_int,
                                      P, P, P, P, P, P, P, P, P, P, P]),
        "moe_layer": (c_int, [ctypes.POINTER(moe_slot_pool), P, P, P, c_int, c_int, c_int, c_int, c_int, P,
                              P, P, P, P, P, P, P, P, P, P, c_size_t, P]),
        "moe_dequant_slot": (c_int, [ctypes.POINTER(moe_slot_pool), c_int, P, P, P]),
        "moe_quant_act": (c_int, [P, c_int, c_int, P, P, P]),
        "moe_pool_check": (c_int, [ctypes.POINTER(moe_slot_pool), P, P, P]),
        "moe_debug_poison": (c_int, [c_int]),
        "moe_bitwidth_plan": (c_int, [P, c_int, c_int, P]),
        "moe_requant_slot": (c_int, [ctypes.POINTER(moe_slot_pool), c_int, c_int, P, P]),
        "moe_profile_enable": (c_int, [c_int]),
        "moe_profile_kernels": (c_int, []),
        "moe_profile_kernel_name": (ctypes.c_char_p, [c_int]),
        "moe_profile_read": (c_int, [c_int, ctypes.POINTER(c_int), ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(python -m moe_expert_layer_topk_amd.build)")
        # torch ships its own HIP runtime (same soname as ROCm's). Load torch
        # first so the library binds to that runtime instead of pulling in a
        # second one, which would see no device.
        import torch  # noqa: F401
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def declared_symbols():
    """Function names declared in include/moe.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def _check(status):
    if status != MOE_OK:
        L = lib()
        msg = L.moe_strerror(status).decode()
        raise MoeError(f"libmoe: {msg} (status {status}, hip error {L.moe_last_hip_error()})")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _ptr(t, dtype=None, numel=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise MoeError(f"{name} holds {t.numel()} elements, needs {numel}")
    return c_void_p(t.data_ptr())


# ---------------------------------------------------------------- route
def route(logits, k, mask=None, ids=None, w=None, err=None, stream=None):
    import torch
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    _check(lib().moe_route(_ptr(logits, torch.float32, T * E, "logits"),
                           _ptr(mask, torch.uint8, E, "mask"), T, E, k,
                           _ptr(ids, torch.int32, T * k, "ids"), _ptr(w, torch.float32, T * k, "w"),
                           _ptr(err, torch.int32, 1, "err"), _stream(stream)))
    return ids, w, err


def route_gemm(x, W_g, k, bias=None, mask=None, logits=None, ids=None, w=None, err=None, stream=None):
    """moe_route_gemm: router gate GEMM then top-k. Returns (logits, ids, w, err)."""
    import torch
    T, H = x.shape
    E = W_g.shape[0]
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if logits is None else logits
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    _check(lib().moe_route_gemm(_ptr(x, torch.bfloat16, T * H, "x"), _ptr(W_g, torch.float32, E * H, "W_g"),
                                _ptr(bias, torch.float32, E, "bias"), _ptr(mask, torch.uint8, E, "mask"), T, H, E, k,
                                _ptr(logits, torch.float32, T * E, "logits"), _ptr(ids, torch.int32, T * k, "ids"),
                                _ptr(w, torch.float32, T * k, "w"), _ptr(err, torch.int32, 1, "err"), _stream(stream)))
    return logits, ids, w, err


# ---------------------------------------------------------------- align
def align_capacity(T, k, E, block_m):
    cap = lib().moe_align_capacity(T, k, E, block_m)
    if cap < 0:
        _check(cap)
    return cap


def align_workspace_bytes(T, k, E, block_m):
    return int(lib().moe_align_workspace_bytes(T, k, E, block_m))


def align(ids, E, block_m, slot_of_expert, out=None, err=None, ws=None, stream=None):
    """Returns dict(sorted_pair, block_slot, counts, seg_offset, n_padded, err)."""
    import torch
    T, k = ids.shape
    dev = ids.device
    cap = align_capacity(T, k, E, block_m)
    if out is None:
        out = _align_out(T, k, E, block_m, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    need = align_workspace_bytes(T, k, E, block_m)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().moe_align(_ptr(ids, torch.int32, T * k, "ids"), T, k, E, block_m,
                           _ptr(slot_of_expert, torch.int32, E, "slot_of_expert"),
                           _ptr(out["sorted_pair"], torch.int32, cap, "sorted_pair"),
                           _ptr(out["block_slot"], torch.int32, cap // block_m, "block_slot"),
                           _ptr(out["counts"], torch.int32, E, "counts"),
                           _ptr(out["seg_offset"], torch.int32, E + 1, "seg_offset"),
                           _ptr(out["n_padded"], torch.int32, 1, "n_padded"),
                           _ptr(err, torch.int32, 1, "err"),
                           _ptr(ws, torch.uint8, need, "ws") if need else None,
                           c_size_t(need), _stream(stream)))
    out = dict(out)
    out["err"] = err
    return out


def _align_out(T, k, E, block_m, dev):
    import torch
    cap = align_capacity(T, k, E, block_m)
    return dict(sorted_pair=torch.empty(cap, dtype=torch.int32, device=dev),
                block_slot=torch.empty(cap // block_m, dtype=torch.int32, device=dev),
                counts=torch.empty(E, dtype=torch.int32, device=dev),
                seg_offset=torch.empty(E + 1, dtype=torch.int32, device=dev),
                n_padded=torch.empty(1, dtype=torch.int32, device=dev))


def route_align_workspace_bytes(T, k, E, block_m):
    return int(lib().moe_route_align_workspace_bytes(T, k, E, block_m))


def route_align(logits, k, block_m, slot_of_expert, mask=None, ids=None, w=None, out=None, err=None, ws=None,
                stream=None):
    """moe_route + moe_align in one call. Returns (ids, w, aligned dict); the
    aligned dict's "err" is i32[2] (route count, align count)."""
    import torch
    T, E = logits.shape
    dev = logits.device
    cap = align_capacity(T, k, E, block_m)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    out = _align_out(T, k, E, block_m, dev) if out is None else out
    err = torch.zeros(2, dtype=torch.int32, device=dev) if err is None else err
    need = route_align_workspace_bytes(T, k, E, block_m)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(lib().moe_route_align(_ptr(logits, torch.float32, T * E, "logits"), _ptr(mask, torch.uint8, E, "mask"),
                                 T, E, k, block_m, _ptr(slot_of_expert, torch.int32, E, "slot_of_expert"),
                                 _ptr(ids, torch.int32, T * k, "ids"), _ptr(w, torch.float32, T * k, "w"),
                                 _ptr(out["sorted_pair"], torch.int32, cap, "sorted_pair"),
                                 _ptr(out["block_slot"], torch.int32, cap // block_m, "block_slot"),
                                 _ptr(out["counts"], torch.int32, E, "counts"),
                                 _ptr(out["seg_offset"], torch.int32, E + 1, "seg_offset"),
                                 _ptr(out["n_padded"], torch.int32, 1, "n_padded"),
                                 _ptr(err, torch.int32, 2, "err"),
                                 _ptr(ws, torch.uint8, need, "ws") if need else None, c_size_t(need),
                                 _stream(stream)))
    out = dict(out)
    out["err"] = err
    return ids, w, out


# ---------------------------------------------------------------- slot pool
def slot_bytes(hidden, inter, fmt):
    return int(lib().moe_slot_bytes(hidden, inter, fmt))


def slot_part_offset(hidden, inter, fmt, part):
    return int(lib().moe_slot_part_offset(hidden, inter, fmt, part))


class SlotPool:
    """A layer's VRAM slot pool: uint8 device tensor [n_slots, stride] plus the
    per-slot format tags (device uint8 [n_slots])."""

    def __init__(self, data, fmt, hidden, inter):
        self.data, self.fmt, self.hidden, self.inter = data, fmt, hidden, inter
        self._c = moe_slot_pool(c_void_p(data.data_ptr()), data.shape[1], data.shape[0],
                                c_void_p(fmt.data_ptr()), hidden, inter)

    @property
    def n_slots(self):
        return self.data.shape[0]

    def c_ref(self):
        return ctypes.byref(self._c)


# ---------------------------------------------------------------- expert FFN
def ffn_workspace_bytes(T, k, E, hidden, inter, block_m, act_mode):
    return int(lib().moe_ffn_workspace_bytes(T, k, E, hidden, inter, block_m, act_mode))


def expert_ffn(pool, x, k, E, topk_w, aligned, block_m, act_mode, out=None, ws=None, stream=None):
    import torch
    T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    need = ffn_workspace_bytes(T, k, E, pool.hidden, pool.inter, block_m, act_mode)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    cap = align_capacity(T, k, E, block_m)
    _check(lib().moe_expert_ffn(pool.c_ref(), _ptr(x, torch.bfloat16, T * H, "x"), T, k, E,
                                _ptr(topk_w, torch.float32, T * k, "topk_w"),
                                _ptr(aligned["sorted_pair"], torch.int32, cap, "sorted_pair"),
                                _ptr(aligned["block_slot"], torch.int32, cap // block_m, "block_slot"),
                                _ptr(aligned["n_padded"], torch.int32, 1, "n_padded"),
                                block_m, act_mode, _ptr(out, torch.bfloat16, T * H, "out"),
                                _ptr(ws, torch.uint8, need, "ws"), c_size_t(ws.numel()), _stream(stream)))
    return out


SLOT_DEFERRED = -2


class Pager:
    """moe_pager: per-layer LRU over VRAM slots (host logic in the library)."""

    def __init__(self, n_layers, E, n_slots):
        self.E, self.n_slots = E, n_slots
        self._p = lib().moe_pager_create(n_layers, E, n_slots)
        if not self._p:
            raise MoeError("moe_pager_create: bad sizes")

    def __del__(self):
        if getattr(self, "_p", None):
            lib().moe_pager_destroy(self._p)
            self._p = None

    def plan(self, layer, needed):
        """needed: host int array. Returns (slot_of_expert [E], fill_expert, fill_slot) as numpy int32."""
        import numpy as np
        nd = np.ascontiguousarray(needed, dtype=np.int32).reshape(-1)
        table = np.empty(self.E, dtype=np.int32)
        fe = np.empty(max(self.n_slots, 1), dtype=np.int32)
        fs = np.empty(max(self.n_slots, 1), dtype=np.int32)
        n = c_int(0)
        _check(lib().moe_pager_plan(self._p, layer, nd.ctypes.data_as(c_void_p), nd.size,
                                    table.ctypes.data_as(c_void_p), fe.ctypes.data_as(c_void_p),
                                    fs.ctypes.data_as(c_void_p), ctypes.byref(n)))
        return table, fe[:n.value].copy(), fs[:n.value].copy()

    def stats(self, layer=-1):
        h, m = ctypes.c_longlong(0), ctypes.c_longlong(0)
        _check(lib().moe_pager_stats(self._p, layer, ctypes.byref(h), ctypes.byref(m)))
        return h.value, m.value


def fp8_pack(slot_bytes_u8, hidden, inter):
    """moe_fp8_pack on a host numpy FP8 slot -> packed numpy uint8."""
    import numpy as np
    src = np.ascontiguousarray(slot_bytes_u8, dtype=np.uint8)
    cap = int(lib().moe_fp8_pack_bound(hidden, inter))
    if cap == 0:
        raise MoeError("moe_fp8_pack: hidden and inter must be multiples of 256")
    out = np.empty(cap, dtype=np.uint8)
    n = int(lib().moe_fp8_pack(src.ctypes.data_as(c_void_p), hidden, inter, out.ctypes.data_as(c_void_p), cap))
    if n == 0:
        raise MoeError("moe_fp8_pack failed")
    return out[:n].copy()


def fp8_unpack(pool, packed_dev, dst_slot, err=None, stream=None):
    import torch
    _check(lib().moe_fp8_unpack(pool.c_ref(), _ptr(packed_dev, torch.uint8, 32, "packed"), int(dst_slot),
                                _ptr(err, torch.int32, 1, "err") if err is not None else None, _stream(stream)))


def pager_fill_packed(pool, h_packed, offsets, sizes, fill_src, fill_slot, staging, copy_stream, err=None):
    """moe_pager_fill_packed: h_packed pinned uint8 (all packed rows back to back),
    offsets / sizes numpy uint64 per bank row; staging a device uint8 buffer."""
    import numpy as np
    import torch
    if not h_packed.is_pinned():
        raise MoeError("the packed host bank must be page-locked (pin_memory=True)")
    off = np.ascontiguousarray(offsets, dtype=np.uint64)
    siz = np.ascontiguousarray(sizes, dtype=np.uint64)
    src = np.ascontiguousarray(fill_src, dtype=np.int32)
    dst = np.ascontiguousarray(fill_slot, dtype=np.int32)
    _check(lib().moe_pager_fill_packed(pool.c_ref(), c_void_p(h_packed.data_ptr()), off.ctypes.data_as(c_void_p),
                                       siz.ctypes.data_as(c_void_p), src.ctypes.data_as(c_void_p),
                                       dst.ctypes.data_as(c_void_p), int(src.size), _ptr(staging, torch.uint8),
                                       staging.numel(), _ptr(err, torch.int32, 1, "err") if err is not None else None,
                                       c_void_p(copy_stream.cuda_stream)))


def pager_fill(pool, h_bank, h_bank_fmt, fill_src, fill_slot, copy_stream):
    """moe_pager_fill: h_bank pinned uint8 [rows, stride], h_bank_fmt pinned uint8 [rows];
    fill_src / fill_slot host int arrays."""
    import numpy as np
    src = np.ascontiguousarray(fill_src, dtype=np.int32)
    dst = np.ascontiguousarray(fill_slot, dtype=np.int32)
    if not (h_bank.is_pinned() and h_bank_fmt.is_pinned()):
        raise MoeError("host bank and format tags must be page-locked (pin_memory=True)")
    _check(lib().moe_pager_fill(pool.c_ref(), c_void_p(h_bank.data_ptr()), h_bank.shape[1],
                                c_void_p(h_bank_fmt.data_ptr()), src.ctypes.data_as(c_void_p),
                                dst.ctypes.data_as(c_void_p), int(src.size), c_void_p(copy_stream.cuda_stream)))


def expert_ffn_pass(pool, x, k, E, topk_w, aligned, block_m, act_mode, last_pass, out, ws, stream=None):
    """moe_expert_ffn_pass: blocks whose slot is SLOT_DEFERRED are left alone;
    the combine into out runs only when last_pass. ws must persist between
    the passes of one sequence."""
    import torch
    T, H = x.shape
    need = ffn_workspace_bytes(T, k, E, pool.hidden, pool.inter, block_m, act_mode)
    cap = align_capacity(T, k, E, block_m)
    _check(lib().moe_expert_ffn_pass(pool.c_ref(), _ptr(x, torch.bfloat16, T * H, "x"), T, k, E,
                                     _ptr(topk_w, torch.float32, T * k, "topk_w"),
                                     _ptr(aligned["sorted_pair"], torch.int32, cap, "sorted_pair"),
                                     _ptr(aligned["block_slot"], torch.int32, cap // block_m, "block_slot"),
                                     _ptr(aligned["n_padded"], torch.int32, 1, "n_padded"),
                                     block_m, act_mode, 1 if last_pass else 0,
                                     _ptr(out, torch.bfloat16, T * H, "out"), _ptr(ws, torch.uint8, need, "ws"),
                                     c_size_t(ws.numel()), _stream(stream)))
    return out


def dequant_slot(pool, slot, w13=None, w2=None, stream=None):
    import torch
    H, I = pool.hidden, pool.inter
    dev = pool.data.device
    w13 = torch.empty((2 * I, H), dtype=torch.float32, device=dev) if w13 is None else w13
    w2 = torch.empty((H, I), dtype=torch.float32, device=dev) if w2 is None else w2
    _check(lib().moe_dequant_slot(pool.c_ref(), slot, _ptr(w13, torch.float32, 2 * I * H, "w13"),
                                  _ptr(w2, torch.float32, H * I, "w2"), _stream(stream)))
    return w13, w2


def quant_act(x, codes=None, exps=None, stream=None):
    """moe_quant_act: e4m3 codes uint8 [rows, cols] and E8M0 bytes uint8 [rows, cols / 128]."""
    import torch
    R, C = x.shape
    codes = torch.empty((R, C), dtype=torch.uint8, device=x.device) if codes is None else codes
    exps = torch.empty((R, C // 128), dtype=torch.uint8, device=x.device) if exps is None else exps
    _check(lib().moe_quant_act(_ptr(x, torch.bfloat16, R * C, "x"), R, C, _ptr(codes, torch.uint8, R * C, "codes"),
                               _ptr(exps, torch.uint8, R * (C // 128), "exps"), _stream(stream)))
    return codes, exps


def pool_check(pool, err=None, status=None, stream=None):
    """moe_pool_check: (err i32[1], status u8[n_slots]) on the device."""
    import torch
    dev = pool.data.device
    err = torch.zeros(1, dtype=torch.int32, device=dev) if err is None else err
    status = torch.empty(pool.n_slots, dtype=torch.uint8, device=dev) if status is None else status
    _check(lib().moe_pool_check(pool.c_ref(), _ptr(err, torch.int32, 1, "err"),
                                _ptr(status, torch.uint8, pool.n_slots, "status"), _stream(stream)))
    return err, status


def bitwidth_plan(counts, n_int4):
    """moe_bitwidth_plan on host arrays: counts int32 [E] -> uint8 [E] of formats."""
    import numpy as np
    c = np.ascontiguousarray(counts, dtype=np.int32)
    out = np.empty(c.size, dtype=np.uint8)
    _check(lib().moe_bitwidth_plan(c.ctypes.data_as(c_void_p), c.size, int(n_int4), out.ctypes.data_as(c_void_p)))
    return out


def requant_slot(pool, src_slot, dst_slot, err=None, stream=None):
    import torch
    _check(lib().moe_requant_slot(pool.c_ref(), int(src_slot), int(dst_slot),
                                  _ptr(err, torch.int32, 1, "err") if err is not None else None, _stream(stream)))


def debug_poison(on=True):
    _check(lib().moe_debug_poison(1 if on else 0))


# ---------------------------------------------------------------- tracing
def profile_enable(on=True):
    _check(lib().moe_profile_enable(1 if on else 0))


def profile_read():
    """{kernel name: (launches, total ms)} for kernels launched since enable."""
    L = lib()
    out = {}
    for i in range(L.moe_profile_kernels()):
        n, ms = c_int(0), ctypes.c_double(0.0)
        _check(L.moe_profile_read(i, ctypes.byref(n), ctypes.byref(ms)))
        if n.value:
            out[L.moe_profile_kernel_name(i).decode()] = (n.value, ms.value)
    return out


# ---------------------------------------------------------------- whole layer
def layer_workspace_bytes(T, k, E, hidden, inter, block_m, act_mode):
    return int(lib().moe_layer_workspace_bytes(T, k, E, hidden, inter, block_m, act_mode))


def layer_call(pool, x, logits, k, slot_of_expert, block_m, act_mode, mask=None, ids=None, w=None, aligned=None,
               err=None, out=None, ws=None, stream=None):
    """moe_layer: route, align and expert FFN in one call. Returns (out, ids,
    w, aligned dict); the aligned dict's "err" is i32[2] (route count, align
    count)."""
    import torch
    T, H = x.shape
    E = logits.shape[1]
    dev = x.device
    cap = align_capacity(T, k, E, block_m)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    aligned = _align_out(T, k, E, block_m, dev) if aligned is None else aligned
    err = torch.zeros(2, dtype=torch.int32, device=dev) if err is None else err
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    need = layer_workspace_bytes(T, k, E, pool.hidden, pool.inter, block_m, act_mode)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib().moe_layer(pool.c_ref(), _ptr(logits, torch.float32, T * E, "logits"),
                           _ptr(mask, torch.uint8, E, "mask"), _ptr(x, torch.bfloat16, T * H, "x"), T, E, k,
                           block_m, act_mode, _ptr(slot_of_expert, torch.int32, E, "slot_of_expert"),
                           _ptr(ids, torch.int32, T * k, "ids"), _ptr(w, torch.float32, T * k, "w"),
                           _ptr(aligned["sorted_pair"], torch.int32, cap, "sorted_pair"),
                           _ptr(aligned["block_slot"], torch.int32, cap // block_m, "block_slot"),
                           _ptr(aligned["counts"], torch.int32, E, "counts"),
                           _ptr(aligned["seg_offset"], torch.int32, E + 1, "seg_offset"),
                           _ptr(aligned["n_padded"], torch.int32, 1, "n_padded"),
                           _ptr(err, torch.int32, 2, "err"), _ptr(out, torch.bfloat16, T * H, "out"),
                           _ptr(ws, torch.uint8, need, "ws"), c_size_t(ws.numel()), _stream(stream)))
    aligned = dict(aligned)
    aligned["err"] = err
    return out, ids, w, aligned


def layer_call_noalloc(pool, x, logits, k, slot_of_expert, block_m, act_mode, mask=None, ids=None, w=None,
                       aligned=None, err=None, out=None, stream=None):
    """moe_layer_noalloc: moe_layer with the library's built-in scratch as its
    workspace. Returns (out, ids, w, aligned dict) like layer_call."""
    import torch
    T, H = x.shape
    E = logits.shape[1]
    dev = x.device
    cap = align_capacity(T, k, E, block_m)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    aligned = _align_out(T, k, E, block_m, dev) if aligned is None else aligned
    err = torch.zeros(2, dtype=torch.int32, device=dev) if err is None else err
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    _check(lib().moe_layer_noalloc(pool.c_ref(), _ptr(logits, torch.float32, T * E, "logits"),
                                   _ptr(mask, torch.uint8, E, "mask"), _ptr(x, torch.bfloat16, T * H, "x"), T, E, k,
                                   block_m, act_mode, _ptr(slot_of_expert, torch.int32, E, "slot_of_expert"),
                                   _ptr(ids, torch.int32, T * k, "ids"), _ptr(w, torch.float32, T * k, "w"),
                                   _ptr(aligned["sorted_pair"], torch.int32, cap, "sorted_pair"),
                                   _ptr(aligned["block_slot"], torch.int32, cap // block_m, "block_slot"),
                                   _ptr(aligned["counts"], torch.int32, E, "counts"),
                                   _ptr(aligned["seg_offset"], torch.int32, E + 1, "seg_offset"),
                                   _ptr(aligned["n_padded"], torch.int32, 1, "n_padded"),
                                   _ptr(err, torch.int32, 2, "err"), _ptr(out, torch.bfloat16, T * H, "out"),
                                   _stream(stream)))
    aligned = dict(aligned)
    aligned["err"] = err
    return out, ids, w, aligned


def layer(pool, x, logits, k, slot_of_expert, block_m, act_mode, mask=None, stream=None, fused=False):
    """route -> align -> expert FFN on one stream; returns (out, route, align).
    fused=False: moe_route, moe_align, moe_expert_ffn; fused=True: moe_route_align
    then moe_expert_ffn; fused="layer": moe_layer. With fused set, the route
    error count is returned as route[2] and align's as aligned["err"]."""
    E = logits.shape[1]
    if fused == "layer":
        out, ids, w, al = layer_call(pool, x, logits, k, slot_of_expert, block_m, act_mode, mask=mask,
                                     stream=stream)
        rerr = al["err"][0:1]
        al["err"] = al["err"][1:2]
        return out, (ids, w, rerr), al
    if fused:
        ids, w, al = route_align(logits, k, block_m, slot_of_expert, mask=mask, stream=stream)
        rerr = al["err"][0:1]
        al["err"] = al["err"][1:2]
    else:
        ids, w, rerr = route(logits, k, mask=mask, stream=stream)
        al = align(ids, E, block_m, slot_of_expert, stream=stream)
    out = expert_ffn(pool, x, k, E, w, al, block_m, act_mode, stream=stream)
    return out, (ids, w, rerr), al
