"""Python binding of libbgtq (Block-GTQ packed-KV path for MI355X).

Argument marshalling only: every step runs in the HIP library.  Device
tensors are torch tensors on a ROCm device (torch supplies device memory and
streams); the library is loaded from this directory and the binding raises if
it is missing.  Function names follow include/bgtq.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbgtq.so")

OK, EINVAL, EBUDGET, ECAPACITY, EDEVICE, EWORKSPACE = 0, -1, -2, -3, -4, -5
TILE = 64
HEAD_DIM = 128
ROPE_PAIRINGS = {"half": 0, "interleaved": 1}  # half-split (j, j+64), interleaved (2j, 2j+1)

EXPORTED = [
    "bgtq_abi_version", "bgtq_last_error", "bgtq_energy", "bgtq_allocate", "bgtq_allocate_device",
    "bgtq_plan_create",
    "bgtq_plan_destroy", "bgtq_plan_sizes", "bgtq_plan_upload", "bgtq_encode_k", "bgtq_encode_v",
    "bgtq_rotate_queries", "bgtq_decode_workspace_size", "bgtq_decode_attn", "bgtq_codebook",
    "bgtq_plan_rotation", "bgtq_plan_bits", "bgtq_profile_enable", "bgtq_profile_read", "bgtq_decode_step",
    "bgtq_fp16_decode_workspace_size", "bgtq_fp16_decode_attn", "bgtq_decode_attn_buffered",
    "bgtq_buffer_append", "bgtq_encode_k_paged", "bgtq_encode_v_paged", "bgtq_decode_attn_paged",
    "bgtq_decode_step_paged", "bgtq_noalloc_scratch_bytes", "bgtq_decode_attn_noalloc", "bgtq_key_logits",
    "bgtq_encode_kv", "bgtq_encode_kv_paged", "bgtq_decode_attn_paged_buffered", "bgtq_decode_step_buffered",
]


class BgtqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("bgtq status %d: %s" % (status, msg))
        self.status = status


class _PlanDesc(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("k_avg_bits", ctypes.c_int32),
                ("v_bits", ctypes.c_int32), ("k_bits", ctypes.POINTER(ctypes.c_int8)),
                ("seed", ctypes.c_uint64), ("layer", ctypes.c_int32), ("rope_pairing", ctypes.c_int32)]


class _Pages(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("n_pages", ctypes.c_int32)]


class _Sizes(ctypes.Structure):
    _fields_ = [("consts", ctypes.c_uint64), ("k_codes", ctypes.c_uint64),
                ("k_norms", ctypes.c_uint64), ("v_codes", ctypes.c_uint64),
                ("v_norms", ctypes.c_uint64)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libbgtq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libbgtq.so is not built (run __graft_entry__.build())")
    # torch first: torch ships its own HIP runtime under the same soname as the
    # system one that libbgtq.so links, and the first one loaded serves the whole
    # process; the library must use torch's, which owns the memory and streams.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I32, I64, U64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    sig = {
        "bgtq_abi_version": (I32, []),
        "bgtq_last_error": (ctypes.c_char_p, []),
        "bgtq_energy": (I32, [P, P, I64, I32, I32, I32, I32, P, P]),
        "bgtq_allocate": (I32, [P, I32, I32, I32, P]),
        "bgtq_allocate_device": (I32, [P, I32, I32, I32, P, P]),
        "bgtq_plan_create": (I32, [ctypes.POINTER(_PlanDesc), ctypes.POINTER(P)]),
        "bgtq_plan_destroy": (None, [P]),
        "bgtq_plan_sizes": (I32, [P, I32, I64, ctypes.POINTER(_Sizes)]),
        "bgtq_plan_upload": (I32, [P, P, P]),
        "bgtq_encode_k": (I32, [P, P, P, I32, I64, I64, I64, P, P, P]),
        "bgtq_encode_v": (I32, [P, P, P, I32, I64, I64, I64, P, P, P]),
        "bgtq_rotate_queries": (I32, [P, P, P, I32, P, P]),
        "bgtq_key_logits": (I32, [P, P, P, I32, P, P, I64, I32, I64, I64, P, P]),
        "bgtq_decode_workspace_size": (I32, [P, I32, I64, ctypes.POINTER(SZ)]),
        "bgtq_decode_attn": (I32, [P, P, P, P, P, P, P, I64, P, I32, I64, ctypes.c_float, P, P, SZ, P]),
        "bgtq_decode_step": (I32, [P, P, P, P, P, P, I32, I64, P, P, P, P, I64, ctypes.c_float, P, P, SZ, P]),
        "bgtq_codebook": (I32, [I32, P, P, P]),
        "bgtq_plan_rotation": (I32, [P, I32, I32, I32, P, ctypes.POINTER(I32)]),
        "bgtq_plan_bits": (I32, [P, P]),
        "bgtq_profile_enable": (I32, [I32]),
        "bgtq_profile_read": (I32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]),
        "bgtq_fp16_decode_workspace_size": (I32, [I32, I32, I32, I64, ctypes.POINTER(SZ)]),
        "bgtq_fp16_decode_attn": (I32, [P, P, P, I32, I32, I32, I64, P, I64, ctypes.c_float, P, P, SZ, P]),
        "bgtq_decode_attn_buffered": (I32, [P, P, P, P, P, P, P, I64, P, I32, I64, ctypes.c_float,
                                            P, P, I32, P, P, I32, P, P, SZ, P]),
        "bgtq_buffer_append": (I32, [P, P, I32, I64, I64, I32, P, P, I32, P, P, I32, P]),
        "bgtq_encode_kv": (I32, [P, P, P, P, I32, I64, I64, I64, P, P, P, P, P]),
        "bgtq_encode_kv_paged": (I32, [P, P, P, P, I32, ctypes.POINTER(_Pages), I64, I64, P, P, P, P, P]),
        "bgtq_encode_k_paged": (I32, [P, P, P, I32, ctypes.POINTER(_Pages), I64, I64, P, P, P]),
        "bgtq_encode_v_paged": (I32, [P, P, P, I32, ctypes.POINTER(_Pages), I64, I64, P, P, P]),
        "bgtq_decode_attn_paged": (I32, [P, P, P, P, P, P, P, ctypes.POINTER(_Pages), P, I32, I64,
                                         ctypes.c_float, P, P, SZ, P]),
        "bgtq_decode_attn_paged_buffered": (I32, [P, P, P, P, P, P, P, ctypes.POINTER(_Pages), P, I32, I64,
                                                  ctypes.c_float, P, P, I32, P, P, I32, P, P, SZ, P]),
        "bgtq_decode_step_buffered": (I32, [P, P, P, P, P, P, I32, I64, P, P, P, P, I64, ctypes.c_float,
                                            P, P, I32, P, P, I32, P, P, SZ, P]),
        "bgtq_decode_step_paged": (I32, [P, P, P, P, P, P, I32, I64, P, P, P, P, ctypes.POINTER(_Pages),
                                         ctypes.c_float, P, P, SZ, P]),
        "bgtq_noalloc_scratch_bytes": (SZ, []),
        "bgtq_decode_attn_noalloc": (I32, [P, P, P, P, P, P, P, I64, P, I32, I64, ctypes.c_float, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != OK:
        raise BgtqError(status, load().bgtq_last_error().decode())


def _need(t, name: str, *, elem: int | None = None, dtype=None, shape=None, device: bool = False) -> None:
    """Check a tensor argument before its address crosses the ABI (the C side cannot tell a
    strided view, a wrong element type or a host tensor from a valid device buffer).
    ``shape`` is a tuple whose None entries match any size."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must have dtype %s (got %s)" % (name, dtype, t.dtype))
    if elem is not None and t.element_size() != elem:
        raise ValueError("%s must have %d-byte elements (got %d)" % (name, elem, t.element_size()))
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and s != d for s, d in zip(shape, t.shape)):
            raise ValueError("%s must have shape %s (got %s)" % (
                name, tuple("*" if s is None else s for s in shape), tuple(t.shape)))
    if device and not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)


def _gpu(**tensors) -> None:
    """Every named tensor must be in GPU memory (checked after the layout checks)."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError("%s must be on the GPU" % name)


def _ptr(t) -> int | None:
    """Device (or host numpy) address of a tensor/array; None passes NULL."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream=None) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def abi_version() -> int:
    return load().bgtq_abi_version()


def codebook(bits: int):
    """(centroids, thresholds, D(b)) of the library's b-bit Lloyd-Max quantiser."""
    c = np.zeros(1 << bits)
    t = np.zeros((1 << bits) - 1)
    d = ctypes.c_double()
    _check(load().bgtq_codebook(bits, c.ctypes.data, t.ctypes.data, ctypes.addressof(d)))
    return c, t, d.value


def _pairing(p) -> int:
    if p not in ROPE_PAIRINGS:
        raise ValueError("rope pairing must be one of %s" % (list(ROPE_PAIRINGS),))
    return ROPE_PAIRINGS[p]


def energy(q_cal, k_cal, n_kv_heads: int, out, stream=None, pairing: str = "half") -> None:
    import torch
    _need(q_cal, "q_cal", elem=2, shape=(None, None, HEAD_DIM))
    n, hq, d = q_cal.shape
    _need(k_cal, "k_cal", elem=2, shape=(n, n_kv_heads, HEAD_DIM))
    _need(out, "energy", dtype=torch.float64, shape=(n_kv_heads, 64))
    _gpu(q_cal=q_cal, k_cal=k_cal, energy=out)
    _check(load().bgtq_energy(_ptr(q_cal), _ptr(k_cal), n, hq, n_kv_heads, d, _pairing(pairing), _ptr(out),
                              _stream(stream)))


def allocate(energy_arr, avg_bits: int) -> np.ndarray:
    """Host greedy allocation: float64 energies [Hkv, 64] (numpy or a CPU tensor) -> int8 widths."""
    e = np.ascontiguousarray(np.asarray(energy_arr.cpu() if hasattr(energy_arr, "cpu") else energy_arr,
                                        dtype=np.float64))
    if e.ndim != 2:
        raise ValueError("energies must be [n_kv_heads, 64]")
    out = np.zeros(e.shape, np.int8)
    _check(load().bgtq_allocate(e.ctypes.data, e.shape[0], e.shape[1], avg_bits, out.ctypes.data))
    return out


def allocate_device(energy_t, avg_bits: int, out, stream=None) -> None:
    """Device allocation: energies already in device memory -> int8 widths in ``out``."""
    import torch
    _need(energy_t, "energy", dtype=torch.float64, shape=(None, 64))
    hkv, nb = energy_t.shape
    _need(out, "bits", elem=1, shape=(hkv, nb))
    _gpu(energy=energy_t, bits=out)
    _check(load().bgtq_allocate_device(_ptr(energy_t), hkv, nb, avg_bits, _ptr(out), _stream(stream)))


@dataclasses.dataclass
class Sizes:
    consts: int
    k_codes: int
    k_norms: int
    v_codes: int
    v_norms: int


class Plan:
    """Host plan for one layer (widths, V width, seed, layer id)."""

    def __init__(self, k_bits: np.ndarray, k_avg_bits: int, v_bits: int, n_q_heads: int,
                 seed: int = 0, layer: int = 0, pairing: str = "half"):
        lib = load()
        kb = np.ascontiguousarray(np.asarray(k_bits, dtype=np.int8))
        self.n_kv_heads = kb.shape[0]
        self.n_q_heads = n_q_heads
        self.k_avg_bits = k_avg_bits
        self.v_bits = v_bits
        self.seed = seed
        self.layer = layer
        self.pairing = pairing
        desc = _PlanDesc(self.n_kv_heads, n_q_heads, HEAD_DIM, k_avg_bits, v_bits,
                         kb.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), seed, layer, _pairing(pairing))
        h = ctypes.c_void_p()
        _check(lib.bgtq_plan_create(ctypes.byref(desc), ctypes.byref(h)))
        self._h = h
        self.k_bits = kb.copy()

    @property
    def handle(self):
        return self._h

    def close(self) -> None:
        if self._h:
            load().bgtq_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sizes(self, batch: int, capacity: int) -> Sizes:
        s = _Sizes()
        _check(load().bgtq_plan_sizes(self._h, batch, capacity, ctypes.byref(s)))
        return Sizes(s.consts, s.k_codes, s.k_norms, s.v_codes, s.v_norms)

    def upload(self, dev_consts, stream=None) -> None:
        _check(load().bgtq_plan_upload(self._h, _ptr(dev_consts), _stream(stream)))

    def rotation(self, kvh: int, tensor: int, width: int) -> np.ndarray | None:
        d = ctypes.c_int32()
        _check(load().bgtq_plan_rotation(self._h, kvh, tensor, width, None, ctypes.byref(d)))
        if d.value == 0:
            return None
        out = np.zeros((d.value, d.value))
        _check(load().bgtq_plan_rotation(self._h, kvh, tensor, width, out.ctypes.data, ctypes.byref(d)))
        return out

    def bits(self) -> np.ndarray:
        out = np.zeros((self.n_kv_heads, 64), np.int8)
        _check(load().bgtq_plan_bits(self._h, out.ctypes.data))
        return out

    def _check_tokens(self, x, name: str) -> None:
        _need(x, name, elem=2, shape=(None, None, self.n_kv_heads, HEAD_DIM))

    def _check_cache(self, k_codes, k_norms, v_codes, v_norms) -> None:
        if k_codes is not None:
            _need(k_codes, "k_codes", elem=4)
        _need(k_norms, "k_norms", elem=2)
        _need(v_codes, "v_codes", elem=4)
        _need(v_norms, "v_norms", elem=2)

    def _check_decode(self, q, seq_lens, out, workspace, lens_name: str = "seq_lens") -> None:
        import torch
        _need(q, "q", elem=2, shape=(None, self.n_q_heads, HEAD_DIM))
        _need(out, "out", elem=2, shape=tuple(q.shape))
        _need(seq_lens, lens_name, dtype=torch.int32, shape=(q.shape[0],))
        _need(workspace, "workspace")

    def _check_new(self, q, k_new, v_new) -> None:
        """The new token's key and value: [batch, Hkv, 128] or [batch, 1, Hkv, 128] (the same memory)."""
        shape = (q.shape[0], 1, self.n_kv_heads, HEAD_DIM) if k_new.dim() == 4 else \
            (q.shape[0], self.n_kv_heads, HEAD_DIM)
        _need(k_new, "k_new", elem=2, shape=shape)
        _need(v_new, "v_new", elem=2, shape=shape)

    def encode_k(self, consts, k, capacity: int, t0: int, k_codes, k_norms, stream=None) -> None:
        self._check_tokens(k, "k")
        _need(k_codes, "k_codes", elem=4)
        _need(k_norms, "k_norms", elem=2)
        _gpu(k=k, k_codes=k_codes, k_norms=k_norms)
        b, n = k.shape[0], k.shape[1]
        _check(load().bgtq_encode_k(self._h, _ptr(consts), _ptr(k), b, capacity, t0, n,
                                    _ptr(k_codes), _ptr(k_norms), _stream(stream)))

    def encode_v(self, consts, v, capacity: int, t0: int, v_codes, v_norms, stream=None) -> None:
        self._check_tokens(v, "v")
        _need(v_codes, "v_codes", elem=4)
        _need(v_norms, "v_norms", elem=2)
        _gpu(v=v, v_codes=v_codes, v_norms=v_norms)
        b, n = v.shape[0], v.shape[1]
        _check(load().bgtq_encode_v(self._h, _ptr(consts), _ptr(v), b, capacity, t0, n,
                                    _ptr(v_codes), _ptr(v_norms), _stream(stream)))

    def encode_kv(self, consts, k, v, capacity: int, t0: int, k_codes, k_norms, v_codes, v_norms,
                  stream=None) -> None:
        """Keys and values of the same tokens in one call (bit-identical to encode_k then encode_v)."""
        self._check_tokens(k, "k")
        self._check_tokens(v, "v")
        _need(v, "v", shape=tuple(k.shape))
        _need(k_codes, "k_codes", elem=4)
        _need(k_norms, "k_norms", elem=2)
        _need(v_codes, "v_codes", elem=4)
        _need(v_norms, "v_norms", elem=2)
        _gpu(k=k, v=v, k_codes=k_codes, k_norms=k_norms, v_codes=v_codes, v_norms=v_norms)
        b, n = k.shape[0], k.shape[1]
        _check(load().bgtq_encode_kv(self._h, _ptr(consts), _ptr(k), _ptr(v), b, capacity, t0, n, _ptr(k_codes),
                                     _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), _stream(stream)))

    def rotate_queries(self, consts, q, q_rot, stream=None) -> None:
        import torch
        _need(q, "q", elem=2, shape=(None, self.n_q_heads, HEAD_DIM))
        _need(q_rot, "q_rot", dtype=torch.float32, shape=tuple(q.shape))
        _gpu(q=q, q_rot=q_rot)
        _check(load().bgtq_rotate_queries(self._h, _ptr(consts), _ptr(q), q.shape[0], _ptr(q_rot),
                                          _stream(stream)))

    def key_logits(self, consts, q_rot, k_codes, k_norms, capacity: int, t0: int, n_k: int, logits,
                   stream=None) -> None:
        """K-only logits q . k_hat of n_q queries per sequence against cache tokens t0 .. t0 + n_k - 1.
        q_rot: float32 [batch, n_q, n_q_heads, 128] (rotate_queries of the [batch * n_q, n_q_heads, 128]
        queries); logits: float32 [batch, n_q_heads, n_q, n_k], written."""
        import torch
        _need(q_rot, "q_rot", dtype=torch.float32, shape=(None, None, self.n_q_heads, HEAD_DIM))
        b, nq = q_rot.shape[0], q_rot.shape[1]
        if k_codes is not None:
            _need(k_codes, "k_codes", elem=4)
        _need(k_norms, "k_norms", elem=2)
        _need(logits, "logits", dtype=torch.float32, shape=(b, self.n_q_heads, nq, n_k))
        _gpu(q_rot=q_rot, k_codes=k_codes, k_norms=k_norms, logits=logits)
        _check(load().bgtq_key_logits(self._h, _ptr(consts), _ptr(q_rot), nq, _ptr(k_codes), _ptr(k_norms),
                                      capacity, b, t0, n_k, _ptr(logits), _stream(stream)))

    def workspace_size(self, batch: int, max_seq_len: int) -> int:
        n = ctypes.c_size_t()
        _check(load().bgtq_decode_workspace_size(self._h, batch, max_seq_len, ctypes.byref(n)))
        return n.value

    def decode_attn(self, consts, q, k_codes, k_norms, v_codes, v_norms, capacity: int, seq_lens,
                    max_seq_len: int, out, workspace, softmax_scale: float | None = None,
                    stream=None) -> None:
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        self._check_decode(q, seq_lens, out, workspace)
        self._check_cache(k_codes, k_norms, v_codes, v_norms)
        _gpu(q=q, seq_lens=seq_lens, out=out, workspace=workspace, k_codes=k_codes, k_norms=k_norms,
             v_codes=v_codes, v_norms=v_norms)
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(load().bgtq_decode_attn(self._h, _ptr(consts), _ptr(q), _ptr(k_codes), _ptr(k_norms),
                                       _ptr(v_codes), _ptr(v_norms), capacity, _ptr(seq_lens), q.shape[0],
                                       max_seq_len, softmax_scale, _ptr(out), _ptr(workspace), ws_bytes,
                                       _stream(stream)))

    def decode_attn_noalloc(self, consts, q, k_codes, k_norms, v_codes, v_norms, capacity: int, seq_lens,
                            max_seq_len: int, out, softmax_scale: float | None = None, stream=None) -> None:
        """decode_attn with the split partials in the library's device scratch (no workspace; calls that
        overlap on one device race)."""
        import torch
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        _need(q, "q", elem=2, shape=(None, self.n_q_heads, HEAD_DIM))
        _need(out, "out", elem=2, shape=tuple(q.shape))
        _need(seq_lens, "seq_lens", dtype=torch.int32, shape=(q.shape[0],))
        self._check_cache(k_codes, k_norms, v_codes, v_norms)
        _gpu(q=q, seq_lens=seq_lens, out=out, k_codes=k_codes, k_norms=k_norms, v_codes=v_codes, v_norms=v_norms)
        _check(load().bgtq_decode_attn_noalloc(self._h, _ptr(consts), _ptr(q), _ptr(k_codes), _ptr(k_norms),
                                               _ptr(v_codes), _ptr(v_norms), capacity, _ptr(seq_lens), q.shape[0],
                                               max_seq_len, softmax_scale, _ptr(out), _stream(stream)))

    def encode_k_paged(self, consts, k, pages: "PagedCache", t0: int, stream=None) -> None:
        self._check_tokens(k, "k")
        _gpu(k=k)
        pg = pages.desc()
        _check(load().bgtq_encode_k_paged(self._h, _ptr(consts), _ptr(k), k.shape[0], ctypes.byref(pg), t0,
                                          k.shape[1], _ptr(pages.k_codes), _ptr(pages.k_norms), _stream(stream)))

    def encode_kv_paged(self, consts, k, v, pages: "PagedCache", t0: int, stream=None) -> None:
        self._check_tokens(k, "k")
        self._check_tokens(v, "v")
        _need(v, "v", shape=tuple(k.shape))
        _gpu(k=k, v=v)
        pg = pages.desc()
        _check(load().bgtq_encode_kv_paged(self._h, _ptr(consts), _ptr(k), _ptr(v), k.shape[0], ctypes.byref(pg),
                                           t0, k.shape[1], _ptr(pages.k_codes), _ptr(pages.k_norms),
                                           _ptr(pages.v_codes), _ptr(pages.v_norms), _stream(stream)))

    def encode_v_paged(self, consts, v, pages: "PagedCache", t0: int, stream=None) -> None:
        self._check_tokens(v, "v")
        _gpu(v=v)
        pg = pages.desc()
        _check(load().bgtq_encode_v_paged(self._h, _ptr(consts), _ptr(v), v.shape[0], ctypes.byref(pg), t0,
                                          v.shape[1], _ptr(pages.v_codes), _ptr(pages.v_norms), _stream(stream)))

    def decode_attn_paged(self, consts, q, pages: "PagedCache", seq_lens, max_seq_len: int, out, workspace,
                          softmax_scale: float | None = None, stream=None) -> None:
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        self._check_decode(q, seq_lens, out, workspace)
        _gpu(q=q, seq_lens=seq_lens, out=out, workspace=workspace)
        pg = pages.desc()
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(load().bgtq_decode_attn_paged(
            self._h, _ptr(consts), _ptr(q), _ptr(pages.k_codes), _ptr(pages.k_norms), _ptr(pages.v_codes),
            _ptr(pages.v_norms), ctypes.byref(pg), _ptr(seq_lens), q.shape[0], max_seq_len, softmax_scale,
            _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))

    def decode_attn_paged_buffered(self, consts, q, pages: "PagedCache", seq_lens, max_seq_len: int,
                                   buf: "Buffer", out, workspace, softmax_scale: float | None = None,
                                   stream=None) -> None:
        """decode_attn_paged with the fp16 sink and recent-window tokens of ``buf`` taken from fp16."""
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        self._check_decode(q, seq_lens, out, workspace)
        _gpu(q=q, seq_lens=seq_lens, out=out, workspace=workspace)
        pg = pages.desc()
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(load().bgtq_decode_attn_paged_buffered(
            self._h, _ptr(consts), _ptr(q), _ptr(pages.k_codes), _ptr(pages.k_norms), _ptr(pages.v_codes),
            _ptr(pages.v_norms), ctypes.byref(pg), _ptr(seq_lens), q.shape[0], max_seq_len, softmax_scale,
            _ptr(buf.k_sink), _ptr(buf.v_sink), buf.n_sink, _ptr(buf.k_recent), _ptr(buf.v_recent), buf.n_recent,
            _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))

    def decode_step_buffered(self, consts, q, k_new, v_new, pos, max_seq_len: int, k_codes, k_norms, v_codes,
                             v_norms, capacity: int, buf: "Buffer", out, workspace,
                             softmax_scale: float | None = None, stream=None) -> None:
        """decode_step that also copies the new token into ``buf`` and attends with its fp16 sink and
        recent window (decode_attn_buffered over pos[b] + 1 tokens)."""
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        self._check_decode(q, pos, out, workspace, "pos")
        self._check_new(q, k_new, v_new)
        self._check_cache(k_codes, k_norms, v_codes, v_norms)
        _gpu(q=q, k_new=k_new, v_new=v_new, pos=pos, out=out, workspace=workspace, k_codes=k_codes,
             k_norms=k_norms, v_codes=v_codes, v_norms=v_norms)
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(load().bgtq_decode_step_buffered(
            self._h, _ptr(consts), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pos), q.shape[0], max_seq_len,
            _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), capacity, softmax_scale, _ptr(buf.k_sink),
            _ptr(buf.v_sink), buf.n_sink, _ptr(buf.k_recent), _ptr(buf.v_recent), buf.n_recent, _ptr(out),
            _ptr(workspace), ws_bytes, _stream(stream)))

    def decode_step_paged(self, consts, q, k_new, v_new, pos, max_seq_len: int, pages: "PagedCache", out,
                          workspace, softmax_scale: float | None = None, stream=None) -> None:
        """decode_step on a paged pool: k_new / v_new appended at token pos[b], then attention over pos[b] + 1."""
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        self._check_decode(q, pos, out, workspace, "pos")
        self._check_new(q, k_new, v_new)
        _gpu(q=q, pos=pos, out=out, workspace=workspace, k_new=k_new, v_new=v_new)
        pg = pages.desc()
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(load().bgtq_decode_step_paged(
            self._h, _ptr(consts), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pos), q.shape[0], max_seq_len,
            _ptr(pages.k_codes), _ptr(pages.k_norms), _ptr(pages.v_codes), _ptr(pages.v_norms), ctypes.byref(pg),
            softmax_scale, _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))

    def decode_attn_buffered(self, consts, q, k_codes, k_norms, v_codes, v_norms, capacity: int, seq_lens,
                             max_seq_len: int, buf: "Buffer", out, workspace, softmax_scale: float | None = None,
                             stream=None) -> None:
        """decode_attn with the fp16 sink and recent-window tokens of ``buf`` taken from fp16."""
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        self._check_decode(q, seq_lens, out, workspace)
        self._check_cache(k_codes, k_norms, v_codes, v_norms)
        _gpu(q=q, seq_lens=seq_lens, out=out, workspace=workspace, k_codes=k_codes, k_norms=k_norms,
             v_codes=v_codes, v_norms=v_norms)
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(load().bgtq_decode_attn_buffered(
            self._h, _ptr(consts), _ptr(q), _ptr(k_codes), _ptr(k_norms), _ptr(v_codes), _ptr(v_norms), capacity,
            _ptr(seq_lens), q.shape[0], max_seq_len, softmax_scale, _ptr(buf.k_sink), _ptr(buf.v_sink),
            buf.n_sink, _ptr(buf.k_recent), _ptr(buf.v_recent), buf.n_recent, _ptr(out), _ptr(workspace),
            ws_bytes, _stream(stream)))

    def decode_step(self, consts, q, k_new, v_new, pos, max_seq_len: int, k_codes, k_norms, v_codes, v_norms,
                    capacity: int, out, workspace, softmax_scale: float | None = None, stream=None) -> None:
        """Append k_new / v_new at token pos[b] of each sequence, then attend q over pos[b] + 1 tokens."""
        if softmax_scale is None:
            softmax_scale = HEAD_DIM ** -0.5
        self._check_decode(q, pos, out, workspace, "pos")
        self._check_cache(k_codes, k_norms, v_codes, v_norms)
        self._check_new(q, k_new, v_new)
        _gpu(q=q, pos=pos, out=out, workspace=workspace, k_codes=k_codes, k_norms=k_norms, v_codes=v_codes,
             v_norms=v_norms, k_new=k_new, v_new=v_new)
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(load().bgtq_decode_step(self._h, _ptr(consts), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(pos),
                                       q.shape[0], max_seq_len, _ptr(k_codes), _ptr(k_norms), _ptr(v_codes),
                                       _ptr(v_norms), capacity, softmax_scale, _ptr(out), _ptr(workspace),
                                       ws_bytes, _stream(stream)))


def fp16_workspace_size(batch: int, n_kv_heads: int, n_q_heads: int, max_seq_len: int) -> int:
    n = ctypes.c_size_t()
    _check(load().bgtq_fp16_decode_workspace_size(batch, n_kv_heads, n_q_heads, max_seq_len, ctypes.byref(n)))
    return n.value


def fp16_decode_attn(q, k, v, seq_lens, max_seq_len: int, out, workspace, softmax_scale: float | None = None,
                     stream=None) -> None:
    """fp16 decode attention over an uncompressed cache k, v [batch][capacity][n_kv_heads][128] (the baseline)."""
    if softmax_scale is None:
        softmax_scale = HEAD_DIM ** -0.5
    import torch
    _need(q, "q", elem=2, shape=(None, None, HEAD_DIM))
    b, hq, _ = q.shape
    _need(k, "k", elem=2, shape=(b, None, None, HEAD_DIM))
    _, cap, hkv, _ = k.shape
    _need(v, "v", elem=2, shape=tuple(k.shape))
    _need(out, "out", elem=2, shape=tuple(q.shape))
    _need(seq_lens, "seq_lens", dtype=torch.int32, shape=(b,))
    _need(workspace, "workspace")
    _gpu(q=q, k=k, v=v, out=out, seq_lens=seq_lens, workspace=workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(load().bgtq_fp16_decode_attn(_ptr(q), _ptr(k), _ptr(v), b, hq, hkv, cap, _ptr(seq_lens), max_seq_len,
                                        softmax_scale, _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


class PagedCache:
    """A paged pool of one layer's packed cache (caller-owned torch tensors, zero-filled): pages of one
    64-token tile per KV head, k_codes [Hkv][n_pages][4 k_avg_bits][64] and so on, plus a device block
    table [batch][max_pages] of int32 page ids (logical tile j of sequence b is page table[b][j])."""

    def __init__(self, plan: "Plan", n_pages: int, block_table, device="cuda"):
        import torch
        hkv = plan.n_kv_heads
        self.plan, self.n_pages = plan, n_pages
        self.block_table = torch.as_tensor(np.ascontiguousarray(block_table, dtype=np.int32)).to(device)
        self.batch, self.max_pages = self.block_table.shape
        s = plan.sizes(1, n_pages * TILE)
        self.consts = torch.zeros(s.consts // 4 + 64, dtype=torch.int32, device=device)
        self.k_codes = torch.zeros((hkv, n_pages, 4 * plan.k_avg_bits, TILE), dtype=torch.int32, device=device)
        self.k_norms = torch.zeros((hkv, n_pages, TILE, 4), dtype=torch.int16, device=device)
        self.v_codes = torch.zeros((hkv, n_pages, HEAD_DIM, 2 * plan.v_bits), dtype=torch.int32, device=device)
        self.v_norms = torch.zeros((hkv, n_pages, TILE), dtype=torch.int16, device=device)
        assert self.k_codes.numel() * 4 == s.k_codes and self.v_codes.numel() * 4 == s.v_codes
        plan.upload(self.consts)

    @property
    def capacity(self) -> int:
        return self.max_pages * TILE

    def desc(self) -> _Pages:
        return _Pages(self.block_table.data_ptr(), self.max_pages, self.n_pages)

    def encode(self, k, v, t0: int, stream=None) -> None:
        self.plan.encode_k_paged(self.consts, k, self, t0, stream)
        self.plan.encode_v_paged(self.consts, v, self, t0, stream)

    def encode_kv(self, k, v, t0: int, stream=None) -> None:
        self.plan.encode_kv_paged(self.consts, k, v, self, t0, stream)


class Buffer:
    """fp16 sink and recent-window buffers of one layer (caller-owned torch tensors):
    k_sink / v_sink [batch][Hkv][n_sink][128], k_recent / v_recent [batch][Hkv][n_recent][128]
    (token t in row t % n_recent)."""

    def __init__(self, batch: int, n_kv_heads: int, n_sink: int = 4, n_recent: int = 128, device="cuda"):
        import torch
        self.batch, self.n_kv_heads, self.n_sink, self.n_recent = batch, n_kv_heads, n_sink, n_recent
        mk = lambda n: (torch.zeros((batch, n_kv_heads, n, HEAD_DIM), dtype=torch.int16, device=device)
                        if n else None)
        self.k_sink, self.v_sink = mk(n_sink), mk(n_sink)
        self.k_recent, self.v_recent = mk(n_recent), mk(n_recent)

    def append(self, k, v, t0: int, stream=None) -> None:
        """Copy new fp16 tokens k, v [batch][n_new][Hkv][128] (positions t0 ..) into the buffers."""
        _need(k, "k", elem=2, shape=(self.batch, None, self.n_kv_heads, HEAD_DIM))
        _need(v, "v", elem=2, shape=tuple(k.shape))
        _gpu(k=k, v=v)
        b, n_new, hkv, _ = k.shape
        _check(load().bgtq_buffer_append(_ptr(k), _ptr(v), b, n_new, t0, hkv, _ptr(self.k_sink),
                                         _ptr(self.v_sink), self.n_sink, _ptr(self.k_recent),
                                         _ptr(self.v_recent), self.n_recent, _stream(stream)))


def profile_enable(on: bool = True) -> None:
    _check(load().bgtq_profile_enable(1 if on else 0))


def profile_read() -> tuple[float, int]:
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load().bgtq_profile_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


class Cache:
    """Device buffers of one layer's packed cache (caller-owned torch tensors, zero-filled)."""

    def __init__(self, plan: Plan, batch: int, capacity: int, device="cuda"):
        import torch
        s = plan.sizes(batch, capacity)
        tiles = (capacity + TILE - 1) // TILE
        hkv = plan.n_kv_heads
        self.plan, self.batch, self.capacity, self.tiles = plan, batch, capacity, tiles
        self.consts = torch.zeros(s.consts // 4 + 64, dtype=torch.int32, device=device)
        self.k_codes = torch.zeros((batch, hkv, tiles, 4 * plan.k_avg_bits, TILE), dtype=torch.int32, device=device)
        self.k_norms = torch.zeros((batch, hkv, tiles, TILE, 4), dtype=torch.int16, device=device)
        self.v_codes = torch.zeros((batch, hkv, tiles, HEAD_DIM, 2 * plan.v_bits), dtype=torch.int32, device=device)
        self.v_norms = torch.zeros((batch, hkv, tiles, TILE), dtype=torch.int16, device=device)
        assert self.k_codes.numel() * 4 == s.k_codes and self.v_codes.numel() * 4 == s.v_codes
        plan.upload(self.consts)

    def encode(self, k, v, t0: int, stream=None) -> None:
        self.plan.encode_k(self.consts, k, self.capacity, t0, self.k_codes, self.k_norms, stream)
        self.plan.encode_v(self.consts, v, self.capacity, t0, self.v_codes, self.v_norms, stream)

    def encode_kv(self, k, v, t0: int, stream=None) -> None:
        self.plan.encode_kv(self.consts, k, v, self.capacity, t0, self.k_codes, self.k_norms, self.v_codes,
                            self.v_norms, stream)

    def step(self, q, k_new, v_new, pos, max_seq_len: int, out, workspace, softmax_scale=None, stream=None) -> None:
        self.plan.decode_step(self.consts, q, k_new, v_new, pos, max_seq_len, self.k_codes, self.k_norms,
                              self.v_codes, self.v_norms, self.capacity, out, workspace, softmax_scale, stream)

    def packed_bytes(self, seq_len: int) -> int:
        """Algorithmic packed bytes read for `seq_len` tokens per sequence (codes + present norms)."""
        kb = self.plan.k_bits
        groups = [len({int(w) for w in row if w > 0}) for row in kb]
        per_head = [4 * 4 * self.plan.k_avg_bits + 2 * g + 16 * self.plan.v_bits + 2 for g in groups]
        return self.batch * seq_len * sum(per_head)
