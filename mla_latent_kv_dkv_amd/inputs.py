"""Seeded synthetic inputs for the MLA decode workloads (no method arithmetic here).

This module is the only thing the fp64 oracle and the GPU library have in
common: it draws numbers, builds page tables and lengths, and nothing else.

Generator (counter based, so any element can be produced on its own and the
host and the GPU produce identical bits):

* SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): element ``i`` of a stream with key ``K`` is
  ``mix64(K + (i+1)*GAMMA)`` with the published GAMMA and mixing constants.
* A roughly normal value is the Irwin-Hall sum of the four 16-bit fields of
  that word, centred: ``s = f0+f1+f2+f3 - 131070`` (an integer, exact in fp32),
  then ``float32(s) * float32(std / sqrt(4*(65536**2-1)/12))`` -- one IEEE fp32
  multiply -- and, for bf16 storage, round-to-nearest-even to bf16.
* A uniform value in [0, 1) is ``(word >> 11) * 2**-53``.

Stream keys are derived on the host from (seed, tensor name, layer) and passed
to the device fill kernel as a 64-bit integer, so only ``mix64`` needs a device
twin (in ``csrc/fill_inputs.hip``).
"""
from __future__ import annotations

import math
import os
import zlib
from dataclasses import dataclass, field

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_IH_STD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)   # std of the 4-field sum
_CHUNK = 1 << 20


def mix64(z):
    """SplitMix64 output mixing of a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, name: str, layer: int = 0) -> int:
    """64-bit stream key of tensor ``name`` (layer ``layer``) under ``seed``."""
    tag = (zlib.crc32(name.encode()) << 16) ^ (layer & 0xFFFF)
    with np.errstate(over="ignore"):
        k = mix64(np.uint64(seed) + GAMMA)
        k = mix64(k ^ (np.uint64(tag) + GAMMA))
    return int(k)


def words(key: int, start: int, n: int) -> np.ndarray:
    """uint64 words ``start .. start+n-1`` of stream ``key``."""
    idx = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(np.uint64(key) + idx * GAMMA)


def normal_scale(std: float) -> np.float32:
    """The single fp32 factor applied to the centred Irwin-Hall integer."""
    return np.float32(std / _IH_STD)


def _normal_chunk(key: int, start: int, n: int, sc: np.float32, out: np.ndarray,
                  bf16: bool = False) -> None:
    z = np.arange(start + 1, start + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z *= GAMMA
        z += np.uint64(key)
        t = z >> np.uint64(30)
        z ^= t
        z *= _M1
        np.right_shift(z, np.uint64(27), out=t)
        z ^= t
        z *= _M2
        np.right_shift(z, np.uint64(31), out=t)
        z ^= t
    m16 = np.uint64(0xFFFF)
    np.bitwise_and(z, m16, out=t)
    s = t.copy()
    for sh in (16, 32):
        np.right_shift(z, np.uint64(sh), out=t)
        t &= m16
        s += t
    np.right_shift(z, np.uint64(48), out=t)
    s += t
    v = s.view(np.int64)
    v -= 131070
    f = v.astype(np.float32)
    f *= sc
    if bf16:
        out[...] = f32_to_bf16_bits(f)
    else:
        out[...] = f


def _normal(key: int, start: int, n: int, std: float, bf16: bool) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    sc = normal_scale(std)
    chunks = [(a, min(n, a + _CHUNK)) for a in range(0, n, _CHUNK)]
    if len(chunks) <= 1:
        for a, b in chunks:
            _normal_chunk(key, start + a, b - a, sc, out[a:b], bf16)
        return out
    from concurrent.futures import ThreadPoolExecutor
    workers = min(16, len(os.sched_getaffinity(0)), len(chunks))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda ab: _normal_chunk(key, start + ab[0], ab[1] - ab[0], sc,
                                              out[ab[0]:ab[1]], bf16), chunks))
    return out


def normal_f32(key: int, start: int, n: int, std: float = 1.0) -> np.ndarray:
    """fp32 values ``start .. start+n-1`` of stream ``key`` (approximately N(0, std^2))."""
    return _normal(key, start, n, std, False)


def normal_bf16_bits(key: int, start: int, n: int, std: float = 1.0) -> np.ndarray:
    """The same values rounded to bf16 (nearest even), as uint16 bit patterns."""
    return _normal(key, start, n, std, True)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns
    (finite inputs; the rounding increment cannot overflow for them)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = b >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def uniform01(key: int, start: int, n: int) -> np.ndarray:
    return (words(key, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


# ----------------------------------------------------------------- workloads --
@dataclass(frozen=True)
class Workload:
    """One decode-step workload: model dims, batch structure and seed."""
    name: str
    hidden: int
    n_heads: int
    d_head: int
    d_latent: int
    d_rope: int
    dtype: str                      # "f32" | "bf16" storage; accumulation is fp32
    batch: int
    context: int                    # fixed length (ignored when ``ragged``)
    seed: int
    num_splits: int = 1
    layers: int = 1
    ragged: tuple = ()              # (lo, hi) for log-uniform lengths, else ()
    permute_pages: bool = True
    cache_from_h: bool = False      # build the cache through the append call
    page_size: int = 64
    rope_base: float = 10000.0
    d_cq: int = 0                   # query compression rank d_c' (0: q^C = W_Q h)
    cache: str = "dtype"            # pool format: "dtype" rows, or "fp8" pages
    chunk: int = 0                  # prefill: the last `chunk` positions of every sequence
                                    # are the step's prompt tokens (0: decode, one token)
    yarn: tuple = ()                # YaRN-stretched RoPE: (scale, orig_len, alpha, beta)
    plan_units: int = 0             # decode attention over a length-proportional plan of
                                    # at most this many units (0: num_splits uniform splits)
    notes: str = field(default="", compare=False)

    @property
    def row(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def fan_in(self, name: str) -> int:
        return {"w_q": self.hidden, "w_qr": self.hidden, "w_dkv": self.hidden,
                "w_kr": self.hidden, "w_uk": self.d_latent, "w_uv": self.d_latent,
                "w_o": self.n_heads * self.d_head, "w_dq": self.hidden,
                "w_uq": self.d_cq}[name]

    def weight_shape(self, name: str) -> tuple:
        nh, dh, dc, dr, H = self.n_heads, self.d_head, self.d_latent, self.d_rope, self.hidden
        return {"w_q": (nh * dh, H), "w_qr": (nh * dr, H), "w_dkv": (dc, H), "w_kr": (dr, H),
                "w_uk": (nh * dh, dc), "w_uv": (nh * dh, dc), "w_o": (H, nh * dh),
                "w_dq": (self.d_cq, H), "w_uq": (nh * dh, self.d_cq)}[name]

    @property
    def weight_names(self) -> tuple:
        """The layer's weights: W_Q, or W_DQ and W_UQ when the query is compressed."""
        if self.d_cq:
            return ("w_dq", "w_uq") + WEIGHT_NAMES[1:]
        return WEIGHT_NAMES


WEIGHT_NAMES = ("w_q", "w_qr", "w_dkv", "w_kr", "w_uk", "w_uv", "w_o")

WORKLOADS = {
    "tiny": Workload("tiny", 64, 4, 16, 32, 8, "f32", 1, 64, 1001, num_splits=1,
                     permute_pages=False, cache_from_h=True),
    "lite": Workload("lite", 2048, 16, 128, 512, 64, "bf16", 32, 4096, 1002, num_splits=8,
                     cache_from_h=True),
    "full": Workload("full", 5120, 128, 128, 512, 64, "bf16", 64, 4096, 1003, num_splits=4),
    "long": Workload("long", 5120, 128, 128, 512, 64, "bf16", 4, 131072, 1004, num_splits=64),
    # ragged: a plan of at most 768 units, three rounds of work units over the 256 CUs
    "ragged": Workload("ragged", 5120, 128, 128, 512, 64, "bf16", 256, 0, 1005, num_splits=16,
                       layers=60, ragged=(512, 32768), plan_units=768),
    # the same shapes with the query's low-rank compression (d_c' = 1536 at full size)
    "tiny-cq": Workload("tiny-cq", 64, 4, 16, 32, 8, "f32", 1, 64, 1006, num_splits=1,
                        permute_pages=False, cache_from_h=True, d_cq=24),
    "lite-cq": Workload("lite-cq", 2048, 16, 128, 512, 64, "bf16", 32, 4096, 1007, num_splits=8,
                        cache_from_h=True, d_cq=512),
    "full-cq": Workload("full-cq", 5120, 128, 128, 512, 64, "bf16", 64, 4096, 1008, num_splits=4,
                        d_cq=1536),
    # the same shapes with the FP8 latent pool (the pool is filled from seeded fp32
    # rows, or built through the FP8 append for the cache-from-h ones)
    "tiny-fp8": Workload("tiny-fp8", 64, 4, 16, 32, 8, "f32", 1, 64, 1009, num_splits=1,
                         permute_pages=False, cache_from_h=True, cache="fp8"),
    "lite-fp8": Workload("lite-fp8", 2048, 16, 128, 512, 64, "bf16", 32, 4096, 1010, num_splits=8,
                         cache_from_h=True, cache="fp8"),
    "full-fp8": Workload("full-fp8", 5120, 128, 128, 512, 64, "bf16", 64, 4096, 1011, num_splits=4,
                         cache="fp8"),
    # chunked prefill: each sequence's last `chunk` positions are prompt tokens of the
    # step, appended and attending causally (cache before them from h, or drawn)
    "tiny-pre": Workload("tiny-pre", 64, 4, 16, 32, 8, "f32", 2, 64, 1012, num_splits=2,
                         cache_from_h=True, page_size=16, chunk=24),
    "lite-pre": Workload("lite-pre", 2048, 16, 128, 512, 64, "bf16", 4, 1024, 1013, num_splits=2,
                         cache_from_h=True, chunk=64),
    "full-pre": Workload("full-pre", 5120, 128, 128, 512, 64, "bf16", 4, 4096, 1014, num_splits=1,
                         chunk=256),
    # YaRN-stretched RoPE: the long-context extension's 4K -> 128K setting (scale 40,
    # alpha 1, beta 32) on the full and long shapes; the tiny shape with a 16-token
    # original window so its 64 positions cross the ramp
    "tiny-yarn": Workload("tiny-yarn", 64, 4, 16, 32, 8, "f32", 1, 64, 1015, num_splits=1,
                          permute_pages=False, cache_from_h=True, yarn=(4.0, 16, 1.0, 32.0)),
    "full-yarn": Workload("full-yarn", 5120, 128, 128, 512, 64, "bf16", 64, 4096, 1016,
                          num_splits=4, yarn=(40.0, 4096, 1.0, 32.0)),
    "long-yarn": Workload("long-yarn", 5120, 128, 128, 512, 64, "bf16", 4, 131072, 1017,
                          num_splits=64, yarn=(40.0, 4096, 1.0, 32.0)),
}


def seq_lengths(w: Workload) -> np.ndarray:
    """Context length of every sequence (the decode token included).  Ragged
    workloads draw L = min(hi, floor(lo * (hi/lo)**u)), u uniform in [0, 1)."""
    if not w.ragged:
        return np.full(w.batch, w.context, dtype=np.int32)
    lo, hi = w.ragged
    u = uniform01(stream_key(w.seed, "lengths"), 0, w.batch)
    return np.minimum(hi, np.floor(lo * np.power(hi / lo, u))).astype(np.int32)


def page_table(w: Workload, lens: np.ndarray):
    """(block_table [B, max_pages] int32, num_pages).  Every sequence owns
    ceil(L/page) pages; physical ids are a seeded permutation (identity when
    ``permute_pages`` is off); unused table entries hold 0."""
    pages = (lens.astype(np.int64) + w.page_size - 1) // w.page_size
    total = int(pages.sum())
    max_pages = int(pages.max())
    if w.permute_pages:
        keys = words(stream_key(w.seed, "page_perm"), 0, total)
        perm = np.argsort(keys, kind="stable").astype(np.int32)
    else:
        perm = np.arange(total, dtype=np.int32)
    bt = np.zeros((w.batch, max_pages), dtype=np.int32)
    off = 0
    for b in range(w.batch):
        bt[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    return bt, total


def tensor_values(w: Workload, name: str, shape, std: float = 1.0, layer: int = 0,
                  start: int = 0, count: int | None = None) -> np.ndarray:
    """Host copy of a seeded tensor in its storage format: fp32 values, or bf16
    bit patterns (uint16) for bf16 workloads.  ``start``/``count`` select a flat
    sub-range (the same elements the device fill writes there)."""
    n = int(np.prod(shape)) if count is None else count
    gen = normal_f32 if w.dtype == "f32" else normal_bf16_bits
    v = gen(stream_key(w.seed, name, layer), start, n, std)
    return v.reshape(shape) if count is None else v


def weight_values(w: Workload, name: str, layer: int = 0) -> np.ndarray:
    return tensor_values(w, name, w.weight_shape(name), 1.0 / math.sqrt(w.fan_in(name)), layer)


def to_f64(w: Workload, arr: np.ndarray) -> np.ndarray:
    """Upcast storage-format values (fp32, or bf16 bits) to fp64."""
    return np.asarray(arr, dtype=np.float64) if w.dtype == "f32" else bf16_bits_to_f64(arr)


def pool_rows(w: Workload, block_table: np.ndarray, seq: int, length: int, layer: int = 0,
              f32: bool = False):
    """Storage-format pool rows of logical positions 0..length-1 of ``seq`` as the
    device fill leaves them (the pool is filled linearly by physical element
    index, stream "pool").  ``f32``: the fp32 values instead, whatever the
    storage type (the source rows of an FP8 pool)."""
    pos = np.arange(length)
    phys = block_table[seq, pos // w.page_size].astype(np.int64) * w.page_size + pos % w.page_size
    key = stream_key(w.seed, "pool", layer)
    # contiguous runs of physical rows share one generator call
    as_f32 = f32 or w.dtype == "f32"
    out = np.empty((length, w.row), dtype=np.float32 if as_f32 else np.uint16)
    j = 0
    while j < length:
        k = j
        while k + 1 < length and phys[k + 1] == phys[k] + 1:
            k += 1
        gen = normal_f32 if as_f32 else normal_bf16_bits
        v = gen(key, int(phys[j]) * w.row, (k - j + 1) * w.row, 1.0)
        out[j:k + 1] = v.reshape(k - j + 1, w.row)
        j = k + 1
    return out


# ------------------------------------------------------- device twin (GPU) --
_inputs_lib = None


def _device_lib():
    global _inputs_lib
    if _inputs_lib is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_inputs.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m mla_latent_kv_dkv_amd.build`")
        lib = ctypes.CDLL(path)
        lib.mla_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                        ctypes.c_void_p]
        lib.mla_fill_normal.restype = ctypes.c_int32
        _inputs_lib = lib
    return _inputs_lib


def fill_device(t, key: int, std: float = 1.0, start: int = 0, stream=None):
    """Fill contiguous device tensor ``t`` (fp32 or bf16) with elements
    start .. start+numel-1 of stream ``key`` -- the same bits ``normal_f32`` /
    ``tensor_values`` give on the host."""
    import ctypes
    import torch
    if not t.is_cuda or not t.is_contiguous() or t.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("fill_device needs a contiguous fp32/bf16 device tensor")
    s = torch.cuda.current_stream() if stream is None else stream
    rc = _device_lib().mla_fill_normal(ctypes.c_void_p(t.data_ptr()), t.numel(),
                                       0 if t.dtype == torch.float32 else 1, key, start,
                                       float(normal_scale(std)), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"mla_fill_normal returned {rc}")
    return t
