"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module holds no attention arithmetic.  It draws i.i.d. standard normal
Q, K, V and dO tensors from numpy's PCG64 generator, rounds them to the
storage dtype (fp32, or bf16 with round-to-nearest-even) and returns both
the storage bits and their exact fp64 values, so that the oracle and the
GPU path start from identical numbers.

Layout of every tensor: [B, H, N, d], d innermost, C-contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "gaussian",
    "round_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "make_storage",
    "exact_of",
]


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, storage dtype, masks and its seed base."""

    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    masks: tuple = ("causal",)
    seed_base: int = 0
    tile: int = 128  # KV tile (rows) the GPU path uses for this workload
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def elems(self) -> int:
        return self.B * self.H * self.N * self.d

    def flops_bwd(self, causal: bool) -> float:
        """Backward FLOP convention: 2.5x the forward's 4*B*H*N^2*d, halved
        when causal.  With a window or block mask: 2.5x 4*B*H*d times the
        exact number of visible (query, key) pairs."""
        if self.window or self.block_spec:
            return 2.5 * 4.0 * self.B * self.H * self.d * self.visible_pairs(causal)
        f = 2.5 * 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if causal else f

    @property
    def window(self) -> int:
        return int(self.extra.get("window", 0))

    @property
    def block_spec(self):
        return self.extra.get("block")

    def block_mask(self):
        """The seeded block mask (bool [N/bs, N/bs]) or None.

        "local_global": each query block sees the key blocks within
        `band` blocks of it, the first `globals` key blocks, and a random
        `density` share of the others (seed = seed_base + 9)."""
        spec = self.block_spec
        if spec is None:
            return None
        nb = self.N // spec["size"]
        qb = np.arange(nb)[:, None]
        kb = np.arange(nb)[None, :]
        rng = np.random.Generator(np.random.PCG64(self.seed_base + 9))
        m = (np.abs(qb - kb) <= spec["band"]) | (kb < spec["globals"])
        m |= rng.random((nb, nb)) < spec["density"]
        return m

    def mask_args(self) -> dict:
        """Keyword arguments of the library's mask (window, block mask)."""
        bm = self.block_mask()
        return {"window": self.window, "block_mask": bm,
                "block_size": 0 if bm is None else self.block_spec["size"]}

    def visible_pairs(self, causal: bool) -> int:
        """Exact count of visible (query, key) pairs under the mask, counted
        per tile pair: a pair of tiles at offset D = q - kv holds T - |e|
        element pairs with i - j = D*T + e for each e in (-T, T)."""
        T = self.tile
        n = self.N // T
        lo = 0 if causal else -(1 << 40)
        hi = (self.window - 1) if self.window else (1 << 40)
        if self.window and not causal:
            lo = -(self.window - 1)
        e = np.arange(-(T - 1), T)
        mult = T - np.abs(e)
        offs = np.arange(-(n - 1), n)
        diff = offs[:, None] * T + e[None, :]
        per_off = ((diff >= lo) & (diff <= hi)).astype(np.int64) @ mult   # by offset D
        q = np.arange(n)[:, None]
        kv = np.arange(n)[None, :]
        cnt = per_off[(q - kv) + (n - 1)]
        bm = self.block_mask()
        if bm is not None:
            bt = self.block_spec["size"] // T
            cnt = cnt * bm[q // bt, kv // bt]
        return int(cnt.sum())


# The five workloads: a tiny fp32 case the oracle finishes in seconds, and four
# bf16 cases at the shapes used for throughput.  Seeds are 1000*id + {0,1,2,3}
# for Q, K, V, dO.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 256, 64, "f32", ("full", "causal"), 1000, 64,
                         "oracle case, 64x64 tiles"),
    "b2h16_n2k_d128_causal": Workload("b2h16_n2k_d128_causal", 2, 16, 2048, 128, "bf16",
                                      ("causal",), 2000),
    "b4h32_n4k_d128_full": Workload("b4h32_n4k_d128_full", 4, 32, 4096, 128, "bf16",
                                    ("full",), 3000),
    "b1h32_n16k_d128_causal": Workload("b1h32_n16k_d128_causal", 1, 32, 16384, 128, "bf16",
                                       ("causal",), 4000),
    "b8h64_n8k_d64": Workload("b8h64_n8k_d64", 8, 64, 8192, 64, "bf16",
                              ("causal", "full"), 5000),
    # special masks (measurement of the window / block-mask extension): a
    # causal sliding window of 4096 keys, and a causal local + global +
    # random block mask over 128-row blocks
    "b1h32_n16k_d128_swa4k": Workload("b1h32_n16k_d128_swa4k", 1, 32, 16384, 128, "bf16",
                                      ("causal",), 6000, extra={"window": 4096}),
    "b1h32_n16k_d128_blocksparse": Workload(
        "b1h32_n16k_d128_blocksparse", 1, 32, 16384, 128, "bf16", ("causal",), 7000,
        extra={"block": {"size": 128, "band": 4, "globals": 2, "density": 0.1}}),
}


def gaussian(shape, seed: int) -> np.ndarray:
    """i.i.d. N(0,1) in float64 from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(size=shape, dtype=np.float64)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 -> bf16 bit pattern (uint16), via fp32, round-to-nearest-even.

    NaN is not expected in these inputs; infinities pass through.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, seed_base: int,
                names=("q", "k", "v", "do")) -> dict:
    """Draw the four input tensors.

    Returns a dict name -> (storage, exact64) where ``storage`` is float32
    (dtype "f32") or uint16 bf16 bits (dtype "bf16"), and ``exact64`` is the
    float64 value of exactly what is stored.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    out = {}
    for i, name in enumerate(names):
        x = gaussian((B, H, N, d), seed_base + i)
        if dtype == "f32":
            s = x.astype(np.float32)
            out[name] = (s, s.astype(np.float64))
        else:
            s = round_to_bf16_bits(x)
            out[name] = (s, bf16_bits_to_f32(s).astype(np.float64))
    return out


def make_storage(B: int, H: int, N: int, d: int, dtype: str, seed_base: int,
                 names=("q", "k", "v", "do")) -> dict:
    """The same tensors as ``make_inputs`` (same seeds, same values), storage
    only: for full-size workloads whose fp64 copies would not fit; the exact
    values of any slice come from ``exact_of``."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    out = {}
    for i, name in enumerate(names):
        x = gaussian((B, H, N, d), seed_base + i)
        out[name] = x.astype(np.float32) if dtype == "f32" else round_to_bf16_bits(x)
        del x
    return out


def exact_of(storage: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 value of exactly what is stored (fp32 values or bf16 bits)."""
    if dtype == "f32":
        return np.asarray(storage, dtype=np.float64)
    return bf16_bits_to_f32(storage).astype(np.float64)


def make_workload_inputs(w: Workload, names=("q", "k", "v", "do")) -> dict:
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed_base, names)
