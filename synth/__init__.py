"""Seeded synthetic inputs for the DSA Lightning Indexer + exact top-K path.

This module only *draws* inputs: Gaussian activations, their quantisation to
OCP FP8 e4m3fn codes with an amax/448 scale (done by torch's own cast), ranges,
paged-cache layouts.  It holds none of the method's arithmetic (no scoring, no
selection, no e4m3 decoding) so that both the CPU oracle and the GPU library
can consume it without sharing computation.

Recipe (fixed draw order per case, CPU ``torch.Generator`` seeded per case):
  q ~ N(0,1) [Q,64,128] -> per-(row,head) scale amax_d|q|/448 -> e4m3 codes
  k ~ N(0,1) [N,128]    -> per-token scale amax/448          -> e4m3 codes
  w ~ N(0, 1/64) [Q,64]
  ranges: causal, row at position t sees keys [0, t+1)

BF16 stream scan (page "Deleting the key transpose puts the DSA indexer scan on its streaming
floor"): per stream b (CPU generator seeded with (seed, b)): q ~ N(0,1) [64,128]
-> BF16 (torch's RNE cast), k ~ N(0,1) [N,128] -> BF16, w ~ N(0, 1/64) [64].

Shapes follow the five workloads of the pages' operating points (Fused Indexer
Top-k page, "2.3 Problem definition" and "6.1 Setup": B=1, 64 heads, d=128,
K=2048, N from 8K to 160K; contest report page (arXiv 2608.14560), "DSA TopK Indexer": paged
decode with 64-token pages).  Real DeepSeek-V3.2 activations are not available;
these Gaussian inputs stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

H = 64          # indexer heads
D = 128         # head dimension
E4M3_MAX = 448.0

# Sampling lattice used by the library's threshold estimator (documented in
# include/idx_topk.h).  Only used here to place adversarial keys on or off it.
SAMPLE_STRIDE = 200
SAMPLE_OFFSET = 100
# x8 keys of the off-lattice outlier block: with the plain keys' ~4096
# candidates, more than a row's 8192+ candidate slots
OUTLIER_KEYS = 6000


@dataclasses.dataclass
class PrefillCase:
    name: str
    q8: np.ndarray        # uint8 [Q,64,128] e4m3fn codes
    q_scale: np.ndarray   # float32 [Q,64]
    k8: np.ndarray        # uint8 [N,128]
    k_scale: np.ndarray   # float32 [N]
    w: np.ndarray         # float32 [Q,64]
    row_start: np.ndarray  # int32 [Q]
    row_end: np.ndarray    # int32 [Q] (exclusive)
    K: int = 2048

    @property
    def Q(self) -> int:
        return int(self.q8.shape[0])

    @property
    def N(self) -> int:
        return int(self.k8.shape[0])

    @property
    def pairs(self) -> int:
        return int((self.row_end.astype(np.int64) - self.row_start).sum())


@dataclasses.dataclass
class DecodeCase:
    name: str
    q8: np.ndarray          # uint8 [B,64,128]
    q_scale: Optional[np.ndarray]  # float32 [B,64] or None (= 1)
    k_cache: np.ndarray     # uint8 [P,page,128]
    k_scale: np.ndarray     # float32 [P,page]
    w: np.ndarray           # float32 [B,64]
    page_table: np.ndarray  # int32 [B,max_pages], -1 = unused
    seq_lens: np.ndarray    # int32 [B]
    page_size: int = 64
    K: int = 2048

    @property
    def B(self) -> int:
        return int(self.q8.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def pairs(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())


@dataclasses.dataclass
class ScanCase:
    name: str
    q16: np.ndarray   # uint16 [B,64,128] BF16 bit patterns
    w: np.ndarray     # float32 [B,64]
    k16: np.ndarray   # uint16 [B,N,128] BF16 bit patterns
    lens: np.ndarray  # int32 [B]
    K: int = 2048

    @property
    def B(self) -> int:
        return int(self.k16.shape[0])

    @property
    def N(self) -> int:
        return int(self.k16.shape[1])

    @property
    def pairs(self) -> int:
        return int(self.lens.astype(np.int64).sum())


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def quantize_e4m3(x: torch.Tensor):
    """Per-slice (last axis) amax/448 scale and e4m3fn codes (torch RNE cast).

    Returns (codes uint8 ndarray, scale float32 ndarray).  Values are clamped to
    +-448 before the cast because torch maps out-of-range values to NaN.
    """
    x = x.float()
    amax = x.abs().amax(dim=-1, keepdim=True)
    amax = torch.where(amax > 0, amax, torch.ones_like(amax))
    scale = (amax / E4M3_MAX).float()
    y = (x / scale).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy().copy(), scale.squeeze(-1).numpy().astype(np.float32).copy()


def _queries(g: torch.Generator, Q: int):
    q = torch.randn(Q, H, D, generator=g)
    q8, qs = quantize_e4m3(q)
    return q8, qs


def _weights(g: torch.Generator, Q: int) -> np.ndarray:
    return (torch.randn(Q, H, generator=g) / 8.0).numpy().astype(np.float32)


def _keys_normal(g: torch.Generator, N: int, heavy_frac: float = 0.0, heavy_mult: float = 8.0):
    k = torch.randn(N, D, generator=g)
    if heavy_frac > 0:
        n_heavy = int(round(N * heavy_frac))
        sel = torch.randperm(N, generator=g)[:n_heavy]
        k[sel] *= heavy_mult
    return quantize_e4m3(k)


def causal_case(name: str, Q: int, N: int, seed: int, key_mode: str = "normal",
                K: int = 2048, positions: Optional[np.ndarray] = None) -> PrefillCase:
    """Q query rows at the last Q positions of an N-token causal context.

    key_mode:
      normal      k ~ N(0,1)
      heavy_tail  1% of key rows scaled x8 before quantisation
      ties16      every key is one of 16 distinct (code vector, scale) pairs
      outlier     a 6000-key block of x8 keys off the sampling lattice, ending
                  at the first row's last position: no sample sees them, so
                  the threshold is taken from the plain keys and the rows
                  keep about 6000 + 4096 candidates, more than the segments
                  hold, and the last ones dropped are outliers (overflow)
      decoy       x8 keys placed exactly on the sampling lattice (every other
                  lattice point), so the sampled threshold lands among them
    """
    g = _gen(seed)
    q8, qs = _queries(g, Q)
    if key_mode == "ties16":
        base = torch.randn(16, D, generator=g)
        b8, bs = quantize_e4m3(base)
        assign = torch.randint(0, 16, (N,), generator=g).numpy()
        k8, ks = b8[assign].copy(), bs[assign].copy()
    elif key_mode == "heavy_tail":
        k8, ks = _keys_normal(g, N, heavy_frac=0.01, heavy_mult=8.0)
    elif key_mode in ("normal", "outlier", "decoy"):
        k = torch.randn(N, D, generator=g)
        if key_mode == "outlier":
            last = int(positions[0]) if positions is not None else N - Q
            pos = []
            p = last
            while len(pos) < OUTLIER_KEYS and p >= 0:
                if (p - SAMPLE_OFFSET) % SAMPLE_STRIDE != 0:
                    pos.append(p)
                p -= 1
            k[torch.tensor(pos)] *= 8.0
        elif key_mode == "decoy":
            lattice = torch.arange(SAMPLE_OFFSET, N, SAMPLE_STRIDE)
            k[lattice[::2]] *= 8.0
        k8, ks = quantize_e4m3(k)
    else:
        raise ValueError(key_mode)
    w = _weights(g, Q)
    if positions is None:
        positions = np.arange(N - Q, N, dtype=np.int64)
    row_start = np.zeros(Q, dtype=np.int32)
    row_end = (positions + 1).astype(np.int32)
    return PrefillCase(name, q8, qs, k8, ks, w, row_start, row_end, K)


def random_case(name: str, Q: int, N: int, seed: int, K: int = 2048,
                min_len: int = 0, max_len: Optional[int] = None,
                key_mode: str = "normal") -> PrefillCase:
    """Small parity case with ragged, arbitrary [start, end) ranges per row."""
    g = _gen(seed)
    q8, qs = _queries(g, Q)
    if key_mode == "heavy_tail":
        k8, ks = _keys_normal(g, N, heavy_frac=0.01)
    else:
        k8, ks = _keys_normal(g, N)
    w = _weights(g, Q)
    max_len = N if max_len is None else min(max_len, N)
    lens = torch.randint(min_len, max_len + 1, (Q,), generator=g).numpy()
    starts = np.array([int(torch.randint(0, N - L + 1, (1,), generator=g).item()) for L in lens])
    return PrefillCase(name, q8, qs, k8, ks, w, starts.astype(np.int32),
                       (starts + lens).astype(np.int32), K)


def decode_case(name: str, seq_lens, seed: int, page_size: int = 64, K: int = 2048,
                max_pages: Optional[int] = None, with_q_scale: bool = False) -> DecodeCase:
    """Paged decode: one query per sequence, keys in a shuffled page pool."""
    g = _gen(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    if with_q_scale:
        q8, qs = _queries(g, B)
    else:
        q = torch.randn(B, H, D, generator=g).clamp(-E4M3_MAX, E4M3_MAX)
        q8, qs = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy(), None
    n_pages = [(int(L) + page_size - 1) // page_size for L in seq_lens]
    P = max(1, sum(n_pages))
    if max_pages is None:
        max_pages = max(1, max(n_pages))
    k = torch.randn(P * page_size, D, generator=g)
    k8, ks = quantize_e4m3(k)
    k8 = k8.reshape(P, page_size, D)
    ks = ks.reshape(P, page_size)
    w = _weights(g, B)
    perm = torch.randperm(P, generator=g).numpy().astype(np.int32)
    table = np.full((B, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        table[b, :n_pages[b]] = perm[o:o + n_pages[b]]
        o += n_pages[b]
    return DecodeCase(name, q8, qs, k8, ks, w, table, seq_lens, page_size, K)


# ---------------------------------------------------------------- workloads

def prefill_smoke(seed: int = 0) -> PrefillCase:
    """64 rows at positions 8128..8191 of an 8192-token context."""
    return causal_case("prefill_smoke_q64_n8192", 64, 8192, seed)


def prefill_chunk(seed: int = 0) -> PrefillCase:
    """4096 rows at the last positions of a 32768-token context."""
    return causal_case("prefill_chunk_q4096_n32768", 4096, 32768, seed)


def long_prefill(seed: int = 0) -> PrefillCase:
    """4096 rows over a 131072-token context, 1% of keys x8 (heavy tail)."""
    return causal_case("long_prefill_q4096_n131072", 4096, 131072, seed, key_mode="heavy_tail")


def adversarial(seed: int = 0) -> List[PrefillCase]:
    """2048 rows at the last positions of a 163840-token context, split into
    four calls with their own key sets: 1024 rows over 16 distinct key
    vectors (massive ties), 256 rows with an off-lattice x8 outlier block of
    6000 keys at the end of their ranges (more candidates than a row holds:
    overflow, exact repair), 256 rows with x8 decoys on the sampling lattice
    (the sampled threshold lands among them: too few candidates, exact
    repair), 512 rows over plain N(0,1) keys."""
    N = 163840
    pos = np.arange(N - 2048, N, dtype=np.int64)
    return [
        causal_case("adversarial_ties16", 1024, N, seed * 16 + 1, "ties16", positions=pos[:1024]),
        causal_case("adversarial_outlier", 256, N, seed * 16 + 2, "outlier", positions=pos[1024:1280]),
        causal_case("adversarial_decoy", 256, N, seed * 16 + 4, "decoy", positions=pos[1280:1536]),
        causal_case("adversarial_normal", 512, N, seed * 16 + 3, "normal", positions=pos[1536:]),
    ]


def adversarial_decoy(seed: int = 0, Q: int = 256) -> PrefillCase:
    """Rows whose sampled threshold lands among on-lattice x8 decoys (underflow)."""
    N = 163840
    pos = np.arange(N - Q, N, dtype=np.int64)
    return causal_case("adversarial_decoy", Q, N, seed * 16 + 4, "decoy", positions=pos)


def random_codes_case(name: str, N: int, starts, ends, seed: int, K: int = 2048) -> PrefillCase:
    """Rows over keys whose e4m3 codes are uniform random bytes (the two NaN
    codes excluded) with per-key scales uniform in [1/896, 1/224): cheap to
    make for very large N.  Queries and weights as in every other case."""
    g = _gen(seed)
    Q = len(starts)
    q8, qs = _queries(g, Q)
    w = _weights(g, Q)
    rng = np.random.default_rng(seed)
    k8 = rng.integers(0, 256, size=(N, D), dtype=np.uint8)
    k8[(k8 & 0x7F) == 0x7F] ^= 0x01
    ks = rng.uniform(1.0 / 896, 1.0 / 224, N).astype(np.float32)
    return PrefillCase(name, q8, qs, k8, ks, w, np.asarray(starts, np.int32), np.asarray(ends, np.int32), K)


def paged_decode_lens(seed: int = 0, B: int = 16) -> np.ndarray:
    """12 lengths from U{1..65536} and 4 from U{1..2048}, at seeded slots."""
    g = _gen(seed * 7919 + 17)
    lens = torch.randint(1, 65537, (B,), generator=g)
    short_slots = torch.randperm(B, generator=g)[:4]
    lens[short_slots] = torch.randint(1, 2049, (4,), generator=g)
    return lens.numpy().astype(np.int32)


def paged_decode(seed: int = 0) -> DecodeCase:
    """Batch 16, one query per sequence, 64-token pages, max 1024 pages."""
    return decode_case("paged_decode_b16", paged_decode_lens(seed), seed, page_size=64,
                       max_pages=1024)


WORKLOADS = {
    "prefill_smoke": prefill_smoke,
    "paged_decode": paged_decode,
    "prefill_chunk": prefill_chunk,
    "long_prefill": long_prefill,
    "adversarial": adversarial,
}


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def scan_stream(seed: int, b: int, N: int):
    """Stream b of a BF16 scan case: (q16 [64,128], w [64], k16 [N,128])."""
    g = _gen(seed * 1000003 + b)
    q16 = _bf16_bits(torch.randn(H, D, generator=g))
    w = (torch.randn(H, generator=g) / 8.0).numpy().astype(np.float32)
    k16 = np.empty((N, D), dtype=np.uint16)
    for i0 in range(0, N, 65536):  # bounded temporaries for long streams
        n = min(65536, N - i0)
        k16[i0:i0 + n] = _bf16_bits(torch.randn(n, D, generator=g))
    return q16, w, k16


def scan_case(name: str, B: int, N: int, seed: int, lens=None, K: int = 2048) -> ScanCase:
    q16 = np.empty((B, H, D), dtype=np.uint16)
    w = np.empty((B, H), dtype=np.float32)
    k16 = np.empty((B, N, D), dtype=np.uint16)
    for b in range(B):
        q16[b], w[b], k16[b] = scan_stream(seed, b, N)
    lens = np.full(B, N, dtype=np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
    return ScanCase(name, q16, w, k16, lens, K)


def bf16_scan(seed: int = 0) -> ScanCase:
    """32 streams x 262144 BF16 keys each (the page's M = 32 operating point), K = 2048."""
    return scan_case("bf16_scan_b32_n262144", 32, 262144, seed)


WORKLOADS["bf16_scan"] = bf16_scan
