"""Seeded input recipes for the five Polar Attention workloads.

The workloads stand in for the pages' evaluation data (FineWeb-Edu at 2K, induction
needle-in-a-haystack to 64K/256K; "ATMA" summary pages, section 3 and the abstract),
none of which is used here.  Shapes follow the 378M / 16-layer model's attention layer:
16 query heads sharing 4 KV heads, head_dim 64, training length 2048.

Random streams.  Every tensor gets its own child of ``SeedSequence(seed)`` (spawn order:
q, k, v, w, pages, needles).  Large tensors are drawn in fixed chunks of
``CHUNK`` elements of the C-order flattened array, chunk ``c`` from the c-th child of the
tensor's stream, so the values do not depend on how many threads draw them.

Precision.  q and k are L2-normalised in float32 (the model normalises them before
attention, "ATMA" technical summary, section 2.1 "Stability Mechanism"), needles are
planted in float32, then bf16 workloads are rounded to nearest-even bf16.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

FLAG_LENGTH_TEMP = 1
FLAG_NULL_FLOOR = 2

CHUNK = 1 << 22          # elements per independent random stream chunk
NEEDLE_NOISE = 0.1       # needle key = normalize(q + 0.1 * unit noise): cosine ~0.995


# --------------------------------------------------------------------------- configs
CONFIGS = {
    # tiny causal fp32, no GQA
    "c1": dict(seed=1001, kind="prefill", B=1, T=256, Hq=4, Hkv=4, d=64, dtype="f32",
               needles="none"),
    # training-length prefill with 5% of key slots planted as near-copies of a later query
    "c2": dict(seed=1002, kind="prefill", B=8, T=2048, Hq=16, Hkv=4, d=64, dtype="bf16",
               needles="copies", needle_frac=0.05),
    # long prefill: one needle per query head, queried by the last row
    "c3": dict(seed=1003, kind="prefill", B=1, T=16384, Hq=16, Hkv=4, d=64, dtype="bf16",
               needles="last_row", needle_heads="all"),
    # extrapolation prefill: 8 needles (even heads), queried by the last row
    "c4": dict(seed=1004, kind="prefill", B=1, T=65536, Hq=16, Hkv=4, d=64, dtype="bf16",
               needles="last_row", needle_heads="even"),
    # paged decode: 16 sequences x 256K KV, shuffled 64-token pages, 1 needle per (b, h)
    "c5": dict(seed=1005, kind="decode", B=16, L=262144, Hq=16, Hkv=4, d=64, dtype="bf16",
               page_size=64, needles="per_head"),
}

BETA_DEFAULT = 8.0       # sqrt(head_dim)
TRAIN_LEN = 2048


# --------------------------------------------------------------------------- helpers
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _normal(ss: np.random.SeedSequence, shape, threads: int = 8) -> np.ndarray:
    """float32 N(0,1) of ``shape`` drawn chunk-wise from children of ``ss``."""
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    n_chunks = max(1, -(-out.size // CHUNK))
    kids = ss.spawn(n_chunks)

    def fill(c):
        g = np.random.Generator(np.random.PCG64(kids[c]))
        g.standard_normal(out=out[c * CHUNK:(c + 1) * CHUNK], dtype=np.float32)

    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(threads, n_chunks)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def _l2_normalize(x: np.ndarray) -> np.ndarray:
    """Unit-normalise the last axis in float32 (the model's q/k precondition)."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def _needle_key(qvec: np.ndarray, g: np.random.Generator) -> np.ndarray:
    z = _l2_normalize(g.standard_normal(qvec.shape[-1], dtype=np.float32))
    return _l2_normalize(qvec.astype(np.float32) + np.float32(NEEDLE_NOISE) * z)


# --------------------------------------------------------------------------- prefill
@dataclasses.dataclass
class PrefillInputs:
    name: str
    dtype: str                 # "bf16" (q/k/v are uint16 bit patterns) or "f32"
    B: int
    T: int
    Hq: int
    Hkv: int
    d: int
    q: np.ndarray              # [B,T,Hq,d]
    k: np.ndarray              # [B,T,Hkv,d]
    v: np.ndarray              # [B,T,Hkv,d]
    beta: np.ndarray           # [Hq] float32
    null_bias: np.ndarray      # [Hq] float32
    count_vec: np.ndarray      # [Hq,d] float32
    train_len: int
    flags: int
    needles: list              # (b, head, key position, query row)

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a


def prefill_inputs(name: str, B: Optional[int] = None, T: Optional[int] = None,
                   Hq: Optional[int] = None, Hkv: Optional[int] = None,
                   seed: Optional[int] = None, flags: int = FLAG_LENGTH_TEMP | FLAG_NULL_FLOOR,
                   train_len: int = TRAIN_LEN, dtype: Optional[str] = None) -> PrefillInputs:
    """Draw a prefill workload; size arguments override the named config's."""
    cfg = dict(CONFIGS[name])
    assert cfg["kind"] == "prefill", name
    B = cfg["B"] if B is None else B
    T = cfg["T"] if T is None else T
    Hq = cfg["Hq"] if Hq is None else Hq
    Hkv = cfg["Hkv"] if Hkv is None else Hkv
    dtype = cfg["dtype"] if dtype is None else dtype
    d = cfg["d"]
    seed = cfg["seed"] if seed is None else seed
    G = Hq // Hkv
    s_q, s_k, s_v, s_w, _s_pages, s_needle = np.random.SeedSequence(seed).spawn(6)
    q = _l2_normalize(_normal(s_q, (B, T, Hq, d)))
    k = _l2_normalize(_normal(s_k, (B, T, Hkv, d)))
    v = _normal(s_v, (B, T, Hkv, d))
    w = (np.float32(0.02) * _normal(s_w, (Hq, d))).astype(np.float32)
    g = np.random.Generator(np.random.PCG64(s_needle))
    needles = []
    mode = cfg["needles"]
    if mode == "copies" and T > 1:
        n_slots = int(round(cfg["needle_frac"] * T))
        for b in range(B):
            for kv in range(Hkv):
                slots = g.choice(T, size=min(n_slots, T), replace=False)
                for j in np.sort(slots):
                    h = int(kv * G + g.integers(0, G))
                    i = int(g.integers(j, T))
                    k[b, j, kv] = _needle_key(q[b, i, h], g)
                    needles.append((b, h, int(j), i))
    elif mode == "last_row" and T > 1:
        heads = range(Hq) if cfg["needle_heads"] == "all" else range(0, Hq, 2)
        for b in range(B):
            used = {kv: set() for kv in range(Hkv)}
            for h in heads:
                kv = h // G
                while True:
                    j = int(g.integers(0, T - 1))
                    if j not in used[kv]:
                        break
                used[kv].add(j)
                k[b, j, kv] = _needle_key(q[b, T - 1, h], g)
                needles.append((b, h, j, T - 1))
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return PrefillInputs(name=name, dtype=dtype, B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, q=q, k=k,
                         v=v, beta=np.full(Hq, BETA_DEFAULT, np.float32),
                         null_bias=np.zeros(Hq, np.float32), count_vec=w,
                         train_len=train_len, flags=flags, needles=needles)


# --------------------------------------------------------------------------- decode
@dataclasses.dataclass
class DecodeInputs:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    q: np.ndarray              # [B,Hq,d]
    k_pool: np.ndarray         # [num_pages,Hkv,page_size,d]
    v_pool: np.ndarray         # [num_pages,Hkv,page_size,d]
    page_table: np.ndarray     # [B,stride] int32 physical page ids
    seq_lens: np.ndarray       # [B] int32
    beta: np.ndarray
    null_bias: np.ndarray
    count_vec: np.ndarray
    train_len: int
    flags: int
    needles: list              # (b, head, logical key position)

    @property
    def num_pages(self) -> int:
        return self.k_pool.shape[0]

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a


def _pool_normal(ss, shape, normalize, dtype, threads=8):
    """Draw a page pool chunk-wise; normalise rows; round to bf16 per chunk (low peak RAM)."""
    total = int(np.prod(shape))
    d = shape[-1]
    out = np.empty(total, dtype=np.uint16 if dtype == "bf16" else np.float32)
    n_chunks = max(1, -(-total // CHUNK))
    kids = ss.spawn(n_chunks)

    def fill(c):
        lo, hi = c * CHUNK, min(total, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(kids[c]))
        x = g.standard_normal(hi - lo, dtype=np.float32).reshape(-1, d)
        if normalize:
            x = _l2_normalize(x)
        out[lo:hi] = (round_bf16(x) if dtype == "bf16" else x).reshape(-1)

    assert CHUNK % d == 0
    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(threads, n_chunks)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def decode_inputs(name: str = "c5", B: Optional[int] = None, L: Optional[int] = None,
                  seq_lens: Optional[Sequence[int]] = None, Hq: Optional[int] = None,
                  Hkv: Optional[int] = None, extra_pages: int = 0, seed: Optional[int] = None,
                  flags: int = FLAG_LENGTH_TEMP | FLAG_NULL_FLOOR,
                  train_len: int = TRAIN_LEN) -> DecodeInputs:
    """Draw a paged-decode workload.

    Each sequence b owns ceil(seq_lens[b]/page_size) pages; the pool holds exactly those
    pages plus ``extra_pages`` unused ones, and the physical ids are a seeded permutation
    of the pool.  Table entries past a sequence's last page are -1.
    """
    cfg = dict(CONFIGS[name])
    assert cfg["kind"] == "decode", name
    B = cfg["B"] if B is None else B
    L = cfg["L"] if L is None else L
    Hq = cfg["Hq"] if Hq is None else Hq
    Hkv = cfg["Hkv"] if Hkv is None else Hkv
    seed = cfg["seed"] if seed is None else seed
    d, P, dtype = cfg["d"], cfg["page_size"], cfg["dtype"]
    G = Hq // Hkv
    lens = np.full(B, L, np.int32) if seq_lens is None else np.asarray(seq_lens, np.int32)
    assert lens.shape == (B,) and (lens >= 1).all()
    n_pages_seq = -(-lens // P)
    stride = int(n_pages_seq.max())
    num_pages = int(n_pages_seq.sum()) + extra_pages
    s_q, s_k, s_v, s_w, s_pages, s_needle = np.random.SeedSequence(seed).spawn(6)
    q32 = _l2_normalize(_normal(s_q, (B, Hq, d)))
    k_pool = _pool_normal(s_k, (num_pages, Hkv, P, d), True, dtype)
    v_pool = _pool_normal(s_v, (num_pages, Hkv, P, d), False, dtype)
    w = (np.float32(0.02) * _normal(s_w, (Hq, d))).astype(np.float32)
    perm = np.random.Generator(np.random.PCG64(s_pages)).permutation(num_pages).astype(np.int32)
    table = np.full((B, stride), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :n_pages_seq[b]] = perm[off:off + n_pages_seq[b]]
        off += n_pages_seq[b]
    g = np.random.Generator(np.random.PCG64(s_needle))
    needles = []
    if cfg["needles"] == "per_head":
        for b in range(B):
            used = {kv: set() for kv in range(Hkv)}
            for h in range(Hq):
                kv = h // G
                while True:
                    j = int(g.integers(0, lens[b]))
                    if j not in used[kv] or len(used[kv]) >= lens[b]:
                        break
                used[kv].add(j)
                key = _needle_key(q32[b, h], g)
                page, slot = table[b, j // P], j % P
                k_pool[page, kv, slot] = round_bf16(key) if dtype == "bf16" else key
                needles.append((b, h, j))
    q = round_bf16(q32) if dtype == "bf16" else q32
    return DecodeInputs(name=name, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, d=d, page_size=P, q=q,
                        k_pool=k_pool, v_pool=v_pool, page_table=table, seq_lens=lens,
                        beta=np.full(Hq, BETA_DEFAULT, np.float32),
                        null_bias=np.zeros(Hq, np.float32), count_vec=w, train_len=train_len,
                        flags=flags, needles=needles)


# --------------------------------------------------------------------------- gradients
@dataclasses.dataclass
class Cotangents:
    """Upstream gradients of the five prefill outputs, and optionally of the plain softmax
    read-out (float32, standard normal)."""
    d_dir: np.ndarray          # [B,T,Hq,d]
    d_count: np.ndarray        # [B,T,Hq,d]
    d_n_eff: np.ndarray        # [B,T,Hq]
    d_gate: np.ndarray         # [B,T,Hq]
    d_lse: np.ndarray          # [B,T,Hq]
    d_attn: Optional[np.ndarray] = None    # [B,T,Hq,d]

    def as_dict(self) -> dict:
        out = dict(dir=self.d_dir, count=self.d_count, n_eff=self.d_n_eff, gate=self.d_gate,
                   lse=self.d_lse)
        if self.d_attn is not None:
            out["attn"] = self.d_attn
        return out


def cotangents(B: int, T: int, Hq: int, d: int = 64, seed: int = 2001,
               n_eff_scale: float = 1.0, attn: bool = False) -> Cotangents:
    """Seeded upstream gradients for the backward pass: one child stream per output (the
    read-out's is the sixth, so asking for it leaves the other five unchanged)."""
    s = np.random.SeedSequence(seed).spawn(6)
    return Cotangents(d_dir=_normal(s[0], (B, T, Hq, d)), d_count=_normal(s[1], (B, T, Hq, d)),
                      d_n_eff=(np.float32(n_eff_scale) * _normal(s[2], (B, T, Hq))).astype(np.float32),
                      d_gate=_normal(s[3], (B, T, Hq)), d_lse=_normal(s[4], (B, T, Hq)),
                      d_attn=_normal(s[5], (B, T, Hq, d)) if attn else None)



# --------------------------------------------------------------------------- paged chunks
@dataclasses.dataclass
class ChunkInputs:
    """A chunked-prefill step: sequences whose first start_pos[b] tokens are cached in
    shuffled pages, plus a chunk of C new tokens (queries, keys, values)."""
    full: PrefillInputs         # the contiguous sequences (T = max start + C)
    start_pos: np.ndarray       # [B] int32
    C: int
    page_size: int
    k_pool: np.ndarray          # [num_pages, Hkv, page, d], prefix already written
    v_pool: np.ndarray
    page_table: np.ndarray      # [B, stride] int32 (-1 past the end)
    max_seq_len: int

    def chunk(self, name: str) -> np.ndarray:
        """q, k or v of the new tokens, [B,C,H,d] (storage dtype)."""
        a = getattr(self.full, name)
        return np.stack([a[b, s:s + self.C] for b, s in enumerate(self.start_pos)])


def chunk_inputs(cfg: str = "c2", B: int = 2, C: int = 256, starts=(0, 700), Hq=None, Hkv=None,
                 train_len: int = TRAIN_LEN, extra_pages: int = 3, seed: int = 3001,
                 page_size: int = 64, full: Optional[PrefillInputs] = None) -> ChunkInputs:
    """Contiguous sequences of length max(starts) + C drawn like ``cfg`` (or the given
    ``full`` sequences); the prefix of each (tokens before its start) is scattered into a
    shuffled page pool, the rest left out."""
    starts = np.asarray(starts, np.int32)[:B]
    T = int(starts.max()) + C
    if full is None:
        full = prefill_inputs(cfg, B=B, T=T, Hq=Hq, Hkv=Hkv, train_len=train_len)
    assert full.T >= T and full.B >= B
    max_seq_len = T
    stride = -(-max_seq_len // page_size)
    num_pages = B * stride + extra_pages
    g = np.random.Generator(np.random.PCG64(seed))
    perm = g.permutation(num_pages)
    table = np.full((B, stride), -1, np.int32)
    k_pool = np.zeros((num_pages, full.Hkv, page_size, full.d), full.k.dtype)
    v_pool = np.zeros_like(k_pool)
    nxt = 0
    for b in range(B):
        L = int(starts[b]) + C
        for pg in range(-(-L // page_size)):
            table[b, pg] = perm[nxt]
            nxt += 1
        for pg in range(int(starts[b]) // page_size + 1):
            lo, hi = pg * page_size, min((pg + 1) * page_size, int(starts[b]))
            if hi > lo:
                pid = table[b, pg]
                k_pool[pid, :, :hi - lo] = full.k[b, lo:hi].transpose(1, 0, 2)
                v_pool[pid, :, :hi - lo] = full.v[b, lo:hi].transpose(1, 0, 2)
    return ChunkInputs(full=full, start_pos=starts, C=C, page_size=page_size, k_pool=k_pool,
                       v_pool=v_pool, page_table=table, max_seq_len=max_seq_len)


# --------------------------------------------------------------------------- memory step
@dataclasses.dataclass
class DeltaInputs:
    """One gated-delta memory step for B sequences whose states live in a slot pool."""
    dtype: str                 # q, k, v storage: "bf16" (bit patterns) or "f32"
    pool: np.ndarray           # [num_slots, H, d_v, d_k] float32
    slots: np.ndarray          # [B] int32, distinct
    q: np.ndarray              # [B, H, d_k]
    k: np.ndarray              # [B, H, d_k]
    v: np.ndarray              # [B, H, d_v]
    alpha: np.ndarray          # [B, H] float32 gate in (0, 1]
    beta: np.ndarray           # [B, H] float32 write strength in (0, 1)

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if self.dtype == "bf16" else a


def delta_inputs(B: int = 256, H: int = 16, num_slots: int = 1024, d_k: int = 64, d_v: int = 64,
                 dtype: str = "bf16", seed: int = 4001) -> DeltaInputs:
    """States N(0, 1/d_k) (a memory of unit-scale writes), q, k, v N(0, 1) (the kernel
    normalises q and k), gates alpha ~ U(0.9, 1) and beta ~ U(0, 1), and a random choice
    of B distinct pool slots."""
    s = np.random.SeedSequence(seed).spawn(6)
    pool = (_normal(s[0], (num_slots, H, d_v, d_k)) / np.float32(np.sqrt(d_k))).astype(np.float32)
    q = _normal(s[1], (B, H, d_k))
    k = _normal(s[2], (B, H, d_k))
    v = _normal(s[3], (B, H, d_v))
    g = np.random.Generator(np.random.PCG64(s[4]))
    alpha = g.uniform(0.9, 1.0, (B, H)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (B, H)).astype(np.float32)
    slots = np.random.Generator(np.random.PCG64(s[5])).permutation(num_slots)[:B].astype(np.int32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return DeltaInputs(dtype=dtype, pool=pool, slots=slots, q=q, k=k, v=v, alpha=alpha, beta=beta)


@dataclasses.dataclass
class DeltaSeqInputs(DeltaInputs):
    """The memory stream over T tokens for B sequences: q, k [B,T,H,d_k], v [B,T,H,d_v],
    alpha, beta [B,T,H]; pool and slots as for one step."""


def delta_seq_inputs(B: int = 32, T: int = 2048, H: int = 16, num_slots: int = 64,
                     d_k: int = 64, d_v: int = 64, dtype: str = "bf16", seed: int = 4101,
                     alpha_range=(0.9, 1.0)) -> DeltaSeqInputs:
    """A prompt or training sequence through the recurrent memory: the step's
    distributions (states N(0, 1/d_k), q, k, v N(0, 1), beta ~ U(0, 1)) drawn per token,
    gates alpha ~ U(alpha_range) per (token, head), B distinct slots."""
    s = np.random.SeedSequence(seed).spawn(6)
    pool = (_normal(s[0], (num_slots, H, d_v, d_k)) / np.float32(np.sqrt(d_k))).astype(np.float32)
    q = _normal(s[1], (B, T, H, d_k))
    k = _normal(s[2], (B, T, H, d_k))
    v = _normal(s[3], (B, T, H, d_v))
    g = np.random.Generator(np.random.PCG64(s[4]))
    alpha = g.uniform(alpha_range[0], alpha_range[1], (B, T, H)).astype(np.float32)
    beta = g.uniform(0.0, 1.0, (B, T, H)).astype(np.float32)
    slots = np.random.Generator(np.random.PCG64(s[5])).permutation(num_slots)[:B].astype(np.int32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return DeltaSeqInputs(dtype=dtype, pool=pool, slots=slots, q=q, k=k, v=v, alpha=alpha,
                          beta=beta)
