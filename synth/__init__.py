"""Seeded synthetic inputs for the top-k selection path.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It holds only input generation (random numbers, score rows, lengths,
block tables); it performs none of the selection arithmetic, so neither side of
a parity comparison can inherit a mistake from it.

Random numbers come from SplitMix64 used as a counter-based generator: the n-th
output of a stream is the SplitMix64 finalizer applied to ``base + n * gamma``,
which is exactly what the sequential SplitMix64 generator returns on its n-th
call (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014; constants of the public-domain reference ``splitmix64.c`` by
S. Vigna). Counter form makes every stream a vectorised numpy expression.
Normals use the Box-Muller transform in float64, then round to float32 (RNE).

Workloads follow the indexer top-k latency study on the lmsys.org page
"Serving GLM5.2 NVFP4 Agentic Workload with SGLang" (section TopK-V2,
Figure 4: target-model verification at batch size 1 with 6 draft tokens, 80K
and 1M input lengths, k = 2048), with indexer-KV pages of 64 tokens (the llm-d
GLM-5.2 page states 64-token KV blocks). The real traffic behind those pages
(an agentic coding replay) is not available; these synthetic rows stand in for
it with the sizes, lengths and tie structure listed in ``CONFIGS``.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math

import numpy as np

_MASK = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix_int(z: int) -> int:
    """SplitMix64 finalizer on a Python int (used for seeding streams)."""
    z &= _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def _mix(z: np.ndarray) -> np.ndarray:
    """SplitMix64 finalizer, vectorised over uint64 (wrapping arithmetic)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_sequence(seed: int, n: int) -> np.ndarray:
    """First ``n`` outputs of SplitMix64 started from state ``seed``."""
    ctr = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(np.uint64(seed & _MASK) + ctr * np.uint64(GAMMA))


class Stream:
    """An independent counter-based stream, keyed by (seed, tag)."""

    def __init__(self, seed: int, *tag: int):
        state = _mix_int(seed * GAMMA + 0x5EED)
        for t in tag:
            state = _mix_int(state ^ _mix_int(t + 1))
        self._state = state
        self._used = 0

    def u64(self, n: int) -> np.ndarray:
        out = splitmix64_sequence((self._state + self._used * GAMMA) & _MASK, n)
        self._used += n
        return out

    def uniform(self, n: int) -> np.ndarray:
        """float64 in [0, 1) from the top 53 bits."""
        return (self.u64(n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)

    def below(self, n: int, bound: int) -> np.ndarray:
        """Integers in [0, bound) by 32-bit multiply-shift (bound < 2**32)."""
        assert 0 < bound < (1 << 32)
        hi = self.u64(n) >> np.uint64(32)
        return ((hi * np.uint64(bound)) >> np.uint64(32)).astype(np.int64)

    def normal(self, n: int) -> np.ndarray:
        """N(0, 1) in float64 by Box-Muller (cosine branch)."""
        u1 = 1.0 - self.uniform(n)          # (0, 1]
        u2 = self.uniform(n)
        return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)

    def permutation(self, n: int) -> np.ndarray:
        """A uniform random permutation of [0, n) (argsort of random keys)."""
        return np.argsort(self.u64(n), kind="stable").astype(np.int64)


@dataclasses.dataclass
class Workload:
    """One batch of top-k inputs, host-resident.

    scores:       float32 [rows, stride]; positions >= lengths[r] hold padding.
    lengths:      int32 [rows]; valid prefix of each row.
    block_table:  int32 [table_rows, table_width]; logical page -> physical page.
    bt_row_stride: 0 when one table is shared by all rows, else table_width.
    """
    name: str
    scores: np.ndarray
    lengths: np.ndarray
    block_table: np.ndarray
    bt_row_stride: int
    page_size: int
    k: int
    seed: int

    @property
    def rows(self) -> int:
        return int(self.scores.shape[0])

    @property
    def stride(self) -> int:
        return int(self.scores.shape[1])

    @property
    def max_len(self) -> int:
        return int(self.lengths.max()) if self.rows else 0

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.scores, self.lengths, self.block_table):
            h.update(np.ascontiguousarray(a).tobytes())
        h.update(f"{self.bt_row_stride},{self.page_size},{self.k}".encode())
        return h.hexdigest()


def page_permutation_tables(st: Stream, tables: int, pages_per_table: int) -> np.ndarray:
    """``tables`` disjoint tables cut from one random permutation of all pages."""
    perm = st.permutation(tables * pages_per_table).astype(np.int32)
    return perm.reshape(tables, pages_per_table)


def _f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def make_c1(seed: int = 1) -> Workload:
    """2 x 8,192 N(0,1); 5% of each row overwritten by copies of other positions."""
    rows, n, ps, k = 2, 8192, 64, 2048
    scores = np.empty((rows, n), np.float32)
    dup = int(n * 0.05)                         # 409 per row
    for r in range(rows):
        st = Stream(seed, 1, r)
        row = _f32(st.normal(n))
        perm = st.permutation(n)
        chosen, rest = perm[:dup], perm[dup:]
        src = rest[st.below(dup, len(rest))]
        row[chosen] = row[src]
        scores[r] = row
    bt = page_permutation_tables(Stream(seed, 2), 1, n // ps)
    lengths = np.full(rows, n, np.int32)
    return Workload("c1_2x8192_ties", scores, lengths, bt, 0, ps, k, seed)


def make_c2(seed: int = 2) -> Workload:
    """7 x 80,000 target-verify rows: 30% exact +0.0, else 2|N(0,1)|; causal tail -inf."""
    rows, n, ps, k = 7, 80_000, 64, 2048
    scores = np.empty((rows, n), np.float32)
    lengths = (79_994 + np.arange(rows)).astype(np.int32)
    for r in range(rows):
        st = Stream(seed, 1, r)
        zero = st.uniform(n) < 0.30
        row = _f32(2.0 * np.abs(st.normal(n)))
        row[zero] = np.float32(0.0)
        row[lengths[r]:] = -np.inf
        scores[r] = row
    bt = page_permutation_tables(Stream(seed, 2), 1, n // ps)
    return Workload("c2_7x80k_verify", scores, lengths, bt, 0, ps, k, seed)


def make_c3(seed: int = 3) -> Workload:
    """7 x 1,000,000 N(0,1) with 1% of positions inside [3.0, 3.0005)."""
    rows, n, ps, k = 7, 1_000_000, 64, 2048
    scores = np.empty((rows, n), np.float32)
    cluster = n // 100
    ulp = 2.0 ** -22                            # float32 spacing on [2, 4)
    for r in range(rows):
        st = Stream(seed, 1, r)
        row = _f32(st.normal(n))
        pos = st.permutation(n)[:cluster]
        j = st.below(cluster, 2098)             # 3.0 + 2097 ulp < 3.0005
        row[pos] = _f32(3.0 + j * ulp)
        scores[r] = row
    bt = page_permutation_tables(Stream(seed, 2), 1, n // ps)
    lengths = np.full(rows, n, np.int32)
    return Workload("c3_7x1m_cluster", scores, lengths, bt, 0, ps, k, seed)


def make_c4(seed: int = 4) -> Workload:
    """64 rows, log-uniform lengths in [512, 200,000], -inf padding, per-row tables."""
    rows, n, ps, k = 64, 200_000, 64, 2048
    st = Stream(seed, 3)
    u = st.uniform(rows)
    lo, hi = math.log(512.0), math.log(float(n))
    lengths = np.clip(np.floor(np.exp(lo + u * (hi - lo))), 512, n).astype(np.int32)
    scores = np.empty((rows, n), np.float32)
    for r in range(rows):
        row = _f32(Stream(seed, 1, r).normal(n))
        row[lengths[r]:] = -np.inf
        scores[r] = row
    pages = n // ps                             # 3,125
    bt = page_permutation_tables(Stream(seed, 2), rows, pages)
    return Workload("c4_64_mixed", scores, lengths, bt, pages, ps, k, seed)


def make_c5(seed: int = 5) -> Workload:
    """256 x 131,072 adversarial ties, four groups of 64 rows."""
    rows, n, ps, k = 256, 131_072, 64, 2048
    scores = np.empty((rows, n), np.float32)
    for r in range(rows):
        st = Stream(seed, 1, r)
        g = r // 64
        if g == 0:                              # one value repeated
            scores[r] = _f32(st.normal(1))[0]
        elif g == 1:                            # 16 distinct values, uniform pick
            vals = _f32(st.normal(16))
            scores[r] = vals[st.below(n, 16)]
        elif g == 2:                            # 1 + U[0, 2^-12): one fp16 bin
            scores[r] = _f32(1.0 + st.below(n, 2048) * 2.0 ** -23)
        else:                                   # N(0,1) sorted descending
            scores[r] = np.sort(_f32(st.normal(n)))[::-1]
    pages = n // ps                             # 2,048
    bt = page_permutation_tables(Stream(seed, 2), rows, pages)
    lengths = np.full(rows, n, np.int32)
    return Workload("c5_256x131k_adversarial", scores, lengths, bt, pages, ps, k, seed)


def make_cp_shard(seed: int = 6) -> Workload:
    """7 x 125,000: one GPU's share of the 1M rows under 8-way context sharding."""
    rows, n, ps, k = 7, 125_000, 64, 2048
    scores = np.empty((rows, n), np.float32)
    for r in range(rows):
        st = Stream(seed, 1, r)
        row = _f32(st.normal(n))
        pos = st.permutation(n)[: n // 100]
        row[pos] = _f32(3.0 + st.below(n // 100, 2098) * 2.0 ** -22)
        scores[r] = row
    pages = (n + ps - 1) // ps
    bt = page_permutation_tables(Stream(seed, 2), 1, pages)
    lengths = np.full(rows, n, np.int32)
    return Workload("cp8_7x125k_shard", scores, lengths, bt, 0, ps, k, seed)


def make_prefill(rows: int = 4096, prefix: int = 80_000, seed: int = 7) -> Workload:
    """A prefill chunk of one request: ``rows`` query tokens whose causal rows
    see ``prefix + t`` positions (t = 0 .. rows-1), N(0,1) scores, -inf past
    each row's length, one shared random page table of 64-token pages.
    This is the ragged prefill top-k the lmsys.org page lists as next work
    (section "What's Next"), at its 80K context length.

    At this size (344 M scores) Box-Muller per score would dominate the run,
    so scores are drawn from a table of 2^20 N(0,1) values, two 20-bit table
    indices per SplitMix64 output (bits 44-63 and 12-31). Values then repeat
    within a row (about 3,400 equal pairs per 80K row), which also exercises
    the position tie-break."""
    ps, k = 64, 2048
    lengths = (prefix + np.arange(rows)).astype(np.int32)
    stride = int(lengths[-1]) + (-int(lengths[-1]) % 4) if rows else 4
    scores = np.empty((rows, stride), np.float32)
    table = _f32(Stream(seed, 5).normal(1 << 20))
    block = 64
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        n = (r1 - r0) * stride
        u = Stream(seed, 1, r0).u64((n + 1) // 2)
        idx = np.empty(2 * u.size, np.int64)
        idx[0::2] = (u >> np.uint64(44)).astype(np.int64)
        idx[1::2] = ((u >> np.uint64(12)) & np.uint64(0xFFFFF)).astype(np.int64)
        scores[r0:r1] = table[idx[:n]].reshape(r1 - r0, stride)
    for r in range(rows):
        scores[r, lengths[r]:] = -np.inf
    bt = page_permutation_tables(Stream(seed, 2), 1, (stride + ps - 1) // ps)
    return Workload(f"prefill_{rows}x{prefix // 1000}k", scores, lengths, bt, 0, ps, k, seed)


def make_plan_split(seed: int = 8, rows: int = 600, long_len: int = 300_000) -> Workload:
    """More rows than the selection kernel plans by itself (so the planning
    kernel writes the work list), four of them long enough to be split across
    workgroups and the rest between k + 1 and 30,000 positions. Per-row
    random page tables; N(0,1) scores, -inf padding."""
    ps, k = 64, 2048
    st = Stream(seed, 4)
    lengths = (k + 1 + st.below(rows, 30_000 - k)).astype(np.int32)
    long_rows = [rows // 8, 3 * rows // 8, 5 * rows // 8, 7 * rows // 8]
    lengths[long_rows] = long_len
    stride = long_len
    scores = np.full((rows, stride), -np.inf, np.float32)
    for r in range(rows):
        scores[r, : lengths[r]] = _f32(Stream(seed, 1, r).normal(int(lengths[r])))
    pages = (stride + ps - 1) // ps
    bt = page_permutation_tables(Stream(seed, 2), rows, pages)
    return Workload(f"plan_split_{rows}", scores, lengths, bt, pages, ps, k, seed)


CONFIGS = {
    1: make_c1,
    2: make_c2,
    3: make_c3,
    4: make_c4,
    5: make_c5,
}


def make_config(i: int, seed: int | None = None) -> Workload:
    """Config ``i`` in 1..5; the seed defaults to the config number."""
    return CONFIGS[i](i if seed is None else seed)


def random_case(seed: int, rows: int, max_len: int, *, k: int | None = None,
                page_size: int = 64, shared_table: bool = False,
                alphabet: int = 0, stride_pad: int = 0,
                special: bool = False, exact_len: bool = False) -> Workload:
    """A small random case for fuzzing.

    ``alphabet`` > 0 draws every score from that many distinct values (heavy
    ties). ``special`` mixes in +0.0, -0.0 and -inf. Lengths are uniform in
    [0, max_len] unless ``exact_len``.
    """
    st = Stream(seed, 9)
    if exact_len:
        lengths = np.full(rows, max_len, np.int32)
    else:
        lengths = st.below(rows, max_len + 1).astype(np.int32)
    stride = max_len + stride_pad
    if alphabet > 0:
        vals = _f32(st.normal(alphabet))
        scores = vals[st.below(rows * stride, alphabet)].reshape(rows, stride)
    else:
        scores = _f32(st.normal(rows * stride)).reshape(rows, stride)
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    if special:
        sel = st.below(rows * stride, 8).reshape(rows, stride)
        scores[sel == 0] = np.float32(0.0)
        scores[sel == 1] = np.float32(-0.0)
        scores[sel == 2] = -np.inf
    for r in range(rows):                       # junk beyond the valid prefix
        scores[r, lengths[r]:] = np.float32(1e30)
    pages = max(1, (stride + page_size - 1) // page_size)
    if shared_table:
        bt = page_permutation_tables(st, 1, pages)
        bt_stride = 0
    else:
        bt = page_permutation_tables(st, rows, pages)
        bt_stride = pages
    if k is None:
        k = int(st.below(1, 2048)[0]) + 1
    return Workload(f"rand{seed}", scores, lengths, bt, bt_stride, page_size, k, seed)


# --- indexer key prologue inputs ---------------------------------------------

@dataclasses.dataclass
class KeyPrologueInputs:
    """One batch of new key tokens for the indexer key prologue.

    k_act:        uint16 [tokens, k_stride] BF16 bit patterns; the first `dim`
                  of each row are the token's key activations.
    weight, bias: float32 [dim] LayerNorm parameters.
    cos_sin:      float32 [max_pos, rope_dim]: per position, the cosines of the
                  rope_dim / 2 pair angles, then their sines (the rotary cache).
    positions:    int32 [tokens]; token_row: int32 [tokens] (-1 = padding).
    block_table:  int32 [rows, pages] (bt_row_stride = pages), or [1, pages]
                  shared (bt_row_stride = 0).
    num_slots:    physical cache slots (pages in the pool x page_size).
    """
    name: str
    k_act: np.ndarray
    dim: int
    weight: np.ndarray
    bias: np.ndarray
    eps: float
    cos_sin: np.ndarray
    rope_dim: int
    positions: np.ndarray
    token_row: np.ndarray
    block_table: np.ndarray
    bt_row_stride: int
    page_size: int
    num_slots: int
    seed: int

    @property
    def tokens(self) -> int:
        return int(self.positions.shape[0])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> BF16 bit patterns, round to nearest even (via FP32)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rnd = ((f >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((f + rnd) >> np.uint64(16)).astype(np.uint16)


def rotary_table(max_pos: int, rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """The serving engines' rotary cache: angle of pair i at position p is
    p * base^(-2i / rope_dim); row p = [cos of the pairs, sin of the pairs],
    evaluated in float64 and rounded to float32."""
    if rope_dim == 0:
        return np.zeros((max_pos, 0), np.float32)
    inv = base ** (-np.arange(0, rope_dim, 2, dtype=np.float64) / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make_key_prologue(tokens: int, seed: int = 11, *, dim: int = 128, rope_dim: int = 64,
                      rows: int = 1, page_size: int = 64, k_stride: int | None = None,
                      pad_every: int = 0, max_pos: int | None = None, shared_table: bool = False,
                      act_scale: float = 3.0) -> KeyPrologueInputs:
    """`tokens` new key tokens spread over `rows` requests; request r's tokens
    take consecutive positions from a random prefix (a chunk of prefill, or a
    few verify tokens of decode). Activations are N(0, act_scale^2) plus a
    per-token offset (so LayerNorm has a mean to remove) and a few outlier
    channels, rounded to BF16. Every request owns a random set of physical
    pages of one shared pool; `pad_every` > 0 marks every pad_every-th token as
    padding (row -1)."""
    st = Stream(seed, 31)
    ks = dim if k_stride is None else k_stride
    x = st.normal(tokens * dim).reshape(tokens, dim) * act_scale
    x += st.normal(tokens)[:, None] * 0.5
    hot = st.below(4, dim)
    x[:, hot] *= 8.0
    k_act = np.zeros((tokens, ks), np.uint16)
    k_act[:, :dim] = bf16_bits(x)
    weight = _f32(1.0 + 0.1 * st.normal(dim))
    bias = _f32(0.05 * st.normal(dim))
    # tokens split as evenly as possible over rows, consecutive positions each
    per = np.full(rows, tokens // rows, np.int64)
    per[: tokens % rows] += 1
    start = st.below(rows, 4096) if rows > 1 or tokens < 4096 else np.zeros(1, np.int64)
    token_row = np.repeat(np.arange(rows, dtype=np.int64), per)
    positions = np.concatenate([start[r] + np.arange(per[r]) for r in range(rows)]) if tokens else \
        np.zeros(0, np.int64)
    need_pos = int(positions.max()) + 1 if tokens else 1
    mp = max(need_pos, max_pos or 0)
    cos_sin = rotary_table(mp, rope_dim)
    pages = (mp + page_size - 1) // page_size
    if shared_table:
        pool = pages
        bt = st.permutation(pool)[None, :].astype(np.int32)
        stride = 0
    else:
        pool = rows * pages
        bt = st.permutation(pool).reshape(rows, pages).astype(np.int32)
        stride = pages
    if pad_every > 0:
        token_row[::pad_every] = -1
    return KeyPrologueInputs(f"key_prologue_{tokens}t_{rows}r", k_act, dim, weight, bias, 1e-6, cos_sin,
                             rope_dim, positions.astype(np.int32), token_row.astype(np.int32), bt, stride,
                             page_size, pool * page_size, seed)


# --- indexer score (MQA logits) inputs ---------------------------------------

@dataclasses.dataclass
class LogitsInputs:
    """Query tokens and a paged FP8 key cache for the indexer's MQA logits.

    q_bf16:   uint16 [tokens, heads, 128] BF16 bits (query prologue input);
    w_raw:    float32 [tokens, heads] raw head-gate weights;
    q_codes:  uint8 [tokens, heads, 128] FP8 E4M3 codes and w: float32
              [tokens, heads] scaled gate weights (logits inputs: random
              codes, drawn independently of q_bf16);
    k_fp8:    uint8 [slots, 128] E4M3 codes; k_scale: float32 [slots] > 0;
    lengths:  int32 [tokens]: token t scores key positions [0, lengths[t]);
    block_table: int32 [1, pages] shared by the tokens (one request).
    """
    name: str
    q_bf16: np.ndarray
    w_raw: np.ndarray
    q_codes: np.ndarray
    w: np.ndarray
    k_fp8: np.ndarray
    k_scale: np.ndarray
    lengths: np.ndarray
    block_table: np.ndarray
    page_size: int
    positions: np.ndarray
    cos_sin: np.ndarray
    rope_dim: int
    seed: int

    @property
    def tokens(self) -> int:
        return int(self.q_codes.shape[0])

    @property
    def heads(self) -> int:
        return int(self.q_codes.shape[1])


def _e4m3_codes(st: Stream, n: int, lo: int = 0x20, span: int = 0x50) -> np.ndarray:
    """Random finite E4M3 codes: magnitude codes in [lo, lo + span) (exponents
    4 to 13 by default, values 2^-3 .. 2^6), random sign. Codes only: no
    value arithmetic."""
    mag = (lo + st.below(n, span)).astype(np.uint8)
    sign = (st.below(n, 2) << 7).astype(np.uint8)
    return mag | sign


def make_logits(tokens: int, keys: int, seed: int = 21, *, heads: int = 64, page_size: int = 64,
                rope_dim: int = 64, with_table: bool = True) -> LogitsInputs:
    """`tokens` query tokens of one request (verify: the last `tokens`
    positions of a context of `keys`), each scoring the causal prefix
    [0, keys - tokens + 1 + t); keys live in a randomly paged FP8 cache.
    with_table=False skips the rotary table (only the query prologue reads it)."""
    st = Stream(seed, 41)
    d = 128
    q_bf16 = bf16_bits(st.normal(tokens * heads * d).reshape(tokens, heads, d) * 2.0)
    w_raw = _f32(st.normal(tokens * heads).reshape(tokens, heads))
    q_codes = _e4m3_codes(st, tokens * heads * d).reshape(tokens, heads, d)
    w = _f32(st.normal(tokens * heads).reshape(tokens, heads) * 0.05)
    pages = (keys + page_size - 1) // page_size
    pool = pages + 3
    bt = st.permutation(pool)[:pages][None, :].astype(np.int32)
    slots = pool * page_size
    k_fp8 = _e4m3_codes(st, slots * d).reshape(slots, d)
    k_scale = _f32(0.001 + st.uniform(slots) * 0.01)
    lengths = (keys - tokens + 1 + np.arange(tokens)).astype(np.int32)
    positions = (lengths - 1).astype(np.int32)
    cos_sin = rotary_table(int(keys), rope_dim) if with_table else np.zeros((0, rope_dim), np.float32)
    return LogitsInputs(f"logits_{tokens}x{keys}", q_bf16, w_raw, q_codes, w, k_fp8, k_scale, lengths, bt,
                        page_size, positions, cos_sin, rope_dim, seed)
