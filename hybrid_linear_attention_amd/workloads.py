"""Seeded synthetic inputs for the GDN mixer core.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the method's arithmetic.  Both the GPU path and the CPU oracle are
fed the tensors it returns (CPU torch tensors; the oracle widens them exactly to
fp64, the GPU path copies them to the device).

Generator: ``numpy.random.Generator(PCG64(seed))`` (seed 1234 + workload id for
the five named workloads) draws the integers (lengths, permutations) and one
key per tensor; a tensor's normal values are float32 draws from keyed block
streams (``_normal``), scaled by the standard deviation in float32 and rounded
to bf16 round-to-nearest-even by torch on the CPU where the storage dtype is
bf16.  Draw order is fixed and documented in ``make_gdn_case``.

Shapes follow the tutorial page's data-structure table (section 01): q/k
[T,16,128], v/z [T,48,128], a/b [T,48], state [R,48,128,128] fp32, conv history
[R,10240,3].
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

# Bit patterns written into slots no request uses, so that a stray write or
# read is visible: a quiet-NaN payload in each storage format.
STATE_SENTINEL_BITS = 0x7FC0DEAD  # float32
HIST_SENTINEL_BITS_F32 = 0x7FC0BEEF
HIST_SENTINEL_BITS_BF16 = 0x7FDE


@dataclass
class GdnDims:
    num_k_heads: int
    num_v_heads: int
    head_dim_k: int
    head_dim_v: int
    conv_taps: int = 4

    @property
    def conv_channels(self) -> int:
        return 2 * self.num_k_heads * self.head_dim_k + self.num_v_heads * self.head_dim_v


FULL_DIMS = GdnDims(16, 48, 128, 128, 4)
TINY_DIMS = GdnDims(2, 6, 16, 16, 4)


@dataclass
class GdnCase:
    dims: GdnDims
    x_qkv: torch.Tensor          # [T, Cqkv]  conv input (pre-conv q|k|v)
    z: torch.Tensor              # [T, Hv, dv]
    a: torch.Tensor              # [T, Hv]    raw decay projection
    b: torch.Tensor              # [T, Hv]    raw write-strength projection
    conv_w: torch.Tensor         # [Cqkv, taps], conv_w[c, i] multiplies x[t-i]
    gamma: torch.Tensor          # [dv] gated-norm gain
    conv_pool: torch.Tensor      # [num_slots, Cqkv, taps-1] oldest -> newest
    state_pool: torch.Tensor     # [num_slots, Hv, dv, dk] fp32
    qsl: torch.Tensor            # [N+1] int32 query_start_loc
    slot_ids: torch.Tensor       # [N] int32
    has_initial: torch.Tensor    # [N] uint8
    used_slots: List[int] = field(default_factory=list)
    meta: Dict = field(default_factory=dict)

    @property
    def num_tokens(self) -> int:
        return int(self.x_qkv.shape[0])

    @property
    def num_reqs(self) -> int:
        return int(self.slot_ids.shape[0])

    @property
    def num_slots(self) -> int:
        return int(self.state_pool.shape[0])


_BLOCK = 1 << 22          # normal draws per keyed block
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _normal(rng, shape, std, dtype, mean=0.0):
    """Normal draws N(mean, std) of one tensor, stored as ``dtype`` (RNE for
    bf16).

    The tensor takes one 63-bit key from the workload's stream ``rng``; its
    elements, in blocks of 2^22, are float32 standard normals from
    ``PCG64(SeedSequence([key, block]))``, scaled by std and shifted by mean in
    float32.  The blocks are independent streams, so they are filled by a
    thread pool and the values do not depend on the thread count."""
    key = int(rng.integers(0, 2 ** 63 - 1))
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=dtype)

    def fill(j):
        s = j * _BLOCK
        e = min(n, s + _BLOCK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([key, j])))
        blk = g.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        if mean != 0.0:
            blk += np.float32(mean)
        out[s:e] = torch.from_numpy(blk).to(dtype)

    nblk = (n + _BLOCK - 1) // _BLOCK
    if nblk <= 1:
        for j in range(nblk):
            fill(j)
    else:
        with ThreadPoolExecutor(min(_THREADS, nblk)) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def _fill_bits(t: torch.Tensor, bits: int):
    if t.dtype == torch.float32:
        t.view(torch.int32).fill_(np.int32(np.uint32(bits).view(np.int32)))
    elif t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(np.int16(np.uint16(bits).view(np.int16)))
    else:
        raise TypeError(t.dtype)


def make_gdn_case(seed: int, dims: GdnDims, lengths: Optional[List[int]] = None,
                  *, random_lengths=None, num_slots: Optional[int] = None,
                  permute_slots: bool = False, act_dtype=torch.bfloat16,
                  pool_dtype=None, weight_dtype=None, state_std: float = 0.0,
                  hist_std: float = 0.0, has_initial: Optional[bool] = None,
                  conv_w_std: float = 0.5, gamma_std: float = 0.0,
                  target_total=None, a_mean: float = 0.0) -> GdnCase:
    """Build one seeded GDN-core workload.

    Draw order from one PCG64 stream:
      1. request lengths (only if ``random_lengths=(n, lo, hi)``: integers in
         [lo, hi] inclusive; with ``target_total=(total, frac)`` the n lengths
         are drawn again, from the same stream, until their sum lies within
         frac of total),
      2. slot permutation of range(num_slots) (only if ``permute_slots``),
      3. initial state of each used slot, in request order (if state_std > 0),
      4. conv history of each used slot, in request order (if hist_std > 0),
      5. x_qkv [T, Cqkv], 6. z [T, Hv, dv] ~ N(0,1), 7. a [T, Hv] ~ N(a_mean, 1),
         8. b [T, Hv] ~ N(0,1),
      9. conv_w [Cqkv, taps] ~ N(0, conv_w_std),
     10. gamma = 1 + N(0, gamma_std) (only if gamma_std > 0, else exactly 1).
    Unused slots carry a NaN sentinel bit pattern.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if random_lengths is not None:
        n, lo, hi = random_lengths
        while True:
            lengths = [int(x) for x in rng.integers(lo, hi + 1, n)]
            if target_total is None or abs(sum(lengths) - target_total[0]) <= target_total[1] * target_total[0]:
                break
    assert lengths is not None
    nreq = len(lengths)
    if num_slots is None:
        num_slots = nreq
    if permute_slots:
        perm = rng.permutation(num_slots)
        slot_ids = [int(x) for x in perm[:nreq]]
    else:
        slot_ids = list(range(nreq))
    pool_dtype = pool_dtype or act_dtype
    weight_dtype = weight_dtype or act_dtype
    C = dims.conv_channels
    nh = dims.conv_taps - 1
    Hv, dv, dk = dims.num_v_heads, dims.head_dim_v, dims.head_dim_k
    T = int(sum(lengths))
    if has_initial is None:
        has_initial = state_std > 0 or hist_std > 0

    state_pool = torch.empty((num_slots, Hv, dv, dk), dtype=torch.float32)
    _fill_bits(state_pool, STATE_SENTINEL_BITS)
    conv_pool = torch.empty((num_slots, C, nh), dtype=pool_dtype)
    _fill_bits(conv_pool, HIST_SENTINEL_BITS_BF16 if pool_dtype == torch.bfloat16
               else HIST_SENTINEL_BITS_F32)
    for s in slot_ids:
        if state_std > 0:
            state_pool[s] = _normal(rng, (Hv, dv, dk), state_std, torch.float32)
        else:
            state_pool[s].zero_()
    for s in slot_ids:
        if hist_std > 0:
            conv_pool[s] = _normal(rng, (C, nh), hist_std, pool_dtype)
        else:
            conv_pool[s].zero_()

    x_qkv = _normal(rng, (T, C), 1.0, act_dtype)
    z = _normal(rng, (T, Hv, dv), 1.0, act_dtype)
    a = _normal(rng, (T, Hv), 1.0, act_dtype, mean=a_mean)
    b = _normal(rng, (T, Hv), 1.0, act_dtype)
    conv_w = _normal(rng, (C, dims.conv_taps), conv_w_std, weight_dtype)
    if gamma_std > 0:
        gamma = (1.0 + _normal(rng, (dv,), gamma_std, torch.float32)).to(weight_dtype)
    else:
        gamma = torch.ones(dv, dtype=weight_dtype)

    qsl = torch.zeros(nreq + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return GdnCase(dims=dims, x_qkv=x_qkv, z=z, a=a, b=b, conv_w=conv_w,
                   gamma=gamma, conv_pool=conv_pool, state_pool=state_pool, qsl=qsl,
                   slot_ids=torch.tensor(slot_ids, dtype=torch.int32),
                   has_initial=torch.full((nreq,), 1 if has_initial else 0,
                                          dtype=torch.uint8),
                   used_slots=slot_ids, meta=dict(seed=seed, lengths=lengths))


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------
def tiny_core(seed: int = 1234) -> GdnCase:
    """Tiny GDN core, fp32 throughout: one sequence of 64 tokens, 2 key heads,
    6 value heads, d_k = d_v = 16, 4-tap conv, zero history and state."""
    return make_gdn_case(seed, TINY_DIMS, [64], act_dtype=torch.float32,
                         pool_dtype=torch.float32, weight_dtype=torch.float32)


def decode_r64(seed: int = 1235) -> GdnCase:
    """Decode step at full shapes: 64 requests x 1 token, 16/48 heads, d = 128,
    state [64,48,128,128] ~ N(0, 0.02) fp32, conv history [64,10240,3] ~ N(0,1)
    bf16, slot r = request r."""
    return make_gdn_case(seed, FULL_DIMS, [1] * 64, state_std=0.02, hist_std=1.0)


def prefill_4096(seed: int = 1236) -> GdnCase:
    """Single-sequence prefill at full shapes: T = 4096, zero state and history."""
    return make_gdn_case(seed, FULL_DIMS, [4096])


VARLEN16_TOTAL = 66000  # the packed batch's stated size, about 66k tokens


def prefill_varlen16(seed: int = 1237) -> GdnCase:
    """Packed varlen prefill: 16 requests of lengths uniform in [256, 8192]
    whose total is about 66k tokens (length vectors are redrawn from the stream
    until the sum is within 2% of 66,000; this seed: 66,292 tokens on the 20th
    draw), slots a seeded permutation of a 64-slot pool, nonzero initial state
    ~ N(0, 0.02) and conv history ~ N(0, 1) per used slot."""
    return make_gdn_case(seed, FULL_DIMS, random_lengths=(16, 256, 8192),
                         target_total=(VARLEN16_TOTAL, 0.02), num_slots=64,
                         permute_slots=True, state_std=0.02, hist_std=1.0)


def spec_verify_r64(seed: int = 1239, tokens: int = 4) -> GdnCase:
    """Speculative verify at full shapes: 64 requests of `tokens` tokens each (the
    last accepted token and tokens - 1 drafts), state ~ N(0, 0.02) and history
    ~ N(0, 1) in slots 0..63 (request r in slot r); slots 64 + tokens r + j
    receive the state and history after token j of request r
    (meta["spec_slots"], int32 [64, tokens])."""
    R = 64
    case = make_gdn_case(seed, FULL_DIMS, [tokens] * R, num_slots=R * (tokens + 1),
                         state_std=0.02, hist_std=1.0)
    case.meta["spec_slots"] = (R + torch.arange(R * tokens, dtype=torch.int32)).reshape(R, tokens)
    return case


# gate values whose maps saturate in float32 and in fp64 alike: softplus(-30)
# and sigmoid(-30) are ~1e-13, so alpha -> 1 and beta -> 0 (and the reverse at +30)
GATE_SATURATE = 30.0
EDGE_KINDS = ("frozen", "write", "forget", "zero_qk", "weak_decay")


def edge_case(kind: str, seed: int, lengths: List[int], num_slots: Optional[int] = None,
              dims: GdnDims = FULL_DIMS) -> GdnCase:
    """Workloads at the gates' and inputs' extremes (the regimes of the tutorial
    page's GDN state lab: a small decay erases the state, a large one keeps
    it; the delta write stores the prediction error).  Built on make_gdn_case
    (state ~ N(0, 0.02), history ~ N(0, 1), slots permuted), then:

      frozen      a = b = -30 everywhere: alpha ~ 1, beta ~ 0 (nothing written)
      write       b = +30: beta ~ 1 (a full delta write of a unit k)
      forget      a = +30: alpha ~ 0 (only the newest write survives)
      zero_qk     the q and k conv inputs of every token of the first request,
                  and of its history, are zero, and its a is lowered by 4 (a weak
                  decay, so that the pure decay it undergoes stays well inside
                  float32's range); in every other request, the q and k inputs
                  of a run of tokens from a quarter to three quarters of its
                  length are zero (q = k = 0 from the run's fourth token on)
      weak_decay  a ~ N(-4, 1): alpha ~ 0.98, a long memory
    """
    if kind not in EDGE_KINDS:
        raise ValueError(kind)
    case = make_gdn_case(seed, dims, list(lengths), num_slots=num_slots or len(lengths) + 3,
                         permute_slots=True, state_std=0.02, hist_std=1.0,
                         a_mean=-4.0 if kind == "weak_decay" else 0.0)
    if kind == "frozen":
        case.a.fill_(-GATE_SATURATE)
        case.b.fill_(-GATE_SATURATE)
    elif kind == "write":
        case.b.fill_(GATE_SATURATE)
    elif kind == "forget":
        case.a.fill_(GATE_SATURATE)
    elif kind == "zero_qk":
        nqk = 2 * dims.num_k_heads * dims.head_dim_k
        qsl = case.qsl.tolist()
        for r in range(case.num_reqs):
            t0, t1 = qsl[r], qsl[r + 1]
            if r == 0:
                case.x_qkv[t0:t1, :nqk] = 0
                case.conv_pool[case.used_slots[0], :nqk] = 0
                case.a[t0:t1] -= 4.0
            else:
                L = t1 - t0
                case.x_qkv[t0 + L // 4:t0 + (3 * L) // 4, :nqk] = 0
    case.meta["edge"] = kind
    return case


@dataclass
class LayerCase:
    core: GdnCase                 # GDN-core tensors (x_qkv/z/a/b unused: made by the projection)
    X: torch.Tensor               # [T, hidden] bf16
    gamma_in: torch.Tensor        # [hidden]
    W_qkvz: torch.Tensor          # [hidden, 2*Hk*dk + 2*Hv*dv]
    W_ba: torch.Tensor            # [hidden, 2*Hv]  (b columns then a columns)
    W_o: torch.Tensor             # [Hv*dv, hidden]
    num_prefill: int = 0
    prefill_len: int = 0
    num_decode: int = 0


def layer_mixed(seed: int = 1238, hidden: int = 5120, num_prefill: int = 8,
                prefill_len: int = 2048, num_decode: int = 256,
                dims: GdnDims = FULL_DIMS) -> LayerCase:
    """Full GDN layer block at hidden 5120, mixed batch: 8 prefill requests of
    2048 tokens (zero state and history) then 256 decode requests of 1 token
    (state ~ N(0, 0.02), history ~ N(0, 1)).  Weights ~ N(0, 0.02), X ~ N(0, 1),
    norm gains 1 + N(0, 0.02), conv taps ~ N(0, 0.5).

    Draw order: decode-slot states, decode-slot histories, X, W_qkvz, W_ba, W_o,
    conv_w, gamma_in, gamma_out.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    C = dims.conv_channels
    nh = dims.conv_taps - 1
    Hv, dv, dk = dims.num_v_heads, dims.head_dim_v, dims.head_dim_k
    nreq = num_prefill + num_decode
    lengths = [prefill_len] * num_prefill + [1] * num_decode
    T = sum(lengths)
    state_pool = torch.zeros((nreq, Hv, dv, dk), dtype=torch.float32)
    conv_pool = torch.zeros((nreq, C, nh), dtype=torch.bfloat16)
    for s in range(num_prefill, nreq):
        state_pool[s] = _normal(rng, (Hv, dv, dk), 0.02, torch.float32)
    for s in range(num_prefill, nreq):
        conv_pool[s] = _normal(rng, (C, nh), 1.0, torch.bfloat16)
    X = _normal(rng, (T, hidden), 1.0, torch.bfloat16)
    W_qkvz = _normal(rng, (hidden, C + Hv * dv), 0.02, torch.bfloat16)
    W_ba = _normal(rng, (hidden, 2 * Hv), 0.02, torch.bfloat16)
    W_o = _normal(rng, (Hv * dv, hidden), 0.02, torch.bfloat16)
    conv_w = _normal(rng, (C, dims.conv_taps), 0.5, torch.bfloat16)
    gamma_in = (1.0 + _normal(rng, (hidden,), 0.02, torch.float32)).to(torch.bfloat16)
    gamma_out = (1.0 + _normal(rng, (dv,), 0.02, torch.float32)).to(torch.bfloat16)
    qsl = torch.zeros(nreq + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    has_initial = torch.tensor([0] * num_prefill + [1] * num_decode, dtype=torch.uint8)
    empty = torch.empty(0)
    core = GdnCase(dims=dims, x_qkv=empty, z=empty, a=empty, b=empty, conv_w=conv_w,
                   gamma=gamma_out, conv_pool=conv_pool, state_pool=state_pool,
                   qsl=qsl, slot_ids=torch.arange(nreq, dtype=torch.int32),
                   has_initial=has_initial, used_slots=list(range(nreq)),
                   meta=dict(seed=seed, lengths=lengths))
    return LayerCase(core=core, X=X, gamma_in=gamma_in, W_qkvz=W_qkvz, W_ba=W_ba,
                     W_o=W_o, num_prefill=num_prefill, prefill_len=prefill_len,
                     num_decode=num_decode)


@dataclass
class GqaDims:
    """Full-attention layer geometry (tutorial page, section 03 GQA lab):
    24 query heads, 4 key/value heads, 256 dims, 64 of them rotated."""
    num_q_heads: int = 24
    num_kv_heads: int = 4
    head_dim: int = 256
    rotary_dim: int = 64


GQA_DIMS = GqaDims()


@dataclass
class GqaCase:
    dims: GqaDims
    q: torch.Tensor              # [R, Hq, D]   new token's query (before rotation)
    gate: torch.Tensor           # [R, Hq, D]   output-gate projection
    k: torch.Tensor              # [R, Hkv, D]  new token's key (before rotation)
    v: torch.Tensor              # [R, Hkv, D]
    k_cache: torch.Tensor        # [num_pages, Hkv, page_size, D] bf16
    v_cache: torch.Tensor        # [num_pages, Hkv, page_size, D] bf16
    block_tables: torch.Tensor   # [R, max_pages] int32 (-1 past each request's pages)
    context_lens: torch.Tensor   # [R] int32, new token included
    page_size: int
    max_context_len: int
    rope_theta: float = 10000.0
    k_scale: float = 1.0         # an e4m3 cache: code c stands for scale * e4m3(c)
    v_scale: float = 1.0

    @property
    def num_reqs(self) -> int:
        return int(self.context_lens.numel())


def make_gqa_case(seed: int, lens: List[int], page_size: int, dims: GqaDims = GQA_DIMS,
                  spare_pages: int = 3, act_dtype=torch.bfloat16, max_context_len: Optional[int] = None,
                  std: float = 1.0, rope_theta: float = 10000.0, cache_dtype=torch.bfloat16,
                  k_scale: float = 1.0, v_scale: float = 1.0) -> GqaCase:
    """Draw order: q, gate, k, v, k_cache, v_cache (normal, `std` for q, k and
    the K cache, 1 otherwise), then one permutation of the physical pages that
    deals each request its pages in table order; spare pages stay unused.
    cache_dtype torch.float8_e4m3fn: the cache draws are converted by torch
    (nearest-even) and kept as uint8 codes, read at k_scale / v_scale."""
    rng = np.random.default_rng(seed)
    R, Hq, Hkv, D = len(lens), dims.num_q_heads, dims.num_kv_heads, dims.head_dim
    q = _normal(rng, (R, Hq, D), std, act_dtype)
    gate = _normal(rng, (R, Hq, D), 1.0, act_dtype)
    k = _normal(rng, (R, Hkv, D), std, act_dtype)
    v = _normal(rng, (R, Hkv, D), 1.0, act_dtype)
    need = [(L + page_size - 1) // page_size for L in lens]
    num_pages = sum(need) + spare_pages
    if cache_dtype == torch.float8_e4m3fn:
        k_cache = _normal(rng, (num_pages, Hkv, page_size, D), std, torch.float32).to(cache_dtype).view(torch.uint8)
        v_cache = _normal(rng, (num_pages, Hkv, page_size, D), 1.0, torch.float32).to(cache_dtype).view(torch.uint8)
    else:
        k_cache = _normal(rng, (num_pages, Hkv, page_size, D), std, torch.bfloat16)
        v_cache = _normal(rng, (num_pages, Hkv, page_size, D), 1.0, torch.bfloat16)
    perm = rng.permutation(num_pages)
    max_pages = max(need) + 1
    bt = np.full((R, max_pages), -1, np.int32)
    at = 0
    for r, n in enumerate(need):
        bt[r, :n] = perm[at:at + n]
        at += n
    return GqaCase(dims=dims, q=q, gate=gate, k=k, v=v, k_cache=k_cache, v_cache=v_cache,
                   block_tables=torch.from_numpy(bt), context_lens=torch.tensor(lens, dtype=torch.int32),
                   page_size=page_size,
                   max_context_len=max(lens) if max_context_len is None else max_context_len,
                   rope_theta=rope_theta, k_scale=k_scale, v_scale=v_scale)


def gqa_decode_r64(seed: int = 1240, page_size: int = 16) -> GqaCase:
    """64 decoding requests with context lengths uniform in [1024, 3072]
    (about 131k cached positions in all: the page's logical-KV example of
    4 GiB at 2 KiB per position per attention layer over 16 layers), pages of
    16 positions."""
    lens = np.random.default_rng(seed).integers(1024, 3073, 64).tolist()
    return make_gqa_case(seed + 1, lens, page_size)


def gqa_decode_r64_fp8(seed: int = 1240, page_size: int = 16) -> GqaCase:
    """The same 64 requests with an fp8 e4m3 KV cache (the server profile's KV
    dtype), scales 1."""
    lens = np.random.default_rng(seed).integers(1024, 3073, 64).tolist()
    return make_gqa_case(seed + 1, lens, page_size, cache_dtype=torch.float8_e4m3fn)


WORKLOADS = {
    "tiny_core": tiny_core,
    "decode_r64": decode_r64,
    "prefill_4096": prefill_4096,
    "prefill_varlen16": prefill_varlen16,
    "layer_mixed": layer_mixed,
    "spec_verify_r64": spec_verify_r64,
    "gqa_decode_r64": gqa_decode_r64,
    "gqa_decode_r64_fp8": gqa_decode_r64_fp8,
}
