"""fp64 CPU oracle of the GQA layer's decode core — TEST INFRASTRUCTURE ONLY.

The full-attention layers that sit between the GDN layers ("Qwen3.8-27B: from
model structure to the vLLM inference dataflow", section 03 MEMORY LABS, GQA /
attention lab, and section 04 PRECISION & CACHE): 24 query heads of 256 and
4 key/value heads of 256, query heads 6j .. 6j+5 sharing key/value head j;
attention softmax(q k^T / sqrt(256)) v over the request's positions; partial
RoPE rotating 64 of each head's 256 dimensions; a sigmoid output gate ahead of
the output projection; K and V held in a paged cache (the PagedAttention card
of section 05 and the glossary's KV page: a logical position maps through the
request's block table to a fixed-size physical page).

One decode step per request r with context length L (the new token included):
  1. q and k of the new token are rotated at position L - 1;
  2. k (rotated) and v are written to the cache at position L - 1;
  3. each query head attends over positions 0 .. L - 1 of its key/value head;
  4. y = o * sigmoid(gate).

Readings taken where the pages are silent (listed in the design notes):
  * rotation pairs dimension i with i + 32 (the rotate-half convention) over the
    first 64 dimensions; pair i turns by position * theta^(-2i/64), theta an
    argument;
  * no q/k normalisation before the rotation (the pages name none);
  * the gate is elementwise over the attention output [Hq, 256];
  * the new token's position is L - 1;
  * cache layout [num_pages, Hkv, page_size, 256]; the stored value of the
    rotated k is its round-to-nearest-even in the cache dtype;
  * an fp8 cache (the server profile's e4m3, section 04) holds OCP e4m3 codes of
    x / scale with one scale per cache (k_scale, v_scale), rounded to nearest-even
    and saturated at +-448; a code c stands for scale * e4m3(c).
"""
import numpy as np

from .oracle import round_bf16


E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Values of OCP e4m3 codes (uint8): sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); 0x7f and 0xff are NaN;
    there is no infinity."""
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((c & 0x7f) == 0x7f, np.nan, s * mag)


def e4m3_round(x):
    """x (fp64) rounded to the nearest e4m3 value, ties to even, saturated at
    +-448: the value the cache stores for x (at scale 1)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # the spacing of e4m3 values around a: 2^(e - 3) in binade [2^e, 2^(e+1)),
    # 2^-9 for the subnormals below 2^-6
    e = np.frexp(np.where(a > 0, a, 1.0))[1].astype(np.float64) - 1.0
    q = np.exp2(np.maximum(e, -6.0) - 3.0)
    r = np.rint(a / q) * q            # rint: round half to even; a / q is exact
    r = np.minimum(r, E4M3_MAX)
    return np.where(a == 0, 0.0 * x, np.copysign(r, x))


def e4m3_encode(x):
    """Codes of the e4m3 values nearest to x (ties to even, saturating); -0 keeps
    its sign (0x80)."""
    r = e4m3_round(x)
    pos = e4m3_decode(np.arange(0x7f))          # codes 0x00 .. 0x7e, increasing
    c = np.searchsorted(pos, np.abs(r)).astype(np.uint8)
    return np.where(np.signbit(r), c | np.uint8(0x80), c).astype(np.uint8)


def rope_partial(x, positions, rotary_dim, theta):
    """Rotate the first rotary_dim dims of every head of x [N, H, D] (fp64) at
    positions [N]: pair i (i < rotary_dim/2) is (x_i, x_{i + rotary_dim/2}),
    turned by angle position * theta^(-2i/rotary_dim).  Dims >= rotary_dim pass
    through."""
    x = np.array(x, dtype=np.float64, copy=True)
    half = rotary_dim // 2
    freq = np.array([float(theta) ** (-2.0 * i / rotary_dim) for i in range(half)])
    ang = np.asarray(positions, dtype=np.float64)[:, None] * freq[None, :]   # [N, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[:, :, :half].copy()
    b = x[:, :, half:rotary_dim].copy()
    x[:, :, :half] = a * c - b * s
    x[:, :, half:rotary_dim] = b * c + a * s
    return x


def _check_paged(block_tables, context_lens, page_size, num_pages):
    """Host-side contract of a paged decode call: every context length >= 1 and
    covered by the request's block table, every page id in range, and the page
    that receives a request's new token read by no other request."""
    R, max_pages = block_tables.shape
    used = []
    for r in range(R):
        L = int(context_lens[r])
        if L < 1 or L > max_pages * page_size:
            raise ValueError(f"request {r}: context length {L} outside [1, {max_pages * page_size}]")
        pages = [int(p) for p in block_tables[r, :(L + page_size - 1) // page_size]]
        if min(pages) < 0 or max(pages) >= num_pages:
            raise ValueError(f"request {r}: page id out of range")
        used.append(pages)
    for r in range(R):
        wp = used[r][(int(context_lens[r]) - 1) // page_size]
        for r2 in range(R):
            if r2 != r and wp in used[r2]:
                raise ValueError(f"page {wp} written by request {r} is read by request {r2}")


def fp8_cache_round(scale):
    """The value an e4m3 cache with this scale stores for x."""
    return lambda x: scale * e4m3_round(np.asarray(x, dtype=np.float64) / scale)


def gqa_decode_paged(q, k, v, gate, k_cache, v_cache, block_tables, context_lens, page_size,
                     rotary_dim, theta, cache_round=round_bf16, v_round=None):
    """One GQA decode step over a paged KV cache.

    q, gate [R, Hq, D]; k, v [R, Hkv, D]; k_cache, v_cache [num_pages, Hkv,
    page_size, D] (the values the cache holds, decoded); block_tables
    [R, max_pages] int; context_lens [R] (new token included).  cache_round
    maps a new k to the value the K cache stores (round_bf16 for a bf16 cache,
    fp8_cache_round(k_scale) for an e4m3 one, None for exact); v_round the
    same for V (default: cache_round).
    Returns y [R, Hq, D], o [R, Hq, D] and the updated caches (copies)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    bt = np.asarray(block_tables)
    lens = np.asarray(context_lens)
    R, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    G = Hq // Hkv
    _check_paged(bt, lens, page_size, kc.shape[0])
    rnd = (lambda t: t) if cache_round is None else cache_round
    vrnd = rnd if v_round is None else v_round
    pos = lens.astype(np.int64) - 1
    qr = rope_partial(q, pos, rotary_dim, theta)
    kr = rope_partial(k, pos, rotary_dim, theta)

    # 2. append the new token
    for r in range(R):
        p = int(pos[r])
        page, off = int(bt[r, p // page_size]), p % page_size
        kc[page, :, off, :] = rnd(kr[r])
        vc[page, :, off, :] = vrnd(v[r])

    # 3. attention over the request's positions, read through the block table
    o = np.zeros((R, Hq, D))
    for r in range(R):
        L = int(lens[r])
        j = np.arange(L)
        pages = bt[r, j // page_size]
        offs = j % page_size
        for h in range(Hq):
            g = h // G
            K = kc[pages, g, offs, :]          # [L, D]
            V = vc[pages, g, offs, :]
            s = K @ qr[r, h] / np.sqrt(D)
            w = np.exp(s - s.max())
            o[r, h] = (w / w.sum()) @ V

    # 4. sigmoid output gate
    y = o / (1.0 + np.exp(-gate))
    return y, o, kc, vc
