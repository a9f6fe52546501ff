"""Small hand-built inputs for tests (no method arithmetic here)."""
import numpy as np

PAGE = 128
D = 128

# E4M3 codes for a few exact values (OCP E4M3FN encoding)
CODE = {0.0: 0x00, 0.5: 0x30, 1.0: 0x38, 2.0: 0x40, -0.5: 0xB0, -1.0: 0xB8, -2.0: 0xC0}


def varlen(seqlen_q, seqlen_k, block_tables=None, spare=0, seed=0):
    """cu_seqlens and a block table (random permutation unless given)."""
    sq = np.asarray(seqlen_q, np.int64)
    sk = np.asarray(seqlen_k, np.int64)
    B = len(sq)
    cu_q = np.zeros(B + 1, np.int32)
    cu_k = np.zeros(B + 1, np.int32)
    cu_q[1:] = np.cumsum(sq)
    cu_k[1:] = np.cumsum(sk)
    pages = (sk + PAGE - 1) // PAGE
    max_pages = int(pages.max())
    bt = np.full((B, max_pages), -1, np.int32)
    if block_tables is None:
        rng = np.random.default_rng(seed)
        perm = rng.permutation(int(pages.sum()) + spare).astype(np.int32)
        off = 0
        for b in range(B):
            bt[b, :pages[b]] = perm[off:off + pages[b]]
            off += pages[b]
    else:
        for b, row in enumerate(block_tables):
            bt[b, :len(row)] = row
    num_pages = int(pages.sum()) + spare
    return cu_q, cu_k, bt, num_pages


def random_codes(rng, shape, max_abs_code=0x5F):
    """Random finite E4M3 codes with |value| <= value(max_abs_code) (no NaN)."""
    mag = rng.integers(0, max_abs_code + 1, size=shape, dtype=np.int64)
    sign = rng.integers(0, 2, size=shape, dtype=np.int64) << 7
    return (mag | sign).astype(np.uint8)


def scatter_pages(rows, cu_k, bt, num_pages, tail_shape, fill=0x7F):
    """Logical token rows [total_k, *tail] -> physical pages [num_pages, 128, *tail]."""
    cache = np.full((num_pages, PAGE) + tuple(tail_shape), fill, np.uint8)
    for b in range(len(cu_k) - 1):
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        for t in range(k1 - k0):
            cache[bt[b, t // PAGE], t % PAGE] = rows[k0 + t]
    return cache
