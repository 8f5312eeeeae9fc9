"""Plain float64 chunk-wise causal attention (oracle; test infrastructure only).

Definition followed.  A streaming DiT splits the latent video into chunks of
frames.  Each query row of chunk c attends to every key position that chunk is
allowed to see: all of its own chunk's tokens (bidirectional inside the chunk)
and the K/V of earlier chunks still held in the rolling cache, whatever their
noise level.  Sources: "Wave Forcing: Towards Speed-of-Light Streaming Video
Generation", abstract (chunk-wise causal attention reaching earlier chunks
before their denoising is complete); hellomarvisaitoday Wave Forcing article,
first paragraph (conditioning on a mixed-noise frontier).  In this API the
visible set of chunk c is the contiguous logical key range
[kv_begin[c], kv_end[c]), which expresses both the block-causal rule and the
rolling window.

For each chunk c, head h and query row i:
    s_j  = scale * sum_d Q[i,h,d] * K[j,h,d]      for j in [kv_begin[c], kv_end[c])
    m    = max_j s_j
    w_j  = exp(s_j - m)
    l    = sum_j w_j
    O[i,h,:]  = sum_j w_j V[j,h,:] / l
    LSE[h,i]  = m + ln l

The only decomposition is over query rows (each row's result depends on that
row alone), done in blocks to bound memory.  No online softmax, no key tiling.
"""
import numpy as np


def _check_chunks(nq, q_off, kv_begin, kv_end, kv_origin, nkeys):
    q_off = [int(x) for x in q_off]
    kv_begin = [int(x) for x in kv_begin]
    kv_end = [int(x) for x in kv_end]
    c = len(q_off) - 1
    if c < 1 or len(kv_begin) != c or len(kv_end) != c:
        raise ValueError("need num_chunks+1 query offsets and num_chunks key ranges")
    if q_off[0] != 0 or q_off[-1] != nq:
        raise ValueError("query offsets must start at 0 and end at the number of query rows")
    for i in range(c):
        if q_off[i + 1] < q_off[i]:
            raise ValueError("query offsets must be non-decreasing")
        if not (kv_origin <= kv_begin[i] < kv_end[i] <= kv_origin + nkeys):
            raise ValueError("chunk %d: key range [%d,%d) empty or outside the given keys"
                             % (i, kv_begin[i], kv_end[i]))
    return q_off, kv_begin, kv_end


def chunk_attention(q, k, v, q_off, kv_begin, kv_end, scale=None, kv_origin=0,
                    row_block=512):
    """Chunk-wise causal attention in float64.

    q            [Nq, H, D] query rows of all chunks, chunk c owning rows
                 [q_off[c], q_off[c+1]).
    k, v         [L, H, D] logical key/value sequence; row r is logical key
                 position kv_origin + r.
    kv_begin/end per-chunk visible logical key range (absolute positions).
    scale        softmax scale; None means 1/sqrt(D).
    Returns (O [Nq, H, D], LSE [H, Nq]), float64, LSE in natural log.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, h, d = q.shape
    if k.shape[1:] != (h, d) or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree: %s %s %s" % (q.shape, k.shape, v.shape))
    q_off, kv_begin, kv_end = _check_chunks(nq, q_off, kv_begin, kv_end, kv_origin, k.shape[0])
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((nq, h, d), dtype=np.float64)
    lse = np.zeros((h, nq), dtype=np.float64)
    for c in range(len(q_off) - 1):
        a, b = kv_begin[c] - kv_origin, kv_end[c] - kv_origin
        for hh in range(h):
            kh = k[a:b, hh, :]
            vh = v[a:b, hh, :]
            for r0 in range(q_off[c], q_off[c + 1], row_block):
                r1 = min(r0 + row_block, q_off[c + 1])
                s = scale * (q[r0:r1, hh, :] @ kh.T)
                m = s.max(axis=1, keepdims=True)
                w = np.exp(s - m)
                l = w.sum(axis=1, keepdims=True)
                o[r0:r1, hh, :] = (w @ vh) / l
                lse[hh, r0:r1] = (m + np.log(l))[:, 0]
    return o, lse


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Combine attention over two disjoint key sets A and B into attention over A u B.

    With LSE_x = ln sum_{j in x} exp(s_j), the union has
    LSE = ln(exp(LSE_a) + exp(LSE_b)) and O = (e^{LSE_a} O_a + e^{LSE_b} O_b) / e^{LSE}.
    Shapes: o [Nq, H, D], lse [H, Nq].
    """
    lse = np.logaddexp(lse_a, lse_b)
    wa = np.exp(lse_a - lse).T[:, :, None]
    wb = np.exp(lse_b - lse).T[:, :, None]
    return wa * o_a + wb * o_b, lse
