"""Plain float64 definitions of sliding-window attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports or calls this module.

Sources (the five pages this method is described on):
  * robocikowo.com glossary entry "Sliding Window Attention" (Polish), the
    opening definition paragraph: query i may take keys only from
    [i-W+1, i] (causal) or [i-W/2, i+W/2] (symmetric); every other logit is
    set to -inf before the softmax, which zeroes its share.
  * aivaro.ru answer 629 "Как работает sliding window attention в Mistral и
    Longformer?" (Russian), section 3: Mistral's window is the previous 4096
    tokens including the token itself; section 4.1: Longformer takes W/2
    neighbours on the left and W/2 on the right.
  * Ultralytics glossary "Sliding Window Attention" (Italian), section
    "Come cresce la finestra con la profondita": the causal window as the
    boolean mask 0 <= i-j < w, its per-layer score count, the reach of the
    last token through stacked layers, and the w-slot circular KV buffer that
    writes position i into slot i mod w.
  * "Finding 15 - sliding-window attention architectures (Mistral-style)
    compile with zero code changes", section "Why this needed no exporter
    changes": attention is Q@K^T + mask, softmax, @V with the window living
    only in an additive mask tensor.
  * "Sliding-window and hybrid attention" (serving guide), section "Check
    yourself": a windowed layer's KV stops growing once it holds W tokens.

Shapes (head-major, contiguous):
  q, out : [B, Hq, T, d]      k, v : [B, Hkv, T, d]
  k_ring, v_ring : [B, Hkv, W, d]
Query head h reads KV head h // (Hq // Hkv) (grouped-query attention with
contiguous groups; the pages only say "GQA 32/8").

Readings of points the pages leave open:
  * symmetric window: |i-j| <= floor(W/2), inclusive on both sides, so an
    interior row sees W+1 keys when W is even;
  * windows are clipped to [0, T): no padding, no sink tokens;
  * scale is an argument (the workloads use 1/sqrt(d));
  * decode: the query at position p is appended first, then sees positions
    [max(0, p-W+1), p]; a sequence with p < 0 holds no tokens and its output
    is defined as zeros;
  * chunked prefill: n new tokens at positions [p, p+n) attend the ring
    (positions before p) and the chunk itself, read before the chunk is
    appended; each output row equals the causal-prefill row of the same
    position over the whole sequence.  Appending n tokens is n single appends
    in order, so when n > W only the last W of them remain;
  * dilated window (aivaro section 4.2, whose example numbers disagree with
    each other under the other reading): the window keeps its number of keys
    and spaces them d apart, so key j is allowed when (i - j) / d is a whole
    number inside the undilated window;
  * global tokens (aivaro section 4.3): added to the window as whole rows and
    columns of the mask; in the causal mode the added pairs keep j <= i, so
    global tokens at the first positions are attention sinks; together with
    a dilation the window part is the dilated one (the union of the masks);
  * decode with sinks: the first S positions are kept in sink slots beside
    the ring and the query sees them together with its window, each
    position once.
"""

import math

import numpy as np

CAUSAL = 0
SYMMETRIC = 1


# --------------------------------------------------------------------------
# The window
# --------------------------------------------------------------------------

def allowed(i, j, T, W, mode):
    """True when query i may attend to key j.

    Causal: j in [i-W+1, i] (robocikowo definition paragraph; Ultralytics mask
    0 <= i-j < w).  Symmetric: j in [i-W/2, i+W/2] (robocikowo definition
    paragraph; aivaro section 4.1), read as |i-j| <= floor(W/2).  Both are
    clipped to the sequence 0 <= j < T.
    """
    if not (0 <= j < T):
        return False
    if mode == CAUSAL:
        return 0 <= i - j <= W - 1
    if mode == SYMMETRIC:
        return abs(i - j) <= W // 2
    raise ValueError("unknown mode %r" % (mode,))


def band(i, T, W, mode):
    """Inclusive key range [lo, hi] that query i may attend to."""
    if mode == CAUSAL:
        return max(0, i - W + 1), i
    if mode == SYMMETRIC:
        h = W // 2
        return max(0, i - h), min(T - 1, i + h)
    raise ValueError("unknown mode %r" % (mode,))


def window_mask(T, W, mode):
    """Boolean [T, T] mask, True where query i (row) may see key j (column).

    Built from the offset i - j exactly as the Ultralytics section builds the
    causal mask; the symmetric mask bounds |i - j| instead.
    """
    pos = np.arange(T)
    offset = pos[:, None] - pos[None, :]
    if mode == CAUSAL:
        return (offset >= 0) & (offset < W)
    if mode == SYMMETRIC:
        return np.abs(offset) <= W // 2
    raise ValueError("unknown mode %r" % (mode,))


def additive_mask(T, W, mode):
    """float64 [T, T]: 0 where allowed, -inf elsewhere (the additive mask
    tensor of Finding 15, "Why this needed no exporter changes")."""
    return np.where(window_mask(T, W, mode), 0.0, -np.inf)


def scores_per_layer(T, W, mode):
    """Number of (query, key) scores one layer computes: the mask's count."""
    return int(window_mask(T, W, mode).sum())


def stacked_reach(T, W, layers, mode=CAUSAL):
    """Reach of the last token after 1..layers stacked windowed layers.

    The Ultralytics section traces how far information travels by multiplying
    the boolean mask by itself: after layer L the set of positions that can
    influence a token is the support of mask^L.  Returns the list of counts
    for the last row, one per layer.
    """
    mask = window_mask(T, W, mode).astype(np.int64)
    reach = mask.copy()
    out = []
    for _ in range(layers):
        out.append(int((reach[-1] > 0).sum()))
        reach = ((mask @ reach) > 0).astype(np.int64)
    return out


def kv_head(h, Hq, Hkv):
    """KV head read by query head h: contiguous groups of Hq // Hkv heads."""
    return h // (Hq // Hkv)


# --------------------------------------------------------------------------
# Attention: three forms of the same definition
#   O = softmax(scale * Q K^T + M) V,   M = 0 inside the window, -inf outside
# --------------------------------------------------------------------------

def _as64(*arrays):
    return [np.asarray(a, dtype=np.float64) for a in arrays]


def _check_shapes(q, k, v):
    B, Hq, T, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    if (Bk, Tk, dk) != (B, T, d) or v.shape != k.shape:
        raise ValueError("shape mismatch q%s k%s v%s" % (q.shape, k.shape, v.shape))
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, T, d


def attention_loop(q, k, v, W, mode, scale):
    """Pure-Python loops over (b, h, i, j, c) for tiny inputs.

    For each query row: score every allowed key, subtract the row maximum,
    exponentiate, normalise, and take the weighted sum of value rows.
    """
    q, k, v = _as64(q, k, v)
    B, Hq, Hkv, T, d = _check_shapes(q, k, v)
    out = np.zeros((B, Hq, T, d))
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            for i in range(T):
                keys = [j for j in range(T) if allowed(i, j, T, W, mode)]
                s = []
                for j in keys:
                    acc = 0.0
                    for c in range(d):
                        acc += float(q[b, h, i, c]) * float(k[b, g, j, c])
                    s.append(scale * acc)
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = sum(e)
                for c in range(d):
                    acc = 0.0
                    for w, j in zip(e, keys):
                        acc += w * float(v[b, g, j, c])
                    out[b, h, i, c] = acc / tot
    return out


def _softmax_rows(S):
    m = S.max(axis=-1, keepdims=True)
    P = np.exp(S - m)
    return P / P.sum(axis=-1, keepdims=True)


def attention_dense(q, k, v, W, mode, scale):
    """Dense [T, T] scores plus the explicit additive mask, for T <= ~4096."""
    q, k, v = _as64(q, k, v)
    B, Hq, Hkv, T, d = _check_shapes(q, k, v)
    M = additive_mask(T, W, mode)
    out = np.empty((B, Hq, T, d))
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            S = scale * (q[b, h] @ k[b, g].T) + M
            out[b, h] = _softmax_rows(S) @ v[b, g]
    return out


def attention_banded(q, k, v, W, mode, scale, block=128, heads=None):
    """Row blocks of `block` queries against the key range their windows
    cover, with the explicit additive mask on that block.  Identical to the
    dense form because every key outside the range is masked to an exact zero
    weight.  `heads` optionally restricts the computation to a list of
    (b, h) pairs; other rows of the result are left as NaN.
    """
    q, k, v = _as64(q, k, v)
    B, Hq, Hkv, T, d = _check_shapes(q, k, v)
    out = np.full((B, Hq, T, d), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    pos = np.arange(T)
    for b, h in pairs:
        g = kv_head(h, Hq, Hkv)
        for r0 in range(0, T, block):
            r1 = min(T, r0 + block)
            lo = band(r0, T, W, mode)[0]
            hi = band(r1 - 1, T, W, mode)[1]
            rows = pos[r0:r1, None]
            cols = pos[None, lo:hi + 1]
            off = rows - cols
            if mode == CAUSAL:
                ok = (off >= 0) & (off < W)
            else:
                ok = np.abs(off) <= W // 2
            M = np.where(ok, 0.0, -np.inf)
            S = scale * (q[b, h, r0:r1] @ k[b, g, lo:hi + 1].T) + M
            out[b, h, r0:r1] = _softmax_rows(S) @ v[b, g, lo:hi + 1]
    return out


def attention_rows(q, k, v, W, mode, scale, b, h, rows):
    """Selected query rows of one (b, h), each over exactly its own window.
    Used to check sampled outputs of full-size problems one by one.
    Returns float64 [len(rows), d]."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    g = kv_head(h, Hq, Hkv)
    res = np.empty((len(rows), d))
    for n, i in enumerate(rows):
        lo, hi = band(int(i), T, W, mode)
        qi = np.asarray(q[b, h, i], dtype=np.float64)
        kk = np.asarray(k[b, g, lo:hi + 1], dtype=np.float64)
        vv = np.asarray(v[b, g, lo:hi + 1], dtype=np.float64)
        s = scale * (kk @ qi)
        p = np.exp(s - s.max())
        res[n] = (p / p.sum()) @ vv
    return res


# --------------------------------------------------------------------------
# Ring-buffer KV cache and decode
# --------------------------------------------------------------------------

def ring_append(k_ring, v_ring, pos, k_new, v_new):
    """Write the new K/V row of each sequence into slot pos mod W, in place.

    Ultralytics ring-buffer paragraph: a buffer of w slots, position i goes
    to slot i mod w and overwrites the oldest entry; robocikowo: only the last
    W tokens per layer are kept, new tokens overwrite the oldest (FIFO).
    Works on any dtype (a bit copy).  k_ring [B, Hkv, W, d], k_new [B, Hkv, d],
    pos [B].  A negative position writes nothing.
    """
    W = k_ring.shape[2]
    for b, p in enumerate(np.asarray(pos).tolist()):
        if p < 0:
            continue
        s = p % W
        k_ring[b, :, s, :] = k_new[b]
        v_ring[b, :, s, :] = v_new[b]


def decode(q, k_ring, v_ring, pos, scale):
    """One query token per sequence against its ring cache.

    q [B, Hq, d]; rings [B, Hkv, W, d]; pos [B] = position of the query,
    whose own K/V row is already in the ring.  The query sees positions
    [max(0, p-W+1), p] (the causal window), stored at slots p' mod W.
    Returns float64 [B, Hq, d]; a sequence with p < 0 gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    out = np.zeros((B, Hq, d))
    for b, p in enumerate(np.asarray(pos).tolist()):
        if p < 0:
            continue
        positions = np.arange(max(0, p - W + 1), p + 1)
        slots = positions % W
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            kk = np.asarray(k_ring[b, g, slots], dtype=np.float64)
            vv = np.asarray(v_ring[b, g, slots], dtype=np.float64)
            s = scale * (kk @ q[b, h])
            e = np.exp(s - s.max())
            out[b, h] = (e / e.sum()) @ vv
    return out


# --------------------------------------------------------------------------
# Chunked prefill into an existing ring
# --------------------------------------------------------------------------

def ring_append_chunk(k_ring, v_ring, pos, k_new, v_new):
    """Append n consecutive tokens per sequence, in place: token i of
    sequence b has position pos[b] + i and goes to slot (pos[b] + i) mod W,
    one token after the other, so a later token overwrites an earlier one
    that maps to the same slot (Ultralytics ring-buffer paragraph; robocikowo
    rolling buffer, FIFO).  k_new [B, Hkv, n, d].  A negative pos[b] writes
    nothing for that sequence.
    """
    n = k_new.shape[2]
    for b, p in enumerate(np.asarray(pos).tolist()):
        if p < 0:
            continue
        for i in range(n):
            ring_append(k_ring[b:b + 1], v_ring[b:b + 1], [p + i], k_new[b:b + 1, :, i],
                        v_new[b:b + 1, :, i])


def prefill_chunk(q, k, v, k_ring, v_ring, pos, W, scale, heads=None, rows=None):
    """Causal windowed attention for a chunk of n new tokens per sequence.

    Token i of sequence b sits at position P = pos[b] + i and sees the causal
    window [max(0, P-W+1), P] (robocikowo definition paragraph; Ultralytics
    mask 0 <= i-j < w).  Positions before pos[b] are read from the ring,
    where position p' lives in slot p' mod W (Ultralytics ring-buffer
    paragraph); positions from pos[b] on are the chunk's own rows k[b, g, p'-pos[b]].
    The ring is read before the chunk is appended to it.

    q [B, Hq, n, d]; k, v [B, Hkv, n, d]; rings [B, Hkv, W, d]; pos [B].
    Returns float64 [B, Hq, n, d]; a sequence with pos[b] < 0 gives zeros.
    `heads` (list of (b, h)) and `rows` (list of chunk rows) restrict the
    computation; entries left out are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    restricted = heads is not None or rows is not None
    out = np.full((B, Hq, n, d), np.nan) if restricted else np.zeros((B, Hq, n, d))
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    row_list = list(range(n)) if rows is None else [int(i) for i in rows]
    pos = np.asarray(pos).tolist()
    for b, h in pairs:
        p = pos[b]
        if p < 0:
            out[b, h, row_list] = 0.0
            continue
        g = kv_head(h, Hq, Hkv)
        for i in row_list:
            P = p + i
            window = np.arange(max(0, P - W + 1), P + 1)
            old = window[window < p]
            new = window[window >= p] - p
            kk = np.concatenate([np.asarray(k_ring[b, g, old % W], dtype=np.float64),
                                 np.asarray(k[b, g, new], dtype=np.float64)])
            vv = np.concatenate([np.asarray(v_ring[b, g, old % W], dtype=np.float64),
                                 np.asarray(v[b, g, new], dtype=np.float64)])
            sc = scale * (kk @ q[b, h, i])
            e = np.exp(sc - sc.max())
            out[b, h, i] = (e / e.sum()) @ vv
    return out


# --------------------------------------------------------------------------
# Dilated sliding window
# --------------------------------------------------------------------------

def dilated_mask(T, W, mode, dilation):
    """Boolean [T, T] mask of the dilated window: query i may see key j when
    i - j is a multiple of the dilation and the quotient m = (i - j) / dilation
    lies in the undilated window (causal 0 <= m <= W-1, symmetric
    |m| <= floor(W/2)), clipped to the sequence.

    aivaro section 4.2 takes every d-th token of the window with gaps, like a
    dilated convolution (robocikowo, dilated-SWA variant): the number of keys
    stays that of the plain window while their span grows d-fold; its example
    W = 512, d = 2 gives 256 keys on each side spanning 1024 positions.  With
    dilation 1 this is window_mask.
    """
    if dilation < 1:
        raise ValueError("dilation must be >= 1")
    pos = np.arange(T)
    offset = pos[:, None] - pos[None, :]
    on_grid = offset % dilation == 0
    m = offset // dilation
    if mode == CAUSAL:
        return on_grid & (m >= 0) & (m <= W - 1)
    if mode == SYMMETRIC:
        return on_grid & (np.abs(m) <= W // 2)
    raise ValueError("unknown mode %r" % (mode,))


def attention_dilated_dense(q, k, v, W, mode, scale, dilation):
    """Dense [T, T] scores plus the dilated additive mask (the additive-mask
    form of Finding 15, "Why this needed no exporter changes")."""
    q, k, v = _as64(q, k, v)
    B, Hq, Hkv, T, d = _check_shapes(q, k, v)
    M = np.where(dilated_mask(T, W, mode, dilation), 0.0, -np.inf)
    out = np.empty((B, Hq, T, d))
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            S = scale * (q[b, h] @ k[b, g].T) + M
            out[b, h] = _softmax_rows(S) @ v[b, g]
    return out


def attention_dilated_rows(q, k, v, W, mode, scale, dilation, b, h, rows):
    """Selected query rows of one (b, h), each over exactly its dilated
    window's keys (for sampled checks of full-size problems).  Returns
    float64 [len(rows), d]."""
    B, Hq, T, d = q.shape
    g = kv_head(h, Hq, k.shape[1])
    res = np.empty((len(rows), d))
    for n, i in enumerate(rows):
        i = int(i)
        if mode == CAUSAL:
            m = np.arange(0, W)
        else:
            m = np.arange(-(W // 2), W // 2 + 1)
        keys = i - dilation * m
        keys = np.sort(keys[(keys >= 0) & (keys < T)])
        qi = np.asarray(q[b, h, i], dtype=np.float64)
        kk = np.asarray(k[b, g, keys], dtype=np.float64)
        vv = np.asarray(v[b, g, keys], dtype=np.float64)
        sc = scale * (kk @ qi)
        e = np.exp(sc - sc.max())
        res[n] = (e / e.sum()) @ vv
    return res


# --------------------------------------------------------------------------
# Sliding window plus global tokens
# --------------------------------------------------------------------------

def global_mask(T, W, mode, global_pos, dilation=1):
    """Boolean [T, T] mask of the window plus global tokens.

    aivaro section 4.3 (Longformer global attention) and robocikowo's global
    tokens entry: a global token attends to every token and every token
    attends to it, on top of the sliding window.  In the causal mode the
    added pairs keep j <= i (no token sees a later one).  global_pos lists
    distinct positions in [0, T).  With dilation > 1 the window is the
    dilated one of section 4.2 (dilated_mask); Longformer combines the two,
    and the global pairs are the same.
    """
    if dilation == 1:
        m = window_mask(T, W, mode).copy()
    else:
        m = dilated_mask(T, W, mode, dilation).copy()
    g = np.zeros(T, dtype=bool)
    g[np.asarray(global_pos, dtype=np.int64)] = True
    extra = g[:, None] | g[None, :]
    if mode == CAUSAL:
        extra &= np.tri(T, dtype=bool)
    return m | extra


def attention_global_dense(q, k, v, W, mode, scale, global_pos, dilation=1):
    """Dense [T, T] scores plus the additive form of global_mask."""
    q, k, v = _as64(q, k, v)
    B, Hq, Hkv, T, d = _check_shapes(q, k, v)
    M = np.where(global_mask(T, W, mode, global_pos, dilation), 0.0, -np.inf)
    out = np.empty((B, Hq, T, d))
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            S = scale * (q[b, h] @ k[b, g].T) + M
            out[b, h] = _softmax_rows(S) @ v[b, g]
    return out


def attention_global_rows(q, k, v, W, mode, scale, global_pos, b, h, rows, dilation=1):
    """Selected query rows of one (b, h) over exactly their keys: the
    (dilated) window, the global keys (j <= i when causal), or, for a global
    row, every key (j <= i when causal).  Returns float64 [len(rows), d]."""
    B, Hq, T, d = q.shape
    g = kv_head(h, Hq, k.shape[1])
    gset = set(int(x) for x in global_pos)
    res = np.empty((len(rows), d))
    for n, i in enumerate(rows):
        i = int(i)
        if i in gset:
            keys = np.arange(0, i + 1) if mode == CAUSAL else np.arange(T)
        else:
            if dilation == 1:
                lo, hi = band(i, T, W, mode)
                window = np.arange(lo, hi + 1)
            else:
                m = np.arange(0, W) if mode == CAUSAL else np.arange(-(W // 2), W // 2 + 1)
                window = i - dilation * m
                window = window[(window >= 0) & (window < T)]
            wset = set(int(x) for x in window)
            extra = [x for x in gset if (x <= i or mode != CAUSAL) and x not in wset]
            keys = np.sort(np.concatenate([window, np.array(extra, dtype=np.int64)]))
        qi = np.asarray(q[b, h, i], dtype=np.float64)
        kk = np.asarray(k[b, g, keys], dtype=np.float64)
        vv = np.asarray(v[b, g, keys], dtype=np.float64)
        sc = scale * (kk @ qi)
        e = np.exp(sc - sc.max())
        res[n] = (e / e.sum()) @ vv
    return res


# --------------------------------------------------------------------------
# Decode with attention sinks
# --------------------------------------------------------------------------

def decode_sinks(q, k_ring, v_ring, k_sink, v_sink, pos, scale):
    """One query token per sequence against its ring plus S sink slots.

    Ultralytics glossary, terms section ("Pozzi di attenzione"): the first
    tokens of a sequence soak up excess attention weight, and StreamingLLM
    keeps them in the cache beside the window.  The query at position p sees
    the positions {0, ..., min(S-1, p)} together with its causal window
    [max(0, p-W+1), p], each position once: window positions come from ring
    slot p' mod W, the sink positions before the window from k_sink[b, :, p'].

    q [B, Hq, d]; rings [B, Hkv, W, d]; sinks [B, Hkv, S, d]; pos [B].
    Returns float64 [B, Hq, d]; a sequence with p < 0 gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, W = k_ring.shape[1], k_ring.shape[2]
    S = k_sink.shape[2]
    out = np.zeros((B, Hq, d))
    for b, p in enumerate(np.asarray(pos).tolist()):
        if p < 0:
            continue
        first = max(0, p - W + 1)
        window = np.arange(first, p + 1)
        sinks = np.arange(0, min(S, first))  # sink positions before the window
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            kk = np.concatenate([np.asarray(k_sink[b, g, sinks], dtype=np.float64),
                                 np.asarray(k_ring[b, g, window % W], dtype=np.float64)])
            vv = np.concatenate([np.asarray(v_sink[b, g, sinks], dtype=np.float64),
                                 np.asarray(v_ring[b, g, window % W], dtype=np.float64)])
            sc = scale * (kk @ q[b, h])
            e = np.exp(sc - sc.max())
            out[b, h] = (e / e.sum()) @ vv
    return out
