"""Plain, slow, fp64 CPU oracle of exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the product path.  Shares no code with the
HIP library.

What is computed, and where the pages define it:

* Forward — the standard (materialised) flow of "Flash Attention 是什么：2026
  最新原理、架构演进与实战详解" (ai.lansai.wang), section 技术原理 › 核心工作机制:
  scores S = Q·Kᵀ (here times the softmax scale, default 1/sqrt(d_k), and with
  future keys masked when causal, both knobs of lqnn.cn "为什么Flash突然成了AI圈的
  高频词" §3.3), a row softmax normalised by the row max and row sum, and the
  weighted sum with V.  The row statistics are kept as the logsumexp
  LSE = m + ln(l), the "max and sum" the same explainer says the forward keeps
  for the backward (技术原理, 重计算 paragraph).
* Backward — the gradient of the forward above, written out from its
  definition (the pages only say the backward recomputes the local attention
  from the saved statistics; 关键术语解析 §5 重计算).  The oracle recomputes
  P from Q and K itself.
* Paged decode — one query per sequence attending to all of that sequence's
  cached keys, which live in fixed 256-token pages of a pool reserved up
  front (0539edu.com "Flash不是那个被时代淘汰的插件" §2); a block table maps
  the sequence's logical page b to a physical page.
* Grouped key/value heads (GQA; MQA when Hkv = 1) — the multi-/grouped-query
  adaptation the explainer names (进阶学习路径 §4): query head h attends with
  key/value head h // (H / Hkv); the K/V gradients sum over the group.
* Packed variable-length batches — the per-sample lengths without padding of
  the explainer's 使用门槛和条件 §4: sequences concatenated token-major
  ([total, H, d]), sequence b owning rows cu[b]..cu[b+1]-1, attention (and
  the causal mask) kept inside each sequence, LSE laid out [H, total].
* Rotary position embedding fused into the forward — the RoPE-with-a-lookup-
  table fusion of 0539edu.com §3: Q and K rows rotated pairwise by angles
  read from cosine / sine tables at each row's position before the scores
  (apply_rope, exact; apply_rope_bf16, the same rotation stored as the bf16
  operands of the products).
* online_forward — the tiled online-softmax recurrence of the explainer's
  关键术语解析 §4 (在线 Softmax: the running max and normaliser update), with
  the partial output rescaled alongside the normaliser and divided by the
  final normaliser once (zwxr.cn §3.1).  Test-only: it exists to show the
  online recurrence equals the two-pass definition; parity uses the
  two-pass functions.

Rows of queries may be processed in blocks (rows are independent); key
blocks are never split in the two-pass functions.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    """Upcast the exact stored values (fp32 or bf16, numpy or torch) to fp64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale · Q Kᵀ for a block of query rows ([r, d] x [n, d] -> [r, n])."""
    return scale * (q_rows @ k.T)


def _mask(s: np.ndarray, rows: np.ndarray, causal: bool) -> np.ndarray:
    """Causal: query i sees keys 0..i only; every later key gets -inf."""
    if causal:
        cols = np.arange(s.shape[1])
        s = np.where(cols[None, :] > rows[:, None], NEG_INF, s)
    return s


def _softmax_rows(s: np.ndarray):
    """Two-pass row softmax: m = row max, E = exp(S - m), l = row sum, P = E / l.

    A row with no visible key (all -inf) gives P = 0, l = 0 and m = -inf, so
    its output is 0 and its logsumexp is -inf rather than NaN; so does a row
    of a sequence with no key at all (zero columns).
    """
    if s.shape[1] == 0:
        return np.zeros_like(s), np.full(s.shape[0], NEG_INF)
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(l[:, None] > 0, e / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, m_safe + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return p, lse


def _dscores(p: np.ndarray, dp: np.ndarray, D: np.ndarray | None = None) -> np.ndarray:
    """dS = P ∘ (dP − D) with D_i = sum_j P_ij dP_ij (softmax Jacobian applied
    row-wise), or the given D."""
    if D is None:
        D = (p * dp).sum(axis=1)
    return p * (dp - D[:, None])


def _forward_head(q, k, v, causal, scale, rows=None, row_block=1024):
    nq = q.shape[0]
    rows = np.arange(nq) if rows is None else np.asarray(rows)
    o = np.zeros((rows.size, v.shape[1]))
    lse = np.zeros(rows.size)
    for r0 in range(0, rows.size, row_block):
        r = rows[r0:r0 + row_block]
        s = _mask(_scores(q[r], k, scale), r, causal)
        p, lse[r0:r0 + r.size] = _softmax_rows(s)
        o[r0:r0 + r.size] = p @ v
    return o, lse


def _check(q, k, v, causal):
    if q.shape[:-2] != k.shape[:-2] or k.shape != v.shape[:-1] + (k.shape[-1],):
        raise ValueError("q, k, v must share leading dims; k and v share their key count")
    if q.shape[-1] != k.shape[-1]:
        raise ValueError("q and k need the same head dimension")
    if causal and q.shape[-2] != k.shape[-2]:
        raise ValueError("causal attention here takes as many queries as keys")


def attention_forward(q, k, v, causal=False, scale=None, row_block=1024):
    """O and LSE of exact attention for inputs of shape [..., N, d].

    Returns (o [..., Nq, dv] fp64, lse [..., Nq] fp64) with LSE the natural
    log of the row sum of exp(scaled, masked scores).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check(q, k, v, causal)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    lead = q.shape[:-2]
    heads = int(np.prod(lead))
    qf = q.reshape((heads,) + q.shape[-2:])
    kf = k.reshape((heads,) + k.shape[-2:])
    vf = v.reshape((heads,) + v.shape[-2:])
    o = np.zeros(qf.shape[:-1] + (vf.shape[-1],))
    lse = np.zeros(qf.shape[:-1])
    for h in range(qf.shape[0]):
        o[h], lse[h] = _forward_head(qf[h], kf[h], vf[h], causal, scale, row_block=row_block)
    return o.reshape(lead + o.shape[-2:]), lse.reshape(lead + lse.shape[-1:])


def attention_forward_rows(q, k, v, rows, causal=False, scale=None):
    """Forward for a subset of query rows of one head ([N, d] inputs).

    Rows are independent in the definition, so a sample of rows is computed
    exactly as the full forward would compute them.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check(q, k, v, causal)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    return _forward_head(q, k, v, causal, scale, rows=np.asarray(rows))


def attention_backward(q, k, v, dout, causal=False, scale=None, row_block=1024, out=None):
    """dQ, dK, dV of L = sum(O * dO) for inputs of shape [..., N, d].

    With P the softmax probabilities of the forward:
      dV = Pᵀ dO;  dP = dO Vᵀ;  D_i = sum_j P_ij dP_ij;
      dS = P ∘ (dP − D);  dQ = scale · dS K;  dK = scale · dSᵀ Q.
    Since O_i = sum_j P_ij V_j, D_i equals sum_d dO_id O_id.  With `out` (the
    forward's output as the caller kept it, e.g. rounded to bf16) D is taken
    as sum_d dO_id out_id instead: the backward of a method that saves O.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    _check(q, k, v, causal)
    if out is not None:
        out = _f64(out)
        assert out.shape == q.shape[:-1] + (v.shape[-1],)
        Dall = (do * out).sum(axis=-1).reshape(-1, q.shape[-2])
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    heads = int(np.prod(q.shape[:-2]))
    qf, kf, vf, dof = (x.reshape((heads,) + x.shape[-2:]) for x in (q, k, v, do))
    dq = np.zeros_like(qf)
    dk = np.zeros_like(kf)
    dv = np.zeros_like(vf)
    for h in range(qf.shape[0]):
        nq = qf.shape[1]
        for r0 in range(0, nq, row_block):
            r = np.arange(r0, min(nq, r0 + row_block))
            s = _mask(_scores(qf[h, r], kf[h], scale), r, causal)
            p, _ = _softmax_rows(s)
            dv[h] += p.T @ dof[h, r]
            dp = dof[h, r] @ vf[h].T
            ds = _dscores(p, dp, None if out is None else Dall[h, r])
            dq[h, r] = scale * (ds @ kf[h])
            dk[h] += scale * (ds.T @ qf[h, r])
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)


def gather_pages(kv_pool, block_table, seq_len, seq, page_size):
    """K and V of one sequence, token by token, through its block table.

    Token t sits in logical page t // page_size, slot t % page_size; the
    table row maps the logical page to a physical page of the pool, whose
    layout is [pages, 2 (K, V), page_size, H, d].
    """
    H, d = kv_pool.shape[3], kv_pool.shape[4]
    K = np.empty((seq_len, H, d))
    V = np.empty((seq_len, H, d))
    for t in range(seq_len):
        page = int(block_table[seq, t // page_size])
        slot = t % page_size
        K[t] = kv_pool[page, 0, slot]
        V[t] = kv_pool[page, 1, slot]
    return K, V


def decode_paged(q, kv_pool, block_table, seq_lens, scale=None, page_size=256):
    """One query token per sequence over its paged KV cache.

    q [S, H, d]; kv_pool [P, 2, page_size, Hkv, d] with Hkv dividing H (query
    head h reads key/value head h // (H // Hkv); Hkv == H is plain multi-head
    attention); block_table [S, max_blocks]; seq_lens [S].  The query sees
    every one of the sequence's L_s cached keys (its own key is already in the
    cache), so no causal mask applies.  A sequence with no cached key has an
    empty softmax: O = 0 and LSE = -inf.  Returns (o [S, H, d], lse [S, H]).
    """
    q, pool = _f64(q), _f64(kv_pool)
    table = np.asarray(_f64(block_table), dtype=np.int64)
    lens = np.asarray(_f64(seq_lens), dtype=np.int64)
    S, H, d = q.shape
    Hkv = pool.shape[3]
    if H % Hkv:
        raise ValueError("the pool's key/value heads must divide the query heads")
    group = H // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((S, H, d))
    lse = np.full((S, H), -np.inf)
    for s in range(S):
        if int(lens[s]) <= 0:
            continue
        K, V = gather_pages(pool, table, int(lens[s]), s, page_size)
        for h in range(H):
            oh, lh = _forward_head(q[s, h][None, :], K[:, h // group], V[:, h // group], False, scale)
            o[s, h], lse[s, h] = oh[0], lh[0]
    return o, lse


def prefill_paged(q, kv_pool, block_table, seq_lens_k, cu_seqlens_q, causal=True, scale=None, page_size=256,
                  rope=None):
    """Chunked prefill over a paged KV cache.

    Sequence b has L = seq_lens_k[b] cached keys (reached through its block
    table as in decode_paged) and n = cu[b+1] - cu[b] new queries, packed in
    q [total_q, H, d].  The queries are the last n positions of the sequence,
    so with the causal mask query i (0-based in its chunk) sees keys
    0 .. i + L - n; without it every query sees all L keys.  A query that
    sees no key has an empty softmax (O = 0, LSE = -inf).  Key/value head of
    query head h: h // (H // Hkv).  rope = (cos, sin, interleaved) rotates the
    queries at their positions as apply_rope_bf16 does (the cached keys are
    used as stored).
    Returns (o [total_q, H, d], lse [H, total_q]).
    """
    q, pool = _f64(q), _f64(kv_pool)
    table = np.asarray(_f64(block_table), dtype=np.int64)
    lens = np.asarray(_f64(seq_lens_k), dtype=np.int64)
    cu = np.asarray(_f64(cu_seqlens_q), dtype=np.int64)
    total, H, d = q.shape
    Hkv = pool.shape[3]
    group = H // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((total, H, d))
    lse = np.full((H, total), -np.inf)
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        n, L = t1 - t0, int(lens[b])
        if n == 0:
            continue
        K, V = gather_pages(pool, table, L, b, page_size)
        positions = np.arange(n) + (L - n)  # absolute position of each query
        qb = q[t0:t1]
        if rope is not None:
            qb = np.swapaxes(apply_rope_bf16(np.swapaxes(qb, 0, 1), np.maximum(positions, 0), *rope), 0, 1)
        for h in range(H):
            s = _mask(_scores(qb[:, h], K[:, h // group], scale), positions, causal)
            p_, lrow = _softmax_rows(s)
            o[t0:t1, h] = p_ @ V[:, h // group]
            lse[h, t0:t1] = lrow
    return o, lse


def apply_rope(x, positions, cos, sin, interleaved=False):
    """Rotary position embedding of rows x [..., n, d] at positions [n], exact.

    Feature pair i of the row at position p is (x_i, x_{i+d/2}) (half split)
    or (x_{2i}, x_{2i+1}) (interleaved); it becomes
    (x·cos[p][i] − y·sin[p][i], x·sin[p][i] + y·cos[p][i]).  The tables are
    inputs (a precomputed lookup, "Flash不是那个被时代淘汰的插件" §3); every
    value is used in fp64.
    """
    x = _f64(x).copy()
    c = _f64(cos)[np.asarray(positions)]  # [n, d/2]
    s = _f64(sin)[np.asarray(positions)]
    d = x.shape[-1]
    if interleaved:
        a, b = x[..., 0::2].copy(), x[..., 1::2].copy()
        x[..., 0::2] = a * c - b * s
        x[..., 1::2] = a * s + b * c
    else:
        a, b = x[..., : d // 2].copy(), x[..., d // 2:].copy()
        x[..., : d // 2] = a * c - b * s
        x[..., d // 2:] = a * s + b * c
    return x


def _bf16_rne(x) -> np.ndarray:
    """Round real values to bf16 (8 significant bits) to nearest, ties to even,
    in one step from the fp64 value (no intermediate fp32 rounding): add half
    of the dropped 45 low mantissa bits of the fp64 encoding, minus one, plus
    the lowest kept bit, then clear the dropped bits.  Defined for zero and
    for magnitudes in bf16's normal range [2^-126, 2^128); anything else
    raises.  Returns fp64 arrays holding the bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    a = np.abs(x)
    if not np.all((a == 0) | ((a >= 2.0 ** -126) & (a < 2.0 ** 128))):
        raise ValueError("bf16 rounding here covers zero and the normal range only")
    u = x.view(np.uint64)
    drop = np.uint64(45)
    keep = (u >> drop) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + keep) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def apply_rope_bf16(x, positions, cos, sin, interleaved=False):
    """The rotation as it is stored for bf16 matrix products.

    The attention products take bf16 operands, so each rotated feature enters
    them as a bf16 value: the exact rotation of apply_rope (fp64 arithmetic on
    the stored bf16 inputs and the fp32 table entries) rounded once to bf16,
    to nearest with ties to even.  Returns fp64 arrays holding those values.
    """
    return _bf16_rne(apply_rope(x, positions, cos, sin, interleaved))


def attention_forward_rope(q, k, v, cos, sin, causal=False, scale=None, interleaved=False, cu_seqlens=None,
                           rotate=apply_rope_bf16):
    """Forward with Q and K rotated first (by default the bf16-stored
    rotation, apply_rope_bf16; pass rotate=apply_rope for the exact one).
    Dense: q [B, H, N, d], k/v [B, Hkv, N, d], positions 0..N-1.  Packed
    (cu_seqlens): [total, heads, d], positions counted from each sequence's
    first row."""
    if cu_seqlens is None:
        N = q.shape[2]
        pos = np.arange(N)
        return attention_forward_gqa(rotate(q, pos, cos, sin, interleaved),
                                     rotate(k, pos, cos, sin, interleaved), v, causal=causal, scale=scale)
    cu = np.asarray(_f64(cu_seqlens), dtype=np.int64)
    pos = np.concatenate([np.arange(cu[b + 1] - cu[b]) for b in range(len(cu) - 1)]).astype(np.int64)
    qr = np.swapaxes(rotate(np.swapaxes(_f64(q), 0, 1), pos, cos, sin, interleaved), 0, 1)
    kr = np.swapaxes(rotate(np.swapaxes(_f64(k), 0, 1), pos, cos, sin, interleaved), 0, 1)
    return attention_forward_varlen(qr, kr, v, cu_seqlens, causal=causal, scale=scale)


def online_forward(q, k, v, causal=False, scale=None, tile=16):
    """Tiled single-pass forward with the online softmax (test-only).

    Keys are visited in tiles of ``tile``.  Per query row a running max m and
    normaliser l are kept; for each tile
      m_new = max(m_old, max(x_tile)),
      l_new = exp(m_old − m_new)·l_old + sum exp(x_tile − m_new),
    and the unnormalised output is rescaled by the same exp(m_old − m_new)
    before the tile's exp(x_tile − m_new)·V is added.  After the last tile the
    output is divided by l once, and LSE = m + ln(l).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    _check(q, k, v, causal)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    lead = q.shape[:-2]
    heads = int(np.prod(lead))
    qf, kf, vf = (x.reshape((heads,) + x.shape[-2:]) for x in (q, k, v))
    nq, nk = qf.shape[1], kf.shape[1]
    o = np.zeros(qf.shape[:-1] + (vf.shape[-1],))
    lse = np.zeros(qf.shape[:-1])
    rows = np.arange(nq)
    for h in range(qf.shape[0]):
        m = np.full(nq, NEG_INF)
        l = np.zeros(nq)
        acc = np.zeros((nq, vf.shape[-1]))
        for j0 in range(0, nk, tile):
            j1 = min(nk, j0 + tile)
            x = scale * (qf[h] @ kf[h, j0:j1].T)
            if causal:
                cols = np.arange(j0, j1)
                x = np.where(cols[None, :] > rows[:, None], NEG_INF, x)
            m_new = np.maximum(m, x.max(axis=1))
            live = np.isfinite(m_new)
            m_ref = np.where(live, m_new, 0.0)
            alpha = np.where(live, np.exp(np.where(live, m - m_ref, 0.0)), 1.0)
            pt = np.exp(x - m_ref[:, None])
            l = alpha * l + pt.sum(axis=1)
            acc = alpha[:, None] * acc + pt @ vf[h, j0:j1]
            m = m_new
        with np.errstate(divide="ignore", invalid="ignore"):
            o[h] = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
            lse[h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return o.reshape(lead + o.shape[-2:]), lse.reshape(lead + lse.shape[-1:])


def _expand_kv(x, H):
    """[B, Hkv, N, d] -> [B, H, N, d]: query head h reads key/value head h // (H/Hkv)."""
    Hkv = x.shape[1]
    if H % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    return np.repeat(x, H // Hkv, axis=1)


def attention_forward_gqa(q, k, v, causal=False, scale=None):
    """Forward with grouped key/value heads: q [B, H, N, d], k/v [B, Hkv, N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    H = q.shape[1]
    return attention_forward(q, _expand_kv(k, H), _expand_kv(v, H), causal=causal, scale=scale)


def attention_backward_gqa(q, k, v, dout, causal=False, scale=None):
    """Gradients for grouped key/value heads: dK, dV [B, Hkv, N, d] sum over each group."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = attention_backward(q, _expand_kv(k, H), _expand_kv(v, H), do, causal=causal, scale=scale)
    g = H // Hkv
    return dq, dk.reshape(B, Hkv, g, N, -1).sum(axis=2), dv.reshape(B, Hkv, g, N, -1).sum(axis=2)


def _unpack(x, t0, t1):
    """Rows t0..t1-1 of a packed [total, heads, d] tensor as [1, heads, L, d]."""
    return np.transpose(x[t0:t1], (1, 0, 2))[None]


def attention_forward_varlen(q, k, v, cu_seqlens, causal=False, scale=None):
    """Packed variable-length forward: q [total, H, d], k/v [total, Hkv, d].

    Returns (o [total, H, d], lse [H, total])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.asarray(_f64(cu_seqlens), dtype=np.int64)
    total, H, d = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((H, total))
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        if t1 == t0:
            continue
        ob, lb = attention_forward_gqa(_unpack(q, t0, t1), _unpack(k, t0, t1), _unpack(v, t0, t1),
                                       causal=causal, scale=scale)
        o[t0:t1] = np.transpose(ob[0], (1, 0, 2))
        lse[:, t0:t1] = lb[0]
    return o, lse


def attention_backward_varlen(q, k, v, dout, cu_seqlens, causal=False, scale=None):
    """Packed variable-length backward; returns dq [total, H, d], dk, dv [total, Hkv, d]."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    cu = np.asarray(_f64(cu_seqlens), dtype=np.int64)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        if t1 == t0:
            continue
        gq, gk, gv = attention_backward_gqa(_unpack(q, t0, t1), _unpack(k, t0, t1), _unpack(v, t0, t1),
                                            _unpack(do, t0, t1), causal=causal, scale=scale)
        dq[t0:t1] = np.transpose(gq[0], (1, 0, 2))
        dk[t0:t1] = np.transpose(gk[0], (1, 0, 2))
        dv[t0:t1] = np.transpose(gv[0], (1, 0, 2))
    return dq, dk, dv
