"""Independent brute-force statement of VSA for tiny inputs (tests only).

Written in matrix form, separately from the oracle's per-row loops: the tile
selection becomes an explicit 0/1 token mask over the dense S x S logit
matrix (-inf where masked), and one softmax per row.  Shares no code with
``oracle/`` or the GPU library.  Method: page "UniServe: serving FastH3 at
its fastest", sections "The FastH3 workload" and "Fused output combination".
"""
import numpy as np

D = 128
T = 64


def widen(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def vsa_dense_masked(q, k, v, g, s_t, s_v, s_a, kk, valid=None):
    """Returns (out float64 [S,H,128], sel int [H,n_v,kk], coarse [H,n_v,128], mask [H,S,S]).
    valid = (text, video, audio) rows at the start of each segment that are
    tokens (default all); the others are padding: never keys, zero outputs,
    and left out of the tile means."""
    Q, K, V, G = (widen(x) for x in (q, k, v, g))
    S, H, _ = Q.shape
    n_v = s_v // T
    vt, vv, va = (s_t, s_v, s_a) if valid is None else valid
    tok = np.zeros(S, dtype=bool)
    tok[:vt] = True
    tok[s_t:s_t + vv] = True
    tok[s_t + s_v:s_t + s_v + va] = True
    alpha = 1.0 / np.sqrt(D)
    out = np.zeros((S, H, D))
    sel = np.zeros((H, n_v, kk), dtype=np.int64)
    coarse = np.zeros((H, n_v, D))
    masks = np.zeros((H, S, S), dtype=bool)
    for h in range(H):
        if n_v:
            # FP32 pooled statistics of the video tiles
            vid_tok = tok[s_t:s_t + s_v].reshape(n_v, T, 1)
            pooled = [((X[s_t:s_t + s_v, h, :].reshape(n_v, T, D) * vid_tok).sum(axis=1)
                       / vid_tok.sum(axis=1)).astype(np.float32).astype(np.float64)
                      for X in (Q, K, V)]
            qb, kb, vb = pooled
            scores = qb @ kb.T                      # [n_v (query tile), n_v (key tile)]
            for u in range(n_v):
                order = sorted(range(n_v), key=lambda w: (-scores[u, w], w))
                sel[h, u] = sorted(order[:kk])
            a = alpha * scores
            wts = np.exp(a - a.max(axis=1, keepdims=True))
            coarse[h] = (wts @ vb) / wts.sum(axis=1, keepdims=True)
        # token-level 0/1 mask expanded from the tile-level mask
        tile_of = np.arange(S) // T
        n_t = s_t // T
        mask = np.zeros((S, S), dtype=bool)
        for i in range(S):
            if s_t <= i < s_t + s_v:
                u = (i - s_t) // T
                allowed_video_tiles = set(n_t + int(w) for w in sel[h, u])
                key_is_video = (np.arange(S) >= s_t) & (np.arange(S) < s_t + s_v)
                mask[i] = ~key_is_video | np.isin(tile_of, list(allowed_video_tiles))
            else:
                mask[i] = True
        mask &= tok[None, :]
        masks[h] = mask
        logits = alpha * (Q[:, h, :] @ K[:, h, :].T)
        logits = np.where(mask, logits, -np.inf)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        o = (p @ V[:, h, :]) / p.sum(axis=1, keepdims=True)
        if n_v:
            vid = slice(s_t, s_t + s_v)
            c_rows = np.repeat(coarse[h], T, axis=0)  # broadcast each tile's output to its 64 rows
            o[vid] = o[vid] + (1.0 / (1.0 + np.exp(-G[vid, h, :]))) * c_rows
        o[~tok] = 0.0
        out[:, h, :] = o
    return out, sel, coarse, masks


def dense_masked_given_sel(q, k, v, s_t, s_v, s_a, sel):
    """Dense attention with the video-to-video keys restricted to a given
    selection sel [H][n_v][k] (video-local tile indices) and no coarse term:
    the attention that a selection rule other than the tile score (for
    instance the SubBlock router) hands to the block-sparse kernel.
    Returns float64 [S][H][128]."""
    Q, K, V = (widen(x) for x in (q, k, v))
    S, H, _ = Q.shape
    n_t = s_t // T
    tile_of = np.arange(S) // T
    key_is_video = (np.arange(S) >= s_t) & (np.arange(S) < s_t + s_v)
    alpha = 1.0 / np.sqrt(D)
    out = np.zeros((S, H, D))
    for h in range(H):
        mask = np.ones((S, S), dtype=bool)
        for i in range(s_t, s_t + s_v):
            allowed = n_t + np.asarray(sel[h, (i - s_t) // T])
            mask[i] = ~key_is_video | np.isin(tile_of, allowed)
        logits = np.where(mask, alpha * (Q[:, h, :] @ K[:, h, :].T), -np.inf)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        out[:, h, :] = (p @ V[:, h, :]) / p.sum(axis=1, keepdims=True)
    return out


def dense_masked_lists(q, k, v, lists):
    """Dense attention in which query tile j of head h may only see the key
    tiles lists[h][j] ([H][N][k], global tile indices): an explicit token-level
    0/1 mask (-inf where 0) over the S x S logits, one softmax per row, no
    coarse term.  The whole-sequence SubBlock router hands such lists to the
    block-sparse kernel.  Returns float64 [S][H][128]."""
    Q, K, V = (widen(x) for x in (q, k, v))
    S, H, _ = Q.shape
    tile_of = np.arange(S) // T
    alpha = 1.0 / np.sqrt(D)
    out = np.zeros((S, H, D))
    for h in range(H):
        mask = np.zeros((S, S), dtype=bool)
        for i in range(S):
            mask[i] = np.isin(tile_of, np.asarray(lists[h][i // T]))
        logits = np.where(mask, alpha * (Q[:, h, :] @ K[:, h, :].T), -np.inf)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        out[:, h, :] = (p @ V[:, h, :]) / p.sum(axis=1, keepdims=True)
    return out
