"""Plain fp64 definition of the offline top-K KL distillation loss and its gradients.

TEST INFRASTRUCTURE ONLY: the GPU library never imports this module, and this
module imports nothing from the GPU library. Inputs arrive as host arrays
(bf16 values already widened exactly to fp32); every step below runs in fp64.

Sources (web pages; the citation names the page and the section):
  [HF]    "Making Knowledge Distillation Cheap Enough to Run at Scale", as
          written up in "Knowledge Distillation 비용 줄이기: offline top-K logits와
          chunked KL 적용 기준" (aibase.it) - sections "offline top-K logits" and
          "what chunked KL loss does" (dense KL expands the cached top-K logits
          into a dense teacher probability grid and compares it with the dense
          student log-probability grid; that dense form is the correctness
          baseline; the chunked and fused forms compute the same loss without the
          grids), and "operations" (cache validation items).
  [REV]   "[논문리뷰] Efficient Knowledge Distillation for LLMs: Offline Top-K
          Logits and a Fused Chunked KL Loss" - section 1 (key terms: the fused
          loss folds the output projection into the loss, chunk by chunk).
  [AIT]   AI Trends summary of the same work - glossary (KL loss, top-K cache,
          chunked KL) and evidence list (all loss variants reach the same loss).
  [PRIM]  "LLM Primer, Chapter 6 - Pruning and Distillation", section 6.2 (the
          loss is the KL divergence between temperature-softened teacher and
          student distributions; MiniLLM's reverse KL is named as the departure).
  [SKD]   "Rethinking Selective Knowledge Distillation" summary (gist.science) -
          Method, section 2 (SE-KD: supervise the top-k% positions ranked by
          student entropy H(q_t)) and section 3 (selective LM head, chunked
          entropy).

Readings where the pages are silent (each is repeated in the design doc):
  * forward KL(p_teacher || q_student) [HF dense KL compares a teacher probability
    grid with a student log-probability grid; PRIM names reverse KL as another
    method's departure];
  * both sides softened by the same T: p = softmax(l/T), q = softmax(z/T) [PRIM 6.2];
  * no T^2 factor on the loss;
  * loss = sum over valid positions of KL_t, divided by the global count N of
    valid positions; N = 0 gives loss 0 and zero gradients;
  * teacher probabilities are renormalised over the K cached entries only;
  * duplicate ids in a row: their probabilities add;
  * a teacher logit of -inf gives p = 0; a row whose K logits are all -inf is a
    missing position and is excluded like a masked row;
  * entropy is in nats over the full vocabulary at T = 1; selection keeps
    floor(num*S/den) positions, highest entropy first, lower index on ties;
  * samples (segments of positions) are ranked by the mean entropy of their
    positions ([SKD] SE-KD3X sample axis); floor(num*B/den) samples are kept,
    highest mean first, lower sample index on ties; a sample without positions
    has mean -inf;
  * teacher targets may also be given as probabilities at K ids (sampled
    sparse targets, [SKD] SE-KD3X class axis): they are used as given,
    renormalised over the row (entries sharing an id add), and the temperature
    then softens the student side only; a row with a negative, NaN or infinite
    value, or with no positive mass, is missing;
  * position signals ([SKD] Method section 1 lists student cross-entropy,
    teacher uncertainty 1 - p_t(y_t), teacher-student KL and student entropy):
    the student side is taken at T = 1 like the entropy, ce_t = log sum_v
    exp(z_tv) - z_{t,y_t}; p_t is the row's KD target (the renormalised top-K
    at T, or the given probabilities), so p_t(y_t) = 0 when y_t is not among
    the row's ids; a label outside [0, V) gives NaN for both, and a missing
    teacher row NaN for the teacher uncertainty;
  * per-sequence top-k%: each segment [offsets[b], offsets[b+1]) keeps
    floor(num*len_b/den) positions by signal, highest first, lower index on
    ties; NaN signals are never kept (a segment then keeps fewer);
  * GLS (global-level selection, named in [SKD] Method section 1 without a
    definition): one threshold for all positions, keep signal >= tau; tau
    may be the smallest value kept by a top-k% selection over a pooled set of
    signals (the per-segment thresholds returned below);
  * sampled sparse targets ([SKD] SE-KD3X class axis, RS-KD: the teacher's
    logits randomly sampled into sparse targets; no procedure is given): N
    token ids drawn per position from the teacher's full softmax p_t =
    softmax(z_t / T) by inverse transform of given uniforms, the cumulative
    mass taken in ascending vocabulary order; the target gives each draw
    probability 1/N (draws of one id add);
  * the teacher cache holds, per position, the K entries of largest teacher
    logit z = h . w_v (before any temperature), ordered by z descending with the
    lower id first among equal logits; the stored logit is z rounded to fp32,
    and then to bf16 when a bf16 cache is asked for.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "teacher_scaled_grid",
    "teacher_distribution",
    "oracle_from_logits",
    "oracle_loss_grads",
    "oracle_rows",
    "oracle_dW_rows",
    "oracle_entropy",
    "oracle_entropy_rows",
    "oracle_select_top_fraction",
    "oracle_entropy_select_kl",
    "oracle_validate_topk",
    "oracle_teacher_topk",
    "oracle_select_samples",
    "oracle_position_signals",
    "oracle_select_by_signal",
    "oracle_select_above",
    "oracle_validate_topk_order",
    "oracle_teacher_sample",
]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _logsumexp_rows(X: np.ndarray) -> np.ndarray:
    """log sum_v exp(X[t, v]) per row, fp64; rows of all -inf give -inf."""
    m = np.max(X, axis=1)
    mf = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        return np.log(np.sum(np.exp(X - mf[:, None]), axis=1)) + mf


def _present_rows(tlogits, T, probs=False):
    """Rows that take part: for logits, a finite teacher log-normaliser (at
    least one finite logit, none +inf/NaN); for probabilities, every value
    finite and >= 0 and a positive sum."""
    tl = _f64(tlogits)
    if tl.shape[1] == 0:
        return np.zeros(tl.shape[0], dtype=bool)
    if probs:
        ok = np.all(np.isfinite(tl) & (tl >= 0.0), axis=1)
        return ok & (np.sum(np.where(np.isfinite(tl) & (tl > 0.0), tl, 0.0), axis=1) > 0.0)
    with np.errstate(invalid="ignore"):
        return np.isfinite(_logsumexp_rows(tl / float(T)))


def teacher_scaled_grid(ids: np.ndarray, tlogits: np.ndarray, V: int, T: float) -> np.ndarray:
    """Dense teacher grid of l/T, -inf off the cached top-K ids [HF, "what chunked KL loss does"].

    Entries that share an id in one row are combined with logaddexp of their
    scaled logits, so that after the softmax their probabilities add.
    """
    ids = np.asarray(ids)
    S, K = ids.shape
    if S and K and (ids.min() < 0 or ids.max() >= V):
        raise ValueError("teacher id out of range [0, V)")
    L = np.full((S, V), -np.inf)
    rows = np.arange(S)
    scaled = _f64(tlogits) / float(T)
    for k in range(K):
        cur = L[rows, ids[:, k]]
        with np.errstate(invalid="ignore"):
            L[rows, ids[:, k]] = np.logaddexp(cur, scaled[:, k])
    return L


def teacher_distribution(ids, tvals, V, T, probs=False):
    """Dense teacher distribution P[t, v] per row, log P, and the rows present.

    probs=False: the cached logits softened by T and renormalised over the
    row's K entries (softmax of the scaled grid; entries sharing an id add)
    [HF "what chunked KL loss does"]. probs=True: the given probabilities
    (sampled sparse targets, [SKD] SE-KD3X) scattered to their ids, entries
    sharing an id adding, renormalised over the row.
    """
    ids = np.asarray(ids)
    if not probs:
        Lt = teacher_scaled_grid(ids, tvals, V, T)
        lse_t = _logsumexp_rows(Lt)
        present = np.isfinite(lse_t)
        lse_t_safe = np.where(present, lse_t, 0.0)
        with np.errstate(invalid="ignore"):
            logP = Lt - lse_t_safe[:, None]
        P = np.where(present[:, None], np.exp(logP), 0.0)
        return P, logP, present
    S, K = ids.shape
    if S and K and (ids.min() < 0 or ids.max() >= V):
        raise ValueError("teacher id out of range [0, V)")
    pv = _f64(tvals)
    present = _present_rows(pv, T, probs=True)
    P = np.zeros((S, V))
    rows = np.arange(S)
    for k in range(K):
        add = np.where(np.isfinite(pv[:, k]) & (pv[:, k] > 0.0), pv[:, k], 0.0)
        P[rows, ids[:, k]] += add
    mass = P.sum(axis=1)
    P = np.where(present[:, None], P / np.where(mass > 0.0, mass, 1.0)[:, None], 0.0)
    with np.errstate(divide="ignore"):
        logP = np.log(P)
    return P, logP, present


def _row_terms(Z, ids, tlogits, T, probs=False):
    """Per-row dense terms of the definition for a block of rows.

    Returns (kl[t], lse[t] = logsumexp(z_t/T), soft[t, v] = softmax(z_t/T) - p_t,
    present[t] = row has at least one finite teacher logit).
    """
    Z = _f64(Z)
    S, V = Z.shape
    P, logP, present = teacher_distribution(ids, tlogits, V, T, probs)   # dense teacher grid
    ZT = Z / float(T)
    lse = _logsumexp_rows(ZT)                                    # log-normaliser of z/T over all V
    with np.errstate(invalid="ignore"):
        logQ = ZT - lse[:, None]
    pos = P > 0.0
    kl = np.zeros(S)
    for t in range(S):                                           # sum over p > 0 only: 0*log 0 = 0
        sel = pos[t]
        kl[t] = np.sum(P[t, sel] * (logP[t, sel] - logQ[t, sel]))
    soft = np.exp(logQ) - P                                      # d KL_t / d(z_t/T)
    return kl, lse, soft, present


def oracle_from_logits(Z, ids, tlogits, T=1.0, mask=None, grad_loss=1.0, probs=False):
    """Loss and logit gradient from given student logits Z[S, V] (dense definition).

    Returns dict(loss, kl_rows, lse, dZ, N, valid); dZ = d loss / d Z.
    """
    Z = _f64(Z)
    S = Z.shape[0]
    kl, lse, soft, present = _row_terms(Z, ids, tlogits, T, probs)
    m = np.ones(S, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    valid = m & present
    N = int(valid.sum())
    if N == 0:
        return dict(loss=0.0, kl_rows=kl, lse=lse, dZ=np.zeros_like(Z), N=0, valid=valid)
    loss = math.fsum(kl[valid]) / N                              # mean over valid positions
    coef = float(grad_loss) / (float(T) * N)
    dZ = np.where(valid[:, None], soft, 0.0) * coef              # (softmax(z/T) - p) / (T N)
    return dict(loss=loss, kl_rows=kl, lse=lse, dZ=dZ, N=N, valid=valid)


def oracle_loss_grads(hidden, W, ids, tlogits, T=1.0, mask=None, grad_loss=1.0, chunk=None,
                      probs=False):
    """Loss, dHidden, dW of the top-K KL loss through the output projection.

    chunk=None: the dense definition (full [S, V] grids) [HF dense KL].
    chunk=C: the same sum taken over row blocks of C, each projected, folded
    into the loss and discarded, with the count N of valid rows taken over all
    rows [REV section 1; HF "what chunked KL loss does"].
    """
    Hd, Wd = _f64(hidden), _f64(W)
    S = Hd.shape[0]
    ids = np.asarray(ids)
    tl = _f64(tlogits)
    if chunk is None:
        Z = Hd @ Wd.T
        r = oracle_from_logits(Z, ids, tl, T, mask, grad_loss, probs)
        dH = r["dZ"] @ Wd                                        # chain rule through z = h W^T
        dW = r["dZ"].T @ Hd
        return dict(loss=r["loss"], kl_rows=r["kl_rows"], lse=r["lse"], dH=dH, dW=dW,
                    N=r["N"], valid=r["valid"])
    C = int(chunk)
    if C <= 0:
        raise ValueError("chunk must be positive")
    m = np.ones(S, dtype=bool) if mask is None else (np.asarray(mask) != 0)
    present = _present_rows(tl, T, probs)
    valid = m & present
    N = int(valid.sum())
    kl_all = np.zeros(S)
    lse_all = np.zeros(S)
    dH = np.zeros_like(Hd)
    dW = np.zeros_like(Wd)
    coef = float(grad_loss) / (float(T) * N) if N else 0.0
    for c0 in range(0, S, C):
        c1 = min(S, c0 + C)
        Zc = Hd[c0:c1] @ Wd.T
        kl, lse, soft, _ = _row_terms(Zc, ids[c0:c1], tl[c0:c1], T, probs)
        kl_all[c0:c1] = kl
        lse_all[c0:c1] = lse
        if N:
            Gc = np.where(valid[c0:c1, None], soft, 0.0) * coef
            dH[c0:c1] = Gc @ Wd
            dW += Gc.T @ Hd[c0:c1]
    loss = math.fsum(kl_all[valid]) / N if N else 0.0
    return dict(loss=loss, kl_rows=kl_all, lse=lse_all, dH=dH, dW=dW, N=N, valid=valid)


def oracle_rows(hidden_rows, W, ids_rows, tl_rows, T, N, grad_loss=1.0, grads=True, probs=False):
    """Per-row outputs for a sample of rows, given the global valid count N.

    Every row of the loss depends only on its own hidden state and cache row,
    so kl_t, lse_t and dHidden_t of sampled rows follow the definition exactly.
    Returns dict(kl_rows, lse, present, dH) for the given rows (all treated as
    valid); grads=False skips dH.
    """
    Hd, Wd = _f64(hidden_rows), _f64(W)
    Z = Hd @ Wd.T
    kl, lse, soft, present = _row_terms(Z, ids_rows, tl_rows, T, probs)
    out = dict(kl_rows=kl, lse=lse, present=present)
    if grads:
        coef = float(grad_loss) / (float(T) * N) if N else 0.0
        G = np.where(present[:, None], soft, 0.0) * coef
        out["dH"] = G @ Wd
    return out


def oracle_dW_rows(hidden, W, ids, tlogits, T, lse, valid, vocab_rows, grad_loss=1.0, probs=False):
    """Rows `vocab_rows` of dW, given every row's student log-normaliser lse_t.

    dW = dZ^T hidden with dZ[t, v] = g (softmax(z_t/T)_v - p_t,v) / (T N) on
    valid rows [HF dense KL, differentiated]; column v of dZ needs only z[:, v]
    (one projection per sampled vocabulary row) and lse. p_t,v is the
    renormalised top-K teacher probability: the sum over the row's cached
    entries with id v of exp(l_k/T - logsumexp_k(l_k/T)) (-inf entries give 0).
    """
    Hd = _f64(hidden)
    vocab_rows = np.asarray(vocab_rows)
    ids = np.asarray(ids)
    valid = np.asarray(valid, dtype=bool)
    N = int(valid.sum())
    if N == 0:
        return np.zeros((len(vocab_rows), Hd.shape[1]))
    Zc = Hd @ _f64(W)[vocab_rows].T                              # z[:, v] for the sampled v
    lse = _f64(lse)
    with np.errstate(invalid="ignore", over="ignore"):
        Q = np.exp(Zc / float(T) - np.where(valid, lse, 0.0)[:, None])
    # teacher probability of each cached entry, Pk[t, k]
    if probs:
        pv = _f64(tlogits)
        use = np.isfinite(pv) & (pv > 0.0)
        mass = np.sum(np.where(use, pv, 0.0), axis=1)
        ok = _present_rows(pv, T, probs=True)
        Pk = np.where(ok[:, None] & use, pv / np.where(mass > 0.0, mass, 1.0)[:, None], 0.0)
    else:
        scaled = _f64(tlogits) / float(T)
        lt = _logsumexp_rows(scaled)                             # teacher log-normaliser per row
        fin = np.isfinite(lt)
        with np.errstate(invalid="ignore"):
            Pk = np.where(fin[:, None], np.exp(scaled - np.where(fin, lt, 0.0)[:, None]), 0.0)
    # Pc[t, j] = sum of Pk[t, k] over the entries whose id is vocab_rows[j]
    # (entries sharing an id add, in the order of k)
    if ids.size and (ids.min() < 0 or ids.max() >= W.shape[0]):
        raise ValueError("teacher id out of range [0, V)")
    uniq, inv = np.unique(vocab_rows, return_inverse=True)
    col = np.full(int(W.shape[0]), -1, dtype=np.int64)
    col[uniq] = np.arange(uniq.shape[0])
    c = col[ids]
    hit = c >= 0
    Pu = np.zeros((ids.shape[0], uniq.shape[0]))
    np.add.at(Pu, (np.nonzero(hit)[0], c[hit]), Pk[hit])
    Pc = Pu[:, inv]
    coef = float(grad_loss) / (float(T) * N)
    G = np.where(valid[:, None], Q - Pc, 0.0) * coef
    return G.T @ Hd


def oracle_entropy_rows(Z):
    """Entropy in nats of softmax(z_t) over the full vocabulary, per row [SKD section 2]."""
    Z = _f64(Z)
    lse = _logsumexp_rows(Z)
    logq = Z - lse[:, None]
    q = np.exp(logq)
    return -np.sum(np.where(q > 0.0, q * logq, 0.0), axis=1)


def oracle_entropy(hidden, W, chunk=None):
    """Student entropy H(q_t), q_t = softmax(hidden_t W^T), per position [SKD sections 2-3].

    chunk bounds the rows projected at once (the chunked-entropy form); the
    result does not depend on it.
    """
    Hd, Wd = _f64(hidden), _f64(W)
    S = Hd.shape[0]
    C = S if chunk is None else int(chunk)
    out = np.zeros(S)
    for c0 in range(0, S, max(C, 1)):
        c1 = min(S, c0 + C)
        out[c0:c1] = oracle_entropy_rows(Hd[c0:c1] @ Wd.T)
    return out


def oracle_select_top_fraction(entropy, num, den):
    """Keep floor(num*S/den) positions, highest entropy first, lower index on ties [SKD section 2].

    Returns (mask uint8 [S], idx int32 ascending, count).
    """
    e = _f64(entropy)
    S = e.shape[0]
    if den <= 0 or num < 0 or num > den:
        raise ValueError("need 0 <= num <= den, den > 0")
    k = (int(num) * S) // int(den)
    order = np.argsort(-e, kind="stable")
    keep = np.sort(order[:k])
    mask = np.zeros(S, dtype=np.uint8)
    mask[keep] = 1
    return mask, keep.astype(np.int32), k


def oracle_entropy_select_kl(hidden, W, ids, tlogits, num=20, den=100, T=1.0, grad_loss=1.0,
                             chunk=None):
    """Entropy-selective variant: entropy over all positions, top num/den kept,
    then the top-K KL loss and gradients over the kept positions only
    [SKD sections 2-3: SE-KD with a selective LM head]."""
    ent = oracle_entropy(hidden, W, chunk=chunk)
    mask, idx, k = oracle_select_top_fraction(ent, num, den)
    r = oracle_loss_grads(hidden, W, ids, tlogits, T=T, mask=mask, grad_loss=grad_loss,
                          chunk=chunk)
    r.update(entropy=ent, mask=mask, idx=idx, count=k)
    return r


def oracle_validate_topk(ids, tlogits, V, probs=False):
    """Cache checks named in [HF "operations"]: token id range and missing positions.

    Returns (n_bad_id, n_empty_row, n_bad_value).
      logits (probs=False): ids outside [0, V); rows whose K logits are all
        -inf; logits that are NaN or +inf.
      probabilities (probs=True, sampled sparse targets, [SKD] SE-KD3X class
        axis): ids outside [0, V); rows with no value that is finite and
        positive (no mass); values that are not finite and >= 0.
    A row counted as empty or holding a bad value takes no part in the loss.
    """
    ids = np.asarray(ids)
    tl = _f64(tlogits)
    n_bad_id = int(np.count_nonzero((ids < 0) | (ids >= V)))
    if probs:
        fin = np.isfinite(tl)
        with np.errstate(invalid="ignore"):
            mass = fin & (tl > 0.0)
            bad = ~(fin & (tl >= 0.0))
        n_empty = int(np.count_nonzero(~np.any(mass, axis=1))) if tl.shape[1] else tl.shape[0]
        return n_bad_id, n_empty, int(np.count_nonzero(bad))
    n_empty = int(np.count_nonzero(np.all(np.isneginf(tl), axis=1))) if tl.size else 0
    n_bad_logit = int(np.count_nonzero(np.isnan(tl) | np.isposinf(tl)))
    return n_bad_id, n_empty, n_bad_logit


def oracle_validate_topk_order(ids, tlogits):
    """The cache's top-K order ([HF "operations"] lists the top-K sorting among
    the cache checks): rows whose K values are not non-increasing (some value
    smaller than the next; a NaN compares with nothing), and rows holding an id
    more than once. Returns (n_unsorted_rows, n_duplicate_rows)."""
    ids = np.asarray(ids)
    tl = _f64(tlogits)
    with np.errstate(invalid="ignore"):
        unsorted = np.any(tl[:, :-1] < tl[:, 1:], axis=1) if tl.shape[1] > 1 else np.zeros(tl.shape[0], bool)
    srt = np.sort(ids, axis=1)
    dup = np.any(srt[:, :-1] == srt[:, 1:], axis=1) if ids.shape[1] > 1 else np.zeros(ids.shape[0], bool)
    return int(np.count_nonzero(unsorted)), int(np.count_nonzero(dup))


def _round_bf16_values(x32: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value (ties to even), as fp32."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


def oracle_teacher_topk(hidden, W, K, out_dtype="f32"):
    """Teacher top-K cache entries for every position.

    [HF "offline top-K logits"]: the teacher's output is computed once and only
    the logits of each position's K most likely tokens are kept; [HF
    "operations"]: the cache holds per-position token ids and logits, and its
    validation checks their top-K order. Softmax is monotone, so the K most
    likely tokens are the K largest logits.

    z = hidden @ W^T in fp64 from the exact inputs. Per row: the K entries of
    largest z, ordered by z descending, the lower id first among equal z.
    Returns (ids int32 [S, K], logits float32 [S, K]): z rounded to fp32, then
    to bf16 (kept as fp32 values) when out_dtype is "bf16".
    """
    Z = _f64(hidden) @ _f64(W).T
    S, V = Z.shape
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    ids = np.empty((S, K), dtype=np.int32)
    vals = np.empty((S, K), dtype=np.float64)
    col = np.arange(V)
    for t in range(S):
        order = np.lexsort((col, -Z[t]))[:K]     # primary: z descending; then id ascending
        ids[t] = order
        vals[t] = Z[t, order]
    logits = vals.astype(np.float32)
    if out_dtype == "bf16":
        logits = _round_bf16_values(logits)
    elif out_dtype != "f32":
        raise ValueError("out_dtype must be 'f32' or 'bf16'")
    return ids, logits


def oracle_select_samples(entropy, offsets, num, den):
    """Keep floor(num*B/den) of B samples by mean student entropy, highest first,
    lower sample index on ties ([SKD] Method section 2, SE-KD3X: the top l% of
    training samples by the mean student entropy of a frozen student's single
    forward pass). Sample b is positions [offsets[b], offsets[b+1]); one with no
    positions has mean -inf.

    Returns (sample mask uint8 [B], kept sample ids int32 ascending, count, means).
    """
    e = _f64(entropy)
    off = np.asarray(offsets, dtype=np.int64)
    B = off.shape[0] - 1
    if B < 0 or np.any(np.diff(off) < 0) or (B > 0 and (off[0] < 0 or off[-1] > e.shape[0])):
        raise ValueError("offsets must be non-decreasing within [0, S]")
    if den <= 0 or num < 0 or num > den:
        raise ValueError("need 0 <= num <= den, den > 0")
    means = np.array([np.mean(e[off[b]:off[b + 1]]) if off[b + 1] > off[b] else -np.inf
                      for b in range(B)])
    k = (int(num) * B) // int(den)
    order = np.argsort(-means, kind="stable")
    keep = np.sort(order[:k])
    mask = np.zeros(B, dtype=np.uint8)
    mask[keep] = 1
    return mask, keep.astype(np.int32), k, means


def oracle_position_signals(hidden, W, ids, tlogits, labels, T=1.0, probs=False, chunk=None):
    """Per-position importance signals ([SKD] Method section 1: student
    cross-entropy, teacher uncertainty 1 - p_t(y_t), student entropy; the
    teacher-student KL per position is oracle_rows' kl_rows).

    entropy_t = H(softmax(z_t)) and ce_t = logsumexp(z_t) - z_{t,y_t}, both at
    T = 1 with z_t = hidden_t W^T; teacher_unc_t = 1 - p_t(y_t) with p_t the
    row's KD target (renormalised top-K softmax at T, or the given
    probabilities), summed over entries sharing the label's id. A label
    outside [0, V) gives NaN ce and teacher_unc; a missing teacher row gives
    NaN teacher_unc. Returns dict(entropy, ce, teacher_unc), fp64 [S].
    """
    Hd, Wd = _f64(hidden), _f64(W)
    S, V = Hd.shape[0], Wd.shape[0]
    y = np.asarray(labels, dtype=np.int64)
    has = (y >= 0) & (y < V)
    C = S if chunk is None else int(chunk)
    ent = np.zeros(S)
    ce = np.full(S, np.nan)
    for c0 in range(0, S, max(C, 1)):
        c1 = min(S, c0 + C)
        Z = Hd[c0:c1] @ Wd.T
        ent[c0:c1] = oracle_entropy_rows(Z)
        lse = _logsumexp_rows(Z)                       # log-normaliser at T = 1
        yy = np.where(has[c0:c1], y[c0:c1], 0)
        zy = Z[np.arange(c1 - c0), yy]                 # the student's logit at the label
        ce[c0:c1] = np.where(has[c0:c1], lse - zy, np.nan)
    tl = _f64(tlogits)
    ids = np.asarray(ids)
    if S and ids.shape[1] and (ids.min() < 0 or ids.max() >= V):
        raise ValueError("teacher id out of range [0, V)")
    present = _present_rows(tl, T, probs)
    tu = np.full(S, np.nan)
    for t in range(S):
        if not (has[t] and present[t]):
            continue
        if probs:
            w = np.where(np.isfinite(tl[t]) & (tl[t] > 0.0), tl[t], 0.0)
        else:
            sc = tl[t] / float(T)
            w = np.exp(sc - np.max(sc))                # -inf entries give 0
        tu[t] = 1.0 - np.sum(w[ids[t] == y[t]]) / np.sum(w)
    return dict(entropy=ent, ce=ce, teacher_unc=tu)


def _check_offsets(off, S):
    B = off.shape[0] - 1
    if B < 0 or np.any(np.diff(off) < 0) or (B > 0 and (off[0] < 0 or off[-1] > S)):
        raise ValueError("offsets must be non-decreasing within [0, S]")
    return B


def oracle_select_by_signal(signal, offsets, num, den):
    """Top-k% positions by a signal, per segment ([SKD] Method section 1,
    top-k% selection; per sequence when offsets are given).

    Segment b is positions [offsets[b], offsets[b+1]) (offsets None: one
    segment [0, S)); it keeps floor(num*len_b/den) positions, highest signal
    first, lower index first among equal values. NaN signals are never kept.
    Returns (mask uint8 [S], idx int32 ascending, count, thresholds [B]) with
    thresholds[b] the smallest kept value of segment b (NaN if none kept).
    """
    x = _f64(signal)
    S = x.shape[0]
    off = np.array([0, S], dtype=np.int64) if offsets is None else np.asarray(offsets, np.int64)
    B = _check_offsets(off, S)
    if den <= 0 or num < 0 or num > den:
        raise ValueError("need 0 <= num <= den, den > 0")
    mask = np.zeros(S, dtype=np.uint8)
    thr = np.full(B, np.nan)
    for b in range(B):
        a, e = int(off[b]), int(off[b + 1])
        cand = np.arange(a, e)[~np.isnan(x[a:e])]
        k = min((int(num) * (e - a)) // int(den), cand.shape[0])
        keep = cand[np.argsort(-x[cand], kind="stable")][:k]
        mask[keep] = 1
        if k > 0:
            thr[b] = np.min(x[keep])
    idx = np.flatnonzero(mask).astype(np.int32)
    return mask, idx, int(idx.shape[0]), thr


def oracle_select_above(signal, tau):
    """GLS reading: one global threshold, keep the positions whose signal is
    >= tau; NaN is never kept. Returns (mask uint8 [S], idx int32, count)."""
    x = _f64(signal)
    with np.errstate(invalid="ignore"):
        mask = (x >= float(tau)).astype(np.uint8)
    idx = np.flatnonzero(mask).astype(np.int32)
    return mask, idx, int(idx.shape[0])


def oracle_teacher_cdf(hidden, W, T):
    """Teacher distribution of the sampled targets: P = softmax(z / T) per row
    (z = hidden W^T, fp64) and F, its cumulative sum over ids 0..v in
    vocabulary order. Returns (P, F), each [S, V] fp64."""
    Z = (_f64(hidden) @ _f64(W).T) / float(T)
    P = np.exp(Z - _logsumexp_rows(Z)[:, None])
    return P, np.cumsum(P, axis=1)


def oracle_teacher_sample(hidden, W, T, uniforms, chunk=None):
    """Sampled sparse teacher targets ([SKD] SE-KD3X class axis, RS-KD): for
    each position t and uniform u in [0, 1), the smallest vocabulary id v with
    F_t(v) > u, where F_t(v) is the cumulative teacher probability
    softmax(z_t / T) over ids 0..v (z_t = hidden_t W^T, fp64). A u at or above
    the last cumulative value (rounding) gives the largest id of positive
    probability. Returns ids int32 [S, N]; a target is (ids, 1/N each)."""
    Hd, Wd = _f64(hidden), _f64(W)
    U = _f64(uniforms)
    S, N = U.shape
    C = S if chunk is None else int(chunk)
    ids = np.zeros((S, N), dtype=np.int32)
    for c0 in range(0, S, max(C, 1)):
        c1 = min(S, c0 + C)
        P, F = oracle_teacher_cdf(Hd[c0:c1], Wd, T)
        for r in range(c1 - c0):
            last = int(np.flatnonzero(P[r] > 0.0)[-1])
            v = np.searchsorted(F[r], U[c0 + r], side="right")     # first F > u
            ids[c0 + r] = np.minimum(v, last)
    return ids
