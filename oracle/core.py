"""CPU oracle of the DiLoCo outer-step merge (quantize -> fp32-domain merge -> Nesterov).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only the tests, the package's smoke check and the benchmark's
``cpu_baseline`` leg use it.  It shares no code with the HIP path.

It is plain and slow on purpose: numpy, one tensor and one learner at a time,
fp64 for every statistic, sum and optimizer step, and the fp32 formula for the
bucket index.  Sources (the pages):

  * INTELLECT-1 reading notes, "Training a 10B Model Across 3 Continents":
      - section 3.2 (worked example): step 4 the pseudo-gradient is the start
        weights minus the learner's end weights; step 5 mu ~ 0, sigma ~ 1.2e-3,
        range +-7.2e-3, 256 buckets of ~5.6e-5, 64 MB -> 16 MB; step 6 the
        learners' pseudo-gradients are averaged with the sum kept in fp32 and
        only int8 on the wire; step 7 Nesterov outer optimizer, lr 0.7,
        momentum 0.9.
      - section 4.1 (uniform quantization with clipping): per-tensor mu and
        sigma; clip to [mu - 6 sigma, mu + 6 sigma]; 256 equal buckets; each
        codebook value is the mean of the data in its bucket, not the midpoint.
      - section 4.2: quantization is for transport only; receivers dequantize
        and accumulate in floating point, because Q(a) + Q(b) != Q(a + b).
  * Decoupled DiLoCo digest, "Resilient, Distributed AI Training at Scale":
      - section "architecture", item 4: P = 24 fragments built by greedy
        bin-packing of whole tensors into balanced fragments (note 1);
      - section "fault tolerance", items 1 and 3: merge once a minimum quorum
        has arrived; learners are weighted (token/step weighted merge).
      - section "architecture": the syncer holds the global fragments, merges
        one fragment at a time and sends the updated fragment back; the
        INTELLECT-1 notes' section 3.2 step 8 likewise has every worker copy the
        updated weights before the next outer step (broadcast, outer_cycle).
      - section "architecture", the second engineering detail, and "fault
        tolerance" item 3: Radial-Directional Averaging averages the outer
        gradients' directions and norms separately (rda_merge); no formula.

Readings taken where the pages are silent:
  * sigma is the population std (ddof = 0) of the whole tensor;
  * lo = fl32(mu - 6 sigma), hi = fl32(mu + 6 sigma), wd = fl32(12 sigma / 256);
  * code = clip(floor(fl32(fl32(x - lo) / wd)), 0, 255), all IEEE fp32 RNE;
  * codebook entries average the *clipped* values; an empty bucket holds its
    midpoint fl32(lo + (c + 1/2) wd); a tensor whose wd is not a normal fp32
    (zero variance) codes every element as 0 and every entry as fl32(mu);
  * weights are normalised as w_i / sum_j w_j in fp64 with a left-to-right sum;
    a zero total is a failed quorum and changes nothing;
  * Nesterov in the PyTorch SGD form: v <- beta v + g; theta <- theta - lr (g + beta v),
    computed in fp64 from the fp32 state and rounded back to fp32 once;
  * Radial-Directional Averaging, per tensor on the dequantized pseudo-gradients:
    g = (sum_i w_i ||x_i||) d / ||d|| with d = sum_i w_i x_i / ||x_i||;
  * NaN or Inf in a pseudo-gradient is outside the contract: the oracle raises;
  * greedy bin-packing = LPT: tensors by size descending (ties: lower index
    first), each onto the least-loaded fragment (ties: lower fragment id).
"""
from __future__ import annotations

import numpy as np

N_BUCKETS = 256
CLIP_SIGMAS = 6.0
FLT_MIN = float(np.finfo(np.float32).tiny)


class NoQuorum(RuntimeError):
    """Raised when every learner weight is zero (no learner arrived)."""


# --- fragment plan (Decoupled DiLoCo: balanced tensor fragmentation) ---------

def fragment_plan(numel, n_fragments):
    """Greedy bin-packing of whole tensors into `n_fragments` balanced fragments.

    Largest tensor first (ties: lower tensor index), each placed on the fragment
    with the smallest load so far (ties: lower fragment id).  Returns
    (fragment_of[T], fragment_numel[P]).
    """
    numel = [int(n) for n in numel]
    loads = [0] * n_fragments
    fragment_of = [0] * len(numel)
    order = sorted(range(len(numel)), key=lambda t: (-numel[t], t))
    for t in order:
        best = 0
        for p in range(1, n_fragments):
            if loads[p] < loads[best]:
                best = p
        fragment_of[t] = best
        loads[best] += numel[t]
    return fragment_of, loads


# --- stage 1: pseudo-gradient (INTELLECT-1 notes, section 3.2 step 4) ---------

def pseudo_gradient(theta_global, theta_learner):
    """Delta = theta_global - theta_learner, one IEEE fp32 subtraction per element."""
    a = np.asarray(theta_global, dtype=np.float32)
    b = np.asarray(theta_learner, dtype=np.float32)
    return np.subtract(a, b, dtype=np.float32)


# --- stage 2: per-tensor quantizer (INTELLECT-1 notes, section 4.1) -----------

def tensor_stats(x):
    """Population mean and std of one tensor's pseudo-gradient, two passes in fp64."""
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = x64.size
    mu = float(np.sum(x64)) / n
    dev = x64 - mu
    var = float(np.sum(dev * dev)) / n
    return mu, float(np.sqrt(var))


def clip_range(mu, sigma):
    """Clip range [mu - 6 sigma, mu + 6 sigma] and the width of one of 256 equal
    buckets, each rounded once to fp32.  Returns (lo, hi, wd, mean32, degenerate)."""
    lo = np.float32(mu - CLIP_SIGMAS * sigma)
    hi = np.float32(mu + CLIP_SIGMAS * sigma)
    wd = np.float32(2.0 * CLIP_SIGMAS * sigma / N_BUCKETS)
    degenerate = not (float(wd) >= FLT_MIN)
    return lo, hi, wd, np.float32(mu), degenerate


def encode(x, lo, wd):
    """Bucket index of every element: floor(fl32(fl32(x - lo) / wd)) clipped to [0, 255]."""
    x = np.asarray(x, dtype=np.float32)
    lo = np.float32(lo)
    wd = np.float32(wd)
    t = np.subtract(x, lo, dtype=np.float32)
    q = np.divide(t, wd, dtype=np.float32)
    c = np.clip(np.floor(q), 0.0, float(N_BUCKETS - 1))
    return c.astype(np.uint8)


def clip_values(x, lo, hi):
    """The clipped pseudo-gradient min(max(x, lo), hi), fp32."""
    return np.minimum(np.maximum(np.asarray(x, np.float32), np.float32(lo)), np.float32(hi))


def histogram(codes, x_clipped):
    """Per-bucket (sum of clipped values in fp64, element count)."""
    codes = np.asarray(codes).astype(np.int64)
    s = np.bincount(codes, weights=np.asarray(x_clipped, np.float32).astype(np.float64),
                    minlength=N_BUCKETS)
    n = np.bincount(codes, minlength=N_BUCKETS)
    return s.astype(np.float64), n.astype(np.int64)


def codebook(bucket_sum, bucket_count, lo, wd):
    """Codebook = mean of the clipped values in each bucket, rounded once to fp32;
    an empty bucket holds its midpoint."""
    cb = np.empty(N_BUCKETS, dtype=np.float32)
    for c in range(N_BUCKETS):
        if bucket_count[c] > 0:
            cb[c] = np.float32(bucket_sum[c] / float(bucket_count[c]))
        else:
            cb[c] = np.float32(float(lo) + (c + 0.5) * float(wd))
    return cb


def quantize_tensor(x, given_range=None):
    """Quantize one learner's pseudo-gradient of one tensor.

    Returns a dict with mu, sigma, lo, hi, wd, mean32, degenerate, codes,
    bucket_sum, bucket_count and codebook.  `given_range` = (lo, hi, wd, mean32)
    skips the statistics and uses that range instead.
    """
    x = np.asarray(x, dtype=np.float32).ravel()
    if not np.isfinite(x).all():
        raise ValueError("non-finite pseudo-gradient: NaN and Inf are outside the method's contract")
    if given_range is None:
        mu, sigma = tensor_stats(x)
        lo, hi, wd, m32, degenerate = clip_range(mu, sigma)
    else:
        lo, hi, wd, m32 = (np.float32(v) for v in given_range)
        mu, sigma = float(m32), float("nan")
        degenerate = not (float(wd) >= FLT_MIN)
    if degenerate:
        codes = np.zeros(x.size, dtype=np.uint8)
        s, n = histogram(codes, clip_values(x, lo, hi))
        cb = np.full(N_BUCKETS, m32, dtype=np.float32)
    else:
        codes = encode(x, lo, wd)
        s, n = histogram(codes, clip_values(x, lo, hi))
        cb = codebook(s, n, lo, wd)
    return dict(mu=mu, sigma=sigma, lo=lo, hi=hi, wd=wd, mean32=m32,
                degenerate=degenerate, codes=codes, bucket_sum=s, bucket_count=n,
                codebook=cb)


def dequantize(codes, cb):
    """fp32 value of every code under its codebook."""
    return np.asarray(cb, np.float32)[np.asarray(codes).astype(np.int64)]


# --- stage 3: weighted merge in the float domain (sections 3.2 step 6, 4.2) ---

def normalize_weights(weights):
    """w_i / sum_j w_j in fp64 (left-to-right sum).  Zero total -> NoQuorum."""
    w = [float(v) for v in weights]
    if any(not (v >= 0.0) for v in w):
        raise ValueError("weights must be >= 0")
    total = 0.0
    for v in w:
        total += v
    if not (total > 0.0):
        raise NoQuorum("no learner present")
    return [v / total for v in w]


def merge(codes_per_learner, codebook_per_learner, w_hat):
    """g = sum_i w_hat_i * cb_i[code_i] in fp64, learners in index order; a learner
    with weight 0 is skipped (never read)."""
    g = None
    for codes, cb, w in zip(codes_per_learner, codebook_per_learner, w_hat):
        if w == 0.0:
            continue
        term = np.float64(w) * dequantize(codes, cb).astype(np.float64)
        g = term if g is None else g + term
    return g


# Averaged directions no longer than this share of their largest possible norm are
# rounding noise of directions that cancel (see rda_merge).
RDA_NULL_DIRECTION = 2.0 ** -40


def rda_merge(codes_per_learner, codebook_per_learner, w_hat):
    """Radial-Directional Averaging (Decoupled DiLoCo digest, "architecture", the
    second engineering detail, and "fault tolerance" item 3): instead of a plain
    mean of the outer gradients, their directions and their norms are averaged
    separately.  The page gives no formula; the reading taken, per tensor, on the
    dequantized pseudo-gradients x_i in fp64, learners in index order, weight-0
    learners skipped:

        r_i = ||x_i||_2                  the learner's norm
        u_i = x_i / r_i                  its direction (none when r_i = 0)
        r   = sum_i w_hat_i r_i          the averaged norm
        d   = sum_i w_hat_i u_i          the averaged direction
        g   = r * d / ||d||_2            (g = 0 when d = 0)

    so g has the averaged norm and points along the averaged direction.
    ||d|| is at most W = sum of w_hat_i over the learners with r_i > 0.  Directions
    that cancel in real arithmetic (d = 0, e.g. constant tensors moved by opposite
    amounts under equal weights) leave only rounding noise in d, about K 2^-53 W,
    which points nowhere in particular; d therefore counts as zero when
    ||d|| <= RDA_NULL_DIRECTION * W."""
    n = len(codes_per_learner[0])
    r = 0.0
    w_moved = 0.0
    d = None
    for codes, cb, w in zip(codes_per_learner, codebook_per_learner, w_hat):
        if w == 0.0:
            continue
        x = dequantize(codes, cb).astype(np.float64)
        r_i = float(np.sqrt(np.sum(x * x)))
        r += w * r_i
        if r_i > 0.0:
            w_moved += w
            term = w * (x / r_i)
            d = term if d is None else d + term
    if d is None:
        return np.zeros(n, np.float64)
    d_norm = float(np.sqrt(np.sum(d * d)))
    if d_norm <= RDA_NULL_DIRECTION * w_moved:
        return np.zeros(n, np.float64)
    return r * (d / d_norm)


# --- stage 4: Nesterov outer step (section 3.2 step 7) ------------------------

def nesterov(theta, momentum, g, lr=0.7, beta=0.9):
    """PyTorch SGD-Nesterov form, dampening 0: v <- beta v + g;
    theta <- theta - lr (g + beta v).  fp64 arithmetic, fp32 state out."""
    th = np.asarray(theta, np.float32).astype(np.float64)
    v = np.asarray(momentum, np.float32).astype(np.float64)
    g = np.asarray(g, np.float64)
    v_new = beta * v + g
    th_new = th - lr * (g + beta * v_new)
    return th_new.astype(np.float32), v_new.astype(np.float32)


# --- one merge call over a fragment -------------------------------------------

def outer_step(theta_g, momentum, theta_L, learner_stride, tensors, weights,
               present=None, lr=0.7, beta=0.9, given_ranges=None, bases=None, rule="mean"):
    """One outer step over the tensors of one fragment.

    theta_g, momentum : fp32 flat arrays (not modified; new copies are returned)
    theta_L           : fp32 [K, learner_stride]
    tensors           : list of (offset, loffset, numel)
    weights           : raw learner weights; 0 = absent
    present           : learners that quantize (default: weight > 0)
    given_ranges      : optional {(i, t): (lo, hi, wd, mean32)} pinned ranges
    bases             : optional list of K fp32 flat arrays laid out like theta_g:
                        learner i's pseudo-gradient is taken against bases[i] (a
                        stale learner's starting point, Decoupled DiLoCo digest,
                        "fault tolerance"); the update is still applied to theta_g
    rule              : "mean" (the weighted mean, merge) or "rda" (Radial-
                        Directional Averaging, rda_merge)

    Returns dict(theta=..., momentum=..., quant={(i, t): quantize_tensor dict},
    g={t: fp64 merged pseudo-gradient}).  Raises NoQuorum when all weights are 0.
    """
    k = theta_L.shape[0]
    w_hat = normalize_weights(weights)
    if present is None:
        present = [1 if w > 0 else 0 for w in weights]
    th = np.array(theta_g, dtype=np.float32, copy=True)
    mom = np.array(momentum, dtype=np.float32, copy=True)
    quant, gs = {}, {}
    for t, (off, loff, n) in enumerate(tensors):
        tg = th[off:off + n]
        codes, cbs, ws = [], [], []
        for i in range(k):
            if not present[i]:
                continue
            base = tg if bases is None else np.asarray(bases[i], np.float32)[off:off + n]
            x = pseudo_gradient(base, theta_L[i, loff:loff + n])
            gr = None if given_ranges is None else given_ranges.get((i, t))
            q = quantize_tensor(x, gr)
            quant[(i, t)] = q
            codes.append(q["codes"])
            cbs.append(q["codebook"])
            ws.append(w_hat[i])
        g = rda_merge(codes, cbs, ws) if rule == "rda" else merge(codes, cbs, ws)
        gs[t] = g
        th[off:off + n], mom[off:off + n] = nesterov(tg, mom[off:off + n], g, lr, beta)
    return dict(theta=th, momentum=mom, quant=quant, g=gs)


# ---------------------------------------------------------------------------
# Sending the update back, and a whole outer step over every fragment.
# ---------------------------------------------------------------------------
def broadcast(theta_g, theta_L, tensors, rows=None):
    """Every learner copies the updated tensors (INTELLECT-1 notes, section 3.2
    step 8; Decoupled DiLoCo digest, "architecture": the syncer sends the updated
    fragment back).  Returns a new [K, stride] array; rows selects learners."""
    out = np.array(theta_L, dtype=np.float32, copy=True)
    for off, loff, n in tensors:
        for i in range(out.shape[0]):
            if rows is None or rows[i]:
                out[i, loff:loff + n] = theta_g[off:off + n]
    return out


def outer_cycle(theta_g, momentum, theta_L, learner_stride, tensors, fragment_first, weights,
                lr=0.7, beta=0.9, send_back=False, rule="mean"):
    """One outer step over every fragment in id order (Decoupled DiLoCo digest,
    "architecture" item 4).  Fragment f owns tensors[fragment_first[f]:
    fragment_first[f + 1]] and merges with weights[f] (0 = learner absent for
    that fragment), by the weighted mean or, with rule "rda", by Radial-
    Directional Averaging (the digest's merge, see rda_merge).  With send_back,
    the fragment's updated tensors are copied to every learner right after its
    merge.  Returns dict(theta, momentum, theta_L, steps={f: outer_step result})."""
    th = np.array(theta_g, dtype=np.float32, copy=True)
    mom = np.array(momentum, dtype=np.float32, copy=True)
    tl = np.array(theta_L, dtype=np.float32, copy=True)
    steps = {}
    for f in range(len(fragment_first) - 1):
        sel = list(tensors[fragment_first[f]:fragment_first[f + 1]])
        if not sel:
            continue
        w = list(weights[f])
        res = outer_step(th, mom, tl, learner_stride, sel, w, [1 if x > 0 else 0 for x in w], lr, beta, rule=rule)
        th, mom = res["theta"], res["momentum"]
        steps[f] = res
        if send_back:
            tl = broadcast(th, tl, sel)
    return dict(theta=th, momentum=mom, theta_L=tl, steps=steps)


def merge_weights(tokens, arrival, quorum, grace):
    """Which learners a fragment's merge takes and with what weight (Decoupled
    DiLoCo digest, "fault tolerance" items 1-3): wait for `quorum` learners, then
    at most `grace` seconds more, and weight every learner that made it by the
    tokens it processed.  arrival[i] = inf (or NaN) means learner i never arrived.
    Returns (weights, merge_time); raises NoQuorum if fewer than `quorum`
    arrived or the merged learners processed no tokens."""
    k = len(tokens)
    came = [i for i in range(k) if np.isfinite(arrival[i])]
    if len(came) < quorum:
        raise NoQuorum(f"{len(came)} of {k} learners arrived, quorum {quorum}")
    # the quorum-th arrival, earlier index first among equal times
    by_time = sorted(came, key=lambda i: (arrival[i], i))
    t_quorum = arrival[by_time[quorum - 1]]
    deadline = t_quorum + grace
    weights = [float(tokens[i]) if i in came and arrival[i] <= deadline else 0.0 for i in range(k)]
    if sum(weights) <= 0.0:
        raise NoQuorum("the merged learners processed no tokens")
    in_time = [arrival[i] for i in came if arrival[i] <= deadline]
    if len(came) == k and max(in_time) < deadline:
        return weights, float(max(in_time))
    return weights, float(deadline)


# ---------------------------------------------------------------------------
# The ring all-reduce with requantization at every hop (INTELLECT-1 notes,
# section 3.2 step 6 and section 4.2): K ranks each hold a pseudo-gradient; a
# message is quantized before it is sent, the receiver dequantizes it and adds it
# to its own fp32 copy, so every hop quantizes a running sum afresh.
# ---------------------------------------------------------------------------
RING_ALIGN = 64


def ring_chunks(n, k):
    """Tensor of n elements cut into k chunks of whole 64-element groups, as
    equal as possible: chunk j = [64 floor(j m / k), 64 floor((j + 1) m / k))
    clipped to n, m = ceil(n / 64).  Chunks may be empty when m < k."""
    m = -(-n // RING_ALIGN)
    bounds = [min(n, RING_ALIGN * ((j * m) // k)) for j in range(k + 1)]
    return [(bounds[j], bounds[j + 1]) for j in range(k)]


def ring_sent_chunk(rank, hop, k):
    """The chunk rank `rank` sends to rank + 1 at reduce-scatter hop `hop`: its own
    chunk first, then each chunk it has just received.  After k - 1 hops the rank
    holds the whole sum of chunk ring_sent_chunk(rank, k - 1, k) = rank + 1."""
    return (rank - hop) % k


def ring_message(x):
    """What the receiver gets for a sent fp32 array: its quantization, dequantized."""
    q = quantize_tensor(x)
    return q, dequantize(q["codes"], q["codebook"])


def ring_outer_step(theta_g, momentum, theta_L, learner_stride, tensors, lr=0.7, beta=0.9, trace=None):
    """One outer step whose K learners (every row of theta_L, equal weights)
    average their pseudo-gradients through a ring, tensor by tensor:

    reduce-scatter, K - 1 hops: at hop s rank r sends its running sum of chunk
      (r - s) mod K, quantized (quantize_tensor on that chunk); rank r + 1 adds
      the dequantized message to its own fp32 value of the chunk: acc = fl32(acc + deQ).
    Rank r then holds the sum of chunk (r + 1) mod K; it divides by K in fp32
      (mean = fl32(sum / K)) and quantizes the mean once.
    all-gather: that message travels the ring unchanged, so every rank ends with
      deQ(Q(mean)) for every chunk; g is that value, and Nesterov updates theta_g.

    Returns dict(theta, momentum, g={t: fp32 array}, messages=[(tensor, hop,
    sender, chunk, quantize_tensor dict)]).  trace, if a list, receives the
    accumulator arrays after every hop."""
    k = theta_L.shape[0]
    th = np.array(theta_g, dtype=np.float32, copy=True)
    mom = np.array(momentum, dtype=np.float32, copy=True)
    gs, messages = {}, []
    for t, (off, loff, n) in enumerate(tensors):
        acc = [pseudo_gradient(th[off:off + n], theta_L[r, loff:loff + n]) for r in range(k)]
        chunks = ring_chunks(n, k)
        for s in range(k - 1):
            sends = []
            for r in range(k):
                c = ring_sent_chunk(r, s, k)
                a, b = chunks[c]
                if b > a:
                    q, d = ring_message(acc[r][a:b])
                    messages.append((t, s, r, c, q))
                    sends.append((r, c, d))
            for r, c, d in sends:  # every rank sends before anyone adds
                a, b = chunks[c]
                dst = (r + 1) % k
                acc[dst][a:b] = np.add(acc[dst][a:b], d, dtype=np.float32)
            if trace is not None:
                trace.append([x.copy() for x in acc])
        g = np.zeros(n, np.float32)
        for r in range(k):
            c = ring_sent_chunk(r, k - 1, k)
            a, b = chunks[c]
            if b > a:
                mean = np.divide(acc[r][a:b], np.float32(k), dtype=np.float32)
                q, d = ring_message(mean)
                messages.append((t, k - 1, r, c, q))
                g[a:b] = d
        gs[t] = g
        th[off:off + n], mom[off:off + n] = nesterov(th[off:off + n], mom[off:off + n], g.astype(np.float64), lr, beta)
    return dict(theta=th, momentum=mom, g=gs, messages=messages)

