"""CPU oracle for the routed Mixture-of-Experts FFN layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may import
this module.  The HIP library never calls it, and it shares no code with the HIP library.

What the layer computes.  The pages (the vLLM-Moet README and its mirrors) describe a
Mixture-of-Experts layer with 384 routed experts per layer, a subset of expert slots resident
on the GPU, the remaining routed experts computed by another tier from the checkpoint's own
bytes, and the "compact" call that computes only the resident slots yet matches the
all-resident path (README, MoET hybrid table, rows "footprint, power" and "identity").  They
do not write the layer's algebra out; this module takes the plain reading of a routed SwiGLU
MoE layer:

    l[t,e]  = fp32( sum_h x[t,h] W_r[e,h] ) (+ bias[e] in fp32)      router logits
    sel(t)  = the k experts with the largest l[t,.], ties to the smaller expert id
    s[t,e]  = softmax_e(l[t,.])   or   1 / (1 + exp(-l[t,e]))          scores
    w[t,j]  = s[t,e_j] / sum_{i<k} s[t,e_i]                            renormalised gates
    FFN_e(x) = W_d,e ( silu(W_g,e x) * (W_u,e x) ),  silu(z) = z / (1 + exp(-z))
    out[t]  = sum_{j<k, slot(e_j) >= 0} w[t,j] FFN_{e_j}(x[t])

with the weights dequantised from their stored bytes and every floating-point step after the
fp32 logits carried out in fp64.  Rows (t, j) whose expert has no resident slot are left out of
the sum and listed instead, as (token, expert, weight), in ascending row order r = t*k + j.

Everything here is written for clarity, not speed: one expert slot at a time, a library matmul
as the only heavy primitive, no blocking and no fusion.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------------
# number formats (decoded from their definitions: bfloat16; OCP 8-bit floating point e4m3fn;
# OCP Microscaling v1.0 e2m1 elements and e8m0 scales)
# ----------------------------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp64: the 16 bits are the high half of an IEEE binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
    S.1111.111 is NaN; exponent 0 is subnormal with value 2^-6 * m/8."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP MX FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is
    subnormal with value m/2; no NaN or infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    return sign * np.where(e == 0, m / 2.0, np.ldexp(1.0 + m / 2.0, e - 1))


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP MX E8M0 scale: 2^(code - 127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def dequant(wdtype: str, w: np.ndarray, s, N: int, K: int) -> np.ndarray:
    """Stored bytes of ONE weight matrix [N, K] (K contiguous) -> fp64 [N, K].

    f32 / bf16: exact.  fp8: e4m3fn code times the fp32 scale of its 128x128 block,
    s[n // 128, k // 128].  mxfp4: byte j of a row holds K index 2j in its low nibble and 2j+1
    in its high nibble; value = e2m1(code) * e8m0(s[n, k // 32])."""
    if wdtype == "f32":
        return np.asarray(w, np.float32).reshape(N, K).astype(np.float64)
    if wdtype == "bf16":
        return bf16_to_f64(np.asarray(w).reshape(N, K))
    if wdtype == "fp8":
        v = e4m3fn_to_f64(np.asarray(w).reshape(N, K))
        sc = np.asarray(s, np.float32).astype(np.float64)
        rows = np.arange(N) // 128
        cols = np.arange(K) // 128
        return v * sc[rows[:, None], cols[None, :]]
    if wdtype == "mxfp4":
        b = np.asarray(w, np.uint8).reshape(N, K // 2)
        codes = np.empty((N, K), np.uint8)
        codes[:, 0::2] = b & 0xF
        codes[:, 1::2] = b >> 4
        sc = e8m0_to_f64(np.asarray(s).reshape(N, K // 32))
        return e2m1_to_f64(codes) * sc[:, np.arange(K) // 32]
    raise ValueError(wdtype)


def activations_f64(x: np.ndarray, xdtype: str) -> np.ndarray:
    """[T,H] activations (fp32 values or bf16 bit patterns) -> fp64, exactly."""
    return bf16_to_f64(x) if xdtype == "bf16" else np.asarray(x, np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# routing: logits, top-k selection, scores, renormalisation
# ----------------------------------------------------------------------------------------------


def router_logits(x64: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """l = x W_r^T evaluated in fp64 and rounded once to fp32 (the logits' precision)."""
    l64 = x64 @ np.asarray(w_router, np.float32).astype(np.float64).T
    return l64.astype(np.float32)


def add_bias(logits32: np.ndarray, bias) -> np.ndarray:
    """Optional per-expert bias, added in fp32."""
    if bias is None:
        return np.asarray(logits32, np.float32)
    return (np.asarray(logits32, np.float32) + np.asarray(bias, np.float32)[None, :]).astype(np.float32)


def select_topk(logits32: np.ndarray, k: int) -> np.ndarray:
    """[T,E] -> [T,k] int32: per token, experts ordered by (logit descending, id ascending),
    first k kept.  Selection on logits equals selection on scores because both score
    functions are strictly increasing in the logit."""
    T, E = logits32.shape
    out = np.empty((T, k), np.int32)
    ids = np.arange(E)
    for t in range(T):
        order = sorted(ids, key=lambda e: (-float(logits32[t, e]), int(e)))
        out[t] = order[:k]
    return out


def scores(logits32: np.ndarray, kind: str) -> np.ndarray:
    """Per-expert scores in fp64: softmax over ALL experts, or the logistic sigmoid."""
    l = np.asarray(logits32, np.float32).astype(np.float64)
    if kind == "softmax":
        z = np.exp(l - l.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    if kind == "sigmoid":
        return 1.0 / (1.0 + np.exp(-l))
    raise ValueError(kind)


def gate_weights(s: np.ndarray, topk_idx: np.ndarray, renorm: bool = True) -> np.ndarray:
    """w[t,j] = s[t,e_j] / sum_i s[t,e_i] (or s[t,e_j] without renormalisation)."""
    picked = np.take_along_axis(s, topk_idx.astype(np.int64), axis=1)
    if not renorm:
        return picked
    return picked / picked.sum(axis=1, keepdims=True)


def near_ties(s: np.ndarray, k: int, margin: float = 1e-5) -> np.ndarray:
    """Token flag: some adjacent gap among its k+1 largest scores is below ``margin``.

    Such a token's selection may legitimately flip when logits are accumulated in a
    different order; its routing is reported apart from the exact comparison."""
    T, E = s.shape
    m = min(k + 1, E)
    top = -np.sort(-s, axis=1)[:, :m]
    if m < 2:
        return np.zeros(T, bool)
    return (np.abs(np.diff(top, axis=1)) < margin).any(axis=1)


def route(logits32: np.ndarray, k: int, score: str, renorm: bool = True, bias=None):
    """Logits (fp32) -> (topk_idx [T,k] int32, topk_w [T,k] fp64, near_tie [T] bool)."""
    l = add_bias(logits32, bias)
    idx = select_topk(l, k)
    s = scores(l, score)
    return idx, gate_weights(s, idx, renorm), near_ties(s, k)


# ----------------------------------------------------------------------------------------------
# histogram, permutation, compact miss list
# ----------------------------------------------------------------------------------------------


def histogram(topk_idx: np.ndarray, E: int) -> np.ndarray:
    """counts[e] = number of (token, choice) rows routed to expert e, absent experts included."""
    counts = np.zeros(E, np.int32)
    for e in np.asarray(topk_idx).reshape(-1):
        counts[e] += 1
    return counts


def row_slots(topk_idx: np.ndarray, slot_map) -> np.ndarray:
    """Slot of each flat row r = t*k + j: slot_map[e] (-1 = not resident), or e itself."""
    e = np.asarray(topk_idx, np.int64).reshape(-1)
    return e.astype(np.int32) if slot_map is None else np.asarray(slot_map, np.int32)[e]


def permute(topk_idx: np.ndarray, slot_map, S: int):
    """Group resident rows by slot, rows of one slot in ascending r.

    Returns slot_offsets [S+1] (slot s owns positions [off[s], off[s+1])), perm [n_res]
    (position -> flat row id) and inv_perm [T*k] (flat row id -> position, -1 for a miss)."""
    slot = row_slots(topk_idx, slot_map)
    R = slot.size
    perm = []
    offsets = [0]
    for s in range(S):
        perm.extend(np.nonzero(slot == s)[0].tolist())
        offsets.append(len(perm))
    perm = np.asarray(perm, np.int32)
    inv = np.full(R, -1, np.int32)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return np.asarray(offsets, np.int32), perm, inv


def miss_list(topk_idx: np.ndarray, topk_w: np.ndarray, slot_map):
    """Rows routed to experts without a resident slot, ascending r: (token, expert, weight).

    The weight is the full-k renormalised gate, so that adding w * FFN_e(x_t) for every listed
    row to the compact output restores the all-resident output."""
    k = topk_idx.shape[1]
    slot = row_slots(topk_idx, slot_map)
    r = np.nonzero(slot < 0)[0]
    return (r // k).astype(np.int32), np.asarray(topk_idx).reshape(-1)[r].astype(np.int32), \
        np.asarray(topk_w, np.float64).reshape(-1)[r]


# ----------------------------------------------------------------------------------------------
# expert FFN and combine
# ----------------------------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def slot_matrices(weights: dict, wdtype: str, s: int, H: int, I: int):
    """fp64 (W_gate [I,H], W_up [I,H], W_down [H,I]) of slot s, from its stored bytes."""
    sg = None if weights.get("s_gu") is None else weights["s_gu"][s]
    sd = None if weights.get("s_d") is None else weights["s_d"][s]
    gu = dequant(wdtype, weights["w_gu"][s], sg, 2 * I, H)
    wd = dequant(wdtype, weights["w_d"][s], sd, H, I)
    return gu[:I], gu[I:], wd


def ffn(x_rows: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, act_quant=None):
    """FFN_e on a batch of fp64 rows [n, H] -> [n, H].  ``act_quant`` (mode-B mirror only)
    is applied to the activations entering each projection pair."""
    xin = x_rows if act_quant is None else act_quant(x_rows)
    a = silu(xin @ wg.T) * (xin @ wu.T)
    ain = a if act_quant is None else act_quant(a)
    return ain @ wd.T


def expert_ffn(weights: dict, wdtype: str, x64: np.ndarray, perm: np.ndarray,
               slot_offsets: np.ndarray, k: int, H: int, I: int, positions=None, act_quant=None):
    """y_perm [n_res, H] fp64: y_perm[p] = FFN_{slot of p}(x[perm[p] // k]).

    ``positions`` (optional boolean mask over perm) restricts the work to some rows; the other
    rows are left as NaN."""
    n = perm.size
    y = np.full((n, H), np.nan)
    S = slot_offsets.size - 1
    for s in range(S):
        lo, hi = int(slot_offsets[s]), int(slot_offsets[s + 1])
        if hi == lo:
            continue
        pos = np.arange(lo, hi)
        if positions is not None:
            pos = pos[positions[lo:hi]]
            if pos.size == 0:
                continue
        wg, wu, wd = slot_matrices(weights, wdtype, s, H, I)
        y[pos] = ffn(x64[perm[pos] // k], wg, wu, wd, act_quant)
    return y


def combine(y_perm: np.ndarray, inv_perm: np.ndarray, topk_w: np.ndarray, T: int, k: int,
            H: int) -> np.ndarray:
    """out[t] = sum over j ascending of w[t,j] * y_perm[inv_perm[t*k+j]], resident rows only;
    a token with no resident row gets a zero row."""
    out = np.zeros((T, H))
    w = np.asarray(topk_w, np.float64).reshape(T, k)
    inv = np.asarray(inv_perm).reshape(T, k)
    for t in range(T):
        for j in range(k):
            p = inv[t, j]
            if p >= 0:
                out[t] += w[t, j] * y_perm[p]
    return out


def combine_tiers(y_a: np.ndarray, inv_a: np.ndarray, y_b: np.ndarray, inv_b: np.ndarray,
                  topk_w: np.ndarray, T: int, k: int, H: int) -> np.ndarray:
    """The combine over two tiers of computed rows (the compact call's resident slots and the
    other tier that computes the rows routed to absent experts -- README, MoET hybrid table,
    row "identity"): row (t, j) takes its output from tier a where it has a position there,
    else from tier b, else adds nothing; j ascending."""
    out = np.zeros((T, H))
    w = np.asarray(topk_w, np.float64).reshape(T, k)
    ia = np.asarray(inv_a).reshape(T, k)
    ib = np.asarray(inv_b).reshape(T, k)
    for t in range(T):
        for j in range(k):
            if ia[t, j] >= 0:
                out[t] += w[t, j] * y_a[ia[t, j]]
            elif ib[t, j] >= 0:
                out[t] += w[t, j] * y_b[ib[t, j]]
    return out


def plan_slots(hist: np.ndarray, S: int) -> np.ndarray:
    """Hot-set placement (the recipes wiki, Home page, expert balance: the experts with the
    largest routing share per byte of weights stay resident; equal sizes here, so the largest
    accumulated counts).  slot_map[e] = rank of e in (count descending, id ascending) when that
    rank is below S, else -1."""
    h = np.asarray(hist, np.int64)
    order = np.lexsort((np.arange(h.size), -h))
    sm = np.full(h.size, -1, np.int32)
    sm[order[:S]] = np.arange(S, dtype=np.int32)
    return sm


def lru_refill(counts, step: int, slot_map, slot_expert, last_use):
    """LRU refill after a call (the pages' full LRU: every resident slot is a spare held by the
    most recently used experts -- vLLM-Moet README, MoET hybrid measurement matrix, 4x RTX 5090
    row).  Slots whose expert took rows in the call are stamped with `step`; the experts that
    missed (rows > 0, no slot), most rows first (ties: smaller id), move into the slots not used
    in the call, least recently used first (ties: smaller slot).  Returns the new slot_map,
    slot_expert, last_use and the moves as (slot, expert) pairs."""
    counts = [int(c) for c in counts]
    sm = [int(v) for v in slot_map]
    se = [int(v) for v in slot_expert]
    lu = [int(v) for v in last_use]
    E, S = len(counts), len(se)
    used = [s for s in range(S) if se[s] >= 0 and counts[se[s]] > 0]
    free = sorted((s for s in range(S) if s not in used), key=lambda s: (lu[s], s))
    for s in used:
        lu[s] = step
    missed = sorted((e for e in range(E) if counts[e] > 0 and sm[e] < 0), key=lambda e: (-counts[e], e))
    moves = list(zip(free, missed))
    for s, e in moves:
        if se[s] >= 0:
            sm[se[s]] = -1
        sm[e] = s
        se[s] = e
        lu[s] = step
    return (np.array(sm, np.int32), np.array(se, np.int32), np.array(lu, np.int64), moves)


# ----------------------------------------------------------------------------------------------
# mode-B activation quantisation mirror (a defined step of the low-precision MFMA path)
# ----------------------------------------------------------------------------------------------


def e4m3fn_round(v: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn value (ties to even), saturating at +-448: fp64 in, fp64 out.

    Normal e4m3fn numbers with exponent e are spaced 2^(e-3); below 2^-6 the spacing is the
    subnormal one, 2^-9."""
    v = np.asarray(v, np.float64)
    mag = np.minimum(np.abs(v), 448.0)
    _, ex = np.frexp(mag)                      # mag = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    q = np.ldexp(1.0, e - 3)
    r = np.round(mag / q) * q                  # numpy rounds halves to even
    return np.sign(v) * np.minimum(r, 448.0)


def act_quant_mx_e4m3_parts(a: np.ndarray, block: int = 32):
    """The two parts of the OCP MX quantisation with E4M3 elements, per row and per ``block``
    consecutive elements: the shared scale exponent X and the element values q (e4m3fn values,
    fp64), so that the quantised activation is q * 2^X.

    X = floor(log2 amax) - 8 (8 is e4m3's largest exponent), kept inside the E8M0 scale range
    [-127, 127] (OCP MX v1.0: E8M0 encodes 2^-127 .. 2^127; finite amax keeps X <= 119, so only
    the lower end binds, for blocks with amax < 2^-118); an all-zero block has X = 0.  Each
    element is e4m3fn(v / 2^X), nearest even, saturated at +-448."""
    a = np.asarray(a, np.float64)
    n, K = a.shape
    assert K % block == 0
    b = a.reshape(n, K // block, block)
    amax = np.abs(b).max(axis=2)
    _, ex = np.frexp(amax)
    X = np.where(amax > 0, np.maximum(ex - 1 - 8, -127), 0)
    q = e4m3fn_round(np.ldexp(b, -X[:, :, None]))
    return X.astype(np.int64), q.reshape(n, K)


def act_quant_mx_e4m3(a: np.ndarray, block: int = 32) -> np.ndarray:
    """The quantised activation q * 2^X (fp64) of ``act_quant_mx_e4m3_parts``."""
    X, q = act_quant_mx_e4m3_parts(a, block)
    n, K = q.shape
    return np.ldexp(q.reshape(n, K // block, block), X[:, :, None]).reshape(n, K)


# ----------------------------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------------------------


def layer(x, xdtype: str, weights: dict, wdtype: str, H: int, I: int, E: int, k: int,
          score: str, renorm: bool = True, w_router=None, logits=None, bias=None,
          slot_map=None, S=None, tokens=None, act_quant=None):
    """Run every stage; returns a dict of all intermediate and final results.

    ``tokens`` (optional index array) limits the FFN and combine to those tokens, for
    full-size checks on a sample; routing and permutation are always computed in full."""
    x64 = activations_f64(x, xdtype)
    T = x64.shape[0]
    S = E if S is None else S
    l32 = router_logits(x64, w_router) if logits is None else np.asarray(logits, np.float32)
    idx, w, tie = route(l32, k, score, renorm, bias)
    counts = histogram(idx, E)
    off, perm, inv = permute(idx, slot_map, S)
    mt, me, mw = miss_list(idx, w, slot_map)
    mask = None
    if tokens is not None:
        want = np.zeros(T, bool)
        want[np.asarray(tokens)] = True
        mask = want[perm // k] if perm.size else np.zeros(0, bool)
    y = expert_ffn(weights, wdtype, x64, perm, off, k, H, I, positions=mask, act_quant=act_quant)
    if tokens is None:
        out = combine(y, inv, w, T, k, H)
    else:
        tk = np.asarray(tokens)
        sub_inv = inv.reshape(T, k)[tk].reshape(-1)
        out = combine(y, sub_inv, np.asarray(w).reshape(T, k)[tk], tk.size, k, H)
    return dict(logits=l32, topk_idx=idx, topk_w=w, near_tie=tie, counts=counts,
                slot_offsets=off, perm=perm, inv_perm=inv, miss_token=mt, miss_expert=me,
                miss_weight=mw, y_perm=y, out=out)
