"""CPU oracle for the redundant-expert MoE dispatch path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke entry
and the benchmark's CPU-baseline leg may import this module.  The product
path (the HIP library and its Python binding) never imports, calls or
falls back to it, and this module imports nothing from the product path.

Plain, slow, obviously correct numpy code: integer work is exact, floating
point is done in float64 from exactly widened inputs and rounded once to
the output type.  Every function names the passage it follows.  Pages
cited (title, then the section or paragraph):

  [ainovat]  "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced Expert
             Parallelism Library for MoE Training" (ainovat.com)
  [repocard] "MoonEP" repository card (findrepo.work): "Why it is worth
             attention", "Strengths", "Considerations"
  [blog]     "MoonEP" walkthrough (moses-y.github.io): "The Problem",
             "What This Does", "How It Is Wired", "How To Use It",
             "Real-World Use"
  [wtf]      "wtf is moonep?" (gitwtfhub.com)

The pages fix the skew metric, the exact S*K-per-rank invariant, the
mechanism (a few redundant experts planned online from the router outputs,
weights prefetched, replica gradients returned home), and the contract (one
contiguous [E+B, H, H'] weight tensor per projection addressed by row index,
plus a planner-produced cu_seqlens).  They do not print the planning
algorithm, its tie-breaks, the token-to-replica assignment, the row order
in the buffer, the activation or the numerics.  Where they are silent this
module takes the plainest reading that meets what they do fix; each such
reading is marked READING.

Notation: R ranks, S tokens per rank, K routed experts per token, E experts,
E_loc = E / R home experts per rank, B replica slots per rank, SK = S*K.
A token copy is (p, s, k); its copy id is (p*S + s)*K + k.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits, f32_to_bf16_bits, bf16_bits_to_f32

STATUS_BAD_EXPERT_ID = 1
STATUS_SLOT_OVERFLOW = 2
HEADER_WORDS = 8


# --------------------------------------------------------------------------------------------
# Skew metric
# --------------------------------------------------------------------------------------------

def maxvio(T, R: int, S: int, K: int, E: int) -> float:
    """max_e T_e / T_bar - 1, with T_bar the per-expert count under perfect balance.

    [ainovat] paragraph defining maxvio.  READING: "tokens" are token-expert
    copies, so perfect balance puts T_bar = R*S*K / E copies on every expert.
    """
    T = np.asarray(T, dtype=np.float64)
    t_bar = R * S * K / E
    return float(T.max() / t_bar - 1.0)


# --------------------------------------------------------------------------------------------
# Planner
# --------------------------------------------------------------------------------------------

def histogram(topk_idx: np.ndarray, E: int):
    """C[p, e] = number of copies (p, s, k) routed to expert e.

    The per-expert token count T_e of [ainovat] (skew-metric paragraph) is
    the column sum of C.  READING: an id outside [0, E) is not counted and
    raises STATUS_BAD_EXPERT_ID; a repeated id within one token counts once
    per copy.
    """
    R = topk_idx.shape[0]
    flat = topk_idx.reshape(R, -1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    C = np.zeros((R, E), dtype=np.int64)
    for p in range(R):
        C[p] = np.bincount(flat[p][valid[p]], minlength=E)
    status = 0 if bool(valid.all()) else STATUS_BAD_EXPERT_ID
    return C, status


@dataclass
class Replica:
    expert: int     # expert e being duplicated
    rank: int       # receiving rank q (never home(e))
    start: int      # first position, in e's copy order, that this replica takes
    count: int      # number of copies it takes
    slot: int = -1  # slot j on rank q (weight row E + j); -1 if dropped for lack of slots


@dataclass
class Plan:
    R: int
    S: int
    K: int
    E: int
    B: int
    status: int
    counts: np.ndarray          # C [R, E]
    T: np.ndarray               # [E]
    keep: np.ndarray            # copies of e that stay on its home rank, [E]
    replicas: list              # Replica, in emission order
    n_donors: int
    n_receivers: int
    n_pieces: int
    max_needed: int             # most replicas any one rank was asked to host by the walk
    rep_first: np.ndarray = field(default=None)
    rep_n: np.ndarray = field(default=None)
    n_relayed: int = 0          # walk replicas placed by the relay fallback
    n_search: int = 0           # steps of the bounded search (0: not run)

    @property
    def E_loc(self):
        return self.E // self.R

    @property
    def SK(self):
        return self.S * self.K

    def home(self, e):
        return e // self.E_loc

    def slot_table(self):
        """(slot_expert, slot_start, slot_count), each [R, B]; empty slots are (-1, 0, 0)."""
        se = np.full((self.R, self.B), -1, np.int64)
        ss = np.zeros((self.R, self.B), np.int64)
        sc = np.zeros((self.R, self.B), np.int64)
        for m in self.replicas:
            if m.slot >= 0:
                se[m.rank, m.slot] = m.expert
                ss[m.rank, m.slot] = m.start
                sc[m.rank, m.slot] = m.count
        return se, ss, sc

    def rows_per_rank(self):
        """n[q, rho]: copies that rank q processes with weight row rho, rho in [0, E+B)."""
        R, E, B = self.R, self.E, self.B
        n = np.zeros((R, E + B), np.int64)
        for e in range(E):
            n[self.home(e), e] = self.keep[e]
        _, _, sc = self.slot_table()
        n[:, E:] = sc
        return n

    def cu_seqlens(self):
        """cu[q] = [0, n[q,0], n[q,0]+n[q,1], ...], E+B+1 entries per rank."""
        n = self.rows_per_rank()
        cu = np.zeros((self.R, self.E + self.B + 1), np.int64)
        cu[:, 1:] = np.cumsum(n, axis=1)
        return cu

    def to_blob(self) -> np.ndarray:
        """int32 words: header, T, keep, rep_first, rep_n, replica list, slot tables.

        header = [status, n_replicas, max_needed, n_donors, n_receivers,
        n_pieces, n_relayed, n_search]; the replica list holds E+R entries of each of
        (expert, rank, slot, start, count), unused entries (-1, -1, -1, 0, 0);
        the slot tables are [R*B] each of (expert, start, count).
        """
        R, E, B = self.R, self.E, self.B
        L = E + R
        re = np.full(L, -1, np.int64); rq = np.full(L, -1, np.int64)
        rs = np.full(L, -1, np.int64); rst = np.zeros(L, np.int64); rc = np.zeros(L, np.int64)
        for i, m in enumerate(self.replicas):
            re[i], rq[i], rs[i], rst[i], rc[i] = m.expert, m.rank, m.slot, m.start, m.count
        se, ss, sc = self.slot_table()
        hdr = np.array([self.status, len(self.replicas), self.max_needed, self.n_donors,
                        self.n_receivers, self.n_pieces, self.n_relayed, self.n_search], np.int64)
        blob = np.concatenate([hdr, self.T, self.keep, self.rep_first, self.rep_n,
                               re, rq, rs, rst, rc, se.ravel(), ss.ravel(), sc.ravel()])
        assert blob.size == plan_words(R, E, B)
        return blob.astype(np.int32)


def plan_words(R: int, E: int, B: int) -> int:
    return HEADER_WORDS + 4 * E + 5 * (E + R) + 3 * R * B


def plan(topk_idx: np.ndarray, E: int, B: int) -> Plan:
    """Online redundant-expert plan from the current router outputs.

    [ainovat] invariant and mechanism paragraphs: every rank must receive
    exactly S*K copies, whatever the skew, by duplicating a few experts onto
    other ranks, planned from this step's routing alone.  [repocard]
    "Strengths" asks for few replicas chosen near-optimally with negligible
    cost.  READING (the pages give no algorithm): a greedy donor-to-receiver
    placement that minimises the replica count in the common cases:

      1. histogram, T_e = sum_p C[p, e]
      2. home(e) = e // E_loc; rank load L_r = sum of T_e over its home
         experts; excess d_r = L_r - S*K
      3. donors (d_r > 0) ordered by (d_r desc, r asc); receivers (d_r < 0)
         by (-d_r desc, r asc)
      4. each donor, taking its home experts by (T_e desc, e asc), cuts one
         piece of a = min(T_e, remaining excess) from each until its excess
         is gone; keep_e = T_e - a
      5. the piece list and the receiver list are walked together; each step
         emits a replica of the current piece's expert on the current
         receiver carrying x = min(piece left, deficit left) copies, taken
         from e's copy order starting at keep_e + (part of the piece already
         emitted); whichever runs out advances
      6. replicas on a receiver take slots 0, 1, ... in emission order; when
         a receiver would need more than B slots the relay fallback
         (``relay_fallback``) re-places the walk's replicas; if it cannot
         place one, a bounded search (``relay_search``) looks for a plan
         with at most one replica per rank; if that fails too, the relay
         fallback's plan stands, its unplaced replicas dropped, and
         STATUS_SLOT_OVERFLOW is set
    """
    R, S, K = topk_idx.shape
    SK = S * K
    E_loc = E // R
    C, status = histogram(topk_idx, E)
    T = C.sum(axis=0)

    # step 2: home loads and excess
    L = np.array([int(T[r * E_loc:(r + 1) * E_loc].sum()) for r in range(R)], np.int64)
    d = L - SK

    # step 3: order donors and receivers
    donors = sorted([r for r in range(R) if d[r] > 0], key=lambda r: (-int(d[r]), r))
    receivers = sorted([r for r in range(R) if d[r] < 0], key=lambda r: (int(d[r]), r))

    # step 4: pieces
    keep = T.copy()
    pieces = []          # (expert, amount)
    for r in donors:
        experts = sorted(range(r * E_loc, (r + 1) * E_loc), key=lambda e: (-int(T[e]), e))
        rem = int(d[r])
        for e in experts:
            if rem == 0:
                break
            a = min(int(T[e]), rem)
            if a == 0:
                continue
            pieces.append((e, a))
            keep[e] -= a
            rem -= a

    # step 5: walk pieces against receivers
    replicas = []
    i = j = 0
    used_piece = used_recv = 0
    while i < len(pieces) and j < len(receivers):
        e, a = pieces[i]
        q = receivers[j]
        need = -int(d[q])
        x = min(a - used_piece, need - used_recv)
        replicas.append(Replica(expert=e, rank=q, start=int(keep[e]) + used_piece, count=x))
        used_piece += x
        used_recv += x
        if used_piece == a:
            i += 1
            used_piece = 0
        if used_recv == need:
            j += 1
            used_recv = 0

    # step 6: slots
    hosted = [0] * R
    for m in replicas:
        m.slot = hosted[m.rank] if hosted[m.rank] < B else -1
        hosted[m.rank] += 1
    max_needed = max(hosted) if R else 0
    n_relayed = n_search = 0
    if max_needed > B:
        replicas, keep, n_relayed, dropped = relay_fallback(replicas, keep, E_loc, R, B)
        if dropped and B >= 1:
            found, keep_s, n_search = relay_search(T, E_loc, R, SK)
            if found is not None:
                replicas = _gather_tile([Replica(expert=f, rank=q, start=0, count=x, slot=0)
                                         for f, q, x in found], keep_s)
                keep, dropped = keep_s, 0
        if dropped:
            status |= STATUS_SLOT_OVERFLOW

    rep_first = np.zeros(E, np.int64)
    rep_n = np.zeros(E, np.int64)
    for idx, m in enumerate(replicas):
        if rep_n[m.expert] == 0:
            rep_first[m.expert] = idx
        rep_n[m.expert] += 1

    return Plan(R=R, S=S, K=K, E=E, B=B, status=status, counts=C, T=T, keep=keep,
                replicas=replicas, n_donors=len(donors), n_receivers=len(receivers),
                n_pieces=len(pieces), max_needed=max_needed, rep_first=rep_first, rep_n=rep_n,
                n_relayed=n_relayed, n_search=n_search)


def relay_fallback(walk, keep, E_loc: int, R: int, B: int):
    """Re-place the walk's replicas when a receiver would need more than B slots.

    [ainovat] invariant paragraph: every rank gets exactly S*K copies
    whatever the skew; the donor-to-receiver walk alone cannot always keep
    within B slots per rank.  READING (the pages give no algorithm; a
    one-hop relay through a donor):

    The walk's replicas (expert f, receiver q, x copies) are taken again in
    emission order.  "Place n copies of e on rank a" means: add them to
    keep_e if a is e's home; else add them to the replica of e that a
    already hosts; else open a replica of e on a in a's next free slot;
    else it fails.  For each walk replica:
      1. place the x copies of f on q directly;
      2. otherwise (q is full) relay through q: for q's replicas (e, c) in
         slot order, the first with keep_e >= x whose home A can take x
         copies of f: q's replica of e grows by x (taken from keep_e), and A
         takes the x copies of f instead of q;
      3. otherwise switch: for q's replicas (e, c) in slot order, the first
         with keep_f >= c whose home-of-f F can take c copies of e: that
         replica becomes a replica of f with c + x copies (c of them taken
         from keep_f), and F takes the c copies of e;
      4. otherwise the replica is dropped (slot -1, its copies get no
         destination).
    Every step keeps each rank's load and each expert's total, so a plan
    with nothing dropped gives every rank exactly S*K copies.  Relays land
    only on donors (homes of pieced experts).  Each walk replica gives at
    most one new entry, so the list never outgrows the walk's.

    Afterwards the entries of each expert are gathered together (experts in
    the order of their first entry, entries of one expert in pass order),
    and an expert's copies are tiled home first, then its entries in that
    order: start = keep_e + the counts of its earlier entries.  When
    nothing overflows the walk's list is returned unchanged.
    Returns (replicas, keep, number of relayed or switched replicas,
    number dropped).
    """
    keep = keep.copy()
    out = []                               # entries in pass order
    on_rank = [[] for _ in range(R)]       # indices into out, in slot order

    def home(e):
        return e // E_loc

    def entry_of(a, e):
        for i in on_rank[a]:
            if out[i].expert == e:
                return i
        return -1

    def can_place(e, a):
        return a == home(e) or entry_of(a, e) >= 0 or len(on_rank[a]) < B

    def place(e, a, n):
        if a == home(e):
            keep[e] += n
            return
        i = entry_of(a, e)
        if i >= 0:
            out[i].count += n
            return
        assert len(on_rank[a]) < B
        out.append(Replica(expert=e, rank=a, start=0, count=n, slot=len(on_rank[a])))
        on_rank[a].append(len(out) - 1)

    relayed = dropped = 0
    for m in walk:
        f, q, x = m.expert, m.rank, m.count
        if can_place(f, q):                                       # 1
            place(f, q, x)
            continue
        done = False
        for i in list(on_rank[q]):                                # 2
            e = out[i].expert
            if keep[e] >= x and can_place(f, home(e)):
                out[i].count += x
                keep[e] -= x
                place(f, home(e), x)
                done = True
                break
        if not done:
            for i in list(on_rank[q]):                            # 3
                e, c = out[i].expert, out[i].count
                if keep[f] >= c and can_place(e, home(f)):
                    out[i].expert = f
                    out[i].count = c + x
                    keep[f] -= c
                    place(e, home(f), c)
                    done = True
                    break
        if done:
            relayed += 1
        else:                                                     # 4
            out.append(Replica(expert=f, rank=q, start=0, count=x, slot=-1))
            dropped += 1

    return _gather_tile(out, keep), keep, relayed, dropped


def _gather_tile(entries, keep):
    """Gather each expert's entries together (experts in the order of their
    first entry, an expert's entries in list order), then tile the expert's
    copies home first: an entry starts at keep_e + the counts of the
    expert's earlier entries."""
    first = {}
    for i, r in enumerate(entries):
        first.setdefault(r.expert, i)
    order = sorted(range(len(entries)), key=lambda i: (first[entries[i].expert], i))
    grouped = [entries[i] for i in order]
    pos = {}
    for r in grouped:
        r.start = int(keep[r.expert]) + pos.get(r.expert, 0)
        pos[r.expert] = pos.get(r.expert, 0) + r.count
    return grouped


SEARCH_BUDGET = 512


def relay_search(T, E_loc: int, R: int, SK: int, budget: int = SEARCH_BUDGET):
    """Bounded search for a plan with at most one replica per rank, run when
    the relay fallback leaves a replica unplaced.

    [ainovat] invariant paragraph: every rank gets exactly S*K copies
    whatever the skew.  READING (the pages give no algorithm).  With one
    replica per rank a rank takes all the copies it lacks from a single
    expert of another rank, and that rank may in turn send out more than its
    own excess and make up the difference the same way (the moves the
    one-hop fallback cannot express).  The search builds such a plan in
    generations:

      generation 0: the receivers (d_r < 0), each needing -d_r copies;
      each rank of a generation, taken by (need desc, r asc), takes its whole
      need from one expert f whose home g has not taken copies (and is not in
      this generation) and has cap_f >= need left, where cap starts at T;
      experts are tried in a fixed order (homes by (d desc, r asc), a home's
      experts by (T desc, e asc)), first those whose home still has that much
      excess left (d_g - out_g >= need), then the others, so that a home
      overshoots only when nothing fits;
      when a generation is placed, every rank that has not taken copies and
      has sent out more than its excess (out_r > d_r) forms the next
      generation, needing out_r - d_r; when none is left the plan is
      complete if every such rank sent out exactly its excess.

    Depth first, undoing a choice when what follows fails; at most `budget`
    placements are tried (the search then gives up).  Each rank takes copies
    at most once, so each hosts at most one replica, and a complete plan
    keeps every rank at exactly SK copies.
    Returns (entries [(expert, rank, count)] in placement order, keep = cap,
    placements tried) or (None, None, placements tried).
    """
    E = R * E_loc
    T = [int(t) for t in T]
    d = [sum(T[r * E_loc:(r + 1) * E_loc]) - SK for r in range(R)]
    homes = sorted(range(R), key=lambda r: (-d[r], r))
    cand = [e for r in homes
            for e in sorted(range(r * E_loc, (r + 1) * E_loc), key=lambda e: (-T[e], e))]
    cap = list(T)
    out = [0] * R
    got = [False] * R
    entries = []
    steps = 0

    def place(pend, i):
        # True: complete; False: no plan below this point; None: budget spent
        nonlocal steps
        if i == len(pend):
            nxt = sorted(((r, out[r] - d[r]) for r in range(R) if not got[r] and out[r] > d[r]),
                         key=lambda t: (-t[1], t[0]))
            if not nxt:
                return all(got[r] or out[r] == d[r] for r in range(R))
            for r, _ in nxt:
                got[r] = True
            res = place(nxt, 0)
            if not res:
                for r, _ in nxt:
                    got[r] = False
            return res
        n, need = pend[i]
        for fitting in (True, False):
            for f in cand:
                g = f // E_loc
                if got[g] or cap[f] < need or (d[g] - out[g] >= need) != fitting:
                    continue
                if steps == budget:
                    return None
                steps += 1
                cap[f] -= need
                out[g] += need
                entries.append((f, n, need))
                res = place(pend, i + 1)
                if res:
                    return True
                cap[f] += need
                out[g] -= need
                entries.pop()
                if res is None:
                    return None
        return False

    pend = sorted(((r, -d[r]) for r in range(R) if d[r] < 0), key=lambda t: (-t[1], t[0]))
    for r, _ in pend:
        got[r] = True
    if place(pend, 0):
        return entries, np.array(cap, np.int64), steps
    return None, None, steps


# --------------------------------------------------------------------------------------------
# Dispatch layout
# --------------------------------------------------------------------------------------------

def layout(topk_idx: np.ndarray, pl: Plan, rank: int):
    """cu_seqlens of ``rank``, the global destination of every copy, and ``rank``'s receive map.

    [ainovat] contract paragraph: dispatch returns cu_seqlens over the E+B
    weight rows and those counts select the active rows.  [blog] "What This
    Does": tokens land directly in their final expert-grouped positions.
    READING:
      * rank q's buffer holds S*K rows grouped by weight row rho = 0..E+B-1
        in ascending rho (home experts at their global id, slot j at E+j);
        cu_seqlens has E+B+1 entries with a leading 0;
      * inside expert e, copies are taken in copy-id order; the first keep_e
        stay home, replica m takes positions [start_m, start_m + count_m);
        each segment keeps that order;
      * dest_pos[c] = q*S*K + row position on q, or -1 when the copy has no
        destination (bad id, or its replica was dropped);
      * src_flat[i] = copy id landing at row i of ``rank``, or -1 if none.
    A stable sort by expert id groups the copies of each expert in copy-id
    order (library sort used as one step).
    """
    R, S, K = topk_idx.shape
    SK = S * K
    E, B = pl.E, pl.B
    E_loc = E // R
    flat = topk_idx.reshape(-1).astype(np.int64)
    key = np.where((flat >= 0) & (flat < E), flat, E)
    order = np.argsort(key, kind="stable")
    first = np.concatenate([[0], np.cumsum(np.bincount(key, minlength=E + 1))])
    cu = pl.cu_seqlens()
    dest = np.full(R * SK, -1, np.int64)
    for e in range(E):
        group = order[first[e]:first[e + 1]]
        h = e // E_loc
        k_e = int(pl.keep[e])
        dest[group[:k_e]] = h * SK + cu[h, e] + np.arange(k_e)
        for m in pl.replicas:
            if m.expert != e or m.slot < 0:
                continue
            dest[group[m.start:m.start + m.count]] = (m.rank * SK + cu[m.rank, E + m.slot]
                                                      + np.arange(m.count))
    src = np.full(SK, -1, np.int64)
    mine = np.nonzero((dest >= rank * SK) & (dest < (rank + 1) * SK))[0]
    src[dest[mine] - rank * SK] = mine
    return cu[rank].astype(np.int32), dest.astype(np.int32), src.astype(np.int32)


def layout_loops(topk_idx: np.ndarray, pl: Plan, rank: int):
    """Per-copy pure-Python version of ``layout`` (same reading), for small inputs.

    Walks the copies in copy-id order with one running counter per expert,
    so it needs no sort; used to cross-check the vectorised version.
    """
    R, S, K = topk_idx.shape
    SK = S * K
    E = pl.E
    E_loc = E // R
    cu = pl.cu_seqlens()
    seen = [0] * E
    dest = [-1] * (R * SK)
    flat = topk_idx.reshape(-1).tolist()
    for c, e in enumerate(flat):
        if not (0 <= e < E):
            continue
        g = seen[e]
        seen[e] += 1
        if g < pl.keep[e]:
            h = e // E_loc
            dest[c] = h * SK + int(cu[h, e]) + g
            continue
        for m in pl.replicas:
            if m.expert == e and m.start <= g < m.start + m.count:
                if m.slot >= 0:
                    dest[c] = m.rank * SK + int(cu[m.rank, E + m.slot]) + (g - m.start)
                break
    src = [-1] * SK
    for c, dpos in enumerate(dest):
        if rank * SK <= dpos < (rank + 1) * SK:
            src[dpos - rank * SK] = c
    return (cu[rank].astype(np.int32), np.array(dest, np.int32), np.array(src, np.int32))


# --------------------------------------------------------------------------------------------
# Permute, grouped GEMM, combine, fold
# --------------------------------------------------------------------------------------------

def permute(x_all: np.ndarray, src_flat: np.ndarray, K: int, row_scale=None, dtype="bf16"):
    """xp[i] = x_all[src_flat[i] // K]: a row gather into expert-grouped order.

    [blog] "What This Does" and [repocard] "Strengths" (the permute is fused
    into dispatch, no extra copy).  Without ``row_scale`` it is a bitwise
    copy; rows with src_flat < 0 are zero.  With ``row_scale`` (indexed by
    copy id) it is the backward of the weighted combine: READING, one IEEE
    fp32 multiply w * x then one rounding to the row type.
    ``x_all`` is uint16 bf16 bits or float32.
    """
    SK = src_flat.shape[0]
    out = np.zeros((SK, x_all.shape[1]), dtype=x_all.dtype)
    for i in range(SK):
        c = int(src_flat[i])
        if c < 0:
            continue
        row = x_all[c // K]
        if row_scale is None:
            out[i] = row
        else:
            w = np.float32(row_scale[c])
            if dtype == "bf16":
                out[i] = f32_to_bf16_bits(w * bf16_bits_to_f32(row))
            else:
                out[i] = w * row.astype(np.float32)
    return out


def _widen(a, dtype):
    return bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, np.float64)


def _narrow(a64, dtype):
    return f64_to_bf16_bits(a64) if dtype == "bf16" else a64.astype(np.float32)


def group_gemm(op: str, a, b, cu, dtype="bf16", out=None):
    """Grouped GEMM over one contiguous weight tensor addressed by row index.

    [ainovat] contract and contiguity paragraphs: segment rho of the rows
    (cu[rho] .. cu[rho+1]) is multiplied by weight row rho of a single
    [E+B, H, H'] tensor; rows with an empty segment are not touched.
    Float64 products from exactly widened inputs, rounded once.

      "fwd":   out[seg] = a[seg] @ W[rho]          a [M, Kd], W [G, Kd, N] -> [M, N]
      "dgrad": out[seg] = a[seg] @ W[rho]^T        a [M, N],  W [G, Kd, N] -> [M, Kd]
      "wgrad": out[rho] += a[seg]^T @ b[seg]       a [M, Kd], b [M, N]     -> fp32 [G, Kd, N]

    READING: output rows outside every segment keep the value of ``out``
    (zeros if not given); wgrad accumulates into fp32 ``out``, one rounding
    per call.
    """
    cu = np.asarray(cu, np.int64)
    G = cu.shape[0] - 1
    if op == "wgrad":
        res = np.array(out, dtype=np.float32, copy=True)
        for rho in range(G):
            lo, hi = int(cu[rho]), int(cu[rho + 1])
            if hi <= lo:
                continue
            acc = _widen(a[lo:hi], dtype).T @ _widen(b[lo:hi], dtype)
            res[rho] = (res[rho].astype(np.float64) + acc).astype(np.float32)
        return res
    M = a.shape[0]
    ncols = b.shape[2] if op == "fwd" else b.shape[1]
    odt = np.uint16 if dtype == "bf16" else np.float32
    res = np.zeros((M, ncols), odt) if out is None else np.array(out, dtype=odt, copy=True)
    for rho in range(G):
        lo, hi = int(cu[rho]), int(cu[rho + 1])
        if hi <= lo:
            continue
        w = _widen(b[rho], dtype)
        prod = _widen(a[lo:hi], dtype) @ (w if op == "fwd" else w.T)
        res[lo:hi] = _narrow(prod, dtype)
    return res


def silu(x64):
    """x * sigma(x), sigma(x) = 1 / (1 + exp(-x)), in float64 (the SiLU / swish-1 function)."""
    x64 = np.asarray(x64, np.float64)
    with np.errstate(over="ignore"):
        return x64 / (1.0 + np.exp(-x64))


def group_gemm_swiglu(a, b, cu, dtype="bf16"):
    """Gated (SwiGLU) up-projection over the grouped weight tensor.

    The pages name no activation; a gated unit is the usual framework
    variant.  READING: W[rho] has 2N' columns interleaved as (gate, up)
    pairs; h = a[seg] @ W[rho] in float64 from exactly widened inputs;
    z[:, j] = silu(h[:, 2j]) * h[:, 2j+1], both z and the pre-activation h
    rounded once to the row type.  Returns (z [M, N'], h [M, 2N']); rows
    outside every segment are zero.
    """
    cu = np.asarray(cu, np.int64)
    G, M, N2 = cu.shape[0] - 1, a.shape[0], b.shape[2]
    odt = np.uint16 if dtype == "bf16" else np.float32
    z = np.zeros((M, N2 // 2), odt)
    h = np.zeros((M, N2), odt)
    for rho in range(G):
        lo, hi = int(cu[rho]), int(cu[rho + 1])
        if hi <= lo:
            continue
        h64 = _widen(a[lo:hi], dtype) @ _widen(b[rho], dtype)
        z[lo:hi] = _narrow(silu(h64[:, 0::2]) * h64[:, 1::2], dtype)
        h[lo:hi] = _narrow(h64, dtype)
    return z, h


def swiglu_backward(dz, h, dtype="bf16"):
    """Gradient of the gated unit with respect to its pre-activation h (interleaved pairs).

    READING: from the stored (rounded) pre-activation g = h[:, 2j],
    u = h[:, 2j+1] and the output gradient dz[:, j], in float64:
    dh[:, 2j] = dz * u * silu'(g), dh[:, 2j+1] = dz * silu(g), with
    silu'(x) = sigma(x) * (1 + x * (1 - sigma(x))); one rounding.
    """
    hh = _widen(h, dtype)
    g, u = hh[:, 0::2], hh[:, 1::2]
    d = _widen(dz, dtype)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-g))
    out = np.empty(hh.shape, np.float64)
    out[:, 0::2] = d * u * sg * (1.0 + g * (1.0 - sg))
    out[:, 1::2] = d * g * sg
    return _narrow(out, dtype)


def group_gemm_rows(op: str, a, b, cu, rows, dtype="bf16"):
    """Selected output rows of ``group_gemm`` ("fwd"/"dgrad"), computed one row at a time.

    For large shapes: each row needs only its own input row and its
    segment's weight row.  Returns (segment of each row, output rows).
    """
    cu = np.asarray(cu, np.int64)
    rows = np.asarray(rows, np.int64)
    seg = np.searchsorted(cu, rows, side="right") - 1
    outs = []
    for r, rho in zip(rows, seg):
        w = _widen(b[rho], dtype)
        x = _widen(a[r:r + 1], dtype)
        outs.append(_narrow(x @ (w if op == "fwd" else w.T), dtype)[0])
    return seg, np.stack(outs) if outs else np.zeros((0,), np.float32)


def wgrad_entries(a, b, cu, rho: int, ii, jj, dtype="bf16", init=None):
    """Selected entries (ii, jj) of a[seg]^T @ b[seg] (+ init) for one weight row rho, fp32."""
    lo, hi = int(cu[rho]), int(cu[rho + 1])
    A = _widen(a[lo:hi][:, ii], dtype)          # [n, len]
    Bm = _widen(b[lo:hi][:, jj], dtype)
    acc = (A * Bm).sum(axis=0)
    if init is not None:
        acc = acc + np.asarray(init, np.float64)
    return acc.astype(np.float32)


def combine(y_all, dest_pos, topk_w, rank: int, S: int, K: int, dtype="bf16", tokens=None):
    """out[s] = sum over k of w[rank, s, k] * y_all[dest_pos of copy (rank, s, k)].

    [blog] "What This Does" / "Real-World Use": combine gathers each token's
    expert outputs back from their expert-grouped positions.  READING: pull
    form, weights are the router's top-K weights, sum in ascending k
    (float64 here), one rounding; copies with dest_pos < 0 add nothing.
    ``tokens`` restricts the computation to those token indices.
    """
    toks = np.arange(S) if tokens is None else np.asarray(tokens, np.int64)
    width = y_all.shape[1]
    acc = np.zeros((toks.size, width), np.float64)
    w = np.asarray(topk_w, np.float32).reshape(-1)
    dp = np.asarray(dest_pos).reshape(-1)
    for t, s in enumerate(toks):
        for k in range(K):
            c = (rank * S + int(s)) * K + k
            d = int(dp[c])
            if d < 0:
                continue
            acc[t] += np.float64(w[c]) * _widen(y_all[d], dtype)
    return _narrow(acc, dtype)


def unpermute_reduce(dxp_all, dest_pos, rank: int, S: int, K: int, dtype="bf16", tokens=None):
    """dx[s] = sum over k of dxp_all[dest_pos of copy (rank, s, k)]: the dispatch's backward.

    [blog] "What This Does" (dispatch places each token's K copies at their
    expert-grouped rows) and "Real-World Use" (the per-layer training loop
    runs backward through the same path).  READING: the dispatch copies a
    token row unchanged to K rows, so the gradient of the token row is the
    plain sum of the K rows' gradients, pulled back through dest_pos the way
    the combine pulls outputs; ascending k in float64, one rounding; copies
    with dest_pos < 0 add nothing.  ``dxp_all`` holds rank q's rows at
    q*S*K ..; ``tokens`` restricts the computation to those token indices.
    """
    toks = np.arange(S) if tokens is None else np.asarray(tokens, np.int64)
    acc = np.zeros((toks.size, dxp_all.shape[1]), np.float64)
    dp = np.asarray(dest_pos).reshape(-1)
    for t, s in enumerate(toks):
        for k in range(K):
            d = int(dp[(rank * S + int(s)) * K + k])
            if d >= 0:
                acc[t] += _widen(dxp_all[d], dtype)
    return _narrow(acc, dtype)


def combine_weight_grad(y_all, dest_pos, dout, rank: int, S: int, K: int, dtype="bf16",
                        tokens=None):
    """dw[s*K + k] = <dout[s], y_all[dest_pos of copy (rank, s, k)]>: the router-weight gradient.

    [blog] "Real-World Use" (backward of the combine that gathers the expert
    outputs).  READING: the combine is linear in each router weight, so the
    weight's gradient is the dot product of the token's output gradient with
    the expert output it scaled; float64 dot product rounded once to float32;
    0 for copies with dest_pos < 0.  ``dout`` holds rank ``rank``'s S token
    rows; the result is [len(tokens), K] (all S tokens by default).
    """
    toks = np.arange(S) if tokens is None else np.asarray(tokens, np.int64)
    out = np.zeros((toks.size, K), np.float64)
    dp = np.asarray(dest_pos).reshape(-1)
    for t, s in enumerate(toks):
        g = _widen(dout[int(s)], dtype)
        for k in range(K):
            d = int(dp[(rank * S + int(s)) * K + k])
            if d >= 0:
                out[t, k] = float(np.dot(g, _widen(y_all[d], dtype)))
    return out.astype(np.float32)


def replica_grad_fold(dw: np.ndarray, pl: Plan, rank: int) -> np.ndarray:
    """Fold replica weight-gradient rows of ``rank`` into their home expert rows.

    [ainovat] mechanism paragraph and [blog] "Real-World Use": in backward,
    the gradients of duplicated experts go back to their home experts.
    READING (one GPU holds the whole [E+B, ...] tensor): for each used slot j
    of ``rank`` in ascending j, dw[e] = fp32(dw[e] + dw[E+j]) and then
    dw[E+j] = 0, so the slot starts the next step clean.
    """
    out = np.array(dw, dtype=np.float32, copy=True)
    se, _, _ = pl.slot_table()
    for j in range(pl.B):
        e = int(se[rank, j])
        if e < 0:
            continue
        out[e] = out[e] + out[pl.E + j]
        out[pl.E + j] = 0.0
    return out


def prefetch(w: np.ndarray, pl: Plan, rank: int) -> np.ndarray:
    """Slot rows of ``rank`` receive a copy of the expert they duplicate.

    [ainovat] mechanism paragraph: duplicated experts' weights are fetched
    before expert compute.  Empty slots are left as they were.
    """
    out = np.array(w, copy=True)
    se, _, _ = pl.slot_table()
    for j in range(pl.B):
        e = int(se[rank, j])
        if e >= 0:
            out[pl.E + j] = out[e]
    return out
