"""Split-plan heuristic, step by step (oracle; test infrastructure).

The pages fix what a plan is but print no formula: a caller builds, on the
host and next to the decode CSR, a split count and a split_indptr per row
(ATOM pull request 2462, "Summary", part 1); a uniform plan depends only on
the row count and config, so graph capture and replay agree (same section);
the persistent kernel instead plans from the real per-row KV lengths on every
call (same page, "Summary", part 2). The constants, tie-breaks and the AUTO
rule below are this library's own choice (spec version 4); the library's C++
planner must produce the same int32 words.

Constants: M_UNIT 128 query rows per work item, N_MAX 256 splits per row,
MIN_SPLIT_KEYS 256, ITEM_OVERHEAD 256 (a work item's fixed cost, in keys),
OCC 1 resident work item per compute unit (a decode workgroup takes nearly
all of a CU's LDS), XCDS 8 (the chiplets whose L2 a launch spreads over).
All arithmetic is integer; cdiv(a, b) = (a + b - 1) // b.

Steps:
1. u = cdiv(H * q_len_max, M_UNIT): M tiles per split. A query row is
   (token i, head h) at index i * H + h of its request row.
2. Mode. AUTO builds the splits of both modes (steps 3 and 4) and estimates
   each plan's duration in keys, a split costing its keys plus ITEM_OVERHEAD:
   UNIFORM's is max(the costliest split, cdiv(u * the sum of split costs,
   OCC*C)), its one-item workgroups being dealt to the compute units as they
   free up; LENGTH_AWARE's is its fullest lane, T - the least room left
   (step 4). AUTO takes LENGTH_AWARE when its estimate is strictly smaller,
   else UNIFORM.
3. UNIFORM: n = clamp(min(cdiv(OCC*C, R*u), cdiv(max L, MIN_SPLIT_KEYS)), 1,
   N_MAX); every row gets n splits; split k of row b covers keys
   [k*L_b // n, (k+1)*L_b // n) (empty ranges are legal).
4. LENGTH_AWARE packs the rows' key ranges into lanes of equal capacity. A
   lane is u workgroups on one chiplet that run the same splits, one M tile
   each, so the u tiles of a split read its keys from one L2 at about the
   same time. X starts at XCDS and halves while (OCC*C) // X < u;
   n_x = (OCC*C) // X slots per chiplet; lam = max(1, n_x // u) lanes per
   chiplet; LAMBDA = X * lam lanes. Lane l (chiplet x = l mod X, k = l // X)
   has members j = 0..u-1, workgroup x + X*(k*u + j).
   Lane capacity T = max(MIN_SPLIT_KEYS + ITEM_OVERHEAD,
   cdiv(sum L + ITEM_OVERHEAD*(R + LAMBDA), LAMBDA),
   cdiv(max L, N_MAX - 1) + ITEM_OVERHEAD); every lane starts with room T.
   A split costs its keys plus ITEM_OVERHEAD. Rows are taken longest first
   (ties by row index); "the roomiest lane" is the lane with the most room,
   the lowest index among equals.
   - A row with L_b = 0 gets one empty split [0, 0) in the roomiest lane;
     its room is unchanged.
   - Otherwise, while keys s < L_b remain, with l the roomiest lane and
     r = room[l] - ITEM_OVERHEAD: if r >= L_b - s, or r < MIN_SPLIT_KEYS, or
     the row already has N_MAX - 1 splits, the split takes the rest
     (n = L_b - s); else it takes n = r. room[l] -= n + ITEM_OVERHEAD.
   So a row is cut only where a lane is full, a lane ends at most one row
   that continues elsewhere, and most rows stay whole.
   Split ids are then assigned in (row, first key) order, so each row's
   splits are consecutive; a lane's splits are listed in id order.
5. split_indptr is the running count of splits per row. Splits of rows with
   more than one split get partial-buffer slots 0, 1, 2, ... in split order;
   the others get -1.
6. UNIFORM: split cost = (end - begin) + ITEM_OVERHEAD. Splits are ranked by
   (-cost, split id). Rank k goes to chiplet k mod XCDS. Each chiplet's item
   list is its splits in rank order, each followed by its M tiles
   m = 0..u-1.
7. UNIFORM: one item per workgroup, G = W = S*u. Workgroup ids are dealt to
   chiplets round-robin (id mod XCDS), so for j < n_min (the shortest
   chiplet list) workgroup XCDS*j + x runs item j of chiplet x; the remaining
   items, taken by (j, x), fill the ids from XCDS*n_min upward in order.
8. LENGTH_AWARE: member j of lane l runs (s, j) for the lane's splits s in
   order. G = 1 + the largest workgroup id that has an item; the other
   workgroups below G have none.
9. Words (int32): a 20-word header [magic 0x4D4C4150, version 4, R, H,
   q_len_max, kv_dtype, C, mode_used (| 0x100 when the caller asked for the
   merge inside the decode kernel, | 0x200 when it asked for fp8 PV
   products), M_UNIT, u, N_MAX, MIN_SPLIT_KEYS,
   ITEM_OVERHEAD, OCC, S, W, G, P, 20, total words], then split_indptr[R+1],
   split_row[S], split_begin[S], split_end[S], split_part[S],
   work_indptr[G+1], item_split[W], item_m[W].
"""
import numpy as np

MAGIC = 0x4D4C4150
VERSION = 4
HEADER_WORDS = 20
M_UNIT = 128
N_MAX = 256
MIN_SPLIT_KEYS = 256
ITEM_OVERHEAD = 256
OCC = 1
XCDS = 8

MODE_AUTO, MODE_UNIFORM, MODE_LENGTH_AWARE = 0, 1, 2
# Bit 8 of the mode: the caller asks for the split merge inside the decode
# kernel. It is recorded in the header's mode word and changes nothing else.
MERGE_IN_KERNEL = 0x100
# Bit 9: the caller asks for the PV products in fp8 (fp8 KV only, not with
# MERGE_IN_KERNEL). Also recorded in the mode word and nothing else.
FP8_PV = 0x200
KV_BF16, KV_FP8 = 0, 1


def cdiv(a, b):
    return (a + b - 1) // b


def clamp(x, lo, hi):
    return max(lo, min(hi, x))


def uniform_splits(lens, u, C):
    """Step 3: (row, begin, end) of every split, in row order."""
    R = len(lens)
    n = clamp(min(cdiv(OCC * C, R * u), cdiv(max(lens), MIN_SPLIT_KEYS)), 1, N_MAX)
    return [(b, k * L // n, (k + 1) * L // n) for b, L in enumerate(lens) for k in range(n)]


def length_aware_splits(lens, u, C):
    """Step 4: the lanes' pieces. Returns (splits in (row, first key) order,
    each split's lane, X, the fullest lane's cost)."""
    R = len(lens)
    X = XCDS
    while X > 1 and (OCC * C) // X < u:
        X //= 2
    lam = max(1, ((OCC * C) // X) // u)
    n_lanes = X * lam
    T = max(MIN_SPLIT_KEYS + ITEM_OVERHEAD, cdiv(sum(lens) + ITEM_OVERHEAD * (R + n_lanes), n_lanes),
            cdiv(max(lens), N_MAX - 1) + ITEM_OVERHEAD)
    room = [T] * n_lanes
    pieces = []   # (row, begin, end, lane) in creation order

    def roomiest():
        best = 0
        for l in range(1, n_lanes):
            if room[l] > room[best]:
                best = l
        return best

    order = sorted(range(R), key=lambda b: (-lens[b], b))
    for b in order:
        L = lens[b]
        if L == 0:
            pieces.append((b, 0, 0, roomiest()))
            continue
        pos, count = 0, 0
        while pos < L:
            lane = roomiest()
            r = room[lane] - ITEM_OVERHEAD
            if r >= L - pos or r < MIN_SPLIT_KEYS or count == N_MAX - 1:
                take = L - pos
            else:
                take = r
            pieces.append((b, pos, pos + take, lane))
            room[lane] -= take + ITEM_OVERHEAD
            pos += take
            count += 1
    pieces.sort(key=lambda p: (p[0], p[1]))
    return [(b, lo, hi) for b, lo, hi, _ in pieces], [lane for *_, lane in pieces], X, n_lanes, T - min(room)


def uniform_estimate(splits, u, C):
    """Step 2: UNIFORM's duration estimate in keys."""
    cost = [hi - lo + ITEM_OVERHEAD for _, lo, hi in splits]
    return max(max(cost), cdiv(u * sum(cost), OCC * C))


def plan_ref(kv_lens, H, q_len_max, kv_dtype, mode, C):
    """Returns the plan as a numpy int32 array of words."""
    lens = [int(x) for x in kv_lens]
    R = len(lens)
    if R < 1 or not (1 <= H <= 128) or not (1 <= q_len_max <= 16) or C < 1:
        raise ValueError("unsupported plan arguments")
    if any(L < 0 for L in lens):
        raise ValueError("negative KV length")

    # 1-4
    u = cdiv(H * q_len_max, M_UNIT)
    flag = mode & (MERGE_IN_KERNEL | FP8_PV)
    mode_req = mode & ~(MERGE_IN_KERNEL | FP8_PV)
    if (flag & FP8_PV) and (kv_dtype != KV_FP8 or (flag & MERGE_IN_KERNEL)):
        raise ValueError("fp8 PV needs fp8 KV and a separate merge")
    if mode_req != MODE_LENGTH_AWARE:
        uni = uniform_splits(lens, u, C)
    if mode_req != MODE_UNIFORM:
        la, la_lane, X, n_lanes, la_est = length_aware_splits(lens, u, C)
    if mode_req == MODE_AUTO:
        mode_used = MODE_LENGTH_AWARE if la_est < uniform_estimate(uni, u, C) else MODE_UNIFORM
    else:
        mode_used = mode_req

    # 3-5: splits (row, key range), partial slots
    if mode_used == MODE_UNIFORM:
        splits = uni
    else:
        splits = la
        lane_splits = [[] for _ in range(n_lanes)]
        for s_id, lane in enumerate(la_lane):
            lane_splits[lane].append(s_id)
    split_row = [b for b, _, _ in splits]
    split_begin = [lo for _, lo, _ in splits]
    split_end = [hi for _, _, hi in splits]
    S = len(split_row)
    nsplit = [0] * R
    for b in split_row:
        nsplit[b] += 1
    split_indptr = [0]
    for nb in nsplit:
        split_indptr.append(split_indptr[-1] + nb)
    split_part = []
    next_slot = 0
    for s_id in range(S):
        if nsplit[split_row[s_id]] > 1:
            split_part.append(next_slot)
            next_slot += 1
        else:
            split_part.append(-1)
    P = next_slot
    W = S * u

    # 6-8: work items and workgroups
    if mode_used == MODE_UNIFORM:
        G = W
        X = XCDS
        cost = [split_end[s_id] - split_begin[s_id] + ITEM_OVERHEAD for s_id in range(S)]
        ranked = sorted(range(S), key=lambda s_id: (-cost[s_id], s_id))
        lists = [[] for _ in range(X)]
        for k, s_id in enumerate(ranked):
            for m in range(u):
                lists[k % X].append((s_id, m))
        order = [None] * W
        n_min = min(len(lst) for lst in lists)
        for x in range(X):
            for j in range(n_min):
                order[XCDS * j + x] = lists[x][j]
        nxt = XCDS * n_min
        tail_len = max(len(lst) for lst in lists)
        for j in range(n_min, tail_len):
            for x in range(X):
                if j < len(lists[x]):
                    order[nxt] = lists[x][j]
                    nxt += 1
        assert nxt == W
        groups = [[it] for it in order]
    else:
        by_wg = {}
        for lane, splits in enumerate(lane_splits):
            x, k = lane % X, lane // X
            for j in range(u):
                if splits:
                    by_wg[x + X * (k * u + j)] = [(s_id, j) for s_id in splits]
        G = 1 + max(by_wg)
        groups = [by_wg.get(g, []) for g in range(G)]

    work_indptr = [0]
    item_split, item_m = [], []
    for grp in groups:
        for (s, m) in grp:
            item_split.append(s)
            item_m.append(m)
        work_indptr.append(len(item_split))

    total = HEADER_WORDS + (R + 1) + 4 * S + (G + 1) + 2 * W
    header = [MAGIC, VERSION, R, H, q_len_max, kv_dtype, C, mode_used | flag, M_UNIT, u,
              N_MAX, MIN_SPLIT_KEYS, ITEM_OVERHEAD, OCC, S, W, G, P, HEADER_WORDS, total]
    words = (header + split_indptr + split_row + split_begin + split_end + split_part
             + work_indptr + item_split + item_m)
    assert len(words) == total
    return np.asarray(words, dtype=np.int64).astype(np.int32)


FIELDS = ["magic", "version", "R", "H", "q_len_max", "kv_dtype", "C", "mode", "M_UNIT", "u",
          "N_MAX", "MIN_SPLIT_KEYS", "ITEM_OVERHEAD", "OCC", "S", "W", "G", "P",
          "header_words", "total_words"]


def unpack_plan(words):
    """Split the words into a dict of named fields and arrays."""
    w = [int(x) for x in words]
    d = dict(zip(FIELDS, w[:HEADER_WORDS]))
    pos = HEADER_WORDS
    R, S, W, G = d["R"], d["S"], d["W"], d["G"]

    def take(n):
        nonlocal pos
        out = w[pos:pos + n]
        pos += n
        return out

    d["split_indptr"] = take(R + 1)
    d["split_row"] = take(S)
    d["split_begin"] = take(S)
    d["split_end"] = take(S)
    d["split_part"] = take(S)
    d["work_indptr"] = take(G + 1)
    d["item_split"] = take(W)
    d["item_m"] = take(W)
    assert pos == d["total_words"] == len(w)
    return d
