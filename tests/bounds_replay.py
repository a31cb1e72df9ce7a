"""Host replay of the global-memory index arithmetic of the selection,
compaction, decoding and AnchorKV kernels.

Each function below re-states, for every workgroup and thread of a launch,
the address expressions of one kernel of the HIP library (the kernel named
in its docstring) and returns the element indices it would read or write in
each global buffer. The integer buffers the kernels read and trust (index
lists, head offsets, budget vectors, the many-workgroup select's per-segment
state and per-chunk counts) are inputs here, so a test can feed arbitrary
values, including values no correct earlier kernel would leave, and check
that every access stays inside the buffer the library was given.

Floating-point data never decides an address in these kernels, so only the
integer inputs are replayed; a membership test on a key is replaced by an
arbitrary choice where its outcome feeds an index (every outcome is then
covered). Indices are Python/numpy integers computed with the kernels'
widths: uint32 arithmetic wraps modulo 2^32 where the kernel's does.
"""
from __future__ import annotations

import numpy as np

U32 = 1 << 32


def _u32(x):
    return np.asarray(x, np.int64) % U32


class Accesses:
    """Per buffer: the list of index arrays touched (reads and writes)."""

    def __init__(self):
        self.by_buffer: dict[str, list[np.ndarray]] = {}

    def add(self, name, idx):
        a = np.asarray(idx, np.int64).ravel()
        if a.size:
            self.by_buffer.setdefault(name, []).append(a)

    def extent(self, name):
        parts = self.by_buffer.get(name)
        if not parts:
            return None
        a = np.concatenate(parts)
        return int(a.min()), int(a.max())

    def check(self, sizes: dict):
        """Asserts every touched index lies in [0, sizes[name])."""
        for name, parts in self.by_buffer.items():
            lo, hi = self.extent(name)
            assert name in sizes, f"untracked buffer {name}"
            assert lo >= 0 and hi < sizes[name], \
                f"{name}: touched [{lo}, {hi}] outside [0, {sizes[name]})"


# ------------------------------------------------------------- k_compact ----

K_ITEMS, K_COMPACT_THREADS = 4, 256


def _search_last_le(table, base, count, value, acc, name):
    """Binary search of the kernels' 'last h in [0, count-1] with
    table[base + h] <= value' (vectorised over value); records the reads."""
    lo = np.zeros(value.shape, np.int64)
    hi = np.full(value.shape, count - 1, np.int64)
    while True:
        act = lo < hi
        if not act.any():
            return lo
        mid = (lo + hi + 1) >> 1
        acc.add(name, base + mid[act])
        cond = np.zeros(value.shape, bool)
        cond[act] = table[base + mid[act]] <= value[act]
        lo = np.where(act & cond, mid, lo)
        hi = np.where(act & ~cond, mid - 1, hi)


def compact_accesses(L, H, n, vecs, kept, idx, offs):
    """k_compact (compact.hip): grid (ceil(kept*vecs / 1024), L), block 256,
    4 items a thread a block-width apart. idx: int32 [L*kept] (arbitrary),
    offs: int32 [L*(H+1)] (arbitrary) or None (uniform: kept % H == 0, as
    the library requires)."""
    acc = Accesses()
    total = kept * vecs
    per_block = K_ITEMS * K_COMPACT_THREADS
    blocks = -(-total // per_block)
    per_head = 0 if offs is not None else kept // H
    base_all = (np.arange(blocks, dtype=np.int64)[:, None] * per_block
                + np.arange(K_COMPACT_THREADS, dtype=np.int64)[None, :]).ravel()
    for l in range(L):
        lim = total
        if offs is not None:
            acc.add("offs", [l * (H + 1) + H])
            e = int(offs[l * (H + 1) + H])
            lim = min(max(e, 0), kept) * vecs
        base = base_all[base_all < lim]            # the others return at once
        for j in range(K_ITEMS):
            item = base + j * K_COMPACT_THREADS
            row = item // vecs
            c = item - row * vecs
            ok = item < lim
            acc.add("idx", l * kept + row[ok])
            pos = np.full(item.shape, -1, np.int64)
            pos[ok] = idx[l * kept + row[ok]]
            if offs is not None:
                h = _search_last_le(offs, l * (H + 1), H, row, acc, "offs")
            else:
                h = row // per_head
            load = (pos >= 0) & (pos < n)
            acc.add("kv", ((l * H + h[load]) * n + pos[load]) * vecs + c[load])
            acc.add("out", l * total + item[ok])
    return acc


def compact_sizes(L, H, n, vecs, kept, offs):
    s = {"idx": L * kept, "kv": L * H * n * vecs, "out": L * kept * vecs}
    if offs is not None:
        s["offs"] = L * (H + 1)
    return s


# -------------------------------------------------------------- k_decode ----

DEC_REC, HEAD_DIM = 128 + 2, 128


def dec_chunk(G):
    """dec_chunk: rows per work item (k_decode_stream for G <= 4, else
    k_decode_phased)."""
    return 512 if G <= 4 else 256


def decode_items(H, kept, ragged, chunk):
    if ragged:
        return -(-kept // chunk) + H
    b = kept // H
    return H * (-(-b // chunk))


def _dec_prefix(offs, l, H, kept, acc, DEC_CHUNK):
    """dec_prefix: effective offsets (clamped into [0, kept], then the
    running maximum) and the per-head work-item prefix."""
    h = np.arange(H + 1, dtype=np.int64)
    if offs is not None:
        acc.add("offs", l * (H + 1) + h)
        x = np.clip(offs[l * (H + 1) + h].astype(np.int64), 0, kept)
    else:
        x = h * (kept // H)
    eo = np.maximum.accumulate(x)
    lens = eo[1:] - eo[:-1]
    cnt = (lens + DEC_CHUNK - 1) // DEC_CHUNK
    pre = np.concatenate([[0], np.cumsum(cnt)])
    return eo, pre


def decode_accesses(L, H, G, kept, offs):
    """k_decode_stream / k_decode_phased (one item of <= dec_chunk(G) kept
    rows of one head per workgroup; every row of the item is read, rows past
    its end clamped to its last) and k_decode_merge (one query head per
    workgroup), decode.hip. offs: int32 [L*(H+1)] (arbitrary) or None
    (uniform, kept % H == 0)."""
    acc = Accesses()
    ragged = offs is not None
    DEC_CHUNK = dec_chunk(G)
    items = decode_items(H, kept, ragged, DEC_CHUNK)
    rec = G * DEC_REC
    for l in range(L):
        eo, pre = _dec_prefix(offs, l, H, kept, acc, DEC_CHUNK)
        its = np.arange(items, dtype=np.int64)
        its = its[its < pre[H]]                    # the others return at once
        if its.size:
            h = _search_last_le(pre, 0, H, its, Accesses(), "lds")
            r0 = eo[h] + (its - pre[h]) * DEC_CHUNK
            r1 = np.minimum(eo[h] + (eo[h + 1] - eo[h]), r0 + DEC_CHUNK)
            assert (r0 < r1).all(), "an item with no rows would clamp its row to r1 - 1 < r0"
            rows = np.minimum(r0[:, None] + np.arange(DEC_CHUNK)[None, :], (r1 - 1)[:, None])
            acc.add("kv_rows", l * kept + rows)
            acc.add("q", ((l * H + h[:, None]) * G + np.arange(G)[None, :]) * HEAD_DIM)
            acc.add("q", ((l * H + h[:, None]) * G + np.arange(G)[None, :]) * HEAD_DIM + HEAD_DIM - 1)
            acc.add("part", (l * items + its) * rec)
            acc.add("part", (l * items + its) * rec + rec - 1)
        for hh in range(H):
            i0, i1 = int(pre[hh]), int(pre[hh + 1])
            for g in range(G):
                acc.add("out", ((l * H + hh) * G + g) * HEAD_DIM + np.array([0, HEAD_DIM - 1]))
                if i0 == i1:
                    continue
                i = np.arange(i0, i1, dtype=np.int64)
                acc.add("part", (l * items + i) * rec + g * DEC_REC)
                acc.add("part", (l * items + i) * rec + g * DEC_REC + HEAD_DIM + 1)
    return acc


def decode_sizes(L, H, G, kept, offs):
    s = {"kv_rows": L * kept, "q": L * H * G * HEAD_DIM, "out": L * H * G * HEAD_DIM,
         "part": L * decode_items(H, kept, offs is not None, dec_chunk(G)) * G * DEC_REC}
    if offs is not None:
        s["offs"] = L * (H + 1)
    return s


# -------------------------------------------------------------- selection ----

SEL_THREADS, M_THREADS, K_CHUNK, K_BINS, K_MAX_GROUPS = 1024, 512, 16384, 2048, 1024
K_MASK_WORDS, K_LIST_CAP, K_SLOTS, K_HIST_BUFS = K_CHUNK // 32, 1024, 3, 3


def _clamp_budget(b, W, n):
    b = int(b)
    return W if b < W else (n if b > n else b)


def seg_span(p, seg, budgets):
    """seg_span (select.hip): what segment `seg` selects and where it writes."""
    if budgets is None:
        return dict(k=p["k"], base=seg * p["budget"], room=p["budget"], off=0, end=p["budget"],
                    reads=[])
    H, W, n, stride = p["H"], p["W"], p["n"], p["stride"]
    l, h = divmod(seg, H)
    off = sum(_clamp_budget(budgets[l * H + j], W, n) for j in range(h))
    b = _clamp_budget(budgets[l * H + h], W, n)
    o = min(off, stride)
    e = min(off + b, stride)
    return dict(k=(b - W) % U32, base=l * stride + o, room=e - o, off=o, end=e,
                reads=[l * H + j for j in range(h + 1)])


def _segment_writes(p, seg, sp, acc, threads):
    """The writes every select variant makes after its members are known:
    the segment's output slots [0, room), head offsets, and (budget vector,
    last head) the row tail."""
    o = np.arange(sp["room"], dtype=np.int64)
    acc.add("idx", sp["base"] + o)
    if p["budgets"] is not None:
        H = p["H"]
        l, h = divmod(seg, H)
        acc.add("head_offsets", [l * (H + 1) + h])
        if h + 1 == H:
            acc.add("head_offsets", [l * (H + 1) + H])
            acc.add("idx", l * p["stride"] + np.arange(sp["end"], p["stride"], dtype=np.int64))
    elif p["adaptive"]:
        acc.add("head_offsets", seg * (p["groups"] + 1) + np.arange(p["groups"] + 1))


def select_resident_accesses(p, budgets=None):
    """k_select (select.hip), global accesses: the score (and weight) loads
    of the segment, guarded by f < len, and the writes of the emission."""
    acc = Accesses()
    length = p["seg_len"]
    for seg in range(p["segments"]):
        sp = seg_span(p, seg, budgets)
        acc.add("budgets", sp["reads"])
        f = seg * length + np.array([0, length - 1]) if length else np.zeros(0)
        acc.add("scores", f)
        if p["two_stage"]:
            acc.add("weight", f)
        _segment_writes(p, seg, sp, acc, SEL_THREADS)
    return acc


def msel_chunk(p, c):
    g = c // p["cpg"]
    cc = c - g * p["cpg"]
    begin = g * p["n_cand"] + cc * K_CHUNK
    end = min(begin + K_CHUNK, (g + 1) * p["n_cand"])
    return g, begin, end


def digit_width(shift):
    return 10 if shift == 41 else (9 if shift == 9 else 11)


def msel_accesses(p, states, ccount, rng, budgets=None, lists=None):
    """k_msel_init, k_msel_hist0, k_msel_hist1, k_msel_filter,
    k_msel_finish and k_msel_emit (select.hip) with arbitrary segment
    states (count), per-chunk counts and list entries. Where a membership
    test decides a rank, each thread's member count is drawn at random
    within its 32 candidates."""
    acc = Accesses()
    S, chunks, W = p["segments"], p["chunks"], p["W"]
    for seg in range(S):
        st = states[seg]
        sp = seg_span(p, seg, budgets)
        acc.add("budgets", sp["reads"])
        acc.add("states", [slot * S + seg for slot in range(K_SLOTS)])
        # init clears the three histograms (stage 1's round 0, round 1,
        # stage 2's round 0), stage 1's finish round 1's; the passes add to
        # bins masked to K_BINS - 1; the picks read thread t's four bins
        # K_BINS - 4 - 4t .. K_BINS - 1 - 4t
        for rnd in range(K_HIST_BUFS):
            acc.add("ghist", (rnd * S + seg) * K_BINS + np.arange(K_BINS))
            t = np.arange(M_THREADS)
            acc.add("ghist", (rnd * S + seg) * K_BINS + (K_BINS - 4 - 4 * t)[:, None] + np.arange(4))
        for c in range(chunks):
            g, begin, end = msel_chunk(p, c)
            # hist0 / hist1 / filter loads: f < end
            if end > begin:
                acc.add("scores", seg * p["seg_len"] + np.array([begin, end - 1]))
                if p["two_stage"]:
                    acc.add("weight", seg * p["seg_len"] + np.array([begin, end - 1]))
            # k_msel_filter: the chunk's mask words and count; list slots
            # base + j (base from an atomic on the state: any uint32) kept
            # below K_LIST_CAP
            words = (seg * chunks + c) * K_MASK_WORDS + np.arange(K_MASK_WORDS)
            acc.add("mask", words)
            if p["two_stage"]:
                acc.add("mask1", words)
            acc.add("ccount", [seg * chunks + c])
            base = int(rng.integers(0, U32))
            slot = _u32(base + np.arange(K_LIST_CAP))
            acc.add("list", seg * K_LIST_CAP + slot[slot < K_LIST_CAP])
        # k_msel_finish: list entries j < count when count <= K_LIST_CAP,
        # else the segment streamed (f < seg_len); members marked from the
        # list's (arbitrary) indices, guarded by f < seg_len
        m = int(_u32(st.get("count", 0)))
        if m <= K_LIST_CAP:
            acc.add("list", seg * K_LIST_CAP + np.arange(m))
        if p["seg_len"]:
            acc.add("scores", seg * p["seg_len"] + np.array([0, p["seg_len"] - 1]))
            if p["two_stage"]:
                acc.add("weight", seg * p["seg_len"] + np.array([0, p["seg_len"] - 1]))
        fl = _u32(lists[seg]) if lists is not None else _u32(rng.integers(0, U32, size=64))
        fl = fl[fl < p["seg_len"]]
        g = fl // p["n_cand"] if p["n_cand"] else fl * 0
        pos = fl - g * p["n_cand"]
        ch = seg * chunks + g * p["cpg"] + pos // K_CHUNK
        acc.add("ccount", ch)
        acc.add("mask", ch * K_MASK_WORDS + (pos % K_CHUNK) // 32)
        # k_msel_emit, per chunk: rank0 = the (arbitrary, uint32) counts of
        # the segment's earlier chunks; its members (set bits of its
        # K_MASK_WORDS words: at most K_CHUNK) staged by rank in LDS take
        # slots rank0 + g*W + i, i < count; a group's last chunk writes the
        # window at rank0 + count + g*W + t, t < W; head offsets
        cc = _u32(ccount[seg])
        for c in range(chunks):
            g, begin, end = msel_chunk(p, c)
            acc.add("ccount", seg * chunks + np.arange(c + 1))
            rank0 = int(_u32(cc[:c].sum()))
            count = int(rng.integers(0, K_CHUNK + 1))
            assert count <= K_MASK_WORDS * 32 == K_CHUNK
            o = rank0 + g * W + np.arange(count, dtype=np.int64)
            acc.add("idx", sp["base"] + o[o < sp["room"]])
            if c - g * p["cpg"] + 1 == p["cpg"]:
                o = rank0 + count + g * W + np.arange(W, dtype=np.int64)
                acc.add("idx", sp["base"] + o[(o >= 0) & (o < sp["room"])])
            if budgets is None and p["adaptive"]:
                if c - g * p["cpg"] == 0:
                    acc.add("head_offsets", [seg * (p["groups"] + 1) + g])
                if c == 0:
                    acc.add("head_offsets", [seg * (p["groups"] + 1) + p["groups"]])
        assert (np.arange(chunks) // p["cpg"]).max(initial=0) < K_MAX_GROUPS
        if budgets is not None:
            H = p["H"]
            l, h = divmod(seg, H)
            acc.add("head_offsets", [l * (H + 1) + h])
            if h + 1 == H:
                acc.add("head_offsets", [l * (H + 1) + H])
                acc.add("idx", l * p["stride"] + np.arange(sp["end"], p["stride"], dtype=np.int64))
    return acc


def msel_pool_accesses(p, in_stride):
    """k_msel_pool (select.hip): per chunk, raw row (seg * groups + g) read
    at positions pos0 - halo .. pos0 + len + halo kept inside [0, n_cand)
    (whole 16-byte units inside it when VEC), the pooled scores written at
    seg * seg_len + begin + e, e < len."""
    acc = Accesses()
    halo = 4
    for seg in range(p["segments"]):
        for c in range(p["chunks"]):
            g, begin, end = msel_chunk(p, c)
            ln, pos0 = end - begin, begin - g * p["n_cand"]
            pos = np.arange(pos0 - halo, pos0 + ln + halo, dtype=np.int64)
            pos = pos[(pos >= 0) & (pos < p["n_cand"])]
            acc.add("raw", (seg * p["groups"] + g) * in_stride + pos)
            acc.add("pooled", seg * p["seg_len"] + begin + np.arange(ln, dtype=np.int64))
    return acc


def select_sizes(p):
    s = {"scores": p["segments"] * p["seg_len"], "budgets": p["L"] * p["H"],
         "states": K_SLOTS * p["segments"], "ghist": K_HIST_BUFS * p["segments"] * K_BINS,
         "ccount": p["segments"] * p.get("chunks", 0),
         "list": p["segments"] * K_LIST_CAP,
         "mask": p["segments"] * p.get("chunks", 0) * K_MASK_WORDS}
    if p["two_stage"]:
        s["weight"] = s["scores"]
        s["mask1"] = s["mask"]
    if p["budgets"] is not None:
        s["idx"] = p["L"] * p["stride"]
        s["head_offsets"] = p["L"] * (p["H"] + 1)
    else:
        s["idx"] = p["segments"] * p["budget"]
        if p["adaptive"]:
            s["head_offsets"] = p["segments"] * (p["groups"] + 1)
    return s


def select_plan(L, H, n, W, budget=0, adaptive=False, two_stage=False, budgets=None, stride=0):
    """The plan kvsel_select / kvsel_select_budgets build (api.hip), for
    arguments those calls accept."""
    n_cand = n - W
    groups = H if adaptive else 1
    p = dict(L=L, H=H, n=n, W=W, n_cand=n_cand, groups=groups, adaptive=adaptive,
             two_stage=two_stage, budgets=budgets, stride=stride,
             budget=budget if budgets is None else 0,
             k=(budget - groups * W) if budgets is None else 0,
             segments=L if adaptive else L * H, seg_len=groups * n_cand)
    p["cpg"] = -(-n_cand // K_CHUNK)
    p["chunks"] = groups * p["cpg"]
    return p


# ------------------------------------------------------------- anchors ----

AS_TILE, RES_ANCHORS, RES_BLOCKS, AS_BLOCK, MAX_ANCHOR_PAD = 64, 256, 16, 256, 2048


def anchor_kpad(k):
    return (k + AS_TILE - 1) // AS_TILE * AS_TILE


def anchor_accesses(L, H, n, k, anchors):
    """k_anchor_gather, k_anchor_assign_res / k_anchor_assign (the slot a
    packed score decodes to, for every half-tile, row code and lane half)
    and k_anchor_self of anchor.hip, with arbitrary anchor positions.
    Buffers: x [L*H*n] rows, anchors [L*H*k], arows [L*H*kpad] rows,
    rinv [L*H*kpad], slot and gamma [L*H*n], and the kernels' LDS tables
    rinv_lds (kResAnchors or kMaxAnchorPad entries)."""
    acc = Accesses()
    kpad = anchor_kpad(k)
    LH = L * H
    a = np.asarray(anchors, np.int64).reshape(LH, k)
    lh = np.arange(LH)[:, None]
    # k_anchor_gather: grid (kpad, L*H); slot s < k reads anchors and, when
    # the position is inside the head, its row of x; every slot writes its
    # row of arows and its rinv entry
    acc.add("anchors", lh * k + np.arange(k)[None, :])
    valid = (a >= 0) & (a < n)
    acc.add("x", (lh * n + a)[valid])
    acc.add("arows", lh * kpad + np.arange(kpad)[None, :])
    acc.add("rinv", lh * kpad + np.arange(kpad)[None, :])
    # assignment: vectors of every key block (reads of x guarded by key < n),
    # the per-slot table copied to LDS, and the decoded slot of every
    # (half-tile bu, row code, lane half) read back from that table
    keys = np.arange(n)
    acc.add("x", (lh * n + keys[None, :]).ravel())
    table = RES_ANCHORS if kpad <= RES_ANCHORS else MAX_ANCHOR_PAD
    acc.add("rinv", lh * kpad + np.arange(kpad)[None, :])
    acc.add("rinv_lds", np.arange(kpad))
    nh = kpad // 32
    bu, code, hf = np.meshgrid(np.arange(nh), np.arange(16), np.arange(2), indexing="ij")
    i = 15 - code
    slot = bu * 32 + 8 * (i >> 2) + 4 * hf + (i & 3)
    acc.add("rinv_lds", slot)                 # gamma's scale of the chosen slot
    # the argmax's scale reads: rows 4j..4j+3 of every half-tile
    j, e = np.meshgrid(np.arange(4), np.arange(4), indexing="ij")
    rows = (np.arange(nh)[:, None, None, None] * 32 + 8 * j[None, None] + 4 * np.arange(2)[None, :, None, None]
            + e[None, None])
    acc.add("rinv_lds", rows)
    acc.add("slot", (lh * n + keys[None, :]).ravel())
    acc.add("gamma", (lh * n + keys[None, :]).ravel())
    # k_anchor_self: positions inside the head write their slot and gamma
    acc.add("slot", (lh * n + a)[valid])
    acc.add("gamma", (lh * n + a)[valid])
    return acc, {"x": LH * n, "anchors": LH * k, "arows": LH * kpad, "rinv": LH * kpad,
                 "slot": LH * n, "gamma": LH * n, "rinv_lds": table}
