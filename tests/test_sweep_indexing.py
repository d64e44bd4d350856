"""Bounds of the sweep kernels' index arithmetic, emulated on the CPU (no GPU needed).

The HIP kernels build per-step row lists in LDS and address LDS tables, workspace records and
logit rows from them.  This test restates that index arithmetic (the same formulas as
draft_sampling_lossless_spec_amd/csrc/spec_cycle.hip and cycle_resident.hip, step by step) and
checks, over every batch size at the edges of a 32-row sub-block and every role mix that can occur,
that each index stays inside the buffer it addresses:

  stepwise sweep (k_sweep_fast): bias-slot list with the DRAFT / CORRECT alignment gap and the
  NO_ROW tail, the staged A-row group against the LDS budget, the per-wave unit spans and their
  (chunk, sub-block) pairs, the chunk-record offsets against the workspace partials;

  resident cycle (k_resident): the vocabulary partition over the workgroups, the tile columns of
  each wave, the LDS carve against the 160 KiB of a workgroup, the bias-slot entries, the per-wave
  record offsets against their areas, and the plain-row items.

Workspace sizes are taken from the library's own spec_workspace_bytes (the C ABI loads without a
GPU); LDS capacities are the kernels' constants, stated below.
"""
import itertools

import numpy as np
import pytest

SUB = 32                 # rows per MFMA sub-block
NT = 256                 # threads per workgroup
LDS_BYTES = 160 * 1024   # LDS of one workgroup on gfx950
MAX_R = 256
CHUNK = 64

BATCHES = [1, 31, 32, 33, 255, 256, 257, 300, 512, 1023, 1024]
POSITIONS = [1, 16, 32]


def role_mixes(B, rng):
    """Role vectors of one step: (draft, correct, plain) flags per request, including the extremes
    (every request drafts and corrects, nothing at all, only corrections)."""
    yield np.ones(B, bool), np.ones(B, bool), np.zeros(B, bool)
    yield np.zeros(B, bool), np.zeros(B, bool), np.zeros(B, bool)
    yield np.zeros(B, bool), np.ones(B, bool), np.zeros(B, bool)
    yield np.ones(B, bool), np.zeros(B, bool), np.ones(B, bool)
    for _ in range(4):
        d = rng.random(B) < rng.random()
        c = rng.random(B) < rng.random()
        p = (rng.random(B) < 0.7) & ~c          # a rejected request neither verifies nor takes a bonus
        yield d, c, p


def lists(d, c, p):
    """Slot layout of one step: DRAFT rows from slot 0, CORRECT rows from the next whole
    sub-block, the gap and the tail up to the last sub-block read NO_ROW."""
    n_draft, n_correct, n_plain = int(d.sum()), int(c.sum()), int(p.sum())
    c0 = -(-n_draft // SUB) * SUB
    n_sb = -(-(c0 + n_correct) // SUB)
    draft_slots = np.arange(n_draft)
    correct_slots = c0 + np.arange(n_correct)
    gap = np.arange(n_draft, c0)
    tail = np.arange(c0 + n_correct, n_sb * SUB)
    return n_draft, n_correct, n_plain, c0, n_sb, draft_slots, correct_slots, gap, tail


def workspace_bytes(B, K, V, R, path):
    from draft_sampling_lossless_spec_amd import binding
    return binding.spec_workspace_bytes(B, K, V, R, binding.BF16, binding.CHUNKED, path)


# ---------------------------------------------------------------------------------------------
# stepwise sweep
# ---------------------------------------------------------------------------------------------
REQ_META = 36            # bytes of the per-request table entry
SA_STRIDE = MAX_R + 8    # bf16 elements per staged A row (padded)
FAST_LDS_CAP = LDS_BYTES - 8 * (NT // 64)   # less the static scan buffer


def bias_slots_max(B):
    return 2 * B + 2 * SUB


def bias_dyn_bytes(B):
    return B * REQ_META + (bias_slots_max(B) + B) * 2


def fast_dyn_bytes(B, g):
    return -(-bias_dyn_bytes(B) // 16) * 16 + g * SA_STRIDE * 2


def sweep_fast_group(B):
    g = 16 * SUB
    while g > SUB and fast_dyn_bytes(B, g) > FAST_LDS_CAP:
        g -= SUB
    return g


@pytest.mark.parametrize("B", BATCHES)
def test_stepwise_sweep_indices_in_bounds(B):
    rng = np.random.default_rng(B)
    G_grid, V, R = 256, 151936, 256
    nrA = -(-V // CHUNK)
    g_stage = sweep_fast_group(B)
    assert g_stage >= SUB and g_stage % SUB == 0
    assert fast_dyn_bytes(B, g_stage) <= FAST_LDS_CAP, "staged A rows overflow the LDS"
    for d, c, p in role_mixes(B, rng):
        n_draft, n_correct, n_plain, c0, n_sb, ds, cs, gap, tail = lists(d, c, p)
        cap = bias_slots_max(B)
        for idx in (ds, cs, gap, tail):
            assert idx.size == 0 or (idx.min() >= 0 and idx.max() < cap), "bias-slot list overflow"
        assert n_plain <= B
        nslots = n_sb * SUB
        assert nslots <= cap
        # no sub-block mixes DRAFT and CORRECT rows
        if n_draft and n_correct:
            assert (ds // SUB).max() < (cs // SUB).min()
        # staged rows: the first kst sub-blocks, every staged row inside the group and the list
        kst = min(g_stage, nslots) // SUB
        rows = np.arange(kst * SUB)
        assert rows.size == 0 or (rows.max() < g_stage and rows.max() < nslots)
        # unit spans of every wave of the grid: (chunk, sub-block) inside (nrA, n_sb)
        nw = G_grid * (NT // 64)
        units = nrA * n_sb
        gw = np.arange(nw, dtype=np.int64)
        u0, u1 = units * gw // nw, units * (gw + 1) // nw
        assert np.all(u0 <= u1) and u1[-1] == units and u0[0] == 0
        assert np.all(u0[1:] == u1[:-1]), "unit spans must tile the units exactly"
        if units:
            u = np.arange(units, dtype=np.int64)
            ch, kk = u // max(n_sb, 1), u % max(n_sb, 1)
            assert ch.max() < nrA and kk.max() < n_sb
            # chunk records: (slot) * nrA + chunk inside the bias partials
            rec = (kk * SUB + SUB - 1) * nrA + ch
            assert rec.max() < cap * nrA


@pytest.mark.parametrize("B,K", list(itertools.product([1, 300, 1024], POSITIONS)))
def test_stepwise_workspace_covers_partials(B, K):
    V, R = 151936, 256
    nrA = -(-V // CHUNK)
    need = 16 * bias_slots_max(B) * nrA * 2 + 16 * B * -(-V // 4096)   # both bias partials, plain partials
    assert workspace_bytes(B, K, V, R, 1) >= need


# ---------------------------------------------------------------------------------------------
# resident cycle
# ---------------------------------------------------------------------------------------------
NW = NT // 64
AG_CHUNKS, LDS_CHUNKS = 2, 2
MAX_CHUNKS = NW * AG_CHUNKS + LDS_CHUNKS
MAX_G = 256
TP = 4096


def n_chunks(V):
    return -(-V // CHUNK)


def chunks_of(g, G, V):
    return n_chunks(V) // G + (1 if g < n_chunks(V) % G else 0)


def chunk_begin(g, G, V):
    n = n_chunks(V)
    return g * (n // G) + (g if g < n % G else n % G)


RES_REQ_META = 40        # bytes of the resident cycle's per-request table entry (ten 32-bit words)


def resident_smem(B):
    o = 4 * 16 * 64 * 16          # W tiles of the LDS chunks
    o += 2 * 16 * 64 * 16         # B operands, double-buffered
    o += B * RES_REQ_META         # per-request table
    o += 2 * B                    # roles, verify lengths
    o += 3 * B * 2                # slots
    o += bias_slots_max(B) * 4 + B * 2   # 32-bit bias entries, plain list
    o = -(-o // 16) * 16
    return o + NW * 16


PAST_END = 0xFFF00000    # byte offset past every logit tensor the resident kernels take (empty slots read there)


def resident_eligible(B, K, V, G, R=256):
    return (V % CHUNK == 0 and R % 16 == 0 and R <= 256 and 1 <= B <= NW * G and B <= 1024
            and 1 <= K <= 32 and B * (K + 1) * V * 2 <= PAST_END and V * R * 2 < 1 << 31
            and -(-n_chunks(V) // G) <= MAX_CHUNKS and -(-V // TP) <= MAX_G)


@pytest.mark.parametrize("B,K,V", [(64, 5, 151936), (256, 16, 151936), (1024, 5, 129280), (512, 16, 151936),
                                   (1024, 32, 151936), (2, 4, 1024), (1024, 12, 163840)])
def test_resident_tile_offsets_fit(B, K, V):
    """The bias tiles are buffer loads with 32-bit byte offsets: row offset + the lane's column base
    + a per-tile immediate (register tiles) or the wave's LDS-tile distance.  For every eligible
    shape the largest offset stays below 2^32, owned pieces lie inside their row, and the A-row
    staging offsets of a previous token stay below the 2^31 marker that reads zeros."""
    G, R = 256, 256
    if not resident_eligible(B, K, V, G):
        assert B * (K + 1) * V * 2 > PAST_END or V % CHUNK or B > NW * G
        pytest.skip("not eligible")
    cb = np.array([chunk_begin(g, G, V) for g in range(G)])
    nc = np.array([chunks_of(g, G, V) for g in range(G)])
    for nrow in (K, K + 1):
        last_row = B * nrow - 1
        for w in range(NW):
            dlds = 2 * (CHUNK * (NW * AG_CHUNKS - AG_CHUNKS * w + (w >> 1)) + 32 * (w & 1))
            assert dlds > 0
            for h in (0, 1):
                col = 2 * (CHUNK * (cb + AG_CHUNKS * w) + 16 * h)           # per workgroup
                base = last_row * 2 * V + col
                for i in range(5):
                    off = ((i >> 1) * 2 * CHUNK + (i & 1) * 64) if i < 4 else dlds
                    top = base + off + 16 + 16
                    assert top.max() < 1 << 32
                    cl = AG_CHUNKS * w + (i >> 1) if i < 4 else NW * AG_CHUNKS + (w >> 1)
                    own = cl < nc
                    # an owned piece ends inside its row
                    assert np.all((col + off + 32)[own] <= 2 * V)
    # A rows: prev * R + h R/2 + 8 w entries, plus 32 i (i < 4) entries, 16 bytes each read
    top = 2 * ((V - 1) * R + R // 2 + 8 * 3) + 64 * 3 + 16
    assert top <= V * R * 2 and V * R * 2 < 1 << 31


@pytest.mark.parametrize("V", [8, 1024, 2048, 3000, 3008, 20000, 129280, 151936, 163840])
def test_resident_vocabulary_partition(V):
    G = 256
    if -(-n_chunks(V) // G) > MAX_CHUNKS:
        pytest.skip("not eligible")
    cb = np.array([chunk_begin(g, G, V) for g in range(G)])
    nc = np.array([chunks_of(g, G, V) for g in range(G)])
    assert nc.max() <= MAX_CHUNKS and nc.sum() == n_chunks(V)
    assert np.all(cb[1:] == cb[:-1] + nc[:-1]), "chunk ranges must tile the vocabulary"
    # every tile column a wave uses: register chunks 2w, 2w+1 and LDS chunk 8 + w/2 (half w&1)
    for g in range(G):
        for w in range(NW):
            for i in range(5):
                cl = AG_CHUNKS * w + (i >> 1) if i < 4 else NW * AG_CHUNKS + (w >> 1)
                f = (i & 1) if i < 4 else (w & 1)
                for h in (0, 1):
                    v0 = CHUNK * (cb[g] + cl) + 32 * f + 16 * h
                    if cl >= nc[g]:
                        continue          # a chunk the workgroup does not own: address clamped
                    assert 0 <= v0 < n_chunks(V) * CHUNK
                    # a piece is loaded only when its first column is inside V (V % 8 == 0)
                    for piece in (v0, v0 + 8):
                        if piece < V:
                            assert piece + 8 <= V


@pytest.mark.parametrize("B", BATCHES)
def test_resident_lds_and_slots_in_bounds(B):
    G = 256
    assert resident_smem(B) <= LDS_BYTES, f"resident LDS carve {resident_smem(B)} B exceeds a workgroup"
    rng = np.random.default_rng(7 + B)
    for d, c, p in role_mixes(B, rng):
        n_draft, n_correct, n_plain, c0, n_sb, ds, cs, gap, tail = lists(d, c, p)
        cap = bias_slots_max(B)
        for idx in (ds, cs, gap, tail):
            assert idx.size == 0 or idx.max() < cap
        # entries pack (previous token + 1) above bit 11 and the request in bits 1..10
        assert B - 1 < 1 << 10 and 163840 + 1 < 1 << 21
        # merges: request b on workgroup b % G, at most NW per workgroup
        assert -(-B // G) <= NW
        # staged B operands: entry e = tid + NT i (i < 4) of 16 k-steps x 64 lanes
        e = np.arange(NT)[:, None] + NT * np.arange(4)[None, :]
        assert e.max() < 16 * 64


@pytest.mark.parametrize("B,K", list(itertools.product(BATCHES, POSITIONS)))
def test_resident_records_in_bounds(B, K):
    G, V, R = 256, 151936, 256
    if not resident_eligible(B, K, V, G):
        pytest.skip("not eligible")
    rec_d = 16 * bias_slots_max(B) * NW * MAX_G
    rec_c = 16 * (B + SUB) * NW * MAX_G
    rec_p = 16 * B * MAX_G
    rng = np.random.default_rng(B * 33 + K)
    for d, c, p in role_mixes(B, rng):
        n_draft, n_correct, n_plain, c0, n_sb, ds, cs, gap, tail = lists(d, c, p)
        slots = np.arange(n_sb * SUB)
        if slots.size:
            ri = ((slots[:, None] * NW + np.arange(NW)[None, :]) * MAX_G + (G - 1))
            assert 16 * (ri.max() + 1) <= rec_d
        if cs.size:
            rc = (((cs - c0)[:, None] * NW + np.arange(NW)[None, :]) * MAX_G + (G - 1))
            assert rc.min() >= 0 and 16 * (rc.max() + 1) <= rec_c
        nrP = -(-V // TP)
        assert nrP <= MAX_G
        if n_plain:
            assert 16 * ((n_plain - 1) * MAX_G + nrP) <= rec_p
            # plain items: (row, item) from a flat index over every wave of the grid
            it = np.arange(n_plain * nrP)
            row, item = it // nrP, it % nrP
            assert row.max() < n_plain and item.max() < nrP
            # a piece is loaded from its own address only when its first column is inside V
            # (V % 8 == 0, so then all eight are); other pieces load column 0 and read -inf
            col = item[:, None] * TP + (np.arange(TP // 512)[None, :] * 64 + np.arange(64)[:, None, None]) * 8
            inside = col < V
            assert np.all(col[inside] + 8 <= V)
    # the library sizes the workspace to hold every record area
    assert workspace_bytes(B, K, V, R, 2) >= rec_d + rec_c + rec_p


PUB_WORDS = 4   # 64-bit words a merge publishes per request and step (three used)


def pub_pack(step, roles, x, lse_q, lse_p):
    """The three words a merge of step `step` publishes (cycle_resident.hip's publish, restated):
    tag step + 1 in the high halves; roles << 28 | x + 1, and the two normalisers' bits below."""
    tag = (step + 1) << 32
    fq = int(np.float32(lse_q).view(np.uint32))
    fp = int(np.float32(lse_p).view(np.uint32))
    return tag | (roles << 28) | (x + 1), tag | fq, tag | fp


def pub_unpack(w0, w1, w2):
    roles = (w0 & 0xFFFFFFFF) >> 28
    x = (w0 & 0x0FFFFFFF) - 1
    lq = np.uint32(w1 & 0xFFFFFFFF).view(np.float32)
    lp = np.uint32(w2 & 0xFFFFFFFF).view(np.float32)
    return [w >> 32 for w in (w0, w1, w2)], roles, x, lq, lp


@pytest.mark.parametrize("B,K", list(itertools.product(BATCHES, POSITIONS)))
def test_resident_published_words(B, K):
    """The per-request words a merge hands to the next step's lists: every (parity, request, word)
    inside the workspace area behind the barrier flags, every one of them cleared at set-up by the
    workgroup that merges the request, and the tag / roles / token / normaliser packing lossless for
    every role set and token (the resident path keeps V <= 10 chunks x 64 columns x 256 workgroups)."""
    G, V, R = 256, 151936, 256
    if not resident_eligible(B, K, V, G):
        pytest.skip("not eligible")
    rec_d = 16 * bias_slots_max(B) * NW * MAX_G
    rec_c = 16 * (B + SUB) * NW * MAX_G
    rec_p = 16 * B * MAX_G
    flags = 8 * (MAX_G * 2 + 2)
    pub = 8 * 2 * B * PUB_WORDS
    assert workspace_bytes(B, K, V, R, 2) >= rec_d + rec_c + rec_p + flags + pub
    # addressing: ((parity B + b) PUB_WORDS + j) over both parities
    par, b, j = np.meshgrid(np.arange(2), np.arange(B), np.arange(PUB_WORDS), indexing="ij")
    idx = ((par * B + b) * PUB_WORDS + j).ravel()
    assert idx.min() == 0 and idx.max() < 2 * B * PUB_WORDS and np.unique(idx).size == idx.size
    # set-up clear: thread i of workgroup g clears word (i % 2P) of request g + G (i / 2P)
    cleared = set()
    for g in range(G):
        for i in range(NW * 2 * PUB_WORDS):
            bb, jj = g + G * (i // (2 * PUB_WORDS)), i % (2 * PUB_WORDS)
            if bb < B:
                assert bb % G == g   # the workgroup that merges (and later publishes) the request
                cleared.add(((jj // PUB_WORDS) * B + bb) * PUB_WORDS + jj % PUB_WORDS)
    assert cleared == set(idx.tolist())
    # packing: a cleared word (tag 0) never matches a polled step s >= 1, and a parity's word of
    # step s - 2 carries tag s - 1
    for step in range(K + 1):
        for roles in range(16):
            for x in (-1, 0, 1, V - 1, 163839):
                lq, lp = np.float32(-11.25 - step), np.float32(np.float32(3.5) * roles)
                tags, r2, x2, lq2, lp2 = pub_unpack(*pub_pack(step, roles, x, lq, lp))
                assert tags == [step + 1] * 3 and (r2, x2) == (roles, x)
                assert lq2 == lq and lp2 == lp
    tags, r2, x2, _, _ = pub_unpack(0, 0, 0)
    assert tags == [0, 0, 0] and r2 == 0 and x2 == -1
    inf_bits = pub_pack(0, 0, -1, -np.inf, np.inf)
    assert np.isneginf(pub_unpack(*inf_bits)[3]) and np.isposinf(pub_unpack(*inf_bits)[4])


# ---------------------------------------------------------------------------------------------
# W-resident acceptance statistics (k_stats_res)
# ---------------------------------------------------------------------------------------------
STATS_BATCH_BYTES = 160 << 20
FLAG_STRIDE = 2


def stats_eligible(B, K, V, R, G=256):
    return (V % CHUNK == 0 and R % 16 == 0 and R <= 256 and B >= 1 and K >= 1
            and B * (K + 1) * V * 2 <= PAST_END and V * R * 2 < 1 << 31
            and -(-n_chunks(V) // G) <= MAX_CHUNKS)


def stats_layout(V, n):
    """Batch rows and the offsets of the statistics kernel's arrays (the formulas of
    resident.h's stats_layout, restated)."""
    a256 = lambda x: -(-x // 256) * 256
    nbr = STATS_BATCH_BYTES // (4 * V) // SUB * SUB
    nbr = min(max(nbr, SUB), -(-max(n, 1) // SUB) * SUB)
    o, off = 0, {}
    for name, size in (("lq", 4 * nbr), ("lp", 4 * nbr), ("part1", 8 * nbr * MAX_G), ("part2", 4 * nbr * MAX_G),
                       ("flags", 8 * (MAX_G * FLAG_STRIDE + 2))):
        off[name] = (o, size)
        o = a256(o + size)
    return nbr, off, o


@pytest.mark.parametrize("B,K,V,R", [(256, 16, 151936, 256), (64, 5, 151936, 256), (300, 3, 2048, 16),
                                     (1, 1, 4096, 256), (9, 32, 64, 16), (1024, 32, 20032, 64),
                                     (40, 5, 20032, 64), (1024, 32, 151936, 256)])
def test_stats_batches_offsets_and_workspace(B, K, V, R):
    """Every listed row falls in exactly one batch; a batch's logits fit the cache budget (or it is
    one sub-block); per-batch arrays are indexed below nbr and MAX_G; the byte offsets of active
    rows stay inside their tensors and those of inactive slots lie past both tensors without
    wrapping; the library's workspace holds the statistics arrays."""
    from draft_sampling_lossless_spec_amd import binding
    if not stats_eligible(B, K, V, R):
        assert B * (K + 1) * V * 2 > PAST_END
        pytest.skip("not eligible")
    n = B * K
    nbr, off, total = stats_layout(V, n)
    assert nbr % SUB == 0 and nbr >= SUB
    assert nbr * 4 * V <= STATS_BATCH_BYTES or nbr == SUB
    covered = np.zeros(n, int)
    for r0 in range(0, n, nbr):
        nb = min(nbr, n - r0)
        assert 0 < nb <= nbr
        covered[r0:r0 + nb] += 1
        lr = np.arange(-(-nb // SUB) * SUB)   # slots of the batch's sub-blocks (the last one ragged)
        assert lr[lr < nb].max() < nbr
    assert np.all(covered == 1)
    # the last batch of the merge after the final barrier
    last_r0 = (n - 1) // nbr * nbr
    assert 0 < n - last_r0 <= nbr
    # record offsets: part1 / part2 [nbr][MAX_G], flags [MAX_G][FLAG_STRIDE] + error word
    assert (nbr - 1) * MAX_G + (MAX_G - 1) < off["part1"][1] // 8
    assert (nbr - 1) * MAX_G + (MAX_G - 1) < off["part2"][1] // 4
    assert MAX_G * FLAG_STRIDE + 1 < off["flags"][1] // 8
    ends = sorted((o, o + s) for o, s in off.values())
    assert all(a[1] <= b[0] for a, b in zip(ends, ends[1:])) and ends[-1][1] <= total
    # logit offsets (bytes): the last row of each tensor, every wave's tiles, plus the inactive marker
    G = 256
    cb = np.array([chunk_begin(g, G, V) for g in range(G)])
    for nrow in (K, K + 1):
        size = B * nrow * 2 * V
        for w in range(NW):
            dlds = 2 * (CHUNK * (NW * AG_CHUNKS - AG_CHUNKS * w + (w >> 1)) + 32 * (w & 1))
            top = (B * nrow - 1) * 2 * V + 2 * (CHUNK * (cb + AG_CHUNKS * w) + 16) + max(3 * 64 + 64, dlds) + 32
            assert top.max() < 1 << 32
        assert size <= PAST_END and PAST_END + 2 * 2 * CHUNK + 64 + 32 + 2 * CHUNK * NW * AG_CHUNKS + 64 < 1 << 32
    # the library's statistics workspace holds these arrays after its sweep arrays
    ws = binding.spec_stats_workspace_bytes(B, K, V, R)
    assert ws >= total
