"""CPU check of the blockwise prefill's workspace indexing, for every compiled instantiation
(bf16 and fp32 operands; chunk 16, 32, 64; dk 32, 64, 128).

The intra-chunk kernel stores the per-chunk blocks the scan reads as 64-lane MFMA operand
fragments; four waves share the stores (csrc/gdn_prefill.h, intra_chunk_kernel phase 2 for
the K and Q row fragments, phase 4 for Z and P').  The scan (inter_chunk_kernel) loads them
per chunk.  Every chunk's fragments are written in one kernel and read in the next, so
"never read before written" comes down to: every fragment the scan loads is stored by the
intra kernel for the same (batch, head, chunk), by exactly one wave, inside that chunk's
range of the array.  This test enumerates both sides' index expressions, restated from the
kernels' loops, and checks that.  A planted regrouping of the Z stores (the group index
taken as wave // 2) is caught, so the check can fail.
"""
import itertools

import pytest

WAVES = 4   # intra-chunk kernel: four waves per work item


def shape(elem, C, dk):
    KB = 32 if elem == "bf16" else 4          # k-values per MFMA
    NT = C // 16                               # token tiles per chunk
    NKD = dk // KB                             # k-blocks over dk
    NKC = (C + KB - 1) // KB                   # k-blocks over a chunk's tokens
    ND = dk // 16                              # dk tiles
    TPG = 2 if elem == "bf16" else 1           # s-tiles per stored Z k-block group
    NG = (NT + TPG - 1) // TPG
    return dict(KB=KB, NT=NT, NKD=NKD, NKC=NKC, ND=ND, TPG=TPG, NG=NG,
                Z_PER_CHUNK=ND * NKC, P_PER_CHUNK=NT * NKC, W_PER_CHUNK=NT * NKD)


def prow(wave, NT):
    """The P row tile a wave owns in phases 2 and 4 (None: none)."""
    pm = 0 if wave == 0 else NT - wave
    return pm if (wave == 0 or pm >= 1) else None


def kept_split(wave, NG):
    """The Z work split of intra_chunk_kernel phase 4: (group, first dk tile, dk tile stride)."""
    return wave % NG, wave // NG, WAVES // NG


def intra_stores(elem, C, dk, split=kept_split):
    """(array, fragment) -> list of waves storing it, for one work item (one chunk)."""
    S = shape(elem, C, dk)
    st = {}

    def put(arr, f, w):
        st.setdefault((arr, f), []).append(w)

    for w in range(WAVES):
        # phase 2: the K and Q row tiles of the wave's P row, as fragments (once per key head)
        m = prow(w, S["NT"])
        if m is not None:
            for kb in range(S["NKD"]):
                put("KF", m * S["NKD"] + kb, w)
                put("QF", m * S["NKD"] + kb, w)
        # phase 4: Z.  fp32 at 64-token chunks and dk = 128: wave w takes s-tile w for dk tiles
        # 0..3 and s-tile 3 - w for 4..7; otherwise k-block groups split over the waves, dk tiles
        # strided
        if elem == "f32" and S["NT"] == 4 and S["ND"] == 8 and split is kept_split:
            for dt in range(S["ND"]):
                u = w if dt < 4 else 3 - w
                for j in range(4):
                    put("Z", dt * S["NKC"] + 4 * u + j, w)
        else:
            zg, dt0, dts = split(w, S["NG"])
            for dt in range(dt0, S["ND"], dts):
                if elem == "bf16":
                    put("Z", dt * S["NKC"] + zg, w)
                else:
                    for j in range(4):
                        put("Z", dt * S["NKC"] + 4 * zg + j, w)
        # phase 4: P', fragments wholly above the diagonal are never stored
        if m is not None:
            if elem == "bf16":
                for kb in range(S["NKC"]):
                    if 2 * kb > m:
                        break
                    put("P", m * S["NKC"] + kb, w)
            else:
                for u in range(S["NT"]):
                    if u > m:
                        break
                    for j in range(4):
                        put("P", m * S["NKC"] + 4 * u + j, w)
    return st


def scan_loads(elem, C, dk):
    """(array, fragment) loaded by the scan for one chunk (chain waves 0..3, output 4..7)."""
    S = shape(elem, C, dk)
    DT, NT = S["ND"], S["NT"]
    TPW = (DT + 3) // 4
    loads = set()
    for w4 in range(4):
        m = w4 % NT
        # chain wave: its K row tile and the Z rows of its state tiles
        for kb in range(S["NKD"]):
            loads.add(("KF", m * S["NKD"] + kb))
        for tw in range(TPW):
            dt = min(w4 + 4 * tw, DT - 1)
            for kb in range(S["NKC"]):
                loads.add(("Z", dt * S["NKC"] + kb))
        # output wave: its Q row tile and P' row tile up to the last block with nonzeros
        for kb in range(S["NKD"]):
            loads.add(("QF", m * S["NKD"] + kb))
        pkmax = (m * 16 + 15) // S["KB"]
        for kb in range(S["NKC"]):
            if kb <= pkmax:
                loads.add(("P", m * S["NKC"] + kb))
    return loads


def coverage_errors(elem, C, dk, split=kept_split):
    S = shape(elem, C, dk)
    per = {"KF": S["W_PER_CHUNK"], "QF": S["W_PER_CHUNK"], "Z": S["Z_PER_CHUNK"],
           "P": S["P_PER_CHUNK"]}
    st = intra_stores(elem, C, dk, split)
    errs = []
    for (arr, f), ws in st.items():
        if not 0 <= f < per[arr]:
            errs.append(f"{arr} fragment {f} stored outside the chunk's {per[arr]} by waves {ws}")
        if len(ws) != 1:
            errs.append(f"{arr} fragment {f} stored by waves {ws}")
    for arr, f in sorted(scan_loads(elem, C, dk)):
        if (arr, f) not in st:
            errs.append(f"{arr} fragment {f} loaded by the scan but never stored")
    return errs


INSTANCES = list(itertools.product(["bf16", "f32"], [16, 32, 64], [32, 64, 128]))


@pytest.mark.parametrize("elem,C,dk", INSTANCES)
def test_every_loaded_fragment_is_stored_once_in_range(elem, C, dk):
    assert coverage_errors(elem, C, dk) == []


@pytest.mark.parametrize("elem,C,dk", INSTANCES)
def test_z_and_kq_stores_cover_the_whole_chunk(elem, C, dk):
    # Z, KF and QF are read in full by the scan's waves (for some shapes by several of them):
    # every fragment of the chunk is stored
    S = shape(elem, C, dk)
    st = intra_stores(elem, C, dk)
    for arr, n in (("Z", S["Z_PER_CHUNK"]), ("KF", S["W_PER_CHUNK"]), ("QF", S["W_PER_CHUNK"])):
        assert {f for (a, f) in st if a == arr} == set(range(n)), arr


def test_planted_regrouping_is_caught():
    # Waves 2 and 3 take the second group of s-tiles (group = wave // 2, dk tiles strided by
    # 2 from wave % 2): a valid split where a chunk has two groups (bf16, 64 tokens), but at 16
    # and 32 tokens there is one group, and waves 2 and 3 store one fragment further on, over
    # another wave's fragment or past the chunk
    regroup = lambda wave, NG: (wave // 2, wave % 2, 2)  # noqa: E731
    bad = {(e, c, d) for (e, c, d) in INSTANCES if e == "bf16" and coverage_errors(e, c, d, regroup)}
    assert bad == {("bf16", c, d) for c in (16, 32) for d in (32, 64, 128)}


def foff(elem, f, lane):
    """Offset, in elements, of fragment f's lane element in an array of stored fragments
    (gdn_device.h, Elem::foff): bf16 fragments of 8 elements one after another; fp32 fragments
    in groups of four whose lane elements are adjacent."""
    if elem == "bf16":
        return (f * 64 + lane) * 8
    return ((f >> 2) * 64 + lane) * 4 + (f & 3)


@pytest.mark.parametrize("elem,C,dk", INSTANCES)
def test_grouped_fragment_offsets_tile_each_chunk(elem, C, dk):
    # The stores and loads address fragment f of a tile as tile_base + foff(f, lane), with the
    # tile bases of the kernels (row tile m of KF/QF: m * NKD fragments; dk tile dt of Z:
    # dt * NKC; row tile m of P': m * NKC).  Within one chunk the offsets must be a bijection
    # onto its elements, and a 16-byte lane group must never straddle two tiles.
    S = shape(elem, C, dk)
    kpl = 8 if elem == "bf16" else 1
    grp = 1 if elem == "bf16" else 4
    for tiles, per_tile in ((S["NT"], S["NKD"]), (S["ND"], S["NKC"]), (S["NT"], S["NKC"])):
        assert per_tile % grp == 0
        seen = set()
        for t in range(tiles):
            base = t * per_tile * 64 * kpl
            for f in range(per_tile):
                for lane in range(64):
                    o = base + foff(elem, f, lane)
                    for e in range(kpl):
                        assert o + e not in seen
                        seen.add(o + e)
                    if f % grp:   # adjacent to the group's first fragment
                        assert o == base + foff(elem, f - f % grp, lane) + f % grp
        assert seen == set(range(tiles * per_tile * 64 * kpl))
