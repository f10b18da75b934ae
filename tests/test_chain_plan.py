"""Host-side planning of a verify pass in model order (sv_pass_chain_image).

CPU-only: the plan image is built in host memory for a stated compute-unit
count, from link descriptors whose pointers are plain integers (never
dereferenced).  Checks the round split, the barrier flags (a link waits iff
its x is an earlier link's xo; the link before it raises the arrivals), the
barrier groups and the buffer rules.  Source of the ordering: Karpathy's
Trick for Faster Local LLMs, "How Uzu optimizes bytes and tokens per pass"
(activations are the values handed from layer to layer).
"""
import numpy as np
import pytest

HDR = np.dtype([("magic", "<u4"), ("version", "<u4"), ("format", "<i4"), ("m", "<i4"),
                ("grid", "<i4"), ("nrounds", "<i4"), ("nlinks", "<i4"), ("nsignals", "<i4"),
                ("spin_limit", "<i4"), ("reserved1", "<u4"), ("group_size", "<i4", (16,)),
                ("pad", "<u4", (6,))])
RND = np.dtype([("codes", "<u8"), ("sz", "<u8"), ("x", "<u8"), ("y", "<u8"), ("xo", "<u8"),
                ("alpha", "<f4"), ("K", "<i4"), ("N", "<i4"), ("xo_cols", "<i4"),
                ("tile0", "<i4"), ("ntiles", "<i4"), ("signal_index", "<i4"), ("flags", "<u4"),
                ("pad", "<i4", (14,))])
WAIT, SIGNAL = 1, 2
H, F = 4096, 12288


def _parse(blob):
    hdr = np.frombuffer(blob, dtype=HDR, count=1)[0]
    rounds = np.frombuffer(blob, dtype=RND, count=int(hdr["nrounds"]), offset=HDR.itemsize)
    return hdr, rounds


class Alloc:
    """Distinct fake device addresses (4 KiB aligned, never dereferenced)."""

    def __init__(self):
        self.top = 1 << 32

    def __call__(self, nbytes):
        a = self.top
        self.top += (nbytes + 4095) // 4096 * 4096 + 4096
        return a


def decoder_chain(layers, m, alloc):
    """Per layer qkv -> o -> gate|up -> down, each input the previous xo."""
    links = []
    h = alloc(m * H * 2)
    for _ in range(layers):
        xq, xg, xd, hn = alloc(m * H * 2), alloc(m * H * 2), alloc(m * F * 2), alloc(m * H * 2)
        for x, N, K, xo, cols in ((h, 3 * H, H, xq, H), (xq, H, H, xg, H),
                                  (xg, 2 * F, H, xd, F), (xd, H, F, hn, H)):
            links.append(dict(x=x, codes=alloc(N * K // 2), scales=alloc(N * K // 16),
                              y=alloc(m * N * 4), xo=xo, xo_cols=cols, alpha=0.0625, K=K, N=N))
        h = hn
    return links


def test_decoder_chain_rounds_and_barriers():
    import verify_pass_sv_amd as sv
    links = decoder_chain(3, 16, Alloc())
    st, grid, blob = sv.sv_pass_chain_image("w4", links, 16, 256)
    assert st == 0 and grid == 256
    hdr, rounds = _parse(blob)
    assert hdr["magic"] == 0x4F565653 and hdr["nlinks"] == 12 and hdr["m"] == 16
    assert hdr["spin_limit"] == 1 << 20
    assert hdr["group_size"].sum() == 256 and set(hdr["group_size"]) == {16}
    # one round per link (qkv 768 tiles = 3 per workgroup, gate|up 1536 = 6)
    assert len(rounds) == 12
    assert [int(r["ntiles"]) for r in rounds] == [768, 256, 1536, 256] * 3
    # every link after the first reads the previous xo: it waits, and the
    # link before it raises the arrivals
    waits = [bool(r["flags"] & WAIT) for r in rounds]
    sigs = [bool(r["flags"] & SIGNAL) for r in rounds]
    assert waits == [False] + [True] * 11
    assert sigs == [True] * 11 + [False]
    assert hdr["nsignals"] == 11
    assert [int(r["signal_index"]) for r in rounds] == [0] + list(range(1, 12))
    for r, d in zip(rounds, links):
        assert (r["x"], r["xo"], r["K"], r["N"], r["xo_cols"]) == \
            (d["x"], d["xo"], d["K"], d["N"], d["xo_cols"])
        assert r["alpha"] == np.float32(0.0625)


def test_two_row_tiles_split_wide_links_into_rounds():
    import verify_pass_sv_amd as sv
    links = decoder_chain(1, 32, Alloc())
    st, grid, blob = sv.sv_pass_chain_image("w4", links, 32, 256)
    assert st == 0 and grid == 256
    hdr, rounds = _parse(blob)
    # at m > 16 a round holds at most 3 tiles per workgroup: gate|up (1536
    # tiles) runs as two rounds of 768; only its first round waits and only
    # its last raises the arrivals
    assert [(int(r["tile0"]), int(r["ntiles"])) for r in rounds] == \
        [(0, 768), (0, 256), (0, 768), (768, 768), (0, 256)]
    assert [int(r["flags"]) for r in rounds] == [SIGNAL, WAIT | SIGNAL, WAIT, SIGNAL, WAIT]


def test_independent_links_do_not_wait_and_small_links_shrink_the_grid():
    import verify_pass_sv_amd as sv
    a = Alloc()
    x = a(8 * 1024 * 2)
    links = [dict(x=x, codes=a(1024 * 512), scales=a(1024 * 64), y=a(8 * 1024 * 4), K=1024,
                  N=N) for N in (1024, 64, 512)]
    st, grid, blob = sv.sv_pass_chain_image("w4", links, 8, 256)
    assert st == 0
    assert grid == 4                            # the smallest link has 4 tiles
    hdr, rounds = _parse(blob)
    assert hdr["nsignals"] == 0 and all(int(r["flags"]) == 0 for r in rounds)
    # 64 tiles over 4 workgroups = 16 per workgroup: rounds of at most 6
    # per workgroup (24 tiles), every workgroup at least one tile
    assert [int(r["ntiles"]) for r in rounds if r["N"] == 1024] == [22, 22, 20]
    assert all(int(r["ntiles"]) >= grid for r in rounds)
    assert sum(hdr["group_size"]) == 4


def test_chain_buffer_rules():
    import verify_pass_sv_amd as sv
    a = Alloc()
    base = decoder_chain(1, 16, a)

    def status(links, m=16, fmt="w4"):
        return sv.sv_pass_chain_image(fmt, links, m, 256)[0]

    assert status(base) == 0
    bad = [dict(d) for d in base]
    bad[1]["x"] += 128                          # x overlaps an earlier xo without being it
    assert status(bad) == 2
    bad = [dict(d) for d in base]
    bad[2]["y"] = bad[3]["x"]                   # a y over another link's input
    assert status(bad) == 2
    bad = [dict(d) for d in base]
    bad[0]["xo"] = bad[0]["x"]                  # a link writes its own input
    assert status(bad) == 2
    bad = [dict(d) for d in base]
    bad[3]["xo"] = bad[1]["x"]                  # a later link writes an earlier input
    assert status(bad) == 2
    bad = [dict(d) for d in base]
    bad[0]["xo_cols"] = 4000                    # not a multiple of 64 channels
    assert status(bad) == 2
    bad = [dict(d) for d in base]
    bad[0]["xo"] += 64                          # xo not 128-byte aligned
    bad[1]["x"] += 64
    assert status(bad) == 3
    assert status(base, fmt="w8") == 0          # W8 chains are built
    assert status(base, fmt="w4_i8") == 4       # int8 chains are not
    assert status(base, m=33) == 2
    bad = [dict(d) for d in base]
    bad[0]["xo"] = 0                            # xo_cols without an xo
    assert status(bad) == 1
