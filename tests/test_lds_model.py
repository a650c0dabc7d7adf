"""The LDS bank model the kernels' chunk permutations are built for, and the
bank probe's patterns (bench.py --lds-probe), on the CPU.

The model (64 banks of 4 bytes; ds_read_b128 in four groups of 16 lanes: per
half-wave the lane quads of even and of odd index parity; ds_read_b64_tr_b16
per half-wave) is the one the probe measured on the GPU: lane 0 shares a
cycle with lanes 1-3, 12-15 and 20-27 only.  Here: every probe pattern is in
bounds and aligned, the model gives that pairing, and under it the kernels'
permutations are conflict-free while the first versions they replaced are
2-way conflicted, as the counters showed."""
import bench

LDS_BYTES = 32768


def test_probe_patterns_in_bounds_and_aligned():
    pats = bench.lds_probe_patterns()
    assert len(pats) == 63 + 10
    for name, kind, offs in pats:
        assert kind in (0, 1) and len(offs) == 64, name
        size = 16 if kind == 0 else 8
        for o in offs:
            if o != bench.LDS_SKIP:
                assert o % size == 0 and 0 <= o <= LDS_BYTES - size, (name, o)


def test_model_pairs_lane0_with_its_group():
    pats = bench.lds_probe_patterns()[:63]
    sharing = [b for b, (_, kind, offs) in enumerate(pats, 1) if bench.lds_model_conflict_degree(kind, offs) > 1]
    assert sharing == [1, 2, 3, 12, 13, 14, 15, 20, 21, 22, 23, 24, 25, 26, 27]


def test_kernel_permutations_under_the_model():
    deg = {name: bench.lds_model_conflict_degree(kind, offs) for name, kind, offs in bench.lds_probe_patterns()[63:]}
    first, current = {}, {}
    for name, d in deg.items():
        if "control" in name:
            assert d == 8, name
        elif "first version" in name:
            first[name] = d
        else:
            current[name] = d
    assert len(first) == 2 and all(d == 2 for d in first.values()), first
    assert len(current) == 6 and all(d == 1 for d in current.values()), current


def test_model_counts_broadcast_once():
    # every lane at the same address is a broadcast, not a conflict
    assert bench.lds_model_conflict_degree(0, [512] * 64) == 1
    assert bench.lds_model_conflict_degree(1, [64] * 64) == 1
