"""The library's host-side tiling rules, restated for tests (no GPU code).

A test that expects a route or a workspace size derives it here, from the
same rule the library applies, so that a change to either side shows up as
a mismatch."""
import math


def packed_blocks(N, C, HW, size):
    """Workgroups per image of the packed-pixel NHWC split route: runs of
    kpx = 16 / gcd(C * size, 16) pixels (whole 16-byte vectors), P = 256 //
    vectors-per-run runs in flight per workgroup, R >= 2 runs per thread
    (as many as keep the grid near 2048 workgroups, whole steps of 4 beyond
    4)."""
    kpx = 16 // math.gcd(C * size, 16)
    sv = kpx * C * size // 16
    runs, P = HW // kpx, 256 // sv
    R = max(2, -(-N * runs // (P * 2048)))
    if R > 4:
        R = -(-R // 4) * 4
    return -(-runs // (P * R))


def packed_applies(C, HW, size):
    """Whether an aligned NHWC image of C channels takes packed runs: a run
    of more than one pixel, H*W a whole number of runs, at most 256 vectors
    a run."""
    kpx = 16 // math.gcd(C * size, 16)
    return kpx > 1 and HW % kpx == 0 and kpx * C * size // 16 <= 256


def nhwc_cluster_fits(C, groups, E, HW):
    """Whether the NHWC channel-block cluster has a plan for E-element
    accesses: channel blocks of whole groups and accesses, at most 256
    accesses and 16 groups each, and an image of at most 64 slices of at most
    16 pixels per thread."""
    cpg = C // groups
    if C % E or cpg < E:
        return False
    unit = cpg // math.gcd(cpg, E) * E
    nb0 = C // unit
    for ncb in range(1, nb0 + 1):
        if nb0 % ncb:
            continue
        cbv, cbg = C // ncb // E, C // ncb // cpg
        if cbv > 256 or cbg > 16:
            continue
        P = 256 // cbv
        if -(-HW // (P * 16)) <= 64:
            return True
    return False


def nhwc_packed_cluster_fits(N, C, groups, size, HW, block_fits):
    """Whether the NHWC cluster takes packed runs for aligned tensors: pixels
    of C channels that are not a whole number of 16-byte vectors, runs of
    kpx = 16 / gcd(C * size, 16) pixels (H*W a whole number of them) of at
    most 256 vectors, at most 16 groups, an image of at most 64 slices of at
    most 16 runs per thread (slices as the library plans them); and then
    preferred when the channel-block form has no plan (block_fits false), or
    the grid (N * slices) has at least 256 workgroups, or at least 96 with at
    least 12 runs per thread."""
    kpx = 16 // math.gcd(C * size, 16)
    if kpx == 1 or HW % kpx or groups > 16:
        return False
    cbv = kpx * C * size // 16
    if cbv > 256:
        return False
    units, P = HW // kpx, 256 // cbv
    k_fit = -(-units // (P * 16))
    if k_fit > 64:
        return False
    K = min(-(-512 // N), units * cbv // 256, 32)
    K = min(max(K, k_fit), 64, units)
    if -(-units // P) <= 6:
        K = 1
    pps = -(-units // K)
    K = -(-units // pps)
    R = -(-pps // P)
    grid = N * K
    return not block_fits or grid >= 256 or (R >= 12 and grid >= 96)
