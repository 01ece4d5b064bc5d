"""A model of the Hessian kernel's host-side token-split plan and work-item
map, for the tests: the plan (number of token splits and tokens per split)
follows the cost model of the library's split planner, and the item map is
the kernel's (super-tile, split) enumeration.  The CPU tests check the plan
against the library's own workspace query and that the item map covers
every (super-tile, 32-token step) exactly once; the GPU tests bound the fp32
running sums of S by the plan's real chain length."""

SUP = 256                 # super-tile edge (features)
STEP = 32                 # tokens per step
CUS = 256
XCD = 8
REG_B = 8                 # work order: blocks of 8 x 8 super-tiles
MAX_CHAIN = 2048
PART_ITEM = 4.0 * 128 * 128 * 4.0     # partial-tile bytes per (super-tile, split)
MAX_PART = 16.0 * 2 ** 30


def upper_tiles(nt):
    return nt * (nt + 1) // 2


def plan(d, n_tok, max_part=MAX_PART):
    """(nsplit, tokens per split) of the statistics kernel."""
    nt = -(-d // SUP)
    ntiles = upper_tiles(nt)
    steps = -(-n_tok // STEP)
    t_step = 1024.0 / 2.1e9
    t_byte = 1.0 / 4.0e12
    best = (1, steps * STEP)
    best_t = 1e30
    max_split = min(64, steps)
    min_split = 1
    while (min_split < max_split and -(-steps // min_split) > MAX_CHAIN and
           (min_split + 1) * ntiles * PART_ITEM <= max_part):
        min_split += 1
    for ns in range(min_split, max_split + 1):
        per = (((steps + ns - 1) // ns) + 1) & ~1
        nsr = -(-steps // per)
        if nsr > 1 and nsr * ntiles * PART_ITEM > max_part:
            continue
        rounds = -(-(ntiles * nsr) // CUS)
        t = rounds * per * t_step + (2.0 * nsr * ntiles * PART_ITEM * t_byte if nsr > 1 else 0.0)
        if t < best_t * 0.999:
            best_t = t
            best = (nsr, per * STEP)
    return best


def workspace_bytes(d, n_tok, max_part=MAX_PART):
    ns, _ = plan(d, n_tok, max_part)
    if ns <= 1:
        return 0
    nt = -(-d // SUP)
    b = ns * upper_tiles(nt) * int(PART_ITEM)
    return -(-b // 256) * 256


def chain_steps(d, n_tok, max_part=MAX_PART):
    """Longest fp32 running sum of S, in 32-token steps."""
    ns, ks = plan(d, n_tok, max_part)
    return min(ks, n_tok) // STEP + (1 if min(ks, n_tok) % STEP else 0)


def blocked_tile(t, nt):
    nb = -(-nt // REG_B)
    for br in range(nb):
        r0 = br * REG_B
        rh = min(REG_B, nt - r0)
        for bc in range(br, nb):
            c0 = bc * REG_B
            cw = min(REG_B, nt - c0)
            size = rh * (rh + 1) // 2 if bc == br else rh * cw
            if t >= size:
                t -= size
                continue
            if bc == br:
                i = 0
                while t >= rh - i:
                    t -= rh - i
                    i += 1
                return r0 + i, r0 + i + t
            return r0 + t // cw, c0 + t % cw
    raise AssertionError("item past the last tile")


def items(d, n_tok):
    """Yield (workgroup, split, ti, tj, first token, token count) of every
    launched workgroup that has an item."""
    nt = -(-d // SUP)
    ns, ks = plan(d, n_tok)
    ntiles = upper_tiles(nt)
    nitems = ntiles * ns
    per_xcd = -(-nitems // XCD)
    for w in range(XCD * per_xcd):
        item = (w % XCD) * per_xcd + w // XCD
        if item >= nitems:
            continue
        split, t = divmod(item, ntiles)
        ti, tj = blocked_tile(t, nt)
        tbeg = split * ks
        tend = min(tbeg + ks, n_tok)
        yield w, split, ti, tj, tbeg, tend - tbeg
