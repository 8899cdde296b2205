"""Blocking of parameters into B x B blocks (oracle; test infrastructure only).

[3DS] "Hyperparameters": ``block_size`` splits every dimension larger than it
into blocks, and 0 means never split.  [DASH] "4. Blocking Strategy": for
B = 1024 a 32000 x 2048 gradient gives 62 full 1024 x 1024 blocks and two
256 x 1024 remainder blocks.  [DASH] "D. DASH for Computer Vision" and [3DS]
"Hyperparameters": tensors of order > 2 are viewed as 2-D by keeping dimension
0 and merging the rest ((E, 3, 16, 16) -> (E, 768)).

Reading taken where the pages are silent: blocks are listed parameter by
parameter, and inside a parameter in row-major order of the block grid; a
ragged block is zero-padded to B x B when stacked.  ``block_size`` 0 makes the
whole parameter one block whose stack side is max(rows, cols).
"""

import numpy as np

# One block-table row: (param, brow, bcol, row0, col0, rows, cols, B).
FIELDS = ("param", "brow", "bcol", "row0", "col0", "rows", "cols", "B")


def reshape_2d(shape):
    """2-D view of a parameter shape: keep dim 0, merge the rest.

    A 1-D shape (n,) becomes (1, n) and a 0-D shape becomes (1, 1).
    """
    shape = tuple(int(s) for s in shape)
    if len(shape) == 0:
        return (1, 1)
    if len(shape) == 1:
        return (1, shape[0])
    rest = 1
    for s in shape[1:]:
        rest *= s
    return (shape[0], rest)


def plan_blocks(shapes2d, block_sizes):
    """Block table for a list of 2-D shapes and per-parameter block sizes.

    Returns an int64 array of shape [nblk, 8] with the columns of ``FIELDS``.
    """
    rows_out = []
    for p, ((m, n), bs) in enumerate(zip(shapes2d, block_sizes)):
        m, n, bs = int(m), int(n), int(bs)
        if m <= 0 or n <= 0:
            continue
        B = max(m, n) if bs == 0 else bs
        nbr = -(-m // B)
        nbc = -(-n // B)
        for br in range(nbr):
            for bc in range(nbc):
                r0 = br * B
                c0 = bc * B
                rows_out.append((p, br, bc, r0, c0, min(B, m - r0), min(B, n - c0), B))
    return np.asarray(rows_out, dtype=np.int64).reshape(-1, 8)


def block_slices(table, b):
    """(row slice, col slice) of block b inside its parameter."""
    _, _, _, r0, c0, rows, cols, _ = (int(x) for x in table[b])
    return slice(r0, r0 + rows), slice(c0, c0 + cols)


def pack_blocks(mats2d, table, B, dtype=None):
    """Stack the blocks of the 2-D matrices into [nblk, B, B], zero padded."""
    nblk = table.shape[0]
    dt = dtype if dtype is not None else (mats2d[0].dtype if len(mats2d) else np.float64)
    out = np.zeros((nblk, B, B), dtype=dt)
    for b in range(nblk):
        p = int(table[b, 0])
        rs, cs = block_slices(table, b)
        blk = mats2d[p][rs, cs]
        out[b, : blk.shape[0], : blk.shape[1]] = blk
    return out


def unpack_blocks(stack, table, shapes2d, dtype=None):
    """Inverse of ``pack_blocks``: the valid region of each block back in place."""
    dt = dtype if dtype is not None else stack.dtype
    mats = [np.zeros(s, dtype=dt) for s in shapes2d]
    for b in range(table.shape[0]):
        p = int(table[b, 0])
        rs, cs = block_slices(table, b)
        rows, cols = int(table[b, 5]), int(table[b, 6])
        mats[p][rs, cs] = stack[b, :rows, :cols]
    return mats
