"""Tile-and-mask model of an elementwise launch -- TEST INFRASTRUCTURE ONLY.

Follows the worked vector-add example of the Triton tutorial page
(accesspath.com, "GPU architecture basics" / "Triton in practice"): n
elements are covered by ceil(n / BLOCK) program instances; instance ``pid``
takes offsets ``pid * BLOCK + arange(BLOCK)`` and a mask ``offsets < n``, so
lanes past the end neither load nor store. The same scheme is the masked
``tl.load``/``tl.store`` of "Lecture 6: GPU Kernels and Triton"
(cs336.sjfarmltd.com), section 3.2.
"""
from __future__ import annotations


def cdiv(a: int, b: int) -> int:
    """Ceiling division for non-negative a and positive b."""
    if b <= 0 or a < 0:
        raise ValueError("cdiv needs a >= 0 and b > 0")
    return (a + b - 1) // b


def programs(n_elements: int, block_size: int):
    """List of (pid, offsets, mask) for every program instance of the grid."""
    grid = cdiv(n_elements, block_size)
    out = []
    for pid in range(grid):
        block_start = pid * block_size
        offsets = [block_start + i for i in range(block_size)]
        mask = [o < n_elements for o in offsets]
        out.append((pid, offsets, mask))
    return out


def covered(n_elements: int, block_size: int):
    """Offsets that some instance loads and stores, in launch order."""
    return [o for _, offs, mask in programs(n_elements, block_size)
            for o, m in zip(offs, mask) if m]
