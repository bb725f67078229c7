"""Host-side bounds checks of kernel index arithmetic (no GPU): the element
ranges a kernel's loads touch, recomputed from the same index formulas on
the CPU, stay inside the buffers the launch gives it.

* summarize_kernel, transposed values v_pt [H, n_t, d, block]: 256 threads,
  thread t reads rows rv + 16 i (rv = t / 16) from token jc = 8 (t % 16),
  8 tokens at a time when block % 8 == 0 (one 16-byte load), else only the
  block's real tokens one by one.  Every element read must lie in the row
  of its block and before the row's last real token.
"""
import numpy as np
import pytest


def _summarize_vpt_reads(H, N, d, block, nbt):
    nb = -(-N // block)
    out = []
    vec_rows = block % 8 == 0
    for h in (0, H - 1):
        for B in (0, nb - 1):
            n_real = min(block, N - B * block)
            vblk = ((h * nbt) + B) * d * block
            for t in range(256):
                rv, jc = t // 16, (t % 16) * 8
                for i in range(d // 16):
                    if jc >= n_real:
                        continue
                    cnt = 8 if vec_rows else min(8, n_real - jc)
                    row = rv + 16 * i
                    lo = vblk + row * block + jc
                    out.append((lo, lo + cnt, vblk + row * block, vblk + row * block + n_real))
    return out


@pytest.mark.parametrize("block", [5, 100, 64, 128, 1, 7])
@pytest.mark.parametrize("d", [64, 128])
def test_summarize_value_reads_stay_in_the_row(block, d):
    H, N = 3, 1000 + block // 2
    nb = -(-N // block)
    total = H * nb * d * block
    for lo, hi, row_lo, row_end in _summarize_vpt_reads(H, N, d, block, nb):
        assert row_lo <= lo and hi <= row_lo + block <= total
        if block % 8:
            assert hi <= row_end          # element reads stop at the last real token
        else:
            assert lo % 8 == 0            # 16-byte aligned vector loads (bf16: 8 elements)
