"""The kernels' work lists in a table image (the ints after the build list), for
the CPU tests of the planner and of append."""
import numpy as np

# record widths of the work lists after the build list: decode unit (first item,
# end item, first output row b * Hq + h * G, layer), decode item (unit, slot_lo,
# slot_hi, gap_lo, then the unit's b, l, h, page_off), prefill tile (unit, row)
DU_INTS, DI_INTS, PI_INTS = 4, 8, 2


def work_lists(t, z, G, Hq):
    """Decode units, decode items and prefill tiles of a table image; checks the
    copies of unit fields the decode records carry against the unit records."""
    U = z.num_units
    w0 = z.table_len + z.num_pages  # work lists follow the build list
    du = t[w0:w0 + DU_INTS * U].reshape(U, DU_INTS)
    i0 = w0 + DU_INTS * U
    items = t[i0:i0 + DI_INTS * z.decode_items].reshape(-1, DI_INTS)
    units = t[int(t[12]):int(t[12]) + 16 * U].reshape(U, 16)  # b, l, h at 1..3, page_off 14
    assert np.array_equal(du[:, 2], units[:, 1] * Hq + units[:, 3] * G)
    assert np.array_equal(du[:, 3], units[:, 2])
    if len(items):
        assert np.array_equal(items[:, 4:8], units[items[:, 0]][:, [1, 2, 3, 14]])
    p0 = i0 + DI_INTS * z.decode_items
    pre = t[p0:p0 + PI_INTS * z.prefill_items].reshape(-1, PI_INTS)
    return du[:, :2], items[:, :4], pre, p0 + PI_INTS * z.prefill_items
