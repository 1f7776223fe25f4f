"""Attention cases that reach every instance of the packed-bit attention
kernel (k_att2), and the rule the launcher uses to pick one, restated from
launch_attend so that a CPU test can check the cases cover them all.

An instance is (record words per half record at most, value tiles, 1 KiB
loads per block, waves, 256-bit records, group <= 4). The launcher takes the
largest record width, the largest number of value columns (each kept code
cut at the record's byte boundaries) and the group of the call."""
import numpy as np

# (workload, average bits, group, tokens, explicit widths as (channels, width)
# runs from the largest eigenvalue down, or None for water-filling)
CASES = [
    (5, 2.0, 7, 2500, None),    # 256-bit records, group 7
    (1, 2.0, 4, 2500, None),    # 256-bit records, group 4
    (5, 1.33, 7, 2500, None),   # 170-bit records, at most 127 columns, group 7: three-word halves
    (5, 1.6, 7, 2500, None),    # 205-bit records, more than 127 columns, group 7
    (5, 1.9, 8, 2500, None),    # 243-bit records, group 8
    (2, 1.2, 3, 2500, None),    # 154-bit records, group 3
    (2, 3.0, 4, 1500, None),    # 384-bit records: halves of up to 8 words, three loads per block
    (2, 1.95, 6, 2500, None),   # 250-bit records (1000-byte blocks: one load), group 6
    (5, 198 / 128, 7, 2500, ((16, 8), (20, 2), (30, 1))),  # 198-bit records, 66 columns, group 7
    (2, 254 / 128, 4, 2500, ((24, 8), (31, 2))),           # 254-bit records: two loads per block
]


def widths(spec, d=128):
    """Channel widths from (channels, width) runs, the rest 0."""
    bits = np.zeros(d, np.uint8)
    j = 0
    for cnt, wd in spec:
        bits[j:j + cnt] = wd
        j += cnt
    return bits


def value_columns(bits):
    """Code pieces of one record: channel j's code, at bit offset sum of the
    earlier widths, cut at every byte boundary it crosses."""
    off, n = 0, 0
    for b in np.asarray(bits, np.int64):
        if b > 0:
            n += (off + b - 1) // 8 - off // 8 + 1
        off += int(b)
    return n


def instance(total_bits_list, bits_list, group):
    """The k_att2 instance launch_attend picks for a call over states with
    these total widths and channel widths, or None for the older kernel."""
    mb = max(total_bits_list)
    mv = max(value_columns(b) for b in bits_list)
    chunks = max(-(-((4 * t) + (12 if (4 * t) % 16 else 0)) // 1024) for t in total_bits_list)
    chunks = max(chunks, 1)
    if group > 8 or mb > 512 or mv > 191:
        return None
    g4 = group <= 4
    if mb <= 256 and chunks <= 1:
        if all(t == 256 for t in total_bits_list):
            return (4, 10, 1, 4, True, g4)
        if not g4 and mv <= 127 and mb <= 192:
            return (3, 8, 1, 4, False, False)
        if not g4 and mv <= 127:
            return (4, 8, 1, 4, False, False)
        return (4, 10, 1, 4, False, g4)
    if mb <= 256:
        return (4, 10, 2, 8, False, False)
    return (8, 12, 3, 8, False, False)


ALL_INSTANCES = {(4, 10, 1, 4, True, True), (4, 10, 1, 4, True, False), (3, 8, 1, 4, False, False),
                 (4, 8, 1, 4, False, False), (4, 10, 1, 4, False, False), (4, 10, 1, 4, False, True),
                 (4, 10, 2, 8, False, False), (8, 12, 3, 8, False, False)}
