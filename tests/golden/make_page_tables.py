"""Writes the small tables in this folder by evaluating formulas printed on the
reference pages (Modern GPU Programming for MLSys (zh), chapter "TMA").  It
imports neither the oracle nor the product; each table's header names the
section it comes from.  Run from this folder: python make_page_tables.py
"""


def sectors_2d():
    lines = ["# Modern GPU Programming for MLSys (zh), chapter 'TMA', section on how TMA writes",
             "# the swizzled layout: 16x128 fp16 tensor, 8x64 box, 128-byte rows of eight 16-byte",
             "# sectors; under 128B the logical sector `col` of row `row` is written to physical",
             "# sector col XOR row.  Under NONE logical sector c stays at physical sector c.",
             "# Table: for each box row r (0..7) the logical sector held by physical sectors 0..7.",
             "# mode row p0 p1 p2 p3 p4 p5 p6 p7"]
    for mode in ("none", "128b"):
        for r in range(8):
            held = [0] * 8
            for col in range(8):
                phys = col ^ r if mode == "128b" else col
                held[phys] = col
            lines.append(f"{mode} {r} " + " ".join(map(str, held)))
    return lines


def atoms_3d():
    lines = ["# Modern GPU Programming for MLSys (zh), chapter 'TMA', section on moving several",
             "# swizzle atoms with a 3D TMA: a 16x256 fp16 matrix; a 16x128 slice is regrouped as",
             "# (group=2, row=16, col=64) with group = j // 64, col = j % 64; group g of the slice",
             "# occupies its own 16 rows x 128 bytes, rows 0-7 and 8-15 of each group are separate",
             "# atoms (four atoms in all), and inside an atom physical sector = logical sector",
             "# XOR (row % 8).",
             "# Table: col_offset group row physical_sector -> global_row global_first_column",
             "# (the physical 16-byte sector holds 8 fp16 starting at that global column)."]
    for off in (0, 128):
        for g in range(2):
            for row in range(16):
                for p in range(8):
                    logical = p ^ (row % 8)
                    j = g * 64 + logical * 8
                    lines.append(f"{off} {g} {row} {p} {row} {off + j}")
    return lines


def bank_sectors():
    lines = ["# Modern GPU Programming for MLSys (zh), chapter 'TMA', section on the grouping",
             "# requirement of 128-byte swizzle: 16x16 grid of 16-byte sectors (256-byte rows),",
             "# 32 banks of 4 bytes taken as 8 bank sectors S0..S7; eight consecutive rows read",
             "# one sector column.  Grouped (two 128-byte groups per row): bank sector =",
             "# local_col XOR (row % 8), col // 8 picks the group, local_col = col % 8.",
             "# Ungrouped (256-byte row stride): bank sector = local_col XOR ((2*row + col//8) % 8).",
             "# The page states the first gives 8 distinct sectors, the second 4 sectors hit twice.",
             "# Table: layout row0 col S0 S1 S2 S3 S4 S5 S6 S7 (hit counts)"]
    for layout in ("grouped", "ungrouped"):
        for row0 in range(9):
            for col in range(16):
                h = [0] * 8
                for row in range(row0, row0 + 8):
                    lc, g = col % 8, col // 8
                    s = lc ^ (row % 8) if layout == "grouped" else lc ^ ((2 * row + g) % 8)
                    h[s] += 1
                lines.append(f"{layout} {row0} {col} " + " ".join(map(str, h)))
    return lines


def txbar_4096():
    return ["# Modern GPU Programming for MLSys (zh), chapter 'TMA', section on waiting for a TMA",
            "# load: two operand tiles of 2048 bytes each share one barrier initialised with an",
            "# expected arrival count of 1; arrive.expect_tx(4096) leaves arrival count 0 and",
            "# 4096 pending bytes; when both copies are done the pending bytes are 0 and the",
            "# phase completes, so a wait on phase 0 succeeds.  The page prints the counts at",
            "# completion as arrival count 0, pending bytes 0.",
            "# Reading (not printed on the page): the operation that completes a phase flips the",
            "# phase and re-arms the arrival count to the count given at init, ready for the next",
            "# phase, as a hardware barrier phase does.  So the last row records the state after",
            "# that re-arm: arrivals_left 1 (the page's 0, re-armed), pending 0, phase 1.",
            "# Table: op argument -> arrivals_left pending_bytes phase try_wait(0)",
            "init 1 -> 1 0 0 0",
            "arrive_expect_tx 4096 -> 0 4096 0 0",
            "complete_tx 2048 -> 0 2048 0 0",
            "complete_tx 2048 -> 1 0 1 1"]


if __name__ == "__main__":
    for name, fn in (("mlc_example_2d_sectors.txt", sectors_2d),
                     ("mlc_example_3d_atoms.txt", atoms_3d),
                     ("mlc_bank_sectors.txt", bank_sectors),
                     ("mlc_txbar_4096.txt", txbar_4096)):
        with open(name, "w") as f:
            f.write("\n".join(fn()) + "\n")
