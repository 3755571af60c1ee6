"""Source transform for the host emulation: prints a kernel source with its
dynamic shared memory routed to the emulator.

The row kernels carve named arrays out of one dynamic LDS block; here each of
them gets its own heap allocation of its declared extent, so AddressSanitizer
reports an index past one array even where the real layout would put it
inside a neighbour.  Any other kernel's dynamic LDS becomes the emulator's
per-workgroup block.

usage: python xform.py SOURCE > OUTPUT
"""
import re
import sys

# extent of each named row-kernel LDS array, in elements
EXTENTS = {"bitmap": "(long)P.bm_wpt * B", "hkey": "P.hs", "hval": "P.hs", "headz": "P.k",
           "headp": "P.k", "headlp": "P.k", "hout": "P.k", "lval": "(long)P.ke * N",
           "lvec": "P.ke", "lslot": "(long)P.ke * N"}


def transform(src):
    src = src.replace("extern __shared__ __align__(16) unsigned char lds[];",
                      "unsigned char* lds = ::emu::dyn_lds;")
    for i, (name, extent) in enumerate(EXTENTS.items()):
        pat = re.compile(r"(\w+)\* " + name +
                         r" = reinterpret_cast<\w+\*>\(lds \+ P\.off_" + name + r"\);")
        src, n = pat.subn(lambda m: f"{m.group(1)}* {name} = ::emu::lds_arr<{m.group(1)}>"
                                    f"({i}, {extent});", src)
        assert n <= 1, name
    return src


if __name__ == "__main__":
    sys.stdout.write(transform(open(sys.argv[1]).read()))
