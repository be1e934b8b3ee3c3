"""The ctypes mirrors of the C-ABI structs match what a C compiler makes of
include/rtv.h: the same size and the same offset for every field, with no
padding between fields, so the binding and the library agree on every byte
they exchange."""
import ctypes
import os
import subprocess

import pytest

from kv_cache_attention_rtv_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRUCTS = [abi.rtv_config, abi.rtv_layout, abi.rtv_window]


def test_struct_layouts_match_the_header(tmp_path):
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "rtv.h"', "int main(void) {"]
    for st in STRUCTS:
        name = st.__name__
        lines.append(f'  printf("{name} sizeof %zu\\n", sizeof({name}));')
        for field, _ in st._fields_:
            lines.append(f'  printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    try:
        subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe)], check=True, capture_output=True, text=True)
    except FileNotFoundError:
        pytest.skip("gcc is not installed")
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        name, field, value = line.split()
        got[(name, field)] = int(value)
    for st in STRUCTS:
        name = st.__name__
        assert got[(name, "sizeof")] == ctypes.sizeof(st), name
        end = 0
        for field, ctype in st._fields_:
            assert got[(name, field)] == getattr(st, field).offset, (name, field)
            # no implicit padding: a field the header holds and the mirror
            # lacks would leave a gap here or at the end
            assert got[(name, field)] == end, (name, field)
            end += ctypes.sizeof(ctype)
        assert got[(name, "sizeof")] == end, name
