"""The ctypes structures of the binding match the C declarations of
include/qkv_epilogue.h field by field (offset, and the struct size), and the
binding's constants match the header's macros, checked against small C
programs that the host compiler builds from the header."""
import ctypes
import json
import os
import re
import shutil
import subprocess

import pytest

from qkv_bias_rope_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = {
    "qkv_epilogue_config_t": B.QkvEpilogueConfig,
    "qkv_epilogue_args_t": B.QkvEpilogueArgs,
    "qkv_proj_args_t": B.QkvProjArgs,
    "qkv_epilogue_plan_t": B.QkvEpiloguePlan,
}


def _c_layout(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "qkv_epilogue.h"',
             "int main(void) {", '    printf("{");']
    first = True
    for cname, cls in STRUCTS.items():
        for fname, _ in cls._fields_:
            sep = "" if first else ","
            first = False
            lines.append(f'    printf("{sep}\\"{cname}.{fname}\\": %zu", offsetof({cname}, {fname}));')
        lines.append(f'    printf(",\\"{cname}.sizeof\\": %zu", sizeof({cname}));')
    lines += ['    printf("}\\n");', "    return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return json.loads(out)


def test_struct_layouts_match_header(tmp_path):
    c = _c_layout(tmp_path)
    for cname, cls in STRUCTS.items():
        for fname, _ in cls._fields_:
            assert getattr(cls, fname).offset == c[f"{cname}.{fname}"], f"{cname}.{fname}"
        assert ctypes.sizeof(cls) == c[f"{cname}.sizeof"], f"sizeof {cname}"


def test_constants_match_header(tmp_path):
    """Every integer macro QKV_* of the header has a binding constant of the
    same name and value (the values as the C compiler sees them)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    hdr = open(os.path.join(ROOT, "include", "qkv_epilogue.h")).read()
    names = [m for m in re.findall(r"^#define (QKV_\w+)[ \t]+\S", hdr, re.M)]
    assert len(names) >= 10
    body = "\n".join(f'    printf("{n} %lld\\n", (long long)({n}));' for n in names)
    src = tmp_path / "consts.c"
    src.write_text(f'#include <stdio.h>\n#include "qkv_epilogue.h"\nint main(void) {{\n{body}\n    return 0;\n}}\n')
    exe = tmp_path / "consts"
    subprocess.run([cc, "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    for line in out.splitlines():
        name, val = line.split()
        assert hasattr(B, name), f"binding lacks {name}"
        assert getattr(B, name) == int(val), f"{name}: binding {getattr(B, name)} != header {val}"
