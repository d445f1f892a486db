"""Wait-state check of compiled matrix-core code (device assembly of this library's own sources).

A matrix-core instruction writes its result registers several cycles after it issues; the compiler
must place enough independent instructions or `s_nop`s before anything else touches them.  The
number it needs per instruction is read off the compiler itself: a straight-line probe kernel per
instruction, whose result is read by the very next vector ALU operation, shows the wait states the
compiler inserts there.  Every path through the library's kernels is then walked forward from each
matrix-core instruction, across branches and joins, and any instruction that reads or writes its
result registers sooner is reported.  A following matrix-core instruction that takes exactly those
registers as its accumulator is exempt (the compiler chains such accumulations back to back), and
so is one that overwrites exactly those registers and takes at least as long (results land in issue
order).
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

# 16-row tiles of every matrix-core instruction the kernels use, with operand types for the probe
PROBE_OPS = {
    "v_mfma_f32_16x16x32_bf16": "acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A8[l], A8[l + 64], acc, 0, 0, 0);",
    "v_mfma_f32_16x16x32_f16": "acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(H8[l], H8[l + 64], acc, 0, 0, 0);",
    "v_mfma_f32_16x16x32_fp8_fp8": "acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(L[l], L[l + 64], acc, 0, 0, 0);",
    "v_mfma_scale_f32_16x16x128_f8f6f4":
        "acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(I8[l], I8[l + 64], acc, 0, 0, 0, 127, 0, 127);",
    "v_smfmac_f32_16x16x64_bf16":
        "acc = __builtin_amdgcn_smfmac_f32_16x16x64_bf16(A8[l], A16[l], acc, idx[l], 0, 0);",
    "v_smfmac_f32_16x16x64_f16": "acc = __builtin_amdgcn_smfmac_f32_16x16x64_f16(H8[l], H16[l], acc, idx[l], 0, 0);",
    "v_smfmac_f32_16x16x128_fp8_fp8":
        "acc = __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(I4[l], I8[l], acc, idx[l], 0, 0);",
}

_PROBE_HEAD = """#include <hip/hip_runtime.h>
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
"""
_PROBE_KERNEL = """__global__ void probe_{n}(const bf16x8* A8, const bf16x16* A16, const f16x8* H8, const f16x16* H16,
    const long* L, const i32x8* I8, const i32x4* I4, const int* idx, f32x4* C) {{
    const int l = threadIdx.x;
    f32x4 acc = C[l];
    {op}
    C[l] = acc + 1.0f;
}}
"""


def _ops(ins: str):
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip() for o in parts[1].split(",")]


def _regs(op: str) -> set:
    m = re.match(r"v\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", op)
    return {int(m.group(1))} if m else set()


def _waits(ins: str) -> int:
    m = re.match(r"s_nop (\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def parse(text: str):
    """Instructions of an assembly listing (labels resolved to instruction indices)."""
    code, labels = [], {}
    for line in text.split("\n"):
        t = line.split(";")[0].rstrip()
        if not t.strip():
            continue
        m = re.match(r"^([.\w$]+):", t)
        if m:
            labels[m.group(1)] = len(code)
            continue
        s = t.strip()
        if s.startswith("."):
            continue
        if t[0] in " \t":
            code.append(s)
    return code, labels


def _successors(code, labels, i):
    op, a = _ops(code[i])
    if op == "s_branch":
        return [labels[a[0]]]
    out = [labels[a[0]]] if op.startswith("s_cbranch") else []
    if op not in ("s_endpgm", "s_setpc_b64"):
        out.append(i + 1)
    return out


def _is_matrix(op: str) -> bool:
    return op.startswith("v_mfma") or op.startswith("v_smfmac")


def _exempt(op: str, args, dst: set, producer: str, need: dict) -> bool:
    """A later matrix-core instruction that takes exactly `dst` as its accumulator, or writes exactly
    `dst` no sooner than the producer does, and reads nothing else of it."""
    if not _is_matrix(op):
        return False
    # dense forms: D, A, B, C, ...; sparse forms: D (= accumulator), A, B, index
    acc_pos = 0 if op.startswith("v_smfmac") else 3
    if len(args) <= acc_pos:
        return False
    others = set()
    for k, x in enumerate(args):
        if k not in (0, acc_pos):
            others |= _regs(x)
    if others & dst:
        return False
    acc, out = _regs(args[acc_pos]), _regs(args[0])
    if acc & dst and acc != dst:
        return False
    if out & dst and (out != dst or need.get(op, 0) < need[producer]):
        return False
    return True


def violations(text: str, need: dict) -> list:
    """(wait states, producer, consumer) for every too-early touch of a matrix-core result."""
    code, labels = parse(text)
    found = {}
    for i, ins in enumerate(code):
        op, a = _ops(ins)
        if op not in need:
            continue
        dst = _regs(a[0])
        stack, seen = [(i + 1, 0)], set()
        while stack:
            pc, w = stack.pop()
            if pc >= len(code) or w >= need[op] or (pc, w) in seen:
                continue
            seen.add((pc, w))
            o, args = _ops(code[pc])
            touched = set()
            for x in args:
                touched |= _regs(x)
            if touched & dst and not _exempt(o, args, dst, op, need):
                found[(i, pc)] = min(w, found.get((i, pc), (w,))[0]), ins, code[pc]
                continue
            for s in _successors(code, labels, pc):
                stack.append((s, w + _waits(code[pc])))
    return list(found.values())


def device_asm(src: str, out: str, flags, hipcc: str) -> str:
    cmd = [hipcc, *flags, "-x", "hip", "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr}")
    with open(out) as f:
        return f.read()


def required_waits(flags, hipcc: str) -> dict:
    """Wait states the compiler puts between each instruction and an ALU read of its result."""
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "probe.hip")
        with open(src, "w") as f:
            f.write(_PROBE_HEAD)
            for n, (name, op) in enumerate(PROBE_OPS.items()):
                f.write(_PROBE_KERNEL.format(n=n, op=op))
        text = device_asm(src, os.path.join(d, "probe.s"), flags, hipcc)
    code, _ = parse(text)
    need = {}
    for i, ins in enumerate(code):
        op, a = _ops(ins)
        if op not in PROBE_OPS:
            continue
        dst, w = _regs(a[0]), 0
        for j in range(i + 1, len(code)):
            o, args = _ops(code[j])
            if o.startswith("v_") and any(_regs(x) & dst for x in args[1:]):
                need[op] = w
                break
            w += _waits(code[j])
    return need
