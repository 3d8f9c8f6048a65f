"""CPU check of the hazard padding around the attention kernel's inline-asm matrix products.

The 64-row pipelined attention kernel (attn_bf16_pipe_kernel with two row blocks per wave) issues its
PV products as inline-asm v_mfma_f32_32x32x16_bf16 with AGPR accumulators.  The compiler schedules
around an asm statement without knowing it is a matrix product, so the hazards it would otherwise pad
are the source's own business:

* a VALU write of a product's A or B register needs two wait states before the product reads it;
* an ordinary read of an accumulator (v_accvgpr_read, a store of AGPR data) needs the product's result
  latency behind it (the source's fences pad 24 wait states);
* an ordinary write of an accumulator (v_accvgpr_write) needs wait states before a product reads it.

This test compiles window_attn.hip to gfx950 assembly with the library's own flags and walks every
instantiation of that kernel in program order, counting one wait state per instruction and N + 1 per
s_nop N.  It fails if any product is closer than that to such a write or read, so a compiler or source
change that moves an instruction into a product's shadow is caught on the CPU, before a GPU runs it.
The walk is linear (a branch into the middle of a window is not followed), which is how the fences are
placed: each sits in the same block as the reads or writes it guards.
"""
import os
import re
import subprocess
import tempfile

import pytest

from sink_window_kv_amd import build as sabuild

VALU_BEFORE_PRODUCT = 2     # wait states between a VALU write of A/B and the product
READ_AFTER_PRODUCT = 20     # wait states between a product and a read of its accumulator
WRITE_BEFORE_PRODUCT = 4    # wait states between an accumulator write and the product that reads it


def _device_asm():
    if not os.path.exists(sabuild.HIPCC):
        pytest.skip("hipcc not found")
    src = os.path.join(sabuild.CSRC, "window_attn.hip")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "window_attn.s")
        cmd = [sabuild.HIPCC, *sabuild.CFLAGS, *sabuild.EXTRA.get("window_attn.hip", []), "--cuda-device-only",
               "-S", src, "-o", out]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-4000:]
        with open(out) as f:
            return f.read()


def _kernels(asm):
    """(name, instruction list, metadata text) of every 64-row pipelined kernel."""
    names = re.findall(r"^(_ZN\S*attn_bf16_pipe_kernelILi\d+ELb[01]ELi2EEEvNS_8AttnArgsE):", asm, re.M)
    out = []
    for n in names:
        body = asm.split("\n" + n + ":", 1)[1].split("s_endpgm", 1)[0]
        ins = []
        for line in body.split("\n"):
            t = line.split(";", 1)[0].strip()
            if t and not t.startswith(".") and not t.endswith(":"):
                ins.append(t)
        meta = re.search(r"\.name:\s+" + re.escape(n) + r"\s*\n(.*?)\.wavefront_size", asm, re.S)
        out.append((n, ins, meta.group(1) if meta else ""))
    return out


def _regs(tok, kind):
    m = re.fullmatch(kind + r"\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(kind + r"(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _operands(ins):
    parts = ins.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def _wait_states(ins):
    op = ins.split()[0]
    return int(ins.split()[1], 0) + 1 if op == "s_nop" else 1


def _agpr_products(ins):
    return [i for i, t in enumerate(ins) if t.startswith("v_mfma") and _operands(t)[0].startswith("a")]


def _check_kernel(ins):
    problems = []
    products = _agpr_products(ins)
    # VALU writes of a product's A/B registers just before it
    for i in products:
        ops = _operands(ins[i])
        ab = _regs(ops[1], "v") | _regs(ops[2], "v")
        ws = 0
        for j in range(i - 1, -1, -1):
            ws += 0 if j == i - 1 else _wait_states(ins[j + 1])
            if ws >= VALU_BEFORE_PRODUCT:
                break
            t = ins[j]
            if t.startswith("v_") and not t.startswith("v_mfma") and _operands(t):
                if _regs(_operands(t)[0], "v") & ab:
                    problems.append(f"VALU write {ws} wait states before a product: {t} -> {ins[i]}")
    # accumulator reads after a product, accumulator writes before one
    for i, t in enumerate(ins):
        op = t.split()[0]
        if not t.startswith("v_mfma") and op != "v_accvgpr_write_b32" and any(o.startswith("a") for o in _operands(t)):
            # reads an AGPR: v_accvgpr_read, or a store of AGPR data
            a = set().union(*(_regs(o, "a") for o in _operands(t)))
            ws = 0
            for j in range(i - 1, -1, -1):
                u = ins[j]
                if u.startswith("v_mfma") and _regs(_operands(u)[0], "a") & a:
                    if ws < READ_AFTER_PRODUCT:
                        problems.append(f"accumulator read {ws} wait states after a product: {u} -> {t}")
                    break
                ws += _wait_states(u)
                if ws >= READ_AFTER_PRODUCT:
                    break
        elif op == "v_accvgpr_write_b32":
            a = _regs(_operands(t)[0], "a")
            ws = 0
            for j in range(i + 1, len(ins)):
                u = ins[j]
                if u.startswith("v_mfma"):
                    ops = _operands(u)
                    if (_regs(ops[0], "a") | _regs(ops[3], "a")) & a:
                        if ws < WRITE_BEFORE_PRODUCT:
                            problems.append(f"accumulator write {ws} wait states before a product: {t} -> {u}")
                        break
                ws += _wait_states(u)
                if ws >= WRITE_BEFORE_PRODUCT or u.startswith("s_branch") or u.startswith("s_cbranch"):
                    break
    return problems


def test_agpr_products_keep_their_hazard_padding():
    kernels = _kernels(_device_asm())
    assert len(kernels) == 4, [k[0] for k in kernels]  # D = 64 and 128, frames of at least one key tile or not
    for name, ins, meta in kernels:
        assert _agpr_products(ins), f"{name}: no AGPR-accumulator products (the asm path is gone)"
        spills = re.search(r"\.vgpr_spill_count:\s+(\d+)", meta)
        assert spills is not None and int(spills.group(1)) == 0, f"{name}: VGPR spills"
        problems = _check_kernel(ins)
        assert not problems, f"{name}:\n" + "\n".join(problems[:20])


def test_hazard_walk_catches_a_planted_violation():
    """The walk itself: a VALU write right before a product, a read or a store of an accumulator right after
    one, and an accumulator write right before one are reported; a read behind 24 wait states is not."""
    ins = ["v_mov_b32_e32 v4, 0",
           "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]",
           "v_accvgpr_read_b32 v20, a3",
           "s_nop 7", "s_nop 7", "s_nop 7",
           "v_accvgpr_read_b32 v21, a3",
           "v_accvgpr_write_b32 a5, v21",
           "v_mfma_f32_32x32x16_bf16 a[0:15], v[12:15], v[8:11], a[0:15]",
           "global_store_dwordx4 v[30:31], a[4:7], off"]
    problems = _check_kernel(ins)
    assert any("VALU write" in p for p in problems)
    assert sum("accumulator read" in p for p in problems) == 2   # the padded read passes, the store does not
    assert any("global_store" in p for p in problems)
    assert any("accumulator write" in p for p in problems)
