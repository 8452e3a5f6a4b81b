"""Static checks of the attention kernels' gfx950 ISA (no GPU needed).

The 128-head decode kernel and the prefill attention kernel issue MFMAs from
inline asm with VGPR accumulators, which the compiler's hazard recognizer
does not see.  These tests compile mla_splitkv.hip and mla_prefill.hip to
assembly with the library's own flags and check:
  * no instruction reads a VGPR written by such an MFMA within 18 wait states
    (an XDL result needs ~11-12 on gfx950; 18 leaves margin), except the next
    MFMA of the same accumulate chain;
  * the kernels that stream tiles by LDS DMA have no scratch reload inside
    any loop that issues MFMAs (the tile loops of the fast path and of the
    16-head-group path): a spill reload is a VMEM access whose own wait would
    also drain the DMAs in flight.
"""
import os
import re
import subprocess

import pytest

from mla_latent_kv_24_amd import build as B

NEED_WAIT_STATES = 18
# the 128-head kernel over a contiguous and over a paged cache
WIDE = ["_ZN3mla19splitkv_wide_kernelILb0EEEvNS_9SplitArgsE",
        "_ZN3mla19splitkv_wide_kernelILb1EEEvNS_9SplitArgsE"]
# every tile-streaming decode kernel, both cache layouts
STREAMING = WIDE + [f"_ZN3mla{k}ILb{p}EEEvNS_9SplitArgsE" for k in ("18splitkv_h16_kernel",) for p in (0, 1)] + \
    [f"_ZN3mla19splitkv_mfma_kernelILi{c}ELb{p}EEEvNS_9SplitArgsE" for c in (2, 4) for p in (0, 1)]
MFMA_V = re.compile(r"^\s*v_mfma\S*\s+v\[(\d+):(\d+)\],\s*(\S+),\s*(\S+),\s*(\S+)")


def _compile(tmp_path_factory, src):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / src.replace(".hip", ".s")
    cmd = [cc, *B.common_flags(), "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return _compile(tmp_path_factory, "mla_splitkv.hip")


@pytest.fixture(scope="module")
def asm_prefill(tmp_path_factory):
    return _compile(tmp_path_factory, "mla_prefill.hip")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operand_regs(line):
    parts = line.split(None, 1)
    body = parts[1] if len(parts) > 1 else ""
    found = set()
    for t in re.findall(r"v\[\d+:\d+\]|\bv\d+\b", body):
        found |= _regs(t)
    return found


def _instructions(text):
    out = []
    for raw in text.splitlines():
        s = raw.strip()
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        out.append(s.split(";")[0].strip())
    return out


def _function(text, name):
    start = text.index(f"{name}:")
    end = text.index(".Lfunc_end", start)
    return text[start:end]


def vgpr_mfma_hazards(instrs, need=NEED_WAIT_STATES):
    """(mfma, reader, wait states) for every read of a VGPR-accumulator MFMA
    result that comes too early."""
    bad = []
    for i, ins in enumerate(instrs):
        m = MFMA_V.match(ins)
        if not m:
            continue
        dst = set(range(int(m.group(1)), int(m.group(2)) + 1))
        ws = 0
        for nxt in instrs[i + 1:i + 60]:
            if nxt.startswith("s_nop"):
                ws += int(nxt.split()[1]) + 1
                continue
            if ws >= need:
                break
            m2 = MFMA_V.match(nxt)
            if m2:
                if (_regs(m2.group(3)) | _regs(m2.group(4))) & dst:
                    bad.append((ins, nxt, ws))
                src_c = _regs(m2.group(5))
                d2 = set(range(int(m2.group(1)), int(m2.group(2)) + 1))
                if src_c & dst and src_c != dst:
                    bad.append((ins, nxt, ws))
                if d2 == dst and src_c == dst:
                    break          # the accumulate chain continues in this MFMA
                ws += 1
                continue
            if _operand_regs(nxt) & dst:
                bad.append((ins, nxt, ws))
            ws += 1
    return bad


def test_checker_flags_an_early_read():
    early = ["v_mfma_f32_32x32x16_bf16 v[18:33], v[2:5], v[6:9], v[18:33]", "s_nop 0",
             "v_mov_b64_e32 v[40:41], v[18:19]"]
    late = early[:1] + ["s_nop 7", "s_nop 7", "s_nop 7"] + early[2:]
    chain = early[:1] + ["v_mfma_f32_32x32x16_bf16 v[18:33], v[2:5], v[6:9], v[18:33]"]
    assert len(vgpr_mfma_hazards(early)) == 1
    assert vgpr_mfma_hazards(late) == []
    assert vgpr_mfma_hazards(chain) == []


def test_no_early_reads_of_vgpr_mfma_results(asm):
    bad = vgpr_mfma_hazards(_instructions(asm))
    assert not bad, bad[:5]


@pytest.mark.parametrize("name", WIDE)
def test_wide_kernel_has_vgpr_score_mfmas(asm, name):
    body = _instructions(_function(asm, name))
    assert sum(1 for s in body if MFMA_V.match(s)) >= 72      # prologue + one step's 36
    assert sum(1 for s in body if re.match(r"v_mfma\S*\s+a\[", s)) >= 32


def mfma_loops(text):
    """Bodies (instruction lists) of the loops of a function's assembly that
    issue MFMAs: from a loop header label to the branch back to it."""
    lines = text.splitlines()
    label_at = {}
    for i, raw in enumerate(lines):
        m = re.match(r"^(\.LBB\d+_\d+):", raw.strip())
        if m:
            label_at[m.group(1)] = i
    loops = []
    for i, raw in enumerate(lines):
        m = re.search(r"\bs_(?:cbranch_\w+|branch)\s+(\.LBB\d+_\d+)", raw)
        if m and m.group(1) in label_at and label_at[m.group(1)] < i:
            body = _instructions("\n".join(lines[label_at[m.group(1)]:i + 1]))
            if any(x.startswith("v_mfma") for x in body):
                loops.append(body)
    return loops


def test_loop_finder_sees_a_backedge():
    text = "\n".join(["k:", ".LBB0_1:", "  v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
                      "  scratch_load_dword v1, off, off", "  s_cbranch_scc1 .LBB0_1", "  s_endpgm"])
    loops = mfma_loops(text)
    assert len(loops) == 1 and any(x.startswith("scratch_load") for x in loops[0])


@pytest.mark.parametrize("name", STREAMING)
def test_streaming_kernel_loops_have_no_scratch_reloads(asm, name):
    loops = mfma_loops(_function(asm, name))
    assert loops
    for body in loops:
        assert not [s for s in body if s.startswith("scratch_load")]


PREFILL = ["_ZN3mla19prefill_attn_kernelILb1EEEvNS_11PrefillArgsE",
           "_ZN3mla19prefill_attn_kernelILb0EEEvNS_11PrefillArgsE"]


def test_prefill_no_early_reads_of_vgpr_mfma_results(asm_prefill):
    body = _instructions(asm_prefill)
    assert sum(1 for x in body if MFMA_V.match(x)) >= 64      # both instances issue VGPR-accumulator MFMAs
    bad = vgpr_mfma_hazards(body)
    assert not bad, bad[:5]


@pytest.mark.parametrize("name", PREFILL)
def test_prefill_attention_loop_has_no_scratch_reloads(asm_prefill, name):
    body = _instructions(_function(asm_prefill, name))
    idx = [i for i, x in enumerate(body) if x.startswith("v_mfma")]
    inside = body[idx[0]:idx[-1]]
    assert not [x for x in inside if x.startswith("scratch_load")]


def test_prefill_asm_mfmas_wait_after_valu_writes(asm_prefill):
    """The prefill kernel's asm MFMAs read sources that VALU code writes just
    before (P, copies of the queries, rescaled accumulators); an MFMA needs 2
    wait states after such a write, and the compiler inserts none for asm:
    each of these MFMAs is emitted right after an s_nop of at least 1."""
    for name in PREFILL:
        body = _instructions(_function(asm_prefill, name))
        for i, ins in enumerate(body):
            if MFMA_V.match(ins):
                assert body[i - 1].startswith("s_nop") and int(body[i - 1].split()[1]) >= 1, (name, i, body[i - 1])

