"""Copies the library's kernel sources for a host build under tests/cpu_emu.

LDS address-space qualifiers are dropped: with -no-pie the static LDS arrays
sit below 4 GiB, so the kernels' 32-bit LDS addresses stay valid pointers.
Each inline-assembly statement is replaced by its emulated meaning (exact text
substitutions, each required to match once, so a change in the sources fails
loudly here instead of being emulated wrongly):
  * the two MFMA forms        -> emu::mfma16x16x32 (zero or running accumulator)
  * the direct-to-LDS load    -> emu::dma16 (16 bytes per lane into 1 KiB of LDS)
  * the LDS store from the accumulation registers -> a 16-byte copy
  * v_max3_f32 and the accumulation-register read  -> plain C++
  * the LDS wait, the wait states and the scalar-register pinning -> nothing
The packed fp32 -> bf16 conversion becomes an explicit round-to-nearest-even
(the host compiler would call a runtime routine for it).  Everything else, the
other builtins included (hip/hip_runtime.h here), is compiled as it is.
"""
import os
import re
import shutil

LDS_SPACE = "__attribute__((address_space(3)))"

SUBS = {
    "gemm_core.hpp": [
        ('  asm volatile("s_mov_b32 m0, %2\\n\\tbuffer_load_dwordx4 %0, %1, 0 offen lds"\n'
         '               :\n'
         '               : "v"(off), "s"(desc), "s"(lds_addr)\n'
         '               : "memory", "m0");',
         '  emu::dma16(desc, off, lds_addr);'),
        ('asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));',
         'acc = emu::mfma16x16x32(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f});'),
        ('asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));',
         'acc = emu::mfma16x16x32(a, b, acc);'),
        ('asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "a"(a) : "memory");',
         'std::memcpy((void*)(uintptr_t)addr, &a, 16);'),
        ('asm volatile("s_nop 7\\n s_nop 7\\n s_nop 7" ::: "memory");', ';'),
        ('asm volatile("" ::"s"(w[i]));', '(void)w[i];'),
        ('return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));',
         'return emu::pack_bf16x2_rne(lo, hi);'),
    ],
    "epilogues.hpp": [
        ('asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");', ';'),
        ('asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));', 'r = fmaxf(fmaxf(a, b), c);'),
    ],
}
# Substitutions whose operands may be any expression: (regex, replacement), each matching once.
REGEX_SUBS = {
    "epilogues.hpp": [
        (r'asm volatile\("v_accvgpr_read_b32 %0, %1" : "=v"\((\w+)\) : "a"\(([^;]*)\)\);', r'\1 = \2;'),
    ],
}
PLAIN = ["kernels.hip", "attention.hip", "fingerprint.hip", "launch.hpp"]


def _code(text: str) -> str:
    return "\n".join(line.split("//")[0] for line in text.splitlines())


def prepare(csrc: str, emu_dir: str, out: str) -> None:
    os.makedirs(out, exist_ok=True)
    for name in list(SUBS) + PLAIN:
        text = open(os.path.join(csrc, name)).read().replace(LDS_SPACE, "")
        for old, new in SUBS.get(name, []):
            assert text.count(old) == 1, (name, old[:60])
            text = text.replace(old, new)
        for pattern, repl in REGEX_SUBS.get(name, []):
            text, n = re.subn(pattern, repl, text)
            assert n == 1, (name, pattern)
        assert "asm" not in _code(text).replace("#include", ""), name
        open(os.path.join(out, name), "w").write(text)
    shutil.copytree(os.path.join(emu_dir, "hip"), os.path.join(out, "hip"), dirs_exist_ok=True)
    shutil.copy(os.path.join(emu_dir, "lib_driver.cpp"), out)
