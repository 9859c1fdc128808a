"""The 64-bit address rebuild that the direct-to-LDS load helper (dma16 in
csrc/gfx950_asm.h) performs on the wave-uniform copy of a pointer: the helper
(csrc/uniform_ptr.h) is compiled here with the host compiler and checked on
addresses whose low word has bit 31 set.  Such a low half comes back from
readfirstlane as a negative int; widening it without going through uint32_t
sign-extends it into the high word, which once produced wrong load addresses
on the GPU.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "head_latent_attention_05_amd", "csrc")

PROGRAM = r'''
#include <cstdio>
#include <cstdint>
#include "uniform_ptr.h"
// stand-in for readfirstlane: identity, returning a signed int like the builtin
static int first(uint32_t x) { return (int)x; }
int main() {
  const uint64_t cases[] = {0x00007f1280000000ull, 0x00007fffffffffffull, 0x0000000080000010ull,
                            0x000012345678abcdull, 0x00000001ffffff00ull, 0x0000000000001000ull};
  int bad = 0;
  for (uint64_t v : cases) {
    const uint64_t r = mla::uniform_u64(v, first);
    if (r != v) { std::printf("%016llx -> %016llx\n", (unsigned long long)v, (unsigned long long)r); ++bad; }
  }
  return bad;
}
'''


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_uniform_pointer_rebuild_keeps_high_word(tmp_path):
    src = tmp_path / "t.cpp"
    src.write_text(PROGRAM)
    exe = tmp_path / "t"
    r = subprocess.run(["g++", "-std=c++17", "-O2", "-I", HEADER_DIR, str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, "address rebuilt wrongly:\n" + r.stdout


def test_dma_helper_uses_the_shared_rebuild():
    """The device helper must take its base address through uniform_u64, the
    function checked above (not an inline copy of the arithmetic)."""
    src = open(os.path.join(HEADER_DIR, "gfx950_asm.h")).read()
    body = src[src.index("void dma16("):src.index("asm volatile(", src.index("void dma16("))]
    assert "uniform_u64(" in body
