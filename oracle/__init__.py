"""CPU oracle for EntroPack-style tile-rANS weight compression.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product (``decode_tile_rans_amd`` and its HIP library) never
imports it, and this package imports nothing from the product: the two share
no code, tables or constants; only the seeded input generators in ``synth``
serve both.

The oracle is deliberately plain: NumPy in float64 (float32 exactly where the
format fixes float32), every step written in the order the method applies it,
vectorised only across independent units (8-wide groups, rANS chains).

Citation keys used in the docstrings (the pages are the only specification):

[ABS]     "EntroPack: Fast and Accurate Entropy-Coded Weight Compression at
          Arbitrary Bitrates" (arXiv 2609.34185), English abstract, as shown on
          the arxivdaily.com and modelscope.ai paper pages.
[SUM]     The same paper's modelscope.ai page, section "摘要" (site summary): the
          only passage that names rANS and says symbol decode, algebraic
          inverse-lattice reconstruction and row rescale run fused on the GPU
          without an intermediate symbol tensor or reconstruction codebook.
[README]  EntroPack README_zh.md (GitHub mirror), sections "快速开始" (quick
          start: target_bpp range, actual_bpp includes metadata), "Config：压缩配置"
          and "性能" (H20 numbers).
[NEWS]    techmoon.xyz article "EntroPack 開源模型壓縮，任意位元率把權重塞進記憶體預算",
          section "任意位元率的本體：目標值、實際值、資料型態與無損選項" (target vs stored
          rate, 2-D lossy only, shape and dtype restored) and the following
          paragraph on the E8 grid and tile-wise entropy coding.

Where the pages are silent (almost every integer detail), the reading taken
is stated at the function that implements it; the full list sits in the
project's design notes.

Functions whose results the tests pin to something other than this code
(closed forms, brute force, IEEE/OCP definitions, round trips) say so.  The
exact symbol model and blob bytes are this project's own format: the pages
print no example, so their bytes are "parity unpinned" beyond round-trip,
invariant and rate-bar pins.
"""
from .codec import compress, decode, parse_blob, Blob  # noqa: F401
from . import e8, numerics, model, rans, rate, gemm  # noqa: F401
