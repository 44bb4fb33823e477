"""Plain fp64 CPU oracle for the folded-Hadamard ternary Packed-linear path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, tables or constants
with the HIP library.

Sources (cited by address and section; no worked example is printed there):

* [P2] kwkr.cn/news/564617 -- teardown of the Ternary-Bonsai-2-27B 2-bit MLX
  pack; sections "ternary weights + folded Hadamard rotation" and
  "packing-format engineering (MLX 2.25 bits vs GGUF)".
* [P3] lpnh.cn/news/2438023 -- guide to the pack's PACK-RUNTIME.md; sections
  "text model loading: artifact.load_model and the Packed module" and
  "affine 2-bit format and Prism contract v1".
* [P1] trdm.cn/news/822023 -- TensorSharp article; used only for the Sylvester
  recurrence (section 2.2) and the ternary-to-code mapping (section 3.2).
"""
from .reference import (  # noqa: F401
    BLOCK_SIZES,
    GROUP,
    CODES_PER_WORD,
    fwht_blocks,
    fwht_signed,
    codes_of,
    dequantize,
    dequantize_rows,
    pack,
    unpack,
    packed_linear,
    packed_linear_rows,
    embed_inverse,
    fold_rotation,
    container_bytes,
    bf16_bits_to_f64,
    f16_to_f64,
)
from .formats import (  # noqa: F401
    PQ2_BLOCK_BYTES,
    PTQ1_BLOCK_BYTES,
    pq2_from_mlx,
    pq2_to_mlx,
    pq2_codes,
    pq2_dequantize_rows,
    pq2_packed_linear,
    ptq1_pack,
    ptq1_unpack,
    ptq1_codes,
    ptq1_dequantize_rows,
    ptq1_packed_linear,
    container_bytes_pq2,
    container_bytes_ptq1,
)
