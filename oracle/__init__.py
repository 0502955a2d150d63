"""CPU oracle for the QLoRA frozen-NF4 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its
Python binding) may import, call, link or execute anything in this package; only
the test-suite, the smoke check and the benchmark's CPU-baseline leg use it.

The oracle is plain NumPy (float64 wherever the pages leave the precision open,
float32 exactly where the encoding fixes it) and shares no code with the HIP
path. Each function names the page passage it follows; pages are cited by title
and section:

  [QLoRA-65B]  "QLoRA는 어떻게 65B 모델을 GPU 한 장에 올렸나" (iq-universe blog,
               ch.4), sections "QLoRA의 수식", "명제 1", "메모리 회계".
  [48GB]       "48GB GPU Fine-Tuning a 65B Model: Where QLoRA Saves GPU Memory"
               (wink.run), sections "LoRA Freezes the Original Weights...",
               "Quantization Keeps the Patterns...", "QLoRA Puts the Two Methods
               in Different Places".
  [GPU-fit]    "8GB, 12GB, 16GB, 24GB GPU에서 몇 B 모델까지 LoRA 학습이 될까"
               (sotaaz), sections "무엇을 돌렸나", "메모리는 어디에 쓰이나".
  [QLoRA-2023] "QLoRA: Efficient Finetuning of Quantized LLMs" (tellworld
               summary), section "How it works".
"""

from .nf4 import (  # noqa: F401
    BLOCK,
    GROUP,
    nf4_codebook,
    nf4_levels_f64,
    nf4_midpoints_f64,
    nf4_thresholds_f32,
    bf16_round,
    block_absmax,
    nearest_level,
    pack_codes,
    unpack_codes,
    double_quant,
    quantize,
    dequant_scales,
    dequantize,
    storage_bytes,
    quantize_absmax,
    dequantize_absmax,
    storage_bytes_absmax,
)
from .qlora import lora_forward, lora_backward, lora_merge, bf16_round_f64  # noqa: F401
from .optim import adamw_step  # noqa: F401
