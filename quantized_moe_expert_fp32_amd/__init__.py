"""MI355X-native routed int4 Mixture-of-Experts layer (HIP/CDNA4 kernels behind a C ABI).

Importing the package loads nothing native; `quantized_moe_expert_fp32_amd.moe`
loads the HIP library and fails loudly when it is missing.
"""

__version__ = "0.1.0"
