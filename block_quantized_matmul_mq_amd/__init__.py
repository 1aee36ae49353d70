"""MI355X-native matmul of GGUF block-quantized weights (Q8_0, Q4_K, Q6_K) with f32 activations.

The compute lives in the HIP library ``libmq.so`` (C ABI declared in
``include/mq.h``); ``block_quantized_matmul_mq_amd.mq`` is its thin ctypes
binding.  ``synth`` makes seeded synthetic inputs.
"""
