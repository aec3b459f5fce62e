"""MI355X-native GPT-2 training step: HIP kernels for gfx950 behind a C ABI.

Importing the package does not load the native library; call
``decoder_only_transformer_train_amd.binding.load()`` (done by ``GPT``) for that.
"""
__all__ = ["synthetic", "configs"]
