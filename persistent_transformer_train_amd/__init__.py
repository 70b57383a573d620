"""MI355X-native GPT training step with live-weight batch-1 decode.

The work runs in libofa.so (HIP for gfx950) behind the C ABI of include/ofa.h;
``persistent_transformer_train_amd.ofa`` is its thin Python binding (importing
it fails when the library has not been built).  ``synth`` draws the seeded
synthetic inputs; ``configs`` holds the five workload configurations.
"""
