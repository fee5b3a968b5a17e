"""MI355X-native large-chunk test-time-training (LaCT) layer.

The compute path is the HIP library ``libttt.so`` (C ABI declared in
``include/ttt.h``); ``test_weight_layers_amd.ttt`` is its thin Python binding.
Importing this package does not load the library: the binding loads it on first
use and raises if it is missing.
"""
