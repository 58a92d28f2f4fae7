"""MI355X-native speech-encoder forward pass (log-mel frontend + Transformer).

The compute runs in the HIP library ``libspeech_encoder.so`` built from
``csrc/`` for gfx950; ``binding`` marshals torch device tensors and streams to
its C ABI.  ``workloads`` draws the seeded synthetic inputs.  Importing this
package loads nothing: the library is opened on first use of ``binding``.
"""
