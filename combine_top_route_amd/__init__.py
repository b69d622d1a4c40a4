"""MI355X-native fused mixture-of-experts layer (forward and backward, one
GPU).  The compute path is the HIP library under csrc/, reached through the
C ABI declared in include/moe.h; `binding` marshals torch tensors to it."""
