"""MI355X-native paged split-KV decode: planner, split decode and log-sum-exp merge.

The compute path is the HIP library built from ``csrc/``; ``binding`` marshals torch tensors into
its C entry points.  ``workloads`` draws seeded synthetic inputs.
"""
